"""The oracle against its pins, and planted mistakes in copies of the oracle
that the pins must catch (all on the CPU)."""
import importlib.util
import os
import types

import pytest

import oracle.gmm_oracle as oracle
from tests import oracle_pins as pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "gmm_oracle.py")


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(oracle)


def _mutant(old: str, new: str) -> types.ModuleType:
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    spec = importlib.util.spec_from_loader("oracle_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


# (description, source anchor, replacement, the pin that must catch it)
MUTATIONS = [
    ("dropped log-determinant", "- 0.5 * maha - half_logdet[k]", "- 0.5 * maha",
     pins.check_log_joint_scipy),
    ("wrong sign of the quadratic", "logw[k] - 0.5 * maha", "logw[k] + 0.5 * maha",
     pins.check_log_joint_bruteforce),
    ("dropped log weight", "out[:, k] = logw[k] - 0.5", "out[:, k] = 0.0 - 0.5",
     pins.check_log_joint_scipy),
    ("log pi instead of log 2pi", "LOG_2PI = math.log(2.0 * math.pi)", "LOG_2PI = math.log(math.pi)",
     pins.check_k1_closed_form),
    ("unshifted log-sum-exp", "return (m + np.log(np.sum(np.exp(L - m)", "return (0 + np.log(np.sum(np.exp(L - 0)",
     pins.check_logz_scipy),
    ("S2 accumulates x not x^2", "S2 += r.T @ (x * x)", "S2 += r.T @ x",
     pins.check_stats_invariants),
    ("N_k summed over components", "Nk += r.sum(axis=0)", "Nk += r.sum(axis=1).sum() / r.shape[1]",
     pins.check_stats_bruteforce),
    ("variance about the old mean", "var = np.maximum(S2 / safe - mu * mu, var_floor)",
     "var = np.maximum(S2 / safe - prev_means * prev_means, var_floor)", pins.check_sklearn_one_step),
    ("variance without the mean term", "var = np.maximum(S2 / safe - mu * mu, var_floor)",
     "var = np.maximum(S2 / safe, var_floor)", pins.check_k1_closed_form),
    ("weights over K", "weights = Nk / float(n_total)", "weights = Nk / float(Nk.shape[0])",
     pins.check_sklearn_one_step),
    ("floor not applied", "var = np.maximum(S2 / safe - mu * mu, var_floor)",
     "var = S2 / safe - mu * mu", pins.check_floor_and_empty),
    ("empty component not kept", "means = np.where(live[:, None], mu, prev_means)", "means = mu",
     pins.check_floor_and_empty),
    ("sample variance in init", "v = np.maximum(np.var(_f64(X), axis=0), var_floor)",
     "v = np.maximum(np.var(_f64(X), axis=0, ddof=1), var_floor)", pins.check_init),
    ("extras ranked ascending", "order = np.lexsort((cand, -rn[cand]))", "order = np.lexsort((cand, rn[cand]))",
     pins.check_soft_assign_bruteforce),
    ("strict threshold", "cand = idx[(rn >= threshold) & (idx != top)]",
     "cand = idx[(rn > threshold + 0.02) & (idx != top)]", pins.check_soft_assign_bruteforce),
    ("lists in descending row order", "for n, lst in enumerate(lists):  # rows in ascending order",
     "for n, lst in reversed(list(enumerate(lists))):", pins.check_soft_assign_bruteforce),
    ("quadratic halved twice", "out[:, k] = logw[k] - 0.5 * maha", "out[:, k] = logw[k] - 0.25 * maha",
     pins.check_two_component_logistic),
    ("gemm form sign slip", "- 2.0 * (X @ (mu * inv).T)", "+ 2.0 * (X @ (mu * inv).T)",
     pins.check_gemm_matches_direct),
    ("argmax tested against the threshold", "kept_rank = others[:m]",
     "kept_rank = np.concatenate(([rn[a]], others[:m]))", pins.check_boundary_rows),
    ("boundary threshold test ignores rank", "kept_rank = others[:m]", "kept_rank = others",
     pins.check_boundary_rows),
    ("no argmax tie", "if rn[a] - others[0] <= eps:", "if False:", pins.check_boundary_rows),
    ("no rank-cut tie", "and others[m - 1] - others[m] <= eps:", "and False:", pins.check_boundary_rows),
    ("rank cut without the threshold", "others[m] >= threshold - eps and ", "", pins.check_boundary_rows),
    ("threshold tested with no extras", """        if m == 0:
            continue
        kept_rank""", """        kept_rank""", pins.check_boundary_rows),
    ("CSR list loses its last row", "for n in ids[offsets[k]:offsets[k + 1]]:",
     "for n in ids[offsets[k]:offsets[k + 1] - 1]:", pins.check_csr_to_lists),
]


@pytest.mark.parametrize("desc,old,new,check", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(desc, old, new, check):
    mod = _mutant(old, new)
    with pytest.raises((AssertionError, ValueError, FloatingPointError)):
        check(mod)


def test_oracle_matches_its_golden_fixture():
    import json
    import numpy as np
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "oracle_tiny.json")))
    X, W, MU, VAR = (np.array(g[k], np.float32) for k in ("X", "weights", "means", "vars"))
    Nk, S1, S2, ll = oracle.estep_stats(X, W, MU, VAR, method="direct")
    for got, key in ((Nk, "Nk"), (S1, "S1"), (S2, "S2"), (ll, "loglik")):
        np.testing.assert_allclose(got, g[key], rtol=1e-13, atol=1e-13)
    w1, mu1, v1 = oracle.mstep(Nk, S1, S2, X.shape[0], g["var_floor"], MU, VAR)
    np.testing.assert_allclose(v1, g["vars1"], rtol=1e-12)
    off, ids, _, _ = oracle.soft_assign(X, W, MU, VAR, g["threshold"], g["max_extra"], method="direct")
    assert off.tolist() == g["offsets"] and ids.tolist() == g["ids"]
