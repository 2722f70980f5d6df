"""The isotropic oracle against its pins, and planted mistakes in copies of it
that the pins must catch (all on the CPU)."""
import importlib.util
import os
import types

import pytest

import oracle.gmm_oracle_iso as oracle_iso
from tests import oracle_iso_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "gmm_oracle_iso.py")


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(oracle_iso)


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    spec = importlib.util.spec_from_loader("oracle_iso_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src.replace(old, new), "oracle_iso_mutant", "exec"), mod.__dict__)
    return mod


MUTATIONS = [
    ("log-determinant without the D factor", "const = logw - 0.5 * D * (LOG_2PI + np.log(v))",
     "const = logw - 0.5 * (LOG_2PI + np.log(v))", pins.check_iso_log_joint_scipy),
    ("distance halved twice", "out[:, k] = const[k] - d2 / (2.0 * v[k])", "out[:, k] = const[k] - d2 / (4.0 * v[k])",
     pins.check_iso_log_joint_scipy),
    ("gemm form sign slip", "- 2.0 * (x @ mu.T)", "+ 2.0 * (x @ mu.T)", pins.check_iso_gemm_matches_direct),
    ("Q without squares", "Q += r.T @ np.sum(x * x, axis=1)", "Q += r.T @ np.sum(x, axis=1)",
     pins.check_iso_stats_invariants),
    ("variance not averaged over D", "var = np.maximum((Q / safe - np.sum(mu * mu, axis=1)) / D, var_floor)",
     "var = np.maximum(Q / safe - np.sum(mu * mu, axis=1), var_floor)", pins.check_iso_k1_closed_form),
    ("variance about the old mean", "var = np.maximum((Q / safe - np.sum(mu * mu, axis=1)) / D, var_floor)",
     "var = np.maximum((Q / safe - np.sum(prev_means * prev_means, axis=1)) / D, var_floor)",
     pins.check_iso_sklearn_one_step),
    ("floor not applied", "var = np.maximum((Q / safe - np.sum(mu * mu, axis=1)) / D, var_floor)",
     "var = (Q / safe - np.sum(mu * mu, axis=1)) / D", pins.check_iso_floor_and_empty),
    ("init takes the largest variance", "v = max(float(np.mean(np.var(x, axis=0))), var_floor)",
     "v = max(float(np.max(np.var(x, axis=0))), var_floor)", pins.check_iso_init),
    ("weights over K", "weights = Nk / float(n_total)", "weights = Nk / float(Nk.shape[0])",
     pins.check_iso_sklearn_one_step),
]


@pytest.mark.parametrize("desc,old,new,check", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(desc, old, new, check):
    with pytest.raises((AssertionError, ValueError, FloatingPointError)):
        check(_mutant(old, new))
