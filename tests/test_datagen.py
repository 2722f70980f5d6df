"""Seeded generators: determinism, prefix property, and the laws' shapes."""
import numpy as np
import torch

from soft_clustering_amd import datagen


def test_same_seed_same_bytes():
    mix = datagen.mixture("mid", 16, 8, seed=0)
    a = datagen.sample(mix, 1000, seed=0)
    b = datagen.sample(mix, 1000, seed=0)
    assert torch.equal(a, b)
    c = datagen.sample(mix, 1000, seed=1)
    assert not torch.equal(a, c)


def test_ranges_are_slices_of_one_sample():
    mix = datagen.mixture("tiny", 8, 16, seed=0)
    n = datagen.CHUNK + 1777
    whole = datagen.sample(mix, n, seed=0)
    part = datagen.sample(mix, 1500, start=datagen.CHUNK - 700, seed=0)
    assert torch.equal(part, whole[datagen.CHUNK - 700: datagen.CHUNK + 800])


def test_strided_buffer_padding_is_nan():
    mix = datagen.mixture("tiny", 8, 16, seed=0)
    x = datagen.sample(mix, 100, seed=0, ldx=12)
    assert x.stride(0) == 12 and x.shape == (100, 8)
    assert torch.isnan(x.as_strided((100, 4), (12, 1), 8)).all()
    assert torch.equal(x, datagen.sample(mix, 100, seed=0))


def test_laws():
    m = datagen.mixture("tiny", 8, 16, seed=0)
    assert m.means.min() >= -10 and m.means.max() <= 10
    assert m.stds.min() >= 0.5 and m.stds.max() <= 2
    assert abs(m.weights.sum() - 1) < 1e-12
    e = datagen.mixture("embed", 64, 32, seed=0)
    assert np.allclose(np.linalg.norm(e.means, axis=1), 1.0)
    x = datagen.sample(e, 500, seed=0)
    assert torch.allclose(torch.linalg.vector_norm(x, dim=1), torch.ones(500), atol=1e-5)
    v = datagen.mixture("ivf", 16, 64, seed=0)
    xi = datagen.sample(v, 2000, seed=0)
    assert torch.equal(xi, torch.round(xi)) and xi.min() >= 0 and xi.max() <= 255


def test_sample_follows_law():
    mix = datagen.mixture("mid", 4, 3, seed=5)
    lab = torch.empty(200_000, dtype=torch.int64)
    x = datagen.sample_into(torch.empty(200_000, 4), mix, 0, seed=5, labels_out=lab).double().numpy()
    lab = lab.numpy()
    freq = np.bincount(lab, minlength=3) / lab.shape[0]
    assert np.all(np.abs(freq - mix.weights) < 5 * np.sqrt(mix.weights / lab.shape[0]))
    for k in range(3):
        xs = x[lab == k]
        assert np.all(np.abs(xs.mean(0) - mix.means[k]) < 6 * mix.stds[k] / np.sqrt(len(xs)))
        assert np.all(np.abs(xs.std(0) / mix.stds[k] - 1) < 0.03)


def test_init_rows_distinct():
    r = datagen.init_rows(1000, 100, seed=1)
    assert len(set(r.tolist())) == 100 and r.min() >= 0 and r.max() < 1000
    assert np.array_equal(r, datagen.init_rows(1000, 100, seed=1))
