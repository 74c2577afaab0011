"""The seeded generators: determinism and the stated distributions."""
import numpy as np

import synth


def test_deterministic():
    a = synth.make_config_layer(1, 4)
    b = synth.make_config_layer(1, 4)
    for f in ("S1", "S2", "alpha", "beta", "gamma", "x"):
        assert getattr(a, f).tobytes() == getattr(b, f).tobytes()
    c = synth.make_config_layer(1, 4, integer=True)
    assert c.x.tobytes() != a.x.tobytes()


def test_shapes_and_types():
    L = synth.make_config_layer(2, 8)
    assert L.S1.shape == (4096, 64) and L.S2.shape == (64, 4096)
    assert L.alpha.shape == (1, 4096) and L.beta.shape == (1, 64) and L.gamma.shape == (1, 4096)
    assert L.x.shape == (8, 4096) and L.x.dtype == np.float16
    assert L.S1.dtype == np.int8 and set(np.unique(L.S1)) == {-1, 1}


def test_bernoulli_and_lognormal():
    L = synth.make_config_layer(3, 1)
    assert abs(L.S2.mean()) < 0.01
    med = float(np.median(L.alpha.astype(np.float64)))
    assert abs(med - np.exp(-3.0)) / np.exp(-3.0) < 0.05


def test_integer_variant():
    L = synth.make_config_layer(1, 4, integer=True)
    assert set(np.unique(L.x.astype(int))) <= set(range(-3, 4))
    assert np.all(L.alpha == 1) and np.all(L.beta == 1) and np.all(L.gamma == 1)


def test_outlier_channels():
    L = synth.make_layer(64, 8, 4096, 1, 64, 4016, outlier_frac=0.01)
    col_rms = np.sqrt((L.x.astype(np.float64) ** 2).mean(axis=0))
    assert np.sum(col_rms > 8) == 41  # ceil(0.01 * 4096) channels scaled x20


def test_zipf_ids():
    B = synth.make_multi_adapter(num_adapters=64, N=8, R=4, M=8, ell=2, T=2048, seed=5000)
    ids = B.ids
    assert ids.dtype == np.int32 and ids.min() >= 0 and ids.max() < 64
    assert np.all(np.diff(ids) >= 0)
    head = np.mean(ids == 0)
    assert 0.2 < head < 0.3  # P(rank 1) = 1 / sum k^-1.1 ~ 0.25
