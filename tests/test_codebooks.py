"""Input-side pins: the truncated E8 table and the Min-Max scalar grid (T10)."""
import numpy as np

import mpq_synth as S
from mpq_synth.codebooks import _e8_points_norm2_at_most


def test_e8_theta_series_shells():
    """Shell sizes of E8 up to norm^2 12 are the theta-series coefficients
    1, 240, 2160, 6720, 17520, 30240, 60480 (240 * sigma_3(k))."""
    pts = _e8_points_norm2_at_most(12)
    n2 = (pts * pts).sum(1)
    counts = {int(k): int((n2 == k).sum()) for k in np.unique(n2)}
    sigma3 = lambda k: sum(d ** 3 for d in range(1, k + 1) if k % d == 0)  # noqa: E731
    assert counts == {0: 1, **{2 * k: 240 * sigma3(k) for k in range(1, 7)}}


def test_e8_codebook_table():
    E = S.e8_codebook()
    assert E.shape == (65536, 8) and E.dtype == np.float32
    E64 = E.astype(np.float64)
    n2 = (E64 ** 2).sum(1)
    # every entry is a lattice point: all-integer or all-half-odd with even sum
    twice = 2 * E64
    assert np.all(twice == np.round(twice))
    integer = np.all(E64 == np.round(E64), axis=1)
    half = np.all(np.abs(E64 - np.round(E64)) == 0.5, axis=1)
    assert np.all(integer | half)
    assert np.all(np.mod(E64.sum(1), 2) == 0)
    assert len({tuple(r) for r in E64.tolist()}) == 65536
    # all shells up to 10, then the first 8655 of shell 12
    assert int((n2 <= 10).sum()) == 56881 and int((n2 == 12).sum()) == 8655
    # ascending (norm^2, x1..x8)
    keys = np.concatenate([n2[:, None], E64], 1)
    assert all(tuple(keys[i]) < tuple(keys[i + 1]) for i in range(0, 65535, 97))
    assert np.all(np.diff(n2) >= 0)
    # fingerprints and RMS
    assert E64[0].tolist() == [0.0] * 8
    assert E64[1].tolist() == [-1, -1, 0, 0, 0, 0, 0, 0]
    assert E64[65535].tolist() == [-1.5, 0.5, 1.5, -2.5, -0.5, 0.5, -0.5, 0.5]
    assert np.isclose(np.sqrt((E64 ** 2).mean()), S.E8_RAW_RMS, rtol=1e-15)
    # exact in bfloat16: at most 8 significant bits (half-integers up to 3)
    assert np.all(np.abs(E64) <= 3)


def test_scalar_grid_min_max():
    """Min-Max rule (NeUQI notes, uniform quantisation): scale = (max-min)/(2^k-1),
    integer zero-point z = round(-min/scale); levels scale*(q - z)."""
    W = np.array([[-1.0, 0.0, 2.5, 0.4], [3.0, 3.0, 3.0, 3.0]], dtype=np.float32)
    E, a, o = S.scalar_grid(W, 3)
    assert E[:, 0].tolist() == list(range(8))
    assert np.isclose(a[0], 3.5 / 7)
    assert np.isclose(o[0], -0.5 * 2)          # z = round(1 / 0.5) = 2
    assert a[1] == 1.0                          # constant row: scale fixed to 1
    lv = a[0] * E[:, 0] + o[0]
    assert np.isclose(lv.min(), -1.0) and np.isclose(lv.max(), 2.5)


def test_config_shapes_small():
    L = S.make_config("c1")
    assert L.W.shape == (64, 256) and L.V.shape == (256, 256) and L.s.shape == (256,)
    assert np.allclose(L.V.T.astype(np.float64) @ L.V, np.eye(256), atol=1e-5)
    assert np.isclose(L.s[3], 4 ** -0.5)
    assert list(S.parity_rows(4096)[:3]) == [0, 64, 128]
    L2 = S.make_layer("x", 8, 64, seed=3, d=8, K=4096)
    assert L2.E.shape == (4096, 8) and np.all(L2.o == 0)
