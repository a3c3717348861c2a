"""The forward-backward E8 denoiser (codebooks that are the first K points of
E8 in (norm, lexicographic) order) against the oracle's scan of the whole
codebook, and against the library's own codebook-scan kernel; codebooks that
are not such a prefix keep the scan kernel.  Tolerances as for every
denoiser test: x_hat and the per-row variance sum 1e-4 relative."""
import numpy as np
import pytest

import mpq_synth as S
from oracle import mpq_oracle as O
from parity_helpers import SOFT_RTOL, dev, host, rel_vec, rel_scalar

pytestmark = pytest.mark.gpu


def oracle_denoise(R1, g1, E, a, o):
    xs, vs = [], []
    for k in range(R1.shape[0]):
        C = O.row_codewords(E, a[k], o[k])
        x, v, _ = O.denoise(R1[k].astype(np.float64), float(g1[k]), C, 8)
        xs.append(x)
        vs.append(v)
    return np.stack(xs), np.stack(vs)


def compare(R1, g1, E, a, o, **kw):
    import post_quantization_solver_amd as mpq
    xh, vt = mpq.denoise(dev(np.asarray(R1, np.float64)), dev(np.asarray(g1, np.float64)), E, dev(a), dev(o), **kw)
    xh, vt = host(xh), host(vt)
    xr, vr = oracle_denoise(R1, g1, E, a, o)
    wx = max(rel_vec(xh[k], xr[k]) for k in range(R1.shape[0]))
    wv = max(rel_scalar(vt[k].astype(np.float64).sum(), vr[k].sum()) for k in range(R1.shape[0]))
    return wx, wv, xh, vt


@pytest.mark.parametrize("K", [1, 240, 1000, 2401, 65536])
@pytest.mark.parametrize("kappa", [0.05, 1.0, 30.0])
def test_e8dp_denoiser(K, kappa):
    import post_quantization_solver_amd as mpq
    E = S.e8_codebook(K)
    assert mpq.codebook_kind(E) == "e8_prefix"
    g = np.random.default_rng(K + int(kappa * 100))
    m, n = 6, 64
    a = (0.3 + g.random(m)).astype(np.float32)
    o = (0.1 * g.standard_normal(m)).astype(np.float32)
    R1 = (g.standard_normal((m, n)) * 1.3 * a[:, None] + o[:, None]).astype(np.float32)
    g1 = (kappa / a.astype(np.float64) ** 2).astype(np.float32)
    wx, wv, xh, vt = compare(R1, g1, E, a, o)
    print(f"[e8dp] K={K} kappa={kappa}: xhat {wx:.2e} sum v {wv:.2e}", flush=True)
    assert wx < 1e-9 and wv < 1e-9    # float64 throughout, like the oracle
    # the codebook-scan kernel on the same inputs agrees too
    wx2, wv2, xs, vs = compare(R1, g1, E, a, o, scan_denoiser=True)
    assert wx2 < SOFT_RTOL and wv2 < SOFT_RTOL


def test_e8dp_underflow_goes_to_exact_pass():
    """Queries far outside the codebook with a sharp posterior: the normaliser
    of the factorised pass underflows float64 and the exact pass takes over."""
    E = S.e8_codebook(65536)
    m, n = 2, 16
    a = np.ones(m, np.float32)
    o = np.zeros(m, np.float32)
    R1 = np.zeros((m, n), np.float32)
    R1[:, 0] = 10.0
    R1[:, 9] = -9.0
    g1 = np.full(m, 600.0, np.float32)
    wx, wv, xh, vt = compare(R1, g1, E, a, o)
    print(f"[e8dp underflow] xhat {wx:.2e} sum v {wv:.2e}", flush=True)
    assert wx < SOFT_RTOL and wv < SOFT_RTOL


def test_non_prefix_codebooks_use_the_scan():
    import post_quantization_solver_amd as mpq
    E = S.e8_codebook(1000)
    shuffled = E[np.random.default_rng(3).permutation(1000)]
    assert mpq.codebook_kind(shuffled) == "generic"
    assert mpq.codebook_kind(np.delete(E, 10, axis=0)) == "generic"
    g = np.random.default_rng(4)
    m, n = 4, 64
    a = np.full(m, 0.7, np.float32)
    o = np.zeros(m, np.float32)
    R1 = (g.standard_normal((m, n)) * 0.9).astype(np.float32)
    g1 = np.full(m, 2.0, np.float32)
    wx, wv, _, _ = compare(R1, g1, shuffled, a, o)
    assert wx < SOFT_RTOL and wv < SOFT_RTOL


def test_layer_with_and_without_e8dp():
    """A whole lattice layer: the forward-backward path and the scan path both
    match the oracle's codes (each teacher-forced stage is covered elsewhere)."""
    import torch
    import post_quantization_solver_amd as mpq
    from oracle.pool import solve_rows
    from parity_helpers import CODE_FRAC, layer_tensors, compare_layer
    L = S.make_layer("e8dp_layer", 12, 128, seed=91, d=8, K=4096, power=0.6, T_vamp=6)
    T = layer_tensors(L)
    refs = solve_rows(L, np.arange(L.m))
    for scan in (False, True):
        out = mpq.quantize_layer(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], T_vamp=L.T_vamp, n_cd=L.n_cd,
                                 damping=L.damping, scan_denoiser=scan)
        torch.cuda.synchronize()
        gpu = {k: (host(v) if v is not None else None) for k, v in out.items()}
        summ = compare_layer(L, np.arange(L.m), gpu, refs)
        print(f"[e8dp layer] scan={scan}: codes {summ['code_agreement']:.5f} traces {summ['trace_rel_max']}",
              flush=True)
        assert summ["code_agreement"] >= CODE_FRAC
        for key, v in summ["trace_rel_max"].items():
            assert v < SOFT_RTOL, (key, v)


@pytest.mark.parametrize("K", [2401, 65536])
def test_e8dp_ragged_and_frozen(K):
    """15 queries (the last wave of four rows of the forward-backward kernel is
    partly empty) and a frozen row (infinite precision: the cavity passes
    through with variance 0) between two live ones; K = 2401 ends in an
    integer point, 65536 in a half-integer one."""
    import post_quantization_solver_amd as mpq
    E = S.e8_codebook(K)
    g = np.random.default_rng(17)
    m, n = 3, 40
    a = (0.5 + g.random(m)).astype(np.float32)
    o = (0.1 * g.standard_normal(m)).astype(np.float32)
    R1 = (g.standard_normal((m, n)) * 1.2 * a[:, None] + o[:, None]).astype(np.float32)
    g1 = (np.array([0.7, 1.0, 4.0]) / a.astype(np.float64) ** 2).astype(np.float32)
    g1[1] = np.inf
    xh, vt = mpq.denoise(dev(R1.astype(np.float64)), dev(g1.astype(np.float64)), E, dev(a), dev(o))
    xh, vt = host(xh), host(vt)
    assert np.array_equal(xh[1], R1[1]) and np.all(vt[1] == 0)
    live = [0, 2]
    xr, vr = oracle_denoise(R1[live], g1[live], E, a[live], o[live])
    for t, k in enumerate(live):
        assert rel_vec(xh[k], xr[t]) < SOFT_RTOL
        assert rel_scalar(vt[k].astype(np.float64).sum(), vr[t].sum()) < SOFT_RTOL


def _e8_map(R1, E, a, o, scan=False):
    import post_quantization_solver_amd as mpq
    g1 = np.ones(R1.shape[0], np.float64)
    return host(mpq.map_codes(dev(np.asarray(R1, np.float64)), dev(g1), E, dev(a), dev(o),
                              scan_denoiser=scan)).astype(np.int64)


def _oracle_nearest(R1, E, a, o):
    return np.stack([O.nearest_codeword(R1[k].astype(np.float64), O.row_codewords(E, a[k], o[k]), 8)
                     for k in range(R1.shape[0])])


@pytest.mark.parametrize("K", [1, 240, 1000, 2401, 65536])
def test_e8_nearest_matches_oracle(K):
    """The max-sum pass over the E8 automaton (round to nearest and the
    marginal MAP) names the oracle's nearest codeword, ties to the lowest
    index, on 15 blocks per row (a partly empty last wave) at several scales."""
    E = S.e8_codebook(K)
    g = np.random.default_rng(K)
    m, n = 4, 120
    a = (0.4 + g.random(m)).astype(np.float32)
    o = (0.1 * g.standard_normal(m)).astype(np.float32)
    scale = np.array([0.6, 1.3, 3.0, 8.0])[:, None]
    R1 = (g.standard_normal((m, n)) * scale * a[:, None] + o[:, None]).astype(np.float32)
    got = _e8_map(R1, E, a, o)
    ref = _oracle_nearest(R1, E, a, o)
    print(f"[e8 nearest] K={K}: {np.mean(got == ref):.4f} agree", flush=True)
    assert np.array_equal(got, ref)
    scan = _e8_map(R1, E, a, o, scan=True)
    assert np.mean(scan == ref) >= 0.99


def test_e8_nearest_exact_ties():
    """Points equidistant from several codewords: the lowest codebook index
    wins, as in the oracle (a = 1, o = 0, dyadic coordinates, exact in float64)."""
    E = S.e8_codebook(65536)
    rows = [np.zeros(8), [0.5, 0.5, 0, 0, 0, 0, 0, 0], [0.25] * 8, [-0.5, 0.5, 0, 0, 0, 0, 0, 0],
            [0.75, 0.25, 0.25, 0.25, 0.25, 0.25, 0.25, 0.25], [1, 0, 0, 0, 0, 0, 0, 0], [0.5] * 8,
            [-1.5, 0, 0.5, 0, 0, 0, 0, 0]]
    R1 = np.asarray(rows, np.float32).reshape(1, -1)
    a = np.ones(1, np.float32)
    o = np.zeros(1, np.float32)
    got = _e8_map(R1, E, a, o)
    ref = _oracle_nearest(R1, E, a, o)
    assert np.array_equal(got, ref), (got, ref)


@pytest.mark.parametrize("K", [2401, 65536])
def test_e8_decoder_equals_automaton(K):
    """The lattice decoder's fast path (blocks whose nearest E8 point is unique
    by a margin and a codeword) and the automaton alone name the same codeword
    for every block: 8192 blocks from well inside the codebook to far outside
    it (scales 0.3 to 12 codeword units), plus exact ties and non-finite
    rows, which the decoder hands to the automaton."""
    import post_quantization_solver_amd as mpq
    E = S.e8_codebook(K)
    g = np.random.default_rng(K + 7)
    m, n = 64, 1024
    a = (0.2 + g.random(m)).astype(np.float32)
    o = (0.05 * g.standard_normal(m)).astype(np.float32)
    scale = np.array([0.3, 0.8, 1.5, 3.0, 6.0, 12.0, 1.0, 2.0] * 8)[:, None]
    R1 = (g.standard_normal((m, n)) * scale * a[:, None] + o[:, None]).astype(np.float32)
    # exact ties (a = 1, o = 0 rows) and a non-finite block
    a[:2] = 1.0
    o[:2] = 0.0
    R1[0, :16] = [0.5, 0.5, 0, 0, 0, 0, 0, 0] + [0.25] * 8
    R1[1, :8] = np.inf
    T = {k: dev(v) for k, v in (("a", a), ("o", o), ("R1", R1.astype(np.float64)))}
    g1 = dev(np.ones(m, np.float64))
    fast = host(mpq.map_codes(T["R1"], g1, E, T["a"], T["o"]))
    slow = host(mpq.map_codes(T["R1"], g1, E, T["a"], T["o"], e8_decode=False))
    print(f"[e8 decoder] K={K}: {np.mean(fast == slow):.6f} agree", flush=True)
    assert np.array_equal(fast, slow)
    ref = _oracle_nearest(R1[2:8], E, a[2:8], o[2:8])
    assert np.array_equal(fast[2:8], ref)
