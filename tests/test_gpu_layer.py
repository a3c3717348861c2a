"""End-to-end parity of mpq_quantize_layer with the oracle on small layers
(all rows), plus edge cases: ragged shapes, r < n, padded lattice codebooks,
frozen rows, T_vamp = 0, n_cd = 0, m = 0, determinism."""
import numpy as np
import pytest

import mpq_synth as S
from oracle import mpq_oracle as O
from parity_helpers import SOFT_RTOL, OBJ_RTOL, CODE_FRAC, dev, host, layer_tensors, compare_layer
from oracle.pool import solve_rows

pytestmark = pytest.mark.gpu


def run_gpu(L, T_vamp=None, n_cd=None, **kw):
    import torch
    import post_quantization_solver_amd as mpq
    T = layer_tensors(L)
    out = mpq.quantize_layer(T["W"], T["s"], T["V"], L.E, T["a"], T["o"],
                             T_vamp=L.T_vamp if T_vamp is None else T_vamp,
                             n_cd=L.n_cd if n_cd is None else n_cd, damping=L.damping, diagnostics=True, **kw)
    torch.cuda.synchronize()
    return {k: (host(v) if v is not None else None) for k, v in out.items()}


CASES = {
    "c1": lambda: S.make_config("c1"),
    "ragged_scalar": lambda: S.make_layer("ragged_scalar", 37, 200, seed=21, d=1, bits=4, power=0.6, r=150, T_vamp=6),
    "scalar_k2": lambda: S.make_layer("scalar_k2", 9, 40, seed=22, d=1, bits=1, power=0.5, T_vamp=5),
    "scalar_k64": lambda: S.make_layer("scalar_k64", 9, 72, seed=23, d=1, bits=6, power=0.5, T_vamp=5),
    "lattice_small": lambda: S.make_layer("lattice_small", 24, 136, seed=24, d=8, power=0.6, T_vamp=6),
    "lattice_k1000_r": lambda: S.make_layer("lattice_k1000_r", 20, 64, seed=25, d=8, K=1000, power=0.5, r=60,
                                            T_vamp=5),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_parity(name):
    L = CASES[name]()
    rows = np.arange(L.m)
    print(f"[layer] {name} m={L.m} n={L.n} r={L.r} K={L.K} d={L.d} T={L.T_vamp}", flush=True)
    gpu = run_gpu(L)
    refs = solve_rows(L, rows)
    summ = compare_layer(L, rows, gpu, refs)
    print(f"  codes {summ['code_agreement']:.5f} rows-equal {summ['rows_codes_equal']}/{summ['n_rows']} "
          f"obj {summ['obj_rel_max']:.2e} traces {summ['trace_rel_max']}", flush=True)
    assert summ["code_agreement"] >= CODE_FRAC
    assert summ["obj_rel_max"] < OBJ_RTOL
    for key, v in summ["trace_rel_max"].items():
        assert v < SOFT_RTOL, (key, v)
    check_counts(L, gpu, refs)


def levels_layer(name, m, n, K, seed, **kw):
    """A scalar layer with a K-level Min-Max grid per row for any K in [2, 64]
    (the synthetic workloads use powers of two): levels 0..K-1, scale
    (max - min) / (K - 1), integer zero point rounded half to even."""
    L = S.make_layer(name, m, n, seed=seed, d=1, bits=4, **kw)
    W64 = np.asarray(L.W, np.float64)
    lo, hi = W64.min(1), W64.max(1)
    scale = (hi - lo) / (K - 1)
    scale = np.where(scale > 0, scale, 1.0)
    zero = np.round(-lo / scale)
    E = np.arange(K, dtype=np.float32).reshape(K, 1)
    return S.Layer(name, L.W, L.s, L.V, E, scale.astype(np.float32), (-scale * zero).astype(np.float32), 1,
                   L.T_vamp, L.n_cd, L.damping)


@pytest.mark.parametrize("K", [3, 5, 12, 33])
def test_layer_parity_levels(K):
    """Scalar grids whose level count is not a power of two: CD's argmin over
    the levels runs over K's next power of two lanes (the lanes past K carry
    no level), within a 16-lane row up to 16 levels and across rows above
    (K = 33).  n = 300 spans a full and a ragged CD tile, r < n."""
    L = levels_layer(f"levels_k{K}", 24, 300, K, seed=70 + K, power=0.6, r=260, T_vamp=5)
    rows = np.arange(L.m)
    print(f"[layer] levels K={K} m={L.m} n={L.n} r={L.r}", flush=True)
    gpu = run_gpu(L)
    refs = solve_rows(L, rows)
    summ = compare_layer(L, rows, gpu, refs)
    print(f"  codes {summ['code_agreement']:.5f} rows-equal {summ['rows_codes_equal']}/{summ['n_rows']} "
          f"obj {summ['obj_rel_max']:.2e} traces {summ['trace_rel_max']}", flush=True)
    assert int(gpu["codes"].max()) <= K - 1
    assert summ["code_agreement"] >= CODE_FRAC
    assert summ["obj_rel_max"] < OBJ_RTOL
    for key, v in summ["trace_rel_max"].items():
        assert v < SOFT_RTOL, (key, v)
    check_counts(L, gpu, refs)


def check_counts(L, gpu, refs):
    """Pass-through events and CD sweeps per row, as the oracle counts them."""
    fb = np.array([r["fallbacks"] for r in refs])
    sw = np.array([next((j + 1 for j, c in enumerate(r["cd_changes"]) if c == 0), L.n_cd) for r in refs])
    assert np.array_equal(gpu["fallbacks"], fb), (gpu["fallbacks"], fb)
    assert np.array_equal(gpu["sweeps"], sw), (gpu["sweeps"], sw)


@pytest.mark.parametrize("eps", [0.05, 0.5])
def test_safeguard_eps(eps):
    """A positive safeguard threshold widens the pass-through rule: more rows
    pass through, and the whole solve still matches the oracle run with the
    same threshold."""
    L = S.make_layer("eps", 24, 96, seed=37, d=1, bits=3, power=0.5, T_vamp=6)
    rows = np.arange(L.m)
    gpu = run_gpu(L, safeguard_eps=eps)
    refs = solve_rows(L, rows, safeguard_eps=eps)
    summ = compare_layer(L, rows, gpu, refs)
    base = solve_rows(L, rows)
    print(f"[safeguard {eps}] codes {summ['code_agreement']:.5f} obj {summ['obj_rel_max']:.2e} pass-through "
          f"{int(gpu['fallbacks'].sum())} (eps 0: {sum(r['fallbacks'] for r in base)})", flush=True)
    assert summ["code_agreement"] >= CODE_FRAC and summ["obj_rel_max"] < OBJ_RTOL
    check_counts(L, gpu, refs)
    assert gpu["fallbacks"].sum() > sum(r["fallbacks"] for r in base)


def test_linear_paths_agree_and_digits_run():
    """The int8 digit GEMM is what the default solve runs (its split kernels
    appear in the profile), the fp64-MFMA path gives way to it only on request,
    and both paths give the same codes and matching traces."""
    import torch
    import post_quantization_solver_amd as mpq
    L = S.make_layer("paths", 48, 320, seed=38, d=1, bits=4, power=0.5, T_vamp=8)
    T = layer_tensors(L)
    outs = {}
    for f64 in (False, True):
        prof = mpq.Profile(("linear1", "linear2", "split"))
        out = mpq.quantize_layer(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], T_vamp=L.T_vamp, n_cd=L.n_cd,
                                 damping=L.damping, profile=prof, linear_f64=f64)
        torch.cuda.synchronize()
        outs[f64] = ({k: host(v) for k, v in out.items() if v is not None}, prof.as_dict())
    (dg, pd), (fp, pf) = outs[False], outs[True]
    assert pd["split"][1] > 0 and pf["split"][1] == 0
    assert pd["linear1"][1] == pf["linear1"][1] == L.T_vamp
    assert np.array_equal(dg["codes"], fp["codes"])
    # beta and gamma1 follow the products directly; gamma2 = eta1 - gamma1 is
    # an ill-conditioned difference, held to the soft-quantity bar
    for k, tol in (("beta_tr", 1e-6), ("gamma1_tr", 1e-6), ("gamma2_tr", SOFT_RTOL)):
        assert np.allclose(dg[k], fp[k], rtol=tol, atol=0), k


def test_long_rows_take_fp64_products():
    """Rows longer than the digit GEMM's inner dimension (n > 32767) run the
    linear module on the fp64 matrix cores and still match the oracle."""
    L = S.make_layer("long", 3, 32776, seed=39, d=1, bits=3, power=0.5, r=24, T_vamp=3)
    rows = np.arange(L.m)
    gpu = run_gpu(L)
    refs = solve_rows(L, rows)
    summ = compare_layer(L, rows, gpu, refs)
    print(f"[long rows] codes {summ['code_agreement']:.5f} obj {summ['obj_rel_max']:.2e}", flush=True)
    assert summ["code_agreement"] >= CODE_FRAC and summ["obj_rel_max"] < OBJ_RTOL
    for key, v in summ["trace_rel_max"].items():
        assert v < SOFT_RTOL, (key, v)


def test_special_cases():
    L = S.make_layer("sp", 12, 48, seed=31, d=1, bits=3, T_vamp=4)
    rows = np.arange(L.m)
    # T_vamp = 0: RTN then CD
    g0 = run_gpu(L, T_vamp=0)
    r0 = solve_rows(L, rows, T_vamp=0)
    assert (g0["codes"] == np.stack([r["codes"] for r in r0])).mean() >= CODE_FRAC
    # n_cd = 0: MAP codes
    g1 = run_gpu(L, n_cd=0)
    r1 = solve_rows(L, rows, n_cd=0)
    assert (g1["codes"] == np.stack([r["map_codes"] for r in r1])).mean() >= CODE_FRAC
    assert g1["cd_changes"] is None
    assert np.all(g1["sweeps"] == 0)


def test_frozen_rows_and_empty():
    import torch
    import post_quantization_solver_amd as mpq
    L = S.make_layer("fz", 6, 32, seed=32, d=1, bits=3, T_vamp=4)
    W = L.W.copy()
    # row 2 exactly on a grid with an exactly representable scale and offset
    a = L.a.copy()
    o = L.o.copy()
    a[2], o[2] = 0.25, -1.0
    W[2] = (np.arange(32) % 8) * 0.25 - 1.0
    L2 = S.Layer("fz", W, L.s, L.V, L.E, a, o, 1, 4, 3, 0.5)
    g = run_gpu(L2)
    assert np.all(g["codes"][2] == np.arange(32) % 8)
    assert np.all(np.isinf(g["beta_tr"][2])) and np.all(np.isinf(g["gamma1_tr"][2]))
    assert np.all(g["cd_changes"][2] == 0)
    assert np.all(np.isfinite(g["beta_tr"][[0, 1, 3, 4, 5]]))
    ref = solve_rows(L2, [2])[0]
    assert ref["frozen"] and list(ref["codes"]) == list(g["codes"][2])
    # m = 0 is a no-op
    T = layer_tensors(L2)
    out = mpq.quantize_layer(T["W"][:0], T["s"], T["V"], L.E, T["a"][:0], T["o"][:0], T_vamp=2, n_cd=1)
    assert out["codes"].shape == (0, 32)


def test_deterministic_and_row_independent():
    L = S.make_layer("det", 16, 64, seed=33, d=8, K=4096, power=0.6, T_vamp=4)
    g1 = run_gpu(L)
    g2 = run_gpu(L)
    for k in ("codes", "beta_tr", "gamma1_tr", "gamma2_tr", "cd_changes"):
        assert np.array_equal(g1[k], g2[k]), k
    # solving a permuted batch permutes the outputs bitwise
    perm = np.random.default_rng(0).permutation(L.m)
    Lp = S.Layer("perm", L.W[perm], L.s, L.V, L.E, L.a[perm], L.o[perm], L.d, L.T_vamp, L.n_cd, L.damping)
    gp = run_gpu(Lp)
    for k in ("codes", "beta_tr", "gamma1_tr"):
        assert np.array_equal(gp[k], g1[k][perm]), k


def test_scale_metamorphic():
    """W and codebook scale x4: identical codes; beta and gamma scale by 1/16."""
    L = S.make_layer("scl", 16, 96, seed=34, d=1, bits=3, T_vamp=6)
    Ls = S.Layer("scl4", L.W * 4, L.s, L.V, L.E, L.a * 4, L.o * 4, 1, 6, 3, 0.5)
    g = run_gpu(L)
    gs = run_gpu(Ls)
    assert np.array_equal(g["codes"], gs["codes"])
    assert np.allclose(gs["beta_tr"], g["beta_tr"] / 16, rtol=1e-5)
    assert np.allclose(gs["gamma1_tr"], g["gamma1_tr"] / 16, rtol=1e-5)


def test_halves_equal_full_solve():
    """Rows are independent problems: solving each half of a 1024-row layer
    alone gives bitwise the rows of the whole layer, for the lattice and the
    scalar CD (the row-compacted gradient updates and the per-row moves see
    different row counts)."""
    for d, extra in ((8, dict(K=1000, r=60)), (1, dict(bits=3))):
        L = S.make_layer("grp", 1024, 64, seed=35, d=d, power=0.6, T_vamp=3, **extra)
        full = run_gpu(L)
        for lo, hi in ((0, 512), (512, 1024)):
            Lh = S.Layer("half", np.ascontiguousarray(L.W[lo:hi]), L.s, L.V, L.E, L.a[lo:hi], L.o[lo:hi], L.d,
                         L.T_vamp, L.n_cd, L.damping)
            part = run_gpu(Lh)
            for k in ("codes", "cd_changes", "beta_tr", "gamma1_tr"):
                assert np.array_equal(part[k], full[k][lo:hi]), (d, lo, k)
        assert full["cd_changes"].sum() > 0


def test_sampled_profile_counts_every_launch():
    """With MPQ_F_PROFILE_SAMPLED the CD scoring category times one launch in
    32 but reports every launch, and its milliseconds scale to all of them;
    the codes do not depend on profiling."""
    import torch
    import post_quantization_solver_amd as mpq
    L = S.make_layer("prof", 1024, 128, seed=36, d=8, K=1000, r=96, power=0.6, T_vamp=2)
    T = layer_tensors(L)
    runs = {}
    for sampled in (False, True):
        prof = mpq.Profile(("cd_score",), sampled=sampled)
        out = mpq.quantize_layer(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], T_vamp=L.T_vamp, n_cd=L.n_cd,
                                 damping=L.damping, profile=prof)
        torch.cuda.synchronize()
        runs[sampled] = (prof.as_dict()["cd_score"], host(out["codes"]))
    (ms_full, n_full), codes_full = runs[False]
    (ms_s, n_s), codes_s = runs[True]
    # 16 blocks x n_cd sweeps
    assert n_full == n_s == (128 // 8) * L.n_cd
    assert ms_full > 0 and 0.2 < ms_s / ms_full < 5.0
    assert np.array_equal(codes_full, codes_s)
