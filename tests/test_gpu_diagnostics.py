"""Parity of the diagnostics and the comparator used by the ablation grid:

  * mpq_objective (float64 layer objective of given codes) against the
    oracle's objective (1e-5 relative; the GPU forms diag(s) V^T once in
    float32, so ~1e-7 is expected);
  * the optional map_codes / objective outputs of mpq_quantize_layer;
  * mpq_greedy (the sequential greedy comparator, reading G3) against the
    oracle's Schur-complement definition: codes >= 99.9 % of blocks,
    objectives 1e-5 relative; and CD started from the greedy codes.
"""
import numpy as np
import pytest

import mpq_synth as S
from oracle import mpq_oracle as O
from oracle.pool import solve_rows, greedy_rows, cd_rows
from parity_helpers import OBJ_RTOL, CODE_FRAC, dev, host, layer_tensors, row_codebook

pytestmark = pytest.mark.gpu

CASES = {
    "scalar3_2tiles": lambda: S.make_layer("dg_s3", 20, 384, seed=61, d=1, bits=3, power=0.5, T_vamp=4),
    "ragged4_lowrank": lambda: S.make_layer("dg_r4", 17, 200, seed=62, d=1, bits=4, power=0.6, r=150, T_vamp=4),
    "grouped_g48": lambda: S.make_layer("dg_g", 15, 200, seed=63, d=1, bits=3, power=0.5, T_vamp=4, group=48),
    "lattice_k1000_2tiles": lambda: S.make_layer("dg_l", 12, 512, seed=64, d=8, K=1000, power=0.6, r=400,
                                                 T_vamp=3),
    "lattice_full": lambda: S.make_layer("dg_lf", 8, 64, seed=65, d=8, power=0.6, T_vamp=3),
}
NAMES = list(CASES)
_CACHE = {}


def layer(name):
    if name not in _CACHE:
        _CACHE[name] = CASES[name]()
    return _CACHE[name]


@pytest.mark.parametrize("name", NAMES)
def test_objective(name):
    import torch
    import post_quantization_solver_amd as mpq
    L = layer(name)
    T = layer_tensors(L)
    rng = np.random.default_rng(7)
    codes = rng.integers(0, L.K, size=(L.m, L.n // L.d)).astype(np.int32)
    f = host(mpq.objective(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], dev(codes), group=L.group))
    ref = np.array([O.codes_objective(L.W[i], codes[i], row_codebook(L, i), L.d, L.s, L.V) for i in range(L.m)])
    rel = float(np.max(np.abs(f - ref) / ref))
    print(f"[objective] {name}: max rel {rel:.2e}", flush=True)
    assert rel < OBJ_RTOL
    # a code outside [0, K) poisons its own row only
    bad = codes.copy()
    bad[1, 0] = L.K
    f2 = host(mpq.objective(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], dev(bad), group=L.group))
    torch.cuda.synchronize()
    assert np.isnan(f2[1]) and np.array_equal(np.delete(f2, 1), np.delete(f, 1))


@pytest.mark.parametrize("name", ["scalar3_2tiles", "grouped_g48", "lattice_k1000_2tiles"])
def test_layer_diagnostic_outputs(name):
    import torch
    import post_quantization_solver_amd as mpq
    L = layer(name)
    T = layer_tensors(L)
    out = mpq.quantize_layer(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], T_vamp=L.T_vamp, n_cd=L.n_cd,
                             damping=L.damping, group=L.group, diagnostics=True)
    f_again = mpq.objective(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], out["codes"], group=L.group)
    torch.cuda.synchronize()
    assert torch.equal(out["objective"], f_again)
    refs = solve_rows(L, np.arange(L.m))
    mc = host(out["map_codes"])
    agree = float(np.mean([np.mean(mc[i] == r["map_codes"]) for i, r in enumerate(refs)]))
    f = host(out["objective"])
    rel = float(np.max([abs(f[i] - r["objective"]) / r["objective"] for i, r in enumerate(refs)]))
    print(f"[diagnostics] {name}: map codes {agree:.5f}, objective vs oracle {rel:.2e}", flush=True)
    assert agree >= CODE_FRAC
    assert rel < OBJ_RTOL
    # without the outputs requested the solve is the same
    plain = mpq.quantize_layer(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], T_vamp=L.T_vamp, n_cd=L.n_cd,
                               damping=L.damping, group=L.group)
    torch.cuda.synchronize()
    assert torch.equal(plain["codes"], out["codes"])


@pytest.mark.parametrize("name", NAMES)
def test_greedy(name):
    import torch
    import post_quantization_solver_amd as mpq
    L = layer(name)
    T = layer_tensors(L)
    print(f"[greedy] {name}: m={L.m} n={L.n} r={L.r} K={L.K} d={L.d} g={L.group}", flush=True)
    codes = mpq.greedy(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], group=L.group)
    torch.cuda.synchronize()
    codes = host(codes)
    rows = np.arange(L.m)
    refs = greedy_rows(L, rows)
    agree = float(np.mean([np.mean(codes[i] == r["codes"]) for i, r in enumerate(refs)]))
    f_gpu = np.array([O.codes_objective(L.W[i], codes[i], row_codebook(L, i), L.d, L.s, L.V) for i in rows])
    f_ref = np.array([r["objective"] for r in refs])
    rel = float(np.max(np.abs(f_gpu - f_ref) / f_ref))
    print(f"  codes {agree:.5f} objective {rel:.2e} (greedy / RTN objective "
          f"{np.mean(f_ref) / np.mean([O.codes_objective(L.W[i], O.nearest_codeword(L.W[i], row_codebook(L, i), L.d), row_codebook(L, i), L.d, L.s, L.V) for i in rows]):.3f})",
          flush=True)
    assert agree >= CODE_FRAC
    assert rel < OBJ_RTOL
    # repeatable
    again = host(mpq.greedy(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], group=L.group))
    assert np.array_equal(again, codes)
    # CD from the greedy start (the greedy + CD cells of the ablation)
    cdc, _ = mpq.cd(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], dev(codes), n_cd=L.n_cd, group=L.group)
    torch.cuda.synchronize()
    cdc = host(cdc)
    cref = cd_rows(L, rows, codes)
    cd_agree = float(np.mean([np.mean(cdc[i] == r["codes"]) for i, r in enumerate(cref)]))
    cd_rel = float(np.max([abs(O.codes_objective(L.W[i], cdc[i], row_codebook(L, i), L.d, L.s, L.V) -
                               r["objective"]) / r["objective"] for i, r in enumerate(cref)]))
    print(f"  greedy + CD: codes {cd_agree:.5f} objective {cd_rel:.2e}", flush=True)
    assert cd_agree >= CODE_FRAC
    assert cd_rel < OBJ_RTOL


def test_greedy_degenerate_operator():
    """s = 0 (H = 0): the damping alone remains and the greedy rounds to nearest."""
    import torch
    import post_quantization_solver_amd as mpq
    L = S.make_layer("dg_zero", 6, 96, seed=66, d=1, bits=3, T_vamp=2)
    T = layer_tensors(L)
    codes = host(mpq.greedy(T["W"], torch.zeros_like(T["s"]), T["V"], L.E, T["a"], T["o"]))
    rtn = np.stack([O.nearest_codeword(L.W[i], row_codebook(L, i), 1) for i in range(L.m)])
    assert np.array_equal(codes, rtn)
