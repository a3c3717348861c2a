"""The allocation-free entry point (mpq_quantize_layer_static, through the C
ABI) against mpq_quantize_layer with a caller workspace: two calls in a row,
the second on a smaller layer (the static array keeps the first call's
contents), each bitwise equal to the regular entry point; a layer whose
workspace exceeds the static array is rejected."""
import numpy as np
import pytest

import mpq_synth as S
from parity_helpers import host, layer_tensors

pytestmark = pytest.mark.gpu

KEYS = ("codes", "beta_tr", "gamma1_tr", "gamma2_tr", "cd_changes")


def solve_both(L):
    import torch
    import post_quantization_solver_amd as mpq
    T = layer_tensors(L)
    cb = mpq.prepare_codebook(L.E)
    kw = dict(T_vamp=L.T_vamp, n_cd=L.n_cd, damping=L.damping)
    ref = mpq.quantize_layer(T["W"], T["s"], T["V"], cb, T["a"], T["o"], **kw)
    got = mpq.quantize_layer_static(T["W"], T["s"], T["V"], cb, T["a"], T["o"], **kw)
    torch.cuda.synchronize()
    return {k: host(ref[k]) for k in KEYS}, {k: host(got[k]) for k in KEYS}


@pytest.mark.parametrize("d", [1, 8])
def test_static_workspace_matches_caller_workspace(d):
    import post_quantization_solver_amd as mpq
    if d == 1:
        big = S.make_layer("st_big", 96, 384, seed=51, d=1, bits=4, power=0.5, T_vamp=6)
        small = S.make_layer("st_small", 24, 136, seed=52, d=1, bits=3, power=0.6, r=100, T_vamp=4)
    else:
        big = S.make_layer("st_big8", 64, 256, seed=53, d=8, K=4096, power=0.6, T_vamp=5)
        small = S.make_layer("st_small8", 16, 64, seed=54, d=8, K=1000, power=0.5, r=60, T_vamp=3)
    for L in (big, small):   # the second call is smaller and finds the first call's data in the array
        assert mpq.workspace_bytes(L.m, L.n, L.r, L.K, L.d) <= mpq.binding.STATIC_WORKSPACE_BYTES
        ref, got = solve_both(L)
        print(f"[static] {L.name} m={L.m} n={L.n} K={L.K}: codes equal {np.mean(ref['codes'] == got['codes']):.4f}",
              flush=True)
        for k in KEYS:
            assert np.array_equal(ref[k], got[k]), (L.name, k)


def test_static_workspace_rejects_large_layers():
    import post_quantization_solver_amd as mpq
    L = S.make_layer("st_large", 1024, 1024, seed=55, d=1, bits=4, power=0.5, T_vamp=2)
    assert mpq.workspace_bytes(L.m, L.n, L.r, L.K, L.d) > mpq.binding.STATIC_WORKSPACE_BYTES
    T = layer_tensors(L)
    with pytest.raises(mpq.MPQError) as e:
        mpq.quantize_layer_static(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], T_vamp=2, n_cd=1)
    assert e.value.status == -5
