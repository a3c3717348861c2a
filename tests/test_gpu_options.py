"""Boundary options and the asynchrony contract of the C ABI on the GPU: the
log-prior hook against the oracle, the finiteness check, and a solve call
that returns while earlier work on its stream is still running."""
import numpy as np
import pytest

import mpq_synth as S
from oracle.pool import solve_rows
from parity_helpers import SOFT_RTOL, OBJ_RTOL, CODE_FRAC, dev, host, layer_tensors, compare_layer

pytestmark = pytest.mark.gpu


def test_log_prior_matches_oracle():
    """A per-level log-prior (key design 1's rho(c)) in the denoiser and the
    marginal MAP: the whole solve against the oracle with the same prior."""
    import torch
    import post_quantization_solver_amd as mpq
    L = S.make_layer("lp", 32, 160, seed=61, d=1, bits=3, power=0.5, T_vamp=6)
    lp = np.random.default_rng(61).normal(0.0, 1.5, L.K).astype(np.float32)
    T = layer_tensors(L)
    out = mpq.quantize_layer(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], T_vamp=L.T_vamp, n_cd=L.n_cd,
                             damping=L.damping, log_prior=dev(lp), diagnostics=True)
    plain = mpq.quantize_layer(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], T_vamp=L.T_vamp, n_cd=L.n_cd,
                               damping=L.damping)
    torch.cuda.synchronize()
    gpu = {k: (host(v) if v is not None else None) for k, v in out.items()}
    rows = np.arange(L.m)
    refs = solve_rows(L, rows, log_prior=lp.astype(np.float64))
    summ = compare_layer(L, rows, gpu, refs)
    print(f"[log prior] codes {summ['code_agreement']:.5f} obj {summ['obj_rel_max']:.2e} "
          f"traces {summ['trace_rel_max']}", flush=True)
    assert summ["code_agreement"] >= CODE_FRAC and summ["obj_rel_max"] < OBJ_RTOL
    for key, v in summ["trace_rel_max"].items():
        assert v < SOFT_RTOL, (key, v)
    map_ref = np.stack([r["map_codes"] for r in refs])
    assert (gpu["map_codes"] == map_ref).mean() >= CODE_FRAC
    assert not np.array_equal(host(plain["gamma1_tr"]), gpu["gamma1_tr"])   # the prior changes the solve


def test_log_prior_needs_scalar_grids():
    import post_quantization_solver_amd as mpq
    L = S.make_layer("lp8", 8, 64, seed=62, d=8, K=1000, power=0.5, r=60, T_vamp=2)
    T = layer_tensors(L)
    with pytest.raises(mpq.MPQError) as e:
        mpq.quantize_layer(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], T_vamp=2, n_cd=1,
                           log_prior=dev(np.zeros(L.K, np.float32)))
    assert e.value.status == -4


def test_check_finite():
    """MPQ_F_CHECK_FINITE: a NaN or infinite input, or a row scale <= 0, gives
    MPQ_ENONFINITE before anything else runs; clean inputs solve as usual."""
    import torch
    import post_quantization_solver_amd as mpq
    L = S.make_layer("fin", 16, 64, seed=63, d=1, bits=3, power=0.5, T_vamp=3)
    T = layer_tensors(L)
    cb = mpq.prepare_codebook(L.E)
    kw = dict(T_vamp=L.T_vamp, n_cd=L.n_cd, damping=L.damping)
    ok = mpq.quantize_layer(T["W"], T["s"], T["V"], cb, T["a"], T["o"], check_finite=True, **kw)
    ref = mpq.quantize_layer(T["W"], T["s"], T["V"], cb, T["a"], T["o"], **kw)
    torch.cuda.synchronize()
    assert np.array_equal(host(ok["codes"]), host(ref["codes"]))
    for name, bad in (("W", float("nan")), ("V", float("inf")), ("s", float("-inf")), ("a", 0.0), ("o", float("nan"))):
        B = {k: v.clone() for k, v in T.items()}
        B[name].view(-1)[3] = bad
        codes = torch.full((L.m, L.n), -7, dtype=torch.int32, device="cuda")
        with pytest.raises(mpq.MPQError) as e:
            mpq.quantize_layer(B["W"], B["s"], B["V"], cb, B["a"], B["o"], check_finite=True,
                               outputs=dict(codes=codes, beta_tr=None, gamma1_tr=None, gamma2_tr=None,
                                            cd_changes=None), **kw)
        assert e.value.status == -8, name
        torch.cuda.synchronize()
        assert int((codes != -7).sum()) == 0, name   # nothing else ran


def test_call_returns_before_queued_work_ends():
    """mpq_quantize_layer only enqueues: called behind a long kernel on the
    same stream it returns while that kernel still runs, and its results are
    those of a call on an idle stream."""
    import torch
    import post_quantization_solver_amd as mpq
    L = S.make_layer("async", 64, 256, seed=64, d=8, K=4096, power=0.6, T_vamp=4)
    T = layer_tensors(L)
    cb = mpq.prepare_codebook(L.E)
    ws = torch.empty(mpq.workspace_bytes(L.m, L.n, L.r, L.K, L.d), dtype=torch.uint8, device="cuda")
    kw = dict(T_vamp=L.T_vamp, n_cd=L.n_cd, damping=L.damping, workspace=ws)
    ref = mpq.quantize_layer(T["W"], T["s"], T["V"], cb, T["a"], T["o"], **kw)
    ref_codes = host(ref["codes"])
    torch.cuda.synchronize()
    done = torch.cuda.Event()
    torch.cuda._sleep(int(3e9))          # about a second of GPU time on this stream
    done.record()
    out = mpq.quantize_layer(T["W"], T["s"], T["V"], cb, T["a"], T["o"], **kw)
    still_running = not done.query()     # the sleep has not finished, so the call did not wait
    torch.cuda.synchronize()
    print(f"[async] sleep still running when the call returned: {still_running}", flush=True)
    assert still_running
    assert np.array_equal(host(out["codes"]), ref_codes)
