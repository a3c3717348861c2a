"""Parity on the five named workloads at full size (n, r, K as benchmarked).

The GPU solves the whole layer in the configuration bench.py times; the
float64 oracle solves a fixed sample of rows (every m/k-th row), which is an
exact comparison because rows are independent problems.  Each stage is also
run teacher-forced: the GPU stage starts from the oracle's own state on the
sampled rows, so a stage's error is measured without the error the stages
before it carried in.

Bars (per sampled row): soft quantities 1e-4 relative (gamma2 and r2 relative
to the operands of gamma2 = eta1 - gamma1); MAP and CD codes >= 99.9 % of
blocks and CD objectives within 1e-5 relative when started from the same
state; end-to-end traces within 1e-4.  End-to-end codes are reported with the
number of rows whose MAP start differs only through the float32 trajectory.
"""
import numpy as np
import pytest

import mpq_synth as S
from oracle import mpq_oracle as O
from oracle.pool import solve_rows
from parity_helpers import (SOFT_RTOL, OBJ_RTOL, CODE_FRAC, dev, host, layer_tensors, compare_layer, rel_vec,
                            rel_scalar)

pytestmark = pytest.mark.gpu

SAMPLE = {"c1": 64, "c2": 16, "c3": 16, "c4": 8, "c5": 4}


def sublayer(L, rows):
    return S.Layer(L.name + "_rows", np.ascontiguousarray(L.W[rows]), L.s, L.V, L.E, L.a[rows], L.o[rows], L.d,
                   L.T_vamp, L.n_cd, L.damping)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_config_parity(name):
    import torch
    import post_quantization_solver_amd as mpq
    print(f"[config] {name}: generating inputs", flush=True)
    L = S.make_config(name, device="cuda")
    T = layer_tensors(L)
    print(f"[config] {name}: m={L.m} n={L.n} r={L.r} K={L.K} d={L.d} T={L.T_vamp} full solve on GPU", flush=True)
    out = mpq.quantize_layer(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], T_vamp=L.T_vamp, n_cd=L.n_cd,
                             damping=L.damping)
    torch.cuda.synchronize()
    gpu = {k: (host(v) if v is not None else None) for k, v in out.items()}
    del T, out
    torch.cuda.empty_cache()
    rows = S.parity_rows(L.m, SAMPLE[name])
    print(f"[config] {name}: oracle on {len(rows)} rows", flush=True)
    refs = solve_rows(L, rows, record=True)
    Ls = sublayer(L, rows)
    Ts = layer_tensors(Ls)
    k_rows = len(rows)
    report = {}

    # (1) end-to-end traces
    summ = compare_layer(L, rows, gpu, refs)
    report["e2e_traces"] = summ["trace_rel_max"]

    # (2) teacher-forced VAMP steps at three iterations
    ytil = dev(np.stack([O.rank_target(Ls.W[k], Ls.s, Ls.V) for k in range(k_rows)]).astype(np.float32))
    worst = {}
    for t in sorted({0, L.T_vamp // 2, L.T_vamp - 1}):
        h = [r["history"][t] for r in refs]
        R1 = dev(np.stack([x["r1"] for x in h]).astype(np.float32))
        g1 = dev(np.array([x["gamma1"] for x in h], dtype=np.float32))
        bt = dev(np.array([x["beta"] for x in h], dtype=np.float32))
        o = mpq.vamp_step(R1, g1, bt, ytil, Ts["s"], Ts["V"], L.E, Ts["a"], Ts["o"], damping=L.damping)
        r1n, g1n, btn = host(R1), host(g1), host(bt)
        for k in range(k_rows):
            nxt = refs[k]["history"][t + 1]["r1"] if t + 1 < L.T_vamp else refs[k]["r1_final"]
            cond = max(1.0, h[k]["eta1"] / h[k]["gamma2"])
            e = dict(xhat1=rel_vec(host(o["xhat1"])[k], h[k]["xhat1"]),
                     eta1=rel_scalar(host(o["eta1"])[k], h[k]["eta1"]),
                     gamma2=rel_scalar(host(o["gamma2"])[k], h[k]["gamma2"]) / cond,
                     r2=rel_vec(host(o["r2"])[k], h[k]["r2"]) / cond,
                     r1=rel_vec(r1n[k], nxt), gamma1=rel_scalar(g1n[k], refs[k]["gamma1_tr"][t + 1]),
                     beta=rel_scalar(btn[k], refs[k]["beta_tr"][t + 1]),
                     fallback=float(bool(host(o["fallback"])[k]) != bool(h[k]["fell_back"])))
            for key, v in e.items():
                worst[key] = max(worst.get(key, 0.0), v)
    report["step"] = worst

    # (3) MAP at the oracle's final state
    R1f = np.stack([r["r1_final"] for r in refs]).astype(np.float32)
    g1f = np.array([r["gamma1_tr"][-1] for r in refs], dtype=np.float32)
    map_gpu = host(mpq.map_codes(dev(R1f), dev(g1f), L.E, Ts["a"], Ts["o"]))
    map_ref = np.stack([r["map_codes"] for r in refs])
    report["map_agree"] = float((map_gpu == map_ref).mean())

    # (4) CD from the oracle's MAP codes
    codes_cd, _ = mpq.cd(Ts["W"], Ts["s"], Ts["V"], L.E, Ts["a"], Ts["o"], dev(map_ref.astype(np.int32)),
                         n_cd=L.n_cd)
    torch.cuda.synchronize()
    codes_cd = host(codes_cd)
    cd_ref = np.stack([r["codes"] for r in refs])
    report["cd_agree"] = float((codes_cd == cd_ref).mean())
    f_cd = np.array([O.codes_objective(Ls.W[k], codes_cd[k], O.row_codewords(L.E, Ls.a[k], Ls.o[k]), L.d, L.s, L.V)
                     for k in range(k_rows)])
    f_ref = np.array([r["objective"] for r in refs])
    report["cd_obj_rel"] = float(np.max(np.abs(f_cd - f_ref) / f_ref))

    # (5) end to end; rows whose GPU MAP start differs from the oracle's
    e2e_rows_diff = int((~(gpu["codes"][rows] == cd_ref).all(1)).sum())
    report["e2e_code_agree"] = summ["code_agreement"]
    report["e2e_obj_rel_max"] = summ["obj_rel_max"]
    report["e2e_obj_rel_mean"] = float(np.mean(summ["obj_rel"]))
    report["e2e_rows_differing"] = f"{e2e_rows_diff}/{k_rows}"
    report["fallbacks"] = int(sum(r["fallbacks"] for r in refs))
    print(f"  {name}: " + ", ".join(f"{k}={v}" for k, v in report.items()), flush=True)

    for key in ("xhat1", "eta1", "gamma2", "r2", "r1", "gamma1", "beta"):
        assert worst[key] < SOFT_RTOL, ("teacher-forced step", key, worst[key])
    assert worst["fallback"] == 0.0
    assert report["map_agree"] >= CODE_FRAC
    assert report["cd_agree"] >= CODE_FRAC
    assert report["cd_obj_rel"] < OBJ_RTOL
    for key, v in summ["trace_rel_max"].items():
        assert v < SOFT_RTOL, ("end-to-end trace", key, v)
