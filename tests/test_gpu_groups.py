"""Parity of group-wise scalar grids (one codebook affine per group of g
consecutive columns; the hyper-parameter paragraph's scalar runs use g = 128)
against the oracle's grouped codebook: every stage teacher-forced, then the
whole layer end to end.

Cases: n = 384 with g = 128 (a 256-column CD tile spans two groups) and a
ragged n = 200 with g = 48 (a shorter last group, every CD tile boundary
inside a group).  Tolerances as for per-row grids: soft quantities 1e-4
relative, codes >= 99.9 % of blocks, objectives 1e-5 relative.
"""
import numpy as np
import pytest

import mpq_synth as S
from oracle import mpq_oracle as O
from oracle.pool import solve_rows
from parity_helpers import SOFT_RTOL, OBJ_RTOL, CODE_FRAC, dev, host, layer_tensors, rel_vec, rel_scalar, \
    compare_layer, row_codebook

pytestmark = pytest.mark.gpu

CASES = {
    "g128_3bit": lambda: S.make_layer("grp3", 24, 384, seed=51, d=1, bits=3, power=0.5, T_vamp=4, group=128),
    "g48_ragged_4bit": lambda: S.make_layer("grp_ragged", 21, 200, seed=52, d=1, bits=4, power=0.6, r=150,
                                            T_vamp=4, group=48),
}
NAMES = list(CASES)
_CACHE = {}


def oracle_runs(name):
    if name not in _CACHE:
        L = CASES[name]()
        rows = np.arange(L.m)
        _CACHE[name] = (L, rows, solve_rows(L, rows, record=True))
    return _CACHE[name]


@pytest.mark.parametrize("name", NAMES)
def test_grouped_prologue(name):
    import post_quantization_solver_amd as mpq
    L, rows, refs = oracle_runs(name)
    T = layer_tensors(L)
    print(f"[group prologue] {name} m={L.m} n={L.n} g={L.group} G={L.a.shape[1]}", flush=True)
    out = mpq.prologue(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], group=L.group)
    rtn, g1, b0 = host(out["rtn_codes"]), host(out["gamma1"]), host(out["beta"])
    agree = float(np.mean([np.mean(rtn[i] == refs[k]["rtn_codes"]) for k, i in enumerate(rows)]))
    wg = max(rel_scalar(g1[i], refs[k]["gamma1_tr"][0]) for k, i in enumerate(rows))
    wb = max(rel_scalar(b0[i], refs[k]["beta_tr"][0]) for k, i in enumerate(rows))
    print(f"  rtn agree {agree:.5f} gamma1 {wg:.2e} beta {wb:.2e}", flush=True)
    assert agree >= CODE_FRAC
    assert wg < SOFT_RTOL and wb < SOFT_RTOL


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("t", [0, 3])
def test_grouped_denoise(name, t):
    import post_quantization_solver_amd as mpq
    L, rows, refs = oracle_runs(name)
    T = layer_tensors(L)
    R1 = np.stack([r["history"][t]["r1"] for r in refs])
    g1 = np.array([r["history"][t]["gamma1"] for r in refs])
    print(f"[group denoise] {name} t={t}", flush=True)
    xh, vt = mpq.denoise(dev(R1), dev(g1), L.E, T["a"], T["o"], group=L.group)
    xh, vt = host(xh), host(vt)
    wx, wv = 0.0, 0.0
    for k, i in enumerate(rows):
        xr, vr, _ = O.denoise(R1[k], float(g1[k]), row_codebook(L, i), L.d)
        wx = max(wx, rel_vec(xh[k], xr))
        wv = max(wv, rel_scalar(vt[k].sum(), vr.sum()))
    print(f"  xhat1 {wx:.2e}  sum v {wv:.2e}", flush=True)
    assert wx < SOFT_RTOL and wv < SOFT_RTOL


@pytest.mark.parametrize("name", NAMES)
def test_grouped_vamp_step(name):
    import post_quantization_solver_amd as mpq
    L, rows, refs = oracle_runs(name)
    T = layer_tensors(L)
    worst = {}
    for t in range(L.T_vamp):
        h = [r["history"][t] for r in refs]
        R1 = dev(np.stack([x["r1"] for x in h]))
        g1 = dev(np.array([x["gamma1"] for x in h]))
        bt = dev(np.array([x["beta"] for x in h]))
        print(f"[group vamp_step] {name} t={t}", flush=True)
        out = mpq.vamp_step(R1, g1, bt, T["W"], T["s"], T["V"], L.E, T["a"], T["o"], damping=L.damping,
                            group=L.group)
        r1n, g1n, btn = host(R1), host(g1), host(bt)
        xh, eta1, g2, fb = (host(out[k]) for k in ("xhat1", "eta1", "gamma2", "fallback"))
        for k in range(len(rows)):
            nxt = refs[k]["history"][t + 1]["r1"] if t + 1 < L.T_vamp else refs[k]["r1_final"]
            g1_ref = refs[k]["gamma1_tr"][t + 1]
            e = dict(xhat1=rel_vec(xh[k], h[k]["xhat1"]), eta1=rel_scalar(eta1[k], h[k]["eta1"]),
                     gamma2=rel_scalar(g2[k], h[k]["gamma2"]), r1=rel_vec(r1n[k], nxt),
                     gamma1=rel_scalar(g1n[k], g1_ref), beta=rel_scalar(btn[k], refs[k]["beta_tr"][t + 1]),
                     fallback=float(bool(fb[k]) != bool(h[k]["fell_back"])))
            for key, v in e.items():
                worst[key] = max(worst.get(key, 0.0), v)
    print("  worst:", {k: f"{v:.2e}" for k, v in worst.items()}, flush=True)
    assert worst["fallback"] == 0.0
    for key in ("xhat1", "eta1", "gamma2", "r1", "gamma1", "beta"):
        assert worst[key] < SOFT_RTOL, (key, worst[key])


@pytest.mark.parametrize("name", NAMES)
def test_grouped_map_and_cd(name):
    import torch
    import post_quantization_solver_amd as mpq
    L, rows, refs = oracle_runs(name)
    T = layer_tensors(L)
    R1 = np.stack([r["r1_final"] for r in refs])
    g1 = np.array([r["gamma1_tr"][-1] for r in refs])
    mc = host(mpq.map_codes(dev(R1), dev(g1), L.E, T["a"], T["o"], group=L.group))
    ref = np.stack([O.map_codes(R1[k], float(g1[k]), row_codebook(L, i), L.d)
                    for k, i in enumerate(rows)])
    map_agree = float((mc == ref).mean())
    start = dev(np.stack([r["map_codes"] for r in refs]).astype(np.int32))
    codes, ch = mpq.cd(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], start, n_cd=L.n_cd, group=L.group)
    torch.cuda.synchronize()
    codes = host(codes)
    cd_ref = np.stack([r["codes"] for r in refs])
    cd_agree = float((codes == cd_ref).mean())
    f_gpu = np.array([O.codes_objective(L.W[i], codes[k], row_codebook(L, i), L.d, L.s, L.V)
                      for k, i in enumerate(rows)])
    f_ref = np.array([r["objective"] for r in refs])
    obj = float(np.max(np.abs(f_gpu - f_ref) / f_ref))
    print(f"[group map/cd] {name} map {map_agree:.5f} cd {cd_agree:.5f} objective {obj:.2e} "
          f"changes gpu {host(ch).sum(0)} ref {np.array([r['cd_changes'] for r in refs]).sum(0)}", flush=True)
    assert map_agree >= CODE_FRAC
    assert cd_agree >= CODE_FRAC
    assert obj < OBJ_RTOL


@pytest.mark.parametrize("name", NAMES)
def test_grouped_layer(name):
    import torch
    import post_quantization_solver_amd as mpq
    L, rows, refs = oracle_runs(name)
    T = layer_tensors(L)
    out = mpq.quantize_layer(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], T_vamp=L.T_vamp, n_cd=L.n_cd,
                             damping=L.damping, group=L.group)
    torch.cuda.synchronize()
    gpu = {k: (host(v) if v is not None else None) for k, v in out.items()}
    summ = compare_layer(L, rows, gpu, refs)
    print(f"[group layer] {name}: codes {summ['code_agreement']:.5f} obj {summ['obj_rel_max']:.2e} "
          f"traces {summ['trace_rel_max']}", flush=True)
    assert summ["code_agreement"] >= CODE_FRAC
    assert summ["obj_rel_max"] < OBJ_RTOL
    for key, v in summ["trace_rel_max"].items():
        assert v < SOFT_RTOL, (key, v)


def test_group_of_whole_row_is_per_row():
    """group >= n is one affine per row: bitwise the per-row solve."""
    import torch
    import post_quantization_solver_amd as mpq
    L = S.make_layer("grp_whole", 16, 96, seed=53, d=1, bits=3, power=0.5, T_vamp=3)
    T = layer_tensors(L)
    a = [mpq.quantize_layer(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], T_vamp=L.T_vamp, n_cd=L.n_cd,
                            damping=L.damping, group=g) for g in (None, 96, 1000)]
    torch.cuda.synchronize()
    for out in a[1:]:
        for key in ("codes", "beta_tr", "gamma1_tr", "gamma2_tr", "cd_changes"):
            assert torch.equal(out[key], a[0][key]), key
