"""Parity of the anchored codebook prior (anchor scale tau; the hyper-parameter
paragraph's default tau = 0.2) against the oracle's explicit per-codeword
log-prior: teacher-forced VAMP steps and end-to-end layers.

Tolerances as for the uniform prior: soft quantities 1e-4 relative, codes
>= 99.9 % of blocks, objectives 1e-5 relative.
"""
import numpy as np
import pytest

import mpq_synth as S
from oracle import mpq_oracle as O
from oracle.pool import solve_rows
from parity_helpers import SOFT_RTOL, OBJ_RTOL, CODE_FRAC, dev, host, layer_tensors, rel_vec, rel_scalar, \
    compare_layer

pytestmark = pytest.mark.gpu

TAU = 0.2

CASES = {
    "scalar3": lambda: S.make_layer("anc_scalar", 24, 96, seed=41, d=1, bits=3, power=0.5, T_vamp=4),
    "lattice_k1000": lambda: S.make_layer("anc_lattice", 16, 64, seed=42, d=8, K=1000, power=0.5, r=60,
                                          T_vamp=4),
}


@pytest.mark.parametrize("name", list(CASES))
def test_anchored_vamp_step(name):
    import post_quantization_solver_amd as mpq
    L = CASES[name]()
    rows = np.arange(L.m)
    refs = solve_rows(L, rows, record=True, anchor_tau=TAU)
    T = layer_tensors(L)
    worst = {}
    for t in range(L.T_vamp):
        h = [r["history"][t] for r in refs]
        R1 = dev(np.stack([x["r1"] for x in h]))
        g1 = dev(np.array([x["gamma1"] for x in h]))
        bt = dev(np.array([x["beta"] for x in h]))
        print(f"[anchor step] {name} t={t}", flush=True)
        out = mpq.vamp_step(R1, g1, bt, T["W"], T["s"], T["V"], L.E, T["a"], T["o"], damping=L.damping,
                            anchor_tau=TAU)
        r1n, g1n = host(R1), host(g1)
        xh, eta1, g2, fb = (host(out[k]) for k in ("xhat1", "eta1", "gamma2", "fallback"))
        for k in range(len(rows)):
            nxt = refs[k]["history"][t + 1]["r1"] if t + 1 < L.T_vamp else refs[k]["r1_final"]
            g1_ref = refs[k]["gamma1_tr"][t + 1]
            e = dict(xhat1=rel_vec(xh[k], h[k]["xhat1"]), eta1=rel_scalar(eta1[k], h[k]["eta1"]),
                     gamma2=rel_scalar(g2[k], h[k]["gamma2"]), r1=rel_vec(r1n[k], nxt),
                     gamma1=rel_scalar(g1n[k], g1_ref), fallback=float(bool(fb[k]) != bool(h[k]["fell_back"])))
            for key, v in e.items():
                worst[key] = max(worst.get(key, 0.0), v)
    print("  worst:", {k: f"{v:.2e}" for k, v in worst.items()}, flush=True)
    assert worst["fallback"] == 0.0
    for key in ("xhat1", "eta1", "gamma2", "r1", "gamma1"):
        assert worst[key] < SOFT_RTOL, (key, worst[key])


@pytest.mark.parametrize("name", list(CASES))
def test_anchored_layer(name):
    import torch
    import post_quantization_solver_amd as mpq
    L = CASES[name]()
    rows = np.arange(L.m)
    T = layer_tensors(L)
    out = mpq.quantize_layer(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], T_vamp=L.T_vamp, n_cd=L.n_cd,
                             damping=L.damping, anchor_tau=TAU)
    torch.cuda.synchronize()
    gpu = {k: (host(v) if v is not None else None) for k, v in out.items()}
    refs = solve_rows(L, rows, anchor_tau=TAU)
    summ = compare_layer(L, rows, gpu, refs)
    print(f"[anchor layer] {name}: codes {summ['code_agreement']:.5f} obj {summ['obj_rel_max']:.2e} "
          f"traces {summ['trace_rel_max']}", flush=True)
    assert summ["code_agreement"] >= CODE_FRAC
    assert summ["obj_rel_max"] < OBJ_RTOL
    for key, v in summ["trace_rel_max"].items():
        assert v < SOFT_RTOL, (key, v)
    # the anchor changes the solve: the uniform-prior run differs somewhere
    plain = mpq.quantize_layer(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], T_vamp=L.T_vamp, n_cd=L.n_cd,
                               damping=L.damping)
    torch.cuda.synchronize()
    assert not np.array_equal(host(plain["gamma1_tr"]), gpu["gamma1_tr"])
