"""Ablation grid and mechanism diagnostics of the MPQ solve on one layer.

    python -m post_quantization_solver_amd.ablation [--config c5] [--T 1 4 8 16] [--S 0 1 3]
                                                    [--group G] [--json FILE] [--markdown FILE]

Reproduces the shape of the ablation table of the papernotes.org MPQ summary
(ablation section, Table 3: VAMP iterations x CD sweeps against a greedy
baseline with and without CD) and the mechanism diagnostics of its key
findings (terminal VAMP precision, fraction of blocks CD changes) on a seeded
synthetic layer -- perplexity needs trained weights and data, so the layer
objective 1/2 ||T (w - w_hat)||^2 stands in for it.  Cells:

  RTN (+ CD S)          T_vamp = 0: round to nearest, then S CD sweeps
  greedy (+ CD S)       the sequential greedy comparator (mpq_greedy), then S sweeps
  MPQ-T (+ CD S)        T VAMP iterations, marginal MAP, S sweeps

Per cell: seconds (one call, inputs resident on the GPU, after one warm-up
call), the layer objective (sum over rows, and relative to RTN), and for MPQ
cells the median terminal precision gamma1^T (raw and in codebook units
gamma1^T a^2), the fraction of blocks whose final code differs from the
marginal-MAP code, and CD moves per block.  Everything runs in the library's
kernels; this module only calls the binding and summarises the results.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np


def _sync():
    import torch
    torch.cuda.synchronize()


def layer_scale(a):
    """Per-row codebook scale (the largest group scale with group-wise grids)."""
    a = np.asarray(a, np.float64)
    return np.abs(a).max(axis=1) if a.ndim == 2 else np.abs(a)


def cell_stats(out, f_rtn_total, a_scale):
    """Summary of one MPQ / RTN cell from quantize_layer(..., diagnostics=True)."""
    f = out["objective"].double().cpu().numpy()
    res = dict(objective=float(f.sum()), objective_vs_rtn=float(f.sum() / f_rtn_total))
    g1 = out.get("gamma1_tr")
    if g1 is not None and g1.shape[1] > 1:
        gT = g1[:, -1].double().cpu().numpy()
        fin = np.isfinite(gT)
        res["gamma1_T_median"] = float(np.median(gT[fin])) if fin.any() else None
        res["gamma1_T_a2_median"] = float(np.median(gT[fin] * a_scale[fin] ** 2)) if fin.any() else None
    codes = out["codes"].cpu().numpy()
    mc = out["map_codes"].cpu().numpy()
    res["cd_changed_fraction"] = float(np.mean(codes != mc))
    ch = out.get("cd_changes")
    res["cd_moves_per_block"] = float(ch.sum().item() / codes.size) if ch is not None and ch.numel() else 0.0
    return res


def run_grid(W, s, V, E, a, o, T_list=(1, 4, 8, 16), S_list=(0, 1, 3), damping=0.5, group=0, log=print):
    """All cells of the grid on device tensors (W, s, V, a, o) and the host
    codebook E.  Returns a list of dicts (one per cell)."""
    import torch
    import post_quantization_solver_amd as mpq
    m, n = W.shape
    r = s.shape[0]
    K, d = np.asarray(E).shape
    ws = torch.empty(max(mpq.workspace_bytes(m, n, r, K, d), 1), dtype=torch.uint8, device=W.device)
    a_scale = layer_scale(a.cpu().numpy())
    kw = dict(damping=damping, workspace=ws, group=group or None, diagnostics=True)

    def timed(fn):
        _sync()
        t0 = time.perf_counter()
        out = fn()
        _sync()
        return out, time.perf_counter() - t0

    # warm-up (library load, first launches)
    mpq.quantize_layer(W, s, V, E, a, o, T_vamp=1, n_cd=1, **kw)
    _sync()
    cells = []
    rtn, t_rtn = timed(lambda: mpq.quantize_layer(W, s, V, E, a, o, T_vamp=0, n_cd=0, **kw))
    f_rtn = float(rtn["objective"].double().sum().item())
    cells.append(dict(cell="RTN", T_vamp=0, S=0, seconds=t_rtn, **cell_stats(rtn, f_rtn, a_scale)))
    for S in S_list:
        if S == 0:
            continue
        out, t = timed(lambda: mpq.quantize_layer(W, s, V, E, a, o, T_vamp=0, n_cd=S, **kw))
        cells.append(dict(cell=f"RTN + CD{S}", T_vamp=0, S=S, seconds=t, **cell_stats(out, f_rtn, a_scale)))
        log(f"  {cells[-1]['cell']}: {t:.3f} s, objective / RTN {cells[-1]['objective_vs_rtn']:.4f}")
    # the greedy comparator, then CD from its codes
    gws = torch.empty(mpq.greedy_workspace_bytes(m, n, r, K, d), dtype=torch.uint8, device=W.device)
    gcodes, t_g = timed(lambda: mpq.greedy(W, s, V, E, a, o, workspace=gws, group=group or None))
    del gws
    f_g = float(mpq.objective(W, s, V, E, a, o, gcodes, workspace=ws, group=group or None).sum().item())
    cells.append(dict(cell="greedy", T_vamp=None, S=0, seconds=t_g, objective=f_g, objective_vs_rtn=f_g / f_rtn))
    log(f"  greedy: {t_g:.3f} s, objective / RTN {f_g / f_rtn:.4f}")
    for S in S_list:
        if S == 0:
            continue
        start = gcodes.clone()
        (codes, ch), t = timed(lambda: mpq.cd(W, s, V, E, a, o, start, n_cd=S, workspace=ws, group=group or None))
        f = float(mpq.objective(W, s, V, E, a, o, codes, workspace=ws, group=group or None).sum().item())
        cells.append(dict(cell=f"greedy + CD{S}", T_vamp=None, S=S, seconds=t_g + t, objective=f,
                          objective_vs_rtn=f / f_rtn, cd_changed_fraction=float((codes != gcodes).double().mean()),
                          cd_moves_per_block=float(ch.sum().item() / codes.numel())))
        log(f"  {cells[-1]['cell']}: {t_g + t:.3f} s, objective / RTN {f / f_rtn:.4f}")
    for T in T_list:
        for S in S_list:
            out, t = timed(lambda: mpq.quantize_layer(W, s, V, E, a, o, T_vamp=T, n_cd=S, **kw))
            name = f"MPQ-{T}" + (f" + CD{S}" if S else "")
            cells.append(dict(cell=name, T_vamp=T, S=S, seconds=t, **cell_stats(out, f_rtn, a_scale)))
            log(f"  {name}: {t:.3f} s, objective / RTN {cells[-1]['objective_vs_rtn']:.4f}, "
                f"gamma1^T median {cells[-1].get('gamma1_T_median')}, "
                f"CD changed {cells[-1]['cd_changed_fraction']:.3g}")
    return cells


def markdown(cells, title):
    hdr = ("| cell | T_vamp | CD sweeps | seconds | objective / RTN | median gamma1^T | median gamma1^T a^2 "
           "| blocks changed by CD | CD moves / block |")
    lines = [f"### {title}", "", hdr, "|" + "---|" * 9]
    for c in cells:
        def fmt(k, spec):
            v = c.get(k)
            return "" if v is None else format(v, spec)
        lines.append(f"| {c['cell']} | {'' if c['T_vamp'] is None else c['T_vamp']} | {c['S']} | "
                     f"{c['seconds']:.3f} | {c['objective_vs_rtn']:.4f} | {fmt('gamma1_T_median', '.4g')} | "
                     f"{fmt('gamma1_T_a2_median', '.4g')} | {fmt('cd_changed_fraction', '.4g')} | "
                     f"{fmt('cd_moves_per_block', '.4g')} |")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--config", default="c5")
    ap.add_argument("--T", type=int, nargs="+", default=[1, 4, 8, 16])
    ap.add_argument("--S", type=int, nargs="+", default=[0, 1, 3])
    ap.add_argument("--group", type=int, default=0)
    ap.add_argument("--json", default="")
    ap.add_argument("--markdown", default="")
    args = ap.parse_args(argv)
    import torch
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import mpq_synth as S
    if not torch.cuda.is_available():
        raise SystemExit("the ablation grid runs on the GPU")
    dev = torch.device("cuda:0")
    L = S.make_config(args.config, device=dev, group=args.group)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)  # noqa: E731
    print(f"[ablation] {L.name}: m={L.m} n={L.n} r={L.r} K={L.K} d={L.d} group={L.group}", flush=True)
    cells = run_grid(t(L.W), t(L.s), t(L.V), L.E, t(L.a), t(L.o), args.T, args.S, L.damping, L.group,
                     log=lambda msg: print(msg, flush=True))
    title = (f"{L.name}: m={L.m} n={L.n} K={L.K} d={L.d}" + (f" g={L.group}" if L.group else "") +
             ", one MI355X, seconds per layer solve")
    if args.json:
        with open(args.json, "w") as fh:
            json.dump(dict(config=L.name, m=L.m, n=L.n, K=L.K, d=L.d, group=L.group, cells=cells), fh, indent=1)
    md = markdown(cells, title)
    if args.markdown:
        with open(args.markdown, "w") as fh:
            fh.write(md)
    print(md, flush=True)


if __name__ == "__main__":
    main()
