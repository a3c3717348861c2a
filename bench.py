"""Benchmark: one MPQ layer solve per step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config c5] [--group G] [--cpu-rows R | --no-cpu] [--no-probe]

A step is one full mpq_quantize_layer call (prologue, T_vamp VAMP
iterations, marginal MAP, 3 CD sweeps) on a seeded synthetic layer whose
inputs are already resident in HBM.  The default workload is the 2-bit E8
lattice layer 4096 x 14336 (Llama-3-8B MLP-down shape), T_vamp = 16.

Prints ONE JSON line: throughput in weights quantized per second, the
roofline of the dominant kernel (timed with HIP events on the library's
stream inside the timed region) against the vendor's peak and against the
rate this GPU reaches on the same instruction (mpq_probe_rate, run after the
timed region; all probed rates are in `measured_peaks`), and the float64
oracle's throughput on a bounded sample of rows of the same layer, run on
the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "weights quantized/sec per layer (T_vamp=16 + 3 CD sweeps), % of MFMA/HBM peak"

# MI355X published peaks
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_BF16_MFMA_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
PEAK_FP64_VALU_TFLOPS = 78.6   # float64 vector and matrix alike on MI355X
CD_MFMA_FLOP_PER_EVAL = 64
# Transcendental issue rate: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz at half
# the fp32 VALU rate on gfx950 -> 19.66e12 exp/s (a throughput probe reads 18.4e12).
EXP_RATE = 256 * 4 * 16 * 2.4e9 / 2
LATTICE_FLOP_PER_EVAL = 36     # 2*8 (distance contraction) + 2*10 (weighted moments)
LATTICE_MFMA_FLOP_PER_EVAL = 128   # bf16 MFMA flops the lattice denoiser issues per eval
SCALAR_FLOP_PER_EVAL = 8       # distance, scaled logit, three moment updates
SPLIT_BF16_PRODUCTS = 6        # linear GEMMs: bf16 cross products per float32 product (hh hm mh hl lh mm)

WORKLOADS = {
    "c1": "3-bit scalar toy layer 64x256, T_vamp=8, 3 CD sweeps",
    "c2": "3-bit scalar Llama-3.2-1B attention projection 2048x2048 (Laplace + 1% outlier columns), T_vamp=16, 3 CD",
    "c3": "4-bit scalar Llama-3.2-1B MLP-down 2048x8192, T_vamp=16, 3 CD",
    "c4": "2-bit E8 lattice Llama-3-8B attention projection 4096x4096, T_vamp=16, 3 CD",
    "c5": "2-bit E8 lattice Llama-3-8B MLP-down 4096x14336 (Student-t rows), T_vamp=16, 3 CD",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def mpq_e8dp_transitions(E):
    import post_quantization_solver_amd as mpq
    return mpq.binding.e8dp_transitions(E)


def dominant_roofline(L, prof, steps, n_cd):
    """Roofline entry for the kernel group with the largest time."""
    m, n, r, K, d = L.m, L.n, L.r, L.K, L.d
    best = max(prof, key=lambda k: prof[k][0])
    ms, launches = prof[best]
    per_launch_s = ms / max(launches, 1) / 1e3
    base = dict(kernel=best, traffic=None, launches=launches, avg_ms=ms / max(launches, 1))
    if best == "denoise" and d == 8 and mpq_e8dp_transitions(L.E) > 0:
        # forward-backward pass over the trimmed E8 automaton: 8 flops per
        # transition per block, on the float64 vector units
        flops = m * (n // d) * 8.0 * mpq_e8dp_transitions(L.E)
        achieved = flops / per_launch_s / 1e12
        return dict(base, bound="alu", achieved=achieved, peak=PEAK_FP64_VALU_TFLOPS, unit="TFLOP/s",
                    frac=achieved / PEAK_FP64_VALU_TFLOPS, path="E8 forward-backward (float64)")
    if best == "denoise":
        evals = m * (n // d) * K
        if d == 8:
            flops = evals * LATTICE_FLOP_PER_EVAL
            peak = LATTICE_FLOP_PER_EVAL * EXP_RATE / 1e12
        else:
            flops = evals * SCALAR_FLOP_PER_EVAL
            peak = SCALAR_FLOP_PER_EVAL * EXP_RATE / 1e12
        achieved = flops / per_launch_s / 1e12
        out = dict(base, bound="alu", achieved=achieved, peak=peak, unit="TFLOP/s", frac=achieved / peak)
        if d == 8:
            # the same launch against the bf16 matrix cores: per 16 queries x 32 codewords
            # it issues two score and two weighted-sum 16x16x32 MFMAs (128 flops per eval)
            mf = evals * LATTICE_MFMA_FLOP_PER_EVAL / per_launch_s / 1e12
            out["secondary"] = dict(bound="mfma", achieved=mf, peak=PEAK_BF16_MFMA_TFLOPS, unit="TFLOP/s",
                                    frac=mf / PEAK_BF16_MFMA_TFLOPS)
        return out
    if best in ("linear1", "linear2"):
        # float32-accurate m x n x r product issued as split-bf16 MFMAs: six
        # bf16 cross products per float32 product, priced at the bf16 peak
        flops = 2.0 * m * n * r
        fp32_equiv = flops / per_launch_s / 1e12
        achieved = SPLIT_BF16_PRODUCTS * fp32_equiv
        return dict(base, bound="mfma", achieved=achieved, peak=PEAK_BF16_MFMA_TFLOPS, unit="TFLOP/s",
                    frac=achieved / PEAK_BF16_MFMA_TFLOPS,
                    secondary=dict(bound="mfma", achieved=fp32_equiv, peak=PEAK_FP32_MFMA_TFLOPS, unit="TFLOP/s",
                                   frac=fp32_equiv / PEAK_FP32_MFMA_TFLOPS,
                                   basis="float32-equivalent vs the fp32 MFMA peak"))
    if best == "cd_score" and d == 8:
        # every sweep scores every codeword for every (row, block): one bf16
        # 16x16x32 MFMA per 16 rows x 16 codewords issues 64 flops per eval
        # (the three-way split of q, the t terms); the method's own work is 2d
        # flops per eval (e . q)
        evals = float(steps) * n_cd * m * (n // d) * K
        secs = ms / 1e3
        issued = evals * CD_MFMA_FLOP_PER_EVAL / secs / 1e12
        algo = evals * 2.0 * d / secs / 1e12
        return dict(base, bound="mfma", achieved=issued, peak=PEAK_BF16_MFMA_TFLOPS, unit="TFLOP/s",
                    frac=issued / PEAK_BF16_MFMA_TFLOPS,
                    secondary=dict(bound="mfma", achieved=algo, peak=PEAK_FP32_MFMA_TFLOPS, unit="TFLOP/s",
                                   frac=algo / PEAK_FP32_MFMA_TFLOPS,
                                   basis="2d flops per eval (float32-equivalent) vs the fp32 MFMA peak"))
    return dict(base, bound="alu", achieved=None, peak=None, unit="TFLOP/s", frac=None)


def measured_peak(roof, probes):
    """The probed counterpart of roof["peak"] (same unit), or None."""
    if roof["peak"] is None:
        return None
    if roof["bound"] == "mfma":
        return probes["mfma_bf16_tflops"]
    if roof.get("path", "").startswith("E8 forward-backward"):
        return probes["valu_f64_tflops"]
    if roof["kernel"] == "denoise":
        # exponential-bound scan: the vendor-derived peak scales with the exp rate
        return roof["peak"] * probes["exp_f32_tops"] * 1e12 / EXP_RATE
    return None


def measured_traffic(config, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by a plain copy's readings), or
    None when there is none or the kernel's sources changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"counters_{config}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("kernels", {}).get(kernel)
    if not rec:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return rec["hbm_bytes_per_launch"] if h.hexdigest() == rec["sources_sha256"] else None


def cpu_baseline(L, rows_count, gpu_codes):
    """Time the float64 oracle on `rows_count` rows of the layer, one worker
    process per row (each solves its row through the whole pipeline)."""
    import numpy as np
    import mpq_synth as S
    from oracle import mpq_oracle as O
    from oracle.pool import solve_rows
    rows = S.parity_rows(L.m, rows_count)
    t0 = time.perf_counter()
    res = solve_rows(L, rows, max_workers=len(rows))
    wall = time.perf_counter() - t0
    agree = float(np.mean([np.mean(gpu_codes[i] == r["codes"]) for i, r in zip(rows, res)]))
    def codebook(i):
        if L.group:
            return O.GroupedCodebook(L.E, L.a[i], L.o[i], L.n, L.d, L.group)
        return O.row_codewords(L.E, L.a[i], L.o[i])
    obj_rel = max(abs(O.codes_objective(L.W[i], gpu_codes[i], codebook(i), L.d, L.s, L.V)
                      - r["objective"]) / r["objective"] for i, r in zip(rows, res))
    value = len(rows) * L.n / wall
    return dict(value=value, unit="weights/s", cores=len(rows), kind="oracle",
                sample=f"{len(rows)} rows (every {max(L.m // len(rows), 1)}-th) of the same layer through the "
                       f"whole pipeline, one single-threaded float64 NumPy worker per row; wall {wall:.1f} s",
                parity=dict(rows=len(rows), code_agreement=agree, obj_rel_max=obj_rel))


def load_or_make(S, name, dev, cache, group=0):
    """The named workload; with `cache`, arrays are saved there once and reloaded."""
    import numpy as np
    fields = ("W", "s", "V", "E", "a", "o")
    path = os.path.join(cache, name + (f"_g{group}" if group else "")) if cache else ""
    if path and all(os.path.exists(os.path.join(path, f + ".npy")) for f in fields):
        ref = S.make_config("c1")  # only for the scalar metadata of the Layer record
        arr = {f: np.load(os.path.join(path, f + ".npy")) for f in fields}
        spec = S.configs._SPECS[name]
        return S.Layer(name, arr["W"], arr["s"], arr["V"], arr["E"], arr["a"], arr["o"], spec["d"],
                       spec.get("T_vamp", 16), ref.n_cd, ref.damping, group=group)
    L = S.make_config(name, device=dev, group=group)
    if path:
        os.makedirs(path, exist_ok=True)
        for f in fields:
            np.save(os.path.join(path, f + ".npy"), getattr(L, f))
    return L


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="c5", choices=sorted(WORKLOADS))
    ap.add_argument("--group", type=int, default=0,
                    help="scalar workloads: group-wise grids of this many columns (0: one grid per row)")
    ap.add_argument("--cpu-rows", type=int, default=0, help="oracle rows for the CPU baseline (0: host cores, <=16)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cache", default="", help="directory for the generated inputs (reused when present)")
    ap.add_argument("--n-cd", type=int, default=None,
                    help="CD sweeps (default: the workload's 3); 0 runs only the prologue, VAMP and MAP, e.g. for "
                         "counter passes over the VAMP kernels")
    ap.add_argument("--no-probe", action="store_true", help="skip the achievable-rate probes")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 times), the reference kernel for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_calibration} MiB 5 times")
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the MPQ layer solve is single-GPU here "
              "(rows would shard across GPUs with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import mpq_synth as S
    import post_quantization_solver_amd as mpq

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    mpq.load_library()
    t0 = time.perf_counter()
    if args.group and S.configs._SPECS[args.config]["d"] != 1:
        print("--group applies to the scalar workloads (c1, c2, c3)", file=sys.stderr)
        sys.exit(2)
    L = load_or_make(S, args.config, dev, args.cache, args.group)
    if args.n_cd is not None:
        L.n_cd = args.n_cd
    log(f"[bench] {args.config}: m={L.m} n={L.n} r={L.r} K={L.K} d={L.d} T={L.T_vamp} S={L.n_cd} "
        f"inputs in {time.perf_counter() - t0:.1f} s")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)  # noqa: E731
    W, s, V, a, o = t(L.W), t(L.s), t(L.V), t(L.a), t(L.o)
    ws = torch.empty(mpq.workspace_bytes(L.m, L.n, L.r, L.K, L.d), dtype=torch.uint8, device=dev)
    kw = dict(T_vamp=L.T_vamp, n_cd=L.n_cd, damping=L.damping, workspace=ws, group=L.group)
    out = None
    for k in range(args.warmup):
        out = mpq.quantize_layer(W, s, V, L.E, a, o, outputs=out, **kw)
        torch.cuda.synchronize()
        log(f"[bench] warmup {k + 1}/{args.warmup} done")

    # timed region: K steps; the single-kernel groups are event-timed on the
    # library's streams (the CD scoring launches one in 32, scaled to all)
    prof = mpq.Profile(("denoise", "linear1", "linear2", "cd_score"), sampled=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        out = mpq.quantize_layer(W, s, V, L.E, a, o, outputs=out, profile=prof, **kw)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / args.steps
    value = L.m * L.n / (ms_per_step / 1e3)
    timed_prof = prof.as_dict()
    log(f"[bench] {args.steps} steps: {ms_per_step:.1f} ms/step, {value / 1e6:.3f} M weights/s")

    # one extra profiled step with every kernel group for the time split
    full = mpq.Profile()
    out = mpq.quantize_layer(W, s, V, L.E, a, o, outputs=out, profile=full, **kw)
    torch.cuda.synchronize()
    split = {k: round(v[0], 3) for k, v in full.as_dict().items()}
    log(f"[bench] kernel ms per step: {split}")
    # candidates are the single-kernel groups (the CD GEMM and update groups
    # each span several kernels and are reported in the split only)
    roof = dominant_roofline(L, {k: v for k, v in timed_prof.items()
                                 if k in ("denoise", "linear1", "linear2", "cd_score")},
                             args.steps, L.n_cd)
    roof["traffic"] = measured_traffic(args.config, roof["kernel"])
    codes = out["codes"].cpu().numpy()

    # achievable rates of the instructions the kernels are bound by, probed on
    # this GPU (outside the timed region; the solver workspace is the scratch)
    probes = None
    if not args.no_probe:
        rates = {k: mpq.probe_rate(k, ws) for k in mpq.binding.PROBE_KINDS}
        probes = dict(mfma_bf16_tflops=rates["mfma_bf16"] / 1e12, mfma_f64_tflops=rates["mfma_f64"] / 1e12,
                      valu_f64_tflops=rates["valu_f64"] / 1e12, exp_f32_tops=rates["exp_f32"] / 1e12,
                      hbm_copy_gbs=rates["hbm_copy"] / 1e9)
        log(f"[bench] probed rates: " + ", ".join(f"{k} {v:.1f}" for k, v in probes.items()))
        measured = measured_peak(roof, probes)
        if measured and roof["achieved"] is not None:
            roof["measured_peak"] = measured
            roof["frac_of_measured"] = roof["achieved"] / measured

    cpu = None
    if not args.no_cpu:
        rows = args.cpu_rows or max(1, min(16, os.cpu_count() or 1))
        log(f"[bench] oracle baseline on {rows} rows ...")
        cpu = cpu_baseline(L, rows, codes)
        log(f"[bench] oracle {cpu['value']:.1f} weights/s; parity on its rows {cpu['parity']}")

    line = dict(metric=METRIC, value=value, unit="weights/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
                ms_per_step=ms_per_step, higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f32",
                data="synthetic",
                config=dict(workload=f"{args.config}: {WORKLOADS[args.config]}" +
                            (f", group-wise grids of {L.group} columns" if L.group else ""), m=L.m, n=L.n, r=L.r,
                            K=L.K, d=L.d, T_vamp=L.T_vamp, n_cd=L.n_cd, damping=L.damping,
                            **({"group": L.group} if L.group else {})),
                roofline=dict(bound=roof["bound"], achieved=roof["achieved"], peak=roof["peak"], unit=roof["unit"],
                              frac=roof["frac"], traffic=roof["traffic"], kernel=roof["kernel"],
                              avg_launch_ms=roof["avg_ms"], launches=roof["launches"],
                              **({"path": roof["path"]} if "path" in roof else {}),
                              **({"measured_peak": roof["measured_peak"], "frac_of_measured": roof["frac_of_measured"]}
                                 if "measured_peak" in roof else {}),
                              **({"secondary": roof["secondary"]} if "secondary" in roof else {})),
                measured_peaks=probes, kernel_ms_per_step=split, cpu_baseline=cpu)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
