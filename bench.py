"""Benchmark: one MPQ layer solve per step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config c5] [--group G] [--cpu-rows R | --no-cpu] [--no-probe]

A step is one full mpq_quantize_layer call (prologue, T_vamp VAMP
iterations, marginal MAP, 3 CD sweeps) on a seeded synthetic layer whose
inputs are already resident in HBM.  The default workload is the 2-bit E8
lattice layer 4096 x 14336 (Llama-3-8B MLP-down shape), T_vamp = 16.

Prints ONE JSON line: throughput in weights quantized per second, the
roofline of the dominant kernel (the method's algorithmic work over the time
measured with HIP events on the library's stream inside the timed region)
against the vendor's peak of the dtype it issues and against the rate this
GPU reaches on the same instruction (mpq_probe_rate, run after the timed
region; all probed rates are in `measured_peaks`), the same for the denoiser
and the linear module together, and the float64 oracle's throughput on a
bounded sample of rows of the same layer, run on the host cores.
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
PEAK_FP64_TFLOPS = 78.6        # float64 matrix and vector alike on MI355X
PEAK_INT8_TOPS = 5000.0        # dense int8 MFMA
DIGITS = 5                     # base-256 digits per operand entry of the digit products (set from --digits)
# Digits a workload runs with unless --digits says otherwise (the library
# default elsewhere).  4 digits split each operand row exact to 2^-31 of its
# largest entry; on the 4096 x 14336 lattice workload that keeps every sampled
# code and trace within the parity bar (tests/test_gpu_configs.py, case c5).
WORKLOAD_DIGITS = {"c5": 4}
DIGIT_PRODUCTS = 15            # int8 digit products per multiply-add of the linear module: DIGITS (DIGITS + 1) / 2
PEAK_HBM_GBS = 8000.0
CD_MFMA_FLOP_PER_EVAL = 64     # bf16 MFMA flops the CD scoring issues per (row, block, codeword)
# Transcendental issue rate: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz at half
# the fp32 VALU rate on gfx950 -> 19.66e12 exp/s (a throughput probe reads 18.4e12).
EXP_RATE = 256 * 4 * 16 * 2.4e9 / 2
LATTICE_FLOP_PER_EVAL = 36     # 2*8 (distance contraction) + 2*10 (weighted moments)
SCALAR_FLOP_PER_EVAL = 8       # distance, scaled logit, three moment updates
TARGET_EVAL_FLOPS = 32     # the target's count of denoiser work per (block, codeword) eval

WORKLOADS = {
    "c1": "3-bit scalar toy layer 64x256, T_vamp=8, 3 CD sweeps",
    "c2": "3-bit scalar Llama-3.2-1B attention projection 2048x2048 (Laplace + 1% outlier columns), T_vamp=16, 3 CD",
    "c3": "4-bit scalar Llama-3.2-1B MLP-down 2048x8192, T_vamp=16, 3 CD",
    "c4": "2-bit E8 lattice Llama-3-8B attention projection 4096x4096, T_vamp=16, 3 CD",
    "c5": "2-bit E8 lattice Llama-3-8B MLP-down 4096x14336 (Student-t rows), T_vamp=16, 3 CD",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def mpq_digits_default():
    import post_quantization_solver_amd as mpq
    return mpq.binding.DIGITS_DEFAULT


def mpq_e8dp_transitions(E):
    import post_quantization_solver_amd as mpq
    return mpq.binding.e8dp_transitions(E)


def group_work(L, kernel, launches, steps, n_cd):
    """Algorithmic work of `launches` launches of a kernel group and the peak
    of the dtype it issues: (flops, peak TFLOP/s, bound, basis)."""
    m, n, r, K, d = L.m, L.n, L.r, L.K, L.d
    if kernel == "denoise" and d == 8 and mpq_e8dp_transitions(L.E) > 0:
        # forward-backward pass over the trimmed E8 automaton: 8 flops per
        # transition per block, float64 on the vector units
        return (launches * m * (n // d) * 8.0 * mpq_e8dp_transitions(L.E), PEAK_FP64_TFLOPS, "alu",
                "E8 forward-backward, 8 flops per automaton transition per block, float64 vector")
    if kernel == "denoise":
        per = LATTICE_FLOP_PER_EVAL if d == 8 else SCALAR_FLOP_PER_EVAL
        return (launches * m * (n // d) * K * per, per * EXP_RATE / 1e12, "alu",
                f"{per} flops and one exponential per (block, codeword)")
    if kernel in ("linear1", "linear2"):
        # one m x n x r product per launch, issued as exact int8 digit
        # products on the int8 matrix cores
        return launches * 2.0 * m * n * r, PEAK_INT8_TOPS, "mfma", "2mnr flops per launch, int8 digit MFMA"
    if kernel == "cd_score" and d == 8:
        # every sweep scores every codeword for every (row, block): the
        # method's own work is 2d flops per eval (e . q); it issues bf16 MFMAs
        evals = float(steps) * n_cd * m * (n // d) * K
        return evals * 2.0 * d, PEAK_BF16_MFMA_TFLOPS, "mfma", "2d flops per (row, block, codeword), bf16 MFMA"
    return None


def dominant_roofline(L, prof, steps, n_cd):
    """Roofline entry for the kernel group with the largest time: the
    method's algorithmic work over the measured time, against the peak of the
    dtype the kernel issues."""
    best = max(prof, key=lambda k: prof[k][0])
    ms, launches = prof[best]
    base = dict(kernel=best, traffic=None, launches=launches, avg_ms=ms / max(launches, 1))
    w = group_work(L, best, launches if best != "cd_score" else 0, steps, n_cd)
    if w is None:
        return dict(base, bound="alu", achieved=None, peak=None, unit="TFLOP/s", frac=None)
    flops, peak, bound, basis = w
    achieved = flops / (ms / 1e3) / 1e12
    out = dict(base, bound=bound, achieved=achieved, peak=peak, unit="TFLOP/s", frac=achieved / peak, basis=basis)
    if best in ("linear1", "linear2"):
        issued = DIGIT_PRODUCTS * achieved
        out["secondary"] = dict(bound="mfma", achieved=issued, peak=PEAK_INT8_TOPS, unit="TOP/s",
                                frac=issued / PEAK_INT8_TOPS,
                                basis=f"int8 MFMA operations as issued ({DIGIT_PRODUCTS} digit products per "
                                      f"multiply-add, {DIGITS} base-256 digits per operand entry), not the "
                                      "method's work",
                                fp64_equivalent=dict(achieved=achieved, peak=PEAK_FP64_TFLOPS,
                                                     frac=achieved / PEAK_FP64_TFLOPS))
    if best == "cd_score":
        issued = flops / (2.0 * L.d) * CD_MFMA_FLOP_PER_EVAL / (ms / 1e3) / 1e12
        out["secondary"] = dict(bound="mfma", achieved=issued, peak=PEAK_BF16_MFMA_TFLOPS, unit="TFLOP/s",
                                frac=issued / PEAK_BF16_MFMA_TFLOPS,
                                basis=f"bf16 MFMA flops as issued ({CD_MFMA_FLOP_PER_EVAL} per eval: split query "
                                      "terms and the quadratic key), not the method's work")
    return out


def denoise_linear_fraction(L, prof, steps):
    """mpq_denoise + mpq_linear together: (a) the fraction of their measured
    time the issuing units would need at peak for the method's algorithmic
    work (sum of work / peak over the sum of times; the linear module's 2mnr
    against the int8 peak it issues on); (a') the same with the linear
    module's work counted as the int8 operations it issues; (b) the work as
    the target counts it (32 flops per block x codeword eval, 4mnr per
    iteration) over the same time, against the fp32 MFMA peak."""
    keys = [k for k in ("denoise", "linear1", "linear2") if k in prof]
    secs = sum(prof[k][0] for k in keys) / 1e3
    if secs <= 0:
        return None
    need = need_issued = 0.0
    for k in keys:
        w = group_work(L, k, prof[k][1], steps, L.n_cd)
        if w is None:
            return None
        need += w[0] / (w[1] * 1e12)
        need_issued += w[0] * (DIGIT_PRODUCTS if k.startswith("linear") else 1) / (w[1] * 1e12)
    T = L.T_vamp * steps
    target_flops = T * (L.m * (L.n // L.d) * L.K * TARGET_EVAL_FLOPS + 4.0 * L.m * L.n * L.r)
    return dict(seconds=secs, frac_of_issuing_peaks=need / secs, frac_of_issuing_peaks_as_issued=need_issued / secs,
                target_count_tflops=target_flops / secs / 1e12,
                target_count_frac_fp32=target_flops / secs / 1e12 / PEAK_FP32_MFMA_TFLOPS,
                basis="(a) sum over denoise, linear 1, linear 2 of algorithmic work / peak of the issued dtype, "
                      "over their summed time; (a') the same with the linear products counted as the int8 digit "
                      "products they issue; (b) 32 flops per (block, codeword) eval + 4mnr per iteration over the "
                      "same time, against the fp32 MFMA peak (the E8 path does far less work than that count)")


def measured_peak(roof, probes):
    """The probed counterpart of roof["peak"] (same unit), or None."""
    if roof["peak"] is None:
        return None
    if roof["kernel"] in ("linear1", "linear2"):
        return None   # the int8 probe reads against the issued rate (roofline.secondary)
    if roof["bound"] == "mfma":
        return probes["mfma_bf16_tflops"]
    if roof.get("basis", "").startswith("E8 forward-backward"):
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
        path = os.path.join(ROOT, f)
        if not os.path.exists(path):
            return None
        h.update(open(path, "rb").read())
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
    model = ""
    try:
        import subprocess
        txt = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        model = next((ln.split(":", 1)[1].strip() for ln in txt.splitlines() if ln.startswith("Model name")), "")
    except Exception:  # noqa: BLE001 - the CPU model is informational
        pass
    agree = float(np.mean([np.mean(gpu_codes[i] == r["codes"]) for i, r in zip(rows, res)]))
    def codebook(i):
        if L.group:
            return O.GroupedCodebook(L.E, L.a[i], L.o[i], L.n, L.d, L.group)
        return O.row_codewords(L.E, L.a[i], L.o[i])
    obj_rel = max(abs(O.codes_objective(L.W[i], gpu_codes[i], codebook(i), L.d, L.s, L.V)
                      - r["objective"]) / r["objective"] for i, r in zip(rows, res))
    value = len(rows) * L.n / wall
    return dict(value=value, unit="weights/s", cores=min(len(rows), os.cpu_count() or 1), kind="oracle",
                host_cpus=os.cpu_count(), cpu_model=model, workers=len(rows),
                sample=f"{len(rows)} rows (every {max(L.m // len(rows), 1)}-th) of the same layer through the "
                       f"whole pipeline, one single-threaded float64 NumPy worker process per row on "
                       f"{os.cpu_count()} host CPUs; wall {wall:.1f} s",
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
    ap.add_argument("--digits", type=int, default=None, choices=[0, 4, 5],
                    help="base-256 digits per operand entry of the int8 digit products (0: the library default; "
                         "unset: the workload's setting, 4 for c5 as its parity test runs it, else the default)")
    ap.add_argument("--no-split", action="store_true",
                    help="skip the extra profiled step that gives the per-group time split (keeps a counter pass "
                         "to one solve's dispatches: rocprofv3 --pmc has crashed in its dispatch interception after "
                         "about 20 000 dispatches in one process)")
    ap.add_argument("--only", choices=["linear", "cd"], default=None,
                    help="run only two calls of the linear module (mpq_linear_step) on the workload's shapes and "
                         "exit: a short program with few dispatches for counter passes over the dominant kernels")
    ap.add_argument("--host-qr", action="store_true",
                    help="draw the orthogonal factor V with NumPy's QR on the host instead of rocSOLVER's (e.g. "
                         "under counter collection, where rocSOLVER's QR has crashed the profiled process); "
                         "V is then another orthogonal draw of the same distribution")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 times), the reference kernel for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    global DIGITS, DIGIT_PRODUCTS
    DIGITS = (args.digits if args.digits is not None else WORKLOAD_DIGITS.get(args.config, 0)) or mpq_digits_default()
    DIGIT_PRODUCTS = DIGITS * (DIGITS + 1) // 2
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
    L = load_or_make(S, args.config, None if args.host_qr else dev, args.cache, args.group)
    if args.n_cd is not None:
        L.n_cd = args.n_cd
    log(f"[bench] {args.config}: m={L.m} n={L.n} r={L.r} K={L.K} d={L.d} T={L.T_vamp} S={L.n_cd} "
        f"inputs in {time.perf_counter() - t0:.1f} s")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)  # noqa: E731
    W, s, V, a, o = t(L.W), t(L.s), t(L.V), t(L.a), t(L.o)
    if args.only == "linear":
        # the linear module alone on a synthetic extrinsic message (r2 near w)
        gen = torch.Generator(device=dev).manual_seed(7)
        R2 = W.double() + 0.01 * torch.randn(W.shape, dtype=torch.float64, device=dev, generator=gen)
        g2 = torch.full((L.m,), 10.0, dtype=torch.float64, device=dev)
        beta = torch.ones(L.m, dtype=torch.float64, device=dev)
        for k in range(2):
            mpq.linear_step(R2, g2, beta, W, s, V, damping=L.damping, digits=DIGITS)
            torch.cuda.synchronize()
            log(f"[bench] linear module call {k + 1}/2 done")
        return
    if args.only == "cd":
        # one CD sweep alone, from the round-to-nearest codes of the prologue
        cb = mpq.prepare_codebook(L.E, dev)
        pro = mpq.prologue(W, s, V, cb, a, o, digits=DIGITS)
        codes = pro["rtn_codes"].clone()
        torch.cuda.synchronize()
        log("[bench] prologue done")
        mpq.cd(W, s, V, cb, a, o, codes, n_cd=1, digits=DIGITS)
        torch.cuda.synchronize()
        log("[bench] one CD sweep done")
        return
    ws = torch.empty(mpq.workspace_bytes(L.m, L.n, L.r, L.K, L.d), dtype=torch.uint8, device=dev)
    kw = dict(T_vamp=L.T_vamp, n_cd=L.n_cd, damping=L.damping, workspace=ws, group=L.group, digits=DIGITS)
    cb = mpq.prepare_codebook(L.E, dev)   # the codebook's device tables, once per layer
    out = None
    for k in range(args.warmup):
        out = mpq.quantize_layer(W, s, V, cb, a, o, outputs=out, **kw)
        torch.cuda.synchronize()
        log(f"[bench] warmup {k + 1}/{args.warmup} done")

    # timed region: K steps; the single-kernel groups are event-timed on the
    # library's stream (the CD scoring launches one in 32, priced at their mean)
    prof = mpq.Profile(("denoise", "linear1", "linear2", "cd_score"), sampled=True, capacity=4096)
    full = mpq.Profile(capacity=32768)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        out = mpq.quantize_layer(W, s, V, cb, a, o, outputs=out, profile=prof, **kw)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / args.steps
    value = L.m * L.n / (ms_per_step / 1e3)
    timed_prof = prof.as_dict()
    log(f"[bench] {args.steps} steps: {ms_per_step:.1f} ms/step, {value / 1e6:.3f} M weights/s")

    # one extra profiled step with every kernel group for the time split
    split = None
    if not args.no_split:
        out = mpq.quantize_layer(W, s, V, cb, a, o, outputs=out, profile=full, **kw)
        torch.cuda.synchronize()
        split = {k: round(v[0], 3) for k, v in full.as_dict().items()}
        log(f"[bench] kernel ms per step: {split}")
    # candidates are the single-kernel groups (the CD GEMM and update groups
    # each span several kernels and are reported in the split only)
    roof = dominant_roofline(L, {k: v for k, v in timed_prof.items()
                                 if k in ("denoise", "linear1", "linear2", "cd_score")},
                             args.steps, L.n_cd)
    roof["traffic"] = measured_traffic(args.config, roof["kernel"])
    dl = denoise_linear_fraction(L, timed_prof, args.steps)
    codes = out["codes"].cpu().numpy()

    # achievable rates of the instructions the kernels are bound by, probed on
    # this GPU (outside the timed region; the solver workspace is the scratch)
    probes = None
    if not args.no_probe:
        rates = {k: mpq.probe_rate(k, ws) for k in mpq.binding.PROBE_KINDS}
        probes = dict(mfma_bf16_tflops=rates["mfma_bf16"] / 1e12, mfma_f64_tflops=rates["mfma_f64"] / 1e12,
                      mfma_i8_tops=rates["mfma_i8"] / 1e12, valu_f64_tflops=rates["valu_f64"] / 1e12,
                      exp_f32_tops=rates["exp_f32"] / 1e12, hbm_copy_gbs=rates["hbm_copy"] / 1e9)
        log(f"[bench] probed rates: " + ", ".join(f"{k} {v:.1f}" for k, v in probes.items()))
        measured = measured_peak(roof, probes)
        if measured and roof["achieved"] is not None:
            roof["measured_peak"] = measured
            roof["frac_of_measured"] = roof["achieved"] / measured
        if roof["kernel"] in ("linear1", "linear2") and "secondary" in roof:
            # the issued int8 rate against the rate this GPU reaches on random digit bytes
            sec = roof["secondary"]
            sec["measured_peak"] = probes["mfma_i8_tops"]
            sec["frac_of_measured"] = sec["achieved"] / probes["mfma_i8_tops"]

    cpu = None
    if not args.no_cpu:
        rows = args.cpu_rows or max(1, min(16, os.cpu_count() or 1))
        log(f"[bench] oracle baseline on {rows} rows ...")
        cpu = cpu_baseline(L, rows, codes)
        log(f"[bench] oracle {cpu['value']:.1f} weights/s; parity on its rows {cpu['parity']}")

    line = dict(metric=METRIC, value=value, unit="weights/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
                ms_per_step=ms_per_step, higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f64",
                data="synthetic",
                config=dict(workload=f"{args.config}: {WORKLOADS[args.config]}" +
                            (f", group-wise grids of {L.group} columns" if L.group else ""), m=L.m, n=L.n, r=L.r,
                            K=L.K, d=L.d, T_vamp=L.T_vamp, n_cd=L.n_cd, damping=L.damping, digits=DIGITS,
                            **({"group": L.group} if L.group else {})),
                roofline=dict(bound=roof["bound"], achieved=roof["achieved"], peak=roof["peak"], unit=roof["unit"],
                              frac=roof["frac"], traffic=roof["traffic"], kernel=roof["kernel"],
                              avg_launch_ms=roof["avg_ms"], launches=roof["launches"],
                              **({"basis": roof["basis"]} if "basis" in roof else {}),
                              **({"measured_peak": roof["measured_peak"], "frac_of_measured": roof["frac_of_measured"]}
                                 if "measured_peak" in roof else {}),
                              **({"secondary": roof["secondary"]} if "secondary" in roof else {})),
                products=f"int8 digit products, {DIGITS} base-256 digits per operand entry "
                         f"({DIGIT_PRODUCTS} per multiply-add, split exact to 2^-{8 * DIGITS - 1} of each row's "
                         "largest entry); float64 VAMP state",
                denoise_linear=dl, measured_peaks=probes, kernel_ms_per_step=split, cpu_baseline=cpu)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
