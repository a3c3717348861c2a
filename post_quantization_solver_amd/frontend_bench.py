"""Timing of the front end on one GPU: activations -> (s, V).

    python -m post_quantization_solver_amd.frontend_bench [--N 262144] [--n 14336] [--r R] [--seed 0]

Draws seeded synthetic activations X (N x n, float32; N = 128 sequences x 2048
tokens by default, the calibration size the MPQ pages use) on the GPU, then
times, each with HIP events on the current stream after one warm-up call:
the RHT of X's rows (mpq_rht), H = X^T X (mpq_gram) and the r largest modes
of H (mpq_factor).  Prints one JSON line with the milliseconds and the
achieved rates (RHT: bytes read + written / s; gram: 2 N n^2 / 2 flops on the
lower triangle / s against the 78.6 TFLOP/s fp64 matrix peak).
"""
from __future__ import annotations

import argparse
import json

PEAK_FP64_TFLOPS = 78.6
PEAK_HBM_GBS = 8000.0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--N", type=int, default=128 * 2048)
    ap.add_argument("--n", type=int, default=14336)
    ap.add_argument("--r", type=int, default=0)
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args(argv)
    import torch
    import post_quantization_solver_amd as mpq
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    N, n = args.N, args.n
    r = args.r or n
    # columns with a decaying scale, so H has a spread spectrum
    scale = torch.exp(-3.0 * torch.arange(n, device=dev, dtype=torch.float32) / n)
    X = torch.randn((N, n), generator=gen, device=dev, dtype=torch.float32) * scale[None, :]
    signs = (torch.randint(0, 2, (n,), generator=gen, device=dev) * 2 - 1).to(torch.float32)
    res = dict(N=N, n=n, r=r)

    def timed(fn):
        st = torch.cuda.current_stream()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        out = fn()
        b.record(st)
        torch.cuda.synchronize()
        return out, a.elapsed_time(b)

    Xw = X[: min(N, 4096)].clone()
    mpq.rht(Xw, signs)
    _, res["rht_ms"] = timed(lambda: mpq.rht(X, signs))
    res["rht_GBps"] = 2 * X.numel() * 4 / (res["rht_ms"] * 1e-3) / 1e9
    res["rht_hbm_frac"] = res["rht_GBps"] / PEAK_HBM_GBS
    gws = torch.empty(int(mpq.load_library().mpq_gram_workspace_bytes(n)), dtype=torch.uint8, device=dev)
    mpq.gram(Xw, workspace=gws)
    H, res["gram_ms"] = timed(lambda: mpq.gram(X, workspace=gws))
    flops = float(N) * n * n   # lower triangle of the 2 N n^2 product
    res["gram_TFLOPs"] = flops / (res["gram_ms"] * 1e-3) / 1e12
    res["gram_fp64_frac"] = res["gram_TFLOPs"] / PEAK_FP64_TFLOPS
    del X, Xw
    torch.cuda.empty_cache()
    fws = torch.empty(int(mpq.load_library().mpq_factor_workspace_bytes(n)), dtype=torch.uint8, device=dev)
    Hw = H[:256, :256].contiguous()
    mpq.factor(Hw, 16)
    (s, V), res["factor_ms"] = timed(lambda: mpq.factor(H, r, workspace=fws))
    res["s_first_last"] = [float(s[0]), float(s[-1])]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
