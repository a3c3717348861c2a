"""Shared helpers for the GPU-vs-oracle parity tests."""
from __future__ import annotations

import numpy as np

# Tolerances (relative): soft quantities, objective; code agreement fraction.
SOFT_RTOL = 1e-4
OBJ_RTOL = 1e-5
CODE_FRAC = 0.999


def dev(x, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def layer_tensors(L, device="cuda"):
    return dict(W=dev(L.W, device), s=dev(L.s, device), V=dev(L.V, device), a=dev(L.a, device), o=dev(L.o, device))


def rel_vec(a, b):
    """||a - b|| / ||b|| for two vectors (float64)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def rel_scalar(a, b):
    a = float(a)
    b = float(b)
    if np.isinf(a) and np.isinf(b):
        return 0.0
    return abs(a - b) / abs(b) if b != 0 else abs(a - b)


def row_codebook(L, i):
    """The oracle's codebook of row i: its codewords, or its group-wise grids."""
    from oracle import mpq_oracle as O
    g = getattr(L, "group", 0)
    if g:
        return O.GroupedCodebook(L.E, L.a[i], L.o[i], L.n, L.d, g)
    return O.row_codewords(L.E, L.a[i], L.o[i])


def objectives(L, rows, codes):
    from oracle import mpq_oracle as O
    out = []
    for k, i in enumerate(rows):
        out.append(O.codes_objective(L.W[i], codes[k], row_codebook(L, i), L.d, L.s, L.V))
    return np.array(out)


def compare_layer(L, rows, gpu, refs, report_only_traces=False):
    """Compare GPU solve outputs (dict of host arrays, indexed by row) with the
    oracle results for `rows`.  Returns a summary dict."""
    codes = gpu["codes"][rows]
    ref_codes = np.stack([r["codes"] for r in refs])
    agree = float((codes == ref_codes).mean())
    f_gpu = objectives(L, rows, codes)
    f_ref = np.array([r["objective"] for r in refs])
    obj_rel = np.abs(f_gpu - f_ref) / np.maximum(f_ref, 1e-300)
    summ = dict(code_agreement=agree, obj_rel_max=float(obj_rel.max()), obj_rel=obj_rel,
                rows_codes_equal=int((codes == ref_codes).all(1).sum()), n_rows=len(rows))
    if gpu.get("beta_tr") is not None:
        tr = {}
        for key in ("beta_tr", "gamma1_tr", "gamma2_tr"):
            g = gpu[key][rows]
            o = np.stack([r[key] for r in refs])
            scale = np.abs(o)
            with np.errstate(invalid="ignore", divide="ignore"):
                rel = np.where(np.isinf(o) & np.isinf(g), 0.0, np.abs(g - o) / scale)
            tr[key] = rel
        summ["trace_rel"] = tr
        summ["trace_rel_max"] = {k: float(np.nanmax(v)) if v.size else 0.0 for k, v in tr.items()}
    return summ
