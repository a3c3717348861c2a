"""Run the float64 oracle over many rows in worker processes.

TEST INFRASTRUCTURE ONLY (used by tests/ and by bench.py's CPU-baseline leg).
Workers are started with the 'spawn' method, import only numpy and the
oracle, and never touch the GPU.  Layer arrays are written once to .npy files
and memory-mapped by every worker, so large factors are not pickled per job;
each worker promotes them to float64 once.  BLAS runs single-threaded in each
worker.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import sys
import tempfile
from concurrent.futures import ProcessPoolExecutor

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_CACHE = {}
_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def _load(path):
    if path not in _CACHE:
        _CACHE.clear()
        arrs = {k: np.load(os.path.join(path, k + ".npy"), mmap_mode="r") for k in ("W", "s", "V", "E", "a", "o")}
        _CACHE[path] = dict(W=arrs["W"], a=arrs["a"], o=arrs["o"], s=np.asarray(arrs["s"], np.float64),
                            V=np.asarray(arrs["V"], np.float64), E=np.asarray(arrs["E"]))
    return _CACHE[path]


def _stage(job):
    """MAP, CD or the greedy comparator of one row (kind 'map': state = (r1,
    gamma1); kind 'cd': state = start codes; kind 'greedy': no state)."""
    if _ROOT not in sys.path:
        sys.path.insert(0, _ROOT)
    from oracle import mpq_oracle as O
    path, i, d, S, kind, state, group = job
    A = _load(path)
    w = np.asarray(A["W"][i], np.float64)
    if group:
        C = O.GroupedCodebook(A["E"], np.asarray(A["a"][i], np.float64), np.asarray(A["o"][i], np.float64),
                              w.shape[0], d, group)
    else:
        C = O.row_codewords(A["E"], float(A["a"][i]), float(A["o"][i]))
    if kind == "map":
        r1, gamma1 = state
        return O.map_codes(np.asarray(r1, np.float64), float(gamma1), C, d)
    if kind == "greedy":
        codes = O.sequential_greedy(w, A["s"], A["V"], C, d)
        return dict(codes=codes, objective=O.codes_objective(w, codes, C, d, A["s"], A["V"]))
    codes, changes = O.block_cd(np.asarray(state, np.int64), w, A["s"], A["V"], C, d, S)
    return dict(codes=codes, changes=changes, objective=O.codes_objective(w, codes, C, d, A["s"], A["V"]))


def _solve(job):
    if _ROOT not in sys.path:
        sys.path.insert(0, _ROOT)
    from oracle import mpq_oracle as O
    path, i, d, T, S, rho, record, tau, group, eps, lp = job
    A = _load(path)
    w = np.asarray(A["W"][i], np.float64)
    if group:
        a, o = np.asarray(A["a"][i], np.float64), np.asarray(A["o"][i], np.float64)
        C = O.GroupedCodebook(A["E"], a, o, w.shape[0], d, group)
    else:
        a, o = float(A["a"][i]), float(A["o"][i])
        C = O.row_codewords(A["E"], a, o)
    res = O.solve_row(w, A["s"], A["V"], A["E"], a, o, d, T, S, rho, record=record, anchor_tau=tau, group=group,
                      safeguard_eps=eps, log_prior=lp)
    res["map_objective"] = O.codes_objective(w, res["map_codes"], C, d, A["s"], A["V"])
    res["rtn_objective"] = O.codes_objective(w, res["rtn_codes"], C, d, A["s"], A["V"])
    res["row"] = int(i)
    return res


def default_workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _run(L, fn, make_jobs, max_workers):
    tmp = tempfile.mkdtemp(prefix="mpq_oracle_")
    try:
        for k in ("W", "s", "V", "E", "a", "o"):
            np.save(os.path.join(tmp, k + ".npy"), np.ascontiguousarray(getattr(L, k)))
        jobs = make_jobs(tmp)
        nw = min(max_workers or default_workers(), len(jobs))
        saved = {k: os.environ.get(k) for k in _THREAD_VARS}
        for k in _THREAD_VARS:
            os.environ[k] = "1"
        try:
            with ProcessPoolExecutor(max_workers=max(nw, 1), mp_context=mp.get_context("spawn")) as ex:
                return list(ex.map(fn, jobs))
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def solve_rows(L, rows, T_vamp=None, n_cd=None, record=False, max_workers=None, anchor_tau=None, safeguard_eps=0.0,
               log_prior=None):
    """Oracle results for the given rows of a layer (attributes W, s, V, E, a,
    o, d, T_vamp, n_cd, damping), in row order; anchor_tau: the anchored prior;
    safeguard_eps: the pass-through threshold; log_prior: one log-prior value
    per base codeword."""
    T = L.T_vamp if T_vamp is None else T_vamp
    S = L.n_cd if n_cd is None else n_cd
    rows = [int(i) for i in rows]
    group = getattr(L, "group", 0)
    lp = None if log_prior is None else np.asarray(log_prior, np.float64)
    return _run(L, _solve, lambda tmp: [(tmp, i, L.d, T, S, L.damping, record, anchor_tau, group, safeguard_eps, lp)
                                        for i in rows], max_workers)


def map_rows(L, rows, r1, gamma1, max_workers=None):
    """Oracle marginal-MAP codes of `rows` at the given (r1[k], gamma1[k])."""
    rows = [int(i) for i in rows]
    g = getattr(L, "group", 0)
    return _run(L, _stage, lambda tmp: [(tmp, i, L.d, 0, "map", (r1[k], gamma1[k]), g) for k, i in enumerate(rows)],
                max_workers)


def cd_rows(L, rows, start_codes, n_cd=None, max_workers=None):
    """Oracle block CD of `rows` from start_codes[k]."""
    S = L.n_cd if n_cd is None else n_cd
    rows = [int(i) for i in rows]
    g = getattr(L, "group", 0)
    return _run(L, _stage, lambda tmp: [(tmp, i, L.d, S, "cd", start_codes[k], g) for k, i in enumerate(rows)],
                max_workers)


def greedy_rows(L, rows, max_workers=None):
    """Oracle sequential-greedy codes (reading G3) of `rows`, with their objectives."""
    rows = [int(i) for i in rows]
    g = getattr(L, "group", 0)
    return _run(L, _stage, lambda tmp: [(tmp, i, L.d, 0, "greedy", None, g) for i in rows], max_workers)
