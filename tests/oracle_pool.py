"""Run the float64 oracle over many rows in worker processes (CPU only).

Workers are started with the 'spawn' method and import only numpy and the
oracle, so they never touch the GPU.
"""
from __future__ import annotations

import os
from concurrent.futures import ProcessPoolExecutor
import multiprocessing as mp

import numpy as np


def _init():
    os.environ["OMP_NUM_THREADS"] = "1"
    os.environ["OPENBLAS_NUM_THREADS"] = "1"


def _solve(args):
    import os, sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    from oracle import mpq_oracle as O
    w, s, V, E, a, o, d, T, n_cd, rho, record = args
    res = O.solve_row(w, s, V, E, a, o, d, T, n_cd, rho, record=record)
    C = O.row_codewords(E, a, o)
    res["map_objective"] = O.codes_objective(w, res["map_codes"], C, d, s, V)
    res["rtn_objective"] = O.codes_objective(w, res["rtn_codes"], C, d, s, V)
    return res


def workers() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def solve_rows(L, rows, T_vamp=None, n_cd=None, record=False, max_workers=None):
    """Oracle results for the given rows of a mpq_synth.Layer."""
    T = L.T_vamp if T_vamp is None else T_vamp
    S = L.n_cd if n_cd is None else n_cd
    jobs = [(L.W[i], L.s, L.V, L.E, float(L.a[i]), float(L.o[i]), L.d, T, S, L.damping, record) for i in rows]
    if len(jobs) == 1 or (max_workers or workers()) == 1:
        _init()
        return [_solve(j) for j in jobs]
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(max_workers=max_workers or workers(), mp_context=ctx, initializer=_init) as ex:
        return list(ex.map(_solve, jobs))
