"""Parity of the ablation grid's cells and diagnostics (terminal gamma1
median, blocks changed by CD, objective relative to RTN) against the oracle
running the same cells row by row: objectives 1e-5 relative, gamma1 medians
1e-4 relative, changed-block fractions equal when the codes agree."""
import numpy as np
import pytest

import mpq_synth as S
from oracle.pool import solve_rows, greedy_rows, cd_rows
from parity_helpers import OBJ_RTOL, SOFT_RTOL, layer_tensors

pytestmark = pytest.mark.gpu

CASES = {
    "scalar3": lambda: S.make_layer("ab_s", 16, 128, seed=71, d=1, bits=3, power=0.5),
    "lattice_k1000": lambda: S.make_layer("ab_l", 8, 64, seed=72, d=8, K=1000, power=0.6, r=60),
}


@pytest.mark.parametrize("name", list(CASES))
def test_ablation_grid(name):
    from post_quantization_solver_amd.ablation import run_grid, layer_scale
    L = CASES[name]()
    T = layer_tensors(L)
    T_list, S_list = (1, 4), (0, 1, 3)
    cells = {c["cell"]: c for c in run_grid(T["W"], T["s"], T["V"], L.E, T["a"], T["o"], T_list, S_list,
                                            L.damping, log=lambda m: None)}
    rows = np.arange(L.m)
    a2 = layer_scale(L.a) ** 2

    f_rtn = sum(r["objective"] for r in solve_rows(L, rows, T_vamp=0, n_cd=0))
    checked = 0
    for Tv in (0,) + T_list:
        for Sc in S_list:
            name_c = ("RTN" if Tv == 0 else f"MPQ-{Tv}") + (f" + CD{Sc}" if Sc else "")
            if name_c not in cells:
                continue
            refs = solve_rows(L, rows, T_vamp=Tv, n_cd=Sc)
            c = cells[name_c]
            f_ref = sum(r["objective"] for r in refs)
            assert abs(c["objective"] - f_ref) / f_ref < OBJ_RTOL, (name_c, c["objective"], f_ref)
            assert abs(c["objective_vs_rtn"] - f_ref / f_rtn) < 1e-4, name_c
            changed = np.mean(np.concatenate([r["codes"] != r["map_codes"] for r in refs]))
            assert abs(c["cd_changed_fraction"] - changed) <= 1e-3, (name_c, c["cd_changed_fraction"], changed)
            if Tv > 0:
                gT = np.array([r["gamma1_tr"][-1] for r in refs])
                fin = np.isfinite(gT)
                assert abs(c["gamma1_T_median"] / np.median(gT[fin]) - 1.0) < SOFT_RTOL, name_c
                assert abs(c["gamma1_T_a2_median"] / np.median(gT[fin] * a2[fin]) - 1.0) < SOFT_RTOL, name_c
            checked += 1
    g = greedy_rows(L, rows)
    f_g = sum(r["objective"] for r in g)
    assert abs(cells["greedy"]["objective"] - f_g) / f_g < OBJ_RTOL
    for Sc in S_list:
        if Sc == 0:
            continue
        cdr = cd_rows(L, rows, [r["codes"] for r in g], n_cd=Sc)
        f_c = sum(r["objective"] for r in cdr)
        assert abs(cells[f"greedy + CD{Sc}"]["objective"] - f_c) / f_c < OBJ_RTOL
        checked += 1
    print(f"[ablation] {name}: {checked + 1} cells match the oracle; objective / RTN: " +
          ", ".join(f"{k} {v['objective_vs_rtn']:.3f}" for k, v in cells.items()), flush=True)
    assert all(c["seconds"] > 0 for c in cells.values())
