"""Seeded synthetic inputs for the MPQ layer solver.

This package builds the arrays that both the GPU library and the CPU oracle
consume: weight matrices, rank-space factors (s, V), base codebooks and the
per-row affine codebook parameters.  It contains none of the solver's
arithmetic; it only draws and arranges inputs.
"""
from .codebooks import e8_codebook, scalar_grid, lattice_row_scale, E8_RAW_RMS
from .configs import Layer, make_config, make_layer, CONFIG_NAMES, orthogonal, parity_rows

__all__ = [
    "e8_codebook", "scalar_grid", "lattice_row_scale", "E8_RAW_RMS",
    "Layer", "make_config", "make_layer", "CONFIG_NAMES", "orthogonal", "parity_rows",
]
