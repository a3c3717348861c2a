"""MPQ post-training-quantization layer solver for AMD Instinct MI355X.

The solver (rank-space VAMP with a blockwise discrete denoiser and an
empirical-Bayes inverse temperature, then marginal MAP and exact block
coordinate descent) runs in hand-written HIP kernels for gfx950 behind the
C ABI of include/mpq.h (libmpq.so).  This package is the thin binding.
"""
from .binding import (  # noqa: F401
    EXPORTS, LIB_PATH, MPQError, PROF_NAMES, PreparedCodebook, Profile, STATUS, cd, codebook_kind, denoise,
    e8dp_transitions, factor, frontend, gram, greedy, greedy_workspace_bytes, linear_step, load_library, map_codes,
    objective, prepare_codebook, probe_rate, prologue, quantize_layer, quantize_layer_static, rht, vamp_step,
    workspace_bytes,
)
