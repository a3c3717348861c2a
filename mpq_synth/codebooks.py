"""Base codebooks and per-row affine parameters.

Every codebook is encoded the same way: a base table E (K x d, float32) shared
by all rows plus a per-row scale a_i and offset o_i, so that row i's codewords
are  c = a_i * e + o_i * 1  for e in E.

* Scalar grids (d = 1): E = {0, 1, ..., K-1}; a_i and o_i come from the
  Min-Max rule (scale = (max - min) / (2^k - 1), integer zero-point
  z = round(-min / scale)) stated on the NeUQI notes page ("Min-Max"
  initialisation of scale and zero-point).  Levels are a_i * (q - z_i).
* E8 lattice (d = 8, K = 65536): the 65536 lowest-norm points of E8 in raw
  half-integer coordinates (exact in bfloat16), ordered by
  (squared norm, x1, ..., x8) ascending.  The MPQ summary only fixes d = 8
  and M_b = 2^16 for the E8P12 setting (hyper-parameter paragraph); the
  truncation and tie order are this package's reading.
"""
from __future__ import annotations

import numpy as np

# RMS over all 65536 x 8 entries of the raw truncated E8 table:
# sqrt(595860 / 524288).  Checked against the enumerated table in tests.
E8_RAW_RMS = float(np.sqrt(595860.0 / 524288.0))


def _e8_points_norm2_at_most(max_norm2: int) -> np.ndarray:
    """All E8 points with squared norm <= max_norm2 (unordered), float64.

    E8 = {x in Z^8 or (Z + 1/2)^8 : sum(x) even}.
    """
    lim = int(np.floor(np.sqrt(max_norm2)))
    ints = np.arange(-lim, lim + 1, dtype=np.int64)
    grid = np.stack(np.meshgrid(*([ints] * 8), indexing="ij"), -1).reshape(-1, 8)
    keep = ((grid * grid).sum(1) <= max_norm2) & (grid.sum(1) % 2 == 0)
    integer_pts = grid[keep].astype(np.float64)

    # half-integer coordinates: 2x is odd; |x| <= sqrt(max_norm2 - 7/4)
    hlim = np.sqrt(max_norm2 - 7 * 0.25)
    odd = np.arange(-int(2 * hlim) - 1, int(2 * hlim) + 2, dtype=np.int64)
    odd = odd[(odd % 2 != 0) & (np.abs(odd) <= 2 * hlim)]
    g2 = np.stack(np.meshgrid(*([odd] * 8), indexing="ij"), -1).reshape(-1, 8)
    # sum(x) = sum(2x)/2 must be an even integer  <=>  sum(2x) % 4 == 0
    keep2 = ((g2 * g2).sum(1) <= 4 * max_norm2) & (g2.sum(1) % 4 == 0)
    half_pts = g2[keep2].astype(np.float64) / 2.0
    return np.concatenate([integer_pts, half_pts], 0)


def e8_codebook(K: int = 65536) -> np.ndarray:
    """First K points of E8 in (norm^2, x1..x8) ascending order, float32 (K x 8)."""
    max_norm2 = 12
    while True:
        pts = _e8_points_norm2_at_most(max_norm2)
        if len(pts) >= K:
            break
        max_norm2 += 2
    n2 = (pts * pts).sum(1)
    keys = tuple(pts[:, j] for j in range(7, -1, -1)) + (n2,)
    order = np.lexsort(keys)
    return np.ascontiguousarray(pts[order][:K].astype(np.float32))


def scalar_grid(W: np.ndarray, bits: int, group: int = 0):
    """Min-Max uniform grid per row, or per group of `group` consecutive columns.

    Returns (E, a, o): E = arange(2^bits) as (K, 1) float32, and float32 a
    (scale) and o (= -scale * zero_point), shape (m,) per row or (m, G) per
    group.  A constant row or group gets scale 1 so its grid stays well defined.
    """
    K = 1 << bits
    W64 = np.asarray(W, dtype=np.float64)
    if group:
        m, n = W64.shape
        G = (n + group - 1) // group
        lo = np.stack([W64[:, k * group:(k + 1) * group].min(1) for k in range(G)], axis=1)
        hi = np.stack([W64[:, k * group:(k + 1) * group].max(1) for k in range(G)], axis=1)
    else:
        lo = W64.min(1)
        hi = W64.max(1)
    scale = (hi - lo) / (K - 1)
    scale = np.where(scale > 0, scale, 1.0)
    zero = np.round(-lo / scale)  # numpy rounds half to even
    E = np.arange(K, dtype=np.float32).reshape(K, 1)
    return E, scale.astype(np.float32), (-scale * zero).astype(np.float32)


def lattice_row_scale(W: np.ndarray, raw_rms: float = E8_RAW_RMS):
    """Per-row scale RMS(w) / RMS(E_raw) and zero offset (float32)."""
    W64 = np.asarray(W, dtype=np.float64)
    rms = np.sqrt((W64 * W64).mean(1))
    rms = np.where(rms > 0, rms, 1.0)
    a = (rms / raw_rms).astype(np.float32)
    return a, np.zeros_like(a)
