"""Seeded synthetic layers.

Five named workloads follow the layer shapes the MPQ pages quantize
(Llama-3.2-1B and Llama-3-8B projections, 3/4-bit scalar and 2-bit E8
lattice); real weights and calibration activations are replaced by seeded
draws:

  c1  64 x 256     N(0,1)                     d=1, 8 levels    s_l = l^-0.5          T=8
  c2  2048 x 2048  Laplace(0,1), 1% cols x 8  d=1, 8 levels    s_l = l^-0.6, 16 x10  T=16
  c3  2048 x 8192  N(0,1)                     d=1, 16 levels   s_l = l^-0.5          T=16
  c4  4096 x 4096  N(0,1)                     d=8, E8 65536    s_l = l^-0.6          T=16
  c5  4096 x 14336 Student-t(5)               d=8, E8 65536    s_l = l^-0.7, 32 x10  T=16

All use r = n, damping 0.5 and 3 CD sweeps.  Arrays are drawn in float64 and
rounded to float32; the float32 arrays are what both sides consume.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .codebooks import e8_codebook, scalar_grid, lattice_row_scale

CONFIG_NAMES = ("c1", "c2", "c3", "c4", "c5")


@dataclass
class Layer:
    name: str
    W: np.ndarray          # m x n float32
    s: np.ndarray          # r float32 (singular values)
    V: np.ndarray          # n x r float32, orthonormal columns
    E: np.ndarray          # K x d float32 base codebook
    a: np.ndarray          # m float32 per-row codebook scale (m x G with group-wise grids)
    o: np.ndarray          # m float32 per-row codebook offset (m x G with group-wise grids)
    d: int
    T_vamp: int
    n_cd: int
    damping: float
    meta: dict = field(default_factory=dict)
    group: int = 0         # > 0: grids per group of this many columns (a, o are m x G)

    @property
    def m(self):
        return self.W.shape[0]

    @property
    def n(self):
        return self.W.shape[1]

    @property
    def r(self):
        return self.s.shape[0]

    @property
    def K(self):
        return self.E.shape[0]


def orthogonal(n: int, rng: np.random.Generator, r: int | None = None, device=None) -> np.ndarray:
    """Q factor of the Householder QR of a seeded n x n standard Gaussian.

    Returns the first r columns (default all) as float32.  With a torch
    device other than the CPU the factorisation runs there (rocSOLVER); the
    Gaussian is always drawn on the host from `rng`.
    """
    r = n if r is None else r
    G = rng.standard_normal((n, n))
    if device is not None and str(device) != "cpu":
        import torch
        Q = torch.linalg.qr(torch.from_numpy(G).to(device), mode="reduced").Q
        Q = Q[:, :r].float().cpu().numpy()
    else:
        Q, _ = np.linalg.qr(G)
        Q = Q[:, :r].astype(np.float32)
    return np.ascontiguousarray(Q)


def spectrum(r: int, power: float, lead: int = 0, lead_factor: float = 10.0) -> np.ndarray:
    """s_l = l^-power for l = 1..r, with the first `lead` modes multiplied."""
    l = np.arange(1, r + 1, dtype=np.float64)
    s = l ** (-power)
    if lead:
        s[:lead] *= lead_factor
    return s.astype(np.float32)


def draw_weights(rng, m, n, dist, outlier_frac=0.0, outlier_factor=8.0, outlier_rng=None):
    if dist == "normal":
        W = rng.standard_normal((m, n))
    elif dist == "laplace":
        W = rng.laplace(0.0, 1.0, (m, n))
    elif dist == "t5":
        W = rng.standard_t(5, (m, n))
    else:
        raise ValueError(dist)
    if outlier_frac > 0:
        k = int(np.round(outlier_frac * n))
        cols = (outlier_rng or rng).choice(n, size=k, replace=False)
        W[:, cols] *= outlier_factor
    return np.ascontiguousarray(W.astype(np.float32))


def make_layer(name, m, n, *, seed, dist="normal", d=1, bits=3, K=None, power=0.5,
               lead=0, r=None, T_vamp=16, n_cd=3, damping=0.5, outlier_frac=0.0,
               device=None, W=None, s=None, V=None, group=0, E=None):
    """General seeded layer.  d = 1 -> Min-Max scalar grid with 2^bits levels
    (per row, or per group of `group` columns); d = 8 -> the first K points of
    E8 (K defaults to 65536), or the given K x 8 codebook E."""
    ss = np.random.SeedSequence(seed)
    w_ss, v_ss, o_ss = ss.spawn(3)
    r = n if r is None else r
    if W is None:
        W = draw_weights(np.random.default_rng(w_ss), m, n, dist, outlier_frac,
                         outlier_rng=np.random.default_rng(o_ss))
    if V is None:
        V = orthogonal(n, np.random.default_rng(v_ss), r=r, device=device)
    if s is None:
        s = spectrum(r, power, lead)
    if d == 1:
        E, a, o = scalar_grid(W, bits, group)
    elif d == 8:
        E = e8_codebook(65536 if K is None else K) if E is None else np.ascontiguousarray(E, dtype=np.float32)
        raw_rms = float(np.sqrt((E.astype(np.float64) ** 2).mean()))
        a, o = lattice_row_scale(W, raw_rms)
    else:
        raise ValueError("d must be 1 or 8")
    if group and d != 1:
        raise ValueError("group-wise grids are generated for scalar codebooks")
    return Layer(name, W, s, V, E, a, o, d, T_vamp, n_cd, damping,
                 meta=dict(seed=seed, dist=dist, power=power, lead=lead), group=int(group))


_SPECS = {
    "c1": dict(m=64, n=256, dist="normal", d=1, bits=3, power=0.5, T_vamp=8),
    "c2": dict(m=2048, n=2048, dist="laplace", outlier_frac=0.01, d=1, bits=3,
               power=0.6, lead=16, T_vamp=16),
    "c3": dict(m=2048, n=8192, dist="normal", d=1, bits=4, power=0.5, T_vamp=16),
    "c4": dict(m=4096, n=4096, dist="normal", d=8, power=0.6, T_vamp=16),
    "c5": dict(m=4096, n=14336, dist="t5", d=8, power=0.7, lead=32, T_vamp=16),
}


def make_config(name: str, device=None, group: int = 0) -> Layer:
    """One of the five named workloads (seed 1000 + index); `group` > 0 gives
    a scalar workload group-wise grids of that many columns (same weights)."""
    idx = CONFIG_NAMES.index(name) + 1
    spec = dict(_SPECS[name])
    m = spec.pop("m")
    n = spec.pop("n")
    L = make_layer(name if not group else f"{name}_g{group}", m, n, seed=1000 + idx, device=device, n_cd=3,
                   damping=0.5, group=group, **spec)
    return L


def parity_rows(m: int, count: int = 64) -> np.ndarray:
    """Fixed row subset: every (m // count)-th row (all rows when m <= count)."""
    if m <= count:
        return np.arange(m)
    step = m // count
    return np.arange(0, step * count, step)
