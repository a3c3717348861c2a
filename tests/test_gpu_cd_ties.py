"""Block CD on exact ties among three or more codewords.

With H = I (V = I, s = 1), a = 1, o = 0 and the first 241 points of E8 (the
origin and the 240 roots), a block's change of the objective is
dF(c) = 1/2 ||c - w||^2 - 1/2 ||x - w||^2, so CD moves each block to the
nearest codeword of w.  Every quantity is a small dyadic number, exact in
float32 and float64 on both sides, so the weights below put the nearest
codewords at exactly equal distance:

  (1, 1, 1, 0, 0, 0, 0, 0)      3 integer roots at distance^2 1
  (1, 1, 1, 1, 0, 0, 0, 0)      6 integer and 8 half-integer roots at 2
  (1, 0, 0, 0, 0, 0, 0, 0)      the origin and 14 roots at 1
  (0, 0, 0, 0, 0, 1, 1, 1)      3 integer roots at 1, late in the order
  (-1, -1, -1, 0, 0, 0, 0, 0)   3 integer roots at 1, negative
  (1/2 x 6, 0, 0)               2 half-integer roots at 1/2

The key-design-3 rule (first argmin of dF, move on a strict decrease) picks
the lowest index among them; the GPU's codes must equal the oracle's.
"""
import numpy as np
import pytest

import mpq_synth as S
from oracle import mpq_oracle as O
from parity_helpers import dev, host

pytestmark = pytest.mark.gpu

TIES = [
    [1, 1, 1, 0, 0, 0, 0, 0],
    [1, 1, 1, 1, 0, 0, 0, 0],
    [1, 0, 0, 0, 0, 0, 0, 0],
    [0, 0, 0, 0, 0, 1, 1, 1],
    [-1, -1, -1, 0, 0, 0, 0, 0],
    [0.5, 0.5, 0.5, 0.5, 0.5, 0.5, 0, 0],
]


def index_of(E, x):
    hit = np.where((E == np.asarray(x, np.float32)[None, :]).all(1))[0]
    assert len(hit) == 1
    return int(hit[0])


def tie_layer(nblocks):
    """Rows of the tie weights (each block one of them, cycled), starting from
    a codeword far from every one of them."""
    E = S.e8_codebook(241)
    m = len(TIES)
    n = 8 * nblocks
    W = np.zeros((m, n), np.float32)
    for i in range(m):
        for b in range(nblocks):
            W[i, 8 * b:8 * b + 8] = TIES[(i + b) % len(TIES)]
    far = [index_of(E, [-1, 0, 0, 0, 0, 0, 0, 1]), index_of(E, [1, 0, 0, 0, 0, 0, 0, -1])]
    codes0 = np.zeros((m, nblocks), np.int32)
    for i in range(m):
        for b in range(nblocks):
            w = W[i, 8 * b:8 * b + 8]
            # the start: whichever of the two far codewords is farther from the block's weights
            d = [float(((E[k] - w) ** 2).sum()) for k in far]
            codes0[i, b] = far[int(np.argmax(d))]
    return E, W, codes0


@pytest.mark.parametrize("nblocks", [1, 3, 40])
def test_cd_exact_ties_take_the_lowest_index(nblocks):
    import torch
    import post_quantization_solver_amd as mpq
    E, W, codes0 = tie_layer(nblocks)
    m, n = W.shape
    s = np.ones(n, np.float32)
    V = np.eye(n, dtype=np.float32)
    a = np.ones(m, np.float32)
    o = np.zeros(m, np.float32)
    print(f"[ties] {m} rows x {nblocks} blocks", flush=True)
    ref = []
    for i in range(m):
        C = O.row_codewords(E, a[i], o[i])
        codes, ch = O.block_cd(codes0[i], W[i], s, V, C, 8, 1)
        ref.append(codes)
    ref = np.stack(ref)
    # sanity: the oracle moved every block to one of its tied nearest codewords, the lowest index
    for i in range(m):
        for b in range(nblocks):
            d = ((E - W[i, 8 * b:8 * b + 8][None, :]) ** 2).sum(1)
            assert ref[i, b] == int(np.flatnonzero(d == d.min())[0])
    cb = mpq.prepare_codebook(E)
    codes = dev(codes0)
    mpq.cd(dev(W), dev(s), dev(V), cb, dev(a), dev(o), codes, n_cd=1)
    torch.cuda.synchronize()
    got = host(codes)
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:8]
