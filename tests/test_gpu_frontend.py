"""Parity of the front end (calibration Gram matrix, random Hadamard
transform, factorisation into (s, V)) with the front-end oracle, and of the
whole chain activations -> (W', s, V) -> solve.

Tolerances: H within 1e-12 of max|H| (float32 products are exact in float64;
only the summation order differs); RHT rows within 5e-6 relative (float32
butterflies, log2 n stages); singular values within 1e-6 of the largest (float64
eigenpairs inside, s and V float32 outputs), eigenvectors |<v, v_ref>| >= 1 - 1e-6 on a spectrum with
distinct modes; the solver's objective on the front end's (s, V) equals the
calibration loss 1/2 ||X'(w' - x)||^2 within 1e-5 relative.
"""
import numpy as np
import pytest

from oracle import frontend_oracle as F
from oracle import mpq_oracle as O
from parity_helpers import OBJ_RTOL, dev, host

pytestmark = pytest.mark.gpu


def activations(N, n, seed, spread=3.0):
    g = np.random.default_rng(seed)
    Q, _ = np.linalg.qr(g.standard_normal((n, n)))
    sig = np.exp(-spread * np.arange(n) / n) * (1.0 + 0.5 * g.random(n))
    X = (g.standard_normal((N, n)) * sig[None, :]) @ Q.T
    return np.ascontiguousarray(X.astype(np.float32))


@pytest.mark.parametrize("N,n", [(5000, 256), (4097, 200), (3, 64), (0, 32)])
def test_gram(N, n):
    import post_quantization_solver_amd as mpq
    X = activations(max(N, 1), n, seed=N + n)[:N]
    H = host(mpq.gram(dev(np.ascontiguousarray(X)) if N else dev(np.zeros((0, n), np.float32))))
    ref = F.gram(X)
    err = np.max(np.abs(H - ref)) / max(np.max(np.abs(ref)), 1e-300) if N else np.max(np.abs(H))
    print(f"[gram] N={N} n={n}: max err {err:.2e}", flush=True)
    assert err <= 1e-12
    assert np.array_equal(H, H.T)


@pytest.mark.parametrize("n", [64, 256, 4096, 28 * 32, 28 * 512])
def test_rht(n):
    import post_quantization_solver_amd as mpq
    g = np.random.default_rng(n)
    A = g.standard_normal((9, n)).astype(np.float32)
    signs = g.choice([-1.0, 1.0], size=n).astype(np.float32)
    out = host(mpq.rht(dev(A.copy()), dev(signs)))
    ref = F.rht_rows(A, signs)
    rel = np.max(np.linalg.norm(out - ref, axis=1) / np.linalg.norm(ref, axis=1))
    print(f"[rht] n={n}: max row rel err {rel:.2e}", flush=True)
    assert rel < 5e-6


@pytest.mark.parametrize("n,r", [(256, 256), (256, 100), (200, 37)])
def test_factor(n, r):
    import post_quantization_solver_amd as mpq
    X = activations(3 * n, n, seed=n + r)
    H = F.gram(X)
    s, V = mpq.factor(dev(H.copy()), r)
    s, V = host(s).astype(np.float64), host(V).astype(np.float64)
    s_ref, V_ref = F.factor(H, r)
    ev_err = np.max(np.abs(s - s_ref)) / s_ref[0]
    align = np.min(np.abs(np.sum(V * V_ref, axis=0)))
    resid = np.max(np.abs(H @ V - V * (s * s)[None, :])) / s_ref[0] ** 2
    print(f"[factor] n={n} r={r}: eigenvalues {ev_err:.2e}, min |<v, v_ref>| {align:.8f}, residual {resid:.2e}",
          flush=True)
    assert ev_err < 1e-6
    assert align > 1 - 1e-6
    assert resid < 1e-6


def test_frontend_chain_to_solver():
    """X, W -> RHT -> H -> (s, V) -> quantize_layer: the solver's objective of the
    returned codes is the calibration loss of the rotated problem."""
    import torch
    import mpq_synth as S
    import post_quantization_solver_amd as mpq
    n, N, m = 256, 1024, 12
    X = activations(N, n, seed=81)
    g = np.random.default_rng(82)
    W = g.standard_normal((m, n)).astype(np.float32)
    signs = g.choice([-1.0, 1.0], size=n).astype(np.float32)
    Wr, s, V = mpq.frontend(dev(X), dev(W), signs=dev(signs))
    Xr = F.rht_rows(X, signs)
    assert np.max(np.abs(host(Wr) - F.rht_rows(W, signs))) < 1e-5
    E, a, o = S.scalar_grid(host(Wr), 3)
    out = mpq.quantize_layer(Wr, s, V, E, dev(a), dev(o), T_vamp=4, n_cd=3, diagnostics=True)
    torch.cuda.synchronize()
    codes = host(out["codes"])
    f = host(out["objective"])
    w_np = host(Wr).astype(np.float64)
    for i in range(m):
        x = O.decode(O.row_codewords(E, a[i], o[i]), codes[i], 1)
        loss = 0.5 * float(np.sum((Xr @ (w_np[i] - x)) ** 2))
        assert abs(f[i] - loss) / loss < OBJ_RTOL, (i, f[i], loss)
    print(f"[frontend chain] objective = calibration loss on {m} rows", flush=True)
