"""Front-end reference oracle: calibration activations -> the solver's inputs.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this module.  The GPU library
never calls it and shares no code with it.

Plain float64 NumPy.  Passages (the papernotes.org MPQ summary, "Overall
framework" and the hyper-parameter paragraph; the ai.info summary's main
findings on random Hadamard transforms):

  * the layer objective is 1/2 (w - w_hat)^T H (w - w_hat) with the
    calibration Gram matrix H = X^T X, and the solver works in the basis of
    its factorisation H = V diag(s^2) V^T (rank r: the r largest modes);
  * incoherence processing is a random Hadamard transform (RHT): weights and
    activations are rotated by the same orthogonal U = Had_n diag(signs) / sqrt(n),
    which leaves W X^T unchanged and conjugates H -> U H U^T, so the spectrum of
    H (and every quantity that depends on H only through its eigenvalues) is
    unchanged.

Readings (the pages name the RHT but print no construction):
  F1  Had_n is the Sylvester matrix for n = 2^k, and for n = 28 * 2^k the
      Kronecker product Had_28 (x) Had_(2^k) (index j = a * 2^k + b), with
      Had_28 the Paley type II matrix built from the quadratic residues mod 13;
      other n are not supported.  The signs are an input (random +-1 drawn by
      the caller).
  F2  the factorisation keeps the r largest eigenvalues, s = sqrt(max(lambda,
      0)) in descending order, V their unit eigenvectors (the sign of each
      column is free: the solver is invariant under column sign flips).
"""
from __future__ import annotations

import numpy as np


def sylvester(k: int) -> np.ndarray:
    """Had_(2^k) by Sylvester's doubling [[H, H], [H, -H]]."""
    H = np.ones((1, 1))
    for _ in range(k):
        H = np.block([[H, H], [H, -H]])
    return H


def quadratic_character(x: int, q: int) -> int:
    x %= q
    if x == 0:
        return 0
    return 1 if any((y * y) % q == x for y in range(1, q)) else -1


def paley2(q: int) -> np.ndarray:
    """Paley construction II, order 2 (q + 1) for a prime q = 1 mod 4:
    Jacobsthal Q[i][j] = chi(j - i), conference matrix C = [[0, 1^T], [1, Q]],
    Had = C (x) [[1, -1], [-1, -1]] + I (x) [[1, 1], [1, -1]]."""
    Q = np.array([[quadratic_character(j - i, q) for j in range(q)] for i in range(q)], dtype=float)
    C = np.zeros((q + 1, q + 1))
    C[0, 1:] = 1.0
    C[1:, 0] = 1.0
    C[1:, 1:] = Q
    return np.kron(C, np.array([[1.0, -1.0], [-1.0, -1.0]])) + np.kron(np.eye(q + 1), np.array([[1.0, 1.0],
                                                                                               [1.0, -1.0]]))


def hadamard(n: int) -> np.ndarray:
    """Had_n of reading F1."""
    k = 0
    m = n
    while m % 2 == 0 and m > 1:
        m //= 2
        k += 1
    if m == 1:
        return sylvester(k)
    if m == 7 and k >= 2:      # n = 28 * 2^(k-2)
        return np.kron(paley2(13), sylvester(k - 2))
    raise ValueError("RHT size must be 2^k or 28 * 2^k")


def rht_matrix(n: int, signs) -> np.ndarray:
    """U = Had_n diag(signs) / sqrt(n) (orthogonal)."""
    return hadamard(n) * np.asarray(signs, np.float64)[None, :] / np.sqrt(n)


def rht_rows(A, signs) -> np.ndarray:
    """Every row a of A mapped to U a.  Rows longer than 4096 use the Kronecker
    form (Had_28 (x) Had_(2^k)) x = vec over (a, b) of Had_28 X Had_(2^k)^T,
    X[a][b] = x[a 2^k + b], instead of forming U (the same product)."""
    A = np.asarray(A, np.float64)
    n = A.shape[1]
    if n <= 4096:
        return A @ rht_matrix(n, signs).T
    Y = A * np.asarray(signs, np.float64)[None, :]
    if n % 28 == 0 and (n // 28) & (n // 28 - 1) == 0:
        P, S = paley2(13), hadamard(n // 28)
        X = Y.reshape(-1, 28, n // 28)
        out = np.einsum("ac,rcb->rab", P, X) @ S.T
    else:
        H = hadamard(n)
        out = Y @ H.T
    return out.reshape(A.shape) / np.sqrt(n)


def gram(X) -> np.ndarray:
    """H = X^T X of the calibration activations X (N x n)."""
    X = np.asarray(X, np.float64)
    return X.T @ X


def factor(H, r: int):
    """Reading F2: (s, V) of the r largest modes of H (eigh)."""
    lam, U = np.linalg.eigh(np.asarray(H, np.float64))
    order = np.argsort(lam)[::-1][:r]
    return np.sqrt(np.maximum(lam[order], 0.0)), U[:, order]
