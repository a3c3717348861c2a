"""Pins of the front-end oracle (calibration Gram matrix, random Hadamard
transform, factorisation into the solver's (s, V)) against closed forms,
library routines and the invariances the pages state; planted slips must fail
them."""
import numpy as np
import pytest
import scipy.linalg

from oracle import frontend_oracle as F
from oracle import mpq_oracle as O


def check_paley28():
    H = F.paley2(13)
    assert H.shape == (28, 28)
    assert set(np.unique(H)) == {-1.0, 1.0}
    assert np.array_equal(H @ H.T, 28.0 * np.eye(28))


def test_paley28_is_hadamard():
    check_paley28()


def check_hadamard_sizes():
    for n in (1, 2, 4, 8, 64, 256, 28, 56, 112, 896):
        H = F.hadamard(n)
        assert H.shape == (n, n)
        assert np.array_equal(H @ H.T, n * np.eye(n)), n
    for n in (2, 16, 128):
        assert np.array_equal(F.hadamard(n), scipy.linalg.hadamard(n))   # Sylvester's construction
    for n in (12, 20, 14, 3):
        with pytest.raises(ValueError):
            F.hadamard(n)


def test_hadamard_sizes():
    check_hadamard_sizes()


def test_hadamard_kronecker_index():
    """For n = 28 * 2^k, entry (a 2^k + b, a' 2^k + b') is Had28[a][a'] Had[b][b']."""
    H = F.hadamard(56)
    P = F.paley2(13)
    S2 = F.sylvester(1)
    for j in range(56):
        for jp in range(0, 56, 5):
            assert H[j, jp] == P[j // 2, jp // 2] * S2[j % 2, jp % 2]


def check_rht_invariances(n=112, N=40, m=5, seed=1):
    g = np.random.default_rng(seed)
    signs = g.choice([-1.0, 1.0], size=n)
    U = F.rht_matrix(n, signs)
    assert np.allclose(U @ U.T, np.eye(n), atol=1e-12)
    X = g.standard_normal((N, n))
    W = g.standard_normal((m, n))
    Xr, Wr = F.rht_rows(X, signs), F.rht_rows(W, signs)
    assert np.allclose(Wr @ Xr.T, W @ X.T, atol=1e-10)                      # W X^T unchanged
    assert np.allclose(F.gram(Xr), U @ F.gram(X) @ U.T, atol=1e-9)         # H -> U H U^T
    ev0 = np.linalg.eigvalsh(F.gram(X))
    ev1 = np.linalg.eigvalsh(F.gram(Xr))
    assert np.allclose(ev0, ev1, atol=1e-9 * ev0.max())                    # spectrum unchanged
    # the signs matter: a different draw is a different rotation
    assert not np.allclose(F.rht_rows(W, signs[::-1]), Wr)


def test_rht_invariances():
    check_rht_invariances()


def check_factor(n=24, N=60, r=24, seed=2):
    g = np.random.default_rng(seed)
    X = g.standard_normal((N, n)) * np.linspace(3.0, 0.1, n)[None, :]
    H = F.gram(X)
    s, V = F.factor(H, r)
    assert np.all(np.diff(s) <= 0) and np.all(s >= 0)
    assert np.allclose(V.T @ V, np.eye(r), atol=1e-12)
    assert np.allclose(H @ V, V * (s * s)[None, :], atol=1e-9 * s[0] ** 2)
    if r == n:
        assert np.allclose((V * (s * s)[None, :]) @ V.T, H, atol=1e-9 * s[0] ** 2)
        # the solver's objective on (s, V) is the calibration loss 1/2 ||X (w - x)||^2
        w = g.standard_normal(n)
        x = g.standard_normal(n)
        assert np.isclose(O.objective(w, x, s, V), 0.5 * np.sum((X @ (w - x)) ** 2), rtol=1e-10)


def test_rht_kronecker_form_matches_matrix():
    """The Kronecker evaluation used for long rows equals the dense U (n = 28 * 256 > 4096)."""
    g = np.random.default_rng(5)
    n = 28 * 256
    signs = g.choice([-1.0, 1.0], size=n)
    A = g.standard_normal((3, n))
    dense = A @ F.rht_matrix(n, signs).T
    assert np.allclose(F.rht_rows(A, signs), dense, atol=1e-10)
    B = g.standard_normal((2, 8192))
    s2 = g.choice([-1.0, 1.0], size=8192)
    assert np.allclose(F.rht_rows(B, s2), B @ F.rht_matrix(8192, s2).T, atol=1e-10)


def test_factor():
    check_factor()
    check_factor(r=10)


def test_factor_rank_deficient():
    """Fewer calibration rows than features: the trailing modes are zero."""
    g = np.random.default_rng(3)
    X = g.standard_normal((6, 16))
    s, V = F.factor(F.gram(X), 16)
    assert np.all(s[6:] < 1e-6 * s[0])
    assert np.allclose((V[:, :6] * (s[:6] ** 2)[None, :]) @ V[:, :6].T, F.gram(X), atol=1e-9)


def test_gram_is_sum_of_outer_products():
    g = np.random.default_rng(4)
    X = g.standard_normal((7, 5))
    ref = sum(np.outer(x, x) for x in X)
    assert np.allclose(F.gram(X), ref, atol=1e-12)


# planted slips --------------------------------------------------------------

def _paley_wrong_kernel(q):
    Q = np.array([[F.quadratic_character(j - i, q) for j in range(q)] for i in range(q)], dtype=float)
    C = np.zeros((q + 1, q + 1))
    C[0, 1:] = 1.0
    C[1:, 0] = 1.0
    C[1:, 1:] = Q
    return np.kron(C, np.array([[1.0, 1.0], [1.0, -1.0]])) + np.kron(np.eye(q + 1), np.array([[1.0, 1.0],
                                                                                             [1.0, -1.0]]))


def _rht_no_scale(n, signs):
    return F.hadamard(n) * np.asarray(signs, float)[None, :]


def _factor_ascending(H, r):
    lam, U = np.linalg.eigh(np.asarray(H, float))
    return np.sqrt(np.maximum(lam[:r], 0.0)), U[:, :r]


@pytest.mark.parametrize("name,fn,checks", [
    ("paley2", _paley_wrong_kernel, [check_paley28, check_hadamard_sizes]),
    ("rht_matrix", _rht_no_scale, [check_rht_invariances]),
    ("factor", _factor_ascending, [lambda: check_factor(r=10)]),
])
def test_pins_catch_frontend_mutation(monkeypatch, name, fn, checks):
    for chk in checks:
        chk()
    monkeypatch.setattr(F, name, fn)
    caught = 0
    for chk in checks:
        try:
            chk()
        except (AssertionError, ValueError):
            caught += 1
    assert caught >= 1
