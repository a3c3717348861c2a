"""Pins for the float64 oracle against facts the pages and the mathematics fix.

Each check is written so that a plausible slip in the oracle (a dropped term,
a wrong sign, a swapped precision, a transposed operand) fails at least one
of them; tests/test_oracle_mutations.py plants such slips and confirms it.
"""
import itertools
import math
import os

import numpy as np
import pytest

from oracle import mpq_oracle as O
import mpq_synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def small_problem(seed=0, n=12, r=9, K=4, d=1, power=0.5):
    g = rng(seed)
    Q, _ = np.linalg.qr(g.standard_normal((n, n)))
    V = Q[:, :r]
    s = np.arange(1, r + 1, dtype=float) ** -power
    w = g.standard_normal(n)
    E = np.arange(K, dtype=float).reshape(K, 1) if d == 1 else g.standard_normal((K, d))
    return w, s, V, E


# ----------------------------------------------------------------------------
# denoiser (key design 1): T1, T5
# ----------------------------------------------------------------------------

def check_denoiser_limits():
    """T1 + T5: normalisation, the hard (gamma -> inf) and flat (gamma -> 0)
    limits, and the closed form for a binary codebook {-a, +a}."""
    g = rng(1)
    C = g.standard_normal((7, 3))
    r = g.standard_normal(12)
    _, _, q = O.denoise(r, 0.7, C, 3, return_q=True)
    assert np.allclose(q.sum(1), 1.0, atol=1e-14)
    # gamma -> inf: one-hot at the nearest codeword (brute force), zero variance
    xh, v, q = O.denoise(r, 1e9, C, 3, return_q=True)
    for b in range(4):
        dists = [sum((C[k, j] - r[3 * b + j]) ** 2 for j in range(3)) for k in range(7)]
        k = dists.index(min(dists))
        assert q[b, k] > 1 - 1e-12
        assert np.allclose(xh[3 * b:3 * b + 3], C[k], atol=1e-9)
        assert v[b] < 1e-9
    # gamma -> 0: posterior = prior (uniform): mean of codewords, total variance
    xh, v, _ = O.denoise(r, 1e-14, C, 3)
    mean = C.mean(0)
    tv = ((C - mean) ** 2).sum(1).mean()
    assert np.allclose(xh.reshape(4, 3), mean[None, :], atol=1e-9)
    assert np.allclose(v, tv, rtol=1e-9)
    # binary codebook: x_hat = a tanh(gamma a r), var = a^2 - x_hat^2
    a = 0.8
    Cb = np.array([[-a], [a]])
    r1 = np.linspace(-2, 2, 9)
    for gam in (0.3, 2.0, 11.0):
        xh, v, _ = O.denoise(r1, gam, Cb, 1)
        ref = a * np.tanh(gam * a * r1)
        assert np.allclose(xh, ref, rtol=1e-12, atol=1e-14)
        assert np.allclose(v, a * a - ref * ref, rtol=1e-10, atol=1e-14)
    # asymmetric binary codebook {c0, c1}: q(c1) = sigmoid(gamma (c1-c0)(r - (c0+c1)/2))
    c0, c1 = -0.3, 1.1
    Cb = np.array([[c0], [c1]])
    for gam in (0.5, 4.0):
        xh, v, _ = O.denoise(r1, gam, Cb, 1)
        p1 = 1.0 / (1.0 + np.exp(-gam * (c1 - c0) * (r1 - 0.5 * (c0 + c1))))
        assert np.allclose(xh, c0 + p1 * (c1 - c0), rtol=1e-12)
        assert np.allclose(v, p1 * (1 - p1) * (c1 - c0) ** 2, rtol=1e-10, atol=1e-15)


def check_denoiser_gaussian_limit():
    """A fine uniform grid over a wide range approximates a flat prior: the
    posterior becomes N(r, 1/gamma) per coordinate (mean r, variance 1/gamma)."""
    h = 0.01
    C = (np.arange(-1000, 1001) * h).reshape(-1, 1)
    r = np.array([0.123, -1.77, 2.5])
    gam = 4.0
    xh, v, _ = O.denoise(r, gam, C, 1)
    assert np.allclose(xh, r, atol=1e-9)
    assert np.allclose(v, 1.0 / gam, rtol=1e-6)
    # 2-d version: trace of covariance = d / gamma
    g2 = np.array(list(itertools.product(np.arange(-120, 121) * 0.05, repeat=2)))
    xh, v, _ = O.denoise(np.array([0.31, -0.42]), 9.0, g2, 2)
    assert np.allclose(xh, [0.31, -0.42], atol=1e-9)
    assert abs(v[0] - 2.0 / 9.0) < 1e-6


def test_denoiser_limits():
    check_denoiser_limits()


def test_denoiser_gaussian_limit():
    check_denoiser_gaussian_limit()


def test_map_is_nearest_under_uniform_prior():
    g = rng(2)
    C = g.standard_normal((50, 8))
    r = g.standard_normal(8 * 20)
    for gam in (0.01, 1.0, 300.0):
        mc = O.map_codes(r, gam, C, 8)
        for b in range(20):
            best = min(range(50), key=lambda k: (sum((C[k, j] - r[8 * b + j]) ** 2 for j in range(8)), k))
            assert mc[b] == best
    # ties go to the lowest index
    C2 = np.array([[1.0], [-1.0], [1.0]])
    assert list(O.map_codes(np.array([0.0, 2.0]), 1.0, C2, 1)) == [0, 0]
    assert list(O.nearest_codeword(np.array([0.0, 2.0]), C2, 1)) == [0, 0]


# ----------------------------------------------------------------------------
# linear module and M-step: T2, T3
# ----------------------------------------------------------------------------

def dense_T(s, V):
    return np.diag(s) @ V.T


def check_linear_module_dense(n=12, r=9, seed=3):
    """T3: the rank-space solve equals the dense LMMSE / ridge solve and
    eta2 = n / tr Sigma2 with Sigma2 = (beta T^T T + gamma2 I)^-1 (numpy.linalg)."""
    w, s, V, _ = small_problem(seed, n, r)
    g = rng(seed + 100)
    r2 = g.standard_normal(n)
    beta, gamma2 = 37.0, 2.5
    T = dense_T(s, V)
    ytil = T @ w
    lin = O.linear_module(r2, gamma2, beta, ytil, s, V)
    A = beta * T.T @ T + gamma2 * np.eye(n)
    xh = np.linalg.solve(A, beta * T.T @ ytil + gamma2 * r2)
    Sig = np.linalg.inv(A)
    assert np.allclose(lin["xhat2"], xh, rtol=1e-11, atol=1e-12)
    assert np.isclose(lin["eta2"], n / np.trace(Sig), rtol=1e-12)
    # extrinsic back: gamma1' = eta2 - gamma2, r1' removes the gamma2 r2 share
    assert np.isclose(lin["gamma1"], n / np.trace(Sig) - gamma2, rtol=1e-11)
    assert np.allclose(lin["gamma1"] * lin["r1"], n / np.trace(Sig) * xh - gamma2 * r2, rtol=1e-10)
    # u is the rank-space residual at r2
    assert np.allclose(lin["u"], ytil - T @ r2, rtol=1e-12, atol=1e-13)


def check_beta_dense(n=12, r=9, seed=4):
    """T2: the printed M-step equals [||y~ - T x_hat2||^2 + tr(T Sigma2 T^T)] / r
    evaluated densely (the EM update of a Gaussian noise precision)."""
    w, s, V, _ = small_problem(seed, n, r)
    g = rng(seed + 7)
    r2 = g.standard_normal(n)
    beta, gamma2 = 12.0, 0.8
    T = dense_T(s, V)
    ytil = T @ w
    lin = O.linear_module(r2, gamma2, beta, ytil, s, V)
    A = beta * T.T @ T + gamma2 * np.eye(n)
    Sig = np.linalg.inv(A)
    xh = Sig @ (beta * T.T @ ytil + gamma2 * r2)
    res = ytil - T @ xh
    inv_beta = (res @ res + np.trace(T @ Sig @ T.T)) / r
    assert np.isclose(O.beta_em(lin["u"], s, beta, gamma2), 1.0 / inv_beta, rtol=1e-12)
    # damping is a convex combination in the precision domain
    assert O.damp_beta(2.0, 6.0, 0.5) == 4.0
    assert O.damp_beta(2.0, 6.0, 1.0) == 6.0
    assert O.damp_beta(2.0, 6.0, 0.25) == 3.0


def test_linear_module_matches_dense_solve():
    for n, r in ((12, 9), (10, 10), (7, 3)):
        check_linear_module_dense(n, r)


def test_beta_mstep_matches_dense_em():
    for n, r in ((12, 9), (9, 9)):
        check_beta_dense(n, r)


# ----------------------------------------------------------------------------
# the message passing itself with a Gaussian prior: T4
# ----------------------------------------------------------------------------

def check_gaussian_prior_fixed_point(n=12, r=9, seed=5):
    """T4: with a Gaussian prior N(mu, sigma^2 I) in the denoiser slot (test
    only) expectation propagation is exact, so VAMP's fixed point is the
    ridge solution (beta T^T T + sigma^-2 I)^-1 (beta T^T y~ + sigma^-2 mu),
    the two posterior means agree and eta1 = eta2."""
    w, s, V, _ = small_problem(seed, n, r)
    g = rng(seed + 11)
    mu = g.standard_normal(n)
    sig2 = 0.37
    beta = 5.0
    T = dense_T(s, V)
    ytil = T @ w

    def gauss_denoiser(r1, gamma1):
        prec = gamma1 + 1.0 / sig2
        return (gamma1 * r1 + mu / sig2) / prec, np.full(n, 1.0 / prec)

    C = np.arange(4, dtype=float).reshape(4, 1)
    st = O.vamp(w, s, V, C, 1, 6, 0.5, 1.0, beta0=beta, denoiser=gauss_denoiser,
                fixed_beta=True, record=True)
    ridge = np.linalg.solve(beta * T.T @ T + np.eye(n) / sig2, beta * T.T @ ytil + mu / sig2)
    last = st["history"][-1]
    assert np.allclose(last["xhat2"], ridge, rtol=1e-10, atol=1e-12)
    assert np.allclose(last["xhat1"], ridge, rtol=1e-10, atol=1e-12)
    assert np.isclose(last["eta1"], last["eta2"], rtol=1e-10)
    assert st["fallbacks"] == 0


def test_gaussian_prior_vamp_reaches_ridge():
    for n, r in ((12, 9), (8, 8)):
        check_gaussian_prior_fixed_point(n, r)


# ----------------------------------------------------------------------------
# CD: T6, T7, T9
# ----------------------------------------------------------------------------

def brute_cd(codes, w, s, V, C, d, n_cd):
    """Independent CD: every candidate is scored by the full objective."""
    codes = list(codes)
    B = len(codes)

    def full(cs):
        return O.objective(w, C[np.array(cs)].reshape(-1), s, V)

    changes = []
    for _ in range(n_cd):
        ch = 0
        for b in range(B):
            cur = full(codes)
            vals = []
            for k in range(C.shape[0]):
                trial = list(codes)
                trial[b] = k
                vals.append(full(trial))
            k = int(np.argmin(vals))
            if vals[k] < cur:
                if k != codes[b]:
                    ch += 1
                codes[b] = k
        changes.append(ch)
        if ch == 0:
            break
    return codes, changes


def check_cd_properties(seed=6, n=16, r=16, d=2, K=9):
    """T6: the Mahalanobis form picks the same codeword as F_b; each accepted
    move lowers the objective by exactly -dF; recomputing u from scratch
    matches the carried residual."""
    g = rng(seed)
    Q, _ = np.linalg.qr(g.standard_normal((n, n)))
    V = Q[:, :r]
    s = np.arange(1, r + 1, dtype=float) ** -0.6
    w = g.standard_normal(n)
    C = g.standard_normal((K, d))
    codes = O.nearest_codeword(w, C, d)
    x = C[codes].reshape(-1)
    u = O.rank_target(w - x, s, V)
    for b in range(n // d):
        sl = slice(b * d, (b + 1) * d)
        Tb = s[:, None] * V[sl, :].T
        gb = Tb.T @ u
        G = Tb.T @ Tb
        D = C - x[sl]
        dF = 0.5 * np.einsum("kj,jl,kl->k", D, G, D) - D @ gb
        mu = x[sl] + np.linalg.solve(G, gb)
        maha = 0.5 * np.einsum("kj,jl,kl->k", C - mu, G, C - mu)
        assert np.argmin(dF) == np.argmin(maha)
        assert np.allclose(dF - dF.min(), maha - maha.min(), atol=1e-10)
        k = int(np.argmin(dF))
        before = O.objective(w, x, s, V)
        if dF[k] < 0:
            x[sl] = C[k]
            u = u - Tb @ D[k]
            after = O.objective(w, x, s, V)
            assert np.isclose(after - before, dF[k], rtol=1e-9, atol=1e-12)
            assert np.allclose(u, O.rank_target(w - x, s, V), atol=1e-12)


def test_cd_properties():
    for seed in range(4):
        check_cd_properties(seed)


def check_cd_bruteforce():
    """T7 (i): T_vamp = 0 gives MAP(w) = RTN followed by CD; it equals an
    independent CD that scores candidates by the full objective."""
    for seed in range(3):
        w, s, V, _ = small_problem(seed + 20, n=10, r=10)
        E = np.arange(4, dtype=np.float32).reshape(4, 1)
        a, o = 0.7, -1.05
        C = O.row_codewords(E, a, o)
        res = O.solve_row(w, s, V, E, a, o, 1, 0, 5, 0.5)
        rtn = O.nearest_codeword(w, C, 1)
        assert list(res["map_codes"]) == list(rtn)
        ref_codes, ref_changes = brute_cd(rtn, w, s, V, C, 1, 5)
        assert list(res["codes"]) == list(ref_codes)
        assert res["cd_changes"][:len(ref_changes)] == ref_changes


def test_cd_matches_bruteforce_objective_cd():
    check_cd_bruteforce()


def test_cd_gibbs_zero_temperature_limit():
    """T7 (ii): the Gibbs block conditional p(c_b | rest) ~ exp(-beta F_b(c))
    at beta = 1e12 puts all its mass on the CD choice."""
    w, s, V, _ = small_problem(31, n=8, r=8)
    C = O.row_codewords(np.arange(4, dtype=float).reshape(4, 1), 0.6, -0.9)
    codes = list(O.nearest_codeword(w, C, 1))
    for b in range(8):
        F = []
        for k in range(4):
            t = list(codes)
            t[b] = k
            F.append(O.objective(w, C[np.array(t)].reshape(-1), s, V))
        F = np.array(F)
        logits = -1e12 * F
        p = np.exp(logits - logits.max())
        p /= p.sum()
        new, _ = O.block_cd(codes, w, s, V, C, 1, 1)
        # one sweep: the first block's choice is the conditional argmax
        if b == 0:
            assert int(np.argmax(p)) == new[0] or F[new[0]] == F.min()
        codes[b] = int(np.argmin(F))


def test_tiny_rows_exhaustive():
    """T9: n = 8, 2-bit scalar (4^8 assignments): CD ends at a blockwise local
    minimum (checked when it stopped on a no-change sweep) no worse than its
    MAP start; the gap to the global minimum is reported, not asserted."""
    gaps = []
    for seed in range(6):
        w, s, V, _ = small_problem(seed + 40, n=8, r=8)
        E = np.arange(4, dtype=float).reshape(4, 1)
        lo, hi = w.min(), w.max()
        a = (hi - lo) / 3
        o = -a * np.round(-lo / a)
        C = O.row_codewords(E, a, o)
        res = O.solve_row(w, s, V, E, a, o, 1, 8, 50, 0.5)
        f_final = res["objective"]
        f_map = O.codes_objective(w, res["map_codes"], C, 1, s, V)
        assert f_final <= f_map + 1e-15
        if res["cd_changes"][-1] == 0 or 0 in res["cd_changes"]:
            for b in range(8):
                for k in range(4):
                    t = np.array(res["codes"])
                    t[b] = k
                    assert O.codes_objective(w, t, C, 1, s, V) >= f_final - 1e-14
        allc = np.array(list(itertools.product(range(4), repeat=8)))
        X = C[allc][..., 0]                      # 65536 x 8
        Tm = dense_T(s, V)
        Ev = 0.5 * (((w[None, :] - X) @ Tm.T) ** 2).sum(1)
        gaps.append(f_final - Ev.min())
        assert Ev.min() <= f_final + 1e-14
    assert min(gaps) >= -1e-14


# ----------------------------------------------------------------------------
# the page's worked example: T8
# ----------------------------------------------------------------------------

def load_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split()
            vals[k] = float(v)
    return vals


def worked_example_instance():
    A = -math.sqrt(0.2)
    Bc = math.sqrt(0.22)
    p = 10 * math.sqrt(0.2) + math.sqrt(0.6)
    q = -(10 * math.sqrt(0.22) - 0.6)
    T = np.array([[1.0, 0.0], [10.0, 1.0]])
    U, sv, Vt = np.linalg.svd(T)
    return np.array([A, Bc, p, q]).reshape(4, 1), sv, Vt.T


def test_worked_example_values():
    """T8: the explainer's greedy-vs-deferred example (errors only)."""
    gold = load_golden("worked_example.txt")
    C, s, V = worked_example_instance()
    w = np.zeros(2)

    def F(k1, k2):
        return O.objective(w, np.array([C[k1, 0], C[k2, 0]]), s, V)

    def block1_alone(k):  # error of block 1 when block 2 exactly compensates
        x1 = C[k, 0]
        return 0.5 * x1 * x1

    assert np.isclose(block1_alone(0), gold["block1_alone_A"], atol=1e-12)
    assert np.isclose(block1_alone(1), gold["block1_alone_B"], atol=1e-12)
    assert np.isclose(min(F(0, k) for k in range(4)) - block1_alone(0), gold["best_block2_after_A"], atol=1e-12)
    assert np.isclose(min(F(1, k) for k in range(4)) - block1_alone(1), gold["best_block2_after_B"], atol=1e-12)
    # greedy: commit block 1 by its own error, then the best block 2
    k1 = int(np.argmin([block1_alone(k) for k in range(4)]))
    greedy = min(F(k1, k) for k in range(4))
    assert k1 == 0 and np.isclose(greedy, gold["greedy_total"], atol=1e-12)
    allF = [F(i, j) for i in range(4) for j in range(4)]
    assert np.isclose(min(allF), gold["deferred_total"], atol=1e-12)


def check_worked_example_mpq():
    """MPQ (VAMP -> MAP -> CD) ends at the deferred 0.29, below greedy 0.40."""
    gold = load_golden("worked_example.txt")
    C, s, V = worked_example_instance()
    w = np.zeros(2)
    for T_vamp in (8, 16):
        res = O.solve_row(w, s, V, C, 1.0, 0.0, 1, T_vamp, 3, 0.5)
        assert np.isclose(res["objective"], gold["deferred_total"], atol=1e-12)
        assert list(res["codes"]) == [1, 3]


def test_worked_example_mpq_reaches_deferred_optimum():
    check_worked_example_mpq()


# ----------------------------------------------------------------------------
# metamorphic relations: T11
# ----------------------------------------------------------------------------

def test_scale_invariance():
    """T11 (a, b): W and the codebook scaled by 2^k leave codes unchanged and
    scale gamma and beta by 2^-2k; s scaled by 2^k scales beta by 2^-2k."""
    L = S.make_layer("t", 4, 32, seed=7, d=1, bits=3, T_vamp=6)
    for i in range(2):
        base = O.solve_row(L.W[i], L.s, L.V, L.E, L.a[i], L.o[i], 1, 6, 3, 0.5)
        sc = O.solve_row(4.0 * L.W[i], L.s, L.V, L.E, 4.0 * L.a[i], 4.0 * L.o[i], 1, 6, 3, 0.5)
        assert list(base["codes"]) == list(sc["codes"])
        assert np.allclose(sc["gamma1_tr"], base["gamma1_tr"] / 16.0, rtol=1e-12)
        assert np.allclose(sc["beta_tr"], base["beta_tr"] / 16.0, rtol=1e-12)
        s2 = O.solve_row(L.W[i], 2.0 * L.s, L.V, L.E, L.a[i], L.o[i], 1, 6, 3, 0.5)
        assert list(base["codes"]) == list(s2["codes"])
        assert np.allclose(s2["beta_tr"], base["beta_tr"] / 4.0, rtol=1e-12)
        assert np.allclose(s2["gamma1_tr"], base["gamma1_tr"], rtol=1e-12)


def test_hyperparameter_special_cases():
    """T11 (d): n_cd = 0 returns the MAP codes; T_vamp = 0 starts CD from RTN."""
    L = S.make_layer("t", 3, 24, seed=8, d=1, bits=3)
    i = 1
    C = O.row_codewords(L.E, L.a[i], L.o[i])
    r0 = O.solve_row(L.W[i], L.s, L.V, L.E, L.a[i], L.o[i], 1, 5, 0, 0.5)
    assert list(r0["codes"]) == list(r0["map_codes"])
    r1 = O.solve_row(L.W[i], L.s, L.V, L.E, L.a[i], L.o[i], 1, 0, 0, 0.5)
    assert list(r1["codes"]) == list(O.nearest_codeword(L.W[i], C, 1))
    assert len(r1["beta_tr"]) == 1 and len(r1["gamma2_tr"]) == 0


def test_frozen_row():
    """G2: a row already on its grid returns the RTN codes and objective 0."""
    w = np.array([-1.0, -0.75, 0.5, 0.0], dtype=np.float32)
    E = np.arange(8, dtype=np.float32).reshape(8, 1)
    s = np.ones(4, dtype=np.float32)
    V = np.eye(4, dtype=np.float32)
    res = O.solve_row(w, s, V, E, 0.25, -1.0, 1, 4, 3, 0.5)
    assert res["frozen"] and res["objective"] == 0.0
    assert list(res["codes"]) == [0, 1, 6, 4]


# ----------------------------------------------------------------------------
# initialisation (hyper-parameter paragraph: r1^0 = w, gamma1^0 = 1 / MSE(w,
# w_rtn); reading R3: beta^0 = r / ||T (w - w_rtn)||^2) and the pass-through
# rule of reading R2, pinned on hand-computed numbers
# ----------------------------------------------------------------------------

def init_instance():
    """w = (0.3, -0.7, 1.2, 0.1) on the levels {-1, 0, 1} (base {0, 1, 2},
    scale 1, offset -1): round to nearest gives (0, -1, 1, 0), errors
    (0.3, 0.3, 0.2, 0.1), squares summing to 0.23 (mean 0.0575).  Rank r = 2 < n = 4:
    V = the first two unit vectors, s = (2, 0.5), so T (w - w_rtn) =
    (2 * 0.3, 0.5 * 0.3) = (0.6, 0.15), squared norm 0.3825."""
    w = np.array([0.3, -0.7, 1.2, 0.1])
    E = np.array([[0.0], [1.0], [2.0]])
    C = O.row_codewords(E, 1.0, -1.0)
    V = np.eye(4)[:, :2]
    s = np.array([2.0, 0.5])
    return w, E, C, V, s


def check_vamp_init_hand():
    w, E, C, V, s = init_instance()
    codes, g1, b0, mse, nrm2 = O.vamp_init(w, s, V, C, 1)
    assert list(codes) == [1, 0, 2, 1]
    assert mse == pytest.approx(0.0575, rel=1e-14)
    assert g1 == pytest.approx(1.0 / 0.0575, rel=1e-12)          # 17.391304...
    assert nrm2 == pytest.approx(0.3825, rel=1e-14)
    assert b0 == pytest.approx(2.0 / 0.3825, rel=1e-12)          # r / ||T e||^2 with r = 2 (not n = 4)
    # and as the whole-row solve records them
    res = O.solve_row(w, s, V, E, 1.0, -1.0, 1, 1, 0, 0.5)
    assert res["gamma1_tr"][0] == pytest.approx(1.0 / 0.0575, rel=1e-12)
    assert res["beta_tr"][0] == pytest.approx(2.0 / 0.3825, rel=1e-12)


def test_vamp_init_hand_computed():
    check_vamp_init_hand()


def check_r2_branch_hand():
    """eta1 <= gamma1: pass the posterior through (r2 = xhat1, gamma2 = eta1);
    eta1 > gamma1: gamma2 = eta1 - gamma1 and r2 = (eta1 xhat1 - gamma1 r1) /
    gamma2, here with r1 = (0.2, 0.4), xhat1 = (0.1, 0.5), gamma1 = 5."""
    r1 = np.array([0.2, 0.4])
    x1 = np.array([0.1, 0.5])
    r2, g2, fb = O.extrinsic_denoiser_to_linear(r1, 5.0, x1, 4.0)
    assert fb and g2 == 4.0 and np.array_equal(r2, x1)
    r2, g2, fb = O.extrinsic_denoiser_to_linear(r1, 5.0, x1, 5.0)      # boundary: not positive -> pass through
    assert fb and g2 == 5.0 and np.array_equal(r2, x1)
    r2, g2, fb = O.extrinsic_denoiser_to_linear(r1, 5.0, x1, 6.0)
    assert not fb and g2 == pytest.approx(1.0)
    assert np.allclose(r2, [6 * 0.1 - 5 * 0.2, 6 * 0.5 - 5 * 0.4], rtol=1e-12)   # (-0.4, 1.0)
    # the safeguard threshold widens the rule: 5.2 <= 5 (1 + 0.05)
    r2, g2, fb = O.extrinsic_denoiser_to_linear(r1, 5.0, x1, 5.2, eps=0.05)
    assert fb and g2 == 5.2 and np.array_equal(r2, x1)
    r2, g2, fb = O.extrinsic_denoiser_to_linear(r1, 5.0, x1, 5.2)
    assert not fb and g2 == pytest.approx(0.2)


def check_r2_in_vamp():
    """On the 64 x 256 toy layer the rule fires; every iteration that took it
    carries r2 = xhat1 and gamma2 = eta1 into the linear module, and every
    other one gamma2 = eta1 - gamma1 > 0."""
    L = S.make_config("c1")
    fired = 0
    for i in range(6):
        C = O.row_codewords(L.E, L.a[i], L.o[i])
        st = O.vamp(L.W[i], L.s, L.V, C, 1, L.T_vamp, L.damping, L.a[i], record=True)
        for h in st["history"]:
            if h["fell_back"]:
                fired += 1
                assert h["gamma2"] == h["eta1"] and h["eta1"] <= h["gamma1"]
                assert np.array_equal(h["r2"], h["xhat1"])
            else:
                assert h["gamma2"] == pytest.approx(h["eta1"] - h["gamma1"], rel=1e-12) and h["gamma2"] > 0
        assert st["fallbacks"] == sum(h["fell_back"] for h in st["history"])
    assert fired > 0


def test_r2_branch_hand_computed():
    check_r2_branch_hand()


def test_r2_branch_inside_vamp():
    check_r2_in_vamp()


def test_log_prior_pins():
    """Key design 1's prior rho(c): a constant log-prior is the uniform prior;
    a prior that leaves two levels the others' probability e^-200 confines the
    posterior mean to between them and the MAP to one of them, while the
    prologue (RTN) and CD ignore it."""
    L = S.make_layer("lp", 4, 48, seed=17, d=1, bits=3, power=0.5, T_vamp=5)
    i = 2
    base = O.solve_row(L.W[i], L.s, L.V, L.E, L.a[i], L.o[i], 1, 5, 3, 0.5, record=True)
    const = O.solve_row(L.W[i], L.s, L.V, L.E, L.a[i], L.o[i], 1, 5, 3, 0.5, record=True,
                        log_prior=np.full(L.K, 3.7))
    assert list(base["codes"]) == list(const["codes"])
    assert np.allclose(base["beta_tr"], const["beta_tr"], rtol=1e-12)
    lp = np.full(L.K, -200.0)
    lp[[2, 5]] = 0.0
    res = O.solve_row(L.W[i], L.s, L.V, L.E, L.a[i], L.o[i], 1, 5, 0, 0.5, record=True, log_prior=lp)
    C = O.row_codewords(L.E, L.a[i], L.o[i])
    lo, hi = sorted((C[2, 0], C[5, 0]))
    for h in res["history"]:
        assert np.all(h["xhat1"] >= lo - 1e-9) and np.all(h["xhat1"] <= hi + 1e-9)
    assert set(np.unique(res["map_codes"])) <= {2, 5}
    assert list(res["rtn_codes"]) == list(base["rtn_codes"])


# ----------------------------------------------------------------------------
# anchored prior (reading A1: hyper-parameter paragraph, tau = 0.2; tau -> inf
# is the unanchored limit)
# ----------------------------------------------------------------------------

def check_anchor_prior(seed=11, nb=40, d=2, K=24):
    """Completing the square: a Gaussian anchor of precision lam at w turns
    the block posterior at (r, gamma) into the unanchored one at
    ((gamma r + lam w) / (gamma + lam), gamma + lam) -- the same softmax,
    derived independently of how the oracle adds the log-prior.  Also the
    limits lam = 0 (uniform prior) and lam -> inf (the codeword nearest w)."""
    g = rng(seed)
    C = g.standard_normal((K, d))
    r = g.standard_normal(nb * d) * 1.3
    w = g.standard_normal(nb * d)
    for gamma, lam in ((0.7, 2.5), (4.0, 0.3), (1e-3, 9.0)):
        xa, va, _ = O.denoise(r, gamma, C, d, anchor=(w, lam))
        reff = (gamma * r + lam * w) / (gamma + lam)
        xu, vu, _ = O.denoise(reff, gamma + lam, C, d)
        assert np.allclose(xa, xu, rtol=1e-10, atol=1e-12)
        assert np.allclose(va, vu, rtol=1e-10, atol=1e-12)
        ma = O.map_codes(r, gamma, C, d, anchor=(w, lam))
        assert np.array_equal(ma, O.nearest_codeword(reff, C, d))
    x0, v0, _ = O.denoise(r, 2.0, C, d, anchor=(w, 0.0))
    xu, vu, _ = O.denoise(r, 2.0, C, d)
    assert np.array_equal(x0, xu) and np.array_equal(v0, vu)
    xs, _, _ = O.denoise(r, 2.0, C, d, anchor=(w, 1e6))
    near_w = O.nearest_codeword(w, C, d)
    assert np.allclose(xs, C[near_w].reshape(-1), atol=1e-6)
    assert np.array_equal(O.map_codes(r, 2.0, C, d, anchor=(w, 1e6)), near_w)
    assert O.anchor_lambda(0.2, 0.5) == pytest.approx(100.0)
    assert O.anchor_lambda(None, 0.5) == 0.0


def test_anchor_prior():
    check_anchor_prior()


def test_anchor_whole_row_limits():
    """tau = None and a huge tau give the unanchored solve; with T_vamp = 0 the
    anchored MAP (centred at w, like the cavity) is round to nearest; at the
    pages' tau = 0.2 CD only lowers the objective from the MAP point."""
    L = S.make_layer("anc", 2, 32, seed=12, d=1, bits=3, T_vamp=4)
    i = 0
    C = O.row_codewords(L.E, L.a[i], L.o[i])
    t0 = O.solve_row(L.W[i], L.s, L.V, L.E, L.a[i], L.o[i], 1, 0, 0, 0.5, anchor_tau=0.05)
    assert list(t0["map_codes"]) == list(O.nearest_codeword(L.W[i], C, 1))
    t2 = O.solve_row(L.W[i], L.s, L.V, L.E, L.a[i], L.o[i], 1, 4, 3, 0.5, anchor_tau=0.2)
    f_map = O.codes_objective(L.W[i], t2["map_codes"], C, 1, L.s, L.V)
    assert np.isfinite(t2["objective"]) and t2["objective"] <= f_map + 1e-15
    base = O.solve_row(L.W[i], L.s, L.V, L.E, L.a[i], L.o[i], 1, 4, 3, 0.5)
    loose = O.solve_row(L.W[i], L.s, L.V, L.E, L.a[i], L.o[i], 1, 4, 3, 0.5, anchor_tau=1e9)
    assert list(base["codes"]) == list(loose["codes"])
    assert np.allclose(base["gamma1_tr"], loose["gamma1_tr"], rtol=1e-9)


# ----------------------------------------------------------------------------
# group-wise grids (reading A2: hyper-parameter paragraph, group size 128 for
# scalar grids)
# ----------------------------------------------------------------------------

def _grouped_problem(seed=13, n=12, r=10, g=4, K=4):
    w, s, V, _ = small_problem(seed, n=n, r=r, K=K)
    E = np.arange(K, dtype=float).reshape(K, 1)
    G = n // g
    lo = np.array([w[k * g:(k + 1) * g].min() for k in range(G)])
    hi = np.array([w[k * g:(k + 1) * g].max() for k in range(G)])
    a = (hi - lo) / (K - 1)
    o = lo.copy()
    return w, s, V, E, a, o, g


def check_grouped_identical_groups():
    """Groups that all carry the row's grid reproduce the per-row solve exactly."""
    w, s, V, E, _, _, g = _grouped_problem()
    a0, o0 = 0.37, -0.61
    G = w.shape[0] // g
    base = O.solve_row(w, s, V, E, a0, o0, 1, 4, 3, 0.5)
    grp = O.solve_row(w, s, V, E, np.full(G, a0), np.full(G, o0), 1, 4, 3, 0.5, group=g)
    assert list(base["codes"]) == list(grp["codes"])
    assert base["objective"] == grp["objective"]
    assert np.array_equal(base["gamma1_tr"], grp["gamma1_tr"])


def check_grouped_local_minimum():
    """With distinct group grids: round to nearest uses each group's own grid,
    every final weight lies on its group's grid, and no single-block change to
    a codeword of the block's own grid lowers the objective (CD's fixed point)."""
    w, s, V, E, a, o, g = _grouped_problem()
    res = O.solve_row(w, s, V, E, a, o, 1, 4, 6, 0.5, group=g)
    grids = [a[k] * E[:, 0] + o[k] for k in range(len(a))]
    for j, k in enumerate(res["rtn_codes"]):
        grid = grids[j // g]
        assert k == int(np.argmin(np.abs(grid - w[j])))
    x = np.array([grids[j // g][k] for j, k in enumerate(res["codes"])])
    f0 = O.objective(w, x, s, V)
    assert abs(f0 - res["objective"]) <= 1e-12 * max(1.0, f0)
    if res["cd_changes"][-1] == 0:   # converged within the sweeps
        for j in range(len(x)):
            for c in grids[j // g]:
                y = x.copy()
                y[j] = c
                assert O.objective(w, y, s, V) >= f0 - 1e-12 * max(1.0, f0)


def test_grouped_identical_groups():
    check_grouped_identical_groups()


def test_grouped_local_minimum():
    check_grouped_local_minimum()


def test_mpq_beats_rtn_on_c1_rows():
    """Sanity on the small workload: MPQ never ends above RTN + CD's start."""
    L = S.make_config("c1")
    better = 0
    for i in range(6):
        res = O.solve_row(L.W[i], L.s, L.V, L.E, L.a[i], L.o[i], 1, 8, 3, 0.5)
        C = O.row_codewords(L.E, L.a[i], L.o[i])
        f_rtn = O.codes_objective(L.W[i], res["rtn_codes"], C, 1, L.s, L.V)
        better += res["objective"] < f_rtn
        assert res["objective"] <= O.codes_objective(L.W[i], res["map_codes"], C, 1, L.s, L.V) + 1e-15
    assert better == 6


# ----------------------------------------------------------------------------
# sequential greedy comparator (reading G3)
# ----------------------------------------------------------------------------

def brute_greedy(w, s, V, C, d, damp):
    """The greedy of G3 computed independently: for every block and candidate,
    the later blocks' best continuous values come from a least-squares solve on
    the stacked operator [T; sqrt(delta) I] (whose Gram matrix is H + delta I)."""
    T = dense_T(s, V)
    n = T.shape[1]
    delta = damp * float(np.mean(np.diag(T.T @ T)))
    A = np.vstack([T, math.sqrt(delta) * np.eye(n)])
    e = np.zeros(n)
    codes = []
    for b in range(n // d):
        hi = (b + 1) * d
        best, bk = np.inf, -1
        for k in range(C.shape[0]):
            eb = e.copy()
            eb[b * d:hi] = w[b * d:hi] - C[k]
            r0 = A[:, :hi] @ eb[:hi]
            if hi < n:
                z = np.linalg.lstsq(A[:, hi:], -r0, rcond=None)[0]
                r0 = r0 + A[:, hi:] @ z
            cost = 0.5 * float(r0 @ r0)
            if bk < 0 or cost < best - 1e-12 * abs(best):
                best, bk = cost, k
        codes.append(bk)
        e[b * d:(b + 1) * d] = w[b * d:(b + 1) * d] - C[bk]
    return np.array(codes)


def check_greedy_bruteforce():
    for seed, n, r, d, K, damp, pw in ((21, 6, 6, 1, 5, 0.0, 0.5), (22, 6, 4, 1, 5, 0.01, 0.5),
                                       (23, 8, 8, 2, 6, 0.0, 0.5), (24, 8, 5, 2, 6, 0.01, 0.5),
                                       (25, 8, 8, 2, 6, 0.3, 0.5), (26, 12, 12, 4, 24, 0.0, 2.0),
                                       (27, 12, 9, 4, 24, 0.01, 2.0)):
        w, s, V, _ = small_problem(seed, n=n, r=r, d=d, power=pw)
        C = rng(seed + 100).standard_normal((K, d))
        got = O.sequential_greedy(w, s, V, C, d, damp=damp)
        ref = brute_greedy(w, s, V, C, d, damp)
        assert list(got) == list(ref), (seed, got, ref)


def test_greedy_matches_least_squares_bruteforce():
    check_greedy_bruteforce()


def check_greedy_worked_example():
    """The explainer's greedy commits block 1 by its own error with block 2
    compensating (A, 0.10) and ends at the printed greedy total 0.40."""
    gold = load_golden("worked_example.txt")
    C, s, V = worked_example_instance()
    w = np.zeros(2)
    codes = O.sequential_greedy(w, s, V, C, 1, damp=0.0)
    assert codes[0] == 0
    assert np.isclose(O.codes_objective(w, codes, C, 1, s, V), gold["greedy_total"], atol=1e-12)


def test_greedy_worked_example():
    check_greedy_worked_example()


def test_greedy_uncoupled_is_round_to_nearest():
    """Diagonal H (V = I): no coupling, so the greedy is round to nearest (d = 1)."""
    g = rng(31)
    n = 10
    w = g.standard_normal(n)
    s = np.abs(g.standard_normal(n)) + 0.1
    E = np.arange(6, dtype=float).reshape(6, 1) * 0.7 - 1.5
    codes = O.sequential_greedy(w, s, np.eye(n), E, 1)
    assert list(codes) == list(O.nearest_codeword(w, E, 1))


def test_greedy_zero_operator_is_round_to_nearest():
    """s = 0 (H = 0): the damping alone remains, so the greedy rounds to nearest."""
    g = rng(33)
    n = 8
    w = g.standard_normal(n)
    Q, _ = np.linalg.qr(g.standard_normal((n, n)))
    E = np.arange(5, dtype=float).reshape(5, 1) * 0.6 - 1.2
    codes = O.sequential_greedy(w, np.zeros(n), Q, E, 1)
    assert list(codes) == list(O.nearest_codeword(w, E, 1))


def test_greedy_last_block_is_best_response():
    """Undamped, the last block has no later blocks to compensate: its code is
    the exact best response to the committed others (CD's block rule)."""
    w, s, V, _ = small_problem(32, n=12, r=12, d=2)
    C = rng(132).standard_normal((7, 2))
    codes = O.sequential_greedy(w, s, V, C, 2, damp=0.0)
    x = C[codes].reshape(-1)
    f = [O.objective(w, np.concatenate([x[:-2], C[k]]), s, V) for k in range(7)]
    assert int(np.argmin(f)) == codes[-1]
