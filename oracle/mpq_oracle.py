"""MPQ reference oracle: plain, slow, float64 NumPy.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this module.  The GPU library
never calls it and shares no code with it.

It solves ONE output row at a time, following the MPQ method as stated on
the papernotes.org summary of "MPQ: A Message-Passing View of Post-Training
Quantization" (section "Method": overall framework and flowchart, key
designs 1-3, and the hyper-parameter paragraph).  Notation follows that
page:

  row weights w (n), blocks of size d (B = n / d), product codebook C^B,
  rank-space operator T = diag(s) V^T (r x n), target y~ = T w,
  objective E_w(w_hat) = 1/2 ||y~ - T w_hat||^2 = 1/2 (w - w_hat)^T H (w - w_hat),
  H = V diag(s^2) V^T,
  cavity (r1, gamma1) -> denoiser -> (x_hat1, eta1) -> extrinsic (r2, gamma2)
  -> Gaussian linear module -> (x_hat2, eta2) -> extrinsic (r1', gamma1'),
  inverse temperature beta updated by the empirical-Bayes M-step with damping,
  then marginal MAP and exact block coordinate descent.

Readings where the pages are silent:
  R1  extrinsic updates use scalar per-row precisions (standard VAMP):
      gamma_out = eta - gamma_in,
      r_out = (eta x_hat - gamma_in r_in) / gamma_out.
  R2  if eta1 <= gamma1 the denoiser's posterior is passed through
      (r2 = x_hat1, gamma2 = eta1); the number of such events is counted.
      A safeguard threshold eps >= 0 widens the rule to eta1 <= gamma1 (1 + eps)
      (eps = 0, the default, is R2 itself).
  R3  beta^0 = r / ||T (w - w_rtn)||^2 (the M-step at the RTN point with
      zero posterior variance).
  R4  damping acts on beta itself: beta' = (1 - rho) beta + rho beta_EM.
  R5  order inside an iteration: denoise(r1^t, gamma1^t) -> linear(beta^t)
      -> M-step with u(r2^t), gamma2^t, beta^t.  The final MAP uses
      (r1^T, gamma1^T).
  R8  blocks are contiguous coordinates [b d, (b+1) d), visited in
      ascending b by CD.
  R9  CD accepts strict improvements only; argmin / argmax ties go to the
      lowest codeword index.
  A1  anchored prior (hyper-parameter paragraph: anchor scale tau = 0.2;
      tau -> infinity is the unanchored limit; the form is not printed):
      rho_b(c) proportional to exp(-||c - w_b||^2 / (2 tau^2 a^2)), a Gaussian
      anchor at the row's own weights whose width is tau codebook units
      (a = the row's codebook scale).  It enters the denoiser and the MAP as a
      per-block log-prior; CD minimises the layer objective alone.
  A2  group-wise grids (hyper-parameter paragraph: scalar grids with group
      size 128): the codebook of block b is a_k e + o_k for the column group k
      of g consecutive weights that holds the block (g a multiple of d); a
      row's blocks keep their own group's codewords in every stage.
  G1  (guard) the denoiser's variance sum is floored at
      n * (1e-12 * a)^2, a = the row's codebook scale; it never binds on
      continuous data.
  G2  (guard) a row whose round-to-nearest point already has zero
      objective (zero RTN error, or an RTN error invisible to T) returns its
      RTN codes, objective 0 and +inf precision traces.
  G3  sequential greedy comparator (the ablation's greedy baseline; the
      explainer's worked example scores a block by its error when the later
      blocks compensate exactly, and the MPQ summary's ablation table names
      the greedy LDLQ baseline; no damping is printed): blocks in ascending
      order, each committed to the codeword that minimises the objective with
      the earlier blocks fixed and the later ones at their best continuous
      values, on the damped H + delta I with delta = 0.01 mean(diag H) (the
      damping customary for greedy solvers; it keeps a rank-deficient H
      factorisable; delta = 1 if H = 0).  Its objective is reported on the
      undamped H.
"""
from __future__ import annotations

import numpy as np

VAR_FLOOR_REL = 1e-24          # G1: per-coordinate variance floor, in units of a^2
GREEDY_DAMP = 0.01             # G3: the greedy comparator's damping, relative to mean(diag H)
_CHUNK_ELEMS = 1 << 22         # block chunking for memory only (blocks are independent)


# ----------------------------------------------------------------------------
# codebook helpers
# ----------------------------------------------------------------------------

def row_codewords(E, a, o):
    """Codewords of one row: c = a * e + o for each base codeword e (K x d)."""
    return float(a) * np.asarray(E, dtype=np.float64) + float(o)


class GroupedCodebook:
    """Reading A2: codewords a_k e + o_k of consecutive column groups of g
    weights (the last group may be shorter).  Stage functions given one of
    these in place of a K x d codebook run group by group."""

    def __init__(self, E, a, o, n, d, g):
        a = np.atleast_1d(np.asarray(a, np.float64))
        o = np.atleast_1d(np.asarray(o, np.float64))
        if g <= 0 or g % d:
            raise ValueError("group size must be a positive multiple of d")
        self.d, self.g, self.n = d, g, n
        self.groups = [(c0, min(n, c0 + g), row_codewords(E, a[k], o[k])) for k, c0 in enumerate(range(0, n, g))]
        if len(self.groups) != a.shape[0] or len(self.groups) != o.shape[0]:
            raise ValueError("one (a, o) per group")
        self.scale = float(np.max(np.abs(a)))

    def block_codebooks(self):
        """The codebook of every block, in block order."""
        out = []
        for c0, c1, C in self.groups:
            out += [C] * ((c1 - c0) // self.d)
        return out

    def decode(self, codes):
        """The weights x of the given block codes."""
        Cb = self.block_codebooks()
        return np.concatenate([Cb[b][k] for b, k in enumerate(np.asarray(codes))])


def decode(C, codes, d):
    """x for the block codes under C (K x d codebook or GroupedCodebook)."""
    if isinstance(C, GroupedCodebook):
        return C.decode(codes)
    return C[np.asarray(codes)].reshape(-1)


def _blocks(x, d):
    return np.asarray(x, dtype=np.float64).reshape(-1, d)


def _chunks(B, K, d):
    step = max(1, _CHUNK_ELEMS // max(1, K * d))
    for b0 in range(0, B, step):
        yield b0, min(B, b0 + step)


def sq_dist(Xb, C):
    """||c - x_b||^2 for every block row of Xb (nb x d) and codeword of C (K x d),
    expanded as ||c||^2 - 2 c.x_b + ||x_b||^2 so the cross term is one matrix
    product (float64; the expansion only changes rounding order)."""
    cc = np.einsum("kj,kj->k", C, C)
    xx = np.einsum("bj,bj->b", Xb, Xb)
    return np.maximum(cc[None, :] - 2.0 * (Xb @ C.T) + xx[:, None], 0.0)


def nearest_codeword(x, C, d):
    """Per-block argmin_c ||x_b - c||^2, ties to the lowest index (round to nearest)."""
    if isinstance(C, GroupedCodebook):
        return np.concatenate([nearest_codeword(np.asarray(x)[c0:c1], Cg, d) for c0, c1, Cg in C.groups])
    Xb = _blocks(x, d)
    B, K = Xb.shape[0], C.shape[0]
    out = np.empty(B, dtype=np.int64)
    for b0, b1 in _chunks(B, K, d):
        out[b0:b1] = np.argmin(sq_dist(Xb[b0:b1], C), axis=1)
    return out


# ----------------------------------------------------------------------------
# stage 1: finite-temperature VAMP in rank space
# ----------------------------------------------------------------------------

def block_logits(r1b, gamma1, C, log_prior=None):
    """log q_b(c) up to a constant: log rho_b(c) - gamma1/2 ||c - r1_b||^2
    (key design 1, the blockwise discrete denoiser).  log_prior: one value
    per codeword (K), or one row per block (nb x K)."""
    L = -0.5 * gamma1 * sq_dist(r1b, C)
    if log_prior is not None:
        lp = np.asarray(log_prior, dtype=np.float64)
        L = L + (lp[None, :] if lp.ndim == 1 else lp)
    return L


def anchor_log_prior(wb, lam, C):
    """Reading A1: log rho_b(c) = -lam/2 ||c - w_b||^2 for the blocks wb (nb x d),
    lam = 1 / (tau a)^2."""
    return -0.5 * float(lam) * sq_dist(wb, C)


def anchor_lambda(tau, a):
    """Precision of the anchored prior (reading A1): 1 / (tau a)^2; 0 when unanchored."""
    if tau is None or not np.isfinite(tau) or tau <= 0:
        return 0.0
    return 1.0 / (float(tau) * float(a)) ** 2


def denoise(r1, gamma1, C, d, log_prior=None, return_q=False, anchor=None):
    """Blockwise discrete denoiser (key design 1).

    For every block: q_b(c) = softmax_c of the block logits, posterior mean
    x_hat1_b = sum_c q_b(c) c and the trace of the posterior covariance
    v_b = sum_c q_b(c) ||c - x_hat1_b||^2.  anchor = (w, lam) adds the
    anchored prior of reading A1.  Returns (x_hat1, v, q or None).
    """
    if isinstance(C, GroupedCodebook):
        parts = [denoise(np.asarray(r1)[c0:c1], gamma1, Cg, d, log_prior, False,
                         None if anchor is None else (np.asarray(anchor[0])[c0:c1], anchor[1]))
                 for c0, c1, Cg in C.groups]
        return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]), None
    R = _blocks(r1, d)
    B, K = R.shape[0], C.shape[0]
    Wb = _blocks(anchor[0], d) if anchor is not None else None
    xhat = np.empty_like(R)
    v = np.empty(B)
    q_all = np.empty((B, K)) if return_q else None
    for b0, b1 in _chunks(B, K, d):
        lp = log_prior
        if anchor is not None and anchor[1] > 0:
            lp = anchor_log_prior(Wb[b0:b1], anchor[1], C)
            if log_prior is not None:
                lp = lp + np.asarray(log_prior, dtype=np.float64)[None, :]
        L = block_logits(R[b0:b1], gamma1, C, lp)
        L = L - L.max(axis=1, keepdims=True)
        q = np.exp(L)
        q /= q.sum(axis=1, keepdims=True)
        xb = q @ C
        xhat[b0:b1] = xb
        v[b0:b1] = np.einsum("bk,bk->b", q, sq_dist(xb, C))
        if return_q:
            q_all[b0:b1] = q
    return xhat.reshape(-1), v, q_all


def extrinsic_denoiser_to_linear(r1, gamma1, xhat1, eta1, eps=0.0):
    """Self-feedback removal on the denoiser side (readings R1, R2; eps: the
    safeguard threshold of R2).

    Returns (r2, gamma2, fell_back)."""
    if eta1 > gamma1 * (1.0 + eps):
        gamma2 = eta1 - gamma1
        r2 = (eta1 * xhat1 - gamma1 * r1) / gamma2
        return r2, gamma2, False
    return np.array(xhat1, dtype=np.float64), eta1, True


def rank_target(w, s, V):
    """y~ = T w with T = diag(s) V^T (compact-SVD projection)."""
    return np.asarray(s, np.float64) * (np.asarray(V, np.float64).T @ np.asarray(w, np.float64))


def linear_module(r2, gamma2, beta, ytil, s, V):
    """Gaussian linear module in the SVD basis (key design 1 + highlights:
    no large-matrix inversion).

    x_hat2 = argmin_x beta/2 ||y~ - T x||^2 + gamma2/2 ||x - r2||^2, solved in
    rank space:  u = y~ - s * (V^T r2),  x_hat2 = r2 + V (D * u) with
    D = beta s / (beta s^2 + gamma2).  Posterior precision
    eta2 = n / tr Sigma2,  tr Sigma2 = (n - r)/gamma2 + sum 1/(beta s^2 + gamma2).
    Extrinsic message back to the denoiser (R1):
    gamma1' = eta2 - gamma2,  r1' = (eta2 x_hat2 - gamma2 r2) / gamma1'.
    """
    s = np.asarray(s, np.float64)
    V = np.asarray(V, np.float64)
    n, r = V.shape
    u = ytil - s * (V.T @ r2)
    den = beta * s * s + gamma2
    z = (beta * s / den) * u
    xhat2 = r2 + V @ z
    trace = (n - r) / gamma2 + np.sum(1.0 / den)
    eta2 = n / trace
    gamma1_new = eta2 - gamma2
    r1_new = (eta2 * xhat2 - gamma2 * r2) / gamma1_new
    return dict(u=u, z=z, xhat2=xhat2, eta2=eta2, gamma1=gamma1_new, r1=r1_new)


def beta_em(u, s, beta, gamma2):
    """Empirical-Bayes M-step for the inverse temperature (key design 2):
    1/beta_EM = (1/r) sum_l [ (gamma2/(beta s_l^2+gamma2))^2 u_l^2 + s_l^2/(beta s_l^2+gamma2) ].
    """
    s = np.asarray(s, np.float64)
    den = beta * s * s + gamma2
    inv = np.mean((gamma2 / den) ** 2 * u * u + s * s / den)
    return 1.0 / inv


def damp_beta(beta, beta_new, rho):
    """Reading R4: beta^{t+1} = (1 - rho) beta^t + rho beta_EM."""
    return (1.0 - rho) * beta + rho * beta_new


def vamp_init(w, s, V, C, d):
    """Initial cavity (hyper-parameter paragraph): r1^0 = w,
    gamma1^0 = 1 / MSE(w, w_rtn); beta^0 by reading R3.
    Returns (rtn_codes, gamma1_0, beta_0, mse, ||T (w - w_rtn)||^2)."""
    w = np.asarray(w, np.float64)
    codes = nearest_codeword(w, C, d)
    w_rtn = decode(C, codes, d)
    mse = float(np.mean((w - w_rtn) ** 2))
    res = rank_target(w - w_rtn, s, V)
    nrm2 = float(res @ res)
    gamma1 = 1.0 / mse if mse > 0 else np.inf
    beta = len(s) / nrm2 if nrm2 > 0 else np.inf
    return codes, gamma1, beta, mse, nrm2


def vamp(w, s, V, C, d, T_vamp, damping, a_scale, beta0=None, denoiser=None,
         fixed_beta=False, record=False, anchor_tau=None, safeguard_eps=0.0, log_prior=None):
    """T_vamp iterations of rank-space VAMP with the beta M-step.

    `denoiser(r1, gamma1) -> (x_hat1, v_blocks)` defaults to the discrete
    codebook denoiser; tests plug in a Gaussian prior to pin the message
    passing itself.  Returns a dict with the final (r1, gamma1, beta), the
    traces and the fallback count.
    """
    w = np.asarray(w, np.float64)
    n = w.shape[0]
    ytil = rank_target(w, s, V)
    codes0, gamma1, beta, _, _ = vamp_init(w, s, V, C, d)
    if beta0 is not None:
        beta = float(beta0)
    if denoiser is None:
        anchor = (w, anchor_lambda(anchor_tau, a_scale))
        denoiser = lambda r, g: denoise(r, g, C, d, log_prior=log_prior, anchor=anchor)[:2]  # noqa: E731
    r1 = w.copy()
    tr_beta, tr_g1, tr_g2, tr_eta1 = [beta], [gamma1], [], []
    hist = []
    fallbacks = 0
    floor = n * VAR_FLOOR_REL * float(a_scale) ** 2
    for _ in range(T_vamp):
        if record:
            hist.append(dict(r1=r1.copy(), gamma1=gamma1, beta=beta))
        xhat1, v = denoiser(r1, gamma1)
        eta1 = n / max(float(np.sum(v)), floor)
        r2, gamma2, fb = extrinsic_denoiser_to_linear(r1, gamma1, xhat1, eta1, safeguard_eps)
        fallbacks += int(fb)
        lin = linear_module(r2, gamma2, beta, ytil, s, V)
        if not fixed_beta:
            beta = damp_beta(beta, beta_em(lin["u"], s, beta, gamma2), damping)
        r1, gamma1 = lin["r1"], lin["gamma1"]
        tr_beta.append(beta)
        tr_g1.append(gamma1)
        tr_g2.append(gamma2)
        tr_eta1.append(eta1)
        if record:
            hist[-1].update(xhat1=xhat1, eta1=eta1, r2=r2, gamma2=gamma2, fell_back=fb,
                            eta2=lin["eta2"], xhat2=lin["xhat2"])
    return dict(r1=r1, gamma1=gamma1, beta=beta, beta_tr=np.array(tr_beta),
                gamma1_tr=np.array(tr_g1), gamma2_tr=np.array(tr_g2),
                eta1_tr=np.array(tr_eta1), fallbacks=fallbacks, rtn_codes=codes0,
                history=hist)


# ----------------------------------------------------------------------------
# stage 2: hard decisions
# ----------------------------------------------------------------------------

def map_codes(r1, gamma1, C, d, log_prior=None, anchor=None):
    """Marginal MAP projection (key design 3): x_b^(0) = argmax_c q_b(c)
    evaluated at (r1^T, gamma1^T); ties to the lowest index.  anchor = (w, lam)
    adds the anchored prior of reading A1."""
    if isinstance(C, GroupedCodebook):
        return np.concatenate([map_codes(np.asarray(r1)[c0:c1], gamma1, Cg, d, log_prior,
                                         None if anchor is None else (np.asarray(anchor[0])[c0:c1], anchor[1]))
                               for c0, c1, Cg in C.groups])
    R = _blocks(r1, d)
    B, K = R.shape[0], C.shape[0]
    Wb = _blocks(anchor[0], d) if anchor is not None else None
    out = np.empty(B, dtype=np.int64)
    for b0, b1 in _chunks(B, K, d):
        lp = log_prior
        if anchor is not None and anchor[1] > 0:
            lp = anchor_log_prior(Wb[b0:b1], anchor[1], C)
            if log_prior is not None:
                lp = lp + np.asarray(log_prior, dtype=np.float64)[None, :]
        out[b0:b1] = np.argmax(block_logits(R[b0:b1], gamma1, C, lp), axis=1)
    return out


def block_cd(codes, w, s, V, C, d, n_cd):
    """Exact block coordinate descent (key design 3; hyper-parameter paragraph:
    at most S_CD sweeps, stop after a sweep with no change).

    Keeps the rank-space residual u = y~ - T x.  For block b with
    T_b = diag(s) V[b rows, :]^T, g = T_b^T u and G_b = T_b^T T_b, the change
    of 1/2 ||u - T_b (c - x_b)||^2 is
        dF(c) = 1/2 (c - x_b)^T G_b (c - x_b) - (c - x_b)^T g,
    minimised over the block's codewords (first argmin); the block moves only
    if dF < 0.  Returns (codes, changes per sweep).
    """
    s = np.asarray(s, np.float64)
    V = np.asarray(V, np.float64)
    codes = np.array(codes, dtype=np.int64)
    x = decode(C, codes, d).copy()
    u = rank_target(np.asarray(w, np.float64) - x, s, V)
    B = x.shape[0] // d
    Cb = C.block_codebooks() if isinstance(C, GroupedCodebook) else [C] * B
    changes = []
    for _ in range(n_cd):
        changed = 0
        for b in range(B):
            sl = slice(b * d, (b + 1) * d)
            Tb = s[:, None] * V[sl, :].T          # r x d
            g = Tb.T @ u
            G = Tb.T @ Tb
            D = Cb[b] - x[sl][None, :]            # K x d : c - x_b
            dF = 0.5 * np.einsum("kj,kj->k", D @ G, D) - D @ g
            k = int(np.argmin(dF))
            if dF[k] < 0.0:
                delta = D[k]
                u = u - Tb @ delta
                x[sl] = Cb[b][k]
                codes[b] = k
                changed += 1
        changes.append(changed)
        if changed == 0:
            break
    return codes, changes


def greedy_hessian(s, V, damp=GREEDY_DAMP):
    """H + delta I with H = V diag(s^2) V^T and delta = damp * mean(diag H) (G3);
    delta = 1 when H = 0 (every code then scores alike, and the greedy rounds
    to nearest)."""
    s = np.asarray(s, np.float64)
    V = np.asarray(V, np.float64)
    H = (V * (s * s)[None, :]) @ V.T
    mean_diag = float(np.mean(np.diag(H)))
    return H + (damp * mean_diag if mean_diag > 0 else 1.0) * np.eye(H.shape[0])


def sequential_greedy(w, s, V, C, d, damp=GREEDY_DAMP):
    """Sequential greedy comparator (reading G3), block by block in ascending
    order on f(e) = 1/2 e^T H e, H the damped greedy_hessian, e = w - x.

    With the earlier blocks committed (e_<) and the later ones free, the
    objective as a function of block b is, up to a constant,
        1/2 (e_b - t_b)^T M_b (e_b - t_b),
    where S = H[>=b, >=b], (t_b, t_>) = -S^{-1} H[>=b, <b] e_< is the best
    continuous completion and M_b = ((S^{-1})[b, b])^{-1} the Schur complement
    that leaves block b after eliminating the later blocks.  Block b takes the
    codeword c minimising it at e_b = w_b - c (first argmin).  Returns codes.
    """
    w = np.asarray(w, np.float64)
    n = w.shape[0]
    B = n // d
    H = greedy_hessian(s, V, damp)
    Cb = C.block_codebooks() if isinstance(C, GroupedCodebook) else [C] * B
    e = np.zeros(n)
    codes = np.zeros(B, dtype=np.int64)
    for b in range(B):
        k = int(np.argmin(greedy_block_costs(H, w, e, Cb[b], d, b)))
        codes[b] = k
        e[b * d:(b + 1) * d] = w[b * d:(b + 1) * d] - Cb[b][k]
    return codes


def greedy_block_costs(H, w, e, Cb, d, b):
    """The greedy's cost of every codeword of block b (sequential_greedy):
    e holds the committed errors w - x of the blocks before b (the rest is
    ignored), H the damped greedy_hessian, Cb the block's K x d codebook."""
    n = w.shape[0]
    lo = b * d
    S = H[lo:, lo:]
    rhs = (H[lo:, :lo] @ e[:lo])[:, None]
    unit = np.zeros((n - lo, d))
    unit[:d, :] = np.eye(d)
    X = np.linalg.solve(S, np.hstack([rhs, unit]))
    t = -X[:d, 0]
    M = np.linalg.inv(X[:d, 1:])
    Eb = np.asarray(w, np.float64)[lo:lo + d][None, :] - Cb - t[None, :]   # K x d : e_b(c) - t_b
    return 0.5 * np.einsum("kj,kj->k", Eb @ M, Eb)


def objective(w, x, s, V):
    """1/2 || T (w - x) ||^2 = 1/2 || s * (V^T (w - x)) ||^2."""
    e = rank_target(np.asarray(w, np.float64) - np.asarray(x, np.float64), s, V)
    return 0.5 * float(e @ e)


def codes_objective(w, codes, C, d, s, V):
    return objective(w, decode(C, codes, d), s, V)


# ----------------------------------------------------------------------------
# the whole row
# ----------------------------------------------------------------------------

def solve_row(w, s, V, E, a, o, d, T_vamp, n_cd, damping, beta0=None, record=False, anchor_tau=None, group=0,
              safeguard_eps=0.0, log_prior=None):
    """MPQ on one row: VAMP (T_vamp iterations) -> marginal MAP -> block CD.
    anchor_tau: the anchored prior of reading A1 (None: uniform prior).
    group > 0: group-wise grids of reading A2 (a, o hold one value per group).
    safeguard_eps: the pass-through threshold of reading R2 (0: R2 itself).
    log_prior: log rho(c), one value per base codeword (key design 1's prior
    of the block posterior; None: uniform), used by the denoiser and the
    marginal MAP; CD minimises the objective alone.

    Returns dict(codes, objective, beta_tr, gamma1_tr, gamma2_tr, eta1_tr,
    cd_changes, fallbacks, map_codes, rtn_codes, frozen[, history]).
    """
    w = np.asarray(w, np.float64)
    if group:
        if anchor_tau is not None and np.isfinite(anchor_tau) and anchor_tau > 0:
            raise ValueError("the anchored prior (A1) is defined for one codebook scale per row")
        C = GroupedCodebook(E, a, o, w.shape[0], d, group)
        a = C.scale   # the variance floor's scale (G1) and, per group, no anchor scale
    else:
        C = row_codewords(E, a, o)
    B = w.shape[0] // d
    rtn, gamma1_0, beta_0, mse, nrm2 = vamp_init(w, s, V, C, d)
    if mse == 0.0 or nrm2 == 0.0:   # G2: the RTN point already has zero objective
        inf = np.inf
        return dict(codes=rtn, objective=0.0, beta_tr=np.full(T_vamp + 1, inf),
                    gamma1_tr=np.full(T_vamp + 1, inf), gamma2_tr=np.full(T_vamp, inf),
                    eta1_tr=np.full(T_vamp, inf), cd_changes=[0] * n_cd, fallbacks=0,
                    map_codes=rtn, rtn_codes=rtn, frozen=True, history=[])
    st = vamp(w, s, V, C, d, T_vamp, damping, a, beta0=beta0, record=record, anchor_tau=anchor_tau,
              safeguard_eps=safeguard_eps, log_prior=log_prior)
    mc = map_codes(st["r1"], st["gamma1"], C, d, log_prior=log_prior, anchor=(w, anchor_lambda(anchor_tau, a)))
    codes, changes = block_cd(mc, w, s, V, C, d, n_cd)
    changes = list(changes) + [0] * (n_cd - len(changes))
    out = dict(codes=codes, objective=codes_objective(w, codes, C, d, s, V),
               beta_tr=st["beta_tr"], gamma1_tr=st["gamma1_tr"], gamma2_tr=st["gamma2_tr"],
               eta1_tr=st["eta1_tr"], cd_changes=changes, fallbacks=st["fallbacks"],
               map_codes=mc, rtn_codes=rtn, frozen=False, r1_final=st["r1"],
               history=st["history"])
    assert codes.shape[0] == B
    return out
