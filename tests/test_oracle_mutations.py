"""Plant plausible slips in the oracle (on the CPU) and confirm the pins catch
each one.  Every mutation is applied with monkeypatch and undone afterwards."""
import numpy as np
import pytest

from oracle import mpq_oracle as O
import test_oracle_pins as P

_orig = {k: getattr(O, k) for k in ("denoise", "extrinsic_denoiser_to_linear", "linear_module",
                                     "beta_em", "block_cd", "rank_target", "block_logits", "anchor_log_prior",
                                     "greedy_hessian", "vamp_init")}


def denoise_var_about_r(r1, gamma1, C, d, log_prior=None, return_q=False, anchor=None):
    xh, v, q = _orig["denoise"](r1, gamma1, C, d, log_prior, True, anchor)
    R = np.asarray(r1, float).reshape(-1, d)
    v = np.einsum("bk,bk->b", q, O.sq_dist(R, C))
    return xh, v, (q if return_q else None)


def logits_no_half(r1b, gamma1, C, log_prior=None):
    return -gamma1 * O.sq_dist(r1b, C)


def logits_wrong_sign(r1b, gamma1, C, log_prior=None):
    return 0.5 * gamma1 * O.sq_dist(r1b, C)


def extr_sign(r1, gamma1, xhat1, eta1, eps=0.0):
    if eta1 > gamma1:
        g2 = eta1 - gamma1
        return (eta1 * xhat1 + gamma1 * r1) / g2, g2, False
    return xhat1.copy(), eta1, True


def extr_no_subtract(r1, gamma1, xhat1, eta1, eps=0.0):
    return (eta1 * xhat1 - gamma1 * r1) / eta1, eta1, False


def extr_pass_gamma1(r1, gamma1, xhat1, eta1, eps=0.0):
    """R2 slip: the pass-through hands on gamma1 instead of eta1."""
    r2, g2, fb = _orig["extrinsic_denoiser_to_linear"](r1, gamma1, xhat1, eta1, eps)
    return (r2, gamma1, fb) if fb else (r2, g2, fb)


def extr_pass_r1(r1, gamma1, xhat1, eta1, eps=0.0):
    """R2 slip: the pass-through keeps the cavity mean r1."""
    r2, g2, fb = _orig["extrinsic_denoiser_to_linear"](r1, gamma1, xhat1, eta1, eps)
    return (np.array(r1, dtype=float), g2, fb) if fb else (r2, g2, fb)


def init_gamma_sum(w, s, V, C, d):
    """gamma1^0 = 1 / sum instead of 1 / mean."""
    codes, g1, b0, mse, nrm2 = _orig["vamp_init"](w, s, V, C, d)
    return codes, 1.0 / (mse * len(w)), b0, mse, nrm2


def init_beta_no_r(w, s, V, C, d):
    """beta^0 without the factor r."""
    codes, g1, b0, mse, nrm2 = _orig["vamp_init"](w, s, V, C, d)
    return codes, g1, 1.0 / nrm2, mse, nrm2


def init_beta_n(w, s, V, C, d):
    """beta^0 with n in place of r."""
    codes, g1, b0, mse, nrm2 = _orig["vamp_init"](w, s, V, C, d)
    return codes, g1, len(w) / nrm2, mse, nrm2


def lin_wrong_D(r2, gamma2, beta, ytil, s, V):
    out = _orig["linear_module"](r2, gamma2, beta, ytil, s, V)
    s = np.asarray(s, float)
    V = np.asarray(V, float)
    z = (beta * s * s / (beta * s * s + gamma2)) * out["u"]
    out["xhat2"] = r2 + V @ z
    out["r1"] = (out["eta2"] * out["xhat2"] - gamma2 * r2) / out["gamma1"]
    return out


def lin_no_null_term(r2, gamma2, beta, ytil, s, V):
    out = _orig["linear_module"](r2, gamma2, beta, ytil, s, V)
    s = np.asarray(s, float)
    eta2 = V.shape[0] / np.sum(1.0 / (beta * s * s + gamma2))
    out["eta2"] = eta2
    out["gamma1"] = eta2 - gamma2
    out["r1"] = (eta2 * out["xhat2"] - gamma2 * r2) / out["gamma1"]
    return out


def lin_no_extrinsic(r2, gamma2, beta, ytil, s, V):
    out = _orig["linear_module"](r2, gamma2, beta, ytil, s, V)
    out["r1"] = out["xhat2"].copy()
    out["gamma1"] = out["eta2"]
    return out


def beta_no_trace(u, s, beta, gamma2):
    s = np.asarray(s, float)
    den = beta * s * s + gamma2
    return 1.0 / np.mean((gamma2 / den) ** 2 * u * u)


def beta_not_squared(u, s, beta, gamma2):
    s = np.asarray(s, float)
    den = beta * s * s + gamma2
    return 1.0 / np.mean((gamma2 / den) * u * u + s * s / den)


def cd_sign(codes, w, s, V, C, d, n_cd):
    s = np.asarray(s, float)
    V = np.asarray(V, float)
    codes = np.array(codes)
    x = C[codes].reshape(-1).copy()
    u = O.rank_target(np.asarray(w, float) - x, s, V)
    changes = []
    for _ in range(n_cd):
        ch = 0
        for b in range(x.shape[0] // d):
            sl = slice(b * d, (b + 1) * d)
            Tb = s[:, None] * V[sl, :].T
            g = Tb.T @ u
            G = Tb.T @ Tb
            D = C - x[sl]
            dF = 0.5 * np.einsum("kj,jl,kl->k", D, G, D) + D @ g
            k = int(np.argmin(dF))
            if dF[k] < 0:
                u = u - Tb @ D[k]
                x[sl] = C[k]
                codes[b] = k
                ch += 1
        changes.append(ch)
        if ch == 0:
            break
    return codes, changes


def anchor_wrong_sign(wb, lam, C):
    return -_orig["anchor_log_prior"](wb, lam, C)


def anchor_no_half(wb, lam, C):
    return 2.0 * _orig["anchor_log_prior"](wb, lam, C)


def grouped_blocks_reversed(self):
    out = []
    for c0, c1, C in reversed(self.groups):
        out += [C] * ((c1 - c0) // self.d)
    return out


def greedy_undamped(s, V, damp=O.GREEDY_DAMP):
    return _orig["greedy_hessian"](s, V, 0.0)


def _greedy_slip(euclid=False, t_sign=-1.0):
    def greedy(w, s, V, C, d, damp=O.GREEDY_DAMP):
        w = np.asarray(w, float)
        n = w.shape[0]
        H = O.greedy_hessian(s, V, damp)
        e = np.zeros(n)
        codes = np.zeros(n // d, dtype=np.int64)
        for b in range(n // d):
            lo = b * d
            unit = np.zeros((n - lo, d))
            unit[:d] = np.eye(d)
            X = np.linalg.solve(H[lo:, lo:], np.hstack([(H[lo:, :lo] @ e[:lo])[:, None], unit]))
            t = t_sign * X[:d, 0]
            M = np.eye(d) if euclid else np.linalg.inv(X[:d, 1:])
            Eb = w[lo:lo + d][None, :] - C - t[None, :]
            k = int(np.argmin(np.einsum("kj,kj->k", Eb @ M, Eb)))
            codes[b] = k
            e[lo:lo + d] = w[lo:lo + d] - C[k]
        return codes
    return greedy


greedy_euclidean_metric = _greedy_slip(euclid=True)
greedy_euclidean_metric.__name__ = "greedy_euclidean_metric"
greedy_target_sign = _greedy_slip(t_sign=1.0)
greedy_target_sign.__name__ = "greedy_target_sign"


def rank_target_transposed(w, s, V):
    return np.asarray(s, float) * (np.asarray(V, float) @ np.asarray(w, float))


MUTATIONS = [
    ("denoise", denoise_var_about_r, [P.check_denoiser_limits]),
    ("block_logits", logits_no_half, [P.check_denoiser_limits]),
    ("block_logits", logits_wrong_sign, [P.check_denoiser_limits]),
    ("extrinsic_denoiser_to_linear", extr_sign, [P.check_gaussian_prior_fixed_point]),
    ("extrinsic_denoiser_to_linear", extr_no_subtract, [P.check_gaussian_prior_fixed_point]),
    ("extrinsic_denoiser_to_linear", extr_pass_gamma1, [P.check_r2_branch_hand, P.check_r2_in_vamp]),
    ("extrinsic_denoiser_to_linear", extr_pass_r1, [P.check_r2_branch_hand, P.check_r2_in_vamp]),
    ("vamp_init", init_gamma_sum, [P.check_vamp_init_hand]),
    ("vamp_init", init_beta_no_r, [P.check_vamp_init_hand]),
    ("vamp_init", init_beta_n, [P.check_vamp_init_hand]),
    ("linear_module", lin_wrong_D, [P.check_gaussian_prior_fixed_point, P.check_linear_module_dense]),
    ("linear_module", lin_no_null_term, [lambda: P.check_linear_module_dense(12, 9)]),
    ("linear_module", lin_no_extrinsic, [P.check_gaussian_prior_fixed_point, P.check_linear_module_dense]),
    ("beta_em", beta_no_trace, [P.check_beta_dense]),
    ("beta_em", beta_not_squared, [P.check_beta_dense]),
    ("block_cd", cd_sign, [P.check_cd_bruteforce, P.check_worked_example_mpq]),
    ("rank_target", rank_target_transposed, [P.check_worked_example_mpq, P.check_cd_bruteforce]),
    ("anchor_log_prior", anchor_wrong_sign, [P.check_anchor_prior]),
    ("anchor_log_prior", anchor_no_half, [P.check_anchor_prior]),
    ("GroupedCodebook.block_codebooks", grouped_blocks_reversed, [P.check_grouped_local_minimum]),
    ("greedy_hessian", greedy_undamped, [P.check_greedy_bruteforce]),
    ("sequential_greedy", greedy_euclidean_metric, [P.check_greedy_bruteforce]),
    ("sequential_greedy", greedy_target_sign, [P.check_greedy_bruteforce, P.check_greedy_worked_example]),
]


@pytest.mark.parametrize("name,fn,checks", MUTATIONS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_pins_catch_mutation(monkeypatch, name, fn, checks):
    for chk in checks:
        chk()  # clean oracle passes
    if "." in name:
        cls, attr = name.split(".")
        monkeypatch.setattr(getattr(O, cls), attr, fn)
    else:
        monkeypatch.setattr(O, name, fn)
    caught = 0
    for chk in checks:
        try:
            with np.errstate(all="ignore"):
                chk()
        except (AssertionError, np.linalg.LinAlgError, ValueError, FloatingPointError):
            caught += 1
    assert caught >= 1, f"mutation {name}/{fn.__name__} not caught"
