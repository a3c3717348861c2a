"""ctypes binding of libmpq.so (the C ABI in include/mpq.h).

Argument marshalling only: every step of the solve runs in the library's HIP
kernels.  Tensors are torch tensors on the GPU (float32 inputs, float64 VAMP
state, int32 codes; contiguous); a base codebook is a CPU float32 tensor or
numpy array, prepared once into device tables by `prepare_codebook` (the entry
points also accept the raw codebook and prepare it on the spot).  Work is
enqueued on torch's current stream.  If the library is missing or fails to
load, every call raises -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmpq.so")

STATUS = {
    0: "MPQ_OK", -1: "MPQ_ENULL", -2: "MPQ_ESHAPE", -3: "MPQ_EPARAM",
    -4: "MPQ_EUNSUPPORTED", -5: "MPQ_EWORKSPACE", -6: "MPQ_EHIP", -7: "MPQ_ESOLVER",
    -8: "MPQ_ENONFINITE", -9: "MPQ_EHOST",
}

EXPORTS = ("mpq_workspace_bytes", "mpq_strerror", "mpq_codebook_bytes", "mpq_codebook_prepare",
           "mpq_profiler_create", "mpq_profiler_destroy", "mpq_quantize_layer", "mpq_quantize_layer_static",
           "mpq_prologue", "mpq_denoise",
           "mpq_vamp_step", "mpq_linear_step", "mpq_map", "mpq_cd", "mpq_objective", "mpq_greedy",
           "mpq_greedy_workspace_bytes", "mpq_gram_workspace_bytes", "mpq_gram", "mpq_rht",
           "mpq_factor_workspace_bytes", "mpq_factor", "mpq_codebook_kind", "mpq_hip_error_name",
           "mpq_e8dp_transitions", "mpq_probe_rate")


class MPQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        detail = _strerror(status)
        if status == -6:
            try:
                detail += ": " + load_library().mpq_hip_error_name().decode()
            except Exception:  # noqa: BLE001 - only used to decorate an error message
                pass
        super().__init__(f"{what} failed: {STATUS.get(status, status)} ({detail})")


F_FIXED_BETA = 1
F_PROFILE = 2
F_NO_E8DP = 4
F_PROFILE_SAMPLED = 8
F_NO_E8_DECODE = 16
F_CHECK_FINITE = 32
F_LINEAR_F64 = 64
DIGITS_DEFAULT = 5   # MPQ_DIGITS_DEFAULT: digits per operand entry of the int8 digit products
PROF_NAMES = ("prologue", "denoise", "extrinsic", "linear1", "beta", "linear2", "map", "cd_gemm", "cd_search",
              "other", "denoise_exact", "cd_score", "split")
PROF_COUNT = len(PROF_NAMES)


class Codebook(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int64), ("d", ctypes.c_int64), ("kind", ctypes.c_int32),
                ("e8_qlast", ctypes.c_int32), ("e8_last2", ctypes.c_int32 * 8), ("tables", ctypes.c_void_p),
                ("magic", ctypes.c_uint64)]


class Options(ctypes.Structure):
    _fields_ = [("beta0", ctypes.c_float), ("flags", ctypes.c_uint32), ("safeguard_eps", ctypes.c_float),
                ("anchor_tau", ctypes.c_float), ("anchor_w", ctypes.c_void_p), ("log_prior", ctypes.c_void_p),
                ("group", ctypes.c_int64),
                ("profiler", ctypes.c_void_p), ("prof_mask", ctypes.c_uint32),
                ("prof_ms", ctypes.POINTER(ctypes.c_double)), ("prof_launches", ctypes.POINTER(ctypes.c_int64)),
                ("map_codes", ctypes.c_void_p), ("objective", ctypes.c_void_p), ("fallbacks", ctypes.c_void_p),
                ("sweeps", ctypes.c_void_p), ("digits", ctypes.c_int32)]


class PreparedCodebook:
    """A codebook's device tables (mpq_codebook_prepare) and its host copy."""

    def __init__(self, cb, device="cuda"):
        import torch
        E = _host_codebook(cb)
        self.E = E
        self.K, self.d = E.shape
        lib = load_library()
        nb = int(lib.mpq_codebook_bytes(self.K, self.d))
        if nb == 0:
            raise MPQError(-2, "mpq_codebook_bytes")
        self.tables = torch.empty(nb, dtype=torch.uint8, device=device)
        self.struct = Codebook()
        rc = lib.mpq_codebook_prepare(E.ctypes.data_as(ctypes.c_void_p), self.K, self.d, _ptr(self.tables), nb,
                                      _stream(), ctypes.byref(self.struct))
        _check(rc, "mpq_codebook_prepare")

    @property
    def kind(self) -> str:
        return "e8_prefix" if self.struct.kind == 1 else "generic"

    def ref(self):
        return ctypes.byref(self.struct)


def prepare_codebook(cb, device="cuda") -> PreparedCodebook:
    """Prepare a base codebook (K x d, host) once into device tables."""
    return cb if isinstance(cb, PreparedCodebook) else PreparedCodebook(cb, device)


class Profile:
    """Host accumulators for the library's per-category event timing, with
    the event pairs (an mpq_profiler) created once.  sampled: time one CD
    scoring launch in 32 and price the rest at their mean
    (MPQ_F_PROFILE_SAMPLED)."""

    def __init__(self, categories=PROF_NAMES, sampled=False, capacity=4096):
        self.sampled = bool(sampled)
        self.ms = (ctypes.c_double * PROF_COUNT)()
        self.launches = (ctypes.c_int64 * PROF_COUNT)()
        self.mask = 0
        for c in categories:
            self.mask |= 1 << PROF_NAMES.index(c)
        self._lib = load_library()
        self.handle = ctypes.c_void_p()
        _check(self._lib.mpq_profiler_create(int(capacity), ctypes.byref(self.handle)), "mpq_profiler_create")

    def reset(self):
        for k in range(PROF_COUNT):
            self.ms[k] = 0.0
            self.launches[k] = 0

    def as_dict(self):
        return {nm: (float(self.ms[k]), int(self.launches[k])) for k, nm in enumerate(PROF_NAMES)
                if self.mask >> k & 1}

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            self._lib.mpq_profiler_destroy(h)
            self.handle = ctypes.c_void_p()


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmpq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m post_quantization_solver_amd.build`")
    # The library registers its GPU code when it is loaded; with a GPU present,
    # initialise the runtime first so that registration does not happen inside
    # the loader (where the runtime's own start-up fails and every later launch
    # from the library reports hipErrorNoDevice).
    try:
        import torch
        if torch.cuda.is_available():
            torch.cuda.init()
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    F = ctypes.c_float
    SZ = ctypes.c_size_t
    OPT = ctypes.POINTER(Options)
    CB = ctypes.POINTER(Codebook)
    lib.mpq_workspace_bytes.argtypes = [I64, I64, I64, I64, I64]
    lib.mpq_workspace_bytes.restype = SZ
    lib.mpq_strerror.argtypes = [I]
    lib.mpq_strerror.restype = ctypes.c_char_p
    lib.mpq_codebook_bytes.argtypes = [I64, I64]
    lib.mpq_codebook_bytes.restype = SZ
    lib.mpq_codebook_prepare.argtypes = [P, I64, I64, P, SZ, P, CB]
    lib.mpq_profiler_create.argtypes = [I, ctypes.POINTER(ctypes.c_void_p)]
    lib.mpq_profiler_destroy.argtypes = [P]
    lib.mpq_profiler_destroy.restype = None
    lib.mpq_quantize_layer.argtypes = [P, I64, I64, P, P, I64, CB, P, P, I, I, F, OPT, P, P, P, P, P, P, SZ, P]
    lib.mpq_quantize_layer_static.argtypes = [P, I64, I64, P, P, I64, CB, P, P, I, I, F, OPT, P, P, P, P, P, P]
    lib.mpq_prologue.argtypes = [P, I64, I64, P, P, I64, CB, P, P, OPT, P, P, P, P, SZ, P]
    lib.mpq_denoise.argtypes = [P, P, I64, I64, CB, P, P, OPT, P, P, P, SZ, P]
    lib.mpq_vamp_step.argtypes = [P, P, P, P, I64, I64, P, P, I64, CB, P, P, F, OPT, P, P, P, P, P, P, SZ, P]
    lib.mpq_linear_step.argtypes = [P, P, P, P, I64, I64, P, P, I64, F, OPT, P, P, P, SZ, P]
    lib.mpq_map.argtypes = [P, P, I64, I64, CB, P, P, OPT, P, P, SZ, P]
    lib.mpq_cd.argtypes = [P, I64, I64, P, P, I64, CB, P, P, I, OPT, P, P, P, SZ, P]
    lib.mpq_objective.argtypes = [P, I64, I64, P, P, I64, CB, P, P, OPT, P, P, P, SZ, P]
    lib.mpq_greedy.argtypes = [P, I64, I64, P, P, I64, CB, P, P, OPT, P, P, SZ, P]
    lib.mpq_greedy_workspace_bytes.argtypes = [I64, I64, I64, I64, I64]
    lib.mpq_greedy_workspace_bytes.restype = SZ
    lib.mpq_gram_workspace_bytes.argtypes = [I64]
    lib.mpq_gram_workspace_bytes.restype = SZ
    lib.mpq_gram.argtypes = [P, I64, I64, P, P, SZ, P]
    lib.mpq_rht.argtypes = [P, I64, I64, P, P]
    lib.mpq_factor_workspace_bytes.argtypes = [I64]
    lib.mpq_factor_workspace_bytes.restype = SZ
    lib.mpq_factor.argtypes = [P, I64, I64, P, P, P, SZ, P]
    lib.mpq_codebook_kind.argtypes = [P, I64, I64]
    lib.mpq_e8dp_transitions.argtypes = [P, I64]
    lib.mpq_e8dp_transitions.restype = I64
    lib.mpq_hip_error_name.argtypes = []
    lib.mpq_hip_error_name.restype = ctypes.c_char_p
    lib.mpq_probe_rate.argtypes = [I, P, SZ, ctypes.POINTER(ctypes.c_double), P]
    for name in EXPORTS[2:]:
        if name.endswith("_bytes") or name in ("mpq_hip_error_name", "mpq_e8dp_transitions", "mpq_profiler_destroy"):
            continue
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def _strerror(status: int) -> str:
    try:
        return load_library().mpq_strerror(int(status)).decode()
    except Exception:  # noqa: BLE001 - only used to decorate an error message
        return "?"


def codebook_kind(cb) -> str:
    """'e8_prefix' if the codebook is the first K points of E8 in (norm, lex)
    order (the forward-backward denoiser applies), else 'generic'."""
    E = _host_codebook(cb.E if isinstance(cb, PreparedCodebook) else cb)
    rc = load_library().mpq_codebook_kind(E.ctypes.data_as(ctypes.c_void_p), E.shape[0], E.shape[1])
    if rc < 0:
        raise MPQError(rc, "mpq_codebook_kind")
    return "e8_prefix" if rc == 1 else "generic"


def e8dp_transitions(cb) -> int:
    """Valid transitions of an E8-prefix codebook's automaton (0 otherwise)."""
    E = _host_codebook(cb.E if isinstance(cb, PreparedCodebook) else cb)
    if E.shape[1] != 8:
        return 0
    return int(load_library().mpq_e8dp_transitions(E.ctypes.data_as(ctypes.c_void_p), E.shape[0]))


PROBE_KINDS = {"mfma_bf16": 0, "mfma_f64": 1, "valu_f64": 2, "exp_f32": 3, "hbm_copy": 4, "mfma_i8": 5}


def probe_rate(kind: str, scratch=None) -> float:
    """Achievable rate of one instruction or of an HBM copy on this GPU
    (mpq_probe_rate): flop/s for "mfma_bf16", "mfma_f64" and "valu_f64",
    int8 operations/s for "mfma_i8" (random operand bytes), lane operations/s
    for "exp_f32", bytes read + written per second for "hbm_copy".  `scratch` (a device tensor, contents overwritten) defaults
    to a fresh 2 GiB buffer."""
    import torch
    if kind not in PROBE_KINDS:
        raise ValueError(f"unknown probe {kind!r}; one of {sorted(PROBE_KINDS)}")
    if scratch is None:
        scratch = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    out = ctypes.c_double(0.0)
    rc = load_library().mpq_probe_rate(PROBE_KINDS[kind], _ptr(scratch), scratch.numel() * scratch.element_size(),
                                       ctypes.byref(out), _stream())
    _check(rc, "mpq_probe_rate")
    return float(out.value)


def workspace_bytes(m, n, r, K, d) -> int:
    return int(load_library().mpq_workspace_bytes(m, n, r, K, d))


def greedy_workspace_bytes(m, n, r, K, d) -> int:
    return int(load_library().mpq_greedy_workspace_bytes(m, n, r, K, d))


# ---------------------------------------------------------------- helpers

def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _dev(t, dtype, name, shape=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _host_codebook(cb):
    arr = cb.detach().cpu().numpy() if hasattr(cb, "detach") else np.asarray(cb)
    arr = np.ascontiguousarray(arr, dtype=np.float32)
    if arr.ndim != 2:
        raise ValueError("codebook must be K x d")
    return arr


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _workspace(m, n, r, K, d, device):
    import torch
    nb = workspace_bytes(m, n, r, K, d)
    if nb == 0:
        raise MPQError(-2, "mpq_workspace_bytes")
    return torch.empty(nb, dtype=torch.uint8, device=device)


def _opts(beta0=None, fixed_beta=False, profile=None, anchor_tau=None, anchor_w=None, group=None, map_codes=None,
          objective=None, scan_denoiser=False, e8_decode=True, safeguard_eps=0.0, fallbacks=None, sweeps=None,
          check_finite=False, linear_f64=False, log_prior=None, digits=None):
    flags = ((F_FIXED_BETA if fixed_beta else 0) | (F_PROFILE if profile is not None else 0) |
             (F_PROFILE_SAMPLED if profile is not None and profile.sampled else 0) |
             (F_NO_E8DP if scan_denoiser else 0) | (0 if e8_decode else F_NO_E8_DECODE) |
             (F_CHECK_FINITE if check_finite else 0) | (F_LINEAR_F64 if linear_f64 else 0))
    o = Options()
    o.beta0 = float(beta0) if beta0 else 0.0
    o.flags = flags
    o.safeguard_eps = float(safeguard_eps or 0.0)
    o.anchor_tau = float(anchor_tau) if anchor_tau else 0.0
    o.anchor_w = anchor_w.data_ptr() if anchor_w is not None else None
    o.group = int(group) if group else 0
    o.log_prior = log_prior.data_ptr() if log_prior is not None else None
    if profile is not None:
        o.profiler = profile.handle
        o.prof_mask = profile.mask
        o.prof_ms = profile.ms
        o.prof_launches = profile.launches
    o.map_codes = map_codes.data_ptr() if map_codes is not None else None
    o.objective = objective.data_ptr() if objective is not None else None
    o.fallbacks = fallbacks.data_ptr() if fallbacks is not None else None
    o.sweeps = sweeps.data_ptr() if sweeps is not None else None
    o.digits = int(digits or 0)
    return ctypes.byref(o), o


def _affine(row_scale, row_offset, m, n, group):
    """Check the per-row (m,) or per-group (m, ceil(n / group)) affine tensors."""
    import torch
    G = 1 if not group or group >= n else -(-n // group)
    for t, nm in ((row_scale, "row_scale"), (row_offset, "row_offset")):
        _dev(t, torch.float32, nm)
        if t.numel() != m * G or t.dim() not in (1, 2) or t.shape[0] != m:
            raise ValueError(f"{nm} has shape {tuple(t.shape)}, expected ({m},) or ({m}, {G})"
                             if G == 1 else f"{nm} has shape {tuple(t.shape)}, expected ({m}, {G})")


def _check(rc, what):
    if rc != 0:
        raise MPQError(rc, what)


# ---------------------------------------------------------------- entry points

def quantize_layer(W, s, V, cb, row_scale, row_offset, T_vamp=16, n_cd=3, damping=0.5, beta0=None,
                   fixed_beta=False, workspace=None, traces=True, profile=None, outputs=None, anchor_tau=None,
                   group=None, diagnostics=False, scan_denoiser=False, safeguard_eps=0.0, check_finite=False,
                   linear_f64=False, log_prior=None, digits=None):
    """Full MPQ solve of one layer (mpq_quantize_layer).

    `cb`: a PreparedCodebook (prepare_codebook) or a raw K x d codebook.
    Returns dict(codes, beta_tr, gamma1_tr, gamma2_tr, cd_changes) of device
    tensors.  `profile` (a Profile) turns on the library's event timing;
    `outputs` (a dict from a previous call) reuses its output tensors;
    `anchor_tau` > 0 selects the anchored codebook prior (None: uniform);
    `log_prior` (device float32, K) is log rho of every base codeword (d = 1);
    `group` > 0 gives every `group` consecutive columns their own affine
    (row_scale and row_offset then m x ceil(n / group)); `diagnostics` adds
    map_codes (the marginal-MAP codes CD starts from), objective (float64,
    per row), fallbacks (pass-through events per row) and sweeps (CD sweeps
    run per row) to the result.
    """
    import torch
    m, n = W.shape
    r = s.shape[0]
    P = prepare_codebook(cb, W.device)
    K, d = P.K, P.d
    dev = W.device
    _dev(W, torch.float32, "W")
    _dev(s, torch.float32, "s", (r,))
    _dev(V, torch.float32, "V", (n, r))
    _affine(row_scale, row_offset, m, n, group)
    if outputs is not None:
        codes, bt, g1, g2, ch = (outputs[k] for k in ("codes", "beta_tr", "gamma1_tr", "gamma2_tr", "cd_changes"))
    else:
        codes = torch.empty((m, n // d if d else 0), dtype=torch.int32, device=dev)
        bt = torch.empty((m, T_vamp + 1), dtype=torch.float32, device=dev) if traces else None
        g1 = torch.empty((m, T_vamp + 1), dtype=torch.float32, device=dev) if traces else None
        g2 = torch.empty((m, T_vamp), dtype=torch.float32, device=dev) if traces and T_vamp > 0 else None
        ch = torch.zeros((m, n_cd), dtype=torch.int32, device=dev) if traces and n_cd > 0 else None
    ws = workspace if workspace is not None else _workspace(m, n, r, K, d, dev)
    mc = torch.empty((m, n // d), dtype=torch.int32, device=dev) if diagnostics else None
    obj = torch.empty(m, dtype=torch.float64, device=dev) if diagnostics else None
    fb = torch.empty(m, dtype=torch.int32, device=dev) if diagnostics else None
    sw = torch.empty(m, dtype=torch.int32, device=dev) if diagnostics else None
    op, _keep = _opts(beta0, fixed_beta, profile, anchor_tau, None, group, mc, obj, scan_denoiser,
                      safeguard_eps=safeguard_eps, fallbacks=fb, sweeps=sw, check_finite=check_finite,
                      linear_f64=linear_f64, log_prior=log_prior, digits=digits)
    rc = load_library().mpq_quantize_layer(
        _ptr(W), m, n, _ptr(s), _ptr(V), r, P.ref(), _ptr(row_scale), _ptr(row_offset), int(T_vamp), int(n_cd),
        float(damping), op, _ptr(codes), _ptr(bt), _ptr(g1), _ptr(g2), _ptr(ch), _ptr(ws), ws.numel(), _stream())
    _check(rc, "mpq_quantize_layer")
    out = dict(codes=codes, beta_tr=bt, gamma1_tr=g1, gamma2_tr=g2, cd_changes=ch)
    if diagnostics:
        out.update(map_codes=mc, objective=obj, fallbacks=fb, sweeps=sw)
    return out


STATIC_WORKSPACE_BYTES = 64 << 20   # MPQ_STATIC_WORKSPACE_BYTES


def quantize_layer_static(W, s, V, cb, row_scale, row_offset, T_vamp=16, n_cd=3, damping=0.5, beta0=None,
                          group=None, outputs=None):
    """mpq_quantize_layer_static: the full solve in the library's static
    per-GPU workspace (no workspace argument; layers whose workspace exceeds
    STATIC_WORKSPACE_BYTES raise MPQ_EWORKSPACE).  `outputs` (a dict from a
    previous call of the same shape) reuses its output tensors.  Returns the
    dict of quantize_layer (codes and traces)."""
    import torch
    m, n = W.shape
    r = s.shape[0]
    P = prepare_codebook(cb, W.device)
    d = P.d
    dev = W.device
    _dev(W, torch.float32, "W")
    _dev(s, torch.float32, "s", (r,))
    _dev(V, torch.float32, "V", (n, r))
    _affine(row_scale, row_offset, m, n, group)
    if outputs is not None:
        codes, bt, g1, g2, ch = (outputs[k] for k in ("codes", "beta_tr", "gamma1_tr", "gamma2_tr", "cd_changes"))
    else:
        codes = torch.empty((m, n // d), dtype=torch.int32, device=dev)
        bt = torch.empty((m, T_vamp + 1), dtype=torch.float32, device=dev)
        g1 = torch.empty((m, T_vamp + 1), dtype=torch.float32, device=dev)
        g2 = torch.empty((m, T_vamp), dtype=torch.float32, device=dev) if T_vamp > 0 else None
        ch = torch.zeros((m, n_cd), dtype=torch.int32, device=dev) if n_cd > 0 else None
    op, _keep = _opts(beta0, group=group)
    rc = load_library().mpq_quantize_layer_static(
        _ptr(W), m, n, _ptr(s), _ptr(V), r, P.ref(), _ptr(row_scale), _ptr(row_offset), int(T_vamp), int(n_cd),
        float(damping), op, _ptr(codes), _ptr(bt), _ptr(g1), _ptr(g2), _ptr(ch), _stream())
    _check(rc, "mpq_quantize_layer_static")
    return dict(codes=codes, beta_tr=bt, gamma1_tr=g1, gamma2_tr=g2, cd_changes=ch)


def prologue(W, s, V, cb, row_scale, row_offset, beta0=None, workspace=None, group=None, linear_f64=False,
             digits=None):
    """RTN codes, gamma1^0 and beta^0 of every row (mpq_prologue); float64 scalars."""
    import torch
    m, n = W.shape
    r = s.shape[0]
    P = prepare_codebook(cb, W.device)
    K, d = P.K, P.d
    dev = W.device
    rtn = torch.empty((m, n // d), dtype=torch.int32, device=dev)
    gamma1 = torch.empty(m, dtype=torch.float64, device=dev)
    beta = torch.empty(m, dtype=torch.float64, device=dev)
    _affine(row_scale, row_offset, m, n, group)
    ws = workspace if workspace is not None else _workspace(m, n, r, K, d, dev)
    op, _keep = _opts(beta0, group=group, linear_f64=linear_f64, digits=digits)
    rc = load_library().mpq_prologue(_ptr(W), m, n, _ptr(s), _ptr(V), r, P.ref(), _ptr(row_scale),
                                     _ptr(row_offset), op, _ptr(rtn), _ptr(gamma1), _ptr(beta), _ptr(ws), ws.numel(),
                                     _stream())
    _check(rc, "mpq_prologue")
    return dict(rtn_codes=rtn, gamma1=gamma1, beta=beta)


def denoise(R1, gamma1, cb, row_scale, row_offset, workspace=None, anchor_tau=None, W=None, group=None,
            scan_denoiser=False):
    """Blockwise denoiser (mpq_denoise): (xhat1, per-block variance trace), float64.
    `scan_denoiser` forces the codebook-scan kernel for E8-prefix codebooks."""
    import torch
    m, n = R1.shape
    P = prepare_codebook(cb, R1.device)
    K, d = P.K, P.d
    dev = R1.device
    _dev(R1, torch.float64, "R1")
    _dev(gamma1, torch.float64, "gamma1", (m,))
    _affine(row_scale, row_offset, m, n, group)
    if anchor_tau:
        _dev(W, torch.float32, "W", (m, n))
    xhat = torch.empty_like(R1)
    vtr = torch.empty((m, n // d), dtype=torch.float64, device=dev)
    ws = workspace if workspace is not None else _workspace(m, n, n, K, d, dev)
    op, _keep = _opts(anchor_tau=anchor_tau, anchor_w=W, group=group, scan_denoiser=scan_denoiser)
    rc = load_library().mpq_denoise(_ptr(R1), _ptr(gamma1), m, n, P.ref(), _ptr(row_scale), _ptr(row_offset), op,
                                    _ptr(xhat), _ptr(vtr), _ptr(ws), ws.numel(), _stream())
    _check(rc, "mpq_denoise")
    return xhat, vtr


def vamp_step(R1, gamma1, beta, W, s, V, cb, row_scale, row_offset, damping=0.5, fixed_beta=False,
              workspace=None, anchor_tau=None, group=None, safeguard_eps=0.0, linear_f64=False, digits=None):
    """One VAMP iteration in place on (R1, gamma1, beta) (float64); returns the
    diagnostics.  W: the layer's weights (float32); with `anchor_tau` > 0 the
    prior is anchored at W."""
    import torch
    m, n = R1.shape
    r = s.shape[0]
    P = prepare_codebook(cb, R1.device)
    K, d = P.K, P.d
    dev = R1.device
    for t, nm in ((R1, "R1"), (gamma1, "gamma1"), (beta, "beta")):
        _dev(t, torch.float64, nm)
    _dev(W, torch.float32, "W", (m, n))
    xhat = torch.empty_like(R1)
    r2 = torch.empty_like(R1)
    eta1 = torch.empty(m, dtype=torch.float64, device=dev)
    gamma2 = torch.empty(m, dtype=torch.float64, device=dev)
    fb = torch.empty(m, dtype=torch.int32, device=dev)
    ws = workspace if workspace is not None else _workspace(m, n, r, K, d, dev)
    _affine(row_scale, row_offset, m, n, group)
    op, _keep = _opts(None, fixed_beta, None, anchor_tau, W if anchor_tau else None, group,
                      safeguard_eps=safeguard_eps, linear_f64=linear_f64, digits=digits)
    rc = load_library().mpq_vamp_step(_ptr(R1), _ptr(gamma1), _ptr(beta), _ptr(W), m, n, _ptr(s), _ptr(V), r,
                                      P.ref(), _ptr(row_scale), _ptr(row_offset), float(damping), op, _ptr(xhat),
                                      _ptr(eta1), _ptr(gamma2), _ptr(r2), _ptr(fb), _ptr(ws), ws.numel(), _stream())
    _check(rc, "mpq_vamp_step")
    return dict(xhat1=xhat, eta1=eta1, gamma2=gamma2, r2=r2, fallback=fb)


def linear_step(R2, gamma2, beta, W, s, V, damping=0.5, fixed_beta=False, workspace=None, linear_f64=False,
                digits=None):
    """The Gaussian linear module + beta M-step (mpq_linear_step): from the
    extrinsic message (R2, gamma2) and beta (updated in place), returns
    (R1, gamma1), the message back to the denoiser (float64)."""
    import torch
    m, n = R2.shape
    r = s.shape[0]
    _dev(R2, torch.float64, "R2")
    _dev(gamma2, torch.float64, "gamma2", (m,))
    _dev(beta, torch.float64, "beta", (m,))
    _dev(W, torch.float32, "W", (m, n))
    _dev(s, torch.float32, "s", (r,))
    _dev(V, torch.float32, "V", (n, r))
    R1 = torch.empty_like(R2)
    gamma1 = torch.empty_like(gamma2)
    ws = workspace if workspace is not None else _workspace(m, n, r, 2, 1, R2.device)
    op, _keep = _opts(None, fixed_beta, linear_f64=linear_f64, digits=digits)
    rc = load_library().mpq_linear_step(_ptr(R2), _ptr(gamma2), _ptr(beta), _ptr(W), m, n, _ptr(s), _ptr(V), r,
                                        float(damping), op, _ptr(R1), _ptr(gamma1), _ptr(ws), ws.numel(), _stream())
    _check(rc, "mpq_linear_step")
    return R1, gamma1


def map_codes(R1, gamma1, cb, row_scale, row_offset, workspace=None, anchor_tau=None, W=None, group=None,
              scan_denoiser=False, e8_decode=True):
    """Marginal MAP codes (mpq_map) at float64 (R1, gamma1); scan_denoiser keeps
    the codebook scan for E8 prefix codebooks too; e8_decode=False finds an E8
    prefix codebook's nearest codewords with the automaton alone (no
    lattice-decoder fast path)."""
    import torch
    m, n = R1.shape
    P = prepare_codebook(cb, R1.device)
    K, d = P.K, P.d
    _dev(R1, torch.float64, "R1")
    _dev(gamma1, torch.float64, "gamma1", (m,))
    _affine(row_scale, row_offset, m, n, group)
    if anchor_tau:
        _dev(W, torch.float32, "W", (m, n))
    codes = torch.empty((m, n // d), dtype=torch.int32, device=R1.device)
    ws = workspace if workspace is not None else _workspace(m, n, n, K, d, R1.device)
    op, _keep = _opts(anchor_tau=anchor_tau, anchor_w=W, group=group, scan_denoiser=scan_denoiser,
                      e8_decode=e8_decode)
    rc = load_library().mpq_map(_ptr(R1), _ptr(gamma1), m, n, P.ref(), _ptr(row_scale), _ptr(row_offset), op,
                                _ptr(codes), _ptr(ws), ws.numel(), _stream())
    _check(rc, "mpq_map")
    return codes


def cd(W, s, V, cb, row_scale, row_offset, codes, n_cd=3, workspace=None, group=None, sweeps=None, digits=None):
    """Block CD from `codes` (a device int32 tensor, updated in place); returns
    (codes, changes per sweep).  `sweeps` (device int32, m) receives the
    sweeps run per row."""
    import torch
    m, n = W.shape
    r = s.shape[0]
    P = prepare_codebook(cb, W.device)
    K, d = P.K, P.d
    _dev(codes, torch.int32, "codes", (m, n // d))
    _affine(row_scale, row_offset, m, n, group)
    ch = torch.zeros((m, max(n_cd, 1)), dtype=torch.int32, device=W.device)
    ws = workspace if workspace is not None else _workspace(m, n, r, K, d, W.device)
    op, _keep = _opts(group=group, sweeps=sweeps, digits=digits)
    rc = load_library().mpq_cd(_ptr(W), m, n, _ptr(s), _ptr(V), r, P.ref(), _ptr(row_scale), _ptr(row_offset),
                               int(n_cd), op, _ptr(codes), _ptr(ch), _ptr(ws), ws.numel(), _stream())
    _check(rc, "mpq_cd")
    return codes, ch[:, :n_cd]


def objective(W, s, V, cb, row_scale, row_offset, codes, workspace=None, group=None):
    """Per-row float64 objective 1/2 ||diag(s) V^T (w - x)||^2 of `codes` (mpq_objective)."""
    import torch
    m, n = W.shape
    r = s.shape[0]
    P = prepare_codebook(cb, W.device)
    K, d = P.K, P.d
    _dev(W, torch.float32, "W")
    _dev(s, torch.float32, "s", (r,))
    _dev(V, torch.float32, "V", (n, r))
    _dev(codes, torch.int32, "codes", (m, n // d))
    _affine(row_scale, row_offset, m, n, group)
    f = torch.empty(m, dtype=torch.float64, device=W.device)
    ws = workspace if workspace is not None else _workspace(m, n, r, K, d, W.device)
    op, _keep = _opts(group=group)
    rc = load_library().mpq_objective(_ptr(W), m, n, _ptr(s), _ptr(V), r, P.ref(), _ptr(row_scale),
                                      _ptr(row_offset), op, _ptr(codes), _ptr(f), _ptr(ws), ws.numel(), _stream())
    _check(rc, "mpq_objective")
    return f


def greedy(W, s, V, cb, row_scale, row_offset, workspace=None, group=None, profile=None):
    """Sequential greedy comparator codes (mpq_greedy); the workspace must hold
    greedy_workspace_bytes(...)."""
    import torch
    m, n = W.shape
    r = s.shape[0]
    P = prepare_codebook(cb, W.device)
    K, d = P.K, P.d
    _dev(W, torch.float32, "W")
    _dev(s, torch.float32, "s", (r,))
    _dev(V, torch.float32, "V", (n, r))
    _affine(row_scale, row_offset, m, n, group)
    codes = torch.empty((m, n // d), dtype=torch.int32, device=W.device)
    if workspace is None:
        nb = greedy_workspace_bytes(m, n, r, K, d)
        if nb == 0:
            raise MPQError(-2, "mpq_greedy_workspace_bytes")
        workspace = torch.empty(nb, dtype=torch.uint8, device=W.device)
    op, _keep = _opts(profile=profile, group=group)
    rc = load_library().mpq_greedy(_ptr(W), m, n, _ptr(s), _ptr(V), r, P.ref(), _ptr(row_scale), _ptr(row_offset),
                                   op, _ptr(codes), _ptr(workspace), workspace.numel(), _stream())
    _check(rc, "mpq_greedy")
    return codes


# ---------------------------------------------------------------- front end

def gram(X, workspace=None):
    """H = X^T X (float64 n x n) of the activations X (device float32 N x n)."""
    import torch
    _dev(X, torch.float32, "X")
    N, n = X.shape
    H = torch.empty((n, n), dtype=torch.float64, device=X.device)
    if workspace is None:
        nb = int(load_library().mpq_gram_workspace_bytes(n))
        if nb == 0:
            raise MPQError(-2, "mpq_gram_workspace_bytes")
        workspace = torch.empty(nb, dtype=torch.uint8, device=X.device)
    _check(load_library().mpq_gram(_ptr(X), N, n, _ptr(H), _ptr(workspace), workspace.numel(), _stream()),
           "mpq_gram")
    return H


def rht(A, signs):
    """Random Hadamard transform of every row of A (device float32, in place); returns A."""
    import torch
    _dev(A, torch.float32, "A")
    rows, n = A.shape
    _dev(signs, torch.float32, "signs", (n,))
    _check(load_library().mpq_rht(_ptr(A), rows, n, _ptr(signs), _stream()), "mpq_rht")
    return A


def factor(H, r, workspace=None):
    """(s, V) of the r largest eigenpairs of H (device float64 n x n, overwritten)."""
    import torch
    _dev(H, torch.float64, "H")
    n = H.shape[0]
    s = torch.empty(r, dtype=torch.float32, device=H.device)
    V = torch.empty((n, r), dtype=torch.float32, device=H.device)
    if workspace is None:
        nb = int(load_library().mpq_factor_workspace_bytes(n))
        if nb == 0:
            raise MPQError(-7, "mpq_factor_workspace_bytes")
        workspace = torch.empty(nb, dtype=torch.uint8, device=H.device)
    _check(load_library().mpq_factor(_ptr(H), n, int(r), _ptr(s), _ptr(V), _ptr(workspace), workspace.numel(),
                                     _stream()), "mpq_factor")
    return s, V


def frontend(X, W, r=None, signs=None):
    """Activations X (N x n) and weights W (m x n) -> (W', s, V) for the solver:
    with `signs` both are rotated by the RHT first (copies; the inputs are
    left unchanged), then H = X'^T X' and its r largest modes (default r = n)."""
    n = X.shape[1]
    if signs is not None:
        X = rht(X.clone(), signs)
        W = rht(W.clone(), signs)
    H = gram(X)
    s, V = factor(H, n if r is None else r)
    return W, s, V
