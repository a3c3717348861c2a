"""Host-side checks of the C ABI: the library loads, exports everything the
header declares, sizes workspaces and rejects bad arguments before touching
the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

import post_quantization_solver_amd as mpq
import mpq_synth as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mpq.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mpq.LIB_PATH):
        from post_quantization_solver_amd import build
        build.build()
    return mpq.load_library()


def declared_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mpq_\w+)\s*\(", txt, flags=re.M)))


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert set(names) == set(mpq.EXPORTS)
    for nm in names:
        assert hasattr(lib, nm), nm


def test_workspace_sizes(lib):
    assert mpq.workspace_bytes(64, 256, 256, 8, 1) > 0
    big = mpq.workspace_bytes(4096, 14336, 14336, 65536, 8)
    assert 2e9 < big < 12e9
    assert mpq.workspace_bytes(4, 10, 11, 8, 1) == 0       # r > n
    assert mpq.workspace_bytes(4, 12, 12, 8, 8) == 0       # n % d
    assert mpq.workspace_bytes(4, 16, 16, 8, 3) == 0       # d unsupported
    assert mpq.workspace_bytes(4, 16, 16, 65, 1) == 0      # K > 64 for scalar grids


FAKE = ctypes.c_void_p(1 << 20)   # never dereferenced: validation fails first
# the marker mpq_codebook_prepare sets in a filled mpq_codebook (library-internal)
CB_MAGIC = 0x4d50514342763200


def fake_codebook(K=8, d=1, kind=0, magic=CB_MAGIC, tables=FAKE):
    """A mpq_codebook as mpq_codebook_prepare would fill it, with tables at a
    fake device address: enough for the host-side validation paths."""
    cb = mpq.binding.Codebook()
    cb.K, cb.d, cb.kind, cb.magic = K, d, kind, magic
    cb.tables = tables
    return cb


def call_layer(lib, m=4, n=16, r=16, K=8, d=1, T=2, ncd=1, rho=0.5, cb=None, ws_bytes=1 << 30, W=FAKE, ws=FAKE,
               opt=None):
    cbs = fake_codebook(K, d) if cb is None else cb
    op = ctypes.byref(opt) if opt is not None else None
    return lib.mpq_quantize_layer(W, m, n, FAKE, FAKE, r, ctypes.byref(cbs), FAKE, FAKE, T, ncd, rho, op, FAKE,
                                  None, None, None, None, ws, ws_bytes, None)


def test_argument_validation(lib):
    assert call_layer(lib, T=-1) == -3
    assert call_layer(lib, ncd=-2) == -3
    assert call_layer(lib, rho=0.0) == -3
    assert call_layer(lib, rho=1.5) == -3
    assert call_layer(lib, rho=float("nan")) == -3
    assert call_layer(lib, d=3, n=18, r=18) == -4
    assert call_layer(lib, d=8, K=256, n=12, r=12) == -2
    assert call_layer(lib, r=17) == -2
    assert call_layer(lib, m=-1) == -2
    assert call_layer(lib, n=65536 + 8, r=8) == -2            # longer rows than the solver takes
    assert call_layer(lib, W=None) == -1
    assert call_layer(lib, m=0) == 0                          # nothing to do
    # an unprepared codebook, or none
    assert call_layer(lib, cb=fake_codebook(magic=0)) == -3
    assert call_layer(lib, cb=fake_codebook(tables=None)) == -1
    assert lib.mpq_quantize_layer(FAKE, 4, 16, FAKE, FAKE, 16, None, FAKE, FAKE, 2, 1, 0.5, None, FAKE, None, None,
                                  None, None, FAKE, 1 << 30, None) == -1
    # workspace too small or misaligned
    assert call_layer(lib, d=8, K=256, ws_bytes=1024) == -5
    assert call_layer(lib, d=8, K=256, ws=ctypes.c_void_p((1 << 20) + 4)) == -5
    assert call_layer(lib, d=8, K=256, ws=None) == -5


def test_codebook_prepare_validation(lib):
    def prep(E, K=None, d=None, tables=FAKE, nbytes=1 << 30, out=True):
        E = np.ascontiguousarray(E, dtype=np.float32)
        K = E.shape[0] if K is None else K
        d = E.shape[1] if d is None else d
        cb = mpq.binding.Codebook()
        return lib.mpq_codebook_prepare(E.ctypes.data_as(ctypes.c_void_p), K, d, tables, nbytes, None,
                                        ctypes.byref(cb) if out else None)
    good = S.e8_codebook(256)
    assert prep(good * np.float32(1.1)) == -4                  # d = 8 codebook not exact in bfloat16
    assert prep(np.zeros((4, 3))) == -4                        # d unsupported
    assert prep(np.zeros((65, 1))) == -2                       # K > 64 for scalar grids
    assert prep(np.array([[0.0], [np.nan]])) == -3             # non-finite level
    assert prep(good, tables=None) == -1
    assert prep(good, out=False) == -1
    assert prep(good, nbytes=1024) == -5                       # table buffer too small
    assert prep(good, tables=ctypes.c_void_p((1 << 20) + 8)) == -5   # misaligned
    assert lib.mpq_codebook_bytes(8, 1) > 0 and lib.mpq_codebook_bytes(65536, 8) > 8 << 20
    assert lib.mpq_codebook_bytes(65, 1) == 0 and lib.mpq_codebook_bytes(8, 3) == 0


def test_group_option_validation(lib):
    Opt = mpq.binding.Options
    assert call_layer(lib, opt=Opt(group=-1)) == -3
    assert call_layer(lib, d=8, K=256, opt=Opt(group=8)) == -4                   # groups need d = 1
    assert call_layer(lib, opt=Opt(group=8, anchor_tau=0.2)) == -4                # and the uniform prior
    # an accepted group option reaches the workspace check
    assert call_layer(lib, opt=Opt(group=8), ws_bytes=1024) == -5
    assert call_layer(lib, opt=Opt(group=64), ws_bytes=1024) == -5                # group >= n: one per row
    assert call_layer(lib, opt=Opt(group=0, anchor_tau=0.2), ws_bytes=1024) == -5


def test_option_validation(lib):
    Opt = mpq.binding.Options
    assert call_layer(lib, opt=Opt(safeguard_eps=-0.1)) == -3
    assert call_layer(lib, opt=Opt(safeguard_eps=float("nan"))) == -3
    assert call_layer(lib, opt=Opt(safeguard_eps=0.5), ws_bytes=1024) == -5       # accepted
    assert call_layer(lib, opt=Opt(flags=mpq.binding.F_PROFILE)) == -1            # profiling needs a profiler
    for bad in (1, 3, 6, -1):                                                     # digits: 4, 5 or 0
        assert call_layer(lib, opt=Opt(digits=bad)) == -3
    for ok in (0, 4, 5):
        assert call_layer(lib, opt=Opt(digits=ok), ws_bytes=1024) == -5
    h = ctypes.c_void_p()
    assert lib.mpq_profiler_create(0, ctypes.byref(h)) == -3
    assert lib.mpq_profiler_create(4, None) == -1
    lib.mpq_profiler_destroy(None)                                                # no-op


def test_linear_step_validation(lib):
    def call(m=4, n=16, r=16, rho=0.5, R2=FAKE, ws_bytes=1 << 30, opt=None):
        return lib.mpq_linear_step(R2, FAKE, FAKE, FAKE, m, n, FAKE, FAKE, r, rho,
                                   ctypes.byref(opt) if opt is not None else None, FAKE, FAKE, FAKE, ws_bytes, None)
    assert call(rho=0.0) == -3
    assert call(r=17) == -2
    assert call(m=-1) == -2
    assert call(m=0) == 0
    assert call(R2=None) == -1
    assert call(ws_bytes=1024) == -5
    assert call(opt=mpq.binding.Options(flags=mpq.binding.F_PROFILE)) == -4
    assert call(opt=mpq.binding.Options(digits=2)) == -3
    assert call(opt=mpq.binding.Options(digits=4), ws_bytes=1024) == -5


def test_frontend_argument_validation(lib):
    assert lib.mpq_rht(FAKE, 4, 12, FAKE, None) == -4          # n neither 2^k nor 28 * 2^k
    assert lib.mpq_rht(FAKE, 4, 32768, FAKE, None) == -4       # longer than the LDS row
    assert lib.mpq_rht(FAKE, -1, 16, FAKE, None) == -2
    assert lib.mpq_rht(FAKE, 0, 16, FAKE, None) == 0
    assert lib.mpq_rht(None, 2, 16, FAKE, None) == -1
    assert lib.mpq_gram(FAKE, 10, 0, FAKE, FAKE, 1 << 30, None) == -2
    assert lib.mpq_gram(FAKE, 10, 16, None, FAKE, 1 << 30, None) == -1
    assert lib.mpq_gram(FAKE, 10, 16, FAKE, FAKE, 16, None) == -5
    assert lib.mpq_factor(FAKE, 16, 17, FAKE, FAKE, FAKE, 1 << 30, None) == -2
    assert lib.mpq_factor(None, 16, 4, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert lib.mpq_gram_workspace_bytes(0) == 0 and lib.mpq_gram_workspace_bytes(256) > 0


@pytest.mark.parametrize("struct_name,cls", [("mpq_options", "Options"), ("mpq_codebook", "Codebook")])
def test_struct_layout_matches_header(tmp_path, struct_name, cls):
    """The ctypes mirrors of the header's structs have its field offsets and
    sizes (compiled with the host C compiler)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    Opt = getattr(mpq.binding, cls)
    names = [f[0] for f in Opt._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"mpq.h\"\nint main(void) {\n" +
                   "".join(f'  printf("%zu\\n", offsetof({struct_name}, {nm}));\n' for nm in names) +
                   f'  printf("%zu\\n", sizeof({struct_name}));\n  return 0;\n}}\n')
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    want = [getattr(Opt, nm).offset for nm in names] + [ctypes.sizeof(Opt)]
    assert got == want


def test_digits_default_matches_header(tmp_path):
    """The binding's DIGITS_DEFAULT is the header's MPQ_DIGITS_DEFAULT."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    src = tmp_path / "dd.c"
    src.write_text('#include <stdio.h>\n#include "mpq.h"\nint main(void) { printf("%d\\n", MPQ_DIGITS_DEFAULT); '
                   'return 0; }\n')
    exe = tmp_path / "dd"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = int(subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout)
    assert got == mpq.binding.DIGITS_DEFAULT


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9):
        assert lib.mpq_strerror(code).decode()
    with pytest.raises(mpq.MPQError):
        mpq.binding._check(-3, "x")


def test_probe_argument_validation(lib):
    import ctypes as C
    out = C.c_double(0.0)
    # rejected before anything reaches the GPU
    assert lib.mpq_probe_rate(0, None, 1 << 30, C.byref(out), None) == -1          # MPQ_ENULL
    fake = C.c_void_p(1 << 20)                                                   # never dereferenced
    assert lib.mpq_probe_rate(0, fake, 1 << 30, None, None) == -1
    assert lib.mpq_probe_rate(6, fake, 1 << 30, C.byref(out), None) == -3        # MPQ_EPARAM
    assert lib.mpq_probe_rate(-1, fake, 1 << 30, C.byref(out), None) == -3
    assert lib.mpq_probe_rate(0, fake, 1 << 20, C.byref(out), None) == -5        # MPQ_EWORKSPACE: < 8 MiB
    assert lib.mpq_probe_rate(4, fake, 128 << 20, C.byref(out), None) == -5      # copy needs 256 MiB
    assert lib.mpq_probe_rate(0, C.c_void_p((1 << 20) + 16), 1 << 30, C.byref(out), None) == -5   # misaligned
    with pytest.raises(ValueError):
        mpq.probe_rate("no_such_probe")
