"""Host-side checks of the C ABI that need no GPU: the library loads,
exports every symbol include/gdn.h declares, and host validation rejects bad
arguments before any HIP call (fail closed, as on "Add request-owned
eight-way MTP serving for Qwen 35B", Clean-install verification; shapes
checked before work, as on "MTP inference: review and commit structure",
Review fixes)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
# GDN_LIB: another build of the library (the host sanitizer run)
LIB = os.environ.get("GDN_LIB") or os.path.join(ROOT, "gated_deltanet_recurrence_conv_amd", "libgdn.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from gated_deltanet_recurrence_conv_amd import build
        build.build()
    return ctypes.CDLL(LIB)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:gdn_status|size_t|const char\*)\s+(gdn_\w+)\s*\(",
                                 text, re.M)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("gdn_conv_step", "gdn_verify", "gdn_commit", "gdn_rewind", "gdn_verify_lazy",
              "gdn_prefill_chunked", "gdn_workspace_size", "gdn_status_string", "gdn_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_binding_exports_same_names():
    from gated_deltanet_recurrence_conv_amd import binding
    for n in declared_functions():
        assert hasattr(binding, n), n


class Dims(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("B", ctypes.c_int32), ("T", ctypes.c_int32),
                ("HV", ctypes.c_int32), ("HK", ctypes.c_int32), ("DK", ctypes.c_int32),
                ("DV", ctypes.c_int32), ("KCONV", ctypes.c_int32), ("S", ctypes.c_int32),
                ("act", ctypes.c_int32), ("out", ctypes.c_int32),
                ("scale", ctypes.c_float), ("l2_eps", ctypes.c_float),
                ("flags", ctypes.c_uint32)]


def good():
    return Dims(1, 8, 2, 32, 16, 128, 128, 4, 3, 1, 0, 1.0, 1e-6, 3)


FAKE = 1 << 20   # aligned, never dereferenced: validation fails before any launch


def verify_call(lib, d, **over):
    args = dict(x=FAKE, w=FAKE, b=None, cs=FAKE, g=FAKE, beta=FAKE, st=FAKE, cur=None, o=FAKE,
                act=None, err=None)
    args.update(over)
    f = lib.gdn_verify
    f.argtypes = [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 12
    return f(ctypes.byref(d), args["x"], args["w"], args["b"], args["cs"], args["g"],
             args["beta"], args["st"], args["cur"], args["o"], args["act"], args["err"], None)


def declared_param_counts():
    """Number of parameters of every function include/gdn.h declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"^\s*(?:gdn_status|size_t|const char\*)\s+(gdn_\w+)\s*\(([^)]*)\)", text, re.M):
        args = m.group(2).strip()
        out[m.group(1)] = 0 if args in ("", "void") else args.count(",") + 1
    return out


def test_binding_declares_every_argument():
    """Each C function the binding calls has ctypes argtypes with the header's
    parameter count, so no 64-bit pointer is ever passed as a C int."""
    from gated_deltanet_recurrence_conv_amd import binding
    src = open(binding.__file__).read()
    called = set(re.findall(r"_lib\.(gdn_\w+)\(", src))
    counts = declared_param_counts()
    assert called <= set(counts)
    for n in called:
        argtypes = getattr(binding._lib, n).argtypes
        assert argtypes is not None, n
        assert len(argtypes) == counts[n], (n, len(argtypes), counts[n])


@pytest.mark.parametrize("field,value,status", [
    ("act", 7, 3), ("out", -1, 3), ("L", 0, 2), ("B", 0, 2), ("T", 0, 2), ("T", 5, 2),
    ("HV", 30, 2), ("DK", 96, 2), ("DV", 8, 2), ("KCONV", 3, 2), ("S", 2, 2)])
def test_verify_rejects_bad_dims(lib, field, value, status):
    d = good()
    setattr(d, field, value)
    assert verify_call(lib, d) == status


def test_verify_rejects_null_and_misaligned(lib):
    assert verify_call(lib, good(), x=None) == 1
    assert verify_call(lib, good(), o=None) == 1
    assert verify_call(lib, good(), st=FAKE + 4) == 4
    assert verify_call(lib, good(), cur=FAKE + 2) == 4
    assert verify_call(lib, good(), g=FAKE + 4) == 4
    f = lib.gdn_verify
    f.argtypes = [ctypes.c_void_p] * 13
    assert f(None, *([FAKE] * 12)) == 1


def test_commit_rewind_conv_prefill_validation(lib):
    d = good()
    lib.gdn_commit.argtypes = [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 7
    assert lib.gdn_commit(ctypes.byref(d), FAKE, FAKE, None, FAKE, None, None, None) == 1
    d.T = 3   # S = 3 < T + 1
    assert lib.gdn_commit(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, None) == 2
    d = good()
    lib.gdn_rewind.argtypes = [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 12
    assert lib.gdn_rewind(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None,
                          None, None, None, None) == 1          # keep missing
    lib.gdn_conv_step.argtypes = [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 6 + \
        [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    d.T = 1024
    assert lib.gdn_conv_step(ctypes.byref(d), FAKE, FAKE, None, FAKE, None, None, 1, None,
                             None) == 1
    d.act = 5
    assert lib.gdn_conv_step(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, None, 1, None,
                             None) == 3
    d = good()
    d.T = 1024
    lib.gdn_prefill_chunked.argtypes = [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 6 + \
        [ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.gdn_prefill_chunked(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE, 32,
                                   None, 0, None, None) == 2    # chunk must be 64
    lib.gdn_prefill_ragged.argtypes = [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 7 + \
        [ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.gdn_prefill_ragged(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE + 2,
                                  64, FAKE, 1 << 40, None, None) == 4   # lengths misaligned
    assert lib.gdn_prefill_ragged(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                  64, FAKE, 16, None, None) == 6        # workspace too small
    lib.gdn_workspace_size.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32]
    lib.gdn_workspace_size.restype = ctypes.c_size_t
    assert lib.gdn_workspace_size(ctypes.byref(d), 32) == 0


def test_prefill_conv_validation(lib):
    """The fused conv + prefill: missing pointers, chunk, workspace size, and
    the shapes it does not serve (fp32 activations, d_k = 16)."""
    f = lib.gdn_prefill_conv_chunked
    f.argtypes = [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 9 + \
        [ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]

    def call(d, conv_w=FAKE, chunk=64, ws_bytes=1 << 40):
        return f(ctypes.byref(d), FAKE, conv_w, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, chunk,
                 FAKE, ws_bytes, None, None)
    d = good()
    d.T = 1024
    assert call(d, conv_w=None) == 1
    assert call(d, chunk=32) == 2
    assert call(d, ws_bytes=16) == 6
    d.act = 0                     # fp32 activations: the two calls serve them
    assert call(d) == 5
    d = good()
    d.DK = 16
    assert call(d) == 5


def test_verify_lazy_validation(lib):
    """Host checks of the fused commit + verify: window length, required
    pointers, a previous window without its inputs, alignment.  Every call
    fails before any launch."""
    f = lib.gdn_verify_lazy
    f.argtypes = [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 16

    def call(d, **over):
        a = dict(xp=FAKE, gp=FAKE, bp=FAKE, kp=FAKE, x=FAKE, w=FAKE, b=None, cs=FAKE, g=FAKE,
                 beta=FAKE, st=FAKE, cur=None, o=FAKE, act=None, err=None)
        a.update(over)
        return f(ctypes.byref(d), a["xp"], a["gp"], a["bp"], a["kp"], a["x"], a["w"], a["b"],
                 a["cs"], a["g"], a["beta"], a["st"], a["cur"], a["o"], a["act"], a["err"], None)

    d = good()
    d.T = 5
    assert call(d) == 2                       # windows are at most 4 tokens
    d = good()
    assert call(d, o=None) == 1               # outputs are required
    assert call(d, xp=None) == 1              # previous window named by keep_prev but missing
    assert call(d, bp=None) == 1
    assert call(d, kp=FAKE + 2) == 4          # int32 arrays: 4-byte alignment
    assert call(d, xp=FAKE + 8) == 4
    d.S = 1                                   # no candidate slots needed ...
    d.T = 0
    assert call(d, kp=None, xp=None, gp=None, bp=None) == 2   # ... but T >= 1


def test_accept_greedy_validation(lib):
    f = lib.gdn_accept_greedy
    f.argtypes = [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 6
    d = good()
    assert f(ctypes.byref(d), None, FAKE, None, FAKE, None, None) == 1    # drafts needed at T = 2
    assert f(ctypes.byref(d), FAKE, None, None, FAKE, None, None) == 1    # targets needed
    assert f(ctypes.byref(d), FAKE, FAKE, None, None, None, None) == 1    # keep needed
    assert f(ctypes.byref(d), FAKE, FAKE, None, FAKE + 2, None, None) == 4
    d.T = 5
    assert f(ctypes.byref(d), FAKE, FAKE, None, FAKE, None, None) == 2


def test_gated_rmsnorm_validation(lib):
    f = lib.gdn_gated_rmsnorm
    f.argtypes = [ctypes.POINTER(Dims), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    d = good()
    assert f(ctypes.byref(d), FAKE, None, FAKE, 1e-6, FAKE, None, None) == 1   # z missing
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE + 2, 1e-6, FAKE, None, None) == 4
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, -1.0, FAKE, None, None) == 2   # eps < 0
    d.DV = 12
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, 1e-6, FAKE, None, None) == 2


def test_tile_counts_fit_32_bits(lib):
    """(layer, row, head) tile counts beyond 2^30 are refused on the host, so
    no grid size or tile index can overflow a 32-bit counter."""
    f = lib.gdn_verify
    f.argtypes = [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 12
    d = Dims(1, 32768, 2, 65536, 65536, 16, 16, 4, 1, 1, 0, 1.0, 1e-6, 3)   # state size in range
    assert f(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None,
             None) == 2


def test_huge_head_counts_refused_without_overflow(lib):
    """Channel counts beyond 32 bits (2*HK*DK + HV*DV) are computed in 64 bits
    and refused."""
    f = lib.gdn_verify
    f.argtypes = [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 12
    d = Dims(1, 1, 2, 1 << 25, 1 << 25, 128, 128, 4, 3, 1, 0, 1.0, 1e-6, 3)
    assert f(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None,
             None) == 2


def test_verify_gated_norm_validation(lib):
    """Host checks of verify / fused commit + verify with the gated-norm
    epilogue: the norm operands are required, aligned, eps >= 0, and the
    window checks of the plain calls still apply.  No call reaches a launch."""
    fv = lib.gdn_verify_gated_norm
    fv.argtypes = ([ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 10 + [ctypes.c_float] +
                   [ctypes.c_void_p] * 4)
    fl = lib.gdn_verify_lazy_gated_norm
    fl.argtypes = ([ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 14 + [ctypes.c_float] +
                   [ctypes.c_void_p] * 4)

    def v(d, z=FAKE, w=FAKE, eps=1e-6, y=FAKE, cur=None):
        return fv(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, cur, z, w, eps, y,
                  None, None, None)

    def lz(d, z=FAKE, w=FAKE, eps=1e-6, y=FAKE):
        return fl(ctypes.byref(d), None, None, None, None, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                  FAKE, None, z, w, eps, y, None, None, None)

    d = good()
    for call in (v, lz):
        assert call(d, z=None) == 1             # gate input required
        assert call(d, w=None) == 1             # norm weight required
        assert call(d, y=None) == 1             # outputs required
        assert call(d, w=FAKE + 8) == 4         # 16-byte alignment
        assert call(d, eps=-1.0) == 2           # eps >= 0
        assert call(d, eps=float("nan")) == 2
    assert v(d, cur=FAKE + 2) == 4
    d.T = 5
    assert v(d) == 2 and lz(d) == 2             # windows are at most 4 tokens
    d = good()
    d.S = 2                                     # verify needs S >= T + 1
    assert v(d) == 2


def test_status_strings_and_version(lib):
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_version.restype = ctypes.c_char_p
    for s in range(8):
        assert lib.gdn_status_string(s).startswith(b"GDN_")
    assert b"gfx950" in lib.gdn_version()


CEILING_HEADER = os.path.join(ROOT, "include", "gdn_ceiling.h")
CEILING_LIB = os.path.join(ROOT, "gated_deltanet_recurrence_conv_amd", "libgdn_ceiling.so")


def test_ceiling_library_exports_its_header():
    """libgdn_ceiling.so (the measured-ceiling loops) exports every function
    include/gdn_ceiling.h declares, its binding has the same names, and it
    refuses bad arguments with -1 before launching anything."""
    if not os.path.exists(CEILING_LIB):
        from gated_deltanet_recurrence_conv_amd import build
        build.build()
    text = open(CEILING_HEADER).read()
    names = sorted(set(re.findall(r"^\s*int\s+(gdn_ceiling_\w+)\s*\(", text, re.M)))
    assert names == ["gdn_ceiling_mfma_bf16", "gdn_ceiling_stream"]
    clib = ctypes.CDLL(CEILING_LIB)
    for n in names:
        assert hasattr(clib, n), n
    from gated_deltanet_recurrence_conv_amd import ceiling
    for n in names:
        assert hasattr(ceiling, n), n
    vp = ctypes.c_void_p
    clib.gdn_ceiling_stream.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_size_t, vp,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    clib.gdn_ceiling_mfma_bf16.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp]
    # too many buffers, no buffers, zero length, no sink for a read-only stream
    assert clib.gdn_ceiling_stream(None, 3, None, 1, 16, None, 1, 4, 1, None) == -1
    assert clib.gdn_ceiling_stream(None, 1, None, 1, 16, None, 1, 4, 1, None) == -1
    assert clib.gdn_ceiling_stream(None, 0, None, 0, 0, None, 1, 4, 1, None) == -1
    assert clib.gdn_ceiling_mfma_bf16(None, 1, 1, None) == -1
    assert clib.gdn_ceiling_mfma_bf16(vp(16), 0, 1, None) == -1
