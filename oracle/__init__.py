"""CPU oracle for the Gated DeltaNet verify / commit / rewind / conv-step /
prefill path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (the HIP library and its
Python binding) never imports it, and it imports nothing from the product.

The arithmetic lives in ``gdn_oracle.c``: plain sequential loops in IEEE
double, one token at a time.  This module only marshals numpy arrays to
float64 copies, calls the C functions and hands back fresh arrays; it never
mutates its arguments.

Page sources, readings and pins are listed in the header of ``gdn_oracle.c``.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FLAG_CONV_SILU = 1
FLAG_QK_L2NORM = 2


def build(force: bool = False) -> str:
    """Compile gdn_oracle.c with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-std=c99", "-Wall",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Dims(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("B", ctypes.c_int32), ("T", ctypes.c_int32),
                ("HV", ctypes.c_int32), ("HK", ctypes.c_int32), ("DK", ctypes.c_int32),
                ("DV", ctypes.c_int32), ("KCONV", ctypes.c_int32), ("S", ctypes.c_int32),
                ("scale", ctypes.c_double), ("l2_eps", ctypes.c_double),
                ("flags", ctypes.c_uint32)]


@dataclass
class Dims:
    L: int
    B: int
    T: int
    HV: int
    HK: int
    DK: int
    DV: int
    KCONV: int = 4
    S: int = 1
    scale: float = 1.0
    l2_eps: float = 1e-6
    flags: int = FLAG_CONV_SILU | FLAG_QK_L2NORM

    @property
    def C(self) -> int:
        return 2 * self.HK * self.DK + self.HV * self.DV

    def _c(self) -> _Dims:
        return _Dims(self.L, self.B, self.T, self.HV, self.HK, self.DK, self.DV, self.KCONV,
                     self.S, float(self.scale), float(self.l2_eps), int(self.flags))


_lib = None


def _bind(lib):
    vp, ip = ctypes.c_void_p, ctypes.c_int
    lib.ora_conv_step.argtypes = [ctypes.POINTER(_Dims)] + [vp] * 6 + [ip]
    lib.ora_conv_step.restype = None
    lib.ora_verify.argtypes = [ctypes.POINTER(_Dims)] + [vp] * 10
    lib.ora_verify.restype = ip
    lib.ora_commit.argtypes = [ctypes.POINTER(_Dims)] + [vp] * 5
    lib.ora_commit.restype = ip
    lib.ora_rewind.argtypes = [ctypes.POINTER(_Dims)] + [vp] * 10
    lib.ora_rewind.restype = ip
    lib.ora_prefill.argtypes = [ctypes.POINTER(_Dims)] + [vp] * 6
    lib.ora_prefill.restype = ip
    lib.ora_accept_greedy.argtypes = [ctypes.POINTER(_Dims)] + [vp] * 5
    lib.ora_accept_greedy.restype = None
    lib.ora_gated_rmsnorm.argtypes = [ctypes.POINTER(_Dims), vp, vp, vp, ctypes.c_double, vp, vp]
    lib.ora_gated_rmsnorm.restype = None
    return lib


def build_sanitized(path: str) -> str:
    """Compile gdn_oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer
    (clang, every report fatal) into `path`; the process that loads it must
    preload the clang sanitizer runtime."""
    clang = "/opt/rocm/llvm/bin/clang"
    subprocess.check_call([clang, "-O1", "-g", "-fno-omit-frame-pointer", "-std=c99", "-Wall",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-shared", "-fPIC", "-o", path, _SRC, "-lm"])
    return path


def _load():
    global _lib
    if _lib is None:
        # GDN_ORACLE_LIB: another build of gdn_oracle.c (the sanitizer run)
        path = os.environ.get("GDN_ORACLE_LIB") or build()
        _lib = _bind(ctypes.CDLL(path))
    return _lib


@contextlib.contextmanager
def library(path: str):
    """Route every call through another build of gdn_oracle.c for the
    duration of the block (used by the mutation test of the pins)."""
    global _lib
    saved = _load()
    _lib = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _f64(a, shape):
    if a is None:
        return None
    out = np.ascontiguousarray(np.asarray(a, dtype=np.float64)).copy()
    if out.size != int(np.prod(shape)):
        raise ValueError("oracle: expected %s elements for shape %s, got %d"
                         % (int(np.prod(shape)), shape, out.size))
    return out.reshape(shape)


def _i32(a, shape):
    if a is None:
        return None
    out = np.ascontiguousarray(np.asarray(a, dtype=np.int32)).copy()
    if out.size != int(np.prod(shape)):
        raise ValueError("oracle: bad int array size for shape %s" % (shape,))
    return out.reshape(shape)


def _u8(a, shape):
    if a is None:
        return None
    out = np.ascontiguousarray(np.asarray(a, dtype=np.uint8)).copy()
    if out.size != int(np.prod(shape)):
        raise ValueError("oracle: bad active size")
    return out.reshape(shape)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _shapes(d: Dims):
    C, km1 = d.C, d.KCONV - 1
    return dict(x=(d.L, d.B, d.T, C), conv_w=(d.L, C, d.KCONV), conv_b=(d.L, C),
                conv_state=(d.L, d.B, km1, C), g=(d.L, d.B, d.T, d.HV),
                beta=(d.L, d.B, d.T, d.HV), state=(d.L, d.B, d.S, d.HV, d.DK, d.DV),
                cur=(d.L, d.B), o=(d.L, d.B, d.T, d.HV, d.DV), keep=(d.B,), active=(d.B,))


def conv_step(d: Dims, x, conv_w, conv_b, conv_state, y_init=None, active=None,
              commit_state=True):
    """Returns (y, conv_state_after).  Rows that are inactive keep y_init."""
    s = _shapes(d)
    x_, w_, b_ = _f64(x, s["x"]), _f64(conv_w, s["conv_w"]), _f64(conv_b, s["conv_b"])
    cs = _f64(conv_state, s["conv_state"])
    y = _f64(y_init, s["x"]) if y_init is not None else np.zeros(s["x"], np.float64)
    act = _u8(active, s["active"])
    _load().ora_conv_step(ctypes.byref(d._c()), _p(x_), _p(w_), _p(b_), _p(cs), _p(y),
                          _p(act), int(bool(commit_state)))
    return y, cs


def verify(d: Dims, x, conv_w, conv_b, conv_state, g, beta, state, cur=None, active=None,
           o_init=None):
    """Returns (state_after, o, err).  Candidate t of row (l, b) lands in slot
    (cur + t + 1) mod S; slot cur and every other input are left as given."""
    s = _shapes(d)
    args = [_f64(x, s["x"]), _f64(conv_w, s["conv_w"]), _f64(conv_b, s["conv_b"]),
            _f64(conv_state, s["conv_state"]), _f64(g, s["g"]), _f64(beta, s["beta"])]
    st = _f64(state, s["state"])
    cu = _i32(cur, s["cur"])
    o = _f64(o_init, s["o"]) if o_init is not None else np.zeros(s["o"], np.float64)
    act = _u8(active, s["active"])
    err = _load().ora_verify(ctypes.byref(d._c()), *[_p(a) for a in args], _p(st), _p(cu),
                             _p(o), _p(act))
    return st, o, err


def commit(d: Dims, x, conv_state, cur, keep, active=None):
    """Returns (conv_state_after, cur_after, err)."""
    s = _shapes(d)
    x_ = _f64(x, s["x"])
    cs = _f64(conv_state, s["conv_state"])
    cu = _i32(cur, s["cur"])
    kp = _i32(keep, s["keep"])
    act = _u8(active, s["active"])
    err = _load().ora_commit(ctypes.byref(d._c()), _p(x_), _p(cs), _p(cu), _p(kp), _p(act))
    return cs, cu, err


def accept_greedy(d: Dims, draft, target, active=None, next_init=None):
    """draft [B][T-1], target [B][T] int32 token ids.  Returns (keep, next);
    next holds next_init (default -1) where nothing is written."""
    B, T = d.B, d.T
    dr = np.ascontiguousarray(np.asarray(draft, np.int32).reshape(B, max(T - 1, 0)))
    tg = np.ascontiguousarray(np.asarray(target, np.int32).reshape(B, T))
    act = None if active is None else np.ascontiguousarray(np.asarray(active, np.uint8).reshape(B))
    keep = np.zeros(B, np.int32)
    nxt = np.full(B, -1, np.int32) if next_init is None else np.array(next_init, np.int32).reshape(B)
    _load().ora_accept_greedy(ctypes.byref(d._c()), _p(dr), _p(tg), _p(act), _p(keep), _p(nxt))
    return keep, nxt


def gated_rmsnorm(d: Dims, o, z, w, eps=1e-6, active=None, y_init=None):
    """o, z [L][B][T][HV][DV]; w [L][DV].  Returns y (y_init where not written)."""
    s = _shapes(d)
    o_ = _f64(o, s["o"])
    z_ = _f64(z, s["o"])
    w_ = _f64(w, (d.L, d.DV))
    act = None if active is None else np.ascontiguousarray(np.asarray(active, np.uint8).reshape(d.B))
    y = _f64(y_init, s["o"]) if y_init is not None else np.zeros(s["o"], np.float64)
    _load().ora_gated_rmsnorm(ctypes.byref(d._c()), _p(o_), _p(z_), _p(w_), float(eps), _p(act), _p(y))
    return y


def rewind(d: Dims, x, conv_w, conv_b, conv_state, g, beta, state, cur, keep, o_init=None,
           want_o=True):
    """Returns (state_after, conv_state_after, o_or_None, err)."""
    s = _shapes(d)
    args = [_f64(x, s["x"]), _f64(conv_w, s["conv_w"]), _f64(conv_b, s["conv_b"])]
    cs = _f64(conv_state, s["conv_state"])
    g_, b_ = _f64(g, s["g"]), _f64(beta, s["beta"])
    st = _f64(state, s["state"])
    cu = _i32(cur, s["cur"])
    kp = _i32(keep, s["keep"])
    o = None
    if want_o:
        o = _f64(o_init, s["o"]) if o_init is not None else np.zeros(s["o"], np.float64)
    err = _load().ora_rewind(ctypes.byref(d._c()), *[_p(a) for a in args], _p(cs), _p(g_),
                             _p(b_), _p(st), _p(cu), _p(kp), _p(o))
    return st, cs, o, err


def prefill(d: Dims, y, g, beta, state, cur=None):
    """Token-sequential prefill over y (post-conv channels).
    Returns (state_after, o, err)."""
    s = _shapes(d)
    y_, g_, b_ = _f64(y, s["x"]), _f64(g, s["g"]), _f64(beta, s["beta"])
    st = _f64(state, s["state"])
    cu = _i32(cur, s["cur"])
    o = np.zeros(s["o"], np.float64)
    err = _load().ora_prefill(ctypes.byref(d._c()), _p(y_), _p(g_), _p(b_), _p(st), _p(cu),
                              _p(o))
    return st, o, err
