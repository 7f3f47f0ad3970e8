"""Thin Python binding of libgdn.so (the C ABI declared in include/gdn.h).

Argument marshalling only: every function takes torch tensors that live on
the GPU (or raw device addresses as ints), checks that each one has the
dtype, size and layout the dims imply -- so that no kernel can be launched
on a buffer smaller than its grid assumes -- and calls the C entry point of
the same name on the current torch stream.  All arithmetic happens in the
HIP kernels; there is no CPU path.  Importing this module fails loudly if
libgdn.so has not been built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libgdn.so is not built (expected at %s); run "
                      "`python -m gated_deltanet_recurrence_conv_amd.build` -- there is no "
                      "fallback path" % LIB_PATH)

# PyTorch ships its own HIP runtime (SONAME libamdhip64.so.7).  Importing
# torch first makes the dynamic loader bind libgdn.so to that same runtime, so
# the process has one HIP runtime and torch's device memory and streams are
# valid in libgdn's calls.  Loading libgdn.so first would pull in a second
# runtime that sees no device.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

GDN_OK = 0
STATUS_NAMES = {0: "GDN_OK", 1: "GDN_E_NULL", 2: "GDN_E_SHAPE", 3: "GDN_E_DTYPE",
                4: "GDN_E_ALIGN", 5: "GDN_E_UNSUPPORTED", 6: "GDN_E_WORKSPACE", 7: "GDN_E_HIP"}
GDN_F32, GDN_BF16 = 0, 1
FLAG_CONV_SILU, FLAG_QK_L2NORM = 1, 2
ERR_KEEP, ERR_SLOT, ERR_INACTIVE_KEEP = 1, 2, 4


class gdn_dims(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("B", ctypes.c_int32), ("T", ctypes.c_int32),
                ("HV", ctypes.c_int32), ("HK", ctypes.c_int32), ("DK", ctypes.c_int32),
                ("DV", ctypes.c_int32), ("KCONV", ctypes.c_int32), ("S", ctypes.c_int32),
                ("act", ctypes.c_int32), ("out", ctypes.c_int32),
                ("scale", ctypes.c_float), ("l2_eps", ctypes.c_float),
                ("flags", ctypes.c_uint32)]


_DT = {"f32": GDN_F32, "fp32": GDN_F32, "float32": GDN_F32, "bf16": GDN_BF16,
       "bfloat16": GDN_BF16}


def make_dims(L, B, T, HV, HK, DK, DV, S=1, act="bf16", out="f32", scale=1.0, l2_eps=1e-6,
              flags=FLAG_CONV_SILU | FLAG_QK_L2NORM, KCONV=4) -> gdn_dims:
    return gdn_dims(int(L), int(B), int(T), int(HV), int(HK), int(DK), int(DV), int(KCONV),
                    int(S), _DT[act] if isinstance(act, str) else int(act),
                    _DT[out] if isinstance(out, str) else int(out), float(scale),
                    float(l2_eps), int(flags))


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.gdn_status_string(status)
        text = "%s: %s" % (where, msg.decode() if msg else STATUS_NAMES.get(status))
        if status == 7:
            text += " (%s)" % _lib.gdn_last_hip_error().decode()
        super().__init__(text)


_vp, _i32 = ctypes.c_void_p, ctypes.c_int32
_D = ctypes.POINTER(gdn_dims)
_lib.gdn_conv_step.argtypes = [_D, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp]
_lib.gdn_verify.argtypes = [_D] + [_vp] * 12
_lib.gdn_commit.argtypes = [_D] + [_vp] * 7
_lib.gdn_rewind.argtypes = [_D] + [_vp] * 12
_lib.gdn_verify_lazy.argtypes = [_D] + [_vp] * 16
_lib.gdn_accept_greedy.argtypes = [_D] + [_vp] * 6
_lib.gdn_gated_rmsnorm.argtypes = [_D, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp]
# (dims, 8 inputs, z, norm_w, eps, y, active, err, stream); the lazy form adds
# x_prev, g_prev, beta_prev and keep_prev in front of x
_lib.gdn_verify_gated_norm.argtypes = [_D] + [_vp] * 10 + [ctypes.c_float] + [_vp] * 4
_lib.gdn_verify_lazy_gated_norm.argtypes = [_D] + [_vp] * 14 + [ctypes.c_float] + [_vp] * 4
_lib.gdn_prefill_ragged.argtypes = [_D, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp,
                                    ctypes.c_size_t, _vp, _vp]
_lib.gdn_prefill_chunked.argtypes = [_D, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp,
                                     ctypes.c_size_t, _vp, _vp]
_lib.gdn_prefill_chunked_noalloc.argtypes = [_D, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp]
_lib.gdn_prefill_conv_chunked.argtypes = [_D] + [_vp] * 9 + [_i32, _vp, ctypes.c_size_t, _vp, _vp]
_lib.gdn_workspace_size.argtypes = [_D, _i32]
_lib.gdn_workspace_size.restype = ctypes.c_size_t
_lib.gdn_status_string.argtypes = [ctypes.c_int]
_lib.gdn_status_string.restype = ctypes.c_char_p
_lib.gdn_version.argtypes = []
_lib.gdn_version.restype = ctypes.c_char_p
_lib.gdn_last_hip_error.argtypes = []
_lib.gdn_last_hip_error.restype = ctypes.c_char_p
for _n in ("gdn_conv_step", "gdn_verify", "gdn_commit", "gdn_rewind", "gdn_verify_lazy",
           "gdn_accept_greedy", "gdn_gated_rmsnorm", "gdn_verify_gated_norm",
           "gdn_verify_lazy_gated_norm", "gdn_prefill_chunked", "gdn_prefill_ragged",
           "gdn_prefill_chunked_noalloc", "gdn_prefill_conv_chunked"):
    getattr(_lib, _n).restype = ctypes.c_int

EXPORTED = ("gdn_conv_step", "gdn_verify", "gdn_commit", "gdn_rewind", "gdn_verify_lazy",
            "gdn_accept_greedy", "gdn_gated_rmsnorm", "gdn_verify_gated_norm",
            "gdn_verify_lazy_gated_norm", "gdn_prefill_chunked", "gdn_prefill_ragged",
            "gdn_prefill_chunked_noalloc", "gdn_prefill_conv_chunked", "gdn_workspace_size",
            "gdn_status_string", "gdn_version", "gdn_last_hip_error")


def _torch():
    import torch
    return torch


def _act_dtype(code):
    torch = _torch()
    return torch.bfloat16 if code == GDN_BF16 else torch.float32


def _arg(t, name, shape=None, dtype=None, optional=False):
    """Device address of a tensor (or an int address) after checking it."""
    if t is None:
        if optional:
            return None
        raise GdnError(1, "%s is required" % name)
    if isinstance(t, int):
        return t
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s: expected a torch.Tensor or a device address" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if t.device.index is not None and t.device.index != torch.cuda.current_device():
        raise ValueError("%s is on %s but the current device is cuda:%d (launches go to the "
                         "current device)" % (name, t.device, torch.cuda.current_device()))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if shape is not None:
        n = 1
        for s in shape:
            n *= int(s)
        if t.numel() != n:
            raise ValueError("%s must hold %d elements for shape %s (got %d)"
                             % (name, n, tuple(shape), t.numel()))
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _shapes(d: gdn_dims):
    C = 2 * d.HK * d.DK + d.HV * d.DV
    return dict(x=(d.L, d.B, d.T, C), conv_w=(d.L, C, d.KCONV), conv_b=(d.L, C),
                conv_state=(d.L, d.B, d.KCONV - 1, C), g=(d.L, d.B, d.T, d.HV),
                state=(d.L, d.B, d.S, d.HV, d.DK, d.DV), cur=(d.L, d.B),
                o=(d.L, d.B, d.T, d.HV, d.DV), rows=(d.B,), err=(1,))


def _check(status, where):
    if status != GDN_OK:
        raise GdnError(status, where)


def gdn_conv_step(d, x, conv_w, conv_b, conv_state, y, active=None, commit_state=True,
                  err=None, stream=None):
    torch, s = _torch(), _shapes(d)
    A, O = _act_dtype(d.act), _act_dtype(d.out)
    _check(_lib.gdn_conv_step(
        ctypes.byref(d), _arg(x, "x", s["x"], A), _arg(conv_w, "conv_w", s["conv_w"], A),
        _arg(conv_b, "conv_b", s["conv_b"], A, True), _arg(conv_state, "conv_state",
                                                             s["conv_state"], A),
        _arg(y, "y", s["x"], O), _arg(active, "active", s["rows"], torch.uint8, True),
        int(bool(commit_state)), _arg(err, "err", s["err"], torch.int32, True),
        _stream(stream)), "gdn_conv_step")


def gdn_verify(d, x, conv_w, conv_b, conv_state, g, beta, state, cur, o, active=None, err=None,
               stream=None):
    torch, s = _torch(), _shapes(d)
    A, O = _act_dtype(d.act), _act_dtype(d.out)
    _check(_lib.gdn_verify(
        ctypes.byref(d), _arg(x, "x", s["x"], A), _arg(conv_w, "conv_w", s["conv_w"], A),
        _arg(conv_b, "conv_b", s["conv_b"], A, True),
        _arg(conv_state, "conv_state", s["conv_state"], A), _arg(g, "g", s["g"], A),
        _arg(beta, "beta", s["g"], A), _arg(state, "state", s["state"], torch.float32),
        _arg(cur, "cur", s["cur"], torch.int32, True), _arg(o, "o", s["o"], O),
        _arg(active, "active", s["rows"], torch.uint8, True),
        _arg(err, "err", s["err"], torch.int32, True), _stream(stream)), "gdn_verify")


def gdn_commit(d, x, conv_state, cur, keep, active=None, err=None, stream=None):
    torch, s = _torch(), _shapes(d)
    A = _act_dtype(d.act)
    _check(_lib.gdn_commit(
        ctypes.byref(d), _arg(x, "x", s["x"], A),
        _arg(conv_state, "conv_state", s["conv_state"], A),
        _arg(cur, "cur", s["cur"], torch.int32), _arg(keep, "keep", s["rows"], torch.int32),
        _arg(active, "active", s["rows"], torch.uint8, True),
        _arg(err, "err", s["err"], torch.int32, True), _stream(stream)), "gdn_commit")


def gdn_rewind(d, x, conv_w, conv_b, conv_state, g, beta, state, cur, keep, o=None, err=None,
               stream=None):
    torch, s = _torch(), _shapes(d)
    A, O = _act_dtype(d.act), _act_dtype(d.out)
    _check(_lib.gdn_rewind(
        ctypes.byref(d), _arg(x, "x", s["x"], A), _arg(conv_w, "conv_w", s["conv_w"], A),
        _arg(conv_b, "conv_b", s["conv_b"], A, True),
        _arg(conv_state, "conv_state", s["conv_state"], A), _arg(g, "g", s["g"], A),
        _arg(beta, "beta", s["g"], A), _arg(state, "state", s["state"], torch.float32),
        _arg(cur, "cur", s["cur"], torch.int32, True),
        _arg(keep, "keep", s["rows"], torch.int32), _arg(o, "o", s["o"], O, True),
        _arg(err, "err", s["err"], torch.int32, True), _stream(stream)), "gdn_rewind")


def gdn_verify_lazy(d, x_prev, g_prev, beta_prev, keep_prev, x, conv_w, conv_b, conv_state, g,
                    beta, state, cur, o, active=None, err=None, stream=None):
    torch, s = _torch(), _shapes(d)
    A, O = _act_dtype(d.act), _act_dtype(d.out)
    _check(_lib.gdn_verify_lazy(
        ctypes.byref(d), _arg(x_prev, "x_prev", s["x"], A, True),
        _arg(g_prev, "g_prev", s["g"], A, True), _arg(beta_prev, "beta_prev", s["g"], A, True),
        _arg(keep_prev, "keep_prev", s["rows"], torch.int32, True),
        _arg(x, "x", s["x"], A), _arg(conv_w, "conv_w", s["conv_w"], A),
        _arg(conv_b, "conv_b", s["conv_b"], A, True),
        _arg(conv_state, "conv_state", s["conv_state"], A), _arg(g, "g", s["g"], A),
        _arg(beta, "beta", s["g"], A), _arg(state, "state", s["state"], torch.float32),
        _arg(cur, "cur", s["cur"], torch.int32, True), _arg(o, "o", s["o"], O),
        _arg(active, "active", s["rows"], torch.uint8, True),
        _arg(err, "err", s["err"], torch.int32, True), _stream(stream)), "gdn_verify_lazy")


def gdn_verify_gated_norm(d, x, conv_w, conv_b, conv_state, g, beta, state, cur, z, norm_w, y,
                          eps=1e-6, active=None, err=None, stream=None):
    """gdn_verify with the gated RMSNorm applied to the outputs in the same
    launch: y = RMSNorm(o) * norm_w * SiLU(z) (z: o's shape in the act dtype,
    norm_w: [L, DV] in the act dtype, y: o's shape in the out dtype)."""
    torch, s = _torch(), _shapes(d)
    A, O = _act_dtype(d.act), _act_dtype(d.out)
    _check(_lib.gdn_verify_gated_norm(
        ctypes.byref(d), _arg(x, "x", s["x"], A), _arg(conv_w, "conv_w", s["conv_w"], A),
        _arg(conv_b, "conv_b", s["conv_b"], A, True),
        _arg(conv_state, "conv_state", s["conv_state"], A), _arg(g, "g", s["g"], A),
        _arg(beta, "beta", s["g"], A), _arg(state, "state", s["state"], torch.float32),
        _arg(cur, "cur", s["cur"], torch.int32, True), _arg(z, "z", s["o"], A),
        _arg(norm_w, "norm_w", (d.L, d.DV), A), float(eps), _arg(y, "y", s["o"], O),
        _arg(active, "active", s["rows"], torch.uint8, True),
        _arg(err, "err", s["err"], torch.int32, True), _stream(stream)), "gdn_verify_gated_norm")


def gdn_verify_lazy_gated_norm(d, x_prev, g_prev, beta_prev, keep_prev, x, conv_w, conv_b,
                               conv_state, g, beta, state, cur, z, norm_w, y, eps=1e-6,
                               active=None, err=None, stream=None):
    """gdn_verify_lazy with the gated RMSNorm of gdn_verify_gated_norm fused
    into the new window's outputs."""
    torch, s = _torch(), _shapes(d)
    A, O = _act_dtype(d.act), _act_dtype(d.out)
    _check(_lib.gdn_verify_lazy_gated_norm(
        ctypes.byref(d), _arg(x_prev, "x_prev", s["x"], A, True),
        _arg(g_prev, "g_prev", s["g"], A, True), _arg(beta_prev, "beta_prev", s["g"], A, True),
        _arg(keep_prev, "keep_prev", s["rows"], torch.int32, True),
        _arg(x, "x", s["x"], A), _arg(conv_w, "conv_w", s["conv_w"], A),
        _arg(conv_b, "conv_b", s["conv_b"], A, True),
        _arg(conv_state, "conv_state", s["conv_state"], A), _arg(g, "g", s["g"], A),
        _arg(beta, "beta", s["g"], A), _arg(state, "state", s["state"], torch.float32),
        _arg(cur, "cur", s["cur"], torch.int32, True), _arg(z, "z", s["o"], A),
        _arg(norm_w, "norm_w", (d.L, d.DV), A), float(eps), _arg(y, "y", s["o"], O),
        _arg(active, "active", s["rows"], torch.uint8, True),
        _arg(err, "err", s["err"], torch.int32, True), _stream(stream)),
        "gdn_verify_lazy_gated_norm")


def gdn_workspace_size(d, chunk=64) -> int:
    return int(_lib.gdn_workspace_size(ctypes.byref(d), int(chunk)))


def gdn_accept_greedy(d, draft_ids, target_ids, keep, active=None, next_ids=None, stream=None):
    torch = _torch()
    B, T = d.B, d.T
    _check(_lib.gdn_accept_greedy(
        ctypes.byref(d), _arg(draft_ids, "draft_ids", (B, T - 1), torch.int32, True) if T > 1 else None,
        _arg(target_ids, "target_ids", (B, T), torch.int32), _arg(active, "active", (B,), torch.uint8, True),
        _arg(keep, "keep", (B,), torch.int32), _arg(next_ids, "next_ids", (B,), torch.int32, True),
        _stream(stream)), "gdn_accept_greedy")


def gdn_gated_rmsnorm(d, o, z, w, y, eps=1e-6, active=None, stream=None):
    s = _shapes(d)
    A, O = _act_dtype(d.act), _act_dtype(d.out)
    _check(_lib.gdn_gated_rmsnorm(
        ctypes.byref(d), _arg(o, "o", s["o"], O), _arg(z, "z", s["o"], A),
        _arg(w, "w", (d.L, d.DV), A), float(eps), _arg(y, "y", s["o"], O),
        _arg(active, "active", s["rows"], _torch().uint8, True), _stream(stream)),
        "gdn_gated_rmsnorm")


def _workspace(d, chunk, workspace):
    need = gdn_workspace_size(d, chunk)
    if workspace is None:
        return None, 0
    if isinstance(workspace, int):
        raise TypeError("workspace must be a tensor so that its size is known")
    ptr = _arg(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise ValueError("workspace holds %d bytes, %d needed" % (nbytes, need))
    return ptr, nbytes


def gdn_prefill_chunked(d, y, g, beta, state, cur, o, chunk=64, workspace=None, err=None,
                        stream=None):
    torch, s = _torch(), _shapes(d)
    A, O = _act_dtype(d.act), _act_dtype(d.out)
    ws_ptr, ws_bytes = _workspace(d, chunk, workspace)
    _check(_lib.gdn_prefill_chunked(
        ctypes.byref(d), _arg(y, "y", s["x"], A), _arg(g, "g", s["g"], A),
        _arg(beta, "beta", s["g"], A), _arg(state, "state", s["state"], torch.float32),
        _arg(cur, "cur", s["cur"], torch.int32, True), _arg(o, "o", s["o"], O), int(chunk),
        ws_ptr, ws_bytes, _arg(err, "err", s["err"], torch.int32, True), _stream(stream)),
        "gdn_prefill_chunked")


def gdn_prefill_conv_chunked(d, x, conv_w, conv_b, conv_state, g, beta, state, cur, o, chunk=64,
                             workspace=None, err=None, stream=None):
    torch, s = _torch(), _shapes(d)
    A, O = _act_dtype(d.act), _act_dtype(d.out)
    ws_ptr, ws_bytes = _workspace(d, chunk, workspace)
    _check(_lib.gdn_prefill_conv_chunked(
        ctypes.byref(d), _arg(x, "x", s["x"], A), _arg(conv_w, "conv_w", s["conv_w"], A),
        _arg(conv_b, "conv_b", s["conv_b"], A, True),
        _arg(conv_state, "conv_state", s["conv_state"], A), _arg(g, "g", s["g"], A),
        _arg(beta, "beta", s["g"], A), _arg(state, "state", s["state"], torch.float32),
        _arg(cur, "cur", s["cur"], torch.int32, True), _arg(o, "o", s["o"], O), int(chunk),
        ws_ptr, ws_bytes, _arg(err, "err", s["err"], torch.int32, True), _stream(stream)),
        "gdn_prefill_conv_chunked")


GDN_NOALLOC_SCRATCH_BYTES = 64 << 20


def gdn_prefill_chunked_noalloc(d, y, g, beta, state, cur, o, chunk=64, err=None, stream=None):
    """gdn_prefill_chunked with the library's static device scratch in place of
    a workspace (no allocation in the call); calls that overlap in time on one
    GPU race."""
    torch, s = _torch(), _shapes(d)
    A, O = _act_dtype(d.act), _act_dtype(d.out)
    _check(_lib.gdn_prefill_chunked_noalloc(
        ctypes.byref(d), _arg(y, "y", s["x"], A), _arg(g, "g", s["g"], A),
        _arg(beta, "beta", s["g"], A), _arg(state, "state", s["state"], torch.float32),
        _arg(cur, "cur", s["cur"], torch.int32, True), _arg(o, "o", s["o"], O), int(chunk),
        _arg(err, "err", s["err"], torch.int32, True), _stream(stream)),
        "gdn_prefill_chunked_noalloc")


def gdn_prefill_ragged(d, y, g, beta, state, cur, o, lengths, chunk=64, workspace=None, err=None,
                       stream=None):
    torch, s = _torch(), _shapes(d)
    A, O = _act_dtype(d.act), _act_dtype(d.out)
    ws_ptr, ws_bytes = _workspace(d, chunk, workspace)
    _check(_lib.gdn_prefill_ragged(
        ctypes.byref(d), _arg(y, "y", s["x"], A), _arg(g, "g", s["g"], A),
        _arg(beta, "beta", s["g"], A), _arg(state, "state", s["state"], torch.float32),
        _arg(cur, "cur", s["cur"], torch.int32, True), _arg(o, "o", s["o"], O),
        _arg(lengths, "lengths", s["rows"], torch.int32), int(chunk),
        ws_ptr, ws_bytes, _arg(err, "err", s["err"], torch.int32, True), _stream(stream)),
        "gdn_prefill_ragged")


def gdn_status_string(status: int) -> str:
    return _lib.gdn_status_string(int(status)).decode()


def gdn_version() -> str:
    return _lib.gdn_version().decode()


def gdn_last_hip_error() -> str:
    return _lib.gdn_last_hip_error().decode()


def raw_library():
    """The loaded ctypes library (for calls with raw pointers)."""
    return _lib
