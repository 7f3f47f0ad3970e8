"""Thin binding of libgdn_ceiling.so (include/gdn_ceiling.h): the hand-written
HBM stream and bf16 matrix-core loops that measure the GPU's sustained
ceilings.  Argument marshalling only; the loops run in HIP.  Measurement
infrastructure, not the Gated DeltaNet path."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn_ceiling.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libgdn_ceiling.so is not built (expected at %s); run "
                      "`python -m gated_deltanet_recurrence_conv_amd.build`" % LIB_PATH)

import torch  # noqa: E402  (bind to torch's HIP runtime first, as binding.py does)

_lib = ctypes.CDLL(LIB_PATH)
_vp = ctypes.c_void_p
_lib.gdn_ceiling_stream.argtypes = [_vp, ctypes.c_int, _vp, ctypes.c_int, ctypes.c_size_t, _vp,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp]
_lib.gdn_ceiling_stream.restype = ctypes.c_int
_lib.gdn_ceiling_mfma_bf16.argtypes = [_vp, ctypes.c_int, ctypes.c_int, _vp]
_lib.gdn_ceiling_mfma_bf16.restype = ctypes.c_int


def _stream_ptr():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_dev(t, name):
    if not (t.is_cuda and t.is_contiguous() and t.data_ptr() % 16 == 0):
        raise ValueError("%s must be a contiguous, 16-byte aligned GPU tensor" % name)


def gdn_ceiling_stream(srcs, dsts, n_vec16, sink=None, grid=1024, unroll=4, nontemporal=True,
                       blocked=False):
    """Streams n_vec16 16-byte vectors from each tensor of srcs into each of dsts
    (grid-stride, or per-workgroup contiguous 64 KiB blocks when blocked)."""
    for i, t in enumerate(list(srcs) + list(dsts)):
        _check_dev(t, "buffer %d" % i)
        if t.numel() * t.element_size() < 16 * n_vec16:
            raise ValueError("buffer %d is smaller than n_vec16 * 16 bytes" % i)
    if not dsts:
        if sink is None:
            raise ValueError("a read-only stream needs a sink tensor")
        _check_dev(sink, "sink")
        if sink.numel() * sink.element_size() < 16 * grid:
            raise ValueError("sink must hold one 16-byte vector per workgroup")
    src_arr = (ctypes.c_void_p * 2)(*[t.data_ptr() for t in srcs], *([0] * (2 - len(srcs))))
    dst_arr = (ctypes.c_void_p * 3)(*[t.data_ptr() for t in dsts], *([0] * (3 - len(dsts))))
    rc = _lib.gdn_ceiling_stream(src_arr, len(srcs), dst_arr, len(dsts), int(n_vec16),
                                 sink.data_ptr() if sink is not None else None, int(grid),
                                 int(unroll), (1 if nontemporal else 0) | (2 if blocked else 0),
                                 _stream_ptr())
    if rc != 0:
        raise RuntimeError("gdn_ceiling_stream failed (%d)" % rc)


def gdn_ceiling_mfma_bf16(out, grid, iters):
    """grid workgroups x 4 waves x iters x 8 bf16 16x16x32 MFMAs; out holds
    grid * 256 * 32 floats."""
    _check_dev(out, "out")
    if out.numel() < grid * 256 * 32 or out.dtype != torch.float32:
        raise ValueError("out must be float32 with grid * 256 * 32 elements")
    rc = _lib.gdn_ceiling_mfma_bf16(out.data_ptr(), int(grid), int(iters), _stream_ptr())
    if rc != 0:
        raise RuntimeError("gdn_ceiling_mfma_bf16 failed (%d)" % rc)
