"""Helpers shared by the GPU parity tests: device copies of the seeded inputs,
the blockwise error metric, and dims for both sides."""
from __future__ import annotations

import numpy as np

import oracle

FLAGS = 3  # SiLU + q/k L2 norm


def torch_mod():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch


def act_dtype(act):
    torch = torch_mod()
    return torch.bfloat16 if act == "bf16" else torch.float32


def dev(a, dtype=None):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda").contiguous()


def host(t) -> np.ndarray:
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def dims_pair(sh, T=None, B=None, L=None, S=None, scale=1.0, flags=FLAGS, out=None, l2_eps=1e-6):
    """(binding dims, oracle dims) for a workloads.Shape."""
    from gated_deltanet_recurrence_conv_amd import binding
    T = sh.T if T is None else T
    B = sh.B if B is None else B
    L = sh.L if L is None else L
    S = sh.S if S is None else S
    out = sh.out if out is None else out
    bd = binding.make_dims(L, B, T, sh.HV, sh.HK, sh.DK, sh.DV, S=S, act=sh.act, out=out,
                           scale=scale, l2_eps=l2_eps, flags=flags)
    od = oracle.Dims(L=L, B=B, T=T, HV=sh.HV, HK=sh.HK, DK=sh.DK, DV=sh.DV, S=S, scale=scale,
                     l2_eps=np.float64(np.float32(l2_eps)), flags=flags)
    return bd, od


def block_err(x, ref, block_axes) -> float:
    """Largest normwise error max|x - r| / max|r| over blocks; block_axes are
    the axes that form one block (e.g. (-2, -1) for a state tile).  A block
    whose reference is all zeros must be all zeros too: any nonzero (or NaN)
    value there gives an infinite error."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    diff = np.abs(x - ref)
    diff = np.where(np.isnan(diff), np.inf, diff)
    num = np.max(diff, axis=block_axes)
    den = np.max(np.abs(ref), axis=block_axes)
    zero = den == 0
    rel = np.where(zero, np.where(num == 0, 0.0, np.inf), num / np.where(zero, 1.0, den))
    return float(np.max(rel)) if rel.size else 0.0


def state_err(x, ref) -> float:
    return block_err(x, ref, (-2, -1))


def out_err(x, ref) -> float:
    """o is [L][B][T][HV][DV]; a block is one (layer, row, head) [T x DV]."""
    x = np.moveaxis(np.asarray(x, np.float64), 2, 3)
    ref = np.moveaxis(np.asarray(ref, np.float64), 2, 3)
    return block_err(x, ref, (-2, -1))


def tol(act):
    return 2e-3 if act == "bf16" else 1e-5
