"""Numpy model of the chunked (WY/UT) form of the gated delta rule, used to
check the algorithm the prefill kernels implement against the sequential
oracle, and to study where bf16 operands may be used.

Per chunk of n <= C tokens starting from state H (d_k x d_v, storage layout
h = S^T), with G_r = sum_{i<=r} g_i, gamma_r = exp(G_r), E_ri = exp(G_r - G_i):

    A   = strictly_lower(diag(beta) E o (K K^T))
    T   = (I + A)^{-1}                              (UT transform)
    U~  = T diag(beta) V,   W~ = T diag(beta gamma) K
    U   = U~ - W~ H
    O   = scale (diag(gamma) Q H + (lower_incl o E o Q K^T) U)
    H'  = gamma_n H + (diag(exp(G_n - G)) K)^T U

(Yang et al., "Parallelizing Linear Transformers with the Delta Rule over
Sequence Length", NeurIPS 2024, applied to the gated rule of "Gated Delta
Networks", ICLR 2025.)  q and k are L2-normalised per token first.  The
chunked recurrence differs from the sequential one only in rounding ("MTP
inference: review and commit structure", Verification and limits).

`bf16` selects emulated bf16 MFMA operands with fp32 accumulation modelled in
float64: each product's operands are exact inputs ('x'), split into hi + lo
bf16 parts ('s', three products, lo x lo dropped) or rounded to bf16 once
('b').  KERNEL_PLAN is the plan the prefill kernels use; `plan` overrides
entries of it.  This module shares no code with the oracle or the HIP path.
"""
from __future__ import annotations

import numpy as np


def _bf16(x):
    x = np.asarray(x, np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + (((u >> 16) & 1) + 0x7FFF)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _split(x):
    x = np.asarray(x, np.float32)
    hi = _bf16(x)
    lo = _bf16(x - hi)
    return hi.astype(np.float64), lo.astype(np.float64)


def _mm(a, b, plan):
    """a @ b with operands 'x' (exact input), 's' (split hi+lo) or 'b' (one
    bf16 rounding); plan = (kind_a, kind_b); None means float64."""
    if plan is None:
        return a @ b
    ka, kb = plan
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if ka == "s" and kb == "s":
        ah, al = _split(a)
        bh, bl = _split(b)
        return ah @ bh + ah @ bl + al @ bh
    if ka == "s":
        ah, al = _split(a)
        bb = b if kb == "x" else _bf16(b).astype(np.float64)
        return ah @ bb + al @ bb
    if kb == "s":
        bh, bl = _split(b)
        aa = a if ka == "x" else _bf16(a).astype(np.float64)
        return aa @ bh + aa @ bl
    aa = a if ka == "x" else _bf16(a).astype(np.float64)
    bb = b if kb == "x" else _bf16(b).astype(np.float64)
    return aa @ bb


# Operand treatment per product, as in the prefill kernels: K K^T and Q K^T
# take the exact bf16 inputs; T diag(beta) is split for U~ and T diag(beta
# gamma / |k|) rounded once for W~; W~ and H are each rounded once inside
# W~ H; H is split inside Q H; P and U are split inside P U; diag(s) U is
# split inside K^T diag(s) U.
KERNEL_PLAN = dict(kk=("x", "x"), qk=("x", "x"), tv=("s", "x"), tk=("b", "x"), wh=("b", "b"),
                   qh=("x", "s"), pu=("s", "s"), ku=("x", "s"))


def chunked_head(q, k, v, g, beta, H0, chunk=64, scale=1.0, l2=True, eps=1e-6, bf16=False,
                 plan=None):
    """q, k (T, dk) raw; v (T, dv); g, beta (T,); H0 (dk, dv).
    Returns (H_T, O)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    T = q.shape[0]
    H = np.array(H0, np.float64)
    O = np.zeros((T, v.shape[1]))
    P = {} if not bf16 else dict(KERNEL_PLAN, **(plan or {}))
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(c0 + chunk, T))
        n = sl.stop - sl.start
        nq = np.sqrt((q[sl] ** 2).sum(1) + eps) if l2 else np.ones(n)
        nk = np.sqrt((k[sl] ** 2).sum(1) + eps) if l2 else np.ones(n)
        G = np.cumsum(g[sl])
        gam = np.exp(G)
        E = np.exp(G[:, None] - G[None, :])
        low_strict = np.tril(np.ones((n, n)), -1)
        low_incl = np.tril(np.ones((n, n)), 0)
        KK = _mm(k[sl], k[sl].T, P.get("kk")) / np.outer(nk, nk)
        A = low_strict * beta[sl][:, None] * E * KK
        Tm = np.linalg.inv(np.eye(n) + A)
        if bf16:
            Tm = Tm.astype(np.float32).astype(np.float64)
        Ut = _mm(Tm * beta[sl][None, :], v[sl], P.get("tv"))
        Wt = _mm(Tm * (beta[sl] * gam / nk)[None, :], k[sl], P.get("tk"))
        U = Ut - _mm(Wt, H, P.get("wh"))
        Pm = low_incl * E * _mm(q[sl], k[sl].T, P.get("qk")) / np.outer(nq, nk) * scale
        O[sl] = (scale * gam / nq)[:, None] * _mm(q[sl], H, P.get("qh")) + _mm(Pm, U, P.get("pu"))
        s = np.exp(G[-1] - G) / nk
        H = gam[-1] * H + _mm(k[sl].T, s[:, None] * U, P.get("ku"))
    return H, O
