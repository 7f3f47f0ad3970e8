"""Brute-force float64 reference used only to pin the oracle on tiny shapes.

It is written in the explicit-matrix form of the gated delta rule, in math
layout (S is d_v x d_k), one token at a time:

    S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = scale * S_t q_t,

with explicit d_k x d_k matrices, and the causal conv as a sum of shifted
window slices weighted per channel.  It shares no code with the oracle
(gdn_oracle.c uses the rank-1 column form on h = S^T) or with the HIP path.

The update is the gated delta rule of "Gated Delta Networks: Improving
Mamba2 with Delta Rule" (Yang, Kautz, Hatamizadeh, ICLR 2025), the mixer the
page "perf(qwen): full-context MTP draft prefill and replay-free rewind"
(Summary item 4) reruns on captured verification inputs.
"""
from __future__ import annotations

import numpy as np


def conv_window(win: np.ndarray, w: np.ndarray, bias, silu: bool) -> np.ndarray:
    """win: (K-1+T, C) window, oldest row first; w: (C, K).  Returns (T, C)."""
    K = w.shape[1]
    T = win.shape[0] - (K - 1)
    out = np.zeros((T, win.shape[1]))
    for j in range(K):
        out += win[j:j + T, :] * w[:, j][None, :]
    if bias is not None:
        out += bias[None, :]
    if silu:
        out = out * (1.0 / (1.0 + np.exp(-out)))
    return out


def l2n(v: np.ndarray, eps: float) -> np.ndarray:
    return v / np.sqrt(np.dot(v, v) + eps)


def run_tokens(y_seq, g_seq, b_seq, h0_storage, HV, HK, DK, DV, scale=1.0, l2=True,
               eps=1e-6):
    """y_seq (T, C) post-conv channels, g_seq/b_seq (T, HV), h0_storage
    (HV, DK, DV).  Returns (list of storage-layout states after each token,
    o of shape (T, HV, DV))."""
    T = y_seq.shape[0]
    group = HV // HK
    S = [np.array(h0_storage[h], dtype=np.float64).T.copy() for h in range(HV)]  # (DV, DK)
    states, outs = [], np.zeros((T, HV, DV))
    eye = np.eye(DK)
    for t in range(T):
        y = np.asarray(y_seq[t], dtype=np.float64)
        for h in range(HV):
            m = h // group
            q = y[m * DK:(m + 1) * DK]
            k = y[HK * DK + m * DK: HK * DK + (m + 1) * DK]
            v = y[2 * HK * DK + h * DV: 2 * HK * DK + (h + 1) * DV]
            if l2:
                q, k = l2n(q, eps), l2n(k, eps)
            a = np.exp(np.float64(g_seq[t][h]))
            bt = np.float64(b_seq[t][h])
            S[h] = a * S[h] @ (eye - bt * np.outer(k, k)) + bt * np.outer(v, k)
            outs[t, h] = scale * (S[h] @ q)
        states.append(np.stack([S[h].T for h in range(HV)]))
    return states, outs


def verify_row(x_lb, cs_lb, w_l, b_l, g_lb, be_lb, h0, HV, HK, DK, DV, scale=1.0, silu=True,
               l2=True, eps=1e-6):
    """One (layer, row) of a verify window.  Returns (candidate states, o)."""
    win = np.concatenate([np.asarray(cs_lb, np.float64), np.asarray(x_lb, np.float64)], axis=0)
    y = conv_window(win, np.asarray(w_l, np.float64), None if b_l is None else
                    np.asarray(b_l, np.float64), silu)
    return run_tokens(y, g_lb, be_lb, h0, HV, HK, DK, DV, scale, l2, eps)
