"""Seeded synthetic inputs for the Gated DeltaNet verify / commit / rewind /
prefill path.

This module is shared by the tests, the benchmark and the smoke check, and
feeds both the HIP path and the CPU oracle.  It holds none of the method's
arithmetic: it only draws random numbers, shapes them to the documented
distributions and rounds them to the activation dtype.  It imports nothing
from the rest of the package.

Every array is returned as numpy; floating arrays are float32 holding values
that are exactly representable in the requested activation dtype (bf16
values are produced by round-to-nearest-even from float32), so the device
copy (torch bf16/fp32) and the oracle's float64 copy hold identical numbers.

Distributions (the pages use real prompts and trained checkpoints, which are
not available; these stand in for them at the pages' shapes):
  x, conv_state ~ N(0, 1); conv_w ~ N(0, 0.5^2); g = -softplus(N(0, 1))
  (so a = exp(g) in (0, 1)); beta = sigmoid(N(0, 1)); state ~ N(0, 0.1^2).
Draw order is fixed: x, conv_state, conv_w, g, beta, state.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np


def bf16_round(a) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + (((u >> 16) & 1) + 0x7FFF)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def _act(a, act: str) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32)
    return bf16_round(a) if act == "bf16" else np.ascontiguousarray(a)


def _softplus(z):
    return np.log1p(np.exp(z))


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


@dataclass(frozen=True)
class Shape:
    """One workload's sizes.  C = 2*HK*DK + HV*DV conv channels."""
    name: str
    L: int
    B: int
    T: int
    HV: int
    HK: int
    DK: int
    DV: int
    S: int
    act: str = "bf16"          # dtype of x, conv_w, conv_state, g, beta, y
    out: str = "f32"           # dtype of o
    KCONV: int = 4
    inactive: tuple = field(default_factory=tuple)

    @property
    def C(self) -> int:
        return 2 * self.HK * self.DK + self.HV * self.DV

    def with_(self, **kw) -> "Shape":
        return replace(self, **kw)


# The workloads the pages' shapes call for.
TINY = Shape("tiny_b1_t2_hv2_hk1_d16_f32", L=1, B=1, T=2, HV=2, HK=1, DK=16, DV=16, S=3,
             act="f32", out="f32")
COHORT = Shape("qwen_verify_cohort_b8_t2_hv32_hk16_d128", L=1, B=8, T=2, HV=32, HK=16,
               DK=128, DV=128, S=3, inactive=(1, 6))
SOLO = Shape("qwen_solo_verify_b1_t3_l30", L=30, B=1, T=3, HV=32, HK=16, DK=128, DV=128, S=4)
REWIND = Shape("qwen_rewind_b8_t4", L=1, B=8, T=4, HV=32, HK=16, DK=128, DV=128, S=5)
PREFILL = Shape("qwen_prefill_b1_4096_in_1024_calls_chunk64", L=1, B=1, T=1024, HV=32, HK=16,
                DK=128, DV=128, S=1)
PREFILL_TOKENS = 4096
PREFILL_CHUNK = 64


def verify_inputs(sh: Shape, seed: int) -> dict:
    """Inputs of one verify/commit/rewind call: x, conv_w, conv_state, g, beta
    (activation dtype), state (fp32, S slots, every slot drawn), cur (int32,
    zeros) and active (uint8, zeros on the shape's inactive rows)."""
    rng = np.random.default_rng(seed)
    L, B, T, C = sh.L, sh.B, sh.T, sh.C
    x = rng.standard_normal((L, B, T, C), dtype=np.float32)
    conv_state = rng.standard_normal((L, B, sh.KCONV - 1, C), dtype=np.float32)
    conv_w = 0.5 * rng.standard_normal((L, C, sh.KCONV), dtype=np.float32)
    g = -_softplus(rng.standard_normal((L, B, T, sh.HV), dtype=np.float32))
    beta = _sigmoid(rng.standard_normal((L, B, T, sh.HV), dtype=np.float32))
    state = 0.1 * rng.standard_normal((L, B, sh.S, sh.HV, sh.DK, sh.DV), dtype=np.float32)
    active = np.ones(B, np.uint8)
    for r in sh.inactive:
        if r < B:
            active[r] = 0
    return dict(x=_act(x, sh.act), conv_w=_act(conv_w, sh.act),
                conv_state=_act(conv_state, sh.act), g=_act(g, sh.act),
                beta=_act(beta, sh.act), state=np.ascontiguousarray(state, np.float32),
                cur=np.zeros((L, B), np.int32), active=active)


def keep_uniform(rng: np.random.Generator, sh: Shape, active=None) -> np.ndarray:
    """keep ~ U{0..T} per row; inactive rows get 0."""
    keep = rng.integers(0, sh.T + 1, size=sh.B).astype(np.int32)
    if active is not None:
        keep[np.asarray(active) == 0] = 0
    return keep


def keep_prefix_acceptance(rng: np.random.Generator, sh: Shape, p: float = 0.8) -> np.ndarray:
    """keep = 1 + number of leading accepted drafts, each accepted with
    probability p, stopping at the first rejection (T-1 drafts per window)."""
    keep = np.ones(sh.B, np.int32)
    for b in range(sh.B):
        for _ in range(sh.T - 1):
            if rng.random() < p:
                keep[b] += 1
            else:
                break
    return keep


def prefill_inputs(sh: Shape, seed: int, tokens: int | None = None, unit_qk: bool = True) -> dict:
    """Post-conv prefill inputs for `tokens` tokens: y = [q | k | v] channels
    (q, k ~ N(0,1), L2-normalised per head when unit_qk, then rounded to the
    activation dtype; v ~ N(0,1)), g, beta, and a zero fp32 state (one slot)."""
    rng = np.random.default_rng(seed)
    T = sh.T if tokens is None else tokens
    L, B = sh.L, sh.B
    q = rng.standard_normal((L, B, T, sh.HK, sh.DK), dtype=np.float32)
    k = rng.standard_normal((L, B, T, sh.HK, sh.DK), dtype=np.float32)
    v = rng.standard_normal((L, B, T, sh.HV, sh.DV), dtype=np.float32)
    if unit_qk:
        q = q / np.sqrt(np.sum(q.astype(np.float64) ** 2, axis=-1, keepdims=True)).astype(np.float32)
        k = k / np.sqrt(np.sum(k.astype(np.float64) ** 2, axis=-1, keepdims=True)).astype(np.float32)
    y = np.concatenate([q.reshape(L, B, T, -1), k.reshape(L, B, T, -1), v.reshape(L, B, T, -1)],
                       axis=-1)
    g = -_softplus(rng.standard_normal((L, B, T, sh.HV), dtype=np.float32))
    beta = _sigmoid(rng.standard_normal((L, B, T, sh.HV), dtype=np.float32))
    state = np.zeros((L, B, sh.S, sh.HV, sh.DK, sh.DV), np.float32)
    return dict(y=_act(y, sh.act), g=_act(g, sh.act), beta=_act(beta, sh.act), state=state,
                cur=np.zeros((L, B), np.int32))


def random_state(sh: Shape, seed: int, std: float = 0.1) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (std * rng.standard_normal((sh.L, sh.B, sh.S, sh.HV, sh.DK, sh.DV),
                                      dtype=np.float32)).astype(np.float32)
