"""Seeded synthetic inputs for the log-linear attention forward and decode step.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic, so both the CPU oracle (``oracle/``) and the GPU library
can take their inputs from it without sharing any computation.

Recipe (one NumPy ``default_rng(seed)`` stream per workload, float32 draws in
C order, in this order: q, k, v, log_a, lambda, then t and states for decode):

* q, k, v ~ N(0, 1) / sqrt(dk); for the Mamba-2-style workloads k is then
  L2-normalised over dk for every (b, h, t).  Workloads that share q and k
  across heads (multi-value attention, the pages' benchmark setup) draw q and
  k for their Hk q/k heads only.
* log_a = -softplus(N(0, 1) + 2)   (strong decay)  or 0 (no decay) or a
  weak-decay variant -softplus(N(0,1)+2) / 1024.
* lambda[b, h, t, l] = softplus(N(0, 1)) with L = bit_length(T - 1) + 1 levels.
* bf16 workloads round q, k, v once to bfloat16 (round-to-nearest-even, via
  torch on the CPU); both sides receive exactly these rounded values.

Everything is returned as CPU torch tensors; callers move them to the device.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


def num_levels(T: int) -> int:
    """Number of lambda levels for a sequence of length T: bit_length(T-1) + 1."""
    if T <= 0:
        raise ValueError("T must be positive")
    return int(T - 1).bit_length() + 1


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x.astype(np.float64)).astype(np.float32)


@dataclasses.dataclass(frozen=True)
class FwdWorkload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    C: int
    dtype: str  # "bf16" or "f32"
    decay: str = "strong"  # "strong", "none", "weak"
    knorm: bool = True
    seed: int = 0
    Hk: int = 0  # q/k heads shared by groups of H / Hk heads (MVA); 0 = one per head

    @property
    def L(self) -> int:
        return num_levels(self.T)

    @property
    def qk_heads(self) -> int:
        return self.Hk or self.H


# The forward workloads the library is measured and checked on.
TINY = FwdWorkload("tiny_T64_fp32", 1, 1, 64, 16, 16, 16, "f32", decay="none", knorm=False)
MAMBA2_T2K = FwdWorkload("mamba2_B8H8_T2048_dk128_dv64", 8, 8, 2048, 128, 64, 64, "bf16")
LM_T16K = FwdWorkload("lm_B2H16_T16384_dk128_dv128", 2, 16, 16384, 128, 128, 64, "bf16")
LONG_T64K = FwdWorkload("long_B1H16_T65536_dk128_dv128", 1, 16, 65536, 128, 128, 64, "bf16")

# The pages' kernel benchmark setup (batch 2, 48 heads, head dim 64, state dim
# 128, chunk 64, q/k shared by all heads as in Mamba-2's multi-value layout),
# at one of its sequence lengths.
PAGES_MVA_T16K = FwdWorkload("pages_mva_B2H48_T16384_dk128_dv64", 2, 48, 16384, 128, 64, 64, "bf16", Hk=1)

FWD_WORKLOADS = {w.name: w for w in (TINY, MAMBA2_T2K, LM_T16K, LONG_T64K, PAGES_MVA_T16K)}


def make_fwd_inputs(w: FwdWorkload):
    """Draw (q, k, v, log_a, lam) for a forward workload as CPU tensors.

    q, k: [B, Hk, T, dk] (Hk = H unless the workload shares q/k across heads);
    v: [B, H, T, dv]; all bf16 or f32; log_a: [B, H, T] f32;
    lam: [B, H, T, L] f32.
    """
    rng = np.random.default_rng(w.seed)
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    Hk = w.qk_heads
    if H % Hk != 0:
        raise ValueError("q/k heads must divide H")
    scale = np.float32(1.0 / math.sqrt(dk))
    q = rng.standard_normal((B, Hk, T, dk), dtype=np.float32) * scale
    k = rng.standard_normal((B, Hk, T, dk), dtype=np.float32) * scale
    v = rng.standard_normal((B, H, T, dv), dtype=np.float32) * scale
    if w.knorm:
        nrm = np.sqrt(np.sum(k.astype(np.float64) ** 2, axis=-1, keepdims=True))
        k = (k / np.maximum(nrm, 1e-12)).astype(np.float32)
    g = rng.standard_normal((B, H, T), dtype=np.float32)
    if w.decay == "none":
        log_a = np.zeros((B, H, T), dtype=np.float32)
    elif w.decay == "strong":
        log_a = -_softplus(g + 2.0)
    elif w.decay == "weak":
        log_a = (-_softplus(g + 2.0) / np.float32(1024.0)).astype(np.float32)
    else:
        raise ValueError(w.decay)
    lam = _softplus(rng.standard_normal((B, H, T, w.L), dtype=np.float32))
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return (
        torch.from_numpy(q).to(tdt),
        torch.from_numpy(k).to(tdt),
        torch.from_numpy(v).to(tdt),
        torch.from_numpy(np.ascontiguousarray(log_a)),
        torch.from_numpy(lam),
    )


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    N: int  # sequences
    H: int
    dk: int
    dv: int
    L: int
    t_max: int  # t ~ U{1 .. t_max}
    dtype: str = "bf16"
    seed: int = 0
    Hk: int = 0  # q/k heads shared by groups of H / Hk heads (MVA); 0 = one per head


DECODE_64x16 = DecodeWorkload("decode_N64_H16_dk128_dv128_L17", 64, 16, 128, 128, 17, 65535)


def live_levels(t_prev: int, L: int) -> list[int]:
    """Levels that may hold non-zero state after processing position t_prev:
    level 0 and level b+1 for every set bit b of t_prev (index bookkeeping
    only, used to shape synthetic decode states)."""
    out = [0]
    for b in range(L - 1):
        if (t_prev >> b) & 1:
            out.append(b + 1)
    return out


def make_decode_inputs(w: DecodeWorkload, t: np.ndarray | None = None):
    """Draw (states, q, k, v, log_a, lam, t) for one decode step.

    states: [N, H, L, dk, dv] f32 holding S_{t-1}; levels that are dead at
    t-1 are exactly 0, live ones are N(0,1)/dk.  q, k: [N, Hk, dk]; v: [N, H, dv]
    (bf16 or f32); log_a: [N, H] f32; lam: [N, H, L] f32; t: [N] int32.
    """
    rng = np.random.default_rng(w.seed)
    N, H, dk, dv, L = w.N, w.H, w.dk, w.dv, w.L
    scale = np.float32(1.0 / math.sqrt(dk))
    Hk = w.Hk or H
    q = rng.standard_normal((N, Hk, dk), dtype=np.float32) * scale
    k = rng.standard_normal((N, Hk, dk), dtype=np.float32) * scale
    v = rng.standard_normal((N, H, dv), dtype=np.float32) * scale
    log_a = -_softplus(rng.standard_normal((N, H), dtype=np.float32) + 2.0)
    lam = _softplus(rng.standard_normal((N, H, L), dtype=np.float32))
    if t is None:
        t = rng.integers(1, w.t_max + 1, size=N).astype(np.int32)
    else:
        t = np.asarray(t, dtype=np.int32)
    states = np.zeros((N, H, L, dk, dv), dtype=np.float32)
    inv = np.float32(1.0 / dk)
    for i in range(N):
        if t[i] <= 0:
            continue
        for lev in live_levels(int(t[i]) - 1, L):
            states[i, :, lev] = rng.standard_normal((H, dk, dv), dtype=np.float32) * inv
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return (
        torch.from_numpy(states),
        torch.from_numpy(q).to(tdt),
        torch.from_numpy(k).to(tdt),
        torch.from_numpy(v).to(tdt),
        torch.from_numpy(log_a),
        torch.from_numpy(lam),
        torch.from_numpy(t),
    )


@dataclasses.dataclass(frozen=True)
class LambdaProjWorkload:
    """Hidden states and per-head projection for the level weights."""
    name: str
    B: int
    T: int
    D: int  # hidden width
    H: int
    L: int
    dtype: str = "bf16"
    bias: bool = True
    seed: int = 0


# The bench forward's shape with hidden width H * dv = 16 * 128.
LAMBDA_LM_T16K = LambdaProjWorkload("lambda_B2T16384_D2048_H16_L15", 2, 16384, 2048, 16, 15)


def make_lambda_proj_inputs(w: LambdaProjWorkload):
    """Draw (x, W, bias): x [B, T, D] ~ N(0, 1); W [H*L, D] ~ N(0, 1) / sqrt(D);
    bias [H*L] ~ N(0, 1) f32 (None when the workload has no bias).  x and W
    are rounded once to bf16 for bf16 workloads."""
    rng = np.random.default_rng(w.seed)
    x = rng.standard_normal((w.B, w.T, w.D), dtype=np.float32)
    W = rng.standard_normal((w.H * w.L, w.D), dtype=np.float32) * np.float32(1.0 / math.sqrt(w.D))
    bias = rng.standard_normal(w.H * w.L, dtype=np.float32)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return (torch.from_numpy(x).to(tdt), torch.from_numpy(W).to(tdt),
            torch.from_numpy(bias) if w.bias else None)


@dataclasses.dataclass(frozen=True)
class GdnWorkload:
    """Log-linear Gated DeltaNet forward inputs."""
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str = "bf16"  # q, k, v storage: "bf16" or "f32"
    decay: str = "weak"  # log_alpha: "strong", "weak" or "none", as for the forward
    seed: int = 0

    @property
    def L(self) -> int:
        return num_levels(self.T)


# The language-model shape of the forward bench, as a Gated DeltaNet layer.
GDN_LM_T16K = GdnWorkload("gdn_B2H16_T16384_dk128_dv128", 2, 16, 16384, 128, 128, seed=3)


def make_gdn_inputs(w: GdnWorkload):
    """Draw (q, k, v, log_alpha, beta, lam) as CPU tensors, in this order:

    q, v ~ N(0, 1) / sqrt(dk); k ~ N(0, 1) L2-normalised over dk (the delta
    rule's keys are unit vectors); log_alpha as log_a of the forward recipe;
    beta = sigmoid(N(0, 1)) in (0, 1); lam[b, h, t, l] = softplus(N(0, 1)).
    q, k, v: [B, H, T, dk|dv] bf16 or f32 (bf16 rounded once, both sides get
    the rounded values); log_alpha, beta: [B, H, T] f32; lam: [B, H, T, L] f32.
    """
    rng = np.random.default_rng(w.seed)
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    scale = np.float32(1.0 / math.sqrt(dk))
    q = rng.standard_normal((B, H, T, dk), dtype=np.float32) * scale
    k = rng.standard_normal((B, H, T, dk), dtype=np.float32)
    k = (k / np.maximum(np.sqrt(np.sum(k.astype(np.float64) ** 2, axis=-1, keepdims=True)),
                        1e-12)).astype(np.float32)
    v = rng.standard_normal((B, H, T, dv), dtype=np.float32) * scale
    g = rng.standard_normal((B, H, T), dtype=np.float32)
    if w.decay == "none":
        log_alpha = np.zeros((B, H, T), dtype=np.float32)
    elif w.decay == "strong":
        log_alpha = -_softplus(g + 2.0)
    elif w.decay == "weak":
        log_alpha = (-_softplus(g + 2.0) / np.float32(1024.0)).astype(np.float32)
    else:
        raise ValueError(w.decay)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T)).astype(np.float64)))).astype(np.float32)
    lam = _softplus(rng.standard_normal((B, H, T, w.L), dtype=np.float32))
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return (torch.from_numpy(q).to(tdt), torch.from_numpy(k).to(tdt), torch.from_numpy(v).to(tdt),
            torch.from_numpy(np.ascontiguousarray(log_alpha)), torch.from_numpy(beta),
            torch.from_numpy(lam))


GDN_DECODE_64x16 = DecodeWorkload("gdn_decode_N64_H16_dk128_dv128_L17", 64, 16, 128, 128, 17, 65535, seed=5)


def make_gdn_decode_inputs(w: DecodeWorkload, t: np.ndarray | None = None):
    """Draw (states, q, k, v, log_alpha, beta, lam, t) for one log-linear Gated
    DeltaNet decode step, in this order: states as make_decode_inputs (levels
    live at t-1 ~ N(0,1)/dk, dead levels exactly 0), q, v ~ N(0,1)/sqrt(dk),
    k ~ N(0,1) L2-normalised, log_alpha = -softplus(N(0,1)+2), beta =
    sigmoid(N(0,1)), lam = softplus(N(0,1)), t ~ U{1..t_max} unless given."""
    rng = np.random.default_rng(w.seed)
    N, H, dk, dv, L = w.N, w.H, w.dk, w.dv, w.L
    if t is None:
        t = rng.integers(1, w.t_max + 1, N).astype(np.int32)
    t = np.asarray(t, dtype=np.int32)
    S = np.zeros((N, H, L, dk, dv), dtype=np.float32)
    for i in range(N):
        if t[i] >= 1:
            for level in live_levels(int(t[i]) - 1, L):
                S[i, :, level] = rng.standard_normal((H, dk, dv), dtype=np.float32) / np.float32(dk)
    scale = np.float32(1.0 / math.sqrt(dk))
    q = rng.standard_normal((N, H, dk), dtype=np.float32) * scale
    k = rng.standard_normal((N, H, dk), dtype=np.float32)
    k = (k / np.maximum(np.sqrt(np.sum(k.astype(np.float64) ** 2, axis=-1, keepdims=True)), 1e-12)).astype(np.float32)
    v = rng.standard_normal((N, H, dv), dtype=np.float32) * scale
    log_alpha = -_softplus(rng.standard_normal((N, H), dtype=np.float32) + 2.0)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((N, H)).astype(np.float64)))).astype(np.float32)
    lam = _softplus(rng.standard_normal((N, H, L), dtype=np.float32))
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return (torch.from_numpy(S), torch.from_numpy(q).to(tdt), torch.from_numpy(k).to(tdt),
            torch.from_numpy(v).to(tdt), torch.from_numpy(np.ascontiguousarray(log_alpha)),
            torch.from_numpy(beta), torch.from_numpy(lam), torch.from_numpy(t))
