"""CPU oracle for log-linear Gated DeltaNet (forward).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library.

Plain fp64 NumPy, no chunking, no WY / UT rearrangement.

What the pages fix.  [P1] "论文阅读：Log-Linear Attention — 基于 Fenwick 树与层次矩阵的
对数线性复杂度注意力机制", section 与已有模型的组合, and [P2] "算力终结者来了！华人天团
「降维打击」注意力瓶颈，AI狂飙进对数时代", section 对Mamba-2和门控DeltaNet的对数线性推广:
a linear-attention model whose output is o_t = sum_{s<=t} c(t,s) v_s becomes
log-linear by weighting each pair with lambda[t, level(t,s)], the Fenwick level
of key s seen from query t ([P1] 层级判定算法, 并行形式), and Gated DeltaNet is
the second model the pages lift this way.

What the pages leave open, read from outside them (parity UNPINNED BY THE
PAGES; every pin below is mathematical):

* The gated delta rule (Yang, Kautz, Hatamizadeh, "Gated Delta Networks:
  Improving Mamba2 with Delta Rule", 2024), with states stored k-major
  (dk x dv, the transpose of the paper's dv x dk):
      S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
      o_t = S_t^T q_t,
  alpha_t = exp(log_alpha[t]) in (0, 1], beta_t in [0, 1].  Unrolled,
      c(t,s) = beta_s q_t^T Phi(t,s) k_s,   Phi(t,s) = A_t A_{t-1} ... A_{s+1},
  with A_r = alpha_r (I - beta_r k_r k_r^T) and Phi(t,t) = I.
* The log-linear lift keeps those coefficients and weights them:
      o_t = sum_{s<=t} lambda[t, level(t,s)] c(t,s) v_s.
  Equivalently every Fenwick bucket holds its own state, each bucket state
  follows the same transitions A_t, the lssb rule of the decode step merges
  them, and o_t = sum_l lambda[t,l] (S_t^l)^T q_t (``loglinear_recurrent``).
  With lambda = 1 on every level this is Gated DeltaNet itself.
"""
from __future__ import annotations

import numpy as np

from .loglinear_oracle import _f64, level_rows, lssb


def gated_delta_recurrent(q, k, v, log_alpha, beta) -> np.ndarray:
    """Gated DeltaNet without the hierarchy, one token at a time.

    q, k: [B, H, T, dk]; v: [B, H, T, dv]; log_alpha, beta: [B, H, T].
    S_t = alpha_t (S_{t-1} - beta_t k_t (k_t^T S_{t-1})) + beta_t k_t v_t^T,
    o_t = S_t^T q_t.  Returns [B, H, T, dv] fp64.
    """
    q, k, v, log_alpha, beta = (_f64(x) for x in (q, k, v, log_alpha, beta))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    out = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv))
            for t in range(T):
                kt, bt = k[b, h, t], beta[b, h, t]
                S = np.exp(log_alpha[b, h, t]) * (S - bt * np.outer(kt, kt @ S))
                S += bt * np.outer(kt, v[b, h, t])
                out[b, h, t] = q[b, h, t] @ S
    return out


def pair_coefficients(q, k, log_alpha, beta) -> np.ndarray:
    """c(t,s) = beta_s q_t^T Phi(t,s) k_s for one (b, h), zero for s > t.

    q, k: [T, dk]; log_alpha, beta: [T].  Row t's vector r = q_t^T Phi(t,s)
    starts at q_t for s = t and moves to s-1 by r <- r A_s; all rows advance
    together, one key position s at a time from T-1 down to 0.
    """
    q, k, log_alpha, beta = (_f64(x) for x in (q, k, log_alpha, beta))
    T = q.shape[0]
    c = np.zeros((T, T))
    R = np.zeros_like(q)
    for s in range(T - 1, -1, -1):
        R[s] = q[s]                    # row s joins with r = q_s (Phi(s,s) = I)
        live = R[s:]                   # rows t >= s hold q_t^T Phi(t,s)
        rk = live @ k[s]
        c[s:, s] = beta[s] * rk
        # r <- r A_s = alpha_s (r - beta_s (r . k_s) k_s^T)
        R[s:] = np.exp(log_alpha[s]) * (live - beta[s] * np.outer(rk, k[s]))
    return c


def loglinear_forward(q, k, v, log_alpha, beta, lam) -> np.ndarray:
    """Log-linear Gated DeltaNet, dense definition, for all (b, h).

    o_t = sum_{s<=t} lam[t, level(t,s)] c(t,s) v_s with c from
    ``pair_coefficients`` and the levels of [P1] 层级判定算法.
    q, k: [B, H, T, dk]; v: [B, H, T, dv]; log_alpha, beta: [B, H, T];
    lam: [B, H, T, L], L = bit_length(T-1) + 1.  Returns [B, H, T, dv] fp64.
    """
    q, k, v, log_alpha, beta, lam = (_f64(x) for x in (q, k, v, log_alpha, beta, lam))
    B, H, T, _ = q.shape
    L = int(T - 1).bit_length() + 1
    if lam.shape[-1] != L:
        raise ValueError(f"lambda has {lam.shape[-1]} levels, expected {L}")
    lev = level_rows(0, T, T)
    causal = lev >= 0
    rows = np.arange(T)[:, None]
    out = np.zeros((B, H, T, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            mh = np.where(causal, lam[b, h][rows, np.maximum(lev, 0)], 0.0)
            c = pair_coefficients(q[b, h], k[b, h], log_alpha[b, h], beta[b, h])
            out[b, h] = (c * mh) @ v[b, h]
    return out


def loglinear_recurrent(q, k, v, log_alpha, beta, lam) -> np.ndarray:
    """The same operator through per-level states, one token at a time.

    Step to t with m = lssb(t) ([P1] 解码：基于 lssb 的状态更新, with the
    transition A_t in place of the scalar decay):
      level m+1  <- A_t (S^0 + ... + S^m)
      levels 1..m <- 0,  levels > m+1 <- A_t S^l
      level 0    <- beta_t k_t v_t^T
    (at t = 0 all levels start empty); o_t = sum_l lam[t,l] (S^l)^T q_t.
    """
    q, k, v, log_alpha, beta, lam = (_f64(x) for x in (q, k, v, log_alpha, beta, lam))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    out = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((L, dk, dv))
            for t in range(T):
                kt, bt, a = k[b, h, t], beta[b, h, t], np.exp(log_alpha[b, h, t])
                if t > 0:
                    m = lssb(t)
                    S[m + 1] = S[: m + 1].sum(axis=0)    # level m+1 is empty here
                    S[: m + 1] = 0.0
                    # A_t applied to every level: alpha (S - beta k (k^T S))
                    S = a * (S - bt * np.einsum("d,le->lde", kt, np.einsum("d,lde->le", kt, S)))
                S[0] = bt * np.outer(kt, v[b, h, t])
                out[b, h, t] = np.einsum("l,d,lde->e", lam[b, h, t], q[b, h, t], S)
    return out



def loglinear_rows(q, k, v, log_alpha, beta, lam, bh: tuple[int, int], rows) -> np.ndarray:
    """Selected output rows of one (b, h), same definition as ``loglinear_forward``.

    For each row t, r = q_t^T Phi(t,s) is carried from s = t down to 0 by
    r <- r A_s, giving c(t,s) = beta_s r . k_s on the way; O(t dk) per row, so
    rows of long sequences can be checked one at a time.
    """
    b, h = bh
    qh, kh, vh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
    la, be, lm = _f64(log_alpha[b, h]), _f64(beta[b, h]), _f64(lam[b, h])
    res = []
    for t in rows:
        t = int(t)
        r = qh[t].copy()
        coef = np.empty(t + 1)
        for s in range(t, -1, -1):
            rk = r @ kh[s]
            coef[s] = be[s] * rk
            r = np.exp(la[s]) * (r - be[s] * rk * kh[s])
        lev = level_rows(t, t + 1, t + 1)[0]
        res.append((coef * lm[t, lev]) @ vh[: t + 1])
    return np.stack(res) if res else np.zeros((0, vh.shape[-1]))


def decode_step(states, q, k, v, log_alpha, beta, lam, t):
    """One decode step of log-linear Gated DeltaNet for every (sequence, head).

    states: [N, H, L, dk, dv] holding the bucket states after t-1 (k-major;
    levels dead at t-1 are 0); q, k: [N, H, dk]; v: [N, H, dv];
    log_alpha, beta: [N, H]; lam: [N, H, L]; t: [N] positions of the tokens.
    Returns (out [N, H, dv], new_states) and leaves ``states`` untouched.

    With m = lssb(t) ([P1] 解码：基于 lssb 的状态更新): level m+1 takes the sum
    of levels 0..m, levels 0..m are emptied, then every level passes through
    A_t = alpha_t (I - beta_t k_t k_t^T), and level 0 receives beta_t k_t v_t^T
    (at t = 0 every level starts empty).  o_t = sum_l lam[l] (S^l)^T q_t.
    Positions outside [0, 2^(L-1)) give a NaN output row and unchanged states.
    """
    S = _f64(states).copy()
    q, k, v, log_alpha, beta, lam = (_f64(x) for x in (q, k, v, log_alpha, beta, lam))
    t = np.asarray(t.detach().cpu().numpy() if hasattr(t, "detach") else t, dtype=np.int64)
    N, H, L, dk, dv = S.shape
    out = np.zeros((N, H, dv))
    for i in range(N):
        ti = int(t[i])
        if ti < 0 or ti >= (1 << (L - 1)):
            out[i] = np.nan
            continue
        for h in range(H):
            lev = S[i, h]
            kk, bt = k[i, h], beta[i, h]
            if ti == 0:
                lev[:] = 0.0
            else:
                m = lssb(ti)
                lev[m + 1] = lev[: m + 1].sum(axis=0)
                lev[: m + 1] = 0.0
                for level in range(L):
                    lev[level] = np.exp(log_alpha[i, h]) * (lev[level] - bt * np.outer(kk, kk @ lev[level]))
            lev[0] = bt * np.outer(kk, v[i, h])
            out[i, h] = np.einsum("l,d,lde->e", lam[i, h], q[i, h], lev)
    return out, S


def states_after(k, v, log_alpha, beta, t: int, L: int) -> np.ndarray:
    """Per-level decode states after the tokens 0..t, for every (b, h).

    By definition the level-l state is the sum over the level-l Fenwick bucket
    of t of Phi(t,s) beta_s k_s v_s^T (k-major, dk x dv); levels with no
    bucket at t are 0.  These are the states a decode step at t+1 starts
    from.  Evaluated by the per-level recurrence of ``loglinear_recurrent``
    (lssb merges, the transition on every level).
    k: [B, H, T, dk], v: [B, H, T, dv], log_alpha, beta: [B, H, T], T > t.
    Returns [B, H, L, dk, dv] fp64.
    """
    k, v, log_alpha, beta = (_f64(x) for x in (k, v, log_alpha, beta))
    B, H, _, dk = k.shape
    dv = v.shape[-1]
    out = np.zeros((B, H, L, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((L, dk, dv))
            for s in range(t + 1):
                ks, bs = k[b, h, s], beta[b, h, s]
                if s > 0:
                    m = lssb(s)
                    S[m + 1] = S[: m + 1].sum(axis=0)
                    S[: m + 1] = 0.0
                    S = np.exp(log_alpha[b, h, s]) * (S - bs * np.einsum("d,le->lde", ks, np.einsum("d,lde->le", ks, S)))
                S[0] = bs * np.outer(ks, v[b, h, s])
            out[b, h] = S
    return out
