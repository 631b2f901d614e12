"""CPU oracle for log-linear attention (forward and O(log T) decode step).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library.

Plain, slow, fp64 NumPy.  It materialises the full lower-triangular mask and
multiplies densely (O(T^2)); the chunkwise / hierarchical algorithm that the GPU
runs is an exact rearrangement of this definition and is deliberately NOT
reproduced here.

Sources (the web pages this follows; cited by title and section):

* [P1] "论文阅读：Log-Linear Attention — 基于 Fenwick 树与层次矩阵的对数线性复杂度注意力机制"
  (paper-reading blog).  Sections used: 前缀的层次化分解 (Fenwick partition of the
  prefix, the t=7 example), 层级判定算法 (level of s as seen from t),
  循环形式与输出计算 (per-level states and lambda-weighted readout),
  并行形式 (O = (QK^T ⊙ M^H) V and its 8x8 pattern table),
  解码：基于 lssb 的状态更新 (decode rule), 与已有模型的组合 (M^S ⊙ M^H).
* [P2] "算力终结者来了！华人天团「降维打击」注意力瓶颈，AI狂飙进对数时代" (news
  write-up).  Sections: 对数线性注意力 (O = (A ⊙ M) V), 特殊结构：Fenwick树划分.
* [P4] "动态线性注意力 — HF Daily Papers".  Section 前置知识 / 多状态线性注意力
  (bucket count ceil(log2(t+1)) + 1, state S = sum over bucket of v k^T).
* [P5] "論文紹介：Log Linear Attention" (journal-club slides), slides 19-21
  (t=7 walk-through, decode update rule).

Readings of points the pages leave open:

* M^S is the Mamba-2 scalar-decay mask M^S[t,s] = exp(cum[t] - cum[s]) with
  cum the inclusive prefix sum of log_a ([P1] 与已有模型的组合 names "the
  original model's semiseparable mask"; its formula is stripped).
* lambda is indexed by the query position t and the level ([P1] 并行形式 table).
* No softmax and no 1/sqrt(dk) scale: the operator is exactly (QK^T ⊙ M) V.
* States are stored k-major, S = sum k v^T (dk x dv), the transpose of the
  pages' v k^T; the readout is o = q^T S.
* lssb(t) is the 0-based index of the lowest set bit.  The decode rule zeroes
  levels 1..lssb(t) (inclusive) and writes the merge to level lssb(t)+1; the
  slide's "0 < l < lssb(t)" is read as a typo because only the inclusive range
  reproduces the parallel form (pinned by the recurrent == parallel test).
* Every kept or merged state is multiplied by a_t = exp(log_a[t]) on the step
  to t; the new level-0 state k_t v_t^T is not decayed (M^S[t,t] = 1).
* At t = 0 all levels are cleared before level 0 receives k_0 v_0^T.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# Index structure: the Fenwick partition of the prefix [0, t]
# --------------------------------------------------------------------------

def fenwick_buckets(t: int) -> list[tuple[int, int, int]]:
    """Partition of the prefix [0, t] into Fenwick buckets.

    Returns a list of (level, lo, hi) with hi exclusive.  Level 0 is the
    size-one sentinel {t}.  The rest of the prefix, [0, t), is cut by starting
    at t and repeatedly removing the lowest set bit: each removal of a low bit
    of value 2^(l-1) cuts off a bucket of that size at level l
    ([P1] 前缀的层次化分解; [P2] 特殊结构：Fenwick树划分).
    """
    if t < 0:
        raise ValueError("t must be >= 0")
    out = [(0, t, t + 1)]
    end = t
    while end:
        low = end & -end              # value of the lowest set bit
        level = low.bit_length()      # 2^(level-1) == low
        out.append((level, end - low, end))
        end -= low
    return out


def level_of(t: int, s: int) -> int:
    """Level of key position s as seen from query position t (s <= t):
    the level of the Fenwick bucket of [0, t] that contains s ([P1] 层级判定算法)."""
    if not 0 <= s <= t:
        raise ValueError("need 0 <= s <= t")
    for level, lo, hi in fenwick_buckets(t):
        if lo <= s < hi:
            return level
    raise AssertionError("buckets do not cover the prefix")


def level_rows(t0: int, t1: int, T: int) -> np.ndarray:
    """Levels for query rows t0..t1-1 against keys 0..T-1, -1 where s > t.

    Filled bucket by bucket from fenwick_buckets, so it is the same rule as
    level_of applied to every pair.
    """
    out = np.full((t1 - t0, T), -1, dtype=np.int16)
    for r, t in enumerate(range(t0, t1)):
        for level, lo, hi in fenwick_buckets(t):
            out[r, lo:hi] = level
    return out


def level_matrix(T: int) -> np.ndarray:
    """Full T x T level matrix (row t = query, column s = key), -1 above the diagonal."""
    return level_rows(0, T, T)


# --------------------------------------------------------------------------
# Forward: O = ((Q K^T) ⊙ M^S ⊙ M^H) V
# --------------------------------------------------------------------------

def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor (bf16 values are exact in fp32)
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def mask_rows(log_a: np.ndarray, lam: np.ndarray, t0: int, t1: int) -> np.ndarray:
    """Rows t0..t1-1 of M = M^S ⊙ M^H for one (batch, head).

    M^H[t, s] = lam[t, level(t, s)]  ([P1] 并行形式)
    M^S[t, s] = exp(cum[t] - cum[s]), cum = inclusive prefix sum of log_a
                ([P1] 与已有模型的组合; Mamba-2 reading, see module docstring)
    Both are zero above the diagonal (s > t).
    """
    log_a = _f64(log_a)
    lam = _f64(lam)
    T = log_a.shape[0]
    cum = np.cumsum(log_a)
    lev = level_rows(t0, t1, T)
    causal = lev >= 0
    rows = np.arange(t0, t1)[:, None]
    mh = np.where(causal, lam[rows, np.maximum(lev, 0)], 0.0)
    diff = np.where(causal, cum[t0:t1, None] - cum[None, :], -np.inf)
    return mh * np.exp(diff)


def forward(q, k, v, log_a, lam, row_block: int = 1024) -> np.ndarray:
    """Dense fp64 forward for all (b, h).

    q, k: [B, H, T, dk]; v: [B, H, T, dv]; log_a: [B, H, T]; lam: [B, H, T, L]
    with L = bit_length(T-1) + 1.  Returns out [B, H, T, dv] float64.
    """
    q, k, v, log_a, lam = (_f64(x) for x in (q, k, v, log_a, lam))
    B, H, T, _ = q.shape
    dv = v.shape[-1]
    L = int(T - 1).bit_length() + 1
    if lam.shape[-1] != L:
        raise ValueError(f"lambda has {lam.shape[-1]} levels, expected {L}")
    out = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            for t0 in range(0, T, row_block):
                t1 = min(T, t0 + row_block)
                m = mask_rows(log_a[b, h], lam[b, h], t0, t1)
                a = q[b, h, t0:t1] @ k[b, h].T          # (QK^T) rows
                out[b, h, t0:t1] = (a * m) @ v[b, h]
    return out


def forward_rows(q, k, v, log_a, lam, bh: tuple[int, int], rows) -> np.ndarray:
    """Selected output rows of one (b, h): o_t = sum_{s<=t} M[t,s] (q_t . k_s) v_s.

    Same definition as ``forward`` evaluated one query row at a time, for
    spot checks at sizes where the full O(T^2) product is too slow.
    """
    b, h = bh
    qh, kh, vh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
    la, lm = _f64(log_a[b, h]), _f64(lam[b, h])
    cum = np.cumsum(la)
    res = []
    for t in rows:
        t = int(t)
        lev = np.empty(t + 1, dtype=np.int64)
        for level, lo, hi in fenwick_buckets(t):
            lev[lo:hi] = level
        m = lm[t, lev] * np.exp(cum[t] - cum[: t + 1])
        res.append((m * (kh[: t + 1] @ qh[t])) @ vh[: t + 1])
    return np.stack(res) if res else np.zeros((0, vh.shape[-1]))


# --------------------------------------------------------------------------
# Decode: per-level states with the lssb merge / promote rule
# --------------------------------------------------------------------------

def lssb(t: int) -> int:
    """0-based index of the lowest set bit of t > 0 ([P1] 解码；[P5] slide 21)."""
    if t <= 0:
        raise ValueError("lssb needs t > 0")
    return (t & -t).bit_length() - 1


def decode_step(states, q, k, v, log_a, lam, t):
    """One decode step for every (sequence, head), in fp64.

    states: [N, H, L, dk, dv] holding S_{t-1} (k-major, S = sum k v^T);
    q, k: [N, H, dk]; v: [N, H, dv]; log_a: [N, H]; lam: [N, H, L];
    t: [N] positions of the incoming tokens.
    Returns (out [N, H, dv], new_states) and leaves ``states`` untouched.

    Update at position t with m = lssb(t)  ([P1] 解码：基于 lssb 的状态更新;
    [P5] slide 21):
      level m+1  <- a_t * (S^0 + S^1 + ... + S^m)   (lower levels promoted)
      levels 1..m <- 0
      levels > m+1 <- a_t * S^l                     (kept, decayed)
      level 0    <- k_t v_t^T                       (the new token)
    At t = 0 every level is cleared first.  Readout ([P1] 循环形式与输出计算):
      o_t = sum_l lam[t, l] * q_t^T S_t^l.
    Positions outside [0, 2^(L-1)) give a NaN output row and unchanged states.
    """
    S = _f64(states).copy()
    q, k, v, log_a, lam = (_f64(x) for x in (q, k, v, log_a, lam))
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
            a = np.exp(log_a[i, h])
            if ti == 0:
                lev[:] = 0.0
            else:
                m = lssb(ti)
                merged = a * lev[: m + 1].sum(axis=0)
                lev[m + 2:] *= a
                lev[1: m + 1] = 0.0
                lev[m + 1] = merged
            lev[0] = np.outer(k[i, h], v[i, h])
            out[i, h] = np.einsum("l,d,lde->e", lam[i, h], q[i, h], lev)
    return out, S


def recurrent_forward(q, k, v, log_a, lam) -> np.ndarray:
    """Run decode_step over t = 0..T-1 from empty states for every (b, h).

    Same inputs and output as ``forward``; used to pin the parallel form to
    the recurrent form ([P1] 解码 and 并行形式 describe the same operator).
    """
    q, k, v, log_a, lam = (_f64(x) for x in (q, k, v, log_a, lam))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    out = np.zeros((B, H, T, dv))
    states = np.zeros((B, H, L, dk, dv))
    for t in range(T):
        o, states = decode_step(states, q[:, :, t], k[:, :, t], v[:, :, t],
                                log_a[:, :, t], lam[:, :, t], np.full(B, t))
        out[:, :, t] = o
    return out


def states_at(k, v, log_a, t: int, L: int) -> np.ndarray:
    """Per-level decode states S_t after the tokens 0..t, for every (b, h).

    By definition ([P1] 循环形式与输出计算; [P4] 多状态线性注意力): the level-l
    state is the decayed sum over the level-l Fenwick bucket of query t,
        S_t^l = sum_{s in bucket l of t} exp(cum[t] - cum[s]) k_s v_s^T,
    stored k-major (dk x dv); levels with no bucket at t are 0.  These are the
    states a decode step at position t+1 starts from (prefill -> decode).
    k: [B, H, T, dk], v: [B, H, T, dv], log_a: [B, H, T] with T > t.
    Returns [B, H, L, dk, dv] fp64.
    """
    k, v, log_a = (_f64(x) for x in (k, v, log_a))
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    if not 0 <= t < T:
        raise ValueError("need 0 <= t < T")
    cum = np.cumsum(log_a, axis=-1)
    S = np.zeros((B, H, L, dk, dv))
    for level, lo, hi in fenwick_buckets(t):
        if level >= L:
            raise ValueError(f"level {level} of t={t} does not fit in L={L}")
        w = np.exp(cum[:, :, t:t + 1] - cum[:, :, lo:hi])          # [B, H, n]
        S[:, :, level] = np.einsum("bhs,bhsd,bhse->bhde", w, k[:, :, lo:hi], v[:, :, lo:hi])
    return S


# --------------------------------------------------------------------------
# Backward (gradients of the forward)
# --------------------------------------------------------------------------

def backward(q, k, v, log_a, lam, dout):
    """Gradients of sum(out * dout) with respect to q, k, v, log_a and lambda.

    Reverse-mode differentiation (torch autograd, fp64, CPU) of the dense
    definition O = ((Q K^T) ⊙ M^S ⊙ M^H) V, one (b, h) at a time, with M^H and
    M^S exactly as in ``mask_rows`` ([P1] 并行形式, 与已有模型的组合).
    Returns (dq, dk, dv, dlog_a, dlam) as float64 arrays shaped like the inputs.
    """
    import torch

    q, k, v, log_a, lam, dout = (_f64(x) for x in (q, k, v, log_a, lam, dout))
    B, H, T, dk = q.shape
    L = int(T - 1).bit_length() + 1
    if lam.shape[-1] != L:
        raise ValueError(f"lambda has {lam.shape[-1]} levels, expected {L}")
    lev = torch.from_numpy(level_matrix(T).astype(np.int64))
    causal = lev >= 0
    idx = lev.clamp(min=0)
    grads = [np.zeros_like(x) for x in (q, k, v, log_a, lam)]
    for b in range(B):
        for h in range(H):
            ts = [torch.tensor(x[b, h], dtype=torch.float64, requires_grad=True)
                  for x in (q, k, v, log_a, lam)]
            tq, tk, tv, tla, tlam = ts
            cum = torch.cumsum(tla, 0)
            diff = torch.where(causal, cum[:, None] - cum[None, :], torch.zeros((), dtype=torch.float64))
            ms = torch.where(causal, torch.exp(diff), torch.zeros((), dtype=torch.float64))
            mh = torch.where(causal, torch.gather(tlam, 1, idx), torch.zeros((), dtype=torch.float64))
            out = ((tq @ tk.T) * mh * ms) @ tv
            (out * torch.from_numpy(dout[b, h])).sum().backward()
            for g, t in zip(grads, ts):
                g[b, h] = t.grad.numpy()
    return tuple(grads)


def _levels_seen_from(s: int, t_end: int) -> np.ndarray:
    """Levels of key s as seen from every query t = s .. t_end-1.

    The bucket walk of ``fenwick_buckets`` run for all those queries at once:
    start at end = t, cut off the bucket (end - low, end] of the lowest set bit
    low of end, and stop at the bucket that holds s.  Level 0 where t == s.
    """
    t = np.arange(s, t_end, dtype=np.int64)
    lev = np.zeros(t.shape, dtype=np.int64)
    end = t.copy()
    todo = t != s
    while np.any(todo):
        low = end & -end
        hit = todo & (end - low <= s) & (s < end)
        lev[hit] = np.log2(low[hit]).astype(np.int64) + 1  # low = 2^(level-1)
        todo &= ~hit
        end = np.where(todo, end - low, end)
    return lev


def backward_rows(q, k, v, log_a, lam, dout, bh: tuple[int, int], rows):
    """dq and dlam at selected query rows of one (b, h), by the chain rule
    written out on the dense definition o_t = sum_{s<=t} M[t,s] (q_t.k_s) v_s,
    M[t,s] = lam[t, level(t,s)] exp(cum[t] - cum[s]):

        dq_t        = sum_{s<=t} M[t,s] (dO_t . v_s) k_s
        dlam[t, l]  = sum over the level-l bucket of t of
                      exp(cum[t] - cum[s]) (q_t . k_s) (dO_t . v_s)

    For spot checks where the full autograd backward is too large.
    Returns (dq [n, dk], dlam [n, L]) float64."""
    b, h = bh
    qh, kh, vh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
    la, lm, do = _f64(log_a[b, h]), _f64(lam[b, h]), _f64(dout[b, h])
    cum = np.cumsum(la)
    L = lm.shape[-1]
    dq, dl = [], []
    for t in rows:
        t = int(t)
        g = np.zeros(L)
        dqt = np.zeros(qh.shape[-1])
        for level, lo, hi in fenwick_buckets(t):
            d = np.exp(cum[t] - cum[lo:hi])
            a = kh[lo:hi] @ qh[t]          # q_t . k_s
            c = vh[lo:hi] @ do[t]          # dO_t . v_s
            g[level] = np.sum(d * a * c)
            dqt += (lm[t, level] * d * c) @ kh[lo:hi]
        dq.append(dqt)
        dl.append(g)
    return np.array(dq).reshape(-1, qh.shape[-1]), np.array(dl).reshape(-1, L)


def backward_cols(q, k, v, log_a, lam, dout, bh: tuple[int, int], cols):
    """dk and dv at selected key positions of one (b, h), by the chain rule on
    the dense definition (see ``backward_rows``):

        dk_s = sum_{t>=s} M[t,s] (dO_t . v_s) q_t
        dv_s = sum_{t>=s} M[t,s] (q_t . k_s) dO_t

    Returns (dk [n, dk], dv [n, dv]) float64."""
    b, h = bh
    qh, kh, vh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
    la, lm, do = _f64(log_a[b, h]), _f64(lam[b, h]), _f64(dout[b, h])
    T = qh.shape[0]
    cum = np.cumsum(la)
    dk, dv = [], []
    for s in cols:
        s = int(s)
        lev = _levels_seen_from(s, T)
        ts = np.arange(s, T)
        m = lm[ts, lev] * np.exp(cum[s:] - cum[s])
        dk.append((m * (do[s:] @ vh[s])) @ qh[s:])
        dv.append((m * (qh[s:] @ kh[s])) @ do[s:])
    return np.array(dk).reshape(-1, kh.shape[-1]), np.array(dv).reshape(-1, vh.shape[-1])


# --------------------------------------------------------------------------
# q and k shared by groups of heads (multi-value attention, MVA)
# --------------------------------------------------------------------------
# [P2] Fig. 4 (the benchmark setup under the figure) runs log-linear Mamba-2
# with MVA: as in Mamba-2, the query / key projections (C and B there) are
# shared by a group of heads while v, the decay and lambda stay per head.
# Reading: Hk q/k heads, Hk dividing H, and head h reads q/k head
# h // (H / Hk) (consecutive heads form a group).  The operator per head is the
# unchanged dense definition above.

def heads_of_qk(x, H: int) -> np.ndarray:
    """q or k [B, Hk, T, d] (or [N, Hk, d]) laid out per head: head h gets
    q/k head h // (H // Hk).  fp64."""
    x = _f64(x)
    Hk = x.shape[1]
    if Hk < 1 or H % Hk != 0:
        raise ValueError(f"{Hk} q/k heads do not divide {H} heads")
    return np.repeat(x, H // Hk, axis=1)


def forward_mva(q, k, v, log_a, lam) -> np.ndarray:
    """Forward with q, k [B, Hk, T, dk] shared by groups of heads; v, log_a,
    lam per head [B, H, ...].  Returns out [B, H, T, dv] float64."""
    H = v.shape[1]
    return forward(heads_of_qk(q, H), heads_of_qk(k, H), v, log_a, lam)


def backward_mva(q, k, v, log_a, lam, dout):
    """Gradients of sum(out * dout) for ``forward_mva``.  A q/k head feeds every
    head of its group, so its gradient is the sum of the per-head gradients
    over the group (chain rule through the repetition)."""
    H, Hk = v.shape[1], q.shape[1]
    dq, dk, dv, dla, dlam = backward(heads_of_qk(q, H), heads_of_qk(k, H), v, log_a, lam, dout)
    B, _, T, d = dq.shape
    G = H // Hk
    return dq.reshape(B, Hk, G, T, d).sum(2), dk.reshape(B, Hk, G, T, d).sum(2), dv, dla, dlam


def decode_step_mva(states, q, k, v, log_a, lam, t):
    """``decode_step`` with q, k [N, Hk, dk] shared by groups of heads."""
    H = states.shape[1]
    return decode_step(states, heads_of_qk(q, H), heads_of_qk(k, H), v, log_a, lam, t)


# --------------------------------------------------------------------------
# lambda from the hidden state
# --------------------------------------------------------------------------
# [P1] 循环形式与输出计算: the level weights lambda_t^l are data dependent and
# non-negative, obtained by a linear projection of the token's hidden
# representation x_t with per-head parameters.  Reading (the map that makes
# them non-negative is not named): softplus of an affine map,
#   lambda[b, h, t, l] = softplus(sum_d x[b, t, d] W[h*L + l, d] + bias[h*L + l]),
# softplus(z) = log(1 + exp(z)).

def softplus(z) -> np.ndarray:
    """log(1 + exp(z)) in fp64, without overflow for large z."""
    z = _f64(z)
    return np.logaddexp(0.0, z)


def lambda_projection(x, W, bias, H: int, L: int) -> np.ndarray:
    """x: [B, T, D]; W: [H*L, D] (row h*L + l holds head h, level l);
    bias: [H*L] or None.  Returns lambda [B, H, T, L] float64."""
    x, W = _f64(x), _f64(W)
    B, T, D = x.shape
    if W.shape != (H * L, D):
        raise ValueError(f"W must be [{H * L}, {D}]")
    z = x.reshape(B * T, D) @ W.T
    if bias is not None:
        z = z + _f64(bias)[None, :]
    lam = softplus(z).reshape(B, T, H, L)
    return np.ascontiguousarray(lam.transpose(0, 2, 1, 3))


def lambda_projection_grad(x, W, bias, dlam, H: int, L: int):
    """Gradient of lambda_projection by the chain rule, in fp64: with
    z = x W^T + bias (rows m = (b, t), columns n = h*L + l),
    dz[m, n] = dlam[b, h, t, l] * sigmoid(z[m, n]) (softplus' = sigmoid),
    dx = dz W, dW = dz^T x, dbias = column sums of dz.
    Returns (dx [B, T, D], dW [H*L, D], dbias [H*L])."""
    x, W, dlam = _f64(x), _f64(W), _f64(dlam)
    B, T, D = x.shape
    if W.shape != (H * L, D) or dlam.shape != (B, H, T, L):
        raise ValueError("shape mismatch")
    X = x.reshape(B * T, D)
    z = X @ W.T
    if bias is not None:
        z = z + _f64(bias)[None, :]
    sig = 0.5 * (1.0 + np.tanh(0.5 * z))  # logistic function, no overflow
    dz = dlam.transpose(0, 2, 1, 3).reshape(B * T, H * L) * sig
    return (dz @ W).reshape(B, T, D), dz.T @ X, dz.sum(axis=0)
