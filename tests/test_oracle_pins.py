"""Pins of the CPU oracle to facts the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (fixtures under tests/golden/, each with its source), closed
forms, special cases that reduce to textbook recurrences, invariants, and
brute force over explicit bucket sets.  Page abbreviations:

[P1] "论文阅读：Log-Linear Attention — 基于 Fenwick 树与层次矩阵的对数线性复杂度注意力机制"
[P4] "动态线性注意力 — HF Daily Papers"
[P5] "論文紹介：Log Linear Attention" (journal-club slides)
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import loglinear_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(rng, B, H, T, dk, dv, decay=0.3, lam_scale=1.0):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    log_a = -decay * rng.random((B, H, T))
    L = int(T - 1).bit_length() + 1
    lam = lam_scale * (0.25 + rng.random((B, H, T, L)))
    return q, k, v, log_a, lam


# ---------------------------------------------------------------- indexing

def test_level_table_8x8_matches_page():
    """[P1] 并行形式: the printed 8x8 lambda-exponent pattern."""
    rows = []
    with open(os.path.join(GOLDEN, "level_table_8x8.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            rows.append([-1 if x == "-" else int(x) for x in line.split()])
    assert np.array_equal(oracle.level_matrix(8), np.array(rows))


def test_t7_partition_matches_pages():
    """[P1] 前缀的层次化分解 and [P5] slides 19-20: t = 7 -> {7},{6},{4,5},{0..3}."""
    with open(os.path.join(GOLDEN, "t7_partition.json")) as f:
        g = json.load(f)
    got = {str(lev): list(range(lo, hi)) for lev, lo, hi in oracle.fenwick_buckets(g["t"])}
    assert got == g["buckets"]


def test_partition_properties_all_t():
    """[P1] 前缀的层次化分解 / [P4] 多状态线性注意力: for every t < 4096 the buckets are
    disjoint and cover [0, t]; one non-empty bucket per set bit of t plus the
    sentinel; bucket l has size 2^(l-1); at most ceil(log2(t+1)) + 1 buckets."""
    for t in range(4096):
        bk = oracle.fenwick_buckets(t)
        covered = np.zeros(t + 1, dtype=int)
        for lev, lo, hi in bk:
            covered[lo:hi] += 1
            assert hi - lo == (1 if lev == 0 else 2 ** (lev - 1))
            if lev > 0:
                assert (t >> (lev - 1)) & 1, "bucket level must match a set bit of t"
        assert np.all(covered == 1)
        assert len(bk) == bin(t).count("1") + 1
        assert len(bk) <= math.ceil(math.log2(t + 1)) + 1


def test_power_of_two_history_is_one_bucket():
    """[P1] 前缀的层次化分解 (t = 8 example): at t = 2^k the whole history [0, t)
    is a single bucket, at level k+1."""
    for kk in range(12):
        t = 1 << kk
        assert sorted(oracle.fenwick_buckets(t)) == [(0, t, t + 1), (kk + 1, 0, t)]


def test_level_closed_form():
    """Closed form level(t,s) = bit_length(t xor s) for s < t (0 at s == t)
    against the bucket walk, every pair up to T = 512."""
    lv = oracle.level_matrix(512)
    t, s = np.tril_indices(512)
    closed = np.array([0 if a == b else int(a ^ b).bit_length() for a, b in zip(t, s)])
    assert np.array_equal(lv[t, s], closed)


def test_chunk_level_example():
    """[P1] 两阶段计算 example (T=8, C=2): levels <= log2(C) stay inside a chunk;
    level 2 links chunk 0->1 and 2->3, level 3 links {0,1} -> {2,3}."""
    with open(os.path.join(GOLDEN, "chunk_levels_T8_C2.json")) as f:
        g = json.load(f)
    T, C = g["T"], g["C"]
    lv = oracle.level_matrix(T)
    inter = {}
    for t in range(T):
        for s in range(t + 1):
            if t // C == s // C:
                assert lv[t, s] <= g["intra_max_level"]
            else:
                inter.setdefault(str(lv[t, s]), set()).add((s // C, t // C))
    assert {k: sorted(map(list, v)) for k, v in inter.items()} == {
        k: sorted(v) for k, v in g["inter"].items()}


# ---------------------------------------------------------------- forward

def test_no_decay_unit_lambda_is_causal_linear_attention():
    """lambda == 1 and log_a == 0: o_t = q_t^T sum_{s<=t} k_s v_s^T (prefix sums
    of outer products, [P1] 循环形式 degenerate case)."""
    rng = np.random.default_rng(1)
    q, k, v, _, _ = _rand_inputs(rng, 1, 2, 37, 5, 3)
    L = int(36).bit_length() + 1
    got = oracle.forward(q, k, v, np.zeros((1, 2, 37)), np.ones((1, 2, 37, L)))
    kv = np.cumsum(np.einsum("bhtd,bhte->bhtde", k, v), axis=2)
    want = np.einsum("bhtd,bhtde->bhte", q, kv)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_level_independent_lambda_is_gated_linear_attention():
    """[P1] 循环形式 退化条件: lambda_t^l = c_t for all l reduces to gated linear
    attention S_t = a_t S_{t-1} + k_t v_t^T, o_t = c_t q_t^T S_t."""
    rng = np.random.default_rng(2)
    B, H, T, dk, dv = 1, 2, 45, 4, 3
    q, k, v, log_a, _ = _rand_inputs(rng, B, H, T, dk, dv, decay=0.5)
    c = 0.5 + rng.random((B, H, T))
    L = int(T - 1).bit_length() + 1
    lam = np.repeat(c[..., None], L, axis=-1)
    got = oracle.forward(q, k, v, log_a, lam)
    want = np.zeros_like(got)
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv))
            for t in range(T):
                S = np.exp(log_a[b, h, t]) * S + np.outer(k[b, h, t], v[b, h, t])
                want[b, h, t] = c[b, h, t] * (q[b, h, t] @ S)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_forward_equals_bucket_brute_force():
    """[P1] 循环形式与输出计算: o_t = sum_l lam_t^l q_t^T S_t^l with
    S_t^l = sum_{s in bucket l} M^S[t,s] k_s v_s^T, by explicit loops."""
    rng = np.random.default_rng(3)
    B, H, T, dk, dv = 1, 1, 23, 3, 2
    q, k, v, log_a, lam = _rand_inputs(rng, B, H, T, dk, dv, decay=0.7)
    got = oracle.forward(q, k, v, log_a, lam)[0, 0]
    for t in range(T):
        o = np.zeros(dv)
        for lev, lo, hi in oracle.fenwick_buckets(t):
            S = np.zeros((dk, dv))
            for s in range(lo, hi):
                decay = math.exp(sum(log_a[0, 0, r] for r in range(s + 1, t + 1)))
                S += decay * np.outer(k[0, 0, s], v[0, 0, s])
            o += lam[0, 0, t, lev] * (q[0, 0, t] @ S)
        np.testing.assert_allclose(got[t], o, rtol=1e-11, atol=1e-12)


def test_one_hot_lambda_selects_one_bucket():
    """With lambda one-hot at level l0 the output is the decayed attention over
    exactly the level-l0 bucket; any bucket-membership error is O(1)."""
    rng = np.random.default_rng(4)
    T, dk, dv = 40, 4, 4
    q, k, v, log_a, _ = _rand_inputs(rng, 1, 1, T, dk, dv, decay=0.1)
    L = int(T - 1).bit_length() + 1
    for l0 in range(L):
        lam = np.zeros((1, 1, T, L))
        lam[..., l0] = 1.0
        got = oracle.forward(q, k, v, log_a, lam)[0, 0]
        cum = np.cumsum(log_a[0, 0])
        for t in range(T):
            want = np.zeros(dv)
            for lev, lo, hi in oracle.fenwick_buckets(t):
                if lev == l0:
                    for s in range(lo, hi):
                        want += math.exp(cum[t] - cum[s]) * (q[0, 0, t] @ k[0, 0, s]) * v[0, 0, s]
            np.testing.assert_allclose(got[t], want, rtol=1e-11, atol=1e-12)


def test_offdiagonal_blocks_rank_one():
    """[P1] HODLR 结构与低秩性: every off-diagonal block of the recursive bisection
    of M = M^S ⊙ M^H has rank 1 (also with the decay mask, [P1] 与已有模型的组合)."""
    rng = np.random.default_rng(5)
    T = 64
    log_a = -0.2 * rng.random(T)
    L = int(T - 1).bit_length() + 1
    lam = 0.5 + rng.random((T, L))
    M = O.mask_rows(log_a, lam, 0, T)
    checked = 0
    size = T
    while size >= 2:
        half = size // 2
        for start in range(0, T, size):
            blk = M[start + half:start + size, start:start + half]
            sv = np.linalg.svd(blk, compute_uv=False)
            assert sv[0] > 0
            assert sv[1] / sv[0] < 1e-12 if len(sv) > 1 else True
            checked += 1
        size = half
    assert checked == T - 1


def test_forward_rows_matches_forward():
    rng = np.random.default_rng(6)
    q, k, v, log_a, lam = _rand_inputs(rng, 2, 2, 50, 4, 3)
    full = oracle.forward(q, k, v, log_a, lam)
    rows = [0, 1, 17, 31, 32, 49]
    got = oracle.forward_rows(q, k, v, log_a, lam, (1, 0), rows)
    np.testing.assert_allclose(got, full[1, 0, rows], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- decode

def test_recurrent_equals_parallel():
    """[P1] 解码：基于 lssb 的状态更新 vs [P1] 并行形式: running the lssb decode rule
    from t = 0 reproduces the dense forward (to rounding)."""
    rng = np.random.default_rng(7)
    q, k, v, log_a, lam = _rand_inputs(rng, 2, 2, 70, 4, 3, decay=0.3)
    dense = oracle.forward(q, k, v, log_a, lam)
    rec = oracle.recurrent_forward(q, k, v, log_a, lam)
    np.testing.assert_allclose(rec, dense, rtol=1e-11, atol=1e-12)


def test_decode_zero_pattern():
    """After the step to t: levels 1..lssb(t) are zero, level lssb(t)+1 holds the
    promoted merge, levels of unset higher bits stay zero."""
    rng = np.random.default_rng(8)
    N, H, L, dk, dv = 6, 1, 8, 3, 2
    ts = np.array([1, 2, 3, 8, 12, 127])
    states = np.zeros((N, H, L, dk, dv))
    for i, t in enumerate(ts):
        prev = t - 1
        states[i, :, 0] = rng.standard_normal((H, dk, dv))
        for b in range(L - 1):
            if (prev >> b) & 1:
                states[i, :, b + 1] = rng.standard_normal((H, dk, dv))
    q = rng.standard_normal((N, H, dk)); k = rng.standard_normal((N, H, dk))
    v = rng.standard_normal((N, H, dv)); log_a = -rng.random((N, H)); lam = rng.random((N, H, L))
    _, new = oracle.decode_step(states, q, k, v, log_a, lam, ts)
    for i, t in enumerate(ts):
        m = oracle.lssb(int(t))
        nz = [bool(np.any(new[i, 0, lev] != 0)) for lev in range(L)]
        want = [True] + [False] * L
        for lev in range(1, L):
            want[lev] = (lev == m + 1) or (lev > m + 1 and (t >> (lev - 1)) & 1 == 1)
        assert nz == want[:L], (t, nz)


def test_decode_out_of_range_t_gives_nan_and_keeps_states():
    rng = np.random.default_rng(9)
    states = rng.standard_normal((3, 1, 4, 2, 2))
    q = rng.standard_normal((3, 1, 2)); v = rng.standard_normal((3, 1, 2))
    out, new = oracle.decode_step(states, q, q, v, np.zeros((3, 1)), np.ones((3, 1, 4)),
                                  np.array([-1, 8, 3]))
    assert np.all(np.isnan(out[:2])) and np.all(np.isfinite(out[2]))
    np.testing.assert_array_equal(new[:2], states[:2])


# ---------------------------------------------------------------- planted mistakes

def _strict_decode_rule(states, q, k, v, log_a, lam, t):
    """The slide's literal 'clear 0 < l < lssb(t)' (exclusive) variant."""
    S = np.array(states, dtype=np.float64).copy()
    N, H, L, dk, dv = S.shape
    out = np.zeros((N, H, dv))
    for i in range(N):
        ti = int(t[i])
        for h in range(H):
            lev = S[i, h]
            a = math.exp(log_a[i, h])
            if ti == 0:
                lev[:] = 0
            else:
                m = O.lssb(ti)
                merged = a * lev[: m + 1].sum(axis=0)
                lev[m + 2:] *= a
                lev[1:m] = 0.0           # exclusive upper end: level m survives
                lev[m + 1] = merged
            lev[0] = np.outer(k[i, h], v[i, h])
            out[i, h] = np.einsum("l,d,lde->e", lam[i, h], q[i, h], lev)
    return out, S


@pytest.mark.parametrize("mistake", ["strict_decode", "decay_sign", "lambda_by_key", "transposed_qk"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    """Plant a plausible mistake in the oracle (CPU only) and check that the
    recurrent == parallel pin or the gated-linear-attention pin rejects it."""
    rng = np.random.default_rng(10)
    q, k, v, log_a, lam = _rand_inputs(rng, 1, 1, 24, 3, 3, decay=0.4)
    if mistake == "strict_decode":
        monkeypatch.setattr(O, "decode_step", _strict_decode_rule)
    elif mistake == "decay_sign":
        real = O.mask_rows
        monkeypatch.setattr(O, "mask_rows", lambda la, lm, t0, t1: real(-np.asarray(la), lm, t0, t1))
    elif mistake == "lambda_by_key":
        def by_key(la, lm, t0, t1):
            la, lm = np.asarray(la, float), np.asarray(lm, float)
            T = la.shape[0]
            cum = np.cumsum(la)
            lev = O.level_rows(t0, t1, T)
            cols = np.arange(T)[None, :].repeat(t1 - t0, 0)
            mh = np.where(lev >= 0, lm[cols, np.maximum(lev, 0)], 0.0)
            return mh * np.exp(np.where(lev >= 0, cum[t0:t1, None] - cum[None, :], -np.inf))
        monkeypatch.setattr(O, "mask_rows", by_key)
    elif mistake == "transposed_qk":
        real_fwd = O.forward
        monkeypatch.setattr(O, "forward", lambda q_, k_, *a, **kw: real_fwd(k_, q_, *a, **kw))
    dense = O.forward(q, k, v, log_a, lam)
    rec = O.recurrent_forward(q, k, v, log_a, lam)
    assert not np.allclose(dense, rec, rtol=1e-6, atol=1e-8)


# ---------------------------------------------------------------- prefill -> decode states

def test_states_at_matches_recurrent_states():
    """The by-definition states at t equal the states the decode rule reaches
    after stepping through 0..t ([P1] 解码：基于 lssb 的状态更新)."""
    q, k, v, la, lam = _rand_inputs(np.random.default_rng(21), 1, 2, 45, 6, 5)
    L = lam.shape[-1]
    states = np.zeros((1, 2, L, 6, 5))
    for t in range(45):
        _, states = oracle.decode_step(states, q[:, :, t], k[:, :, t], v[:, :, t], la[:, :, t],
                                       lam[:, :, t], np.full(1, t))
        if t in (0, 1, 6, 7, 8, 31, 44):
            np.testing.assert_allclose(oracle.states_at(k, v, la, t, L), states, rtol=1e-12, atol=1e-13)


def test_states_at_readout_is_the_parallel_output():
    """o_t = sum_l lambda[t, l] q_t^T S_t^l reproduces the dense forward row t
    ([P1] 循环形式与输出计算 and 并行形式 describe one operator)."""
    q, k, v, la, lam = _rand_inputs(np.random.default_rng(5), 2, 1, 70, 8, 4)
    L = lam.shape[-1]
    full = oracle.forward(q, k, v, la, lam)
    for t in (0, 5, 32, 63, 69):
        S = oracle.states_at(k, v, la, t, L)
        o = np.einsum("bhl,bhd,bhlde->bhe", lam[:, :, t], q[:, :, t], S)
        np.testing.assert_allclose(o, full[:, :, t], rtol=1e-11, atol=1e-12)


def test_states_at_zero_pattern():
    """Level 0 always holds k_t v_t^T; level l >= 1 is non-zero exactly when bit
    l-1 of t is set ([P1] 前缀的层次化分解: one bucket per set bit)."""
    _, k, v, la, _ = _rand_inputs(np.random.default_rng(9), 1, 1, 200, 4, 4)
    L = 9
    for t in (0, 1, 2, 3, 100, 127, 128, 199):
        S = oracle.states_at(k, v, la, t, L)[0, 0]
        np.testing.assert_allclose(S[0], np.outer(k[0, 0, t], v[0, 0, t]))
        for l in range(1, L):
            assert (np.abs(S[l]).max() > 0) == bool((t >> (l - 1)) & 1), (t, l)


# ---------------------------------------------------------------- backward

def _loss(q, k, v, la, lam, dout):
    return float(np.sum(oracle.forward(q, k, v, la, lam) * dout))


def test_backward_matches_finite_differences():
    """Every gradient entry against central differences of the (NumPy) forward."""
    rng = np.random.default_rng(17)
    q, k, v, la, lam = _rand_inputs(rng, 1, 1, 9, 3, 2, decay=0.4)
    dout = rng.standard_normal((1, 1, 9, 2))
    grads = oracle.backward(q, k, v, la, lam, dout)
    eps = 1e-6
    for x, g in zip((q, k, v, la, lam), grads):
        num = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            old = x[i]
            x[i] = old + eps
            fp = _loss(q, k, v, la, lam, dout)
            x[i] = old - eps
            fm = _loss(q, k, v, la, lam, dout)
            x[i] = old
            num[i] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_backward_causal_linear_attention_closed_form():
    """lambda = 1, no decay: out = tril(Q K^T) V, whose gradients are the
    textbook products (dV = S^T dO, dQ = tril(dO V^T) K, dK = tril(dO V^T)^T Q)."""
    rng = np.random.default_rng(4)
    T, dk, dv = 33, 5, 4
    q, k, v, _, _ = _rand_inputs(rng, 1, 1, T, dk, dv)
    la = np.zeros((1, 1, T))
    lam = np.ones((1, 1, T, int(T - 1).bit_length() + 1))
    dout = rng.standard_normal((1, 1, T, dv))
    dq, dk_, dv_, _, _ = oracle.backward(q, k, v, la, lam, dout)
    Q, K, V, dO = q[0, 0], k[0, 0], v[0, 0], dout[0, 0]
    S = np.tril(Q @ K.T)
    G = np.tril(dO @ V.T)
    np.testing.assert_allclose(dv_[0, 0], S.T @ dO, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dq[0, 0], G @ K, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk_[0, 0], G.T @ Q, rtol=1e-12, atol=1e-12)


def test_backward_decay_gradient_identity():
    """d log_a[r] = sum_{t >= r} (dO_t . O_t - v_t . dV_t): the decay of token r
    sits in exactly the pairs s < r <= t (reverse prefix sum of row minus column
    sums of dM ⊙ M)."""
    rng = np.random.default_rng(8)
    q, k, v, la, lam = _rand_inputs(rng, 2, 1, 40, 4, 3, decay=0.5)
    dout = rng.standard_normal((2, 1, 40, 3))
    _, _, dv_, dla, _ = oracle.backward(q, k, v, la, lam, dout)
    out = oracle.forward(q, k, v, la, lam)
    dc = np.sum(dout * out, -1) - np.sum(v * dv_, -1)
    want = np.flip(np.cumsum(np.flip(dc, -1), -1), -1)
    np.testing.assert_allclose(dla, want, rtol=1e-10, atol=1e-11)


def test_backward_lambda_gradient_euler_identity():
    """out is linear in lambda, so sum_l lambda[t,l] dlam[t,l] = dO_t . O_t."""
    rng = np.random.default_rng(12)
    q, k, v, la, lam = _rand_inputs(rng, 1, 2, 50, 4, 3, decay=0.2)
    dout = rng.standard_normal((1, 2, 50, 3))
    dlam = oracle.backward(q, k, v, la, lam, dout)[4]
    out = oracle.forward(q, k, v, la, lam)
    np.testing.assert_allclose(np.sum(lam * dlam, -1), np.sum(dout * out, -1), rtol=1e-10, atol=1e-11)
    # entries of levels no pair reaches are exactly zero (row t uses levels <= bit_length(t))
    for t in range(50):
        assert not np.any(dlam[:, :, t, t.bit_length() + 1:])


# ---------------------------------------------------- q/k shared across heads

def test_mva_forward_bucket_brute_force():
    """q, k shared by groups of heads ([P2] Fig. 4 setup: MVA): every head's
    output by explicit bucket loops, reading q/k head h // (H / Hk)."""
    rng = np.random.default_rng(41)
    B, H, Hk, T, dk, dv = 2, 6, 2, 11, 3, 2
    q, k, v, log_a, lam = _rand_inputs(rng, B, H, T, dk, dv, decay=0.6)
    q, k = q[:, :Hk], k[:, :Hk]
    got = oracle.forward_mva(q, k, v, log_a, lam)
    assert got.shape == (B, H, T, dv)
    for b in range(B):
        for h in range(H):
            g = h // (H // Hk)
            for t in range(T):
                o = np.zeros(dv)
                for lev, lo, hi in oracle.fenwick_buckets(t):
                    for s in range(lo, hi):
                        decay = math.exp(sum(log_a[b, h, r] for r in range(s + 1, t + 1)))
                        o += lam[b, h, t, lev] * decay * (q[b, g, t] @ k[b, g, s]) * v[b, h, s]
                np.testing.assert_allclose(got[b, h, t], o, rtol=1e-11, atol=1e-12)


def test_mva_one_group_per_head_is_the_plain_forward():
    rng = np.random.default_rng(42)
    q, k, v, log_a, lam = _rand_inputs(rng, 1, 3, 17, 4, 2)
    np.testing.assert_array_equal(oracle.forward_mva(q, k, v, log_a, lam), oracle.forward(q, k, v, log_a, lam))


def test_mva_backward_matches_finite_differences():
    """Gradients of the shared q / k (summed over their group) and of the
    per-head v, log_a, lambda against central differences of forward_mva."""
    rng = np.random.default_rng(43)
    B, H, Hk, T, dk, dv = 1, 4, 2, 7, 2, 2
    q, k, v, la, lam = _rand_inputs(rng, B, H, T, dk, dv, decay=0.4)
    q, k = q[:, :Hk].copy(), k[:, :Hk].copy()
    dout = rng.standard_normal((B, H, T, dv))
    grads = oracle.backward_mva(q, k, v, la, lam, dout)
    assert grads[0].shape == q.shape and grads[1].shape == k.shape

    def loss():
        return float((oracle.forward_mva(q, k, v, la, lam) * dout).sum())

    eps = 1e-6
    for x, g in zip((q, k, v, la, lam), grads):
        num = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            old = x[i]
            x[i] = old + eps
            fp = loss()
            x[i] = old - eps
            fm = loss()
            x[i] = old
            num[i] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_mva_decode_is_the_per_head_decode_on_repeated_qk():
    """decode_step_mva against decode_step with q / k written out per head by
    hand (not through heads_of_qk)."""
    rng = np.random.default_rng(44)
    N, H, Hk, L, dk, dv = 3, 4, 2, 6, 3, 2
    S = rng.standard_normal((N, H, L, dk, dv))
    q = rng.standard_normal((N, Hk, dk))
    k = rng.standard_normal((N, Hk, dk))
    v = rng.standard_normal((N, H, dv))
    la = -rng.random((N, H))
    lam = rng.random((N, H, L))
    t = np.array([5, 12, 0])
    qh = np.stack([q[:, h // 2] for h in range(H)], axis=1)
    kh = np.stack([k[:, h // 2] for h in range(H)], axis=1)
    o1, s1 = oracle.decode_step_mva(S, q, k, v, la, lam, t)
    o2, s2 = oracle.decode_step(S, qh, kh, v, la, lam, t)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


# ------------------------------------------------- lambda from the hidden state

def test_softplus_closed_forms():
    """softplus(0) = ln 2; softplus(z) - softplus(-z) = z; large z -> z;
    very negative z -> exp(z)."""
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=0, abs=1e-15)
    z = np.linspace(-30, 30, 61)
    np.testing.assert_allclose(oracle.softplus(z) - oracle.softplus(-z), z, rtol=0, atol=1e-12)
    assert oracle.softplus(800.0) == 800.0
    assert oracle.softplus(-50.0) == pytest.approx(math.exp(-50.0), rel=1e-12)


def test_lambda_projection_brute_force():
    """[P1] 循环形式与输出计算: per-head linear map of x_t, made non-negative
    (softplus reading), by explicit loops over every output element."""
    rng = np.random.default_rng(51)
    B, T, D, H, L = 2, 5, 7, 3, 4
    x = rng.standard_normal((B, T, D))
    W = rng.standard_normal((H * L, D))
    bias = rng.standard_normal(H * L)
    got = oracle.lambda_projection(x, W, bias, H, L)
    assert got.shape == (B, H, T, L)
    for b in range(B):
        for h in range(H):
            for t in range(T):
                for l in range(L):
                    z = sum(x[b, t, d] * W[h * L + l, d] for d in range(D)) + bias[h * L + l]
                    assert got[b, h, t, l] == pytest.approx(math.log1p(math.exp(z)), rel=1e-12)
    assert np.all(got > 0)


def test_lambda_projection_one_hot_rows_land_in_place():
    """A one-hot row of W copies one hidden coordinate to exactly one
    (head, level) slot: the output layout is [B, H, T, L]."""
    B, T, D, H, L = 1, 3, 4, 2, 3
    x = np.arange(B * T * D, dtype=np.float64).reshape(B, T, D) / 10.0
    W = np.zeros((H * L, D))
    W[1 * L + 2, 3] = 1.0          # head 1, level 2 <- x[..., 3]
    got = oracle.lambda_projection(x, W, None, H, L)
    want = np.full((B, H, T, L), math.log(2.0))
    want[0, 1, :, 2] = np.log1p(np.exp(x[0, :, 3]))
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=0)


def test_lambda_projection_grad_matches_central_differences():
    """The gradient of F = sum(dlam * lambda_projection(x, W, bias)) with
    respect to every entry of x, W and bias, against central differences of
    lambda_projection itself (pins the chain rule, the sigmoid factor and the
    [B, H, T, L] <-> (row, column) layout)."""
    rng = np.random.default_rng(52)
    B, T, D, H, L = 2, 3, 4, 2, 3
    x = rng.standard_normal((B, T, D))
    W = rng.standard_normal((H * L, D))
    bias = rng.standard_normal(H * L)
    dlam = rng.standard_normal((B, H, T, L))
    dx, dW, db = oracle.lambda_projection_grad(x, W, bias, dlam, H, L)

    def F(x_, W_, b_):
        return float(np.sum(dlam * oracle.lambda_projection(x_, W_, b_, H, L)))

    eps = 1e-6
    for arr, grad, name in ((x, dx, "dx"), (W, dW, "dW"), (bias, db, "dbias")):
        assert grad.shape == arr.shape, name
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            fp = F(x, W, bias)
            arr[idx] = old - eps
            fm = F(x, W, bias)
            arr[idx] = old
            assert grad[idx] == pytest.approx((fp - fm) / (2 * eps), rel=1e-6, abs=1e-8), (name, idx)


def test_lambda_projection_grad_sigmoid_limits():
    """One input column, one output: dz -> dlam for z >> 0 (softplus is the
    identity there) and dz -> dlam * e^z for z << 0; dbias = dz."""
    x = np.ones((1, 1, 1))
    dlam = np.full((1, 1, 1, 1), 2.0)
    for z, want in ((40.0, 2.0), (-40.0, 2.0 * math.exp(-40.0))):
        _, _, db = oracle.lambda_projection_grad(x, np.zeros((1, 1)), np.array([z]), dlam, 1, 1)
        assert db[0] == pytest.approx(want, rel=1e-12)


# ---------------------------------------------------- level_of and sampled backward

def test_level_of_matches_page_table_and_partition():
    """level_of (one pair at a time) against the printed 8x8 table ([P1] 并行形式),
    the t = 7 partition ([P1] 前缀的层次化分解; [P5] slides 19-20), and the
    closed form bit_length(t xor s) for every pair s <= t < 64; s > t is refused."""
    rows = []
    with open(os.path.join(GOLDEN, "level_table_8x8.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            rows.append([-1 if x == "-" else int(x) for x in line.split()])
    for t in range(8):
        for s in range(t + 1):
            assert oracle.level_of(t, s) == rows[t][s], (t, s)
    with open(os.path.join(GOLDEN, "t7_partition.json")) as f:
        g = json.load(f)
    for lev, members in g["buckets"].items():
        for s in members:
            assert oracle.level_of(g["t"], s) == int(lev)
    for t in range(64):
        for s in range(t + 1):
            assert oracle.level_of(t, s) == (0 if s == t else int(t ^ s).bit_length())
    with pytest.raises(ValueError):
        oracle.level_of(3, 4)


def test_levels_seen_from_key_match_level_matrix():
    """The column-wise bucket walk used by backward_cols against the row-wise
    level matrix, every key s < 300."""
    T = 300
    lv = oracle.level_matrix(T)
    for s in range(T):
        assert np.array_equal(O._levels_seen_from(s, T), lv[s:, s]), s


@pytest.mark.parametrize("seed,T,decay", [(21, 37, 0.4), (22, 70, 0.0), (23, 64, 1.5)])
def test_sampled_backward_matches_autograd(seed, T, decay):
    """backward_rows / backward_cols (chain rule written out per row / column)
    against the fp64 autograd backward of the dense definition, every row and
    every column of a few (b, h)."""
    rng = np.random.default_rng(seed)
    q, k, v, la, lam = _rand_inputs(rng, 2, 2, T, 5, 3, decay=decay)
    dout = rng.standard_normal((2, 2, T, 3))
    dq, dk_, dv_, _, dlam = oracle.backward(q, k, v, la, lam, dout)
    idx = list(range(T))
    for bh in [(0, 1), (1, 0)]:
        gq, gl = oracle.backward_rows(q, k, v, la, lam, dout, bh, idx)
        gk, gv = oracle.backward_cols(q, k, v, la, lam, dout, bh, idx)
        np.testing.assert_allclose(gq, dq[bh], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(gl, dlam[bh], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(gk, dk_[bh], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(gv, dv_[bh], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("mistake", ["dq_no_lambda", "dk_wrong_side", "dv_untransposed_decay"])
def test_sampled_backward_planted_mistakes_are_caught(mistake):
    """A dropped lambda, a q/k side swap or a decay taken the wrong way in the
    sampled formulas must fail the autograd comparison above."""
    rng = np.random.default_rng(31)
    T = 40
    q, k, v, la, lam = _rand_inputs(rng, 1, 1, T, 4, 3, decay=0.4)
    dout = rng.standard_normal((1, 1, T, 3))
    dq, dk_, dv_, _, _ = oracle.backward(q, k, v, la, lam, dout)
    Q, K, V, dO = q[0, 0], k[0, 0], v[0, 0], dout[0, 0]
    cum = np.cumsum(la[0, 0])
    lv = oracle.level_matrix(T)
    t, s = 29, 11
    if mistake == "dq_no_lambda":
        ss = np.arange(t + 1)
        bad = (np.exp(cum[t] - cum[ss]) * (V[ss] @ dO[t])) @ K[ss]
        assert not np.allclose(bad, dq[0, 0, t], rtol=1e-6)
    elif mistake == "dk_wrong_side":
        ts = np.arange(s, T)
        m = lam[0, 0, ts, lv[ts, s]] * np.exp(cum[ts] - cum[s])
        bad = (m * (dO[ts] @ V[s])) @ K[ts]
        assert not np.allclose(bad, dk_[0, 0, s], rtol=1e-6)
    else:
        ts = np.arange(s, T)
        m = lam[0, 0, ts, lv[ts, s]] * np.exp(cum[s] - cum[ts])
        bad = (m * (Q[ts] @ K[s])) @ dO[ts]
        assert not np.allclose(bad, dv_[0, 0, s], rtol=1e-6)
    gq, _ = oracle.backward_rows(q, k, v, la, lam, dout, (0, 0), [t])
    gk, gv = oracle.backward_cols(q, k, v, la, lam, dout, (0, 0), [s])
    np.testing.assert_allclose(gq[0], dq[0, 0, t], rtol=1e-10)
    np.testing.assert_allclose(gk[0], dk_[0, 0, s], rtol=1e-10)
    np.testing.assert_allclose(gv[0], dv_[0, 0, s], rtol=1e-10)
