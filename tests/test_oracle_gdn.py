"""Pins of the log-linear Gated DeltaNet oracle (oracle/gated_deltanet.py).

The pages name the model but print neither the delta rule nor its chunkwise
form, so this oracle is "parity unpinned by the pages": its pins are the
mathematics of the published gated delta rule and the reductions it must
obey.  Each test checks the oracle against something other than itself:

* brute force with explicit dk x dk transition matrices on tiny inputs;
* lambda = 1 on every level must give Gated DeltaNet itself, run as its
  one-token recurrence (fixes the order of the transition products and the
  sign of the delta term);
* the dense definition must equal the per-level recurrence with the lssb
  merges of [P1] 解码：基于 lssb 的状态更新 (two unrelated evaluations);
* with mutually orthogonal keys the delta terms vanish and the model must be
  the log-linear Mamba-2 operator (the pinned ``oracle.forward``) with
  beta-scaled values ([P1] 与已有模型的组合: the same hierarchy on both models);
* closed forms: a key written twice with beta = 1 is erased from the older
  bucket; beta = 0 writes nothing; one token gives lam * beta (q . k) v.

[P1] "论文阅读：Log-Linear Attention — 基于 Fenwick 树与层次矩阵的对数线性复杂度注意力机制"
"""
import numpy as np
import pytest

import oracle
from oracle import gated_deltanet as G


def _inputs(rng, B, H, T, dk, dv, decay=0.4, unit_keys=True):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, dv))
    log_alpha = -decay * rng.random((B, H, T))
    beta = rng.random((B, H, T))
    L = int(T - 1).bit_length() + 1
    lam = 0.25 + rng.random((B, H, T, L))
    return q, k, v, log_alpha, beta, lam


def test_brute_force_explicit_transitions():
    """o_t = sum_s lam[t, level(t,s)] beta_s q_t^T (A_t ... A_{s+1}) k_s v_s with
    every A_r = alpha_r (I - beta_r k_r k_r^T) built as a matrix."""
    rng = np.random.default_rng(0)
    T, dk, dv = 9, 3, 2
    q, k, v, la, beta, lam = _inputs(rng, 1, 1, T, dk, dv, unit_keys=False)
    A = [np.exp(la[0, 0, r]) * (np.eye(dk) - beta[0, 0, r] * np.outer(k[0, 0, r], k[0, 0, r]))
         for r in range(T)]
    want = np.zeros((T, dv))
    for t in range(T):
        for s in range(t + 1):
            phi = np.eye(dk)
            for r in range(s + 1, t + 1):
                phi = A[r] @ phi
            c = beta[0, 0, s] * q[0, 0, t] @ phi @ k[0, 0, s]
            want[t] += lam[0, 0, t, oracle.level_of(t, s)] * c * v[0, 0, s]
    got = G.loglinear_forward(q, k, v, la, beta, lam)[0, 0]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("unit_keys", [True, False])
def test_unit_lambda_is_gated_deltanet(unit_keys):
    """lam = 1 on every level: both oracle forms reduce to the one-token
    recurrence S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T."""
    rng = np.random.default_rng(1)
    q, k, v, la, beta, lam = _inputs(rng, 2, 1, 37, 8, 5, unit_keys=unit_keys)
    lam[:] = 1.0
    want = G.gated_delta_recurrent(q, k, v, la, beta)
    np.testing.assert_allclose(G.loglinear_forward(q, k, v, la, beta, lam), want, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(G.loglinear_recurrent(q, k, v, la, beta, lam), want, rtol=1e-10, atol=1e-11)


def test_dense_equals_level_recurrence():
    """Random lambda over T = 70 (lssb merges up to level 7, a ragged end):
    the dense pair-coefficient form equals the per-level state recurrence."""
    rng = np.random.default_rng(2)
    q, k, v, la, beta, lam = _inputs(rng, 1, 2, 70, 6, 4)
    want = G.loglinear_recurrent(q, k, v, la, beta, lam)
    np.testing.assert_allclose(G.loglinear_forward(q, k, v, la, beta, lam), want, rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("decay", [0.0, 2.0])
def test_orthogonal_keys_reduce_to_loglinear_mamba2(decay):
    """Pairwise orthogonal keys (T <= dk): (I - beta_r k_r k_r^T) k_s = k_s for
    r != s, so c(t,s) = beta_s exp(cum[t] - cum[s]) (q_t . k_s) and the model is
    the log-linear Mamba-2 operator with values beta_s v_s."""
    rng = np.random.default_rng(3)
    B, H, T, dk, dv = 1, 2, 13, 16, 3
    q, _, v, la, beta, lam = _inputs(rng, B, H, T, dk, dv, decay=decay)
    k = np.empty((B, H, T, dk))
    for h in range(H):
        basis, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
        k[0, h] = basis[:T] * (0.5 + rng.random((T, 1)))      # orthogonal, not unit
    got = G.loglinear_forward(q, k, v, la, beta, lam)
    want = oracle.forward(q, k, beta[..., None] * v, la, lam)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_rewrite_with_unit_beta_erases_older_bucket():
    """beta = 1, no decay, the same unit key u at t = 0 and 1: the write at
    t = 1 removes u's old value from the state, so the level-1 pair (1, 0)
    carries c = q^T (I - u u^T) u = 0 and o_1 = lam[1, 0] (q . u) v_1."""
    rng = np.random.default_rng(4)
    dk, dv = 5, 3
    u = rng.standard_normal(dk)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((1, 1, 2, dk))
    k = np.stack([u, u])[None, None]
    v = rng.standard_normal((1, 1, 2, dv))
    la = np.zeros((1, 1, 2))
    beta = np.ones((1, 1, 2))
    lam = np.array([[[[1.3, 0.7], [0.6, 2.1]]]])
    out = G.loglinear_forward(q, k, v, la, beta, lam)[0, 0]
    np.testing.assert_allclose(out[1], 0.6 * (q[0, 0, 1] @ u) * v[0, 0, 1], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(out[0], 1.3 * (q[0, 0, 0] @ u) * v[0, 0, 0], rtol=1e-13)


def test_zero_beta_writes_nothing_and_one_token_closed_form():
    rng = np.random.default_rng(5)
    q, k, v, la, beta, lam = _inputs(rng, 1, 1, 20, 4, 3)
    assert not np.any(G.loglinear_forward(q, k, v, la, np.zeros_like(beta), lam))
    q1, k1, v1, la1, b1, lam1 = (x[:, :, :1] for x in (q, k, v, la, beta, lam))
    want = lam1[0, 0, 0, 0] * b1[0, 0, 0] * (q1[0, 0, 0] @ k1[0, 0, 0]) * v1[0, 0, 0]
    np.testing.assert_allclose(G.loglinear_forward(q1, k1, v1, la1, b1, lam1[..., :1])[0, 0, 0], want,
                               rtol=1e-13)


def test_rows_match_dense():
    """The one-row evaluation used for long sequences equals the dense form."""
    rng = np.random.default_rng(6)
    q, k, v, la, beta, lam = _inputs(rng, 2, 2, 150, 8, 3)
    dense = G.loglinear_forward(q, k, v, la, beta, lam)
    rows = [0, 1, 63, 64, 65, 127, 128, 149]
    for bh in [(0, 1), (1, 0)]:
        np.testing.assert_allclose(G.loglinear_rows(q, k, v, la, beta, lam, bh, rows), dense[bh][rows],
                                   rtol=1e-11, atol=1e-12)


def test_decode_chain_equals_dense():
    """Decode steps from empty states over t = 0..T-1 reproduce the dense
    definition row by row (the step of [P1] 解码：基于 lssb 的状态更新 with the
    transition A_t on every level), and levels dead at t hold exactly 0."""
    rng = np.random.default_rng(7)
    B, H, T, dk, dv = 2, 1, 40, 5, 3
    q, k, v, la, beta, lam = _inputs(rng, B, H, T, dk, dv)
    L = lam.shape[-1]
    want = G.loglinear_forward(q, k, v, la, beta, lam)
    S = np.zeros((B, H, L, dk, dv))
    for t in range(T):
        o, S = G.decode_step(S, q[:, :, t], k[:, :, t], v[:, :, t], la[:, :, t], beta[:, :, t],
                             lam[:, :, t], np.full(B, t))
        np.testing.assert_allclose(o, want[:, :, t], rtol=1e-10, atol=1e-12)
        live = {0} | {b + 1 for b in range(L - 1) if (t >> b) & 1}
        for level in range(L):
            assert np.any(S[:, :, level]) == (level in live), (t, level)


def test_decode_out_of_range_position():
    rng = np.random.default_rng(8)
    S = rng.standard_normal((2, 1, 4, 3, 2))
    q, k = rng.standard_normal((2, 1, 3)), rng.standard_normal((2, 1, 3))
    v, la, beta = rng.standard_normal((2, 1, 2)), -rng.random((2, 1)), rng.random((2, 1))
    lam = rng.random((2, 1, 4))
    o, S2 = G.decode_step(S, q, k, v, la, beta, lam, np.array([8, 3]))
    assert np.all(np.isnan(o[0])) and np.array_equal(S2[0], S[0])
    assert np.all(np.isfinite(o[1]))


def test_states_after_brute_force():
    """The level states after t equal the bucket sums of Phi(t,s) beta_s k_s v_s^T
    built from explicit transition matrices over the Fenwick buckets of t
    ([P1] 前缀的层次化分解), and a decode step from them gives row t+1 of
    the dense definition."""
    rng = np.random.default_rng(9)
    T, dk, dv = 14, 3, 2
    q, k, v, la, beta, lam = _inputs(rng, 1, 1, T, dk, dv)
    L = lam.shape[-1]
    A = [np.exp(la[0, 0, r]) * (np.eye(dk) - beta[0, 0, r] * np.outer(k[0, 0, r], k[0, 0, r])) for r in range(T)]
    dense = G.loglinear_forward(q, k, v, la, beta, lam)
    for t in (0, 5, 7, 12):
        got = G.states_after(k, v, la, beta, t, L)[0, 0]
        want = np.zeros_like(got)
        for level, lo, hi in oracle.fenwick_buckets(t):
            for s in range(lo, hi):
                phi = np.eye(dk)
                for r in range(s + 1, t + 1):
                    phi = A[r] @ phi
                want[level] += beta[0, 0, s] * np.outer(phi @ k[0, 0, s], v[0, 0, s])
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-13)
        o, _ = G.decode_step(got[None, None], q[:, :, t + 1], k[:, :, t + 1], v[:, :, t + 1], la[:, :, t + 1],
                             beta[:, :, t + 1], lam[:, :, t + 1], np.array([t + 1]))
        np.testing.assert_allclose(o[0, 0], dense[0, 0, t + 1], rtol=1e-10, atol=1e-12)
