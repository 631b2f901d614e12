"""GPU parity of the backward (loglinear_bwd / _f32) against the oracle's
gradients of the dense definition (fp64 autograd).

Tolerance per gradient: max |gpu - oracle| <= tol * RMS(oracle gradient), with
tol = 1e-4 for fp32 inputs (fp32 matrix-core arithmetic) and the bf16 bound
2e-2 for bf16 inputs, the same bound as the bf16 forward (the bf16 path runs
bf16 matrix cores with hi/lo splits of its fp32 operands; its measured error
is ~1e-3 of the RMS at most, in d log_a under strong decay).  The oracle
receives the same (bf16-rounded) inputs and the forward output `out` is the
oracle's, so the backward is checked on its own; one pipeline case feeds the
GPU forward's output instead.
"""
import numpy as np
import pytest
import torch

import log_linear_attention_attn_amd as ll
import oracle
import workloads as W
from gpu_util import BF16_TOL, announce, assert_parity, have_gpu, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

BWD_TOL = 1e-4
NAMES = ("dq", "dk", "dv", "dlog_a", "dlam")

CASES = [
    # (B, H, T, dk, dv, C, dtype, decay)
    (1, 1, 1, 16, 16, 16, "f32", "weak"),        # one token
    (1, 2, 64, 16, 16, 64, "f32", "weak"),       # one chunk
    (1, 2, 200, 32, 32, 16, "f32", "weak"),      # ragged, several chunk levels
    (1, 1, 777, 64, 32, 32, "f32", "strong"),
    (2, 1, 300, 128, 64, 64, "bf16", "weak"),
    (1, 1, 1000, 128, 128, 64, "bf16", "none"),  # every level carries weight
    (1, 2, 1024, 64, 128, 32, "bf16", "weak"),   # T a power of two
    (1, 2, 700, 128, 128, 64, "bf16", "strong"), # strong decay: heavy-tailed gradients
    (1, 1, 3000, 128, 64, 64, "bf16", "weak"),   # 47 chunks, six chunk-level bits, ragged
    (1, 2, 500, 32, 96, 64, "bf16", "strong"),   # contraction widths 32 and 96 on the bf16 kernels
    (1, 1, 4200, 128, 128, 64, "bf16", "weak"),  # 66 chunks: chunk-level bits 0-6, ragged
    # reverse sweeps' row records over two (b,h): 64-row blocks that end inside
    # a chunk, three 1024-row decay-gradient scan blocks per (b,h), the last ragged
    (2, 1, 2500, 128, 128, 64, "bf16", "none"),
]


def _inputs(case, seed):
    B, H, T, dk, dv, C, dtype, decay = case
    w = W.FwdWorkload("bwd", B, H, T, dk, dv, C, dtype, decay=decay, seed=seed)
    q, k, v, la, lam = W.make_fwd_inputs(w)
    dout = torch.from_numpy(np.random.default_rng(seed + 1).standard_normal((B, H, T, dv)).astype(np.float32))
    return w, (q, k, v, la, lam), dout


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}T{}dk{}dv{}C{}_{}_{}".format(*c))
def test_bwd_matches_oracle(case):
    w, inp, dout = _inputs(case, seed=case[2] + case[3])
    q, k, v, la, lam = inp
    out = torch.from_numpy(oracle.forward(*inp).astype(np.float32))
    announce(f"bwd {case}")
    dq_, dk_, dv_, dla, dlam = to_dev(q, k, v, la, lam)
    grads = ll.bwd(dq_, dk_, dv_, dla, dlam, out.cuda(), dout.cuda(), C=w.C)
    torch.cuda.synchronize()
    want = oracle.backward(q, k, v, la, lam, dout)
    tol = BWD_TOL if case[6] == "f32" else BF16_TOL
    for name, g, ref in zip(NAMES, grads, want):
        assert_parity(g.cpu().numpy(), ref, tol, f"{name} {case}")


def test_bwd_after_gpu_forward():
    """The pipeline as a trainer runs it: GPU forward, then the backward with
    the GPU forward's output (bf16 path; its rounding enters d log_a)."""
    case = (1, 2, 1000, 128, 64, 64, "bf16", "weak")
    w, inp, dout = _inputs(case, seed=5)
    announce("bwd after the GPU forward")
    dev = to_dev(*inp)
    out = ll.fwd(*dev, C=w.C)
    grads = ll.bwd(*dev, out, dout.cuda(), C=w.C)
    torch.cuda.synchronize()
    want = oracle.backward(*inp, dout)
    for name, g, ref in zip(NAMES, grads, want):
        assert_parity(g.cpu().numpy(), ref, BF16_TOL, f"{name} pipeline")


def test_bwd_deterministic():
    case = (1, 2, 500, 64, 64, 32, "bf16", "weak")
    w, inp, dout = _inputs(case, seed=9)
    dev = to_dev(*inp)
    out = ll.fwd(*dev, C=w.C)
    announce("bwd determinism")
    g1 = ll.bwd(*dev, out, dout.cuda(), C=w.C)
    g2 = ll.bwd(*dev, out, dout.cuda(), C=w.C)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("decay", ["none", "weak"])
def test_bwd_256_chunks_sampled(decay):
    """T=16384, C=64: 256 chunks, so the bf16 sweeps run chunk-level bits 0-7
    (the bench's backward shape per head).  dq and dlambda on sampled query
    rows and dk, dv on sampled key columns against the oracle's per-row /
    per-column chain rule; no or weak decay so every level carries weight."""
    B, H, T = 1, 2, 16384
    w = W.FwdWorkload("bwd256", B, H, T, 128, 128, 64, "bf16", decay=decay, seed=7)
    q, k, v, la, lam = W.make_fwd_inputs(w)
    dout = torch.from_numpy(np.random.default_rng(8).standard_normal((B, H, T, 128)).astype(np.float32))
    announce(f"bwd 256 chunks sampled {decay}")
    dev = to_dev(q, k, v, la, lam)
    out = ll.fwd(*dev, C=64)
    grads = [g.cpu().numpy() for g in ll.bwd(*dev, out, dout.cuda(), C=64)]
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    fixed = []
    for n in (1, 2, 4, 8, 16, 32, 64, 96, 128, 129, 192, 255):
        fixed += [n * 64 - 1, n * 64]
    idx = sorted(set(fixed) | set(rng.integers(0, T, 24).tolist()))
    for bh in [(0, 0), (0, 1)]:
        dq, dlam = oracle.backward_rows(q, k, v, la, lam, dout, bh, idx)
        dk_, dv_ = oracle.backward_cols(q, k, v, la, lam, dout, bh, idx)
        assert_parity(grads[0][bh][idx], dq, BF16_TOL, f"dq rows {decay} {bh}")
        assert_parity(grads[4][bh][idx], dlam, BF16_TOL, f"dlam rows {decay} {bh}")
        assert_parity(grads[1][bh][idx], dk_, BF16_TOL, f"dk cols {decay} {bh}")
        assert_parity(grads[2][bh][idx], dv_, BF16_TOL, f"dv cols {decay} {bh}")


def test_bwd_ten_segments_sampled():
    """T=20000, C=64: 313 chunks, so the reverse register-state sweeps for dK
    and dV run ten 32-chunk segments (four segment-level bits, the pre-pass
    with five register levels) and a ragged last segment of 25 chunks whose
    last chunk is partial.  Sampled rows of dq, dlambda and columns of dk, dv
    at every segment boundary, weak decay so the segment-level states carry
    weight."""
    B, H, T = 1, 1, 20000
    w = W.FwdWorkload("bwd313", B, H, T, 128, 128, 64, "bf16", decay="weak", seed=11)
    q, k, v, la, lam = W.make_fwd_inputs(w)
    dout = torch.from_numpy(np.random.default_rng(12).standard_normal((B, H, T, 128)).astype(np.float32))
    announce("bwd ten segments sampled")
    dev = to_dev(q, k, v, la, lam)
    out = ll.fwd(*dev, C=64)
    grads = [g.cpu().numpy() for g in ll.bwd(*dev, out, dout.cuda(), C=64)]
    torch.cuda.synchronize()
    seg = 32 * 64
    fixed = [0, T - 1, T - 2, 288 * 64, 312 * 64, 312 * 64 - 1]
    for g in range(1, 10):
        fixed += [g * seg - 1, g * seg]
    rng = np.random.default_rng(13)
    idx = sorted(set(fixed) | set(rng.integers(0, T, 16).tolist()))
    bh = (0, 0)
    dq, dlam = oracle.backward_rows(q, k, v, la, lam, dout, bh, idx)
    dk_, dv_ = oracle.backward_cols(q, k, v, la, lam, dout, bh, idx)
    assert_parity(grads[0][bh][idx], dq, BF16_TOL, "dq rows T=20000")
    assert_parity(grads[4][bh][idx], dlam, BF16_TOL, "dlam rows T=20000")
    assert_parity(grads[1][bh][idx], dk_, BF16_TOL, "dk cols T=20000")
    assert_parity(grads[2][bh][idx], dv_, BF16_TOL, "dv cols T=20000")


@pytest.mark.parametrize("scale", [(8.0, 1e-6), (0.05, 1e3)], ids=["big_qk_tiny_dout", "small_qk_big_dout"])
def test_bwd_input_scales(scale):
    """The fp16 register-state sweeps (dQ, dK, dV and the in-chunk dlambda)
    carry power-of-two scales per row, per score tile and per level state so
    that no fp16 operand leaves fp16's normal range: q and k scaled by 8 with
    dO by 1e-6, and q, k by 0.05 with dO by 1e3, against the oracle on the
    same (bf16-rounded) inputs.  T=4200: three 32-chunk segments, weak decay."""
    sq, sd = scale
    case = (1, 1, 4200, 128, 128, 64, "bf16", "weak")
    w, inp, dout = _inputs(case, seed=21)
    q, k, v, la, lam = inp
    q = (q.float() * sq).to(q.dtype)
    k = (k.float() * sq).to(k.dtype)
    dout = dout * sd
    inp = (q, k, v, la, lam)
    out = torch.from_numpy(oracle.forward(*inp).astype(np.float32))
    announce(f"bwd input scales {scale}")
    grads = ll.bwd(*to_dev(*inp), out.cuda(), dout.cuda(), C=64)
    torch.cuda.synchronize()
    want = oracle.backward(*inp, dout)
    for name, g, ref in zip(NAMES, grads, want):
        assert_parity(g.cpu().numpy(), ref, BF16_TOL, f"{name} scales {scale}")
