"""GPU parity of the forward (loglinear_fwd / _f32 / _ex) against the CPU oracle.

Tolerances: max |gpu - oracle| <= 2e-2 * RMS(oracle) for bf16 inputs (the
bf16 bound; the bf16 kernels split every fp32 operand of a bf16 product into
hi + lo terms, ~2^-16 relative, and the register-state sweep keeps its
bucket states in scaled fp16, 2^-11 relative per merge), 1e-4 * RMS for fp32
inputs (fp32 matrix-core arithmetic); the level table is bit-exact; repeated
runs are bitwise identical.
"""
import dataclasses

import numpy as np
import pytest
import torch

import log_linear_attention_attn_amd as ll
import oracle
import workloads as W
from gpu_util import BF16_TOL, F32_TOL, announce, assert_parity, have_gpu, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _run(w, seg_log2=-1, inputs=None):
    q, k, v, la, lam = inputs if inputs is not None else W.make_fwd_inputs(w)
    announce(f"fwd {w} seg_log2={seg_log2}")
    dq, dk_, dv_, dla, dlam = to_dev(q, k, v, la, lam)
    out = ll.fwd_ex(dq, dk_, dv_, dla, dlam, C=w.C, seg_log2=seg_log2)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (q, k, v, la, lam)


def _tol(w):
    return BF16_TOL if w.dtype == "bf16" else F32_TOL


# ---------------------------------------------------------------- index path

@pytest.mark.parametrize("T", [1, 2, 7, 8, 100, 4096])
def test_level_table_bit_exact(T):
    announce(f"level_table T={T}")
    got = ll.level_table(T).cpu().numpy().astype(np.int16)
    assert np.array_equal(got, oracle.level_matrix(T))


# ---------------------------------------------------------------- small cases, full oracle

def test_tiny_fp32_workload():
    """T=64, dk=dv=16, fp32, C=16, no decay, seed 0: the small workload in full."""
    w = W.TINY
    got, inp = _run(w)
    want = oracle.forward(*inp)
    assert_parity(got, want, F32_TOL, w.name)
    out2 = ll.fwd(*to_dev(*inp), C=w.C)  # the plain loglinear_fwd_f32 entry point
    torch.cuda.synchronize()
    assert_parity(out2.cpu().numpy(), want, F32_TOL, w.name + " (loglinear_fwd_f32)")


SMALL = []
for dtype in ("bf16", "f32"):
    for C in (16, 32, 64):
        for decay in ("none", "weak", "strong"):
            SMALL.append(W.FwdWorkload(f"small_{dtype}_C{C}_{decay}", 1, 2, 777, 64, 32, C, dtype,
                                       decay=decay, seed=C))


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("seg_log2", [0, 2, -1])
def test_small_parity(w, seg_log2):
    """Ragged T = 777 over several chunks and segments, every chunk size,
    no / weak / strong decay, explicit and automatic segment sizes."""
    got, inp = _run(w, seg_log2)
    assert_parity(got, oracle.forward(*inp), _tol(w), f"{w.name} seg{seg_log2}")


SHAPES = [
    # (B, H, T, dk, dv, C)
    (1, 1, 1, 16, 16, 16),        # single token
    (1, 1, 15, 16, 16, 16),       # shorter than one chunk
    (2, 1, 64, 32, 16, 64),       # exactly one chunk
    (1, 3, 130, 48, 48, 64),      # dk / dv padded, ragged tail of 2
    (1, 1, 1024, 128, 128, 64),   # 16 chunks
    (2, 2, 515, 96, 80, 32),
    (1, 1, 2049, 128, 64, 16),    # 129 chunks of 16: deep chunk-level tree
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}H{}T{}dk{}dv{}C{}".format(*s))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_shapes_parity(shape, dtype):
    B, H, T, dk, dv, C = shape
    w = W.FwdWorkload("shape", B, H, T, dk, dv, C, dtype, decay="weak", seed=T)
    for s in (-1, 1):
        got, inp = _run(w, s)
        assert_parity(got, oracle.forward(*inp), _tol(w), f"{shape} {dtype} seg{s}")


def test_one_hot_lambda_isolates_every_level():
    """fp32, no decay, lambda one-hot at one level: the output is the attention
    over exactly that Fenwick bucket, so a bucket-membership or level-index
    error anywhere gives an O(1) mismatch."""
    B, H, T, dk, dv, C = 1, 1, 700, 32, 16, 16
    w = W.FwdWorkload("onehot", B, H, T, dk, dv, C, "f32", decay="none", knorm=False, seed=11)
    q, k, v, la, _ = W.make_fwd_inputs(w)
    L = W.num_levels(T)
    for lev in range(L):
        lam = torch.zeros(B, H, T, L)
        lam[..., lev] = 1.0
        for s in (0, 2):
            got, inp = _run(w, s, (q, k, v, la, lam))
            assert_parity(got, oracle.forward(*inp), F32_TOL, f"one-hot level {lev} seg{s}")


def test_mamba2_T2048_full():
    """B=8, H=8, T=2048, dk=128, dv=64, bf16, C=64: every output against the oracle."""
    w = W.MAMBA2_T2K
    got, inp = _run(w)
    assert_parity(got, oracle.forward(*inp), BF16_TOL, w.name)


@pytest.mark.parametrize("decay", ["none", "weak"])
@pytest.mark.parametrize("base", [W.MAMBA2_T2K, W.LM_T16K], ids=lambda w: w.name)
def test_weak_decay_coverage(base, decay):
    """The workloads' strong decay makes distant levels negligible; without
    decay (or with weak decay) every inter-chunk level carries weight."""
    w = dataclasses.replace(base, name=base.name + "_" + decay, B=1, H=2, decay=decay)
    got, inp = _run(w)
    if w.T <= 4096:
        assert_parity(got, oracle.forward(*inp), BF16_TOL, w.name)
    else:
        rows = _sample_rows(w.T, w.C, 48, seed=3, seg_chunks=64)
        for bh in [(0, 0), (0, 1)]:
            want = oracle.forward_rows(*inp, bh, rows)
            assert_parity(got[bh[0], bh[1], rows], want, BF16_TOL, f"{w.name} {bh}")


def _sample_rows(T, C, n, seed, seg_chunks=16):
    """Random rows plus fixed ones: the ends of the sequence and of its first
    chunk, every segment boundary of a plan with seg_chunks chunks per segment
    (first row of each segment and the rows either side of it), and the first
    rows of chunks n whose lowest set bit is 4..7 (the chunks that read a
    freshly merged deep bucket state) with the last row before each."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, C - 1, C, T // 2, T // 2 - 1, T - C, T - 2, T - 1]
    seg = seg_chunks * C
    for x in range(seg, T, seg):
        fixed += [x - 1, x, x + 1]
    N = (T + C - 1) // C
    deep = [n for n in range(1, N) if 4 <= (n & -n).bit_length() - 1 <= 7]
    for n in deep[:24]:
        fixed += [n * C - 1, n * C, n * C + 37]
    rows = sorted(set(fixed) | set(rng.integers(0, T, n).tolist()))
    return [r for r in rows if 0 <= r < T]


@pytest.mark.parametrize("w", [W.LM_T16K, W.LONG_T64K], ids=lambda w: w.name)
def test_full_size_sampled_rows(w):
    """Full-size workloads in the launch configuration the bench uses
    (loglinear_fwd), checked on sampled rows of a few (b, h) pairs."""
    q, k, v, la, lam = W.make_fwd_inputs(w)
    announce(f"fwd full-size {w.name}")
    out = ll.fwd(*to_dev(q, k, v, la, lam), C=w.C)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(0)
    pairs = [(0, 0), (w.B - 1, w.H - 1)] + [(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(2)]
    rows = _sample_rows(w.T, w.C, 40, seed=1, seg_chunks=64 if w.T <= 16384 else 128)
    for bh in pairs[: 4 if w.T <= 16384 else 2]:
        want = oracle.forward_rows(q, k, v, la, lam, bh, rows)
        assert_parity(got[bh[0], bh[1], rows], want, BF16_TOL, f"{w.name} {bh}")


def test_deterministic_bitwise():
    w = dataclasses.replace(W.MAMBA2_T2K, B=2, H=4)
    q, k, v, la, lam = to_dev(*W.make_fwd_inputs(w))
    announce("determinism")
    a = ll.fwd(q, k, v, la, lam, C=64)
    b = ll.fwd(q, k, v, la, lam, C=64)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_caller_workspace_matches_owned():
    w = dataclasses.replace(W.MAMBA2_T2K, B=1, H=4, decay="weak")
    q, k, v, la, lam = to_dev(*W.make_fwd_inputs(w))
    n = ll.fwd_workspace_size(1, 4, w.T, w.dk, w.dv, w.C, 2)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    announce("caller workspace")
    a = ll.fwd_ex(q, k, v, la, lam, C=64, seg_log2=2)
    b = ll.fwd_ex(q, k, v, la, lam, C=64, seg_log2=2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


RS_CASES = [
    # (B, H, T, dk, dv, decay, seg_log2)
    (1, 2, 64, 128, 64, "none", -1),     # one chunk
    (1, 1, 65, 128, 64, "weak", 0),      # ragged tail of one token
    (2, 1, 1000, 128, 128, "weak", 2),
    (1, 2, 1000, 96, 64, "strong", 0),   # dk padded to 128
    (1, 1, 3000, 128, 192, "none", 3),   # three 64-column groups
    (1, 1, 4096, 128, 64, "weak", 4),
    (1, 1, 20000, 128, 64, "weak", 3),   # 313 chunks: the ten-slot instantiation
]


@pytest.mark.parametrize("case", RS_CASES, ids=lambda c: "B{}H{}T{}dk{}dv{}_{}_s{}".format(*c))
def test_register_state_kernel_parity(case):
    """The register-state sweep (bucket states in registers) forced on every
    shape class it covers, against the oracle and against the LDS-state sweep."""
    B, H, T, dk, dv, decay, s = case
    w = W.FwdWorkload("rs", B, H, T, dk, dv, 64, "bf16", decay=decay, seed=T + dv)
    q, k, v, la, lam = W.make_fwd_inputs(w)
    dq, dk_, dv_, dla, dlam = to_dev(q, k, v, la, lam)
    announce(f"register-state kernel {case}")
    rs = ll.fwd_ex(dq, dk_, dv_, dla, dlam, C=64, seg_log2=s, kernel=ll.KERNEL_REGISTER_STATE)
    lds = ll.fwd_ex(dq, dk_, dv_, dla, dlam, C=64, seg_log2=s, kernel=ll.KERNEL_LDS_STATE)
    torch.cuda.synchronize()
    want = oracle.forward(q, k, v, la, lam)
    assert_parity(rs.cpu().numpy(), want, BF16_TOL, f"register-state {case}")
    assert_parity(lds.cpu().numpy(), want, BF16_TOL, f"lds-state {case}")


@pytest.mark.parametrize("scale", [(8.0, 1e-4), (0.05, 1e3)], ids=["big_qk_small_v", "small_qk_big_v"])
def test_register_state_input_scales(scale):
    """The register-state sweep's fp16 operands (Q per chunk, the level states
    per wave) carry power-of-two scales chosen from their maxima, so extreme
    input magnitudes stay inside fp16's normal range: q, k scaled by 8 with v
    by 1e-4, and q, k by 0.05 with v by 1e3, weak decay, 16-chunk segments."""
    sq, sv = scale
    w = W.FwdWorkload("rs_scale", 1, 1, 4096, 128, 128, 64, "bf16", decay="weak", seed=31)
    q, k, v, la, lam = W.make_fwd_inputs(w)
    q = (q.float() * sq).to(q.dtype)
    k = (k.float() * sq).to(k.dtype)
    v = (v.float() * sv).to(v.dtype)
    announce(f"register-state input scales {scale}")
    out = ll.fwd_ex(*to_dev(q, k, v, la, lam), C=64, seg_log2=4, kernel=ll.KERNEL_REGISTER_STATE)
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy(), oracle.forward(q, k, v, la, lam), BF16_TOL, f"register-state scales {scale}")


def test_register_state_kernel_rejects_other_shapes():
    w = W.FwdWorkload("rs_no", 1, 1, 128, 128, 48, 64, "bf16")
    dq, dk_, dv_, dla, dlam = to_dev(*W.make_fwd_inputs(w))
    with pytest.raises(ll.LogLinearError):
        ll.fwd_ex(dq, dk_, dv_, dla, dlam, C=64, kernel=ll.KERNEL_REGISTER_STATE)


# ------------------------------------------------ the bench's launch plans, deep merges weighted

DEEP = [
    # (B, H, T, decay, seg_log2): seg_log2 6 is the plan at B=2 H=16 T=16384;
    # 7 with more than 256 chunks is the ten-slot plan of B=1 H=16 T=65536
    (1, 1, 16384, "none", 6),
    (1, 2, 16384, "weak", 6),
    (1, 1, 20000, "none", 7),
    (1, 1, 65536, "weak", 7),
]


@pytest.mark.parametrize("case", DEEP, ids=lambda c: "B{}H{}T{}_{}_s{}".format(*c))
def test_register_state_deep_merges(case):
    """Register-state sweep at the segment sizes the bench's plans use, with no
    or weak decay so the in-register merges at lssb 4..7 and the segment-
    spanning node states all carry weight; sampled rows include every
    segment boundary and the chunks that read a freshly merged deep state."""
    B, H, T, decay, s = case
    w = W.FwdWorkload("deep", B, H, T, 128, 128, 64, "bf16", decay=decay, seed=T + s)
    q, k, v, la, lam = W.make_fwd_inputs(w)
    announce(f"register-state deep merges {case}")
    out = ll.fwd_ex(*to_dev(q, k, v, la, lam), C=64, seg_log2=s, kernel=ll.KERNEL_REGISTER_STATE)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rows = _sample_rows(T, 64, 48, seed=5, seg_chunks=1 << s)
    for bh in [(b, h) for b in range(B) for h in range(H)]:
        want = oracle.forward_rows(q, k, v, la, lam, bh, rows)
        assert_parity(got[bh[0], bh[1], rows], want, BF16_TOL, f"deep {case} {bh}")


def test_bench_shape_weak_decay_auto_plan():
    """B=2, H=16, T=16384 (the bench's shape and automatic plan) with weak
    decay, on sampled rows of two (b, h) pairs."""
    w = dataclasses.replace(W.LM_T16K, name="lm_weak", decay="weak")
    q, k, v, la, lam = W.make_fwd_inputs(w)
    announce("bench shape, weak decay, automatic plan")
    out = ll.fwd(*to_dev(q, k, v, la, lam), C=64)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rows = _sample_rows(w.T, w.C, 40, seed=7, seg_chunks=64)
    for bh in [(0, 3), (1, 15)]:
        want = oracle.forward_rows(q, k, v, la, lam, bh, rows)
        assert_parity(got[bh[0], bh[1], rows], want, BF16_TOL, f"lm weak auto {bh}")


WIDE_CASES = [
    # (B, H, T, dk, decay, seg_log2): dv = 128
    (1, 2, 64, 128, "none", 3),      # one chunk
    (1, 1, 65, 128, "weak", 3),      # ragged tail of one token
    (2, 1, 1000, 128, "weak", 3),
    (1, 2, 1000, 96, "strong", 4),   # dk padded to 128
    (1, 1, 3000, 128, "none", 4),
    (1, 1, 4096, 128, "weak", 5),
    (1, 1, 8000, 128, "none", 5),
    (1, 1, 9000, 128, "weak", 6),
    (1, 1, 20000, 128, "weak", 6),   # ten chunk-level bits
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=lambda c: "B{}H{}T{}dk{}_{}_s{}".format(*c))
def test_wide_kernel_parity(case):
    """The full-width sweep (one workgroup per (b,h, segment), all 128 dv
    columns) forced on each segment size it is built for, against the oracle:
    full output up to T=4096, sampled rows (every segment boundary, chunks
    reading freshly merged deep states) beyond."""
    B, H, T, dk, decay, s = case
    w = W.FwdWorkload("wide", B, H, T, dk, 128, 64, "bf16", decay=decay, seed=T + dk + s)
    q, k, v, la, lam = W.make_fwd_inputs(w)
    announce(f"wide kernel {case}")
    out = ll.fwd_ex(*to_dev(q, k, v, la, lam), C=64, seg_log2=s, kernel=ll.KERNEL_WIDE)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    if T <= 4096:
        assert_parity(got, oracle.forward(q, k, v, la, lam), BF16_TOL, f"wide {case}")
    else:
        rows = _sample_rows(T, 64, 48, seed=11, seg_chunks=1 << s)
        for bh in [(b, h) for b in range(B) for h in range(H)]:
            want = oracle.forward_rows(q, k, v, la, lam, bh, rows)
            assert_parity(got[bh[0], bh[1], rows], want, BF16_TOL, f"wide {case} {bh}")


def test_wide_kernel_rejects_other_shapes():
    w = W.FwdWorkload("wide_no", 1, 1, 128, 128, 64, 64, "bf16")
    dq, dk_, dv_, dla, dlam = to_dev(*W.make_fwd_inputs(w))
    with pytest.raises(ll.LogLinearError):
        ll.fwd_ex(dq, dk_, dv_, dla, dlam, C=64, kernel=ll.KERNEL_WIDE)
    w = W.FwdWorkload("wide_no2", 1, 1, 4096, 128, 128, 64, "bf16")
    dq, dk_, dv_, dla, dlam = to_dev(*W.make_fwd_inputs(w))
    with pytest.raises(ll.LogLinearError):  # a segment size it is not built for
        ll.fwd_ex(dq, dk_, dv_, dla, dlam, C=64, seg_log2=2, kernel=ll.KERNEL_WIDE)
