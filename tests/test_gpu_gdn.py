"""GPU parity of the log-linear Gated DeltaNet forward (loglinear_gdn_fwd)
against the fp64 oracle (oracle/gated_deltanet.py; parity unpinned by the
pages, pinned by the mathematics in tests/test_oracle_gdn.py).

Tolerance: max |gpu - oracle| <= GDN_TOL * RMS(oracle).  The kernels run
fp32 end to end (fp32 matrix cores); bf16 inputs are rounded once and the
oracle gets the same rounded values, so the bound is the same for both input
types.  Error sources: fp32 products of length <= 128 (~1e-6 relative), the
in-chunk triangular solve (unit-diagonal, entries |beta (k.k) Gamma| < 1 for
unit keys) and the in-chunk prefix sums of log alpha, taken as a compensated
sum so that the rounding of the running sum (|g| up to ~150 under strong
decay) does not reach the decay factors; GDN_TOL = 1e-4 leaves room for the
chunk-to-chunk carries of the bucket states (measured <= 4.7e-6).
"""
import numpy as np
import pytest
import torch

import log_linear_attention_attn_amd as ll
import workloads as W
from oracle import gated_deltanet as G
from gpu_util import announce, assert_parity, have_gpu, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

GDN_TOL = 1e-4

CASES = [
    # (B, H, T, dk, dv, dtype, decay)
    (1, 1, 1, 64, 16, "f32", "weak"),        # one token
    (1, 2, 64, 64, 16, "f32", "none"),       # one full chunk
    (1, 1, 200, 64, 32, "f32", "strong"),    # ragged, four chunks
    (2, 1, 300, 128, 64, "bf16", "weak"),
    (1, 1, 1000, 128, 128, "bf16", "none"),  # 16 chunks, chunk-level bits 0-3
    (1, 2, 700, 128, 48, "f32", "weak"),     # three column slices (grid not a multiple of 8)
    (1, 1, 4200, 128, 32, "f32", "weak"),    # 66 chunks: chunk-level bits 0-6, ragged
    (1, 1, 2500, 64, 64, "bf16", "none"),    # dk = 64, 40 chunks
    (1, 1, 4200, 128, 64, "bf16", "strong"), # strong decay over 66 chunks: in-chunk gammas underflow to 0
]


def _run(case, seed):
    B, H, T, dk, dv, dtype, decay = case
    w = W.GdnWorkload("gdn", B, H, T, dk, dv, dtype, decay, seed=seed)
    inp = W.make_gdn_inputs(w)
    announce(f"gdn {case}")
    got = ll.gdn_fwd(*to_dev(*inp))
    torch.cuda.synchronize()
    return inp, got.cpu().numpy()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}T{}dk{}dv{}_{}_{}".format(*c))
def test_gdn_matches_oracle(case):
    inp, got = _run(case, seed=case[2] + case[4])
    want = G.loglinear_forward(*inp)
    assert_parity(got, want, GDN_TOL, f"gdn {case}")


def test_gdn_unit_lambda_is_gated_deltanet():
    """lambda = 1 on every level: the GPU result is Gated DeltaNet's own
    one-token recurrence (oracle.gated_delta_recurrent)."""
    w = W.GdnWorkload("gdn", 1, 2, 300, 64, 32, "f32", "weak", seed=4)
    q, k, v, la, beta, lam = W.make_gdn_inputs(w)
    lam = torch.ones_like(lam)
    announce("gdn unit lambda")
    got = ll.gdn_fwd(*to_dev(q, k, v, la, beta, lam)).cpu().numpy()
    assert_parity(got, G.gated_delta_recurrent(q, k, v, la, beta), GDN_TOL, "gdn unit lambda")


def test_gdn_headline_shape_sampled_rows():
    """B=2 H=16 T=16384 dk=dv=128 (256 chunks, chunk-level bits 0-7, 256
    workgroups), weak decay so every level carries weight: sampled rows of
    two heads against the one-row oracle, at chunk and Fenwick boundaries."""
    w = W.GDN_LM_T16K
    inp = W.make_gdn_inputs(w)
    announce("gdn B2H16 T16384 sampled")
    dev = to_dev(*inp)
    ws = torch.empty(ll.gdn_workspace_size(w.B, w.H, w.T, w.dk, w.dv), dtype=torch.uint8, device="cuda")
    got = ll.gdn_fwd(*dev, workspace=ws)
    again = ll.gdn_fwd(*dev)
    torch.cuda.synchronize()
    assert torch.equal(got, again), "workspace and allocating calls differ"
    got = got.cpu().numpy()
    rng = np.random.default_rng(5)
    fixed = [0, 63, 64, 127, 128, 1023, 1024, 4095, 4096, 8191, 8192, 12287, 16320, 16383]
    rows = sorted(set(fixed) | set(rng.integers(0, w.T, 6).tolist()))
    for bh in [(0, 0), (1, 15)]:
        want = G.loglinear_rows(*inp, bh, rows)
        assert_parity(got[bh][rows], want, GDN_TOL, f"gdn T16384 rows {bh}")


def test_gdn_deterministic():
    w = W.GdnWorkload("gdn", 1, 2, 900, 128, 32, "bf16", "weak", seed=6)
    dev = to_dev(*W.make_gdn_inputs(w))
    announce("gdn determinism")
    a = ll.gdn_fwd(*dev)
    b = ll.gdn_fwd(*dev)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("T,decay", [(65536, "weak"), (8192, "none")], ids=["T65536_weak", "T8192_none"])
def test_gdn_long_sampled_rows(T, decay):
    """One (b,h), one 16-column slice: T = 65536 walks 1024 chunks with ten
    chunk-level bits (the sweep's LDS at 124 KiB); T = 8192 ends exactly on a
    chunk boundary with 128 chunks.  Sampled rows at chunk, Fenwick and
    end-of-sequence boundaries against the one-row oracle."""
    w = W.GdnWorkload("gdn_long", 1, 1, T, 128, 16, "bf16", decay, seed=T % 97)
    inp = W.make_gdn_inputs(w)
    announce(f"gdn long T={T} {decay}")
    got = ll.gdn_fwd(*to_dev(*inp)).cpu().numpy()
    fixed = [0, 63, 64, 4095, 4096, T // 2 - 1, T // 2, T - 65, T - 64, T - 1]
    rows = sorted(set(r for r in fixed if r < T) | set(np.random.default_rng(3).integers(0, T, 4).tolist()))
    want = G.loglinear_rows(*inp, (0, 0), rows)
    assert_parity(got[0, 0][rows], want, GDN_TOL, f"gdn T={T} rows")


def _decode_case(w, t=None):
    S, q, k, v, la, beta, lam, tt = W.make_gdn_decode_inputs(w, t)
    dS = S.cuda()
    o = ll.gdn_decode_step(dS, *to_dev(q, k, v, la, beta, lam, tt))
    torch.cuda.synchronize()
    want_o, want_S = G.decode_step(S, q, k, v, la, beta, lam, tt)
    return o.cpu().numpy(), dS.cpu().numpy(), want_o, want_S, S.numpy()


def test_gdn_decode_full_workload():
    """64 sequences x 16 heads, dk = dv = 128, L = 17, random t: outputs and
    every updated state against the oracle step; levels dead at t are 0."""
    w = W.GDN_DECODE_64x16
    announce("gdn decode 64x16")
    o, S, want_o, want_S, _ = _decode_case(w)
    assert_parity(o, want_o, GDN_TOL, "gdn decode out")
    assert_parity(S, want_S, 1e-5, "gdn decode states")
    assert np.array_equal(S == 0, want_S == 0)


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 64, 20), ("bf16", 128, 200)])
def test_gdn_decode_special_positions(dtype, dk, dv):
    """t = 0 (every level cleared), powers of two (one merged bucket), odd t,
    the last valid position 2^(L-1) - 1, and out-of-range positions (NaN
    output, states untouched); dv not a multiple of 64."""
    Lv = 9
    t = np.array([0, 1, 2, 64, 127, 128, 255, 256, 300, -1], dtype=np.int32)
    w = W.DecodeWorkload("gdn_dec_special", len(t), 3, dk, dv, Lv, 255, dtype=dtype, seed=dk + dv)
    announce(f"gdn decode special {dtype} {dk} {dv}")
    o, S, want_o, want_S, S0 = _decode_case(w, t)
    ok = (t >= 0) & (t < 256)
    assert_parity(o[ok], want_o[ok], GDN_TOL, "gdn decode special out")
    assert_parity(S[ok], want_S[ok], 1e-5, "gdn decode special states")
    assert np.all(np.isnan(o[~ok]))
    assert np.array_equal(S[~ok], S0[~ok])


def test_gdn_decode_chain_matches_forward():
    """Decode steps on the GPU from empty states over t = 0..T-1 give the GPU
    forward's rows (two GPU kernels that share no code path)."""
    B, H, T, dk, dv = 2, 2, 130, 64, 32
    wf = W.GdnWorkload("gdn_chain", B, H, T, dk, dv, "f32", "weak", seed=9)
    q, k, v, la, beta, lam = to_dev(*W.make_gdn_inputs(wf))
    announce("gdn decode chain")
    fwd = ll.gdn_fwd(q, k, v, la, beta, lam)
    S = torch.zeros((B, H, lam.shape[-1], dk, dv), dtype=torch.float32, device="cuda")
    outs = []
    for t in range(T):
        tt = torch.full((B,), t, dtype=torch.int32, device="cuda")
        outs.append(ll.gdn_decode_step(S, q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                       v[:, :, t].contiguous(), la[:, :, t].contiguous(),
                                       beta[:, :, t].contiguous(), lam[:, :, t].contiguous(), tt))
    dec = torch.stack(outs, dim=2)
    torch.cuda.synchronize()
    assert_parity(dec.cpu().numpy(), fwd.cpu().numpy(), GDN_TOL, "gdn decode chain vs forward")


@pytest.mark.parametrize("T", [1, 37, 64, 65, 200, 4200, 8192])
def test_gdn_prefill_states(T):
    """The prefill's decode states at T-1 against the oracle's level states
    (one ragged or full last chunk, in-chunk buckets of every size, chunk-level
    buckets up to bit 6), with two extra levels that must be 0."""
    w = W.GdnWorkload("gdn_prefill", 1, 2, T, 128 if T > 100 else 64, 32, "f32", "weak", seed=T)
    inp = W.make_gdn_inputs(w)
    announce(f"gdn prefill T={T}")
    out, st = ll.gdn_prefill(*to_dev(*inp), L=w.L + 2)
    torch.cuda.synchronize()
    want = G.states_after(inp[1], inp[2], inp[3], inp[4], T - 1, w.L + 2)
    assert_parity(st.cpu().numpy(), want, GDN_TOL, f"gdn prefill states T={T}")
    assert not st[:, :, w.L:].any()
    assert torch.equal(out, ll.gdn_fwd(*to_dev(*inp)))


def test_gdn_prefill_then_decode_matches_forward():
    """Prefill over the first 300 tokens, then decode steps 300..339 from its
    states: the rows equal the GPU forward over all 340 tokens."""
    B, H, T0, T, dk, dv = 2, 2, 300, 340, 128, 64
    wf = W.GdnWorkload("gdn_handoff", B, H, T, dk, dv, "bf16", "none", seed=13)
    q, k, v, la, beta, lam = to_dev(*W.make_gdn_inputs(wf))
    announce("gdn prefill then decode")
    full = ll.gdn_fwd(q, k, v, la, beta, lam)
    L = lam.shape[-1]
    _, S = ll.gdn_prefill(q[:, :, :T0].contiguous(), k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous(),
                          la[:, :, :T0].contiguous(), beta[:, :, :T0].contiguous(),
                          lam[:, :, :T0, :W.num_levels(T0)].contiguous(), L=L)
    rows = []
    for t in range(T0, T):
        tt = torch.full((B,), t, dtype=torch.int32, device="cuda")
        rows.append(ll.gdn_decode_step(S, q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                       v[:, :, t].contiguous(), la[:, :, t].contiguous(),
                                       beta[:, :, t].contiguous(), lam[:, :, t].contiguous(), tt))
    dec = torch.stack(rows, dim=2)
    torch.cuda.synchronize()
    assert_parity(dec.cpu().numpy(), full[:, :, T0:].cpu().numpy(), GDN_TOL, "gdn prefill -> decode")
