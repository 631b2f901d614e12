"""GPU parity of the prefill -> decode handoff (loglinear_prefill and the
final_states option of loglinear_fwd_ex): the per-level decode states at
position T-1 against the oracle's states by definition, and decode steps that
continue from them against the dense forward of the longer sequence.

Tolerances as for the forward: max |gpu - oracle| <= 2e-2 * RMS(oracle) for
bf16 inputs, 1e-4 * RMS for fp32 inputs (outputs and states alike).
"""
import numpy as np
import pytest
import torch

import log_linear_attention_attn_amd as ll
import oracle
import workloads as W
from gpu_util import BF16_TOL, F32_TOL, announce, assert_parity, have_gpu, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

CASES = [
    # (B, H, T, dk, dv, C, dtype, decay, extra levels, seg_log2, kernel)
    (1, 2, 1, 16, 16, 16, "f32", "weak", 0, -1, ll.KERNEL_AUTO),          # one token
    (1, 1, 15, 32, 16, 16, "f32", "strong", 3, -1, ll.KERNEL_AUTO),       # inside one chunk, extra levels
    (1, 2, 200, 32, 32, 16, "f32", "weak", 1, 1, ll.KERNEL_AUTO),
    (2, 1, 777, 64, 32, 32, "bf16", "none", 0, 2, ll.KERNEL_AUTO),        # LDS-state sweep, ragged
    (1, 2, 1000, 128, 64, 64, "bf16", "weak", 2, 2, ll.KERNEL_REGISTER_STATE),
    (1, 2, 1000, 128, 64, 64, "bf16", "weak", 2, 2, ll.KERNEL_LDS_STATE),
    (1, 1, 3000, 96, 128, 64, "bf16", "strong", 0, 3, ll.KERNEL_REGISTER_STATE),  # dk padded
    (1, 1, 4096, 128, 128, 64, "bf16", "none", 0, -1, ll.KERNEL_AUTO),    # T a power of two
    (1, 1, 4095, 128, 64, 64, "bf16", "none", 0, -1, ll.KERNEL_AUTO),     # every level live
    (1, 2, 3000, 128, 128, 64, "bf16", "weak", 1, 3, ll.KERNEL_WIDE),     # full-width sweep, node levels
    (1, 1, 4095, 96, 128, 64, "bf16", "none", 0, 4, ll.KERNEL_WIDE),
]


def _tol(dtype):
    return BF16_TOL if dtype == "bf16" else F32_TOL


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}T{}dk{}dv{}C{}_{}_{}_L+{}_s{}_k{}".format(*c))
def test_prefill_states_match_definition(case):
    B, H, T, dk, dv, C, dtype, decay, extra, s, kernel = case
    w = W.FwdWorkload("prefill", B, H, T, dk, dv, C, dtype, decay=decay, seed=T + dk)
    q, k, v, la, lam = W.make_fwd_inputs(w)
    Ls = W.num_levels(T) + extra
    announce(f"prefill {case}")
    dq, dk_, dv_, dla, dlam = to_dev(q, k, v, la, lam)
    states = torch.full((B, H, Ls, dk, dv), float("nan"), device="cuda")  # every element must be written
    out = ll.fwd_ex(dq, dk_, dv_, dla, dlam, C=C, seg_log2=s, kernel=kernel, final_states=states)
    torch.cuda.synchronize()
    tol = _tol(dtype)
    assert_parity(out.cpu().numpy(), oracle.forward(q, k, v, la, lam), tol, f"out {case}")
    want = oracle.states_at(k, v, la, T - 1, Ls)
    got = states.cpu().numpy()
    assert_parity(got, want, tol, f"states {case}")
    # levels with no bucket at T-1 are exactly zero
    for l in range(1, Ls):
        if not ((T - 1) >> (l - 1)) & 1:
            assert not np.any(got[:, :, l]), f"level {l} should be empty"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_entry_point_matches_fwd_ex(dtype):
    w = W.FwdWorkload("prefill_ep", 1, 2, 300, 64, 64, 32 if dtype == "f32" else 64, dtype, decay="weak", seed=3)
    q, k, v, la, lam = to_dev(*W.make_fwd_inputs(w))
    announce(f"prefill entry point {dtype}")
    out1, st1 = ll.prefill(q, k, v, la, lam, C=w.C, L=W.num_levels(w.T) + 1)
    st2 = torch.empty_like(st1)
    out2 = ll.fwd_ex(q, k, v, la, lam, C=w.C, final_states=st2)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(st1, st2)


@pytest.mark.parametrize("dtype,T,C", [("bf16", 1000, 64), ("bf16", 1024, 64), ("f32", 333, 16)])
def test_decode_continues_from_prefill(dtype, T, C):
    """Prefill T tokens, then decode tokens T..T+5 one step at a time from the
    emitted states: the decode outputs equal rows T..T+5 of the dense forward
    over all T+6 tokens."""
    steps = 6
    dk, dv = (128, 64) if dtype == "bf16" else (32, 16)
    w = W.FwdWorkload("chain", 1, 2, T + steps, dk, dv, C, dtype, decay="weak", seed=T)
    q, k, v, la, lam = W.make_fwd_inputs(w)
    Lfull = lam.shape[-1]
    want = oracle.forward(q, k, v, la, lam)
    dq, dk_, dv_, dla, dlam = to_dev(q, k, v, la, lam)
    announce(f"prefill+decode {dtype} T={T}")
    out, states = ll.prefill(dq[:, :, :T].contiguous(), dk_[:, :, :T].contiguous(), dv_[:, :, :T].contiguous(),
                             dla[:, :, :T].contiguous(), dlam[:, :, :T, :W.num_levels(T)].contiguous(),
                             C=C, L=Lfull)
    tol = _tol(dtype)
    for i in range(steps):
        t = T + i
        o = ll.decode_step(states, dq[:, :, t].contiguous(), dk_[:, :, t].contiguous(), dv_[:, :, t].contiguous(),
                           dla[:, :, t].contiguous(), dlam[:, :, t].contiguous(),
                           torch.full((1,), t, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        assert_parity(o.cpu().numpy(), want[:, :, t], tol, f"decode t={t} after prefill {T}")
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy(), want[:, :, :T], tol, f"prefill out T={T}")


@pytest.mark.parametrize("T,decay,s,kernel", [(16384, "none", 6, "rs"), (20000, "weak", 7, "rs"),
                                              (16384, "none", 5, "wide"), (20000, "weak", 6, "wide")])
def test_prefill_states_at_bench_plans(T, decay, s, kernel):
    """Prefill states at the bench's segment sizes (64-chunk segments at
    T=16384, the ten-slot kernel with 128-chunk segments beyond 256 chunks),
    with no or weak decay so every inter-chunk level carries weight."""
    w = W.FwdWorkload("prefill_deep", 1, 1, T, 128, 128, 64, "bf16", decay=decay, seed=T)
    q, k, v, la, lam = W.make_fwd_inputs(w)
    Ls = W.num_levels(T)
    announce(f"prefill at bench plan T={T} s={s}")
    states = torch.full((1, 1, Ls, 128, 128), float("nan"), device="cuda")
    ll.fwd_ex(*to_dev(q, k, v, la, lam), C=64, seg_log2=s,
              kernel=ll.KERNEL_REGISTER_STATE if kernel == "rs" else ll.KERNEL_WIDE, final_states=states)
    torch.cuda.synchronize()
    want = oracle.states_at(k, v, la, T - 1, Ls)
    assert_parity(states.cpu().numpy(), want, BF16_TOL, f"states T={T} s={s}")
