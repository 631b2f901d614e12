"""GPU parity with q and k shared by groups of heads (multi-value attention,
the layout of the pages' log-linear Mamba-2 benchmark): forward (both sweep
kernels, several segmentations), prefill states, decode step and backward
against the oracle's *_mva functions.

Tolerances as for the per-head paths: forward, states and decode
max |gpu - oracle| <= 2e-2 * RMS(oracle) for bf16 inputs and 1e-4 * RMS for
fp32 inputs; backward 1e-4 * RMS of each gradient for fp32 inputs and the
bf16 bound for bf16 inputs.
"""
import numpy as np
import pytest
import torch

import log_linear_attention_attn_amd as ll
import oracle
import workloads as W
from gpu_util import BF16_TOL, F32_TOL, announce, assert_parity, have_gpu, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _tol(dtype):
    return BF16_TOL if dtype == "bf16" else F32_TOL


FWD_CASES = [
    # (B, H, Hk, T, dk, dv, C, dtype, decay, seg_log2, kernel)
    (1, 4, 1, 1000, 128, 128, 64, "bf16", "weak", 2, ll.KERNEL_REGISTER_STATE),  # ragged, segments
    (2, 6, 2, 700, 128, 64, 64, "bf16", "strong", -1, ll.KERNEL_AUTO),
    (1, 4, 2, 1000, 128, 64, 64, "bf16", "none", 1, ll.KERNEL_LDS_STATE),
    (1, 6, 3, 300, 32, 16, 16, "f32", "weak", 1, ll.KERNEL_AUTO),
    (2, 2, 1, 129, 64, 32, 32, "f32", "strong", 0, ll.KERNEL_AUTO),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "B{}H{}Hk{}T{}dk{}dv{}C{}_{}_{}_s{}_k{}".format(*c))
def test_mva_forward_and_prefill(case):
    B, H, Hk, T, dk, dv, C, dtype, decay, s, kernel = case
    w = W.FwdWorkload("mva", B, H, T, dk, dv, C, dtype, decay=decay, seed=T + H, Hk=Hk)
    q, k, v, la, lam = W.make_fwd_inputs(w)
    assert q.shape[1] == Hk and v.shape[1] == H
    announce(f"mva fwd {case}")
    dq, dk_, dv_, dla, dlam = to_dev(q, k, v, la, lam)
    Ls = W.num_levels(T)
    states = torch.full((B, H, Ls, dk, dv), float("nan"), device="cuda")
    out = ll.fwd_ex(dq, dk_, dv_, dla, dlam, C=C, seg_log2=s, kernel=kernel, final_states=states)
    torch.cuda.synchronize()
    tol = _tol(dtype)
    assert_parity(out.cpu().numpy(), oracle.forward_mva(q, k, v, la, lam), tol, f"out {case}")
    want = oracle.states_at(oracle.heads_of_qk(k, H), v, la, T - 1, Ls)
    assert_parity(states.cpu().numpy(), want, tol, f"states {case}")
    # the plain entry point and prefill route shared q/k through loglinear_fwd_ex
    out2 = ll.fwd(dq, dk_, dv_, dla, dlam, C=C)
    out3, st3 = ll.prefill(dq, dk_, dv_, dla, dlam, C=C)
    torch.cuda.synchronize()
    assert_parity(out2.cpu().numpy(), oracle.forward_mva(q, k, v, la, lam), tol, f"fwd {case}")
    assert_parity(st3.cpu().numpy(), want, tol, f"prefill states {case}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mva_decode_step(dtype):
    w = W.DecodeWorkload("mva_decode", 6, 8, 64, 32, 9, 255, dtype=dtype, seed=5, Hk=2)
    S, q, k, v, la, lam, t = W.make_decode_inputs(w, t=np.array([1, 2, 7, 64, 255, 0]))
    announce(f"mva decode {dtype}")
    dS, dq, dk_, dv_, dla, dlam, dt = to_dev(S, q, k, v, la, lam, t)
    out = ll.decode_step(dS, dq, dk_, dv_, dla, dlam, dt)
    torch.cuda.synchronize()
    want_o, want_s = oracle.decode_step_mva(S, q, k, v, la, lam, t)
    tol = _tol(dtype)
    assert_parity(out.cpu().numpy(), want_o, tol, f"decode out {dtype}")
    assert_parity(dS.cpu().numpy(), want_s, tol, f"decode states {dtype}")


BWD_CASES = [
    # (B, H, Hk, T, dk, dv, C, dtype, decay)
    (1, 4, 2, 200, 32, 32, 16, "f32", "weak"),
    (1, 4, 1, 300, 128, 64, 64, "bf16", "strong"),
    (2, 6, 3, 130, 64, 32, 32, "bf16", "none"),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "B{}H{}Hk{}T{}dk{}dv{}C{}_{}_{}".format(*c))
def test_mva_backward(case):
    B, H, Hk, T, dk, dv, C, dtype, decay = case
    w = W.FwdWorkload("mva_bwd", B, H, T, dk, dv, C, dtype, decay=decay, seed=T + dk, Hk=Hk)
    inp = W.make_fwd_inputs(w)
    dout = torch.from_numpy(np.random.default_rng(T).standard_normal((B, H, T, dv)).astype(np.float32))
    out = torch.from_numpy(oracle.forward_mva(*inp).astype(np.float32))
    announce(f"mva bwd {case}")
    grads = ll.bwd(*to_dev(*inp), out.cuda(), dout.cuda(), C=C)
    torch.cuda.synchronize()
    want = oracle.backward_mva(*inp, dout)
    for name, g, ref in zip(("dq", "dk", "dv", "dlog_a", "dlam"), grads, want):
        assert g.shape == ref.shape, name
        assert_parity(g.cpu().numpy(), ref, 1e-4 if dtype == "f32" else BF16_TOL, f"{name} {case}")
