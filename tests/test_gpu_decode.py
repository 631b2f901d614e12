"""GPU parity of the decode step (loglinear_decode_step / _f32) against the
CPU oracle, and of a chain of decode steps against the GPU forward.

The decode step is fp32 arithmetic on exact inputs, so outputs must match the
oracle to 1e-4 * RMS and states to 1e-5 * RMS(states); the set of zero and
non-zero levels after a step is compared exactly.
"""
import numpy as np
import pytest
import torch

import log_linear_attention_attn_amd as ll
import oracle
import workloads as W
from gpu_util import F32_TOL, announce, assert_parity, have_gpu, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _step(w, t=None):
    states, q, k, v, la, lam, tt = W.make_decode_inputs(w, t)
    announce(f"decode {w} t[:4]={tt[:4].tolist()}")
    dS, dq, dk_, dv_, dla, dlam, dt = to_dev(states, q, k, v, la, lam, tt)
    out = ll.decode_step(dS, dq, dk_, dv_, dla, dlam, dt)
    torch.cuda.synchronize()
    want_out, want_S = oracle.decode_step(states, q, k, v, la, lam, tt)
    return out.cpu().numpy(), dS.cpu().numpy(), want_out, want_S, states.numpy(), tt.numpy()


def _check_states(got_S, want_S, what):
    # exact zero / non-zero pattern per level
    gz = np.any(got_S != 0, axis=(-1, -2))
    wz = np.any(want_S != 0, axis=(-1, -2))
    assert np.array_equal(gz, wz), f"{what}: live-level pattern differs"
    assert_parity(got_S, want_S, 1e-5, what + " states")


def test_decode_workload_64x16():
    """64 sequences x 16 heads, dk=dv=128, L=17, t ~ U{1..65535}, bf16 q/k/v."""
    w = W.DECODE_64x16
    out, S, want_out, want_S, _, _ = _step(w)
    assert_parity(out, want_out, F32_TOL, w.name)
    _check_states(S, want_S, w.name)


def test_decode_special_positions():
    """t = 0 (all levels cleared), powers of two (one history bucket), the
    largest valid t, and odd / even mixes, on a small shape with fp32 inputs."""
    L = 9
    ts = np.array([0, 1, 2, 3, 4, 7, 8, 64, 200, 255, 128, 129], dtype=np.int32)
    w = W.DecodeWorkload("decode_special", len(ts), 3, 32, 48, L, 255, dtype="f32", seed=5)
    out, S, want_out, want_S, _, _ = _step(w, ts)
    assert_parity(out, want_out, F32_TOL, "special t")
    _check_states(S, want_S, "special t")


def test_decode_out_of_range_t():
    """t < 0 or t >= 2^(L-1): NaN output row, states untouched; other rows normal."""
    L = 6
    ts = np.array([-1, 32, 5, 1000], dtype=np.int32)
    w = W.DecodeWorkload("decode_oob", len(ts), 2, 16, 16, L, 31, dtype="bf16", seed=6)
    out, S, want_out, _, S_in, _ = _step(w, ts)
    assert np.all(np.isnan(out[[0, 1, 3]]))
    np.testing.assert_array_equal(S[[0, 1, 3]], S_in[[0, 1, 3]])
    assert_parity(out[2], want_out[2], F32_TOL, "in-range row")


def test_decode_chain_equals_forward():
    """Decode steps t = 0..T-1 from empty states reproduce the GPU forward
    (recurrent form == parallel form, on the GPU), fp32 inputs."""
    B, H, T, dk, dv = 1, 2, 150, 32, 32
    wf = W.FwdWorkload("chain", B, H, T, dk, dv, 16, "f32", decay="weak", seed=9)
    q, k, v, la, lam = to_dev(*W.make_fwd_inputs(wf))
    L = W.num_levels(T)
    announce("decode chain vs forward")
    fwd = ll.fwd(q, k, v, la, lam, C=16)
    S = torch.zeros(B, H, L, dk, dv, device="cuda")
    outs = []
    for t in range(T):
        tt = torch.full((B,), t, dtype=torch.int32, device="cuda")
        o = ll.decode_step(S, q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                           la[:, :, t].contiguous(), lam[:, :, t].contiguous(), tt)
        outs.append(o)
    rec = torch.stack(outs, dim=2)
    torch.cuda.synchronize()
    assert_parity(rec.cpu().numpy(), fwd.cpu().numpy(), F32_TOL, "chain vs fwd")
