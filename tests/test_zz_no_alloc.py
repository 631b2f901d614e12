"""GPU check of the allocation-free forward (loglinear_fwd_noalloc) against
loglinear_fwd: the same kernels and plan, so the outputs must be bitwise
equal.  Consecutive calls share the library's static scratch, the later ones
on smaller inputs, so a stale value left by an earlier call would show."""
import numpy as np
import pytest
import torch

import log_linear_attention_attn_amd as ll
import oracle
import workloads as W
from gpu_util import BF16_TOL, announce, assert_parity, have_gpu, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

CASES = [
    # (B, H, T, dk, dv, C, decay): the register-state plan with segment and
    # block states, then smaller inputs (fewer segments), then the LDS-state
    # plan (dk = 64, C = 32)
    (2, 4, 4096, 128, 128, 64, "weak"),
    (1, 2, 1000, 128, 64, 64, "none"),
    (1, 1, 777, 64, 32, 32, "weak"),
]


def test_noalloc_matches_fwd_on_consecutive_calls():
    for i, (B, H, T, dk, dv, C, decay) in enumerate(CASES):
        assert ll.fwd_workspace_size(B, H, T, dk, dv, C) > 0, "the case must use the scratch"
        w = W.FwdWorkload("noalloc", B, H, T, dk, dv, C, "bf16", decay=decay, seed=40 + i)
        q, k, v, la, lam = W.make_fwd_inputs(w)
        dev = to_dev(q, k, v, la, lam)
        announce(f"fwd_noalloc call {i}: B={B} H={H} T={T} dk={dk} dv={dv} C={C} {decay}")
        want = ll.fwd(*dev, C=C)
        out = torch.full((B, H, T, dv), float("nan"), device="cuda")
        got = ll.fwd_noalloc(*dev, C=C, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, want), f"call {i}: differs from loglinear_fwd"
        if T <= 1000:
            assert_parity(got.cpu().numpy(), oracle.forward(q, k, v, la, lam), BF16_TOL, f"noalloc call {i}")


def test_noalloc_rejects_oversized_plan():
    w = W.FwdWorkload("noalloc_big", 1, 1, 64, 16, 16, 16, "bf16")
    q, k, v, la, lam = to_dev(*W.make_fwd_inputs(w))
    assert ll.fwd_workspace_size(1, 1, 65536, 128, 1024, 16) > ll.NOALLOC_SCRATCH_BYTES
    # shape-consistent tensors are not needed: the size check comes first on the host
    with pytest.raises(ll.LogLinearError):
        big = [torch.empty(0, device="cuda")] * 6
        st = ll.lib().loglinear_fwd_noalloc(*[ll._ptr(t) for t in big], 1, 1, 65536, 128, 1024, 16, None)
        ll._raise(st, "loglinear_fwd_noalloc")
