"""GPU parity of the level-weight projection (loglinear_lambda_proj) and of
its gradient (loglinear_lambda_proj_bwd) against the oracle's
lambda_projection / lambda_projection_grad (fp64).  bf16 inputs are exact in
fp32 and the accumulation is fp32, so the bound is
max |gpu - oracle| <= 1e-4 * RMS(oracle) for both input types, per output."""
import numpy as np
import pytest
import torch

import log_linear_attention_attn_amd as ll
import oracle
import workloads as W
from gpu_util import F32_TOL, announce, assert_parity, have_gpu, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

CASES = [
    # (B, T, D, H, L, dtype, bias)
    (1, 1, 8, 1, 1, "bf16", True),          # one row, one output column
    (2, 300, 256, 4, 9, "bf16", True),      # ragged rows, one partial column tile
    (1, 1000, 2048, 16, 15, "bf16", True),  # the bench shape's width, 240 columns
    (1, 200, 512, 48, 15, "bf16", False),   # 720 columns: three column blocks, no bias
    (1, 130, 64, 20, 15, "f32", True),      # fp32, two column blocks
    (3, 77, 100, 3, 7, "f32", False),       # D not a multiple of the 64-wide K slice
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}T{}D{}H{}L{}_{}_bias{}".format(*c))
def test_lambda_proj_matches_oracle(case):
    B, T, D, H, L, dtype, bias = case
    w = W.LambdaProjWorkload("lp", B, T, D, H, L, dtype, bias, seed=T + D)
    x, Wt, b = W.make_lambda_proj_inputs(w)
    announce(f"lambda_proj {case}")
    dx, dW = to_dev(x, Wt)
    db = b.cuda() if b is not None else None
    out = torch.full((B, H, T, L), float("nan"), device="cuda")  # every element must be written
    got = ll.lambda_proj(dx, dW, db, H, L, out=out)
    torch.cuda.synchronize()
    want = oracle.lambda_projection(x, Wt, b, H, L)
    g = got.cpu().numpy()
    assert np.all(g > 0), "softplus output must be positive"
    assert_parity(g, want, F32_TOL, f"lambda {case}")


def test_lambda_proj_feeds_the_forward():
    """The projection's output used as the forward's lambda: the result equals
    the oracle forward on the oracle's lambda (bf16 forward tolerance)."""
    B, H, T, dk, dv, D = 1, 2, 300, 64, 64, 128
    L = W.num_levels(T)
    fw = W.FwdWorkload("lp_fwd", B, H, T, dk, dv, 64, "bf16", decay="weak", seed=3)
    q, k, v, la, _ = W.make_fwd_inputs(fw)
    x, Wt, b = W.make_lambda_proj_inputs(W.LambdaProjWorkload("lp_fwd", B, T, D, H, L, "bf16", seed=4))
    announce("lambda_proj -> fwd")
    dq, dk_, dv_, dla, dx, dW = to_dev(q, k, v, la, x, Wt)
    lam = ll.lambda_proj(dx, dW, b.cuda(), H, L)
    out = ll.fwd(dq, dk_, dv_, dla, lam, C=64)
    torch.cuda.synchronize()
    lam_ref = oracle.lambda_projection(x, Wt, b, H, L)
    from gpu_util import BF16_TOL
    assert_parity(out.cpu().numpy(), oracle.forward(q, k, v, la, lam_ref), BF16_TOL, "fwd with projected lambda")


BWD_CASES = [
    # (B, T, D, H, L, dtype)
    (1, 1, 8, 1, 1, "bf16"),          # one row, one output column
    (2, 300, 256, 4, 9, "bf16"),      # ragged rows (600), 36 columns
    (1, 1000, 2048, 16, 15, "bf16"),  # the bench shape's width, 240 columns, four row splits
    (3, 77, 200, 20, 15, "bf16"),     # 231 rows, 300 columns (3 tiles), D = 200 (ragged tile)
    (2, 50, 100, 3, 7, "bf16"),       # D % 8 != 0: the small-tile kernels
    (3, 77, 100, 3, 7, "f32"),        # D not a multiple of the 64-wide tile
    (1, 130, 64, 20, 15, "f32"),      # 300 columns: five column tiles
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "B{}T{}D{}H{}L{}_{}".format(*c))
def test_lambda_proj_bwd_matches_oracle(case):
    """The gradient from the GPU's own lambda (as a training step chains it)
    against the chain rule in fp64; two calls are bitwise equal.  Where the
    forward does not take the shape (bf16 rows need D % 8 == 0) lambda is the
    oracle's, rounded to fp32."""
    B, T, D, H, L, dtype = case
    w = W.LambdaProjWorkload("lpb", B, T, D, H, L, dtype, True, seed=T + 2 * D)
    x, Wt, b = W.make_lambda_proj_inputs(w)
    dlam = torch.from_numpy(np.random.default_rng(T + D).standard_normal((B, H, T, L)).astype(np.float32))
    announce(f"lambda_proj_bwd {case}")
    dx_, dW_ = to_dev(x, Wt)
    if dtype == "bf16" and D % 8:
        lam = torch.from_numpy(oracle.lambda_projection(x, Wt, b, H, L).astype(np.float32)).cuda()
    else:
        lam = ll.lambda_proj(dx_, dW_, b.cuda(), H, L)
    gx, gW, gb = ll.lambda_proj_bwd(dx_, dW_, lam, dlam.cuda())
    gx2, gW2, gb2 = ll.lambda_proj_bwd(dx_, dW_, lam, dlam.cuda())
    torch.cuda.synchronize()
    want = oracle.lambda_projection_grad(x, Wt, b, dlam, H, L)
    for name, g, ref in zip(("dx", "dW", "dbias"), (gx, gW, gb), want):
        assert tuple(g.shape) == ref.shape, name
        assert_parity(g.cpu().numpy(), ref, F32_TOL, f"{name} {case}")
    assert torch.equal(gx, gx2) and torch.equal(gW, gW2) and torch.equal(gb, gb2)


def test_lambda_proj_bwd_empty_batch_gives_zero_weight_gradients():
    """No rows: the weight and bias gradients are sums over nothing."""
    D, H, L = 16, 2, 3
    x = torch.empty((0, 5, D), dtype=torch.bfloat16, device="cuda")
    Wt = torch.ones((H * L, D), dtype=torch.bfloat16, device="cuda")
    lam = torch.empty((0, H, 5, L), device="cuda")
    announce("lambda_proj_bwd empty")
    gx, gW, gb = ll.lambda_proj_bwd(x, Wt, lam, lam.clone())
    torch.cuda.synchronize()
    assert gx.shape == (0, 5, D)
    assert torch.equal(gW.cpu(), torch.zeros(H * L, D)) and torch.equal(gb.cpu(), torch.zeros(H * L))



def test_lambda_proj_bwd_unaligned_rows_take_the_general_kernels():
    """bf16 x starting 2 bytes past a 16-byte boundary: the gradient takes the
    small-tile kernels (the matrix-core path needs 16-byte aligned rows) and
    still matches the oracle."""
    B, T, D, H, L = 1, 200, 256, 4, 9
    w = W.LambdaProjWorkload("lpb_unaligned", B, T, D, H, L, "bf16", True, seed=7)
    x, Wt, b = W.make_lambda_proj_inputs(w)
    dlam = torch.from_numpy(np.random.default_rng(8).standard_normal((B, H, T, L)).astype(np.float32))
    announce("lambda_proj_bwd unaligned x")
    store = torch.empty(B * T * D + 1, dtype=torch.bfloat16, device="cuda")
    xu = store[1:].view(B, T, D)  # contiguous, data pointer 2 bytes past the allocation
    xu.copy_(x.cuda())
    assert xu.data_ptr() % 16 != 0
    dW_ = Wt.cuda()
    lam = torch.from_numpy(oracle.lambda_projection(x, Wt, b, H, L).astype(np.float32)).cuda()
    gx, gW, gb = ll.lambda_proj_bwd(xu, dW_, lam, dlam.cuda())
    torch.cuda.synchronize()
    want = oracle.lambda_projection_grad(x, Wt, b, dlam, H, L)
    for name, g, ref in zip(("dx", "dW", "dbias"), (gx, gW, gb), want):
        assert_parity(g.cpu().numpy(), ref, F32_TOL, f"{name} unaligned")
