"""HIP graph capture of the library's calls (the serving-loop use): the forward
with a caller workspace and the decode step allocate nothing and issue no
memsets, so they can be captured once and replayed.  Each replay is checked
against the eager result, with eager work and synchronisations between the
replays."""
import numpy as np
import pytest
import torch

import log_linear_attention_attn_amd as ll
import workloads as W
from gpu_util import announce, have_gpu, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def test_forward_graph_replays_match_eager():
    w = W.FwdWorkload("graph", 1, 2, 1000, 128, 64, 64, "bf16", decay="weak", seed=11)
    q, k, v, la, lam = to_dev(*W.make_fwd_inputs(w))
    ws = torch.empty(max(ll.fwd_workspace_size(w.B, w.H, w.T, w.dk, w.dv, w.C, 2), 1), dtype=torch.uint8,
                     device="cuda")
    announce("forward graph capture")
    eager = ll.fwd_ex(q, k, v, la, lam, C=w.C, seg_log2=2, workspace=ws).clone()
    out = torch.empty_like(eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ll.fwd_ex(q, k, v, la, lam, C=w.C, out=out, seg_log2=2, workspace=ws)
    for _ in range(3):
        out.fill_(float("nan"))            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


def test_decode_graph_replays_match_eager():
    wd = W.DecodeWorkload("graph_decode", 8, 4, 64, 64, 11, 1023, seed=3)
    S, q, k, v, la, lam, t = W.make_decode_inputs(wd)
    dq, dk_, dv_, dla, dlam, dt = to_dev(q, k, v, la, lam, t)
    announce("decode graph capture")
    S_eager = S.cuda()
    o_eager = ll.decode_step(S_eager, dq, dk_, dv_, dla, dlam, dt).clone()
    S_graph = S.cuda()
    out = torch.empty_like(o_eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ll.decode_step(S_graph, dq, dk_, dv_, dla, dlam, dt, out=out)
    for _ in range(3):
        # every replay starts from the same states as the eager step did
        S_graph.copy_(S.cuda())
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_eager)
        assert torch.equal(S_graph, S_eager)


def test_gdn_forward_graph_replays_match_eager():
    """The Gated DeltaNet forward with a caller workspace (preparation and
    level sweep) captured once and replayed."""
    w = W.GdnWorkload("graph_gdn", 1, 2, 700, 128, 32, "bf16", "weak", seed=12)
    q, k, v, la, beta, lam = to_dev(*W.make_gdn_inputs(w))
    ws = torch.empty(ll.gdn_workspace_size(w.B, w.H, w.T, w.dk, w.dv), dtype=torch.uint8, device="cuda")
    announce("gdn forward graph capture")
    eager = ll.gdn_fwd(q, k, v, la, beta, lam, workspace=ws).clone()
    out = torch.empty_like(eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ll.gdn_fwd(q, k, v, la, beta, lam, out=out, workspace=ws)
    for _ in range(3):
        out.fill_(float("nan"))
        ws.fill_(7)                        # the workspace's contents on entry must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
