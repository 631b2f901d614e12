"""Benchmark of the log-linear attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 300] [--workload NAME] [--no-cpu-baseline]
                    [--headline-only] [--pass fwd|bwd|decode|lambda|gdn]

A step is one loglinear_fwd_ex call (segment-state, node and sweep kernels,
caller-owned workspace) over one batch of synthetic inputs already resident in
HBM.  Prints ONE JSON line.  At the default workload the line also carries,
each timed the same way:
  "configs"     the forward at B=8 H=8 T=2048 dk=128 dv=64 (L=12) and at
                B=1 H=16 T=65536 dk=dv=128 (L=17), each with its own roofline;
  "bwd"         the backward (gradients of q, k, v, log_a, lambda) of the
                headline workload;
  "prefill"     the forward plus the decode states at T-1;
  "decode"      one decode step of 64 sequences x 16 heads, L = 17;
  "lambda_proj" the level-weight projection at the same B, T, H, L with hidden
                width 2048, and its gradient;
  "gdn"         the log-linear Gated DeltaNet forward at the same B, H, T, dk, dv,
                and its decode step at the decode step's shapes;
  "pages_context" the pages' own speed statements (context, not a target).
The backward and the configs run before the headline forward is timed.
--pass bwd / decode / lambda / gdn time only the backward, the decode step, the
projection or the Gated DeltaNet forward.
Default workload: log-linear Mamba-2 forward, B=2, H=16, T=16384, dk=dv=128,
bf16 q/k/v, fp32 log_a / lambda / out, L=15, C=64.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd tokens/sec + TFLOP/s vs bf16 MFMA peak, log-linear Mamba-2 at T=16K"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 matrix

# What the pages say about speed, restated, with the hardware they name.
# Context only: they print no runtime or throughput figure for this path.
PAGES_CONTEXT = (
    "Context, not a target: the pages publish no kernel time or throughput for this path. "
    "In their words restated: a custom Triton chunkwise kernel for log-linear Mamba-2 overtakes "
    "FlashAttention-2 in forward+backward kernel time once sequences pass roughly 8K tokens, "
    "and the whole log-linear Mamba-2 model trains faster than a Transformer at 32K; all on one "
    "NVIDIA H100, batch 2, 48 heads, head dim 64, state dim 128, chunk 64, Mamba-2 with "
    "multi-value attention against FlashAttention-2 with grouped-query attention, lengths up to "
    "131K, precision not stated (paper-reading blog, experiment results / training efficiency; "
    "news write-up, Fig. 4 and its setup; journal-club slides, slide 39)."
)


def algorithmic_flops(B, H, T, dk, dv, C):
    """Multiply-adds x2 the method must do (not the dense work it avoids):
    causal intra-chunk pairs, chunk states, popcount-weighted inter-chunk reads."""
    N = -(-T // C)
    intra = 0
    for n in range(N):
        c = min(C, T - n * C)
        intra += c * (c + 1) // 2 * 2 * (dk + dv)
    states = (N - 1) * 2 * C * dk * dv
    inter = sum(bin(n).count("1") for n in range(N)) * 2 * C * dk * dv
    return B * H * (intra + states + inter)


def algorithmic_bytes(B, H, T, dk, dv, L, in_bytes=2):
    """Minimal HBM traffic: q, k, v, log_a, lambda read once, fp32 out written once."""
    per = (2 * dk + dv) * in_bytes + 4 + 4 * L + 4 * dv
    return B * H * T * per


def algorithmic_flops_bwd(B, H, T, dk, dv, C):
    """dQ, dK and dV each have the forward's pair structure (causal in-chunk
    pairs, chunk states, popcount-weighted bucket reads), and the in-chunk
    dlambda needs the two score matrices q.k and dO.v once more."""
    N = -(-T // C)
    pairs = sum(min(C, T - n * C) * (min(C, T - n * C) + 1) // 2 for n in range(N))
    return 3 * algorithmic_flops(B, H, T, dk, dv, C) + B * H * pairs * 2 * (dk + dv)


def algorithmic_bytes_bwd(B, H, T, dk, dv, L, in_bytes=2):
    """q, k, v, log_a, lambda, out and dout read once; fp32 dq, dk, dv, dlog_a,
    dlambda written once."""
    per = (2 * dk + dv) * in_bytes + 4 + 4 * L + 4 * dv + 4 * dv + 4 * (2 * dk + dv) + 4 + 4 * L
    return B * H * T * per


def decode_bytes(t, H, L, dk, dv, in_bytes=2):
    """HBM bytes one decode step must move for the positions t (one per
    sequence, all H heads): with m = lssb(t), read S^0..S^m and the live levels
    above m+1, write S^0..S^(m+1) (levels 1..m cleared) and those live levels;
    plus q, k, v, log_a, lambda, out and t.  t = 0 writes every level."""
    lvl = dk * dv * 4
    total = 0
    for x in t:
        x = int(x)
        if x == 0:
            rd, wr = 0, L
        else:
            m = (x & -x).bit_length() - 1
            high = bin(x >> (m + 1)).count("1")
            rd, wr = m + 1 + high, m + 2 + high
        total += H * ((rd + wr) * lvl + (2 * dk + dv) * in_bytes + 4 + 4 * L + 4 * dv) + 4
    return total


def bench_decode(dev, steps: int, warmup: int):
    """One decode step (loglinear_decode_step) for 64 sequences x 16 heads,
    dk = dv = 128, L = 17, t ~ U{1..65535}: states [64,16,17,128,128] fp32
    (1.14 GB) resident in HBM and updated in place.  Every timed step repeats
    the step at the same positions, so each moves the same bytes."""
    import torch
    import log_linear_attention_attn_amd as ll
    import workloads as W
    w = W.DECODE_64x16
    S, q, k, v, la, lam, t = W.make_decode_inputs(w)
    t_host = t.numpy().copy()
    S, q, k, v, la, lam, t = (x.to(dev) for x in (S, q, k, v, la, lam, t))
    out = torch.empty(w.N, w.H, w.dv, dtype=torch.float32, device=dev)
    for _ in range(warmup):
        ll.decode_step(S, q, k, v, la, lam, t, out=out)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        ll.decode_step(S, q, k, v, la, lam, t, out=out)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    nbytes = decode_bytes(t_host, w.H, w.L, w.dk, w.dv, 2 if w.dtype == "bf16" else 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    del S
    return {
        "workload": w.name, "N": w.N, "H": w.H, "dk": w.dk, "dv": w.dv, "L": w.L,
        "t": "U{1..65535} per sequence, seed 0", "steps": steps, "ms_per_step": ms,
        "tokens_per_s": w.N / (ms * 1e-3), "algorithmic_bytes": nbytes,
        "roofline": {"kernel": "decode_kernel", "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS},
    }


def bench_gdn_decode(dev, steps: int, warmup: int):
    """One log-linear Gated DeltaNet decode step (loglinear_gdn_decode_step) for
    64 sequences x 16 heads, dk = dv = 128, L = 17, t ~ U{1..65535}, timed like
    bench_decode.  It moves the Mamba-2 step's bytes plus beta: each live level
    is read once and written once."""
    import torch
    import log_linear_attention_attn_amd as ll
    import workloads as W
    w = W.GDN_DECODE_64x16
    S, q, k, v, la, beta, lam, t = W.make_gdn_decode_inputs(w)
    t_host = t.numpy().copy()
    S, q, k, v, la, beta, lam, t = (x.to(dev) for x in (S, q, k, v, la, beta, lam, t))
    out = torch.empty(w.N, w.H, w.dv, dtype=torch.float32, device=dev)
    for _ in range(warmup):
        ll.gdn_decode_step(S, q, k, v, la, beta, lam, t, out=out)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        ll.gdn_decode_step(S, q, k, v, la, beta, lam, t, out=out)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    nbytes = decode_bytes(t_host, w.H, w.L, w.dk, w.dv, 2 if w.dtype == "bf16" else 4) + w.N * w.H * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    del S
    return {
        "workload": w.name, "N": w.N, "H": w.H, "dk": w.dk, "dv": w.dv, "L": w.L,
        "t": f"U{{1..65535}} per sequence, seed {w.seed}", "steps": steps, "ms_per_step": ms,
        "tokens_per_s": w.N / (ms * 1e-3), "algorithmic_bytes": nbytes,
        "roofline": {"kernel": "gdn_decode_kernel", "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS},
    }


def bench_lambda(dev, steps: int, warmup: int):
    """The level-weight projection (loglinear_lambda_proj) at the bench
    forward's shape: x [2, 16384, 2048] bf16 (hidden width H * dv), W [240, 2048]
    bf16, bias fp32 -> lambda [2, 16, 16384, 15] fp32; three x buffers rotated."""
    import torch
    import log_linear_attention_attn_amd as ll
    import workloads as W
    w = W.LAMBDA_LM_T16K
    x, Wt, b = W.make_lambda_proj_inputs(w)
    xs = [x.to(dev)] + [x.to(dev) for _ in range(2)]
    Wt, b = Wt.to(dev), b.to(dev)
    out = torch.empty(w.B, w.H, w.T, w.L, dtype=torch.float32, device=dev)
    for i in range(warmup):
        ll.lambda_proj(xs[i % 3], Wt, b, w.H, w.L, out=out)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        ll.lambda_proj(xs[i % 3], Wt, b, w.H, w.L, out=out)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    ib = 2 if w.dtype == "bf16" else 4
    nbytes = w.B * w.T * w.D * ib + w.H * w.L * (w.D * ib + 4) + w.B * w.H * w.T * w.L * 4
    flops = 2 * w.B * w.T * w.D * w.H * w.L
    gbs = nbytes / (ms * 1e-3) / 1e9
    # gradient (loglinear_lambda_proj_bwd) from the last lambda and a fixed
    # dlambda: dx = dz W and dW = dz^T x (+ dbias); bf16 inputs on bf16 matrix
    # cores with dz split hi/lo, fp32 inputs on fp32 matrix cores
    dlam = torch.randn(w.B, w.H, w.T, w.L, generator=torch.Generator().manual_seed(0)).to(dev)
    bsteps, bwarm = max(3, steps // 2), 3
    for i in range(bwarm):
        ll.lambda_proj_bwd(xs[i % 3], Wt, out, dlam)
    torch.cuda.synchronize()
    start.record()
    for i in range(bsteps):
        ll.lambda_proj_bwd(xs[i % 3], Wt, out, dlam)
    stop.record()
    torch.cuda.synchronize()
    bms = start.elapsed_time(stop) / bsteps
    bflops = 2 * flops + w.B * w.T * w.H * w.L * 2
    bbytes = (w.B * w.T * w.D * (ib + 4) + w.H * w.L * (w.D * (ib + 4) + 4)
              + 2 * w.B * w.H * w.T * w.L * 4)
    btf = bflops / (bms * 1e-3) / 1e12
    bgbs = bbytes / (bms * 1e-3) / 1e9
    # bf16 inputs: bf16 matrix cores (dz split hi/lo), intensity ~137 flop/B is
    # below the bf16 ridge -> HBM-bound; fp32 inputs: fp32 matrix cores, above
    # the fp32 ridge (~20 flop/B) -> bound by the fp32 matrix peak.  The rate
    # is over the whole call (dz kernel, the two products, the in-order sums).
    if w.dtype == "bf16":
        broof = {"kernel": "whole gradient (lam_dz16_kernel, lam_mm16_kernel x2, sums)", "bound": "hbm",
                 "achieved": bgbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": bgbs / PEAK_HBM_GBS}
    else:
        broof = {"kernel": "lam_gemm_kernel", "bound": "mfma", "achieved": btf, "peak": PEAK_FP32_TFLOPS,
                 "unit": "TFLOP/s", "frac": btf / PEAK_FP32_TFLOPS}
    return {
        "workload": w.name, "B": w.B, "T": w.T, "D": w.D, "H": w.H, "L": w.L, "dtype": w.dtype,
        "steps": steps, "ms_per_step": ms, "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
        "tflops": flops / (ms * 1e-3) / 1e12,
        "roofline": {"kernel": "lambda_proj_kernel", "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS},
        "bwd": {"steps": bsteps, "ms_per_step": bms, "algorithmic_flops": bflops, "algorithmic_bytes": bbytes,
                "tflops": btf, "roofline": broof},
    }


def sweep_kernel(w) -> str:
    """The sweep kernel the automatic plan launches for workload w."""
    rs = (w.dtype == "bf16" and w.C == 64 and w.dk > 64 and w.dv % 64 == 0
          and -(-w.T // 64) <= 1024)
    return "fwd_rs_kernel" if rs else "fwd_sweep_kernel"


def upload_fwd(w, dev, nsets: int = 1, base=None):
    """Device input sets (nsets buffers holding the same values), the output
    and the caller-owned workspace for timing workload w; base: the host
    inputs, made here when not given."""
    import torch
    import log_linear_attention_attn_amd as ll
    import workloads as W
    if base is None:
        base = W.make_fwd_inputs(w)
    sets = [[t.to(dev) for t in base]]
    sets += [[t.clone() for t in sets[0]] for _ in range(nsets - 1)]
    out = torch.empty(w.B, w.H, w.T, w.dv, dtype=torch.float32, device=dev)
    return sets, out


def bench_fwd(w, dev, K: int, Wm: int, seg_log2: int = -1, nsets: int = 1, uploaded=None):
    """Time K forwards (loglinear_fwd_ex, caller-owned workspace, so no device
    allocation inside the timed loop) of workload w after Wm untimed ones.

    Inputs are rotated over nsets buffers holding the same values, so that a
    workload smaller than the 256 MB last-level cache does not find its inputs
    there on the next step.  The step time comes from K steps with no
    instrumentation; a second pass of K steps with four events per step,
    re-recorded around the library's kernels (each event is one more packet
    between two dependent kernels), gives the per-kernel times, and the
    sweep's time divides the algorithmic bytes for the roofline record.
    uploaded: what upload_fwd returned, so the host-to-device copies need not
    sit between measurements."""
    import torch
    import log_linear_attention_attn_amd as ll
    sets, out = uploaded if uploaded is not None else upload_fwd(w, dev, nsets)
    ws_bytes = ll.fwd_workspace_size(w.B, w.H, w.T, w.dk, w.dv, w.C, seg_log2)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def timed(input_sets, n_warm=Wm):
        def step(i, ev=None):
            q, k, v, la, lam = input_sets[i % len(input_sets)]
            ll.fwd_ex(q, k, v, la, lam, C=w.C, out=out, seg_log2=seg_log2, workspace=ws, phase_events=ev)

        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
        for s_ in evs:
            for e in s_:
                e.record()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(n_warm):
            step(i)
        torch.cuda.synchronize()
        # the step time: K steps as a caller runs them, no events between kernels
        t0 = time.perf_counter()
        start.record()
        for i in range(K):
            step(i)
        stop.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_step = start.elapsed_time(stop) / K
        # the per-kernel times: K more steps with the phase events
        for i in range(K):
            step(i, evs[i])
        torch.cuda.synchronize()
        phases = [[s_[j].elapsed_time(s_[j + 1]) for j in range(3)] for s_ in evs]
        return ms_step, wall, phases

    ms, wall, phases = timed(sets)
    seg_ms, node_ms, sweep_ms = (sum(p[j] for p in phases) / K for j in range(3))
    step_ms = sorted(sum(p) for p in phases)
    del sets

    flops = algorithmic_flops(w.B, w.H, w.T, w.dk, w.dv, w.C)
    in_bytes = 2 if w.dtype == "bf16" else 4
    abytes = algorithmic_bytes(w.B, w.H, w.T, w.dk, w.dv, w.L, in_bytes)
    if w.Hk:
        # q and k are read once per q/k head, not once per head
        abytes -= w.B * (w.H - w.Hk) * w.T * 2 * w.dk * in_bytes
    tflops = flops / (ms * 1e-3) / 1e12
    sweep_gbs = abytes / (sweep_ms * 1e-3) / 1e9
    step_gbs = abytes / (ms * 1e-3) / 1e9
    floor_ms = max(flops / (PEAK_BF16_TFLOPS * 1e12), abytes / (PEAK_HBM_GBS * 1e9)) * 1e3
    traffic = load_traffic(w.name)
    rec = {
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
                   "C": w.C, "L": w.L, "inputs": f"{w.dtype} q/k/v, fp32 log_a/lambda/out",
                   "decay": w.decay, "seed": w.seed, "qk_heads": w.qk_heads},
        "steps": K, "warmup": Wm,
        "ms_per_step": ms,
        "tokens_per_s": w.B * w.T / (ms * 1e-3),
        "head_tokens_per_s": w.B * w.H * w.T / (ms * 1e-3),
        "tflops": tflops,
        "frac_bf16_peak": tflops / PEAK_BF16_TFLOPS,
        "algorithmic_flops": flops,
        "algorithmic_bytes": abytes,
        "roofline_floor_ms": floor_ms,
        "frac_roofline_step": floor_ms / ms,
        "hbm_gbs_step": step_gbs,
        "kernels_ms": {"seg_state": seg_ms, "seg_node": node_ms, "fwd_sweep": sweep_ms},
        "median_ms_per_step": step_ms[len(step_ms) // 2],
        "wall_ms_per_step": wall / K * 1e3,
        "workspace_bytes": ws_bytes,
        "roofline": {
            "kernel": sweep_kernel(w),
            "bound": "hbm",
            "achieved": sweep_gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": sweep_gbs / PEAK_HBM_GBS,
            "traffic": traffic,
            "mfma_tflops": flops / (sweep_ms * 1e-3) / 1e12,
            "note": "achieved = algorithmic bytes of the whole forward / the sweep kernel's "
                    "event-timed duration; traffic = its rocprofv3 FETCH_SIZE + WRITE_SIZE "
                    "bytes per launch (calibrated on a plain copy), null when taken on other sources",
        },
        "source_hash": source_hash(),
    }
    return rec


def bwd_record(w, dev, K: int, Wm: int, base=None):
    """The backward of workload w timed like the forward (see bench_bwd)."""
    import numpy as np
    import torch
    import log_linear_attention_attn_amd as ll
    import workloads as W
    q, k, v, la, lam = [t.to(dev) for t in (base if base is not None else W.make_fwd_inputs(w))]
    out = ll.fwd(q, k, v, la, lam, C=w.C)
    dout = torch.from_numpy(np.random.default_rng(w.seed + 1).standard_normal(tuple(out.shape))
                            .astype(np.float32)).to(dev)
    for _ in range(Wm):
        ll.bwd(q, k, v, la, lam, out, dout, C=w.C)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(K):
        ll.bwd(q, k, v, la, lam, out, dout, C=w.C)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / K
    flops = algorithmic_flops_bwd(w.B, w.H, w.T, w.dk, w.dv, w.C)
    abytes = algorithmic_bytes_bwd(w.B, w.H, w.T, w.dk, w.dv, w.L, 2 if w.dtype == "bf16" else 4)
    tflops = flops / (ms * 1e-3) / 1e12
    bf16 = w.dtype == "bf16" and w.C == 64
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    return {
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv, "C": w.C,
                   "L": w.L, "inputs": f"{w.dtype} q/k/v, fp32 log_a/lambda/out/dout", "pass": "backward"},
        "steps": K, "warmup": Wm, "ms_per_step": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3),
        "tflops": tflops, "algorithmic_flops": flops, "algorithmic_bytes": abytes,
        "hbm_gbs_algorithmic": abytes / (ms * 1e-3) / 1e9,
        "roofline": {"kernel": ("whole backward (fp16 matrix cores: the dQ, dV and dK register-state sweeps "
                                "on power-of-two scaled fp16 operands, the in-chunk dlambda and v . dV inside "
                                "the dV sweep, one row pass for dlambda and dc)"
                                if bf16 else "whole backward (fp32 matrix-core arithmetic)"),
                     "bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": tflops / peak, "traffic": None},
    }


def gdn_algorithmic_flops(B, H, T, dk, dv, C=64):
    """Matrix-product flops of the chunkwise log-linear Gated DeltaNet forward,
    counted as dense products (no credit for the triangular shapes): per chunk
    K K^T and Q K^T (2 C^2 dk each), the WY rows and the transformed queries
    (2 C^2 dk each), the in-chunk coefficients (2 C^3) and the triangular solve
    (C^3 / 3); per chunk and 16-column slice summed over dv, the in-chunk
    output and Tb V (2 C^2 dv each), the chunk's own state (2 C dk dv) and, per
    live bucket level, its output, W S and carried state (3 x 2 C dk dv)."""
    N = (T + C - 1) // C
    live = sum(bin(n).count("1") for n in range(N))
    per_chunk = 8 * C * C * dk + 2 * C ** 3 + C ** 3 / 3 + 4 * C * C * dv + 2 * C * dk * dv
    return B * H * (N * per_chunk + live * 6 * C * dk * dv)


def gdn_record(dev, K: int, Wm: int):
    """Log-linear Gated DeltaNet forward (loglinear_gdn_fwd: the chunk
    preparation and level sweep kernels, caller-owned workspace) at
    B=2 H=16 T=16384 dk=dv=128, timed over K calls after Wm untimed ones."""
    import torch
    import log_linear_attention_attn_amd as ll
    import workloads as W
    w = W.GDN_LM_T16K
    q, k, v, la, beta, lam = [t.to(dev) for t in W.make_gdn_inputs(w)]
    out = torch.empty(w.B, w.H, w.T, w.dv, dtype=torch.float32, device=dev)
    ws = torch.empty(ll.gdn_workspace_size(w.B, w.H, w.T, w.dk, w.dv), dtype=torch.uint8, device=dev)
    for _ in range(Wm):
        ll.gdn_fwd(q, k, v, la, beta, lam, out=out, workspace=ws)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(K):
        ll.gdn_fwd(q, k, v, la, beta, lam, out=out, workspace=ws)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / K
    flops = gdn_algorithmic_flops(w.B, w.H, w.T, w.dk, w.dv)
    tflops = flops / (ms * 1e-3) / 1e12
    return {
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv, "C": 64,
                   "L": w.L, "inputs": f"{w.dtype} q/k/v, fp32 log_alpha/beta/lambda/out", "decay": w.decay},
        "steps": K, "warmup": Wm, "ms_per_step": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3),
        "tflops": tflops, "algorithmic_flops": flops, "workspace_bytes": ws.numel(),
        "roofline": {"kernel": "whole call: chunk preparation + level sweep (fp32 matrix cores)",
                     "bound": "mfma", "achieved": tflops, "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / PEAK_FP32_TFLOPS, "traffic": None},
    }


def bench_prefill(sets, w, steps: int, warmup: int):
    """Forward plus the decode states at T-1 (loglinear_prefill) on the same
    inputs: the extra cost over the forward is the state emit of the last
    segment and the in-chunk handoff kernel."""
    import torch
    import log_linear_attention_attn_amd as ll
    dev = sets[0][0].device
    states = torch.empty(w.B, w.H, w.L, w.dk, w.dv, dtype=torch.float32, device=dev)
    out = torch.empty(w.B, w.H, w.T, w.dv, dtype=torch.float32, device=dev)
    for i in range(warmup):
        ll.prefill(*sets[i % len(sets)], C=w.C, out=out, states=states)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        ll.prefill(*sets[i % len(sets)], C=w.C, out=out, states=states)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    return {"ms_per_step": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3),
            "states_bytes": states.numel() * 4, "L": w.L}


def source_hash() -> str:
    from log_linear_attention_attn_amd.profiling import source_hash as h
    return h()


def load_traffic(workload: str):
    """HBM traffic per sweep launch from committed rocprofv3 --pmc summaries,
    or None when they are missing or were taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"fwd_sweep_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def calibrate_copy(mib: int):
    """A plain device-to-device copy of a known size, for scaling the
    FETCH_SIZE / WRITE_SIZE counters (run under rocprofv3 --pmc)."""
    import torch
    n = mib * 1024 * 1024
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 3}))


def cpu_baseline(w, budget_s: float = 12.0):
    """The CPU oracle (fp64 NumPy, dense O(T^2)) on whole (b, h) head-sequences
    of the same workload until ~budget_s of work; rate in the metric's unit."""
    import numpy as np
    import oracle
    import workloads as W
    threads, blas = 0, "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([i.get("num_threads", 0) for i in info] or [0])
        blas = ",".join(sorted({f"{i.get('internal_api')}:{i.get('version')}" for i in info
                                if i.get("user_api") == "blas"})) or blas
    except Exception:
        pass
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu)
    except OSError:
        pass
    q, k, v, la, lam = W.make_fwd_inputs(w)
    done, t0 = 0, time.perf_counter()
    while True:
        b, h = divmod(done, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        g = h // (w.H // w.qk_heads)  # the q/k head this head reads
        qs = (slice(b, b + 1), slice(g, g + 1))
        oracle.forward(q[qs], k[qs], v[sl], la[sl], lam[sl])
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s or done >= w.B * w.H:
            break
    tokens = done * w.T / w.H   # one token = one position of one batch row, all H heads
    return {
        "value": tokens / el, "unit": "tokens/s", "cores": threads or len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"oracle.forward (fp64 NumPy, dense masked QK^T V) on {done} of {w.B * w.H} (b,h) "
                  f"head-sequences of T={w.T}, {el:.1f} s; rate = {done}*T/H tokens / time",
        "seconds_per_head_sequence": el / done,
        "full_config_seconds_extrapolated": el / done * w.B * w.H,
        "cpu": cpu,
        "blas": blas,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first: the GPU clocks take ~0.1 s of load to reach steady state")
    ap.add_argument("--workload", default="lm_B2H16_T16384_dk128_dv128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline forward (no other configs, backward, prefill, "
                         "decode or projection objects)")
    ap.add_argument("--seg-log2", type=int, default=-1)
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd", "decode", "lambda", "gdn"], default="fwd",
                    help="time the forward (default, the headline; its line also carries one "
                         "decode and one lambda-projection measurement), the backward, or only the "
                         "decode step or the lambda projection")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import log_linear_attention_attn_amd as ll
    import workloads as W

    w = W.FWD_WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.which == "bwd":
        bench_bwd(args, w, dev)
        return
    if args.which == "lambda":
        rec = bench_lambda(dev, args.steps, args.warmup)
        print(json.dumps({
            "metric": "lambda projection GB/s (algorithmic HBM bytes / time)", "value": rec["roofline"]["achieved"],
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": rec["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": rec["dtype"], "data": "synthetic",
            "config": {k: rec[k] for k in ("workload", "B", "T", "D", "H", "L")},
            "roofline": rec["roofline"], "tflops": rec["tflops"], "bwd": rec["bwd"]}))
        return
    if args.which == "gdn":
        rec = gdn_record(dev, args.steps, args.warmup)
        print(json.dumps({
            "metric": "log-linear Gated DeltaNet fwd tokens/sec", "value": rec["tokens_per_s"],
            "unit": "tokens/s", "n_gpus": 1, "steps": rec["steps"], "warmup": rec["warmup"],
            "ms_per_step": rec["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic", "config": rec["config"],
            "roofline": rec["roofline"], "tflops": rec["tflops"],
            "algorithmic_flops": rec["algorithmic_flops"],
            "decode": bench_gdn_decode(dev, args.steps, args.warmup)}))
        return
    if args.which == "decode":
        rec = bench_decode(dev, args.steps, args.warmup)
        gbs = rec["roofline"]["achieved"]
        print(json.dumps({
            "metric": "decode step GB/s (algorithmic HBM bytes / time), 64 sequences x 16 heads, L=17",
            "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": rec["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": rec["workload"], "N": rec["N"], "H": rec["H"], "dk": rec["dk"],
                       "dv": rec["dv"], "L": rec["L"], "t": rec["t"]},
            "roofline": rec["roofline"], "tokens_per_s": rec["tokens_per_s"],
            "algorithmic_bytes": rec["algorithmic_bytes"]}))
        return
    K, Wm = args.steps, args.warmup
    # the backward and the other configs first: they are part of the line, and
    # they bring the GPU clocks to steady state before the headline is timed
    # (all inputs are drawn and uploaded first, so the GPU does not idle
    # between the measurements)
    extra = {}
    base = W.make_fwd_inputs(w)
    full = args.workload == W.LM_T16K.name and not args.headline_only
    aux = [(x, upload_fwd(x, dev, 3 if x is W.MAMBA2_T2K else 1)) for x in (W.MAMBA2_T2K, W.LONG_T64K)] if full else []
    head = upload_fwd(w, dev, 3, base)
    if full:
        aux_w = max(Wm, 20)
        extra["bwd"] = bwd_record(w, dev, max(3, K // 4), 3, base=base)
        extra["configs"] = {x.name: bench_fwd(x, dev, K, aux_w, uploaded=xu) for x, xu in aux}
    del aux
    rec_f = bench_fwd(w, dev, K, Wm, args.seg_log2, uploaded=head)
    sets, out = head
    del head
    rec = {
        "metric": METRIC,
        "value": rec_f["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": rec_f["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": rec_f["config"],
    }
    rec.update({k: v for k, v in rec_f.items() if k not in ("config", "ms_per_step", "tokens_per_s")})
    rec.update(extra)
    if full:
        rec["prefill"] = bench_prefill(sets, w, K, Wm)
        rec["decode"] = bench_decode(dev, K, Wm)
        rec["lambda_proj"] = bench_lambda(dev, K, Wm)
        rec["gdn"] = gdn_record(dev, max(3, K // 4), 3)
        rec["gdn"]["decode"] = bench_gdn_decode(dev, K, Wm)
        # the same shapes with log_a = 0 (no decay), timed last so its launches
        # do not sit among the headline's in a trace: the instruction stream is
        # the same, only the data (and with it the power draw) differs
        zero = [[q, k, v, torch.zeros_like(la), lam] for q, k, v, la, lam in sets]
        rz = bench_fwd(w, dev, K, max(Wm, 20), args.seg_log2, uploaded=(zero, out))
        rec["no_decay"] = {"ms_per_step": rz["ms_per_step"], "kernels_ms": rz["kernels_ms"],
                           "note": "log_a = 0, other inputs as the headline"}
        del zero
    del sets
    rec["pages_context"] = PAGES_CONTEXT
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec))


def bench_bwd(args, w, dev):
    """Backward (loglinear_bwd) of the same workload: gradients of sum(out * dout)
    for a random dout; inputs and out resident in HBM, timed over K steps."""
    r = bwd_record(w, dev, args.steps, args.warmup)
    rec = {
        "metric": "bwd tokens/sec (gradients of q, k, v, log_a, lambda), log-linear Mamba-2",
        "value": r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": r["steps"],
        "warmup": r["warmup"], "ms_per_step": r["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": r["config"],
    }
    rec.update({k: v for k, v in r.items() if k not in rec and k != "tokens_per_s"})
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
