"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import sys

import numpy as np
import torch

BF16_TOL = 2e-2   # max |gpu - oracle| <= BF16_TOL * RMS(oracle) for bf16 inputs
F32_TOL = 1e-4    # same bound for fp32 inputs


def have_gpu() -> bool:
    return torch.cuda.is_available()


def announce(msg: str):
    """Name the case about to run on the GPU (flushed, so a crash still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(*ts, device="cuda"):
    return [t.to(device).contiguous() for t in ts]


def rel_max_err(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    rms = float(np.sqrt(np.mean(want ** 2)))
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    return err / rms if rms > 0 else err


def assert_parity(got, want, tol, what=""):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    r = rel_max_err(got, want)
    print(f"  {what}: max|err|/RMS = {r:.3e} (tol {tol:.1e})", flush=True)
    assert r <= tol, f"{what}: max|err|/RMS = {r:.3e} > {tol:.1e}"
