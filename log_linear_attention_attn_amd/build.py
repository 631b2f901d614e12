"""Build libloglinear.so (HIP, gfx950) in-tree with hipcc.

    python -m log_linear_attention_attn_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libloglinear.so")
SOURCES = ["loglinear_fwd.hip", "loglinear_sweep_rs.hip", "loglinear_sweep_wide.hip", "loglinear_decode.hip", "loglinear_bwd.hip", "loglinear_bwd16.hip", "loglinear_bwd_rev.hip", "loglinear_lambda.hip",
           "loglinear_lambda_bwd.hip", "loglinear_noalloc.hip", "loglinear_gdn.hip",
           "loglinear_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def build_command(out: str = LIB, extra: list[str] | None = None) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-pass-failed",
        "-I", INCLUDE, "-I", CSRC,
        "-o", out,
        *[os.path.join(CSRC, s) for s in SOURCES],
        *(extra or []),
    ]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libloglinear.so; returns its path."""
    tmp = LIB + ".tmp"
    cmd = build_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
