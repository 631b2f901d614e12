"""Static check of the gfx950 assembly this package builds: find instructions
that read a matrix-core (MFMA) destination register fewer than MIN_WAIT wait
states after the MFMA along some control-flow path.

The hardware does not interlock a VALU / LDS / memory read of an MFMA result;
the compiler must separate them with independent instructions or s_nop.  One
build of this library produced such a read right after a branch (stale
accumulator lane, wrong chunk state), so every build is scanned.

    python -m log_linear_attention_attn_amd.isa_check   # exit 1 if any found
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

from . import build as _build

MIN_WAIT = 8  # the compiler's own separation after a 16x16x32 bf16 / f16 MFMA
# opcodes whose results need longer: the compiler's own straight-line
# separation (a 16x16x4 fp32 MFMA runs more passes)
MIN_WAIT_BY_OP = {"v_mfma_f32_16x16x4_f32": 10}


def _regs(tok: str) -> set:
    m = re.match(r"([av])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([av])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _functions(text: str) -> dict:
    funcs, cur = {}, None
    for line in text.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur = m.group(1)
            funcs[cur] = []
            continue
        if cur is not None:
            funcs[cur].append(line)
            if "s_endpgm" in line:
                cur = None
    return funcs


def _need(op: str, min_wait: int) -> int:
    return max(min_wait, MIN_WAIT_BY_OP.get(op, min_wait))


def scan(asm_text: str, min_wait: int = MIN_WAIT) -> list[str]:
    limit = max([min_wait] + list(MIN_WAIT_BY_OP.values()))
    found = []
    for fn, body in _functions(asm_text).items():
        ins, labels = [], {}
        for line in body:
            s = line.split(";")[0].strip()
            if not s:
                continue
            if s.endswith(":"):
                labels[s[:-1]] = len(ins)
                continue
            if s.startswith("."):
                continue
            parts = s.replace(",", " ").split()
            ins.append((parts[0], parts[1:], s))
        preds = {i: [] for i in range(len(ins))}
        for i, (op, args, _) in enumerate(ins):
            if i + 1 < len(ins) and op not in ("s_branch", "s_endpgm", "s_setpc_b64"):
                preds[i + 1].append(i)
            if (op.startswith("s_cbranch") or op == "s_branch") and args and args[0] in labels:
                if labels[args[0]] < len(ins):
                    preds[labels[args[0]]].append(i)
        for i, (op, args, s) in enumerate(ins):
            if "mfma" in op:
                continue
            srcs = set()
            for a in args[1:]:
                srcs |= _regs(a)
            if op.startswith(("ds_write", "global_store", "buffer_store")):
                for a in args:
                    srcs |= _regs(a)
            if not srcs:
                continue
            stack, seen = [(p, 0) for p in preds[i]], set()
            while stack:
                j, w = stack.pop()
                if (j, w) in seen or w >= limit:
                    continue
                seen.add((j, w))
                op2, args2, s2 = ins[j]
                if "mfma" in op2 and _regs(args2[0]) & srcs:
                    if w < _need(op2, min_wait):
                        found.append(f"{fn}: '{s}' reads the result of '{s2}' after {w} wait states")
                    continue
                step = int(args2[0], 0) + 1 if op2 == "s_nop" else 1
                for p in preds[j]:
                    stack.append((p, w + step))
    return found


def device_asm() -> str:
    """Compile every source for gfx950 to device assembly (not a library)."""
    out = []
    with tempfile.TemporaryDirectory() as td:
        for src in _build.SOURCES:
            if not src.endswith(".hip"):
                continue
            path = os.path.join(td, src + ".s")
            cmd = [c for c in _build.build_command(path) if c not in ("-shared", "-fPIC")]
            cmd = [c for c in cmd if not c.endswith((".hip", ".cpp"))]
            cmd += ["--cuda-device-only", "-S", os.path.join(_build.CSRC, src)]
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(res.stderr)
            with open(path) as f:
                out.append(f.read())
    return "\n".join(out)


if __name__ == "__main__":
    bad = scan(device_asm())
    for b in bad:
        print(b)
    print(f"{len(bad)} MFMA result read(s) with fewer wait states than required "
          f"({MIN_WAIT}, or per opcode {MIN_WAIT_BY_OP})")
    sys.exit(1 if bad else 0)
