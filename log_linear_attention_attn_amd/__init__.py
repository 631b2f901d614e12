"""Log-linear attention on MI355X (gfx950): thin ctypes binding of libloglinear.so.

Every step of the computation runs in the HIP kernels of libloglinear.so; this
module only checks tensor metadata, passes device pointers and the current HIP
stream, and turns status codes into exceptions.  There is no CPU fallback: if
the library is not built, every call raises.

Entry points (same names as the C ABI in include/loglinear.h):
    fwd(q, k, v, log_a, lam, C=64, out=None)            bf16 or fp32 q/k/v
    fwd_ex(..., seg_log2=-1, workspace=None)            explicit options
    prefill(q, k, v, log_a, lam, C=64, L=None)          forward + decode states at T-1
    bwd(q, k, v, log_a, lam, out, dout, C=64)           gradients of sum(out * dout)
    fwd_workspace_size(B, H, T, dk, dv, C, seg_log2=-1)
    gdn_fwd(q, k, v, log_alpha, beta, lam, out=None, workspace=None)   log-linear Gated DeltaNet
    gdn_workspace_size(B, H, T, dk, dv)
    gdn_decode_step(states, q, k, v, log_alpha, beta, lam, t, out=None)   its decode step
    gdn_prefill(q, k, v, log_alpha, beta, lam, L=None, workspace=None)     forward + states at T-1
    decode_step(states, q, k, v, log_a, lam, t, out=None)
    level_table(T, device=None)                          int8 [T, T]
    num_levels(T)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LogLinearError", "lib", "library_path", "num_levels", "fwd", "fwd_ex", "prefill", "bwd",
    "fwd_workspace_size", "decode_step", "level_table", "strerror", "gdn_fwd", "gdn_workspace_size",
    "gdn_decode_step", "gdn_prefill",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libloglinear.so")
_lib = None

LL_BF16, LL_F32 = 0, 1
EXPORTED_SYMBOLS = (
    "loglinear_num_levels", "loglinear_fwd", "loglinear_fwd_f32", "loglinear_fwd_ex",
    "loglinear_prefill", "loglinear_prefill_f32", "loglinear_bwd", "loglinear_bwd_f32",
    "loglinear_bwd_ex", "loglinear_fwd_workspace_size",
    "loglinear_decode_step", "loglinear_decode_step_f32", "loglinear_decode_step_ex",
    "loglinear_level_table", "loglinear_lambda_proj", "loglinear_lambda_proj_bwd",
    "loglinear_strerror", "loglinear_fwd_noalloc", "loglinear_gdn_fwd", "loglinear_gdn_workspace_size",
    "loglinear_gdn_decode_step", "loglinear_gdn_prefill",
)

# bytes of the static scratch behind loglinear_fwd_noalloc (the header's
# LOGLINEAR_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


class LogLinearError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({strerror(status)})")
        self.status = status


class _States(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("N", ctypes.c_int), ("H", ctypes.c_int),
                ("L", ctypes.c_int), ("dk", ctypes.c_int), ("dv", ctypes.c_int)]


class _FwdOpts(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("seg_log2", ctypes.c_int), ("kernel", ctypes.c_int),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("phase_events", ctypes.c_void_p), ("final_states", ctypes.POINTER(_States)),
                ("qk_heads", ctypes.c_int)]


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libloglinear.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m log_linear_attention_attn_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    fwd_args = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i]
    L.loglinear_num_levels.argtypes = [i]
    L.loglinear_num_levels.restype = i
    L.loglinear_fwd.argtypes = fwd_args + [vp]
    L.loglinear_fwd.restype = i
    L.loglinear_fwd_f32.argtypes = fwd_args + [vp]
    L.loglinear_fwd_f32.restype = i
    L.loglinear_fwd_ex.argtypes = fwd_args + [ctypes.POINTER(_FwdOpts), vp]
    L.loglinear_fwd_ex.restype = i
    L.loglinear_fwd_noalloc.argtypes = fwd_args + [vp]
    L.loglinear_fwd_noalloc.restype = i
    pre_args = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(_States), i, i, i, i, i, i, vp]
    L.loglinear_prefill.argtypes = pre_args
    L.loglinear_prefill.restype = i
    L.loglinear_prefill_f32.argtypes = pre_args
    L.loglinear_prefill_f32.restype = i
    bwd_args = [vp] * 12 + [i, i, i, i, i, i, vp]
    L.loglinear_bwd.argtypes = bwd_args
    L.loglinear_bwd.restype = i
    L.loglinear_bwd_f32.argtypes = bwd_args
    L.loglinear_bwd_f32.restype = i
    L.loglinear_bwd_ex.argtypes = bwd_args[:-1] + [i, i, vp]
    L.loglinear_bwd_ex.restype = i
    L.loglinear_fwd_workspace_size.argtypes = [i, i, i, i, i, i, i]
    L.loglinear_fwd_workspace_size.restype = sz
    dec_args = [ctypes.POINTER(_States), vp, vp, vp, vp, vp, vp, vp, vp]
    L.loglinear_decode_step.argtypes = dec_args
    L.loglinear_decode_step.restype = i
    L.loglinear_decode_step_f32.argtypes = dec_args
    L.loglinear_decode_step_f32.restype = i
    L.loglinear_decode_step_ex.argtypes = dec_args[:-1] + [i, i, vp]
    L.loglinear_decode_step_ex.restype = i
    L.loglinear_lambda_proj.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, vp]
    L.loglinear_lambda_proj.restype = i
    L.loglinear_lambda_proj_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
    L.loglinear_lambda_proj_bwd.restype = i
    L.loglinear_level_table.argtypes = [vp, i, vp]
    L.loglinear_level_table.restype = i
    L.loglinear_gdn_fwd.argtypes = [vp] * 7 + [i] * 6 + [vp, sz, vp]
    L.loglinear_gdn_fwd.restype = i
    L.loglinear_gdn_workspace_size.argtypes = [i] * 5
    L.loglinear_gdn_decode_step.argtypes = [ctypes.POINTER(_States)] + [vp] * 8 + [i, vp]
    L.loglinear_gdn_decode_step.restype = i
    L.loglinear_gdn_prefill.argtypes = [vp] * 8 + [i] * 7 + [vp, sz, vp]
    L.loglinear_gdn_prefill.restype = i
    L.loglinear_gdn_workspace_size.restype = sz
    L.loglinear_strerror.argtypes = [i]
    L.loglinear_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def strerror(status: int) -> str:
    try:
        return lib().loglinear_strerror(int(status)).decode()
    except Exception:  # library missing: still report the number
        return "unknown"


def num_levels(T: int) -> int:
    return int(lib().loglinear_num_levels(int(T)))


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else ctypes.c_void_p(0)


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_dev(name: str, t: torch.Tensor, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _raise(status: int, what: str):
    if status != 0:
        raise LogLinearError(status, what)


def _qk_heads(q, v) -> int:
    """qk_heads argument of the C ABI: 0 when every head has its own q / k,
    else the number of q / k heads (shared by groups of v heads, MVA)."""
    Hk, H = q.shape[1], v.shape[1]
    if Hk == H:
        return 0
    if Hk < 1 or H % Hk != 0:
        raise ValueError(f"q/k heads ({Hk}) must divide the heads of v ({H})")
    return Hk


def fwd_workspace_size(B, H, T, dk, dv, C, seg_log2=-1) -> int:
    n = lib().loglinear_fwd_workspace_size(B, H, T, dk, dv, C, seg_log2)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes")
    return int(n)


KERNEL_AUTO, KERNEL_LDS_STATE, KERNEL_REGISTER_STATE, KERNEL_WIDE = 0, 1, 2, 3


def fwd_ex(q, k, v, log_a, lam, C: int = 64, out=None, seg_log2: int = -1, workspace=None,
           phase_events=None, kernel: int = KERNEL_AUTO, final_states=None):
    """Log-linear attention forward through loglinear_fwd_ex.

    q, k: [B, Hk, T, dk]; v: [B, H, T, dv] (all bf16 or all fp32), Hk = H or
    a divisor of H (q / k shared by H / Hk heads each, MVA);
    log_a: [B, H, T] fp32; lam: [B, H, T, L] fp32 with L = num_levels(T).
    phase_events: None or 4 recorded torch.cuda.Event(enable_timing=True)
    objects, re-recorded before / between / after the library's kernels.
    final_states: None or an fp32 [B, H, Ls, dk, dv] tensor that receives the
    decode states at position T-1 (see prefill).
    Returns out [B, H, T, dv] fp32 (allocated unless given).
    """
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q, k, v must be bfloat16 or float32")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    B, Hk, T, dk = q.shape
    H, dv = v.shape[1], v.shape[-1]
    qk_heads = _qk_heads(q, v)
    L = num_levels(T) if T > 0 else 0
    _check_dev("q", q, q.dtype, (B, Hk, T, dk), dev)
    _check_dev("k", k, q.dtype, (B, Hk, T, dk), dev)
    _check_dev("v", v, q.dtype, (B, H, T, dv), dev)
    _check_dev("log_a", log_a, torch.float32, (B, H, T), dev)
    _check_dev("lam", lam, torch.float32, (B, H, T, L), dev)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
    _check_dev("out", out, torch.float32, (B, H, T, dv), dev)
    ev = None
    if phase_events is not None:
        if len(phase_events) != 4:
            raise ValueError("phase_events needs 4 events")
        ev = (ctypes.c_void_p * 4)(*[e.cuda_event for e in phase_events])
        if not all(ev):
            raise ValueError("record each phase event once before passing it")
    fin = None
    if final_states is not None:
        if final_states.dim() != 5:
            raise ValueError("final_states must be [B, H, Ls, dk, dv]")
        _check_dev("final_states", final_states, torch.float32, (B, H, final_states.shape[2], dk, dv), dev)
        fin = _States(final_states.data_ptr(), B, H, final_states.shape[2], dk, dv)
    opts = _FwdOpts(LL_BF16 if q.dtype == torch.bfloat16 else LL_F32, int(seg_log2), int(kernel),
                    _ptr(workspace), workspace.numel() * workspace.element_size() if workspace is not None else 0,
                    ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None,
                    ctypes.pointer(fin) if fin is not None else None, qk_heads)
    st = lib().loglinear_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(lam), _ptr(out),
                                B, H, T, dk, dv, int(C), ctypes.byref(opts), _stream(dev))
    _raise(st, "loglinear_fwd_ex")
    return out


def fwd(q, k, v, log_a, lam, C: int = 64, out=None):
    """Log-linear attention forward (loglinear_fwd for bf16, loglinear_fwd_f32 for
    fp32; q / k shared across heads go through loglinear_fwd_ex)."""
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q, k, v must be bfloat16 or float32")
    if q.dim() == 4 and v.dim() == 4 and q.shape[1] != v.shape[1]:
        return fwd_ex(q, k, v, log_a, lam, C=C, out=out)
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = num_levels(T) if T > 0 else 0
    _check_dev("q", q, q.dtype, (B, H, T, dk), dev)
    _check_dev("k", k, q.dtype, (B, H, T, dk), dev)
    _check_dev("v", v, q.dtype, (B, H, T, dv), dev)
    _check_dev("log_a", log_a, torch.float32, (B, H, T), dev)
    _check_dev("lam", lam, torch.float32, (B, H, T, L), dev)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
    _check_dev("out", out, torch.float32, (B, H, T, dv), dev)
    f = lib().loglinear_fwd if q.dtype == torch.bfloat16 else lib().loglinear_fwd_f32
    st = f(_ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(lam), _ptr(out), B, H, T, dk, dv, int(C),
           _stream(dev))
    _raise(st, "loglinear_fwd")
    return out


def fwd_noalloc(q, k, v, log_a, lam, C: int = 64, out=None):
    """loglinear_fwd_noalloc: the bf16 forward with its workspace in the
    library's static device scratch (no allocation inside the call; calls that
    overlap on one GPU race).  Same result as fwd.  `out` is allocated here
    unless given, so a caller that must not allocate passes it."""
    if q.dtype != torch.bfloat16:
        raise TypeError("q, k, v must be bfloat16")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = num_levels(T) if T > 0 else 0
    _check_dev("q", q, q.dtype, (B, H, T, dk), dev)
    _check_dev("k", k, q.dtype, (B, H, T, dk), dev)
    _check_dev("v", v, q.dtype, (B, H, T, dv), dev)
    _check_dev("log_a", log_a, torch.float32, (B, H, T), dev)
    _check_dev("lam", lam, torch.float32, (B, H, T, L), dev)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
    _check_dev("out", out, torch.float32, (B, H, T, dv), dev)
    st = lib().loglinear_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(lam), _ptr(out),
                                     B, H, T, dk, dv, int(C), _stream(dev))
    _raise(st, "loglinear_fwd_noalloc")
    return out


def prefill(q, k, v, log_a, lam, C: int = 64, L: int | None = None, out=None, states=None):
    """Forward plus the per-level decode states at position T-1
    (loglinear_prefill / loglinear_prefill_f32).

    Returns (out [B, H, T, dv] fp32, states [B, H, L, dk, dv] fp32); L defaults
    to num_levels(T) and may be larger so decoding can continue past 2^(L-1).
    q / k shared across heads go through loglinear_fwd_ex's final_states.
    """
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q, k, v must be bfloat16 or float32")
    if q.dim() == 4 and v.dim() == 4 and q.shape[1] != v.shape[1]:
        B, _, T, dk = q.shape
        H, dv = v.shape[1], v.shape[-1]
        Ls = int(L) if L is not None else max(num_levels(T) if T > 0 else 0, 1)
        if states is None:
            states = torch.empty((B, H, Ls, dk, dv), dtype=torch.float32, device=q.device)
        out = fwd_ex(q, k, v, log_a, lam, C=C, out=out, final_states=states)
        return out, states
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    Lf = num_levels(T) if T > 0 else 0
    _check_dev("q", q, q.dtype, (B, H, T, dk), dev)
    _check_dev("k", k, q.dtype, (B, H, T, dk), dev)
    _check_dev("v", v, q.dtype, (B, H, T, dv), dev)
    _check_dev("log_a", log_a, torch.float32, (B, H, T), dev)
    _check_dev("lam", lam, torch.float32, (B, H, T, Lf), dev)
    Ls = int(L) if L is not None else max(Lf, 1)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
    _check_dev("out", out, torch.float32, (B, H, T, dv), dev)
    if states is None:
        states = torch.empty((B, H, Ls, dk, dv), dtype=torch.float32, device=dev)
    _check_dev("states", states, torch.float32, (B, H, Ls, dk, dv), dev)
    desc = _States(states.data_ptr(), B, H, Ls, dk, dv)
    f = lib().loglinear_prefill if q.dtype == torch.bfloat16 else lib().loglinear_prefill_f32
    st = f(_ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(lam), _ptr(out), ctypes.byref(desc),
           B, H, T, dk, dv, int(C), _stream(dev))
    _raise(st, "loglinear_prefill")
    return out, states


def bwd(q, k, v, log_a, lam, out, dout, C: int = 64):
    """Gradients of sum(out * dout) with respect to q, k, v, log_a and lam
    (loglinear_bwd / loglinear_bwd_f32); out is the forward's output.

    Returns (dq, dk, dv, dlog_a, dlam), all fp32, shaped like the inputs.  With
    q / k shared across heads (MVA) dq and dk are summed over each group
    (loglinear_bwd_ex).
    """
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q, k, v must be bfloat16 or float32")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    B, Hk, T, dk = q.shape
    H, dv = v.shape[1], v.shape[-1]
    qk_heads = _qk_heads(q, v)
    L = num_levels(T) if T > 0 else 0
    _check_dev("q", q, q.dtype, (B, Hk, T, dk), dev)
    _check_dev("k", k, q.dtype, (B, Hk, T, dk), dev)
    _check_dev("v", v, q.dtype, (B, H, T, dv), dev)
    _check_dev("log_a", log_a, torch.float32, (B, H, T), dev)
    _check_dev("lam", lam, torch.float32, (B, H, T, L), dev)
    _check_dev("out", out, torch.float32, (B, H, T, dv), dev)
    _check_dev("dout", dout, torch.float32, (B, H, T, dv), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    gq, gk = torch.empty((B, Hk, T, dk), **f32), torch.empty((B, Hk, T, dk), **f32)
    gv = torch.empty((B, H, T, dv), **f32)
    gla, glam = torch.empty((B, H, T), **f32), torch.empty((B, H, T, L), **f32)
    ptrs = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(lam), _ptr(out), _ptr(dout), _ptr(gq), _ptr(gk),
            _ptr(gv), _ptr(gla), _ptr(glam), B, H, T, dk, dv, int(C))
    if qk_heads:
        st = lib().loglinear_bwd_ex(*ptrs, LL_BF16 if q.dtype == torch.bfloat16 else LL_F32, qk_heads,
                                    _stream(dev))
    else:
        f = lib().loglinear_bwd if q.dtype == torch.bfloat16 else lib().loglinear_bwd_f32
        st = f(*ptrs, _stream(dev))
    _raise(st, "loglinear_bwd")
    return gq, gk, gv, gla, glam


def decode_step(states, q, k, v, log_a, lam, t, out=None):
    """One decode step; updates ``states`` [N, H, L, dk, dv] fp32 in place.

    q, k: [N, Hk, dk] with Hk = H or a divisor of H (shared by H / Hk heads
    each, MVA); v: [N, H, dv] (bf16 or fp32); log_a: [N, H] fp32;
    lam: [N, H, L] fp32; t: [N] int32.  Returns out [N, H, dv] fp32.
    """
    dev = states.device
    if dev.type != "cuda":
        raise ValueError("states must be on a GPU device")
    N, H, L, dk, dv = states.shape
    _check_dev("states", states, torch.float32, (N, H, L, dk, dv), dev)
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q, k, v must be bfloat16 or float32")
    Hk = q.shape[1] if q.dim() == 3 else H
    if Hk < 1 or H % Hk != 0:
        raise ValueError(f"q/k heads ({Hk}) must divide the heads of the states ({H})")
    _check_dev("q", q, q.dtype, (N, Hk, dk), dev)
    _check_dev("k", k, q.dtype, (N, Hk, dk), dev)
    _check_dev("v", v, q.dtype, (N, H, dv), dev)
    _check_dev("log_a", log_a, torch.float32, (N, H), dev)
    _check_dev("lam", lam, torch.float32, (N, H, L), dev)
    _check_dev("t", t, torch.int32, (N,), dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    _check_dev("out", out, torch.float32, (N, H, dv), dev)
    desc = _States(states.data_ptr(), N, H, L, dk, dv)
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(lam), _ptr(t), _ptr(out))
    if Hk != H:
        st = lib().loglinear_decode_step_ex(*args, LL_BF16 if q.dtype == torch.bfloat16 else LL_F32, Hk,
                                            _stream(dev))
    else:
        f = lib().loglinear_decode_step if q.dtype == torch.bfloat16 else lib().loglinear_decode_step_f32
        st = f(*args, _stream(dev))
    _raise(st, "loglinear_decode_step")
    return out


def lambda_proj(x, W, bias, H: int, L: int, out=None):
    """Level weights from the hidden state (loglinear_lambda_proj):
    lambda[b, h, t, l] = softplus(x[b, t] . W[h*L + l] + bias[h*L + l]).

    x: [B, T, D] and W: [H*L, D], both bf16 or both fp32; bias: [H*L] fp32 or
    None.  Returns lambda [B, H, T, L] fp32 (allocated unless given).
    """
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("x, W must be bfloat16 or float32")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    B, T, D = x.shape
    _check_dev("x", x, x.dtype, (B, T, D), dev)
    _check_dev("W", W, x.dtype, (H * L, D), dev)
    if bias is not None:
        _check_dev("bias", bias, torch.float32, (H * L,), dev)
    if out is None:
        out = torch.empty((B, H, T, L), dtype=torch.float32, device=dev)
    _check_dev("out", out, torch.float32, (B, H, T, L), dev)
    st = lib().loglinear_lambda_proj(_ptr(x), _ptr(W), _ptr(bias), _ptr(out), B, T, D, int(H), int(L),
                                     LL_BF16 if x.dtype == torch.bfloat16 else LL_F32, _stream(dev))
    _raise(st, "loglinear_lambda_proj")
    return out


def lambda_proj_bwd(x, W, lam, dlam, want_bias: bool = True):
    """Gradient of lambda_proj (loglinear_lambda_proj_bwd): from the forward's
    lambda [B, H, T, L] and the incoming dlambda (both fp32), returns
    (dx [B, T, D], dW [H*L, D], dbias [H*L] or None), all fp32.
    x: [B, T, D] and W: [H*L, D] as for lambda_proj."""
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("x, W must be bfloat16 or float32")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    B, T, D = x.shape
    if lam.dim() != 4:
        raise ValueError("lambda must be [B, H, T, L]")
    H, L = int(lam.shape[1]), int(lam.shape[3])
    _check_dev("x", x, x.dtype, (B, T, D), dev)
    _check_dev("W", W, x.dtype, (H * L, D), dev)
    _check_dev("lambda", lam, torch.float32, (B, H, T, L), dev)
    _check_dev("dlambda", dlam, torch.float32, (B, H, T, L), dev)
    dx = torch.empty((B, T, D), dtype=torch.float32, device=dev)
    dW = torch.empty((H * L, D), dtype=torch.float32, device=dev)
    db = torch.empty((H * L,), dtype=torch.float32, device=dev) if want_bias else None
    st = lib().loglinear_lambda_proj_bwd(_ptr(x), _ptr(W), _ptr(lam), _ptr(dlam), _ptr(dx), _ptr(dW), _ptr(db),
                                         B, T, D, H, L, LL_BF16 if x.dtype == torch.bfloat16 else LL_F32,
                                         _stream(dev))
    _raise(st, "loglinear_lambda_proj_bwd")
    return dx, dW, db


def level_table(T: int, device=None):
    """GPU-computed level table (int8 [T, T], -1 above the diagonal)."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    lev = torch.empty((T, T), dtype=torch.int8, device=dev)
    _raise(lib().loglinear_level_table(_ptr(lev), int(T), _stream(dev)), "loglinear_level_table")
    return lev


def gdn_workspace_size(B, H, T, dk, dv) -> int:
    n = lib().loglinear_gdn_workspace_size(B, H, T, dk, dv)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid or unsupported sizes")
    return int(n)


def gdn_fwd(q, k, v, log_alpha, beta, lam, out=None, workspace=None):
    """Log-linear Gated DeltaNet forward through loglinear_gdn_fwd.

    q, k: [B, H, T, dk]; v: [B, H, T, dv] (all bf16 or all fp32);
    log_alpha, beta: [B, H, T] fp32; lam: [B, H, T, L] fp32, L = num_levels(T).
    workspace: None (the library allocates) or a uint8 device tensor of at
    least gdn_workspace_size(...) bytes.  Returns out [B, H, T, dv] fp32.
    """
    out = _gdn_check(q, k, v, log_alpha, beta, lam, out)
    return _gdn_call(q, k, v, log_alpha, beta, lam, out, workspace, None)


def gdn_prefill(q, k, v, log_alpha, beta, lam, L=None, workspace=None, out=None):
    """loglinear_gdn_prefill: the Gated DeltaNet forward plus the decode
    states at T-1, [B, H, L, dk, dv] fp32 with L = num_levels(T) unless given
    (more levels are written as 0).  Returns (out, states)."""
    out = _gdn_check(q, k, v, log_alpha, beta, lam, out)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    Ls = int(L) if L is not None else num_levels(T)
    states = torch.empty((B, H, Ls, dk, dv), dtype=torch.float32, device=q.device)
    _gdn_call(q, k, v, log_alpha, beta, lam, out, workspace, states)
    return out, states


def _gdn_check(q, k, v, log_alpha, beta, lam, out):
    """Metadata checks of the Gated DeltaNet calls; returns out (allocated unless given)."""
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q, k, v must be bfloat16 or float32")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = num_levels(T) if T > 0 else 0
    _check_dev("q", q, q.dtype, (B, H, T, dk), dev)
    _check_dev("k", k, q.dtype, (B, H, T, dk), dev)
    _check_dev("v", v, q.dtype, (B, H, T, dv), dev)
    _check_dev("log_alpha", log_alpha, torch.float32, (B, H, T), dev)
    _check_dev("beta", beta, torch.float32, (B, H, T), dev)
    _check_dev("lam", lam, torch.float32, (B, H, T, L), dev)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
    _check_dev("out", out, torch.float32, (B, H, T, dv), dev)
    return out


def _gdn_call(q, k, v, log_alpha, beta, lam, out, workspace, states):
    dev = q.device
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    dtype = LL_BF16 if q.dtype == torch.bfloat16 else LL_F32
    if states is not None:
        st = lib().loglinear_gdn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(lam),
                                         _ptr(out), _ptr(states), states.shape[2], B, H, T, dk, dv, dtype,
                                         _ptr(workspace), nbytes, _stream(dev))
        _raise(st, "loglinear_gdn_prefill")
        return out
    st = lib().loglinear_gdn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(lam),
                                 _ptr(out), B, H, T, dk, dv,
                                 LL_BF16 if q.dtype == torch.bfloat16 else LL_F32,
                                 _ptr(workspace), nbytes, _stream(dev))
    _raise(st, "loglinear_gdn_fwd")
    return out


def gdn_decode_step(states, q, k, v, log_alpha, beta, lam, t, out=None):
    """One log-linear Gated DeltaNet decode step (loglinear_gdn_decode_step);
    updates ``states`` [N, H, L, dk, dv] fp32 in place.

    q, k: [N, H, dk]; v: [N, H, dv] (bf16 or fp32); log_alpha, beta: [N, H]
    fp32; lam: [N, H, L] fp32; t: [N] int32.  Returns out [N, H, dv] fp32.
    """
    dev = states.device
    if dev.type != "cuda":
        raise ValueError("states must be on a GPU device")
    N, H, L, dk, dv = states.shape
    _check_dev("states", states, torch.float32, (N, H, L, dk, dv), dev)
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q, k, v must be bfloat16 or float32")
    _check_dev("q", q, q.dtype, (N, H, dk), dev)
    _check_dev("k", k, q.dtype, (N, H, dk), dev)
    _check_dev("v", v, q.dtype, (N, H, dv), dev)
    _check_dev("log_alpha", log_alpha, torch.float32, (N, H), dev)
    _check_dev("beta", beta, torch.float32, (N, H), dev)
    _check_dev("lam", lam, torch.float32, (N, H, L), dev)
    _check_dev("t", t, torch.int32, (N,), dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    _check_dev("out", out, torch.float32, (N, H, dv), dev)
    desc = _States(states.data_ptr(), N, H, L, dk, dv)
    st = lib().loglinear_gdn_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                         _ptr(beta), _ptr(lam), _ptr(t), _ptr(out),
                                         LL_BF16 if q.dtype == torch.bfloat16 else LL_F32, _stream(dev))
    _raise(st, "loglinear_gdn_decode_step")
    return out
