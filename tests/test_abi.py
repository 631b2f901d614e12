"""Host-side checks of the C ABI: the library loads, exports every symbol that
include/loglinear.h declares, and rejects bad arguments before touching the
GPU (so these run on a machine without one)."""
import ctypes
import os
import re

import pytest

import log_linear_attention_attn_amd as ll

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "loglinear.h")

LL_OK, LL_ERR_NULL, LL_ERR_SHAPE, LL_ERR_UNSUPPORTED, LL_ERR_HIP, LL_ERR_WORKSPACE = 0, -1, -2, -3, -4, -5

pytestmark = pytest.mark.skipif(not os.path.exists(ll.library_path()),
                                reason="libloglinear.so not built (run __graft_entry__.build())")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(loglinear_\w+)\s*\(", text)))


def test_header_declarations_all_exported():
    declared = _declared_functions()
    assert set(declared) == set(ll.EXPORTED_SYMBOLS)
    L = ll.lib()
    for name in declared:
        assert hasattr(L, name), name


def test_num_levels():
    for T, L in [(0, 0), (1, 1), (2, 2), (3, 3), (64, 7), (65, 8), (2048, 12), (16384, 15), (65536, 17)]:
        assert ll.num_levels(T) == L


def _fwd(B=1, H=1, T=64, dk=16, dv=16, C=16, ptr=1, f=None):
    L = ll.lib()
    p = ctypes.c_void_p(ptr) if ptr else ctypes.c_void_p(0)
    fn = f or L.loglinear_fwd
    return fn(p, p, p, p, p, p, B, H, T, dk, dv, C, ctypes.c_void_p(0))


def test_fwd_argument_errors():
    assert _fwd(C=48) == LL_ERR_SHAPE          # not a power of two
    assert _fwd(C=128) == LL_ERR_UNSUPPORTED   # power of two without a kernel
    assert _fwd(C=0) == LL_ERR_SHAPE
    assert _fwd(dk=8) == LL_ERR_SHAPE
    assert _fwd(dk=24) == LL_ERR_SHAPE
    assert _fwd(dk=256) == LL_ERR_UNSUPPORTED
    assert _fwd(dv=0) == LL_ERR_SHAPE
    assert _fwd(dv=2048) == LL_ERR_UNSUPPORTED
    assert _fwd(B=-1) == LL_ERR_SHAPE
    assert _fwd(T=-5) == LL_ERR_SHAPE
    assert _fwd(ptr=0) == LL_ERR_NULL
    assert _fwd(ptr=0, f=ll.lib().loglinear_fwd_f32) == LL_ERR_NULL


def test_fwd_empty_is_noop():
    # zero-sized problems succeed without touching (NULL) pointers or the GPU
    assert _fwd(B=0, ptr=0) == LL_OK
    assert _fwd(H=0, ptr=0) == LL_OK
    assert _fwd(T=0, ptr=0) == LL_OK


def test_fwd_ex_options():
    L = ll.lib()
    p = ctypes.c_void_p(1)
    assert L.loglinear_fwd_ex(p, p, p, p, p, p, 1, 1, 64, 16, 16, 16, None, None) == LL_ERR_NULL
    bad = ll._FwdOpts(7, -1, 0, None, 0, None)
    assert L.loglinear_fwd_ex(p, p, p, p, p, p, 1, 1, 64, 16, 16, 16, ctypes.byref(bad), None) == LL_ERR_SHAPE
    bad = ll._FwdOpts(0, 13, 0, None, 0, None)
    assert L.loglinear_fwd_ex(p, p, p, p, p, p, 1, 1, 64, 16, 16, 16, ctypes.byref(bad), None) == LL_ERR_SHAPE
    # a caller workspace smaller than required is rejected before any launch
    need = ll.fwd_workspace_size(1, 1, 4096, 64, 64, 64, 1)
    assert need > 0
    small = ll._FwdOpts(0, 1, 0, ctypes.c_void_p(256), need - 1, None)
    assert L.loglinear_fwd_ex(p, p, p, p, p, p, 1, 1, 4096, 64, 64, 64, ctypes.byref(small), None) == LL_ERR_WORKSPACE
    # kernel selection: out-of-range value, and the register-state kernel on sizes it does not cover
    bad = ll._FwdOpts(0, -1, 4, None, 0, None)
    assert L.loglinear_fwd_ex(p, p, p, p, p, p, 1, 1, 64, 16, 16, 16, ctypes.byref(bad), None) == LL_ERR_SHAPE
    # the full-width kernel: dv = 128, C = 64, 64 < dk <= 128, bf16, its segment sizes only
    wide = ll._FwdOpts(0, -1, 3, None, 0, None)
    assert L.loglinear_fwd_ex(p, p, p, p, p, p, 1, 1, 64, 16, 16, 16, ctypes.byref(wide), None) == LL_ERR_UNSUPPORTED
    assert L.loglinear_fwd_ex(p, p, p, p, p, p, 1, 1, 4096, 128, 64, 64, ctypes.byref(wide), None) == LL_ERR_UNSUPPORTED
    wide2 = ll._FwdOpts(0, 2, 3, None, 0, None)
    assert L.loglinear_fwd_ex(p, p, p, p, p, p, 1, 1, 4096, 128, 128, 64, ctypes.byref(wide2), None) == LL_ERR_UNSUPPORTED
    widef = ll._FwdOpts(1, -1, 3, None, 0, None)
    assert L.loglinear_fwd_ex(p, p, p, p, p, p, 1, 1, 4096, 128, 128, 64, ctypes.byref(widef), None) == LL_ERR_UNSUPPORTED
    rs = ll._FwdOpts(0, -1, 2, None, 0, None)
    assert L.loglinear_fwd_ex(p, p, p, p, p, p, 1, 1, 64, 16, 16, 16, ctypes.byref(rs), None) == LL_ERR_UNSUPPORTED
    assert L.loglinear_fwd_ex(p, p, p, p, p, p, 1, 1, 64, 128, 48, 64, ctypes.byref(rs), None) == LL_ERR_UNSUPPORTED
    f32 = ll._FwdOpts(1, -1, 2, None, 0, None)
    assert L.loglinear_fwd_ex(p, p, p, p, p, p, 1, 1, 64, 128, 64, 64, ctypes.byref(f32), None) == LL_ERR_UNSUPPORTED


def test_workspace_size_formula():
    # one segment -> no scratch
    assert ll.fwd_workspace_size(1, 1, 64, 16, 16, 16, 4) == 0
    def a256(x):
        return -(-x // 256) * 256

    # B=2,H=16,T=16384,dk=dv=128,C=64, 16-chunk segments: 16 segments; the
    # state kernel already has 32 * 15 * 2 = 960 >= 512 workgroups, so the
    # state blocks are the segments (15 used + 1 slot)
    BH, nseg, dv, dkp = 32, 16, 128, 128
    st = BH * dv * dkp * 4
    assert ll.fwd_workspace_size(2, 16, 16384, 128, 128, 64, 4) == (
        st * 16 + st * nseg + a256(BH * nseg * 4) + a256(BH * 16 * 4))
    # 64-chunk segments: 4 segments, 32 * 3 * 2 = 192 workgroups -> blocks of
    # 16 chunks (768 workgroups): 12 blocks + 1 slot
    nseg, nblk1 = 4, 13
    assert ll.fwd_workspace_size(2, 16, 16384, 128, 128, 64, 6) == (
        st * nblk1 + st * nseg + a256(BH * nseg * 4) + a256(BH * nblk1 * 4))
    with pytest.raises(ValueError):
        ll.fwd_workspace_size(1, 1, 64, 10, 16, 16)


def test_decode_argument_errors():
    L = ll.lib()
    p = ctypes.c_void_p(1)
    assert L.loglinear_decode_step(None, p, p, p, p, p, p, p, None) == LL_ERR_NULL
    for N, H, Lv, dk, dv, want in [
        (1, 1, 0, 16, 16, LL_ERR_SHAPE), (1, 1, 32, 16, 16, LL_ERR_SHAPE),
        (1, 1, 4, 6, 16, LL_ERR_SHAPE), (1, 1, 4, 16, 2, LL_ERR_SHAPE),
        (-1, 1, 4, 16, 16, LL_ERR_SHAPE), (1, 1, 4, 2048, 16, LL_ERR_UNSUPPORTED),
        (0, 4, 4, 16, 16, LL_OK), (1, 1, 4, 16, 16, LL_ERR_NULL),
    ]:
        desc = ll._States(0, N, H, Lv, dk, dv)
        assert L.loglinear_decode_step(ctypes.byref(desc), p, p, p, p, p, p, p, None) == want, (N, H, Lv, dk, dv)


def test_level_table_argument_errors():
    L = ll.lib()
    assert L.loglinear_level_table(ctypes.c_void_p(1), 0, None) == LL_ERR_SHAPE
    assert L.loglinear_level_table(ctypes.c_void_p(1), 9000, None) == LL_ERR_SHAPE
    assert L.loglinear_level_table(None, 16, None) == LL_ERR_NULL


def test_strerror():
    for s in (LL_OK, LL_ERR_NULL, LL_ERR_SHAPE, LL_ERR_UNSUPPORTED, LL_ERR_HIP, LL_ERR_WORKSPACE):
        assert ll.strerror(s) and ll.strerror(s) != "unknown status"
    assert ll.strerror(42) == "unknown status"


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 16, 16)
    lam = torch.zeros(1, 1, 16, ll.num_levels(16))
    with pytest.raises(ValueError):
        ll.fwd(q, q, q, torch.zeros(1, 1, 16), lam, C=16)


def test_prefill_argument_errors():
    """States buffers that do not match the forward are rejected before any
    GPU work; a zero-sized problem is a no-op."""
    L = ll.lib()
    p = ctypes.c_void_p(1)
    B, H, T, dk, dv, C = 2, 3, 100, 32, 16, 16  # num_levels(100) = 8
    assert L.loglinear_prefill(p, p, p, p, p, p, None, B, H, T, dk, dv, C, None) == LL_ERR_NULL
    for N_, H_, Lv, dk_, dv_, want in [
        (1, 3, 8, 32, 16, LL_ERR_SHAPE),    # N != B
        (2, 2, 8, 32, 16, LL_ERR_SHAPE),    # H differs
        (2, 3, 7, 32, 16, LL_ERR_SHAPE),    # fewer levels than T needs
        (2, 3, 32, 32, 16, LL_ERR_SHAPE),   # more than 31 levels
        (2, 3, 8, 16, 16, LL_ERR_SHAPE),    # dk differs
        (2, 3, 8, 32, 32, LL_ERR_SHAPE),    # dv differs
        (2, 3, 8, 32, 16, LL_ERR_NULL),     # shapes fine, NULL data
    ]:
        desc = ll._States(0, N_, H_, Lv, dk_, dv_)
        for f in (L.loglinear_prefill, L.loglinear_prefill_f32):
            assert f(p, p, p, p, p, p, ctypes.byref(desc), B, H, T, dk, dv, C, None) == want, (N_, H_, Lv, dk_, dv_)
    desc = ll._States(0, 0, H, 8, dk, dv)
    assert L.loglinear_prefill(p, p, p, p, p, p, ctypes.byref(desc), 0, H, T, dk, dv, C, None) == LL_OK
    # the same checks through loglinear_fwd_ex's final_states option
    bad = ll._States(0, 1, H, 8, dk, dv)
    opts = ll._FwdOpts(0, -1, 0, None, 0, None, ctypes.pointer(bad))
    assert L.loglinear_fwd_ex(p, p, p, p, p, p, B, H, T, dk, dv, C, ctypes.byref(opts), None) == LL_ERR_SHAPE


def test_bwd_argument_errors():
    L = ll.lib()
    p = ctypes.c_void_p(1)
    args = [p] * 12
    assert L.loglinear_bwd(*args, 1, 1, 64, 16, 16, 48, None) == LL_ERR_SHAPE       # C not a power of two
    assert L.loglinear_bwd(*args, 1, 1, 64, 24, 16, 16, None) == LL_ERR_SHAPE       # dk not a multiple of 16
    assert L.loglinear_bwd(*args, 1, 1, 16 * 5000, 16, 16, 16, None) == LL_ERR_UNSUPPORTED  # > 4096 chunks
    assert L.loglinear_bwd(*([ctypes.c_void_p(0)] + args[1:]), 1, 1, 64, 16, 16, 16, None) == LL_ERR_NULL
    assert L.loglinear_bwd(*[ctypes.c_void_p(0)] * 12, 0, 1, 64, 16, 16, 16, None) == LL_OK  # empty: no-op
    assert L.loglinear_bwd_f32(*args, 1, 1, 64, 16, 16, 48, None) == LL_ERR_SHAPE


def test_qk_heads_must_divide_heads():
    """qk_heads that do not divide H are rejected before any GPU work."""
    L = ll.lib()
    p = ctypes.c_void_p(1)
    bad = ll._FwdOpts(0, -1, 0, None, 0, None, None, 3)
    assert L.loglinear_fwd_ex(p, p, p, p, p, p, 1, 4, 64, 16, 16, 16, ctypes.byref(bad), None) == LL_ERR_SHAPE
    neg = ll._FwdOpts(0, -1, 0, None, 0, None, None, -2)
    assert L.loglinear_fwd_ex(p, p, p, p, p, p, 1, 4, 64, 16, 16, 16, ctypes.byref(neg), None) == LL_ERR_SHAPE
    assert L.loglinear_bwd_ex(*([p] * 12), 1, 4, 64, 16, 16, 16, 0, 3, None) == LL_ERR_SHAPE
    assert L.loglinear_bwd_ex(*([p] * 12), 1, 4, 64, 16, 16, 16, 7, 2, None) == LL_ERR_SHAPE  # dtype
    desc = ll._States(1, 2, 4, 8, 16, 16)
    assert L.loglinear_decode_step_ex(ctypes.byref(desc), p, p, p, p, p, p, p, 0, 3, None) == LL_ERR_SHAPE
    assert L.loglinear_decode_step_ex(ctypes.byref(desc), p, p, p, p, p, p, p, 5, 2, None) == LL_ERR_SHAPE


def test_lambda_proj_argument_errors():
    L = ll.lib()
    p = ctypes.c_void_p(16)
    assert L.loglinear_lambda_proj(p, p, None, p, 1, 4, 16, 2, 3, 2, None) == LL_ERR_SHAPE      # dtype
    assert L.loglinear_lambda_proj(p, p, None, p, 1, 4, 12, 2, 3, 0, None) == LL_ERR_SHAPE      # D % 8 (bf16)
    assert L.loglinear_lambda_proj(p, p, None, p, 1, 4, 16, 2, 0, 0, None) == LL_ERR_SHAPE      # L
    assert L.loglinear_lambda_proj(p, p, None, p, 1, 4, 16, 2, 32, 0, None) == LL_ERR_SHAPE     # L > 31
    assert L.loglinear_lambda_proj(p, p, None, p, 0, 4, 16, 2, 3, 0, None) == LL_OK            # empty
    assert L.loglinear_lambda_proj(None, p, None, p, 1, 4, 16, 2, 3, 0, None) == LL_ERR_NULL
    q = ctypes.c_void_p(18)  # not 16-byte aligned
    assert L.loglinear_lambda_proj(q, p, None, p, 1, 4, 16, 2, 3, 0, None) == LL_ERR_SHAPE


def test_lambda_proj_bwd_argument_errors():
    L = ll.lib()
    p = ctypes.c_void_p(16)
    args = [p] * 7
    assert L.loglinear_lambda_proj_bwd(*args, 1, 4, 16, 2, 3, 2, None) == LL_ERR_SHAPE       # dtype
    assert L.loglinear_lambda_proj_bwd(*args, 1, 4, 16, 2, 0, 0, None) == LL_ERR_SHAPE       # L
    assert L.loglinear_lambda_proj_bwd(*args, 1, 4, 16, 2, 32, 0, None) == LL_ERR_SHAPE      # L > 31
    assert L.loglinear_lambda_proj_bwd(*args, 1, 4, 0, 2, 3, 0, None) == LL_ERR_SHAPE        # D
    assert L.loglinear_lambda_proj_bwd(*args, 1, 4, 16, 4096, 31, 0, None) == LL_ERR_UNSUPPORTED  # H*L
    assert L.loglinear_lambda_proj_bwd(*args, 1 << 16, 1 << 16, 16, 2, 3, 0, None) == LL_ERR_UNSUPPORTED
    assert L.loglinear_lambda_proj_bwd(p, p, p, p, None, p, p, 1, 4, 16, 2, 3, 0, None) == LL_ERR_NULL
    assert L.loglinear_lambda_proj_bwd(p, None, p, p, p, p, p, 0, 4, 16, 2, 3, 0, None) == LL_ERR_NULL



def test_misaligned_pointers_are_rejected():
    """Pointers the kernels access with 16-byte vectors must be 16-byte
    aligned; any other is LL_ERR_SHAPE, returned on the host before any GPU work."""
    L = ll.lib()
    good, bad = ctypes.c_void_p(256), ctypes.c_void_p(258)
    # forward: q, ..., out (one misaligned at a time); log_a may be anywhere
    fwd_args = [good] * 6
    for i in (0, 1, 2, 4, 5):
        a = list(fwd_args)
        a[i] = bad
        assert L.loglinear_fwd(*a, 1, 1, 64, 16, 16, 16, None) == LL_ERR_SHAPE, i
    # backward: q, k, v, log_a, lambda, out, dout, grads
    bwd_args = [good] * 12
    for i in (0, 2, 6, 7, 9, 11):
        a = list(bwd_args)
        a[i] = bad
        assert L.loglinear_bwd(*a, 1, 1, 64, 16, 16, 16, None) == LL_ERR_SHAPE, i
    # decode: the state buffer and out (q, k, v are read one element at a time)
    desc = ll._States(258, 1, 1, 4, 16, 16)
    assert L.loglinear_decode_step(ctypes.byref(desc), good, good, good, good, good, good, good, None) == LL_ERR_SHAPE
    desc = ll._States(256, 1, 1, 4, 16, 16)
    assert L.loglinear_decode_step(ctypes.byref(desc), good, good, good, good, good, good, bad, None) == LL_ERR_SHAPE
    # a caller workspace must be 256-byte aligned
    opts = ll._FwdOpts(ll.LL_BF16, 2, 0, ctypes.c_void_p(256 + 16), 1 << 30, None, None, 0)
    assert L.loglinear_fwd_ex(*fwd_args, 1, 1, 4096, 128, 64, 64, ctypes.byref(opts), None) == -5


def test_fwd_noalloc_rejects_sizes_beyond_its_scratch():
    """loglinear_fwd_noalloc checks its workspace against the static scratch
    on the host, before any HIP call: a plan that needs more is
    LL_ERR_WORKSPACE, argument errors are reported as for loglinear_fwd."""
    L = ll.lib()
    p = ctypes.c_void_p(256)
    fn = L.loglinear_fwd_noalloc
    # B=H=1, T=65536, dk=128, dv=1024, C=16: the automatic plan needs 256 MiB
    assert ll.fwd_workspace_size(1, 1, 65536, 128, 1024, 16, -1) > ll.NOALLOC_SCRATCH_BYTES
    assert fn(p, p, p, p, p, p, 1, 1, 65536, 128, 1024, 16, None) == LL_ERR_WORKSPACE
    # the bench shapes fit
    assert ll.fwd_workspace_size(2, 16, 16384, 128, 128, 64, -1) <= ll.NOALLOC_SCRATCH_BYTES
    assert ll.fwd_workspace_size(1, 16, 65536, 128, 128, 64, -1) <= ll.NOALLOC_SCRATCH_BYTES
    assert fn(p, p, p, p, p, p, 1, 1, 64, 16, 16, 48, None) == LL_ERR_SHAPE
    assert fn(None, p, p, p, p, p, 1, 1, 64, 16, 16, 16, None) == LL_ERR_NULL
    assert fn(p, p, p, p, p, p, 0, 1, 64, 16, 16, 16, None) == LL_OK


def test_gdn_argument_errors():
    """loglinear_gdn_fwd rejects bad sizes, pointers and workspaces on the host."""
    L = ll.lib()
    p = ctypes.c_void_p(1 << 20)   # 16-byte aligned, never dereferenced

    def call(B=1, H=1, T=64, dk=64, dv=16, dtype=0, ws=None, nbytes=0, ptr=p):
        return L.loglinear_gdn_fwd(ptr, p, p, p, p, p, p, B, H, T, dk, dv, dtype, ws, nbytes, None)

    assert call(dk=32) == LL_ERR_UNSUPPORTED
    assert call(dk=256) == LL_ERR_UNSUPPORTED
    assert call(dv=24) == LL_ERR_UNSUPPORTED
    assert call(dv=0) == LL_ERR_SHAPE
    assert call(B=-1) == LL_ERR_SHAPE
    assert call(dtype=7) == LL_ERR_SHAPE
    assert call(T=64 * 8193, dk=128) == LL_ERR_UNSUPPORTED   # 14 chunk-level bits: states exceed LDS
    assert call(ptr=None) == LL_ERR_NULL
    assert call(B=0, ptr=None) == LL_OK
    assert call(ptr=ctypes.c_void_p((1 << 20) + 8)) == LL_ERR_SHAPE
    need = L.loglinear_gdn_workspace_size(1, 1, 64, 64, 16)
    assert call(ws=p, nbytes=need - 1) == LL_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p((1 << 20) + 16), nbytes=need) == LL_ERR_WORKSPACE
    # 4 (3 dk + 128) * 64 bytes per chunk, plus one float per chunk (each part 256-byte aligned)
    for B, H, T, dk in [(1, 1, 64, 64), (2, 16, 16384, 128), (1, 2, 4200, 128)]:
        n = B * H * ((T + 63) // 64)
        want = ((n * 4 * (3 * dk + 128) * 64 + 255) // 256 + (n * 4 + 255) // 256) * 256
        assert L.loglinear_gdn_workspace_size(B, H, T, dk, 16) == want
    assert L.loglinear_gdn_workspace_size(1, 1, 64, 48, 16) == ctypes.c_size_t(-1).value


def test_gdn_decode_argument_errors():
    L = ll.lib()
    p = ctypes.c_void_p(1 << 20)

    def call(N=1, H=1, Lv=5, dk=64, dv=16, dtype=0, data=1 << 20, ptr=p):
        st = ll._States(data, N, H, Lv, dk, dv)
        return L.loglinear_gdn_decode_step(ctypes.byref(st), ptr, p, p, p, p, p, p, p, dtype, None)

    assert L.loglinear_gdn_decode_step(None, p, p, p, p, p, p, p, p, 0, None) == LL_ERR_NULL
    assert call(dk=32) == LL_ERR_UNSUPPORTED
    assert call(dk=6) == LL_ERR_SHAPE
    assert call(dv=2) == LL_ERR_SHAPE
    assert call(dv=2048) == LL_ERR_UNSUPPORTED
    assert call(Lv=0) == LL_ERR_SHAPE
    assert call(Lv=32) == LL_ERR_SHAPE
    assert call(N=-1) == LL_ERR_SHAPE
    assert call(dtype=3) == LL_ERR_SHAPE
    assert call(N=0, ptr=None) == LL_OK
    assert call(ptr=None) == LL_ERR_NULL
    assert call(data=(1 << 20) + 4) == LL_ERR_SHAPE


def test_gdn_prefill_argument_errors():
    L = ll.lib()
    p = ctypes.c_void_p(1 << 20)

    def call(states=p, Ls=7, T=64, B=1):
        return L.loglinear_gdn_prefill(p, p, p, p, p, p, p, states, Ls, B, 1, T, 64, 16, 0, None, 0, None)

    assert call(states=None) == LL_ERR_NULL
    assert call(Ls=6) == LL_ERR_SHAPE              # T = 64 has L = 7 levels
    assert call(Ls=32) == LL_ERR_SHAPE
    assert call(states=ctypes.c_void_p((1 << 20) + 4)) == LL_ERR_SHAPE
    assert call(states=None, B=0) == LL_OK
