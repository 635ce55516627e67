"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_03_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "gdn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.lib_path()):
        pytest.fail("libgdn.so is not built (run __graft_entry__.build())")
    return gdn.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(gdn.EXPORTS)
    raw = ctypes.CDLL(gdn.lib_path())
    for n in names:
        assert hasattr(raw, n), n


def test_version_and_status_strings(lib):
    assert gdn.version() >= 100
    for code in range(5):
        assert gdn.status_string(code)
    assert "unknown" in gdn.status_string(99)


def test_workspace_query(lib):
    # one entry per (chunk slot, value head).  Staged path (bf16, d_k = 128,
    # d_v a multiple of 32): T's non-zero bf16 fragments (four whole, two
    # half) + gamma, s, g: 5,888 bytes.  Chained path (every other one-pass
    # problem): M and P in fp32, C x C each, + a 256-float gate block.
    staged = 5 * 1024 + 768
    chained = lambda c: (2 * c * c + 256) * 4
    w = gdn.chunk_fwd_workspace_bytes(4, 4096, 16, 16, 128, 128, gdn.GDN_BF16, 64, 0)
    assert 4 * 64 * 16 * staged <= w < 4 * 64 * 16 * staged + 4096
    packed = gdn.chunk_fwd_workspace_bytes(1, 1000, 2, 4, 128, 128, gdn.GDN_BF16, 64, 5)
    assert (16 + 5) * 4 * staged <= packed < (16 + 5) * 4 * staged + 4096
    general = gdn.chunk_fwd_workspace_bytes(1, 1000, 2, 4, 64, 128, gdn.GDN_BF16, 64, 5)
    assert (16 + 5) * 4 * chained(64) <= general < (16 + 5) * 4 * chained(64) + 4096
    f32 = gdn.chunk_fwd_workspace_bytes(1, 64, 1, 1, 16, 16, gdn.GDN_F32, 16, 0)
    assert 4 * chained(16) <= f32 < 4 * chained(16) + 4096
    assert gdn.chunk_fwd_workspace_bytes(1, 64, 1, 1, 48, 64, gdn.GDN_BF16, 64, 0) == 0
    assert gdn.chunk_fwd_workspace_bytes(1, 64, 1, 1, 64, 64, gdn.GDN_BF16, 48, 0) == 0
    assert gdn.chunk_fwd_workspace_bytes(1, 64, 1, 1, 64, 64, 7, 64, 0) == 0


def fwd(lib, fn, B=1, T=8, H_qk=1, H_v=1, d_k=64, d_v=64, dtype=0, ptrs=True, cu=None, n=0,
        extra=()):
    p = ctypes.c_void_p(0x1000) if ptrs else None
    args = [B, T, H_qk, H_v, d_k, d_v, dtype, p, p, p, p, p, cu, n, None, p, None]
    return getattr(lib, fn)(*args, *extra)


@pytest.mark.parametrize("fn,extra", [("gdn_recurrent_fwd", (None,)),
                                      ("gdn_kda_recurrent_fwd", (None,)),
                                      ("gdn_chunk_fwd", (64, None, 0, None)),
                                      ("gdn_kda_chunk_fwd", (64, None, 0, None)),
                                      ("gdn_chunk_fwd_noalloc", (64, None))])
def test_argument_errors_are_reported_before_launch(lib, fn, extra):
    # every case below fails validation, so no kernel is launched
    assert fwd(lib, fn, d_k=48, extra=extra) == 2
    assert fwd(lib, fn, d_v=256, extra=extra) == 2
    assert fwd(lib, fn, dtype=5, extra=extra) == 2
    assert fwd(lib, fn, H_qk=3, H_v=4, extra=extra) == 2
    assert fwd(lib, fn, B=-1, extra=extra) == 1
    assert fwd(lib, fn, ptrs=False, extra=extra) == 1
    assert fwd(lib, fn, B=2, cu=ctypes.c_void_p(0x1000), n=2, extra=extra) == 1
    assert fwd(lib, fn, B=2, n=3, extra=extra) == 1
    # a packed batch with tokens but no sequence
    assert fwd(lib, fn, B=1, T=8, cu=ctypes.c_void_p(0x1000), n=0, extra=extra) == 1
    # more than 2^31 - 1 tokens (token and chunk indices are 32-bit in the kernels)
    assert fwd(lib, fn, B=2, T=(1 << 30) + 1, d_k=16, d_v=16, extra=extra) == 2
    # a tensor that does not start on a 16-byte boundary
    args = [1, 8, 1, 1, 64, 64, 0] + [ctypes.c_void_p(0x1000)] * 5 + [None, 0, None, ctypes.c_void_p(0x1008), None]
    assert getattr(lib, fn)(*args, *extra) == 1


def test_chunk_workspace_errors(lib):
    p = ctypes.c_void_p(0x1000)
    args = [1, 8, 1, 1, 64, 64, 0, p, p, p, p, p, None, 0, None, p, None]
    assert lib.gdn_chunk_fwd(*args, 48, p, 1 << 30, None) == 2   # unsupported chunk
    assert lib.gdn_chunk_fwd(*args, 64, None, 1 << 30, None) == 3  # no workspace
    assert lib.gdn_chunk_fwd(*args, 64, p, 16, None) == 3          # too small
    assert lib.gdn_chunk_fwd(*args, 64, ctypes.c_void_p(0x1001), 1 << 30, None) == 3  # misaligned


def test_decode_argument_errors(lib):
    p = ctypes.c_void_p(0x1000)
    assert lib.gdn_decode_step(1, 1, 1, 48, 64, 0, p, p, p, p, p, p, p, None) == 2
    assert lib.gdn_decode_step(1, 1, 1, 64, 64, 0, p, p, p, p, p, None, p, None) == 1
    assert lib.gdn_decode_step(1, 2, 3, 64, 64, 0, p, p, p, p, p, p, p, None) == 2
    assert lib.gdn_decode_step(1, 1, 1, 64, 64, 0, p, p, p, p, p, ctypes.c_void_p(0x1008), p, None) == 1
    for fn in (lib.gdn_decode_step, lib.gdn_kda_decode_step):
        assert fn(1, 1, 1, 48, 64, 0, p, p, p, p, p, p, p, None) == 2
        assert fn(1, 2, 3, 64, 64, 0, p, p, p, p, p, p, p, None) == 2
    # the per-channel rates are read 16 bytes at a time
    assert lib.gdn_kda_decode_step(1, 1, 1, 64, 64, 0, p, p, p, ctypes.c_void_p(0x1004), p, p, p, None) == 1
    args = [1, 8, 1, 1, 64, 64, 0, p, p, p, ctypes.c_void_p(0x1004), p, None, 0, None, p, None, None]
    assert lib.gdn_kda_recurrent_fwd(*args) == 1


def prologue(lib, B=1, T=8, H_qk=1, H_v=1, d_k=64, d_v=64, dtype=0, ptrs=True, cu=None, n=0, eps=1e-6,
             q_scale=1.0):
    p = ctypes.c_void_p(0x1000) if ptrs else None
    return lib.gdn_block_prologue(B, T, H_qk, H_v, d_k, d_v, dtype, p, p, p, p, p, p, None, None, None, p, p, p,
                                  None, eps, q_scale, cu, n, p, p, p, p, p, None)


def test_block_argument_errors(lib):
    p = ctypes.c_void_p(0x1000)
    assert prologue(lib, d_k=48) == 2
    assert prologue(lib, H_qk=3, H_v=4) == 2
    assert prologue(lib, dtype=5) == 2
    assert prologue(lib, ptrs=False) == 1
    assert prologue(lib, eps=-1.0) == 1
    assert prologue(lib, eps=float("nan")) == 1
    assert prologue(lib, q_scale=float("inf")) == 1
    assert prologue(lib, B=2, cu=p, n=2) == 1      # a packed batch has B == 1
    assert prologue(lib, cu=p, n=0) == 1           # ... and at least one sequence
    # the grid bound (one wave per 16 tokens and head at most): 2^17 x 3 * 2^15 exceeds 32 bits
    assert prologue(lib, B=1, T=1 << 21, H_qk=1 << 15, H_v=1 << 15, d_k=16, d_v=16) == 2
    # a token's row of one tensor must stay below 2^24 bytes: 2^15 heads x 128 x 4 bytes = 2^24
    assert prologue(lib, B=1, T=8, H_qk=1 << 15, H_v=1 << 15, d_k=128, d_v=128) == 2
    assert lib.gdn_block_epilogue(1, 8, 1, 48, 0, p, p, None, 1e-6, p, None) == 2
    assert lib.gdn_block_epilogue(1, 8, 1, 64, 0, p, None, None, 1e-6, p, None) == 1
    assert lib.gdn_block_epilogue(1, 8, 1, 64, 0, p, p, None, -1.0, p, None) == 1
    assert lib.gdn_block_epilogue(1, 8, 1, 64, 0, p, ctypes.c_void_p(0x1004), None, 1e-6, p, None) == 1
    q = ctypes.c_void_p(0x1002)
    assert lib.gdn_block_prologue(1, 8, 1, 1, 64, 64, 0, p, q, p, p, p, p, None, None, None, p, p, p,
                                  None, 1e-6, 1.0, None, 0, p, p, p, p, p, None) == 1
    assert lib.gdn_block_epilogue(0, 8, 1, 64, 0, None, None, None, 1e-6, None, None) == 0  # nothing to do


def _gpu_present():
    """True wherever a GPU could be reached: a kernel driver device node
    exists, or torch sees a device.  The test below must never launch on a
    real GPU, whatever torch reports."""
    if os.path.exists("/dev/kfd") or os.path.exists("/dev/dri"):
        return True
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu_present(), reason="drives launches with placeholder pointers: hosts without a GPU only")
def test_host_path_reaches_launch_without_gpu(lib):
    """Valid arguments run the host-side geometry and launch sequencing; with no
    GPU present the launch fails and is reported as GDN_ERROR_LAUNCH (4).
    Regression: the token-by-token path once divided by its (zero) chunk size."""
    p = ctypes.c_void_p(0x1000)
    base = [1, 8, 1, 1, 64, 64, 0, p, p, p, p, p, None, 0, None, p, None]
    assert lib.gdn_recurrent_fwd(*base, None) == 4
    ws = ctypes.c_void_p(0x100000)
    assert lib.gdn_chunk_fwd(*base, 64, ws, 1 << 30, None) == 4
    assert lib.gdn_chunk_fwd_segmented(*base, 64, 0, ws, 1 << 30, None) == 4
    assert lib.gdn_chunk_fwd_segmented(*base, 64, 1, ws, 1 << 30, None) == 4
    assert lib.gdn_decode_step(2, 1, 1, 64, 64, 1, p, p, p, p, p, p, p, None) == 4
    assert lib.gdn_kda_recurrent_fwd(*base, None) == 4
    assert lib.gdn_kda_chunk_fwd(*base, 64, ws, 1 << 30, None) == 4
    grads = [p, None, p, p, p, p, p, None]  # d_o, dhT, dq, dk, dv, dalpha, dbeta, dh0
    assert lib.gdn_chunk_bwd(*base[:15], *grads, 64, ws, 1 << 30, None) == 4
    assert lib.gdn_chunk_fwd_noalloc(*base, 64, None) == 4   # no device: the scratch has no address
    assert lib.gdn_kda_decode_step(2, 1, 1, 64, 64, 1, p, p, p, p, p, p, p, None) == 4
    assert prologue(lib) == 4
    assert lib.gdn_block_epilogue(1, 8, 1, 64, 0, p, p, None, 1e-6, p, None) == 4


def test_segment_plan_and_workspace(lib):
    bf = gdn.GDN_BF16
    # a full batch runs in one pass; a few long units are cut into segments
    assert gdn.chunk_fwd_plan_segments(4, 4096, 16, 16, 128, 128, bf, 64, 0) == 0
    assert gdn.chunk_fwd_plan_segments(1, 65536, 16, 16, 128, 128, bf, 64, 0) == 128
    seg = gdn.chunk_fwd_plan_segments(1, 65536, 2, 2, 128, 128, bf, 64, 0)
    assert seg == 64
    assert gdn.chunk_fwd_plan_segments(1, 4096, 1, 1, 128, 128, bf, 64, 0) == 0   # too short to cut
    assert gdn.chunk_fwd_plan_segments(1, 8192, 1, 1, 128, 128, bf, 64, 0) == 64
    assert lib.gdn_chunk_fwd_plan_segments(1, 64, 1, 1, 48, 64, bf, 64, 0) == -1
    # gdn_chunk_fwd's query covers the planned form
    one = gdn.chunk_fwd_segmented_workspace_bytes(1, 65536, 2, 2, 128, 128, bf, 64, 0, 0)
    planned = gdn.chunk_fwd_segmented_workspace_bytes(1, 65536, 2, 2, 128, 128, bf, 64, 0, seg)
    assert gdn.chunk_fwd_workspace_bytes(1, 65536, 2, 2, 128, 128, bf, 64, 0) == planned
    nseg = 1024 // seg + (1024 % seg > 0)
    # + segment offsets, maps [seg, H, 128, 256] and entry states [seg, H, 128, 128] in fp32
    assert planned >= one + nseg * 2 * 128 * (256 + 128) * 4
    assert gdn.chunk_fwd_workspace_bytes(4, 4096, 16, 16, 128, 128, bf, 64, 0) == \
        gdn.chunk_fwd_segmented_workspace_bytes(4, 4096, 16, 16, 128, 128, bf, 64, 0, 0)
    # packed: a bound for every cu_seqlens with these totals
    packed = gdn.chunk_fwd_segmented_workspace_bytes(1, 1000, 2, 4, 64, 32, gdn.GDN_F32, 32, 5, 2)
    assert packed > gdn.chunk_fwd_segmented_workspace_bytes(1, 1000, 2, 4, 64, 32, gdn.GDN_F32, 32, 5, 0)
    assert gdn.chunk_fwd_segmented_workspace_bytes(1, 1000, 2, 4, 64, 32, gdn.GDN_F32, 32, 5, -1) == 0


def test_segmented_argument_errors(lib):
    p = ctypes.c_void_p(0x1000)
    base = [1, 8, 1, 1, 64, 64, 0, p, p, p, p, p, None, 0, None, p, None]
    assert lib.gdn_chunk_fwd_segmented(*base, 64, -1, p, 1 << 30, None) == 1   # negative length
    assert lib.gdn_chunk_fwd_segmented(*base, 48, 2, p, 1 << 30, None) == 2    # unsupported chunk
    assert lib.gdn_chunk_fwd_segmented(*base, 64, 2, None, 1 << 30, None) == 3  # no workspace
    assert lib.gdn_chunk_fwd_segmented(*base, 64, 2, p, 64, None) == 3          # too small
    # a segment longer than 2^31 - 1 tokens
    assert lib.gdn_chunk_fwd_segmented(*base, 64, 1 << 26, p, 1 << 30, None) == 2
    bad = list(base)
    bad[2] = 3
    bad[3] = 4
    assert lib.gdn_chunk_fwd_segmented(*bad, 64, 2, p, 1 << 30, None) == 2      # H_v not a multiple of H_qk


def test_kda_chunk_workspace(lib):
    bf = gdn.GDN_BF16
    # one entry per (chunk slot, value head): 64 fragments of 512 operand-type
    # elements (T, P, Khat, Qhat, Ktil^T) + 128 fp32 decay factors
    entry = 64 * 512 * 2 + 512
    w = gdn.kda_chunk_fwd_workspace_bytes(4, 4096, 16, 16, 128, 128, bf, 64, 0)
    assert 4 * 64 * 16 * entry <= w < 4 * 64 * 16 * entry + 4096
    f32 = gdn.kda_chunk_fwd_workspace_bytes(1, 100, 1, 2, 32, 32, gdn.GDN_F32, 32, 0)
    assert f32 >= 4 * 2 * (64 * 512 * 4 + 512)
    assert gdn.kda_chunk_fwd_workspace_bytes(1, 64, 1, 1, 48, 64, bf, 64, 0) == 0
    p = ctypes.c_void_p(0x1000)
    args = [1, 8, 1, 1, 64, 64, 0, p, p, p, p, p, None, 0, None, p, None]
    assert lib.gdn_kda_chunk_fwd(*args, 48, p, 1 << 30, None) == 2
    assert lib.gdn_kda_chunk_fwd(*args, 64, None, 1 << 30, None) == 3
    assert lib.gdn_kda_chunk_fwd(*args, 64, p, 64, None) == 3
    misaligned = list(args)
    misaligned[10] = ctypes.c_void_p(0x1004)                    # alpha (read 16 bytes at a time)
    assert lib.gdn_kda_chunk_fwd(*misaligned, 64, p, 1 << 30, None) == 1


def test_noalloc_argument_errors(lib):
    p = ctypes.c_void_p(0x1000)
    base = [1, 8, 1, 1, 64, 64, 0, p, p, p, p, p, None, 0, None, p, None]
    assert lib.gdn_chunk_fwd_noalloc(*base, 48, None) == 2          # unsupported chunk
    # a problem whose scratch exceeds the 32 MiB array: rejected before any launch
    big = [8, 4096, 16, 16, 128, 128, 1, p, p, p, p, p, None, 0, None, p, None]
    assert gdn.chunk_fwd_workspace_bytes(8, 4096, 16, 16, 128, 128, 1, 64, 0) > (32 << 20)
    assert lib.gdn_chunk_fwd_noalloc(*big, 64, None) == 3


def test_backward_workspace_and_argument_errors(lib):
    """gdn_chunk_bwd: workspace sizes and argument errors, all before any launch."""
    bf, f32 = gdn.GDN_BF16, gdn.GDN_F32
    # one fp32 entry per (chunk slot, value head): M, P and Gamma . K K^T
    # (C x C each), 256 gate values, the chunk's start state and end gradient
    # (d_k x d_v each), U and dY (C x d_v each)
    def entry(C, dk, dv):
        return 4 * (3 * C * C + 256 + 2 * dk * dv + 2 * C * dv)
    w = gdn.chunk_bwd_workspace_bytes(4, 4096, 16, 16, 128, 128, bf, 64, 0)
    ents = 4 * 64 * 16 * entry(64, 128, 128)        # no per-value-head parts: one value head per qk head
    assert ents <= w < ents + 4096
    packed = gdn.chunk_bwd_workspace_bytes(1, 1000, 2, 4, 64, 32, f32, 32, 5)
    ents = (32 + 5) * 4 * entry(32, 64, 32)
    parts = 2 * 1000 * 4 * 64 * 4                    # per-value-head dq and dk under grouped heads
    assert ents + parts <= packed < ents + parts + 4096
    assert gdn.chunk_bwd_workspace_bytes(1, 64, 1, 1, 48, 64, bf, 64, 0) == 0
    assert gdn.chunk_bwd_workspace_bytes(1, 64, 1, 1, 64, 64, bf, 48, 0) == 0
    p = ctypes.c_void_p(0x1000)
    ws = ctypes.c_void_p(0x100000)
    fwd = [1, 8, 1, 1, 64, 64, 0, p, p, p, p, p, None, 0, None]
    good = [p, None, p, p, p, p, p, None]
    assert lib.gdn_chunk_bwd(*fwd, None, *good[1:], 64, ws, 1 << 30, None) == 1      # d_o missing
    assert lib.gdn_chunk_bwd(*fwd, *good[:2], None, *good[3:], 64, ws, 1 << 30, None) == 1  # dq missing
    assert lib.gdn_chunk_bwd(*fwd, *good, 48, ws, 1 << 30, None) == 2                 # chunk
    assert lib.gdn_chunk_bwd(*fwd, *good, 64, ws, 16, None) == 3                      # workspace too small
    assert lib.gdn_chunk_bwd(*fwd, *good, 64, ctypes.c_void_p(0x100010), 1 << 30, None) == 3  # misaligned
    assert lib.gdn_chunk_bwd(*fwd, *good[:7], ctypes.c_void_p(0x1004), 64, ws, 1 << 30, None) == 1  # dh0
    bad_dtype = [1, 8, 1, 1, 64, 64, 5] + fwd[7:]
    assert lib.gdn_chunk_bwd(*bad_dtype, *good, 64, ws, 1 << 30, None) == 2
