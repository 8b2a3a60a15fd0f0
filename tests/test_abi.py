"""The C ABI library without a GPU: it loads, exports every function that
include/attn.h declares, its structs match the ctypes mirrors, and every
malformed call is rejected on the host with the documented status before any
HIP call is made."""

import ctypes
import math
import os
import re
import subprocess
import tempfile

import pytest

import exact_io_aware_06_amd as ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def _lib():
    if not os.path.exists(ea.library_path()):
        pytest.fail("libattn.so is not built; run `python -m exact_io_aware_06_amd.build`")
    return ea.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function():
    lib = _lib()
    names = _declared_functions()
    assert names == ["attn_abi_version", "attn_bwd", "attn_bwd_workspace_size", "attn_fwd",
                     "attn_fwd_splitkv", "attn_fwd_splitkv_noalloc",
                     "attn_fwd_splitkv_num_splits", "attn_fwd_splitkv_workspace_size",
                     "attn_fwd_varlen", "attn_last_error"]
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", ea.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (attn_\w+)", out))
    assert set(names) <= exported


def test_abi_version_matches_header():
    m = re.search(r"#define ATTN_ABI_VERSION (\d+)", open(HEADER).read())
    assert _lib().attn_abi_version() == int(m.group(1))


def test_struct_layout_matches_header():
    src = r"""
    #include <stdio.h>
    #include <stddef.h>
    #include "attn.h"
    int main(void) {
      printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(attn_tensor_t),
             offsetof(attn_tensor_t, dtype), offsetof(attn_tensor_t, shape),
             offsetof(attn_tensor_t, stride), sizeof(attn_mask_t),
             offsetof(attn_mask_t, kv_len), offsetof(attn_mask_t, window),
             offsetof(attn_mask_t, window_left), offsetof(attn_mask_t, window_right),
             sizeof(attn_status_t));
      return 0;
    }
    """
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), c, "-o", exe],
                       check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                               check=True).stdout.split()]
    T, M = ea.AttnTensor, ea.AttnMask
    assert vals == [ctypes.sizeof(T), T.dtype.offset, T.shape.offset, T.stride.offset,
                    ctypes.sizeof(M), M.kv_len.offset, M.window.offset, M.window_left.offset,
                    M.window_right.offset, 4]


# ------------------------------------------------------------ host-side rejections

def _desc(shape, dtype=ea.ATTN_BF16, data=0x10000, stride=None):
    if stride is None:
        stride = [shape[1] * shape[2] * shape[3], shape[2] * shape[3], shape[3], 1]
    return ea.make_desc(data, dtype, shape, stride)


def _call(q=None, k=None, v=None, o=None, lse=None, mask=None, causal=0, scale=0.125,
          **over):
    B, H, N, d = over.get("shape", (2, 4, 64, 64))
    q = q or _desc((B, H, N, d))
    k = k or _desc((B, H, N, d), data=0x20000)
    v = v or _desc((B, H, N, d), data=0x30000)
    o = o or _desc((B, H, N, d), data=0x40000)
    lse = lse or _desc((B, H, N, 1), ea.ATTN_F32, data=0x50000, stride=[H * N, N, 1, 1])
    _lib()
    return ea.attn_fwd_raw(q, k, v, mask, causal, scale, o, lse, 0)


def test_null_descriptor():
    lib = _lib()
    d = _desc((1, 1, 8, 64))
    rc = lib.attn_fwd(None, ctypes.byref(d), ctypes.byref(d), None, 0, 0.125,
                      ctypes.byref(d), ctypes.byref(d), None)
    assert rc == ea.ATTN_ERR_INVALID
    assert "non-NULL" in ea.last_error()


@pytest.mark.parametrize("scale", [math.inf, -math.inf, math.nan])
def test_non_finite_scale_is_invalid(scale):
    assert _call(scale=scale) == ea.ATTN_ERR_INVALID
    assert "scale" in ea.last_error()


@pytest.mark.parametrize("scale", [0.0, -0.0, -0.1, -8.0])
def test_non_positive_scale_is_unsupported(scale):
    # well formed, but the kernels scale the row maximum of the raw dot
    # products and need scale > 0
    assert _call(scale=scale) == ea.ATTN_ERR_UNSUPPORTED
    assert "scale" in ea.last_error()


def test_unsupported_head_dim():
    s = (1, 2, 16, 96)
    assert _call(shape=s, q=_desc(s), k=_desc(s), v=_desc(s), o=_desc(s)) == ea.ATTN_ERR_UNSUPPORTED
    assert "head dimension" in ea.last_error()


def test_dtype_mismatch_and_unknown_dtype():
    s = (2, 4, 64, 64)
    assert _call(k=_desc(s, ea.ATTN_F32)) == ea.ATTN_ERR_INVALID
    assert _call(q=_desc(s, 7), k=_desc(s, 7), v=_desc(s, 7), o=_desc(s, 7)) == ea.ATTN_ERR_UNSUPPORTED
    bad_lse = _desc((2, 4, 64, 1), ea.ATTN_BF16, stride=[256, 64, 1, 1])
    assert _call(lse=bad_lse) == ea.ATTN_ERR_INVALID


def test_shape_mismatches():
    assert _call(o=_desc((2, 4, 63, 64))) == ea.ATTN_ERR_INVALID
    assert _call(k=_desc((2, 4, 64, 128))) == ea.ATTN_ERR_INVALID
    assert _call(v=_desc((2, 4, 32, 64))) == ea.ATTN_ERR_INVALID
    assert _call(k=_desc((1, 4, 64, 64)), v=_desc((1, 4, 64, 64))) == ea.ATTN_ERR_INVALID
    # key/value heads must divide query heads
    assert _call(k=_desc((2, 3, 64, 64)), v=_desc((2, 3, 64, 64))) == ea.ATTN_ERR_INVALID
    assert "divide" in ea.last_error()
    lse = _desc((2, 4, 64, 2), ea.ATTN_F32)
    assert _call(lse=lse) == ea.ATTN_ERR_INVALID


def test_negative_extent_and_stride():
    assert _call(q=_desc((2, 4, -1, 64), stride=[1, 1, 1, 1])) == ea.ATTN_ERR_INVALID
    assert _call(q=_desc((2, 4, 64, 64), stride=[-16384, 4096, 64, 1])) == ea.ATTN_ERR_UNSUPPORTED


def test_layout_requirements():
    s = (2, 4, 64, 64)
    assert _call(q=_desc(s, stride=[16384, 4096, 64, 2])) == ea.ATTN_ERR_UNSUPPORTED
    assert "contiguous" in ea.last_error()
    assert _call(q=_desc(s, data=0x10002)) == ea.ATTN_ERR_UNSUPPORTED
    assert "aligned" in ea.last_error()
    assert _call(k=_desc(s, stride=[16384, 4096, 68, 1], data=0x20000)) == ea.ATTN_ERR_UNSUPPORTED
    lse = _desc((2, 4, 64, 1), ea.ATTN_F32, data=0x50000, stride=[256, 64, 2, 1])
    assert _call(lse=lse) == ea.ATTN_ERR_UNSUPPORTED
    # 64 key rows must span < 2 GiB (32-bit tile offsets)
    big = 1 << 24
    assert _call(k=_desc(s, stride=[64 * big, 64 * big, big, 1], data=0x20000)) == ea.ATTN_ERR_UNSUPPORTED
    assert "row stride" in ea.last_error()


def test_bias_checks():
    m = ea.AttnMask()
    b = _desc((1, 4, 64, 32), ea.ATTN_F32, data=0x60000)
    m.bias = ctypes.pointer(b)
    assert _call(mask=m) == ea.ATTN_ERR_INVALID          # Nk mismatch
    b2 = _desc((1, 4, 64, 64), ea.ATTN_BF16, data=0x60000)
    m.bias = ctypes.pointer(b2)
    assert _call(mask=m) == ea.ATTN_ERR_INVALID          # dtype
    b3 = _desc((3, 4, 64, 64), ea.ATTN_F32, data=0x60000)
    m.bias = ctypes.pointer(b3)
    assert _call(mask=m) == ea.ATTN_ERR_INVALID          # batch extent neither 1 nor B
    b4 = _desc((1, 4, 64, 64), ea.ATTN_F32, data=0x60000, stride=[0, 4096, 64, 2])
    m.bias = ctypes.pointer(b4)
    assert _call(mask=m) == ea.ATTN_ERR_UNSUPPORTED      # last dimension not contiguous
    b5 = _desc((1, 4, 64, 64), ea.ATTN_F32, data=0x60002)
    m.bias = ctypes.pointer(b5)
    assert _call(mask=m) == ea.ATTN_ERR_UNSUPPORTED      # not 4-byte aligned


def test_empty_problem_is_a_no_op():
    # B == 0: nothing to compute, nothing enqueued, OK (no GPU needed)
    s = (0, 4, 64, 64)
    lse = _desc((0, 4, 64, 1), ea.ATTN_F32, stride=[256, 64, 1, 1])
    assert _call(q=_desc(s), k=_desc(s), v=_desc(s), o=_desc(s), lse=lse) == ea.ATTN_OK
    assert ea.last_error() == ""
    s = (2, 4, 0, 64)
    lse = _desc((2, 4, 0, 1), ea.ATTN_F32, stride=[0, 0, 1, 1])
    assert _call(q=_desc(s), o=_desc(s), lse=lse) == ea.ATTN_OK


def test_python_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        ea.attn_fwd(q, q, q)


def test_no_undefined_kernel_symbols():
    # hipcc can silently drop a kernel's host stub (leaving an undefined
    # symbol that only fails when the library is loaded on the GPU machine)
    out = subprocess.run(["nm", "-D", "--undefined-only", ea.library_path()],
                         capture_output=True, text=True, check=True).stdout
    missing = [ln for ln in out.splitlines() if "attn" in ln]
    assert not missing, missing


# ------------------------------------------------------------ split-key entry points

def test_splitkv_workspace_size():
    ws = ea.splitkv_workspace_size
    # [num_splits, B, H, Nq, d] partial outputs + [num_splits, B, H, Nq] LSEs, fp32
    assert ws(2, 3, 5, 128, 4) == 4 * 2 * 3 * 5 * 129 * 4
    assert ws(8, 32, 1, 64, 1) == 8 * 32 * 65 * 4
    assert ws(0, 3, 5, 128, 4) == 0
    for bad in [(2, 3, 5, 128, 0), (2, 3, 5, 128, 1025), (-1, 3, 5, 128, 2), (2, 3, 5, 2048, 2)]:
        assert ws(*bad) == -1, bad


def test_splitkv_num_splits_choice():
    n = ea.splitkv_num_splits
    # decoding: 8 x 32 single-row tiles -> 2 splits make 512 workgroups,
    # one round on 256 CUs
    assert n(8, 32, 1, 16384, 128) == 2
    # 8 key/value heads: the 4 query heads of a group share a workgroup, so
    # there are 64 workgroups per split -> 8 splits
    assert n(8, 32, 1, 16384, 128, Hk=8) == 8
    assert n(8, 32, 1, 16384, 128, Hk=5) == 1      # Hk must divide H
    # one sequence, 32 heads, 64K keys: 16 splits of 4096 keys
    assert n(1, 32, 1, 65536, 128) == 16
    # every split keeps at least 256 keys
    assert n(1, 1, 1, 1000, 128) == 3
    assert n(1, 1, 1, 200, 64) == 1
    # enough query tiles already: no split
    assert n(2, 32, 4096, 4096, 128) == 1
    # empty or unsupported shapes: no split
    assert n(0, 32, 1, 4096, 128) == 1 and n(1, 1, 1, 4096, 96) == 1
    assert 1 <= n(1, 1, 1, 1 << 30, 128) <= 1024


def _split_call(num_splits=4, workspace=0x70000, ws_bytes=1 << 30, dtype=ea.ATTN_BF16,
                shape=(2, 4, 1, 64), nk=1024):
    B, H, Nq, d = shape
    q = _desc((B, H, Nq, d), dtype)
    k = _desc((B, H, nk, d), dtype, data=0x20000)
    v = _desc((B, H, nk, d), dtype, data=0x30000)
    o = _desc((B, H, Nq, d), dtype, data=0x40000)
    lse = _desc((B, H, Nq, 1), ea.ATTN_F32, data=0x50000, stride=[H * Nq, Nq, 1, 1])
    _lib()
    return ea.attn_fwd_splitkv_raw(q, k, v, None, 0, 0.125, num_splits, workspace, ws_bytes,
                                   o, lse, 0)


def test_splitkv_rejections():
    # every call below needs more than one split, so it is refused before
    # any kernel could be enqueued
    assert _split_call(num_splits=0) == ea.ATTN_ERR_INVALID
    assert "num_splits" in ea.last_error()
    assert _split_call(num_splits=1025) == ea.ATTN_ERR_INVALID
    assert _split_call(dtype=ea.ATTN_F32) == ea.ATTN_ERR_UNSUPPORTED
    assert "bf16" in ea.last_error()
    assert _split_call(workspace=0) == ea.ATTN_ERR_INVALID
    assert "workspace" in ea.last_error()
    assert _split_call(workspace=0x70008) == ea.ATTN_ERR_INVALID
    need = ea.splitkv_workspace_size(2, 4, 1, 64, 4)
    assert _split_call(ws_bytes=need - 1) == ea.ATTN_ERR_INVALID
    assert "too small" in ea.last_error()
    # the check is against the split count actually used: 1024 keys in
    # requested 7 splits -> splits of 192 keys -> 6 splits
    need6 = ea.splitkv_workspace_size(2, 4, 1, 64, 6)
    assert _split_call(num_splits=7, ws_bytes=need6 - 4) == ea.ATTN_ERR_INVALID
    assert "6 splits" in ea.last_error()
    # the common argument checks still apply
    assert _split_call(shape=(2, 4, 1, 96)) == ea.ATTN_ERR_UNSUPPORTED


# ------------------------------------------------------------ packed sequences

def _varlen_call(shape0=1, cu_q=0x80000, cu_k=0x90000, num_seqs=3, max_q=64, mask=None,
                 dtype=ea.ATTN_BF16):
    T, H, d = 256, 4, 64
    q = _desc((shape0, H, T, d), dtype, stride=[T * H * d, d, H * d, 1])
    k = _desc((shape0, H, T, d), dtype, data=0x20000, stride=[T * H * d, d, H * d, 1])
    v = _desc((shape0, H, T, d), dtype, data=0x30000, stride=[T * H * d, d, H * d, 1])
    o = _desc((shape0, H, T, d), dtype, data=0x40000, stride=[T * H * d, d, H * d, 1])
    lse = _desc((shape0, H, T, 1), ea.ATTN_F32, data=0x50000, stride=[H * T, T, 1, 1])
    lib = _lib()
    return lib.attn_fwd_varlen(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                               ctypes.c_void_p(cu_q), ctypes.c_void_p(cu_k), num_seqs, max_q,
                               ctypes.byref(mask) if mask is not None else None, 0, 0.125,
                               ctypes.byref(o), ctypes.byref(lse), None)


def test_varlen_rejections():
    # every call below is refused on the host before any launch
    assert _varlen_call(shape0=2) == ea.ATTN_ERR_INVALID
    assert "packed" in ea.last_error()
    assert _varlen_call(cu_q=0) == ea.ATTN_ERR_INVALID
    assert _varlen_call(cu_k=0x90002) == ea.ATTN_ERR_INVALID
    assert _varlen_call(num_seqs=-1) == ea.ATTN_ERR_INVALID
    assert _varlen_call(max_q=-5) == ea.ATTN_ERR_INVALID
    m = ea.AttnMask()
    m.kv_len = 0x70000
    assert _varlen_call(mask=m) == ea.ATTN_ERR_INVALID
    assert "kv_len" in ea.last_error()
    # nothing to compute: OK without touching the device
    assert _varlen_call(num_seqs=0) == ea.ATTN_OK
    assert _varlen_call(max_q=0) == ea.ATTN_OK


# ------------------------------------------------------------------ backward

def _bwd_call(dtype=ea.ATTN_BF16, workspace=0xA0000, ws_bytes=1 << 20, dq_shape=None,
              dout_dtype=None, q_stride=None, dout_stride=None):
    B, H, N, d = 2, 4, 64, 64
    q = _desc((B, H, N, d), dtype, stride=q_stride)
    k = _desc((B, H, N, d), dtype, data=0x20000)
    v = _desc((B, H, N, d), dtype, data=0x30000)
    o = _desc((B, H, N, d), dtype, data=0x40000)
    lse = _desc((B, H, N, 1), ea.ATTN_F32, data=0x50000, stride=[H * N, N, 1, 1])
    do = _desc((B, H, N, d), dout_dtype if dout_dtype is not None else dtype, data=0x60000,
               stride=dout_stride)
    dq = _desc(dq_shape or (B, H, N, d), dtype, data=0x70000)
    dk = _desc((B, H, N, d), dtype, data=0x80000)
    dv = _desc((B, H, N, d), dtype, data=0x90000)
    lib = _lib()
    return lib.attn_bwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(o),
                        ctypes.byref(lse), ctypes.byref(do), None, 0, 0.125,
                        ctypes.c_void_p(workspace), ws_bytes, ctypes.byref(dq), ctypes.byref(dk),
                        ctypes.byref(dv), None)


def test_bwd_workspace_size():
    assert ea.bwd_workspace_size(2, 4, 64) == 8 * 2 * 4 * 64
    assert ea.bwd_workspace_size(-1, 4, 64) == -1


def test_bwd_rejections():
    # every call below is refused on the host before any launch
    assert _bwd_call(dtype=ea.ATTN_F32) == ea.ATTN_ERR_UNSUPPORTED
    assert "bf16" in ea.last_error()
    assert _bwd_call(dq_shape=(2, 4, 63, 64)) == ea.ATTN_ERR_INVALID
    assert "shape" in ea.last_error()
    assert _bwd_call(dout_dtype=ea.ATTN_F32) == ea.ATTN_ERR_INVALID
    assert _bwd_call(workspace=0) == ea.ATTN_ERR_INVALID
    assert _bwd_call(workspace=0xA0004) == ea.ATTN_ERR_INVALID
    assert _bwd_call(ws_bytes=8 * 2 * 4 * 64 - 1) == ea.ATTN_ERR_INVALID
    assert "too small" in ea.last_error()
    # 64 rows of q or dout must span < 2 GiB (the dK/dV kernel's tile
    # offsets are 32-bit): 64 * 2^24 bf16 elements is exactly 2 GiB
    big = 1 << 24
    for kw in ("q_stride", "dout_stride"):
        assert _bwd_call(**{kw: [64 * big, 64 * big, big, 1]}) == ea.ATTN_ERR_UNSUPPORTED
        assert "row stride" in ea.last_error()
        # just under the limit the stride is accepted: the call gets as far
        # as the (too small) workspace, which is checked after the strides
        assert _bwd_call(ws_bytes=8, **{kw: [64 * big, 64 * big, big - 8, 1]}) == ea.ATTN_ERR_INVALID
        assert "too small" in ea.last_error()


def _bwd_empty_call(q_shape, kv_shape, dk_data=0x80000):
    q = _desc(q_shape)
    k = _desc(kv_shape, data=0x20000)
    v = _desc(kv_shape, data=0x30000)
    o = _desc(q_shape, data=0x40000)
    B, H, N, _ = q_shape
    lse = _desc((B, H, N, 1), ea.ATTN_F32, data=0x50000, stride=[H * N, N, 1, 1])
    do = _desc(q_shape, data=0x60000)
    dq = _desc(q_shape, data=0x70000)
    dk = _desc(kv_shape, data=dk_data)
    dv = _desc(kv_shape, data=0x90000)
    lib = _lib()
    return lib.attn_bwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(o),
                        ctypes.byref(lse), ctypes.byref(do), None, 0, 0.125, None, 0,
                        ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), None)


def test_bwd_empty_query_side():
    # no query rows, or no query heads, with keys present: dK and dV must be
    # zeroed, so their layout is checked on the host first (a misaligned dk
    # is refused before any launch); with no keys either there is nothing to
    # write and the call returns OK without touching the device
    assert _bwd_empty_call((2, 4, 0, 64), (2, 2, 300, 64), dk_data=0x80002) == \
        ea.ATTN_ERR_UNSUPPORTED
    assert "dk" in ea.last_error()
    assert _bwd_empty_call((2, 0, 10, 64), (2, 2, 300, 64), dk_data=0x80002) == \
        ea.ATTN_ERR_UNSUPPORTED
    assert _bwd_empty_call((2, 4, 0, 64), (2, 2, 0, 64)) == ea.ATTN_OK
    assert _bwd_empty_call((0, 4, 10, 64), (0, 2, 300, 64)) == ea.ATTN_OK


def _noalloc_call(shape_q, Nk, num_splits, dtype=ea.ATTN_BF16):
    B, H, Nq, d = shape_q
    q = _desc(shape_q, dtype)
    k = _desc((B, H, Nk, d), dtype, data=0x20000)
    v = _desc((B, H, Nk, d), dtype, data=0x30000)
    o = _desc(shape_q, dtype, data=0x40000)
    lse = _desc((B, H, Nq, 1), ea.ATTN_F32, data=0x50000, stride=[H * Nq, Nq, 1, 1])
    lib = _lib()
    return lib.attn_fwd_splitkv_noalloc(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), None,
                                        0, 0.125, num_splits, ctypes.byref(o), ctypes.byref(lse),
                                        None)


def test_noalloc_rejections():
    # refused on the host before the scratch array is looked up or anything
    # is enqueued: partials beyond the scratch size, f32, bad split counts;
    # an empty problem is a no-op
    assert ea.NOALLOC_SCRATCH_BYTES == int(re.search(
        r"#define ATTN_NOALLOC_SCRATCH_BYTES \((\d+) \* 1024 \* 1024\)",
        open(HEADER).read()).group(1)) << 20
    # 2 splits x 8 x 32 x 64 rows x 129 x 4 bytes = 16.9 MB > 8 MiB
    assert _noalloc_call((8, 32, 64, 128), 4096, 2) == ea.ATTN_ERR_UNSUPPORTED
    assert "scratch" in ea.last_error()
    assert _noalloc_call((1, 2, 1, 128), 4096, 4, dtype=ea.ATTN_F32) == ea.ATTN_ERR_UNSUPPORTED
    assert _noalloc_call((1, 2, 1, 128), 4096, 0) == ea.ATTN_ERR_INVALID
    assert _noalloc_call((1, 2, 1, 128), 4096, 1025) == ea.ATTN_ERR_INVALID
    assert _noalloc_call((0, 2, 1, 128), 4096, 4) == ea.ATTN_OK
