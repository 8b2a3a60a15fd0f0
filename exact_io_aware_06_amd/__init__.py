"""Fused exact attention forward for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libattn.so``, whose C ABI is declared in
``include/attn.h``. The binding only marshals arguments: it allocates the
outputs with PyTorch, passes device pointers, shapes, strides and the current
HIP stream, and raises on a non-OK status. Every arithmetic step of the
forward runs in the HIP kernels; there is no CPU fallback, and using this
module without the built library or without a GPU raises.

    from exact_io_aware_06_amd import attn_fwd
    o, lse = attn_fwd(q, k, v, causal=True)    # q, k, v: [B, H, N, d] on cuda

For few query rows against many keys (decoding), ``attn_fwd_splitkv``
computes the same function with the keys split across workgroups and the
partial results merged by their log-sum-exps.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

__all__ = ["attn_fwd", "attn_fwd_raw", "attn_fwd_splitkv", "attn_fwd_splitkv_raw",
           "attn_fwd_splitkv_noalloc", "NOALLOC_SCRATCH_BYTES",
           "attn_fwd_varlen", "prepare_varlen_call", "attn_bwd", "prepare_bwd_call",
           "bwd_workspace_size",
           "splitkv_num_splits", "splitkv_workspace_size", "prepare_call", "AttnError", "load_library", "library_path",
           "AttnTensor", "AttnMask", "ATTN_OK", "ATTN_ERR_INVALID",
           "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_HIP", "ATTN_BF16", "ATTN_F32"]

HERE = os.path.dirname(os.path.abspath(__file__))

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3
ATTN_BF16, ATTN_F32 = 0, 1
NOALLOC_SCRATCH_BYTES = 8 * 1024 * 1024   # ATTN_NOALLOC_SCRATCH_BYTES of include/attn.h
_STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID", 2: "ATTN_ERR_UNSUPPORTED", 3: "ATTN_ERR_HIP"}


class AttnTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class AttnMask(ctypes.Structure):
    _fields_ = [("bias", ctypes.POINTER(AttnTensor)), ("kv_len", ctypes.c_void_p),
                ("window", ctypes.c_int32), ("window_left", ctypes.c_int32),
                ("window_right", ctypes.c_int32)]


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def library_path() -> str:
    return os.environ.get("ATTN_LIBRARY", os.path.join(HERE, "libattn.so"))


_lib = None


def load_library():
    """Load ``libattn.so`` (built in-tree by ``exact_io_aware_06_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m exact_io_aware_06_amd.build` "
            "(the forward has no CPU fallback)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(AttnTensor)
    lib.attn_fwd.argtypes = [P, P, P, ctypes.POINTER(AttnMask), ctypes.c_int, ctypes.c_float,
                             P, P, ctypes.c_void_p]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd_splitkv.argtypes = [P, P, P, ctypes.POINTER(AttnMask), ctypes.c_int,
                                     ctypes.c_float, ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_int64, P, P, ctypes.c_void_p]
    lib.attn_fwd_splitkv.restype = ctypes.c_int
    lib.attn_fwd_splitkv_noalloc.argtypes = [P, P, P, ctypes.POINTER(AttnMask), ctypes.c_int,
                                             ctypes.c_float, ctypes.c_int32, P, P,
                                             ctypes.c_void_p]
    lib.attn_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.attn_fwd_splitkv_workspace_size.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int32]
    lib.attn_fwd_splitkv_workspace_size.restype = ctypes.c_int64
    lib.attn_fwd_splitkv_num_splits.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int] * 2
    lib.attn_fwd_splitkv_num_splits.restype = ctypes.c_int32
    lib.attn_fwd_varlen.argtypes = [P, P, P, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.POINTER(AttnMask), ctypes.c_int,
                                    ctypes.c_float, P, P, ctypes.c_void_p]
    lib.attn_fwd_varlen.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [P, P, P, P, P, P, ctypes.POINTER(AttnMask), ctypes.c_int,
                             ctypes.c_float, ctypes.c_void_p, ctypes.c_int64, P, P, P,
                             ctypes.c_void_p]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd_workspace_size.argtypes = [ctypes.c_int64] * 3
    lib.attn_bwd_workspace_size.restype = ctypes.c_int64
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def make_desc(data_ptr: int, dtype: int, shape, stride) -> AttnTensor:
    t = AttnTensor()
    t.data = data_ptr
    t.dtype = dtype
    for i in range(4):
        t.shape[i] = int(shape[i])
        t.stride[i] = int(stride[i])
    return t


def attn_fwd_raw(q: AttnTensor, k: AttnTensor, v: AttnTensor, mask: Optional[AttnMask],
                 causal: bool, scale: float, o: AttnTensor, lse: AttnTensor,
                 stream: int = 0) -> int:
    """Call the C entry point with prepared descriptors; returns the status."""
    lib = load_library()
    return lib.attn_fwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                        ctypes.byref(mask) if mask is not None else None,
                        1 if causal else 0, float(scale), ctypes.byref(o),
                        ctypes.byref(lse), ctypes.c_void_p(stream))


def attn_fwd_splitkv_raw(q: AttnTensor, k: AttnTensor, v: AttnTensor, mask: Optional[AttnMask],
                         causal: bool, scale: float, num_splits: int, workspace: int,
                         workspace_bytes: int, o: AttnTensor, lse: AttnTensor,
                         stream: int = 0) -> int:
    """Call the split-key C entry point with prepared descriptors; returns the status."""
    lib = load_library()
    return lib.attn_fwd_splitkv(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                ctypes.byref(mask) if mask is not None else None,
                                1 if causal else 0, float(scale), int(num_splits),
                                ctypes.c_void_p(workspace), int(workspace_bytes),
                                ctypes.byref(o), ctypes.byref(lse), ctypes.c_void_p(stream))


def splitkv_workspace_size(B: int, H: int, Nq: int, d: int, num_splits: int) -> int:
    """Workspace bytes ``attn_fwd_splitkv`` needs (-1 for invalid arguments)."""
    return int(load_library().attn_fwd_splitkv_workspace_size(B, H, Nq, d, num_splits))


def splitkv_num_splits(B: int, H: int, Nq: int, Nk: int, d: int, causal: bool = False,
                       has_bias: bool = False, Hk: Optional[int] = None) -> int:
    """The library's split count for this shape (1: no split); Hk: key/value
    heads (default H)."""
    return int(load_library().attn_fwd_splitkv_num_splits(
        B, H, H if Hk is None else Hk, Nq, Nk, d, 1 if causal else 0, 1 if has_bias else 0))


def last_error() -> str:
    return load_library().attn_last_error().decode()


def _torch_desc(t, name):
    import torch
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, H, N, d], got {tuple(t.shape)}")
    if t.dtype == torch.bfloat16:
        dt = ATTN_BF16
    elif t.dtype == torch.float32:
        dt = ATTN_F32
    else:
        raise TypeError(f"{name}: dtype {t.dtype} is not supported (bfloat16 or float32)")
    return make_desc(t.data_ptr(), dt, t.shape, t.stride())


def _prepare(q, k, v, bias, kv_len, scale, out, lse, window=None):
    import torch
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k and v must be GPU tensors (no CPU path exists)")
    B, H, Nq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dev = q.device
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=q.dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    if lse.dim() != 3 or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 [B, H, Nq] tensor")
    qd, kd, vd, od = (_torch_desc(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")))
    ld = make_desc(lse.data_ptr(), ATTN_F32, (*lse.shape, 1), (*lse.stride(), 1))
    mask = None
    keep = []
    if bias is not None or kv_len is not None or window is not None:
        mask = AttnMask()
        if window is not None:
            wl, wr = window
            mask.window = 1
            mask.window_left = -1 if wl is None else int(wl)
            mask.window_right = -1 if wr is None else int(wr)
        if bias is not None:
            if bias.dtype != torch.float32 or not bias.is_cuda or bias.dim() != 4:
                raise ValueError("bias must be a float32 4-D GPU tensor")
            bias_desc = make_desc(bias.data_ptr(), ATTN_F32, bias.shape, bias.stride())
            keep.append(bias_desc)
            mask.bias = ctypes.pointer(bias_desc)
        if kv_len is not None:
            if kv_len.dtype != torch.int32 or not kv_len.is_cuda or kv_len.numel() != B:
                raise ValueError("kv_len must be an int32 GPU tensor with B entries")
            if not kv_len.is_contiguous():
                raise ValueError("kv_len must be contiguous")
            mask.kv_len = kv_len.data_ptr()
    return scale, out, lse, (qd, kd, vd, od, ld, mask, keep)


def attn_fwd_splitkv(q, k, v, bias=None, kv_len=None, causal: bool = False,
                     scale: Optional[float] = None, num_splits: Optional[int] = None,
                     workspace=None, out=None, lse=None, window=None):
    """``attn_fwd`` with the keys split across workgroups (flash-decoding).

    Same arguments and result as ``attn_fwd`` (bfloat16 only). num_splits
    defaults to the library's choice for the shape. workspace: optional
    uint8 GPU tensor of at least ``splitkv_workspace_size(B, H, Nq, d,
    num_splits)`` bytes; allocated here when not given.
    """
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if num_splits is None:
        num_splits = splitkv_num_splits(B, H, Nq, Nk, d, causal, bias is not None, k.shape[1])
    scale, out, lse, (qd, kd, vd, od, ld, mask, _keep) = _prepare(q, k, v, bias, kv_len, scale,
                                                                    out, lse, window)
    need = splitkv_workspace_size(B, H, Nq, d, num_splits)
    if need < 0:
        raise AttnError(ATTN_ERR_INVALID, f"invalid split count {num_splits} for this shape")
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = attn_fwd_splitkv_raw(qd, kd, vd, mask, causal, scale, num_splits,
                                  workspace.data_ptr(), ws_bytes, od, ld, stream)
    if rc != ATTN_OK:
        raise AttnError(rc, last_error())
    return out, lse


def attn_fwd_splitkv_noalloc(q, k, v, bias=None, kv_len=None, causal: bool = False,
                             scale: Optional[float] = None, num_splits: Optional[int] = None,
                             out=None, lse=None, window=None):
    """``attn_fwd_splitkv`` without a workspace: the library keeps the split
    partials in its own per-device scratch array (NOALLOC_SCRATCH_BYTES), so
    the C call allocates nothing. Outputs are allocated here when not given.
    Calls that overlap on one device race on the array (use one stream)."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if num_splits is None:
        num_splits = splitkv_num_splits(B, H, Nq, Nk, d, causal, bias is not None, k.shape[1])
    scale, out, lse, (qd, kd, vd, od, ld, mask, _keep) = _prepare(q, k, v, bias, kv_len, scale,
                                                                    out, lse, window)
    lib = load_library()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = lib.attn_fwd_splitkv_noalloc(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd),
                                          ctypes.byref(mask) if mask is not None else None,
                                          1 if causal else 0, float(scale), int(num_splits),
                                          ctypes.byref(od), ctypes.byref(ld),
                                          ctypes.c_void_p(stream))
    if rc != ATTN_OK:
        raise AttnError(rc, last_error())
    return out, lse


def prepare_call(q, k, v, bias=None, kv_len=None, causal: bool = False,
                 scale: Optional[float] = None, out=None, lse=None, split: bool = False,
                 num_splits: Optional[int] = None, workspace=None, window=None):
    """Marshal the arguments once; return ``(enqueue, out, lse)``.

    ``enqueue()`` launches the forward (``split``: the split-key forward) on
    the stream that was current when this was called, with no per-call
    argument marshalling, and raises AttnError on a non-OK status. The
    tensors must stay alive and in place while ``enqueue`` is used.
    """
    import torch
    B, H, Nq, d = q.shape
    scale, out, lse, (qd, kd, vd, od, ld, mask, keep) = _prepare(q, k, v, bias, kv_len, scale,
                                                                   out, lse, window)
    lib = load_library()
    stream = torch.cuda.current_stream(q.device).cuda_stream
    refs = (qd, kd, vd, od, ld, mask, keep)
    mp = ctypes.byref(mask) if mask is not None else None
    args = [ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), mp, 1 if causal else 0,
            float(scale)]
    if split:
        if num_splits is None:
            num_splits = splitkv_num_splits(B, H, Nq, k.shape[2], d, causal, bias is not None,
                                            k.shape[1])
        need = splitkv_workspace_size(B, H, Nq, d, num_splits)
        if need < 0:
            raise AttnError(ATTN_ERR_INVALID, f"invalid split count {num_splits} for this shape")
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        args += [int(num_splits), ctypes.c_void_p(workspace.data_ptr()),
                 workspace.numel() * workspace.element_size()]
        fn = lib.attn_fwd_splitkv
    else:
        fn = lib.attn_fwd
    args += [ctypes.byref(od), ctypes.byref(ld), ctypes.c_void_p(stream)]

    def enqueue(_refs=refs, _ws=workspace):
        rc = fn(*args)
        if rc != ATTN_OK:
            raise AttnError(rc, last_error())

    return enqueue, out, lse


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                    causal: bool = False, scale: Optional[float] = None, window=None,
                    out=None, lse=None):
    """Attention over packed variable-length sequences (no padding).

    q: [total_q, H, d], k and v: [total_k, Hk, d] (token-major packing,
    last dimension contiguous), bfloat16 or float32 GPU tensors.
    cu_seqlens_q / cu_seqlens_k: int32 [num_seqs + 1] GPU tensors of
    cumulative offsets; sequence s owns rows cu_seqlens_q[s]:cu_seqlens_q[s+1]
    and keys cu_seqlens_k[s]:cu_seqlens_k[s+1]. max_seqlen_q: at least the
    longest query sequence. causal / window apply per sequence (bottom-right
    aligned). Returns (o [total_q, H, d], lse [H, total_q] float32).
    """
    enqueue, out, lse = prepare_varlen_call(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                                            causal, scale, window, out, lse)
    enqueue()
    return out, lse


def prepare_varlen_call(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                        causal: bool = False, scale: Optional[float] = None, window=None,
                        out=None, lse=None):
    """``attn_fwd_varlen``'s arguments marshalled once; returns ``(enqueue,
    out, lse)`` like ``prepare_call``.

    q: [total_q, H, d], k and v: [total_k, Hk, d] (token-major packing,
    last dimension contiguous), bfloat16 or float32 GPU tensors.
    cu_seqlens_q / cu_seqlens_k: int32 [num_seqs + 1] GPU tensors of
    cumulative offsets; sequence s owns rows cu_seqlens_q[s]:cu_seqlens_q[s+1]
    and keys cu_seqlens_k[s]:cu_seqlens_k[s+1]. max_seqlen_q: at least the
    longest query sequence. causal / window apply per sequence (bottom-right
    aligned). Returns (o [total_q, H, d], lse [H, total_q] float32).
    """
    import torch
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k and v must be GPU tensors (no CPU path exists)")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.dim() != 3:
            raise ValueError(f"{n} must be 3-D [total, heads, d], got {tuple(t.shape)}")
    for cu, n in ((cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k")):
        if cu.dtype != torch.int32 or not cu.is_cuda or cu.dim() != 1 or not cu.is_contiguous():
            raise ValueError(f"{n} must be a contiguous 1-D int32 GPU tensor")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold num_seqs + 1 offsets")
    Tq, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, Tq), dtype=torch.float32, device=q.device)
    if lse.shape != (H, Tq) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 [H, total_q] tensor")

    def view4(t, name):
        # [total, heads, d] seen as [1, heads, total, d]
        dd = _torch_desc(t.unsqueeze(0), name)
        st = t.stride()
        return make_desc(t.data_ptr(), dd.dtype, (1, t.shape[1], t.shape[0], t.shape[2]),
                         (t.numel(), st[1], st[0], st[2]))

    qd, kd, vd, od = view4(q, "q"), view4(k, "k"), view4(v, "v"), view4(out, "out")
    ld = make_desc(lse.data_ptr(), ATTN_F32, (1, H, Tq, 1), (lse.numel(), lse.stride(0),
                                                              lse.stride(1), 1))
    mask = None
    if window is not None:
        mask = AttnMask()
        wl, wr = window
        mask.window = 1
        mask.window_left = -1 if wl is None else int(wl)
        mask.window_right = -1 if wr is None else int(wr)
    lib = load_library()
    stream = torch.cuda.current_stream(q.device).cuda_stream
    refs = (qd, kd, vd, od, ld, mask)
    args = [ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd),
            ctypes.c_void_p(cu_seqlens_q.data_ptr()), ctypes.c_void_p(cu_seqlens_k.data_ptr()),
            cu_seqlens_q.numel() - 1, int(max_seqlen_q),
            ctypes.byref(mask) if mask is not None else None, 1 if causal else 0,
            float(scale), ctypes.byref(od), ctypes.byref(ld), ctypes.c_void_p(stream)]

    def enqueue(_refs=refs):
        rc = lib.attn_fwd_varlen(*args)
        if rc != ATTN_OK:
            raise AttnError(rc, last_error())

    return enqueue, out, lse


def bwd_workspace_size(B: int, H: int, Nq: int) -> int:
    """Workspace bytes ``attn_bwd`` needs (-1 for invalid extents)."""
    return int(load_library().attn_bwd_workspace_size(B, H, Nq))


def prepare_bwd_call(q, k, v, o, lse, dout, bias=None, kv_len=None, causal: bool = False,
                     scale: Optional[float] = None, window=None, dq=None, dk=None, dv=None,
                     workspace=None):
    """The backward's arguments marshalled once; returns ``(enqueue, dq, dk,
    dv)``. Inputs as for ``attn_bwd``."""
    import torch
    B, H, Nq, d = q.shape
    scale, _, lse, (qd, kd, vd, od, ld, mask, keep) = _prepare(q, k, v, bias, kv_len, scale,
                                                               o, lse, window)
    if not dout.is_cuda or dout.dtype != q.dtype or dout.shape != q.shape:
        raise ValueError("dout must be a GPU tensor with q's shape and dtype")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = bwd_workspace_size(B, H, Nq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    dod, dqd, dkd, dvd = (_torch_desc(t, n) for t, n in ((dout, "dout"), (dq, "dq"),
                                                          (dk, "dk"), (dv, "dv")))
    lib = load_library()
    stream = torch.cuda.current_stream(q.device).cuda_stream
    refs = (qd, kd, vd, od, ld, mask, keep, dod, dqd, dkd, dvd, workspace)
    args = [ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), ctypes.byref(od),
            ctypes.byref(ld), ctypes.byref(dod), ctypes.byref(mask) if mask is not None else None,
            1 if causal else 0, float(scale), ctypes.c_void_p(workspace.data_ptr()),
            workspace.numel() * workspace.element_size(), ctypes.byref(dqd), ctypes.byref(dkd),
            ctypes.byref(dvd), ctypes.c_void_p(stream)]

    def enqueue(_refs=refs):
        rc = lib.attn_bwd(*args)
        if rc != ATTN_OK:
            raise AttnError(rc, last_error())

    return enqueue, dq, dk, dv


def attn_bwd(q, k, v, o, lse, dout, bias=None, kv_len=None, causal: bool = False,
             scale: Optional[float] = None, window=None, dq=None, dk=None, dv=None,
             workspace=None):
    """Gradients (dq, dk, dv) of ``attn_fwd`` for the upstream gradient dout.

    q, k, v, bias, kv_len, causal, scale, window: as passed to ``attn_fwd``
    (bfloat16 only); o, lse: what it returned. dk and dv of a key/value head
    sum over the query heads that read it; no gradient is returned for the
    bias. Deterministic.
    """
    enqueue, dq, dk, dv = prepare_bwd_call(q, k, v, o, lse, dout, bias, kv_len, causal, scale,
                                           window, dq, dk, dv, workspace)
    enqueue()
    return dq, dk, dv


def attn_fwd(q, k, v, bias=None, kv_len=None, causal: bool = False,
             scale: Optional[float] = None, out=None, lse=None, window=None):
    """O = softmax_row(scale * Q K^T + bias) V and the row log-sum-exp.

    q: [B, H, Nq, d], k and v: [B, Hk, Nk, d] (Hk divides H), bfloat16 or
    float32 CUDA/HIP tensors with a contiguous last dimension. bias: optional
    float32 [B|1, H|1, Nq, Nk], added unscaled. kv_len: optional int32 [B] on
    the same device; keys at or past kv_len[b] are masked. causal hides key j
    from query i when j > i + (Nk - Nq). window: optional (left, right) —
    key j takes part only if i + (Nk - Nq) - left <= j <= i + (Nk - Nq) +
    right; None or a negative value leaves that side open (causal sets right
    to 0). scale defaults to 1/sqrt(d).
    Returns (o [B, H, Nq, d] in q's dtype, lse [B, H, Nq] float32).
    """
    import torch
    scale, out, lse, (qd, kd, vd, od, ld, mask, _keep) = _prepare(q, k, v, bias, kv_len, scale,
                                                                    out, lse, window)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = attn_fwd_raw(qd, kd, vd, mask, causal, scale, od, ld, stream)
    if rc != ATTN_OK:
        raise AttnError(rc, last_error())
    return out, lse
