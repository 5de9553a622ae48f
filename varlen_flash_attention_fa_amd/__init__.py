"""Python binding of libfa_varlen.so (MI355X / gfx950 varlen flash-attention forward).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/fa_varlen.h``.  torch is used for
device memory and the current stream.  There is no CPU fallback: if the shared
library has not been built, importing the low-level functions raises.

Low-level names mirror the C ABI (``fa_varlen_check``, ``fa_varlen_workspace_bytes``,
``fa_varlen_fwd``, ``fa_padded_check``, ``fa_padded_workspace_bytes``, ``fa_padded_fwd``,
``fa_kv_append_check``, ``fa_kv_append``, ``fa_last_error``) and take :class:`FaTensor`
descriptors; :func:`varlen_fwd`, :func:`padded_fwd` and :func:`kv_append` are the
tensor-level convenience wrappers.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

__all__ = [
    "FaTensor", "FlashAttnError", "lib_path", "load", "fa_varlen_check",
    "fa_varlen_workspace_bytes", "fa_varlen_fwd", "fa_last_error", "varlen_fwd", "desc",
    "fa_varlen_set_kernel_events", "fa_varlen_fwd_static", "FA_STATIC_SCRATCH_BYTES", "fa_kv_append_check", "fa_kv_append", "kv_append",
    "fa_padded_check", "fa_padded_workspace_bytes", "fa_padded_fwd", "padded_fwd",
    "FA_DTYPE_BF16", "FA_DTYPE_I32", "FA_DTYPE_F16", "FA_DTYPE_F32", "STATUS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfa_varlen.so")

FA_DTYPE_BF16 = 1
FA_DTYPE_I32 = 2
FA_DTYPE_F16 = 3
FA_DTYPE_F32 = 4
STATUS = {0: "FA_OK", 1: "FA_ERR_RANK", 2: "FA_ERR_CONTIGUOUS", 3: "FA_ERR_SHAPE",
          4: "FA_ERR_PAGE_SIZE", 5: "FA_ERR_HEAD_DIM", 6: "FA_ERR_DTYPE", 7: "FA_ERR_ARGUMENT",
          8: "FA_ERR_WORKSPACE", 9: "FA_ERR_DEVICE", 10: "FA_ERR_HIP"}


class FaTensor(ctypes.Structure):
    """Mirror of ``fa_tensor``: data pointer, dtype, rank, shape[4], stride[4] (elements)."""

    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class FlashAttnError(ValueError):
    def __init__(self, code: int, message: str):
        super().__init__(message)
        self.code = code
        self.status = STATUS.get(code, str(code))


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libfa_varlen.so is not built; run varlen_flash_attention_fa_amd/build.py "
                           "(or __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(FaTensor)
    lib.fa_varlen_check.argtypes = [P, P, P, P, ctypes.c_int32, P, ctypes.c_int32, P]
    lib.fa_varlen_check.restype = ctypes.c_int
    lib.fa_varlen_workspace_bytes.argtypes = [P, P, P, ctypes.c_int32, P, ctypes.c_int32,
                                              ctypes.POINTER(ctypes.c_size_t)]
    lib.fa_varlen_workspace_bytes.restype = ctypes.c_int
    lib.fa_varlen_fwd.argtypes = [P, P, P, P, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, P,
                                  ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_int32, P,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.fa_varlen_fwd.restype = ctypes.c_int
    lib.fa_varlen_fwd_static.argtypes = [P, P, P, P, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, P,
                                         ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_int32, P,
                                         ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_varlen_fwd_static.restype = ctypes.c_int
    lib.fa_varlen_set_kernel_events.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_varlen_set_kernel_events.restype = ctypes.c_int
    lib.fa_padded_check.argtypes = [P, P, P, P, P]
    lib.fa_padded_check.restype = ctypes.c_int
    lib.fa_padded_workspace_bytes.argtypes = [P, P, P, ctypes.POINTER(ctypes.c_size_t)]
    lib.fa_padded_workspace_bytes.restype = ctypes.c_int
    lib.fa_padded_fwd.argtypes = [P, P, P, P, ctypes.c_float, ctypes.c_int32, ctypes.c_int32, P,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.fa_padded_fwd.restype = ctypes.c_int
    lib.fa_kv_append_check.argtypes = [P, P, ctypes.c_int32, P, P, P, ctypes.c_int32]
    lib.fa_kv_append_check.restype = ctypes.c_int
    lib.fa_kv_append.argtypes = [P, P, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, P, P, P,
                                 ctypes.c_int32, ctypes.c_void_p]
    lib.fa_kv_append.restype = ctypes.c_int
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def desc(shape: Sequence[int], stride: Optional[Sequence[int]] = None, dtype: int = FA_DTYPE_BF16,
         data: int = 0) -> FaTensor:
    """Descriptor from explicit shape/strides (row-major strides by default)."""
    shape = [int(s) for s in shape]
    if stride is None:
        stride, acc = [], 1
        for s in reversed(shape):
            stride.insert(0, acc)
            acc *= max(1, s)
    t = FaTensor()
    t.data = data or None
    t.dtype = dtype
    t.rank = len(shape)
    for i in range(min(4, len(shape))):
        t.shape[i] = shape[i]
        t.stride[i] = int(stride[i])
    return t


def _tdesc(t) -> FaTensor:
    import torch
    dt = {torch.bfloat16: FA_DTYPE_BF16, torch.int32: FA_DTYPE_I32, torch.float16: FA_DTYPE_F16,
          torch.float32: FA_DTYPE_F32}.get(t.dtype, 0)
    return desc(list(t.shape), list(t.stride()), dt, t.data_ptr())


def _ref(d: Optional[FaTensor]):
    return ctypes.byref(d) if d is not None else None


def fa_last_error() -> str:
    return load().fa_last_error().decode("utf-8", "replace")


def _raise_on(rc: int) -> None:
    if rc != 0:
        raise FlashAttnError(rc, fa_last_error())


def _check_seqlens(named) -> None:
    """Offsets arrays go to the C ABI as bare pointers, so their layout is checked here.

    A strided array gets the pages' text ("seqlens_q has to be contiguous", page
    "flash-attn-varlen expects input tensors of rank 3", Related errors); dtype and
    rank, which the pages do not show, get their own."""
    import torch
    texts = {"seqlens_q": "seqlens_q has to be contiguous", "seqlens_k": "seqlens_k has to be contiguous",
             "seqlens_new": "seqlens_new has to be contiguous"}
    for name, t in named:
        if t.dtype != torch.int32 or t.dim() != 1:
            raise FlashAttnError(7, "%s must be a 1-d int32 tensor (got %s, %d-d)" % (name, t.dtype, t.dim()))
        if not t.is_contiguous():
            raise FlashAttnError(2, texts[name])


def fa_varlen_check(q: FaTensor, k: FaTensor, v: FaTensor, out: Optional[FaTensor], batch: int,
                    block_table: Optional[FaTensor], page_block_size: int,
                    alibi_slopes: Optional[FaTensor] = None) -> int:
    """Shape/stride/dtype contract only (host code, no GPU needed).  Returns the status."""
    return load().fa_varlen_check(_ref(q), _ref(k), _ref(v), _ref(out), int(batch),
                                  _ref(block_table), int(page_block_size or 0), _ref(alibi_slopes))


def fa_varlen_workspace_bytes(q: FaTensor, k: FaTensor, v: FaTensor, batch: int,
                              block_table: Optional[FaTensor], page_block_size: int) -> int:
    n = ctypes.c_size_t(0)
    rc = load().fa_varlen_workspace_bytes(_ref(q), _ref(k), _ref(v), int(batch), _ref(block_table),
                                          int(page_block_size or 0), ctypes.byref(n))
    _raise_on(rc)
    return int(n.value)


def fa_varlen_fwd(q: FaTensor, k: FaTensor, v: FaTensor, out: FaTensor, cu_seqlens_q: int,
                  cu_seqlens_k: int, batch: int, block_table: Optional[FaTensor],
                  page_block_size: int, softmax_scale: float, window_left: int, window_right: int,
                  softmax_lse: int, workspace: int, workspace_bytes: int, stream: int,
                  alibi_slopes: Optional[FaTensor] = None) -> int:
    """Raw C-ABI call with descriptors and integer device addresses.  Returns the status."""
    return load().fa_varlen_fwd(_ref(q), _ref(k), _ref(v), _ref(out), cu_seqlens_q or None,
                                cu_seqlens_k or None, int(batch), _ref(block_table),
                                int(page_block_size or 0), float(softmax_scale), int(window_left),
                                int(window_right), _ref(alibi_slopes), softmax_lse or None,
                                workspace or None, int(workspace_bytes), stream or None)


# size of the scratch array fa_varlen_fwd_static uses on each GPU (FA_STATIC_SCRATCH_BYTES)
FA_STATIC_SCRATCH_BYTES = 64 << 20


def fa_varlen_fwd_static(q: FaTensor, k: FaTensor, v: FaTensor, out: FaTensor, cu_seqlens_q: int,
                         cu_seqlens_k: int, batch: int, block_table: Optional[FaTensor],
                         page_block_size: int, softmax_scale: float, window_left: int, window_right: int,
                         softmax_lse: int, stream: int, alibi_slopes: Optional[FaTensor] = None) -> int:
    """Raw C-ABI call of the allocation-free entry (no workspace).  Returns the status."""
    return load().fa_varlen_fwd_static(_ref(q), _ref(k), _ref(v), _ref(out), cu_seqlens_q or None,
                                       cu_seqlens_k or None, int(batch), _ref(block_table),
                                       int(page_block_size or 0), float(softmax_scale), int(window_left),
                                       int(window_right), _ref(alibi_slopes), softmax_lse or None,
                                       stream or None)


def fa_varlen_set_kernel_events(start_event: int, stop_event: int) -> int:
    """Measurement hook: bracket the main kernel of later calls with these hipEvent_t handles."""
    return load().fa_varlen_set_kernel_events(start_event or None, stop_event or None)


def fa_padded_check(q: FaTensor, k: FaTensor, v: FaTensor, out: Optional[FaTensor],
                    alibi_slopes: Optional[FaTensor] = None) -> int:
    """Contract of the padded entry only (host code, no GPU needed).  Returns the status."""
    return load().fa_padded_check(_ref(q), _ref(k), _ref(v), _ref(out), _ref(alibi_slopes))


def fa_padded_workspace_bytes(q: FaTensor, k: FaTensor, v: FaTensor) -> int:
    n = ctypes.c_size_t(0)
    _raise_on(load().fa_padded_workspace_bytes(_ref(q), _ref(k), _ref(v), ctypes.byref(n)))
    return int(n.value)


def fa_padded_fwd(q: FaTensor, k: FaTensor, v: FaTensor, out: FaTensor, softmax_scale: float,
                  window_left: int, window_right: int, softmax_lse: int, workspace: int,
                  workspace_bytes: int, stream: int, alibi_slopes: Optional[FaTensor] = None) -> int:
    """Raw C-ABI call of the padded entry.  Returns the status."""
    return load().fa_padded_fwd(_ref(q), _ref(k), _ref(v), _ref(out), float(softmax_scale), int(window_left),
                                int(window_right), _ref(alibi_slopes), softmax_lse or None, workspace or None,
                                int(workspace_bytes), stream or None)


def padded_fwd(q, k, v, softmax_scale: Optional[float] = None, window_left: int = -1,
               window_right: int = -1, return_lse: bool = False, out=None, workspace=None, stream=None,
               alibi_slopes=None):
    """Forward over padded (B, Sq, H, D) / (B, Sk, Hk, D) device tensors.

    Returns ``out`` (B, Sq, H, D) bf16, plus ``lse`` (B, H, Sq) fp32 if ``return_lse``.
    """
    import torch
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(q.shape[-1])
    dq, dk, dv = _tdesc(q), _tdesc(k), _tdesc(v)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    dout = _tdesc(out)
    dal = _tdesc(alibi_slopes) if alibi_slopes is not None else None
    _raise_on(fa_padded_check(dq, dk, dv, dout, dal))
    nbytes = fa_padded_workspace_bytes(dq, dk, dv)
    if nbytes and (workspace is None or workspace.numel() * workspace.element_size() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    lse = None
    if return_lse:
        lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    _raise_on(fa_padded_fwd(dq, dk, dv, dout, softmax_scale, window_left, window_right,
                            lse.data_ptr() if lse is not None else 0,
                            workspace.data_ptr() if (nbytes and workspace is not None) else 0, nbytes,
                            int(stream), dal))
    return (out, lse) if return_lse else out


def fa_kv_append_check(k_new: FaTensor, v_new: FaTensor, batch: int, block_table: FaTensor,
                       k_cache: FaTensor, v_cache: FaTensor, page_block_size: int) -> int:
    """Contract of the paged append only (host code, no GPU needed).  Returns the status."""
    return load().fa_kv_append_check(_ref(k_new), _ref(v_new), int(batch), _ref(block_table),
                                     _ref(k_cache), _ref(v_cache), int(page_block_size or 0))


def fa_kv_append(k_new: FaTensor, v_new: FaTensor, cu_seqlens_new: int, cu_seqlens_k: int, batch: int,
                 block_table: FaTensor, k_cache: FaTensor, v_cache: FaTensor, page_block_size: int,
                 stream: int) -> int:
    """Raw C-ABI call with descriptors and integer device addresses.  Returns the status."""
    return load().fa_kv_append(_ref(k_new), _ref(v_new), cu_seqlens_new or None, cu_seqlens_k or None,
                               int(batch), _ref(block_table), _ref(k_cache), _ref(v_cache),
                               int(page_block_size or 0), stream or None)


def kv_append(k_new, v_new, cu_seqlens_new, cu_seqlens_k, block_table, k_cache, v_cache,
              page_block_size: Optional[int] = None, stream=None):
    """Write new tokens' K/V rows into a paged cache in place (device tensors).

    k_new/v_new (total_new, Hk, D) bf16; cu_seqlens_new / cu_seqlens_k int32 (batch+1,),
    the latter counting keys after the append; block_table (batch, max_blocks) int32;
    k_cache/v_cache (num_blocks, P, Hk, D) bf16.  New token j of sequence b lands at
    logical key Lk_b - Lnew_b + j.  Enqueues on torch's current stream (or ``stream``).
    """
    import torch
    _check_seqlens((("seqlens_new", cu_seqlens_new), ("seqlens_k", cu_seqlens_k)))
    batch = cu_seqlens_new.shape[0] - 1
    if cu_seqlens_k.shape[0] != batch + 1:
        raise FlashAttnError(7, "cu_seqlens_new and cu_seqlens_k must both have batch+1 entries")
    if page_block_size is None:
        page_block_size = k_cache.shape[1] if k_cache.dim() == 4 else 0
    if stream is None:
        stream = torch.cuda.current_stream(k_cache.device).cuda_stream
    rc = fa_kv_append(_tdesc(k_new), _tdesc(v_new), cu_seqlens_new.data_ptr(), cu_seqlens_k.data_ptr(),
                      batch, _tdesc(block_table), _tdesc(k_cache), _tdesc(v_cache), page_block_size,
                      int(stream))
    _raise_on(rc)
    return k_cache, v_cache


def varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, block_table=None,
               page_block_size: Optional[int] = None, softmax_scale: Optional[float] = None,
               window_left: int = -1, window_right: int = -1, return_lse: bool = False,
               out=None, workspace=None, stream=None, alibi_slopes=None):
    """Varlen flash-attention forward on device tensors.

    q (total_q, H, D) bf16 or fp16; k/v (total_k, Hk, D) or paged (num_blocks, P, Hk, D), q's dtype,
    with ``block_table`` (batch, max_blocks) int32; cu_seqlens_* int32 (batch+1,).
    Returns ``out`` (same shape as q), plus ``lse`` (H, total_q) fp32 if
    ``return_lse``.  Allocates out / lse / workspace with torch when not given and
    enqueues on torch's current stream (or ``stream``).
    """
    import torch
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(q.shape[-1])
    _check_seqlens((("seqlens_q", cu_seqlens_q), ("seqlens_k", cu_seqlens_k)))
    batch = cu_seqlens_q.shape[0] - 1
    if cu_seqlens_k.shape[0] != batch + 1:
        raise FlashAttnError(7, "cu_seqlens_q and cu_seqlens_k must both have batch+1 entries")
    dq, dk, dv = _tdesc(q), _tdesc(k), _tdesc(v)
    dbt = _tdesc(block_table) if block_table is not None else None
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format) if q.dim() == 3 else \
            torch.empty(0, device=q.device, dtype=q.dtype)
    dout = _tdesc(out)
    dal = _tdesc(alibi_slopes) if alibi_slopes is not None else None
    rc = fa_varlen_check(dq, dk, dv, dout, batch, dbt, page_block_size or 0, dal)
    _raise_on(rc)
    nbytes = fa_varlen_workspace_bytes(dq, dk, dv, batch, dbt, page_block_size or 0)
    if nbytes and (workspace is None or workspace.numel() * workspace.element_size() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    lse = None
    if return_lse:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = fa_varlen_fwd(dq, dk, dv, dout, cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), batch,
                       dbt, page_block_size or 0, softmax_scale, window_left, window_right,
                       lse.data_ptr() if lse is not None else 0,
                       workspace.data_ptr() if (nbytes and workspace is not None) else 0,
                       nbytes, int(stream), dal)
    _raise_on(rc)
    return (out, lse) if return_lse else out
