"""fp64 CPU oracle for varlen (paged) softmax attention -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and the two share no code.

The arithmetic lives in ``fa_oracle.c`` (plain C, double precision); this module
builds it with gcc and marshals arrays.  See the header of ``fa_oracle.c`` for the
definition it follows and the passages it cites.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB = os.path.join(_HERE, "libfa_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile ``fa_oracle.c`` into ``libfa_oracle.so`` (strict IEEE, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-std=c11",
                               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        f = lib.fa_oracle_attention_t
        P = ctypes.c_void_p
        f.argtypes = [P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int64,
                      ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int, P, ctypes.c_int,
                      ctypes.c_double, ctypes.c_int, ctypes.c_int, P, P, P, ctypes.c_int, ctypes.c_int,
                      P, ctypes.c_int64]
        f.restype = ctypes.c_int
        w = lib.fa_oracle_widen
        w.argtypes = [P, ctypes.c_int64, ctypes.c_int, P]
        w.restype = None
        g = lib.fa_oracle_kv_append
        g.argtypes = [P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int, P,
                      ctypes.c_int, ctypes.c_int, ctypes.c_int64, P, P]
        g.restype = ctypes.c_int
        _lib = lib
    return _lib


DTYPES = {"bf16": 0, "f16": 1}


def _dtype_of(t) -> str:
    """'bf16' or 'f16' for a torch tensor; uint16 bit arrays are taken as bf16."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return {torch.bfloat16: "bf16", torch.float16: "f16"}[t.dtype]
    except ImportError:  # pragma: no cover
        pass
    return "bf16"


def _bits(t) -> np.ndarray:
    """bf16 / fp16 tensor or uint16 array -> contiguous uint16 numpy array of its bits."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            assert t.dtype in (torch.bfloat16, torch.float16), t.dtype
            return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(t)
    assert a.dtype == np.uint16
    return a


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def attention(q, k, v, cu_seqlens_q, cu_seqlens_k, block_table=None, page_block_size: int = 0,
              softmax_scale: float = 1.0, window_left: int = -1, window_right: int = -1,
              token_sel: Optional[np.ndarray] = None, nthreads: Optional[int] = None,
              alibi_slopes=None) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 attention over host bf16 or fp16 inputs (q, k, v of one element type).

    q: (total_q, H, D); k, v: (total_k, Hk, D) or, with ``block_table``,
    (num_blocks, page_block_size, Hk, D).  Returns ``out`` (total_q, H, D) float64
    and ``lse`` (H, total_q) float64 (natural log).  Rows not selected by
    ``token_sel`` are returned as NaN.  ``alibi_slopes``: None, (H,) or (batch, H)
    slopes; key j of query row i then gets -slope * |i + Lk - Lq - j| added to its
    scaled score.
    """
    lib = _load()
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    assert qb.ndim == 3
    total_q, H, D = qb.shape
    cu_q = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    cu_k = np.ascontiguousarray(cu_seqlens_k, dtype=np.int32)
    batch = cu_q.shape[0] - 1
    if block_table is not None:
        assert kb.ndim == 4 and kb.shape == vb.shape and kb.shape[1] == page_block_size
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        assert bt.ndim == 2 and bt.shape[0] == batch
        kv_rows, page, Hk, width = kb.shape[0], page_block_size, kb.shape[2], bt.shape[1]
        bt_ptr = bt.ctypes.data
    else:
        assert kb.ndim == 3 and kb.shape == vb.shape
        kv_rows, page, Hk, width, bt_ptr, bt = kb.shape[0], 0, kb.shape[1], 0, None, None
    assert kb.shape[-1] == D
    out = np.full((total_q, H, D), np.nan, dtype=np.float64)
    lse = np.full((H, total_q), np.nan, dtype=np.float64)
    sel = None
    if token_sel is not None:
        sel = np.ascontiguousarray(token_sel, dtype=np.uint8)
        assert sel.shape == (total_q,)
    al, al_sb = None, 0
    if alibi_slopes is not None:
        al = np.ascontiguousarray(np.asarray(alibi_slopes, dtype=np.float64))
        assert al.shape in ((H,), (batch, H)), al.shape
        al_sb = H if al.ndim == 2 else 0
    dt = _dtype_of(q)
    assert _dtype_of(k) == dt and _dtype_of(v) == dt, "q, k and v must share one element type"
    rc = lib.fa_oracle_attention_t(qb.ctypes.data, total_q, H, D, kb.ctypes.data, vb.ctypes.data,
                                   kv_rows, page, Hk, cu_q.ctypes.data, cu_k.ctypes.data, batch,
                                   bt_ptr, width, float(softmax_scale), int(window_left),
                                   int(window_right), None if sel is None else sel.ctypes.data,
                                   out.ctypes.data, lse.ctypes.data,
                                   int(nthreads or default_threads()), DTYPES[dt],
                                   None if al is None else al.ctypes.data, al_sb)
    if rc != 0:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)
    return out, lse


def widen(bits, dtype: str) -> np.ndarray:
    """The oracle's exact widening of 16-bit values ('bf16' or 'f16') to float64."""
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(a.shape, dtype=np.float64)
    _load().fa_oracle_widen(a.ctypes.data, a.size, DTYPES[dtype], out.ctypes.data)
    return out


def attention_workload(wl, token_sel=None, nthreads=None, alibi_slopes=None):
    """Convenience: run the oracle on an object with the workload fields."""
    return attention(wl.q, wl.k, wl.v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.block_table,
                     wl.page_block_size, wl.softmax_scale, wl.window_left, wl.window_right,
                     token_sel=token_sel, nthreads=nthreads, alibi_slopes=alibi_slopes)


def attention_padded(q, k, v, softmax_scale: float = 1.0, window_left: int = -1, window_right: int = -1,
                     nthreads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 attention over padded batch-major inputs: every batch element is an
    independent sequence (the non-varlen FlashAttention the pages point padded
    callers to), so batch element b is one call of :func:`attention` on q[b],
    k[b], v[b].

    q: (B, Sq, H, D); k, v: (B, Sk, Hk, D) bf16 (any strides).  Returns ``out``
    (B, Sq, H, D) float64 and ``lse`` (B, H, Sq) float64 (natural log).
    """
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    out = np.zeros((B, Sq, H, D), dtype=np.float64)
    lse = np.zeros((B, H, Sq), dtype=np.float64)
    cu_q = np.array([0, Sq], dtype=np.int32)
    cu_k = np.array([0, Sk], dtype=np.int32)
    for b in range(B):
        o, l = attention(q[b], k[b], v[b], cu_q, cu_k, None, 0, softmax_scale, window_left, window_right,
                         nthreads=nthreads)
        out[b] = o
        lse[b] = l
    return out, lse


def kv_append(k_new, v_new, cu_seqlens_new, cu_seqlens_k, block_table, k_pool, v_pool, strict=True):
    """Reference paged K/V append; returns new (k_pool, v_pool) uint16 arrays (inputs untouched).

    k_new/v_new (total_new, Hk, D) bf16; pools (num_blocks, P, Hk, D) bf16; new token j
    of sequence b goes to logical position Lk_b - Lnew_b + j.  A token whose position or
    block id falls outside the table or the pool is skipped; with ``strict`` that raises
    ValueError instead of returning.
    """
    lib = _load()
    kn, vn = _bits(k_new), _bits(v_new)
    kp, vp = _bits(k_pool).copy(), _bits(v_pool).copy()
    assert kn.ndim == 3 and kn.shape == vn.shape and kp.ndim == 4 and kp.shape == vp.shape
    cu_n = np.ascontiguousarray(cu_seqlens_new, dtype=np.int32)
    cu_k = np.ascontiguousarray(cu_seqlens_k, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    rc = lib.fa_oracle_kv_append(kn.ctypes.data, vn.ctypes.data, kn.shape[0], kn.shape[1], kn.shape[2],
                                 cu_n.ctypes.data, cu_k.ctypes.data, cu_n.shape[0] - 1,
                                 bt.ctypes.data, bt.shape[1], kp.shape[1], kp.shape[0],
                                 kp.ctypes.data, vp.ctypes.data)
    if rc == -1 or (rc != 0 and strict):
        raise ValueError("oracle kv_append rejected its arguments (code %d)" % rc)
    return kp, vp
