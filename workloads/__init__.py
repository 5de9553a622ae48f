"""Seeded synthetic inputs for varlen (paged) flash-attention forward.

This module only draws inputs: sequence lengths, the physical-block permutation
of a paged K/V pool and N(0,1) bf16 tensors.  It holds none of the attention
arithmetic, so both the fp64 oracle (under ``oracle/``) and the HIP path can be
fed from it without sharing any part of the method.

Layouts follow the contract the pages quote for candle's ``FlashAttentionVarLen``
(pages "flash-attn-varlen expects input tensors of rank 3" and
"flash-attn-varlen paged expects k/v tensors of rank 4", sections Source and
What it means):

* q: rank 3 ``(total_q, num_heads, head_dim)``
* k/v non-paged: rank 3 ``(total_k, num_heads_k, head_dim)``
* k/v paged: rank 4 ``(num_blocks, page_block_size, num_heads_k, head_dim)``
  read through a per-sequence ``block_table`` of physical block ids.

Draw order for a seed is fixed: lengths -> block permutation -> q -> k -> v.
Values are ``standard_normal(float32)`` rounded to bf16 (round to nearest even,
as torch's CPU cast does).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

__all__ = [
    "Workload", "CONFIGS", "make_config", "make_custom", "make_append", "append_config", "make_padded",
    "alibi_slopes",
    "PADDED", "normal_bf16",
    "lengths_for", "C4_TOTAL",
]

# Tensors above this many elements are drawn in parallel chunks, each from a
# child generator seeded from the parent stream (deterministic for a seed).
_CHUNK = 1 << 24
C4_TOTAL = 65536


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


TORCH_DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16}


def normal_bf16(rng: np.random.Generator, shape: Sequence[int], dtype: str = "bf16") -> torch.Tensor:
    """N(0,1) float32 draws rounded (nearest even) to bf16, or to fp16 with
    ``dtype="f16"``, shape ``shape`` (CPU tensor).  The draws do not depend on dtype."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = torch.empty(n, dtype=TORCH_DTYPES[dtype])
    if n <= _CHUNK:
        if n:
            out.copy_(torch.from_numpy(rng.standard_normal(n, dtype=np.float32)))
        return out.reshape(shape)
    nchunks = (n + _CHUNK - 1) // _CHUNK
    seeds = rng.integers(0, 2**63 - 1, size=nchunks, dtype=np.int64)

    def fill(c: int) -> None:
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        g = np.random.Generator(np.random.PCG64(int(seeds[c])))
        buf = g.standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi].copy_(torch.from_numpy(buf))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


@dataclass
class Workload:
    """One call's inputs on the host.  ``k``/``v`` are rank 3 (non-paged) or rank 4 (paged)."""

    name: str
    seed: int
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    cu_seqlens_q: np.ndarray
    cu_seqlens_k: np.ndarray
    block_table: Optional[np.ndarray]
    page_block_size: int
    softmax_scale: float
    window_left: int
    window_right: int
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.cu_seqlens_q.shape[0] - 1)

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    @property
    def lens_q(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_q.astype(np.int64))

    @property
    def lens_k(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_k.astype(np.int64))

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_heads_k(self) -> int:
        return int(self.k.shape[-2])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[2])


def _cu(lens: Sequence[int]) -> np.ndarray:
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    assert cu[-1] < 2**31
    return cu.astype(np.int32)


def _f32(x: float) -> float:
    return float(np.float32(x))


def _c4_lengths(rng: np.random.Generator, batch: int = 8, lo: int = 1024, hi: int = 16384,
                total: int = C4_TOTAL) -> List[int]:
    """Log-uniform lengths in [lo, hi] rescaled so they sum to exactly ``total``.

    Draw x_i = exp(U(ln lo, ln hi)); bisect a scale s so that
    sum(clip(round(s*x_i), lo, hi)) hits ``total``; put any residual on the
    largest length that is not clamped.
    """
    x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=batch))

    def tot(s: float) -> np.ndarray:
        return np.clip(np.round(s * x), lo, hi).astype(np.int64)

    a, b = 1e-6, 1e6
    for _ in range(200):
        mid = math.sqrt(a * b)
        if tot(mid).sum() < total:
            a = mid
        else:
            b = mid
    L = tot(b)
    resid = total - int(L.sum())
    order = np.argsort(-L, kind="stable")
    for idx in order:
        if resid == 0:
            break
        nv = int(np.clip(L[idx] + resid, lo, hi))
        resid -= nv - int(L[idx])
        L[idx] = nv
    assert int(L.sum()) == total, (L, total)
    return [int(v) for v in L]


# Config table: the five workloads (plus the head_dim-512 MQA variant of the
# large-head decode) with the shapes the problem statement gives for them.
CONFIGS = {
    "c1": dict(desc="non-paged varlen causal, seqlens {17,64,5}, H4/Hk2, D64",
               num_heads=4, num_heads_k=2, head_dim=64, page=0, width=0,
               window_left=-1, window_right=0, scale=1.0 / 8.0),
    "c2": dict(desc="paged decode, 64 seqs, q_len 1, kv U[1,4096], P32, H32/Hk8, D128",
               num_heads=32, num_heads_k=8, head_dim=128, page=32, width=128,
               window_left=-1, window_right=0, scale=1.0 / math.sqrt(128)),
    "c3": dict(desc="paged chunked prefill, 16 seqs, q U[1,512], prefix U[0,8192], P64, H32/Hk8, D128",
               num_heads=32, num_heads_k=8, head_dim=128, page=64, width=136,
               window_left=-1, window_right=0, scale=1.0 / math.sqrt(128)),
    "c4": dict(desc="non-paged long prefill, 8 seqs log-uniform [1024,16384] sum 65536, H64/Hk8, D128, window_left 4096",
               num_heads=64, num_heads_k=8, head_dim=128, page=0, width=0,
               window_left=4096, window_right=0, scale=1.0 / math.sqrt(128)),
    "c5a": dict(desc="paged spec-decode, 32 seqs, q_len 4, kv U[1024,32768], P128, D256, H16/Hk16",
                num_heads=16, num_heads_k=16, head_dim=256, page=128, width=256,
                window_left=-1, window_right=0, scale=1.0 / math.sqrt(256)),
    "c5b": dict(desc="paged spec-decode MQA, 32 seqs, q_len 4, kv U[1024,32768], P128, D512, H16/Hk1",
                num_heads=16, num_heads_k=1, head_dim=512, page=128, width=256,
                window_left=-1, window_right=0, scale=1.0 / math.sqrt(512)),
}

DEFAULT_SEEDS = {"c1": 1001, "c2": 1002, "c3": 1003, "c4": 1004, "c5a": 1005, "c5b": 1005}


def lengths_for(name: str, rng: np.random.Generator):
    """(lens_q, lens_k) for a config, drawn first from ``rng``."""
    if name == "c1":
        L = [17, 64, 5]
        return L, list(L)
    if name == "c2":
        lk = rng.integers(1, 4096, size=64, endpoint=True)
        return [1] * 64, [int(x) for x in lk]
    if name == "c3":
        lq = rng.integers(1, 512, size=16, endpoint=True)
        pre = rng.integers(0, 8192, size=16, endpoint=True)
        return [int(x) for x in lq], [int(a + b) for a, b in zip(lq, pre)]
    if name == "c4":
        L = _c4_lengths(rng)
        return L, list(L)
    if name in ("c5a", "c5b"):
        lk = rng.integers(1024, 32768, size=32, endpoint=True)
        return [4] * 32, [int(x) for x in lk]
    raise KeyError(name)


def make_custom(lens_q: Sequence[int], lens_k: Sequence[int], num_heads: int, num_heads_k: int,
                head_dim: int, *, seed: int = 0, page: int = 0, width: int = 0,
                window_left: int = -1, window_right: int = 0, scale: Optional[float] = None,
                spare: float = 0.1, poison: bool = False, rng: Optional[np.random.Generator] = None,
                name: str = "custom", dtype: str = "bf16") -> Workload:
    """Build a workload from explicit lengths.

    ``page > 0`` makes a paged pool of ``ceil((1+spare) * sum(ceil(Lk/page)))``
    blocks (at least one); sequence b takes the next ``ceil(Lk_b/page)`` ids of a
    random permutation.  ``width`` is the block_table width (0 = the smallest
    that fits).  With ``poison`` the spare blocks and the slots past each
    sequence's last token hold NaN and unused block_table entries are -1, so any
    stray read shows up in the output.
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    lens_q = [int(x) for x in lens_q]
    lens_k = [int(x) for x in lens_k]
    assert len(lens_q) == len(lens_k)
    batch = len(lens_q)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    total_q = sum(lens_q)
    total_k = sum(lens_k)
    block_table = None
    if page > 0:
        pages = [(lk + page - 1) // page for lk in lens_k]
        need = sum(pages)
        num_blocks = max(1, int(math.ceil((1.0 + spare) * need)))
        w = max([1] + pages) if width <= 0 else width
        assert w >= max([0] + pages), "block_table width too small"
        perm = rng.permutation(num_blocks).astype(np.int32)
        bt = np.full((batch, w), -1 if poison else 0, dtype=np.int32)
        pos = 0
        for b, np_ in enumerate(pages):
            bt[b, :np_] = perm[pos:pos + np_]
            pos += np_
        block_table = bt
        q = normal_bf16(rng, (total_q, num_heads, head_dim), dtype)
        k = normal_bf16(rng, (num_blocks, page, num_heads_k, head_dim), dtype)
        v = normal_bf16(rng, (num_blocks, page, num_heads_k, head_dim), dtype)
        if poison:
            used = np.zeros((num_blocks, page), dtype=bool)
            for b in range(batch):
                for j in range(lens_k[b]):
                    used[bt[b, j // page], j % page] = True
            mask = torch.from_numpy(~used)
            k[mask] = float("nan")
            v[mask] = float("nan")
    else:
        q = normal_bf16(rng, (total_q, num_heads, head_dim), dtype)
        k = normal_bf16(rng, (total_k, num_heads_k, head_dim), dtype)
        v = normal_bf16(rng, (total_k, num_heads_k, head_dim), dtype)
    return Workload(name=name, seed=seed, q=q, k=k, v=v, cu_seqlens_q=_cu(lens_q),
                    cu_seqlens_k=_cu(lens_k), block_table=block_table, page_block_size=page,
                    softmax_scale=_f32(scale), window_left=int(window_left),
                    window_right=int(window_right))


def make_append(lens_new: Sequence[int], lens_k: Sequence[int], num_heads_k: int, head_dim: int, *,
                page: int, seed: int = 0, width: int = 0, spare: float = 0.1):
    """Inputs of a paged K/V append: a random pool (as ``make_custom`` builds it)
    plus new rows.  Returns (wl, k_new, v_new, cu_seqlens_new); ``wl.q`` is k_new
    (its head count is num_heads_k), ``wl.cu_seqlens_k`` counts keys after the append.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    wl = make_custom(lens_new, lens_k, num_heads_k, num_heads_k, head_dim, page=page, width=width,
                     spare=spare, rng=rng, seed=seed, name="append")
    v_new = normal_bf16(rng, tuple(wl.q.shape))
    return wl, wl.q, v_new, wl.cu_seqlens_q


def alibi_slopes(num_heads: int, batch: int = 0, seed: Optional[int] = None) -> np.ndarray:
    """ALiBi slopes as float32: (num_heads,), or (batch, num_heads) when batch > 0.
    Without a seed, the geometric sequence 2^(-8 h / num_heads), h = 1..num_heads, of
    the ALiBi paper (Press et al., 2022); with a seed, uniform draws in [0, 1)."""
    if seed is None:
        s = 2.0 ** (-8.0 * np.arange(1, num_heads + 1) / num_heads)
        out = np.tile(s, (batch, 1)) if batch > 0 else s
    else:
        rng = np.random.Generator(np.random.PCG64(seed))
        out = rng.random((batch, num_heads) if batch > 0 else (num_heads,))
    return np.ascontiguousarray(out, dtype=np.float32)


def make_padded(B: int, Sq: int, Sk: int, num_heads: int, num_heads_k: int, head_dim: int, *,
                seed: int = 0, layout: str = "bshd", dtype: str = "bf16"):
    """Padded inputs q (B, Sq, H, D), k/v (B, Sk, Hk, D) bf16, drawn q, k, v in that
    order.  ``layout="bhsd"`` draws them head-major, (B, H, S, D) contiguous, and
    returns (B, S, H, D) views of those (strided, not mergeable into tokens)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if layout == "bhsd":
        q = normal_bf16(rng, (B, num_heads, Sq, head_dim), dtype).transpose(1, 2)
        k = normal_bf16(rng, (B, num_heads_k, Sk, head_dim), dtype).transpose(1, 2)
        v = normal_bf16(rng, (B, num_heads_k, Sk, head_dim), dtype).transpose(1, 2)
    else:
        q = normal_bf16(rng, (B, Sq, num_heads, head_dim), dtype)
        k = normal_bf16(rng, (B, Sk, num_heads_k, head_dim), dtype)
        v = normal_bf16(rng, (B, Sk, num_heads_k, head_dim), dtype)
    return q, k, v


# Padded (non-varlen) workloads, batch-major with uniform lengths: the long-prefill
# batch at a uniform length, and a decode batch at a uniform cache length.
PADDED = {
    "p4": dict(desc="padded prefill (8, 8192) H64/Hk8 D128, causal, window_left 4096",
               B=8, Sq=8192, Sk=8192, num_heads=64, num_heads_k=8, head_dim=128, window_left=4096,
               window_right=0, seed=1004),
    "p2": dict(desc="padded decode (64, q 1, kv 4096) H32/Hk8 D128",
               B=64, Sq=1, Sk=4096, num_heads=32, num_heads_k=8, head_dim=128, window_left=-1,
               window_right=0, seed=1002),
}


def append_config(name: str, seed: Optional[int] = None, dtype: str = "bf16") -> Workload:
    """Paged workload whose last ``lens_q[b]`` keys per sequence are the tokens an
    append writes.  Paged configs are used as they are; the long-prefill config
    (non-paged) gets a page-64 pool holding its whole sequences (Lq = Lk), and
    its ``q`` has num_heads_k heads (the new K rows' shape)."""
    cfg = CONFIGS[name]
    if cfg["page"] > 0:
        return make_config(name, seed, dtype=dtype)
    seed = DEFAULT_SEEDS[name] if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    lens_q, lens_k = lengths_for(name, rng)
    wl = make_custom(lens_q, lens_k, cfg["num_heads_k"], cfg["num_heads_k"], cfg["head_dim"], seed=seed,
                     page=64, rng=rng, name=name + "-paged", dtype=dtype)
    wl.extra["desc"] = cfg["desc"].replace("non-paged", "paged (P64)")
    return wl


def make_config(name: str, seed: Optional[int] = None, *, poison: bool = False, dtype: str = "bf16") -> Workload:
    """The named workload (``c1`` ... ``c5b``) for ``seed`` (default: its timing seed)."""
    cfg = CONFIGS[name]
    if seed is None:
        seed = DEFAULT_SEEDS[name]
    rng = np.random.Generator(np.random.PCG64(seed))
    lens_q, lens_k = lengths_for(name, rng)
    wl = make_custom(lens_q, lens_k, cfg["num_heads"], cfg["num_heads_k"], cfg["head_dim"],
                     seed=seed, page=cfg["page"], width=cfg["width"],
                     window_left=cfg["window_left"], window_right=cfg["window_right"],
                     scale=cfg["scale"], poison=poison, rng=rng, name=name, dtype=dtype)
    wl.extra["desc"] = cfg["desc"]
    return wl
