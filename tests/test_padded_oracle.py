"""Pins for the oracle's padded (batch-major, non-varlen) attention.

The padded entry treats every batch element as one sequence.  Pinned against
torch's batched fp64 scaled_dot_product_attention on (B, H, S, D) tensors with
band masks from ``tril``/``triu`` and ``repeat_interleave``d K/V heads (a
library routine that shares nothing with the oracle's C code), and against the
varlen oracle with uniform cu_seqlens (bit-exact)."""
import numpy as np
import pytest
import torch

import workloads as W


def band(Sq, Sk, wl, wr):
    m = torch.ones(Sq, Sk, dtype=torch.bool)
    if wr >= 0:
        m = m.tril(diagonal=Sk - Sq + wr)
    if wl >= 0:
        m = m.triu(diagonal=Sk - Sq - wl)
    return m


CASES = [
    # B, Sq, Sk, H, Hk, D, wl, wr, layout
    (3, 17, 17, 4, 2, 32, -1, 0, "bshd"),
    (2, 5, 40, 8, 2, 16, -1, 0, "bhsd"),
    (2, 1, 33, 4, 1, 64, -1, -1, "bshd"),
    (4, 12, 9, 2, 2, 8, 3, 2, "bhsd"),
]


@pytest.mark.parametrize("case", CASES)
def test_matches_torch_batched_sdpa(oracle_mod, case):
    B, Sq, Sk, H, Hk, D, wl, wr, layout = case
    q, k, v = W.make_padded(B, Sq, Sk, H, Hk, D, seed=11, layout=layout)
    scale = 0.3
    out, lse = oracle_mod.attention_padded(q, k, v, scale, wl, wr)
    mask = band(Sq, Sk, wl, wr)
    rows_ok = mask.any(dim=1)
    qh = q.double().permute(0, 2, 1, 3)                                   # B, H, Sq, D
    kh = k.double().repeat_interleave(H // Hk, dim=2).permute(0, 2, 1, 3)  # B, H, Sk, D
    vh = v.double().repeat_interleave(H // Hk, dim=2).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=scale)
    ref = ref.permute(0, 2, 1, 3).numpy()
    ok = rows_ok.numpy()
    assert np.abs(out[:, ok] - ref[:, ok]).max() < 1e-12
    assert (out[:, ~ok] == 0).all()
    # lse: log-sum-exp of the masked scaled scores, from torch
    s = torch.einsum("bhqd,bhkd->bhqk", qh, kh) * scale
    s = s.masked_fill(~mask, float("-inf"))
    ref_lse = torch.logsumexp(s, dim=-1).numpy()
    assert np.allclose(lse[:, :, ok], ref_lse[:, :, ok], atol=1e-12, rtol=0)
    assert np.isneginf(lse[:, :, ~ok]).all()


def test_equals_varlen_with_uniform_offsets(oracle_mod):
    B, Sq, Sk, H, Hk, D = 3, 7, 20, 4, 2, 32
    q, k, v = W.make_padded(B, Sq, Sk, H, Hk, D, seed=12, layout="bhsd")
    out, lse = oracle_mod.attention_padded(q, k, v, 0.2, 5, 0)
    o2, l2 = oracle_mod.attention(q.reshape(B * Sq, H, D), k.reshape(B * Sk, Hk, D), v.reshape(B * Sk, Hk, D),
                                  np.arange(B + 1, dtype=np.int32) * Sq, np.arange(B + 1, dtype=np.int32) * Sk,
                                  softmax_scale=0.2, window_left=5, window_right=0)
    assert np.array_equal(out.reshape(B * Sq, H, D), o2)
    assert np.array_equal(lse.transpose(1, 0, 2).reshape(H, B * Sq), l2)
