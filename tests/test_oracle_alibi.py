"""Pins for the oracle's ALiBi term: key j of query row i gets -slope * |a - j|
(a = i + Lk - Lq) added to its scaled score.

Checked against torch fp64 SDPA with the bias passed as a float attention mask
(a library routine), against a geometric-series closed form, and for zero
slopes against the plain call (bit-exact)."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from test_oracle_pins import lib_mask


def sdpa_alibi(wl, slopes):
    H, Hk = wl.num_heads, wl.num_heads_k
    G = H // Hk
    out = np.zeros((wl.q.shape[0], H, wl.head_dim))
    valid = np.zeros(wl.q.shape[0], bool)
    for b in range(wl.batch):
        q0, q1 = int(wl.cu_seqlens_q[b]), int(wl.cu_seqlens_q[b + 1])
        Lq, Lk = q1 - q0, int(wl.lens_k[b])
        if wl.paged:
            P = wl.page_block_size
            kb = torch.stack([wl.k[wl.block_table[b, j // P], j % P] for j in range(Lk)])
            vb = torch.stack([wl.v[wl.block_table[b, j // P], j % P] for j in range(Lk)])
        else:
            k0 = int(wl.cu_seqlens_k[b])
            kb, vb = wl.k[k0:k0 + Lk], wl.v[k0:k0 + Lk]
        mask = lib_mask(Lq, Lk, wl.window_left, wl.window_right)
        ok = mask.any(dim=1)
        valid[q0:q1] = ok.numpy()
        sl = torch.as_tensor(np.asarray(slopes, np.float64).reshape(-1, H)[b if np.ndim(slopes) == 2 else 0])
        a = torch.arange(Lq, dtype=torch.float64)[:, None] + Lk - Lq
        dist = (a - torch.arange(Lk, dtype=torch.float64)[None, :]).abs()
        bias = -sl[:, None, None] * dist[None]                        # H, Lq, Lk
        bias = bias.masked_fill(~mask[None], float("-inf"))
        qh = wl.q[q0:q1].double().permute(1, 0, 2)
        kh = kb.double().repeat_interleave(G, dim=1).permute(1, 0, 2)
        vh = vb.double().repeat_interleave(G, dim=1).permute(1, 0, 2)
        rows = ok.nonzero().flatten()
        o = torch.nn.functional.scaled_dot_product_attention(qh[:, rows], kh, vh, attn_mask=bias[:, rows],
                                                             scale=float(wl.softmax_scale))
        out[q0 + rows.numpy()] = o.permute(1, 0, 2).numpy()
    return out, valid


CASES = [
    # lens_q, lens_k, H, Hk, D, page, wl, wr, per-batch slopes
    ([17, 64, 5], [17, 64, 5], 4, 2, 32, 0, -1, 0, False),
    ([1, 3, 2], [40, 130, 64], 8, 2, 32, 32, -1, 0, True),
    ([9, 30], [40, 30], 4, 4, 16, 0, 6, 3, False),
    ([12, 7], [12, 20], 2, 1, 8, 0, -1, -1, True),
]


@pytest.mark.parametrize("case", CASES)
def test_matches_torch_sdpa_with_bias(oracle_mod, case):
    lq, lk, H, Hk, D, P, wl_, wr_, per_batch = case
    wl = W.make_custom(lq, lk, H, Hk, D, seed=41, page=P, window_left=wl_, window_right=wr_)
    slopes = W.alibi_slopes(H, batch=len(lq) if per_batch else 0, seed=42 if per_batch else None)
    out, _ = oracle_mod.attention_workload(wl, alibi_slopes=slopes)
    ref, valid = sdpa_alibi(wl, slopes)
    assert np.abs(out[valid] - ref[valid]).max() < 1e-12
    assert (out[~valid] == 0).all()


def test_zero_slopes_equal_plain_call(oracle_mod):
    wl = W.make_custom([5, 9], [30, 9], 4, 2, 32, seed=43)
    o1, l1 = oracle_mod.attention_workload(wl)
    o2, l2 = oracle_mod.attention_workload(wl, alibi_slopes=np.zeros(4, np.float32))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_geometric_series_closed_form(oracle_mod):
    """Q = 0, one causal query over n keys: weights e^{-s d}, d = 0..n-1 (distance
    from the last key), so lse = log((1 - e^{-s n}) / (1 - e^{-s})) and, with
    v_j = j, out = sum_d (n-1-d) e^{-s d} / sum_d e^{-s d}."""
    n, s = 50, 0.25
    q = torch.zeros(1, 1, 8, dtype=torch.bfloat16)
    k = torch.zeros(n, 1, 8, dtype=torch.bfloat16)
    v = torch.arange(n, dtype=torch.float32)[:, None, None].expand(n, 1, 8).to(torch.bfloat16)
    out, lse = oracle_mod.attention(q, k, v, np.array([0, 1], np.int32), np.array([0, n], np.int32),
                                    softmax_scale=1.0, window_left=-1, window_right=0,
                                    alibi_slopes=np.array([s], np.float32))
    r = math.exp(-s)
    z = (1 - r ** n) / (1 - r)
    assert abs(lse[0, 0] - math.log(z)) < 1e-12
    # sum_d (n-1-d) r^d = (n-1) z - r (1 - n r^{n-1} + (n-1) r^n) / (1 - r)^2
    num = (n - 1) * z - r * (1 - n * r ** (n - 1) + (n - 1) * r ** n) / (1 - r) ** 2
    assert np.allclose(out[0, 0], num / z, rtol=0, atol=1e-12)
