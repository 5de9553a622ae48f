"""Pins for the oracle's paged K/V append (the write that precedes paged attention).

Round trip: take a paged workload, poison the slots of each sequence's last
Lnew keys with NaN, append those keys' true rows (gathered here by plain
indexing of the block table) and compare the whole pool bit-exactly with the
original; then the attention oracle on the rebuilt pool equals the one on the
original.  This fixes the position rule (new tokens are the last Lnew keys of
Lk), the page/slot mapping and that no other slot is touched.
"""
import numpy as np
import torch

import workloads as W


def _split_new(wl, lnew):
    """Rows of each sequence's last lnew[b] keys, gathered from the pool, and a poisoned pool."""
    P = wl.page_block_size
    k_rows, v_rows = [], []
    kp = wl.k.clone()
    vp = wl.v.clone()
    for b in range(wl.batch):
        lk = int(wl.lens_k[b])
        for pos in range(lk - lnew[b], lk):
            blk, slot = wl.block_table[b, pos // P], pos % P
            k_rows.append(wl.k[blk, slot].clone())
            v_rows.append(wl.v[blk, slot].clone())
            kp[blk, slot] = float("nan")
            vp[blk, slot] = float("nan")
    Hk, D = wl.num_heads_k, wl.head_dim
    k_new = torch.stack(k_rows) if k_rows else torch.zeros(0, Hk, D, dtype=torch.bfloat16)
    v_new = torch.stack(v_rows) if v_rows else torch.zeros(0, Hk, D, dtype=torch.bfloat16)
    cu_new = np.zeros(wl.batch + 1, np.int32)
    cu_new[1:] = np.cumsum(lnew)
    return k_new, v_new, cu_new, kp, vp


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_round_trip_restores_pool_bit_exact(oracle_mod):
    wl = W.make_custom([3, 1, 20, 5, 0], [70, 33, 200, 5, 9], 4, 2, 64, seed=21, page=32, spare=0.3)
    lnew = [3, 1, 20, 5, 0]
    k_new, v_new, cu_new, kp, vp = _split_new(wl, lnew)
    assert np.isnan(kp.float().numpy()).any()
    k2, v2 = oracle_mod.kv_append(k_new, v_new, cu_new, wl.cu_seqlens_k, wl.block_table, kp, vp)
    assert np.array_equal(k2, bits(wl.k)) and np.array_equal(v2, bits(wl.v))


def test_round_trip_attention_unchanged(oracle_mod):
    wl = W.make_custom([1, 4, 2], [40, 130, 64], 8, 2, 32, seed=22, page=64)
    k_new, v_new, cu_new, kp, vp = _split_new(wl, [1, 4, 2])
    k2, v2 = oracle_mod.kv_append(k_new, v_new, cu_new, wl.cu_seqlens_k, wl.block_table, kp, vp)
    wl2 = W.Workload(name="rebuilt", seed=0, q=wl.q,
                     k=torch.from_numpy(k2.view(np.int16)).view(torch.bfloat16).reshape(wl.k.shape),
                     v=torch.from_numpy(v2.view(np.int16)).view(torch.bfloat16).reshape(wl.v.shape),
                     cu_seqlens_q=wl.cu_seqlens_q, cu_seqlens_k=wl.cu_seqlens_k,
                     block_table=wl.block_table, page_block_size=64, softmax_scale=wl.softmax_scale,
                     window_left=-1, window_right=0)
    o1, l1 = oracle_mod.attention_workload(wl)
    o2, l2 = oracle_mod.attention_workload(wl2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_rejects_positions_outside_table(oracle_mod):
    wl = W.make_custom([2], [40], 2, 1, 16, seed=23, page=32)
    k_new = wl.k[0, :2].clone()
    cu_new = np.array([0, 2], np.int32)
    bad_cu_k = np.array([0, 1], np.int32)   # fewer keys than new tokens -> negative position
    try:
        oracle_mod.kv_append(k_new, k_new, cu_new, bad_cu_k, wl.block_table, wl.k, wl.v)
    except ValueError:
        return
    raise AssertionError("expected a rejection")
