"""Seeded input generator: determinism and the shapes each workload promises."""
import numpy as np
import torch

import workloads as W


def test_same_seed_same_inputs():
    a = W.make_config("c3", seed=1)
    b = W.make_config("c3", seed=1)
    assert torch.equal(a.q.view(torch.int16), b.q.view(torch.int16))
    assert torch.equal(a.k.view(torch.int16), b.k.view(torch.int16))
    assert np.array_equal(a.block_table, b.block_table)
    c = W.make_config("c3", seed=2)
    assert not np.array_equal(a.cu_seqlens_k, c.cu_seqlens_k)


def test_large_tensors_are_deterministic():
    g1 = np.random.Generator(np.random.PCG64(5))
    g2 = np.random.Generator(np.random.PCG64(5))
    x = W.normal_bf16(g1, (3, W._CHUNK + 17))
    y = W.normal_bf16(g2, (3, W._CHUNK + 17))
    assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert abs(float(x.float().mean())) < 1e-3 and abs(float(x.float().std()) - 1) < 1e-3


def test_config_shapes():
    c1 = W.make_config("c1")
    assert list(c1.lens_q) == [17, 64, 5] and list(c1.lens_k) == [17, 64, 5]
    assert c1.q.shape == (86, 4, 64) and c1.k.shape == (86, 2, 64) and not c1.paged
    assert c1.softmax_scale == 0.125 and (c1.window_left, c1.window_right) == (-1, 0)
    c2 = W.make_config("c2")
    assert c2.batch == 64 and set(c2.lens_q) == {1}
    assert c2.lens_k.min() >= 1 and c2.lens_k.max() <= 4096
    assert c2.block_table.shape == (64, 128) and c2.k.shape[1:] == (32, 8, 128)
    need = int(sum((c2.lens_k + 31) // 32))
    assert c2.k.shape[0] == int(np.ceil(1.1 * need))
    used = np.concatenate([c2.block_table[b, :(c2.lens_k[b] + 31) // 32] for b in range(64)])
    assert len(set(used.tolist())) == len(used)      # distinct physical blocks
    c3 = W.make_config("c3")
    assert c3.lens_q.min() >= 1 and c3.lens_q.max() <= 512
    pre = c3.lens_k - c3.lens_q
    assert pre.min() >= 0 and pre.max() <= 8192 and c3.block_table.shape == (16, 136)


def test_c4_lengths_sum_and_range():
    for seed in (1004, 1, 2, 3):
        rng = np.random.Generator(np.random.PCG64(seed))
        lq, lk = W.lengths_for("c4", rng)
        assert sum(lq) == W.C4_TOTAL and lq == lk and len(lq) == 8
        assert min(lq) >= 1024 and max(lq) <= 16384


def test_c5_lengths():
    rng = np.random.Generator(np.random.PCG64(1005))
    lq, lk = W.lengths_for("c5a", rng)
    assert lq == [4] * 32 and min(lk) >= 1024 and max(lk) <= 32768


def test_poison_marks_unused_slots():
    w = W.make_custom([1, 2], [33, 64], 2, 1, 8, seed=3, page=32, poison=True)
    assert (w.block_table[0, 2:] == -1).all() and (w.block_table[1, 2:] == -1).all()
    blk = w.block_table[0, 1]
    assert torch.isnan(w.k[blk, 1:].float()).all() and not torch.isnan(w.k[blk, 0].float()).any()
