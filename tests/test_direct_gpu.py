"""GPU parity of direct calls: a call with at most 16 sequences whose keys are not
split into chunks runs without the planner -- its attention workgroups cover
(sequence, row tile, K/V head) and read their sequence's offsets themselves.

Each case runs once as a direct call and once with FA_DIRECT=0 (the planner's
work list); the two must give the same bits (the work items are the same, only
their source differs), and the direct result must meet the oracle bar of
tests/test_parity_gpu.py (bf16/fp16 out max |d| <= 2e-2, mean |d| <= 2e-3, lse
within parity_util.lse_bound).  Cases: empty sequences (no queries, no keys),
all queries in one sequence (every other sequence's workgroups exit), 16
sequences at the largest direct grid, both kernel paths, head dims 64 to 512,
fp16, paged K/V, windows, ALiBi and the padded entry.
"""
import numpy as np
import pytest
import torch

import varlen_flash_attention_fa_amd as fa
import workloads as W
from parity_util import assert_close, run_hip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()


def _same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def _both(monkeypatch, fn):
    monkeypatch.delenv("FA_DIRECT", raising=False)
    direct = fn()
    monkeypatch.setenv("FA_DIRECT", "0")
    planned = fn()
    monkeypatch.delenv("FA_DIRECT")
    return direct, planned


CASES = [
    # name, lens_q, lens_k, H, Hk, D, page, wl, wr, dtype
    ("prefill-empty-seqs", [0, 37, 300, 5, 0], [10, 37, 500, 0, 64], 8, 2, 128, 0, -1, 0, "bf16"),
    ("prefill-empty-seqs-paged", [0, 37, 300, 5, 0], [10, 37, 500, 0, 64], 8, 2, 128, 32, -1, 0, "bf16"),
    ("one-seq-holds-all-rows", [0, 0, 257, 0], [3, 0, 300, 7], 4, 2, 64, 32, -1, 0, "bf16"),
    ("sixteen-seqs", [64] * 16, [64] * 16, 8, 8, 128, 0, -1, 0, "bf16"),
    ("decode-kind-wr1", [1] * 12, [1, 2, 31, 32, 33, 100, 255, 256, 257, 400, 511, 512], 32, 8, 128, 32, -1, 0, "bf16"),
    ("decode-kind-wr4", [8, 8, 8, 8], [20, 300, 8, 512], 16, 4, 128, 64, -1, 0, "bf16"),
    ("prefill-window-f16", [200, 33, 90], [200, 33, 150], 4, 4, 64, 0, 40, 0, "f16"),
    ("prefill-d256-two-sided", [70, 130], [90, 130], 4, 2, 256, 32, 7, 5, "bf16"),
    ("decode-d512-mqa", [4, 4, 4], [300, 17, 512], 16, 1, 512, 128, -1, 0, "bf16"),
    ("prefill-noncausal-odd-d", [33, 5, 61], [40, 5, 61], 4, 2, 13, 0, -1, -1, "bf16"),
]


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[c[0] for c in CASES])
def test_direct_matches_planner_and_oracle(oracle_mod, monkeypatch, idx):
    name, lq, lk, H, Hk, D, P, wl_, wr_, dt = CASES[idx]
    print("case", name, flush=True)
    wl = W.make_custom(lq, lk, H, Hk, D, seed=1200 + idx, page=P, window_left=wl_, window_right=wr_,
                       poison=P > 0, dtype=dt)
    (o_d, l_d), (o_p, l_p) = _both(monkeypatch, lambda: run_hip(wl))
    assert _same_bits(o_d, o_p), name + ": direct and planned outputs differ"
    assert torch.equal(l_d, l_p), name + ": direct and planned lse differ"
    ref_o, ref_l = oracle_mod.attention_workload(wl)
    assert_close(o_d, l_d, ref_o, ref_l, what=name, n_keys=int(max([1] + list(wl.lens_k))))


def test_direct_alibi(oracle_mod, monkeypatch):
    wl = W.make_custom([130, 5, 64], [300, 5, 64], 8, 2, 128, seed=1250, page=64)
    slopes = W.alibi_slopes(8, batch=3, seed=1251)
    d = "cuda"

    def run():
        out, lse = fa.varlen_fwd(wl.q.to(d), wl.k.to(d), wl.v.to(d), torch.from_numpy(wl.cu_seqlens_q).to(d),
                                 torch.from_numpy(wl.cu_seqlens_k).to(d), block_table=torch.from_numpy(wl.block_table).to(d),
                                 page_block_size=wl.page_block_size, softmax_scale=wl.softmax_scale,
                                 window_left=wl.window_left, window_right=wl.window_right, return_lse=True,
                                 alibi_slopes=torch.from_numpy(slopes).to(d))
        torch.cuda.synchronize()
        return out, lse

    (o_d, l_d), (o_p, l_p) = _both(monkeypatch, run)
    assert _same_bits(o_d, o_p) and torch.equal(l_d, l_p)
    ref_o, ref_l = oracle_mod.attention_workload(wl, alibi_slopes=slopes)
    assert_close(o_d, l_d, ref_o, ref_l, what="alibi")


def test_direct_padded(oracle_mod, monkeypatch):
    q, k, v = W.make_padded(3, 70, 90, 8, 2, 128, seed=1260)
    scale = 1.0 / np.sqrt(128)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()

    def run():
        out, lse = fa.padded_fwd(qd, kd, vd, softmax_scale=scale, window_left=-1, window_right=0, return_lse=True)
        torch.cuda.synchronize()
        return out, lse

    (o_d, l_d), (o_p, l_p) = _both(monkeypatch, run)
    assert _same_bits(o_d, o_p) and torch.equal(l_d, l_p)
    ref_o, ref_l = oracle_mod.attention_padded(q, k, v, scale, -1, 0)
    # padded lse is (B, H, Sq): compare as varlen rows (B*Sq, H, D) / (H, B*Sq)
    o = o_d.reshape(3 * 70, 8, 128)
    lse = l_d.permute(1, 0, 2).reshape(8, 3 * 70)
    assert_close(o, lse, ref_o.reshape(3 * 70, 8, 128), np.ascontiguousarray(
        np.transpose(ref_l, (1, 0, 2)).reshape(8, 3 * 70)), what="padded", n_keys=90)
