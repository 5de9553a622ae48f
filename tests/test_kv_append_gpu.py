"""GPU parity of the paged K/V append (fa_kv_append through the C ABI).

The append moves bf16 bits, so the bar is bit-exact: the whole pool after the
HIP append equals the oracle's pool (every slot, written or not).  Small cases
cover each head-dim path (16-byte units and element units), page sizes, empty
sequences, sequences that are all new, strided inputs, the metadata the kernel
skips and batches past the LDS-staged lookup.  The full-size cases append each
workload's query-length worth of tokens into its own pool after poisoning
those slots, and must restore the pool exactly.
"""
import numpy as np
import pytest
import torch

import varlen_flash_attention_fa_amd as fa
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()


def bits(t):
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def run_append(k_new, v_new, cu_new, cu_k, bt, k_pool, v_pool):
    dev = "cuda"
    kp, vp = k_pool.to(dev), v_pool.to(dev)
    fa.kv_append(k_new.to(dev) if k_new.device.type == "cpu" else k_new,
                 v_new.to(dev) if v_new.device.type == "cpu" else v_new,
                 torch.from_numpy(np.ascontiguousarray(cu_new, np.int32)).to(dev),
                 torch.from_numpy(np.ascontiguousarray(cu_k, np.int32)).to(dev),
                 torch.from_numpy(np.ascontiguousarray(bt, np.int32)).to(dev), kp, vp)
    torch.cuda.synchronize()
    return kp, vp


def assert_pool_equal(kp, vp, ref_k, ref_v, what):
    gk, gv = bits(kp), bits(vp)
    bad_k = int((gk != ref_k).sum())
    bad_v = int((gv != ref_v).sum())
    assert bad_k == 0 and bad_v == 0, "%s: %d K and %d V elements differ" % (what, bad_k, bad_v)


CASES = [
    # name, lens_new, lens_k, Hk, D, page
    ("decode-d128-hk8", [1] * 9, [1, 31, 32, 33, 255, 256, 257, 1000, 2100], 8, 128, 32),
    ("chunk-d128-p64", [130, 5, 64, 1, 0], [700, 5, 300, 64, 12], 8, 128, 64),
    ("all-new-d64", [40, 100], [40, 100], 2, 64, 32),
    ("spec-d256-p128", [4, 4, 4], [1030, 2049, 4], 16, 256, 128),
    ("mqa-d512", [4, 1, 7], [1100, 2500, 300], 1, 512, 128),
    ("odd-d13", [33, 5], [40, 5], 2, 13, 32),
    ("odd-d100", [70, 1], [90, 600], 1, 100, 64),
    ("d40-hk3", [3, 9], [77, 300], 3, 40, 32),
]


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[c[0] for c in CASES])
def test_small_cases_bit_exact(oracle_mod, idx):
    name, ln, lk, Hk, D, P = CASES[idx]
    wl, k_new, v_new, cu_new = W.make_append(ln, lk, Hk, D, page=P, seed=300 + idx)
    print("case", name, flush=True)
    kp, vp = run_append(k_new, v_new, cu_new, wl.cu_seqlens_k, wl.block_table, wl.k, wl.v)
    rk, rv = oracle_mod.kv_append(k_new, v_new, cu_new, wl.cu_seqlens_k, wl.block_table, wl.k, wl.v)
    assert not np.array_equal(rk, bits(wl.k)) or sum(ln) == 0
    assert_pool_equal(kp, vp, rk, rv, name)


def test_strided_inputs(oracle_mod):
    """k_new/v_new as views with padded token and head strides; pools with a padded slot stride."""
    ln, lk, Hk, D, P = [5, 17], [60, 17], 2, 64, 32
    wl, k_new, v_new, cu_new = W.make_append(ln, lk, Hk, D, page=P, seed=7)
    big_k = torch.zeros(k_new.shape[0], Hk + 1, D + 8, dtype=torch.bfloat16)
    big_v = torch.zeros_like(big_k)
    big_k[:, :Hk, :D] = k_new
    big_v[:, :Hk, :D] = v_new
    dev = "cuda"
    pk = torch.zeros(wl.k.shape[0], P, Hk + 2, D, dtype=torch.bfloat16)
    pv = torch.zeros_like(pk)
    pk[:, :, :Hk] = wl.k
    pv[:, :, :Hk] = wl.v
    pk_d, pv_d = pk.to(dev), pv.to(dev)
    kd, vd = pk_d[:, :, :Hk], pv_d[:, :, :Hk]
    assert not kd.is_contiguous()
    fa.kv_append(big_k.to(dev)[:, :Hk, :D], big_v.to(dev)[:, :Hk, :D],
                 torch.from_numpy(cu_new).to(dev), torch.from_numpy(wl.cu_seqlens_k).to(dev),
                 torch.from_numpy(wl.block_table).to(dev), kd, vd)
    torch.cuda.synchronize()
    rk, rv = oracle_mod.kv_append(k_new, v_new, cu_new, wl.cu_seqlens_k, wl.block_table, wl.k, wl.v)
    assert_pool_equal(kd, vd, rk, rv, "strided")
    # the padding heads stay zero
    assert not bits(pk_d[:, :, Hk:]).any()


def test_skipped_metadata(oracle_mod):
    """Tokens at negative positions, past the table, or on block ids outside the pool are skipped."""
    ln, lk, Hk, D, P = [3, 2, 4, 2], [50, 40, 70, 33], 2, 64, 32
    wl, k_new, v_new, cu_new = W.make_append(ln, lk, Hk, D, page=P, seed=8, width=3)
    cu_k = wl.cu_seqlens_k.copy()
    bt = wl.block_table.copy()
    # sequence 1: two new tokens but only one key -> the first lands at position -1
    cu_k[2:] -= 39
    # sequence 2: 70 keys in a table of width 3 (96 slots) but the last block id is out of the pool
    bt[2, 2] = wl.k.shape[0] + 5
    # sequence 3: the block holding its new keys is -1
    bt[3, 1] = -1
    kp, vp = run_append(k_new, v_new, cu_new, cu_k, bt, wl.k, wl.v)
    with pytest.raises(ValueError):
        oracle_mod.kv_append(k_new, v_new, cu_new, cu_k, bt, wl.k, wl.v)
    # the oracle writes every valid token and skips the rest
    rk, rv = oracle_mod.kv_append(k_new, v_new, cu_new, cu_k, bt, wl.k, wl.v, strict=False)
    assert_pool_equal(kp, vp, rk, rv, "skipped metadata")


@pytest.mark.parametrize("batch", [255, 256, 600, 2047, 2600])
def test_batch_sizes_each_lookup(oracle_mod, batch):
    """Offsets staged one per lane (batch + 1 <= 256), eight per lane (<= 2048), or
    searched in global memory (larger batches)."""
    rng = np.random.Generator(np.random.PCG64(batch))
    ln = rng.integers(0, 3, batch).tolist()
    lk = [int(a) + int(b) for a, b in zip(ln, rng.integers(0, 70, batch))]
    wl, k_new, v_new, cu_new = W.make_append(ln, lk, 1, 64, page=32, seed=batch)
    kp, vp = run_append(k_new, v_new, cu_new, wl.cu_seqlens_k, wl.block_table, wl.k, wl.v)
    rk, rv = oracle_mod.kv_append(k_new, v_new, cu_new, wl.cu_seqlens_k, wl.block_table, wl.k, wl.v)
    assert_pool_equal(kp, vp, rk, rv, "batch %d" % batch)


def test_empty_calls_write_nothing():
    wl, k_new, v_new, cu_new = W.make_append([0, 0], [5, 9], 2, 64, page=32, seed=10)
    kp, vp = run_append(k_new, v_new, cu_new, wl.cu_seqlens_k, wl.block_table, wl.k, wl.v)
    assert np.array_equal(bits(kp), bits(wl.k)) and np.array_equal(bits(vp), bits(wl.v))


def _last_key_rows(wl, lnew):
    """Flat pool rows (block * P + slot) of each sequence's last lnew[b] keys."""
    P = wl.page_block_size
    lk = wl.lens_k
    rows = []
    for b in range(wl.batch):
        pos = np.arange(lk[b] - lnew[b], lk[b])
        rows.append(wl.block_table[b, pos // P].astype(np.int64) * P + pos % P)
    return np.concatenate(rows) if rows else np.zeros(0, np.int64)


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5a", "c5b"])
def test_full_size_round_trip(name):
    """Each workload appends its own query-length worth of tokens (its last keys);
    the long-prefill batch writes its whole sequences into a page-64 pool."""
    wl = W.append_config(name)
    print("round trip", name, flush=True)
    lnew = wl.lens_q
    rows = torch.from_numpy(_last_key_rows(wl, lnew)).cuda()
    dev = "cuda"
    k0, v0 = wl.k.to(dev), wl.v.to(dev)
    Hk, D = k0.shape[2], k0.shape[3]
    kflat, vflat = k0.view(-1, Hk, D), v0.view(-1, Hk, D)
    k_new, v_new = kflat[rows].clone(), vflat[rows].clone()
    kp, vp = k0.clone(), v0.clone()
    kp.view(-1, Hk, D)[rows] = float("nan")
    vp.view(-1, Hk, D)[rows] = float("nan")
    fa.kv_append(k_new, v_new, torch.from_numpy(wl.cu_seqlens_q).to(dev),
                 torch.from_numpy(wl.cu_seqlens_k).to(dev), torch.from_numpy(wl.block_table).to(dev),
                 kp, vp)
    torch.cuda.synchronize()
    assert torch.equal(kp.view(torch.int16), k0.view(torch.int16)), name + ": K pool differs"
    assert torch.equal(vp.view(torch.int16), v0.view(torch.int16)), name + ": V pool differs"
