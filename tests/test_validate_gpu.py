"""GPU tests of the FA_VALIDATE=1 metadata check of fa_varlen_fwd and fa_kv_append.

By default the kernels trust the offsets and the block table (they only clamp
them into the tensors given).  With FA_VALIDATE=1 the library copies them to the
host first and rejects decreasing offsets, offsets past the rows, a sequence with
more keys than its block-table row holds, and a block id outside the pool among
the pages a sequence's keys (appended rows) use -- with FA_ERR_ARGUMENT and no
launch, so the output keeps what it held.  Valid metadata gives the same bits as
without the check.  Every rejected case is rejected on the host: no kernel ever
sees the bad metadata.
"""
import numpy as np
import pytest
import torch

import varlen_flash_attention_fa_amd as fa
import workloads as W
from parity_util import to_dev

pytestmark = pytest.mark.gpu

ARG = 7  # FA_ERR_ARGUMENT


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()


@pytest.fixture()
def validate(monkeypatch):
    monkeypatch.setenv("FA_VALIDATE", "1")


def _paged(poison=False):
    return W.make_custom([1, 5, 3], [70, 200, 33], 8, 2, 128, seed=41, page=32, poison=poison)


def _call(wl, d, cu_q=None, cu_k=None, bt=None, out=None):
    return fa.varlen_fwd(d["q"], d["k"], d["v"], d["cu_q"] if cu_q is None else cu_q,
                         d["cu_k"] if cu_k is None else cu_k, block_table=d["bt"] if bt is None else bt,
                         page_block_size=wl.page_block_size or None, softmax_scale=wl.softmax_scale,
                         window_left=wl.window_left, window_right=wl.window_right, out=out)


def _i32(xs):
    return torch.tensor(xs, dtype=torch.int32, device="cuda")


def _rejected(fn, text):
    with pytest.raises(fa.FlashAttnError) as e:
        fn()
    assert e.value.code == ARG and "FA_VALIDATE" in str(e.value) and text in str(e.value), str(e.value)


@pytest.mark.parametrize("poison", [False, True])
def test_valid_metadata_same_bits(monkeypatch, poison):
    # poisoned tables hold -1 past each sequence's last page: not a used page, so accepted
    wl = _paged(poison)
    d = to_dev(wl)
    ref = _call(wl, d)
    torch.cuda.synchronize()
    monkeypatch.setenv("FA_VALIDATE", "1")
    got = _call(wl, d)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))


def test_decreasing_query_offsets(validate):
    wl = _paged()
    d = to_dev(wl)
    out = torch.full_like(d["q"], 7.0)
    _rejected(lambda: _call(wl, d, cu_q=_i32([0, 4, 1, 9]), out=out), "cu_seqlens_q must be non-decreasing")
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "nothing may be written after a rejected call"


def test_query_offset_past_rows(validate):
    wl = _paged()
    d = to_dev(wl)
    total_q = d["q"].shape[0]
    _rejected(lambda: _call(wl, d, cu_q=_i32([0, 1, 6, total_q + 1])), "entry 3 is %d" % (total_q + 1))


def test_packed_key_offset_past_rows(validate):
    wl = W.make_custom([4, 9], [30, 50], 4, 2, 64, seed=42)
    d = to_dev(wl)
    total_k = d["k"].shape[0]
    _rejected(lambda: _call(wl, d, cu_k=_i32([0, 30, total_k + 5])), "cu_seqlens_k must be non-decreasing")


@pytest.mark.parametrize("bad", [-1, "pool"])
def test_block_id_outside_the_pool(validate, bad):
    wl = _paged()
    d = to_dev(wl)
    bt = d["bt"].clone()
    nblk = d["k"].shape[0]
    bt[1, 5] = nblk if bad == "pool" else -1  # sequence 1 has 200 keys: pages 0..6 are used
    _rejected(lambda: _call(wl, d, bt=bt), "block_table[1][5] = %d is outside the pool of %d blocks"
              % (int(bt[1, 5]), nblk))


def test_more_keys_than_the_table_holds(validate):
    wl = _paged()
    d = to_dev(wl)
    width = d["bt"].shape[1]
    lk = width * 32 + 1
    _rejected(lambda: _call(wl, d, cu_k=_i32([0, 70, 70 + lk, 70 + lk + 33])), "sequence 1 has %d keys" % lk)


# ------------------------------------------------------------------ append

def _append_case():
    return W.make_append([2, 0, 5], [40, 17, 90], 2, 64, page=32, seed=43)


def _append(wl, k_new, v_new, cu_new, cu_k=None, bt=None):
    kp, vp = wl.k.cuda(), wl.v.cuda()
    fa.kv_append(k_new.cuda(), v_new.cuda(), _i32(list(cu_new)),
                 _i32(list(wl.cu_seqlens_k if cu_k is None else cu_k)),
                 torch.from_numpy(np.ascontiguousarray(wl.block_table if bt is None else bt, np.int32)).cuda(), kp, vp)
    torch.cuda.synchronize()
    return kp, vp


def test_append_valid_same_bits(monkeypatch):
    wl, k_new, v_new, cu_new = _append_case()
    ka, va = _append(wl, k_new, v_new, cu_new)
    monkeypatch.setenv("FA_VALIDATE", "1")
    kb, vb = _append(wl, k_new, v_new, cu_new)
    assert torch.equal(ka.view(torch.int16), kb.view(torch.int16))
    assert torch.equal(va.view(torch.int16), vb.view(torch.int16))


def test_append_more_rows_than_keys(validate):
    wl, k_new, v_new, cu_new = _append_case()
    cu_k = [0, 1, 18, 108]  # sequence 0: 2 new rows, 1 key after the append
    _rejected(lambda: _append(wl, k_new, v_new, cu_new, cu_k=cu_k), "sequence 0 appends 2 rows but has 1 keys")


def test_append_block_id_outside_the_pool_where_rows_land(validate):
    wl, k_new, v_new, cu_new = _append_case()
    bt = np.array(wl.block_table, copy=True)
    nblk = wl.k.shape[0]
    bt[2, 2] = nblk  # sequence 2: keys 85..89 are new, page 2 (keys 64..95)
    _rejected(lambda: _append(wl, k_new, v_new, cu_new, bt=bt), "block_table[2][2] = %d" % nblk)


def test_append_bad_block_id_where_no_row_lands_accepted(validate):
    wl, k_new, v_new, cu_new = _append_case()
    bt = np.array(wl.block_table, copy=True)
    bt[2, 0] = -1  # page 0 of sequence 2 holds old keys only: not touched by the append
    _append(wl, k_new, v_new, cu_new, bt=bt)
