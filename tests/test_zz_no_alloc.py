"""The allocation-free entry fa_varlen_fwd_static through the C ABI.

It must give what fa_varlen_fwd gives with a caller-owned workspace (same
kernels: bit-identical out and lse) and stay within the oracle's bar, on two
calls in a row where the second is smaller than the first (the scratch keeps
the first call's contents), and it must reject shapes whose scratch would
exceed FA_STATIC_SCRATCH_BYTES without touching the output.
"""
import numpy as np
import pytest
import torch

import varlen_flash_attention_fa_amd as fa
import workloads as W
from parity_util import assert_close, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()


def _descs(d):
    dbt = fa._tdesc(d["bt"]) if d["bt"] is not None else None
    return fa._tdesc(d["q"]), fa._tdesc(d["k"]), fa._tdesc(d["v"]), dbt


def run_pair(wl, stream):
    """(out, lse) of fa_varlen_fwd with a workspace and of fa_varlen_fwd_static."""
    d = to_dev(wl)
    dq, dk, dv, dbt = _descs(d)
    nbytes = fa.fa_varlen_workspace_bytes(dq, dk, dv, wl.batch, dbt, wl.page_block_size)
    assert 0 < nbytes <= fa.FA_STATIC_SCRATCH_BYTES
    res = []
    for static in (False, True):
        out = torch.full_like(d["q"], float("nan"))
        lse = torch.full((wl.num_heads, wl.q.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
        args = (dq, dk, dv, fa._tdesc(out), d["cu_q"].data_ptr(), d["cu_k"].data_ptr(), wl.batch, dbt,
                wl.page_block_size, wl.softmax_scale, wl.window_left, wl.window_right, lse.data_ptr())
        with torch.cuda.stream(stream):
            if static:
                rc = fa.fa_varlen_fwd_static(*args, stream.cuda_stream)
            else:
                ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
                rc = fa.fa_varlen_fwd(*args, ws.data_ptr(), nbytes, stream.cuda_stream)
        assert rc == 0, fa.fa_last_error()
        stream.synchronize()
        res.append((out, lse))
    return res


def test_static_entry_matches_workspace_entry(oracle_mod):
    stream = torch.cuda.Stream()
    # first call: a split decode batch (partials, combine, adaptive chunk);
    # second call, smaller: a prefill batch that reads a shorter work list from
    # the same scratch
    first = W.make_custom([1] * 24 + [4] * 8, list(range(90, 90 + 32 * 97, 97)), 16, 4, 128, seed=61, page=32)
    second = W.make_custom([70, 5, 130], [70, 300, 900], 8, 2, 64, seed=62, page=64, window_left=200)
    for wl, what in ((first, "decode"), (second, "prefill, smaller")):
        (o_ws, l_ws), (o_st, l_st) = run_pair(wl, stream)
        assert torch.equal(o_ws.view(torch.int16), o_st.view(torch.int16)), what
        assert torch.equal(l_ws, l_st), what
        ref_o, ref_l = oracle_mod.attention_workload(wl)
        assert_close(o_st, l_st, ref_o, ref_l, what="static " + what, n_keys=int(max(wl.lens_k)))


def test_static_entry_rejects_oversize_scratch():
    # a decode batch over 1.28M-key block tables: its split partials alone would
    # need more than the static scratch holds
    wl = W.make_custom([1, 1, 1, 1], [100, 200, 300, 400], 16, 4, 128, seed=63, page=32, width=40000)
    d = to_dev(wl)
    dq, dk, dv, dbt = _descs(d)
    assert fa.fa_varlen_workspace_bytes(dq, dk, dv, wl.batch, dbt, 32) > fa.FA_STATIC_SCRATCH_BYTES
    out = torch.full_like(d["q"], 7.0)
    rc = fa.fa_varlen_fwd_static(dq, dk, dv, fa._tdesc(out), d["cu_q"].data_ptr(), d["cu_k"].data_ptr(),
                                 wl.batch, dbt, 32, wl.softmax_scale, -1, 0, 0, 0)
    torch.cuda.synchronize()
    assert fa.STATUS[rc] == "FA_ERR_WORKSPACE"
    assert "static scratch" in fa.fa_last_error()
    assert torch.all(out == 7.0)
