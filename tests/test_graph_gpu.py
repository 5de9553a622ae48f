"""HIP-graph capture of the forward (GPU).

A serving loop captures its decode step once and replays it with new contents
in the same buffers.  The forward has to allow that: it enqueues kernels only
(no allocation, memset or host synchronisation inside the call), and the
device planner reads the offsets at run time, so a replay with new sequence
lengths (within the shapes and bounds of the captured call) computes the new
work list.  Each case captures one call, then replays it several times with
new q and new offsets copied into the captured buffers; after every replay the
program's own eager call on the same inputs (into other buffers) must give the
same bits, and the replay's output must change with its inputs.  Cases: split
decode (planner, attention, combine), prefill through the planner, a direct
call (no planner), the allocation-free entry, and an append followed by the
forward (one decode step).
"""
import numpy as np
import pytest
import torch

import varlen_flash_attention_fa_amd as fa
import workloads as W
from parity_util import to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()


def _same(a, b):
    if a.dtype in (torch.bfloat16, torch.float16):
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def _cu(lens):
    return torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))


def _split(rng, total, n, lo=0):
    """n non-negative lengths (each >= lo) summing to total."""
    cuts = np.sort(rng.integers(0, total - n * lo + 1, size=n - 1))
    return (np.diff(np.concatenate([[0], cuts, [total - n * lo]])) + lo).astype(np.int64)


def _capture(fn):
    """Warm up fn on a side stream, then capture it into a graph; returns (graph, fn's result)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = fn()
    torch.cuda.synchronize()
    return g, res


def _replay_and_check(g, captured, set_inputs, eager, what):
    """Replay g after set_inputs(i); compare the captured outputs with eager() bit for bit."""
    prev = None
    for i in range(REPLAYS):
        set_inputs(i)
        torch.cuda.synchronize()
        print("%s: replay %d" % (what, i), flush=True)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in captured]
        ref = eager()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(got, ref)):
            assert _same(a, b), "%s: replay %d, output %d differs from the eager call" % (what, i, j)
        if prev is not None:
            assert not _same(got[0], prev[0]), "%s: replay %d did not recompute" % (what, i)
        prev = got


def _fwd(d, wl, out=None, ws=None):
    return fa.varlen_fwd(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], block_table=d["bt"],
                         page_block_size=wl.page_block_size or None, softmax_scale=wl.softmax_scale,
                         window_left=wl.window_left, window_right=wl.window_right, return_lse=True,
                         out=out, workspace=ws)


def _workspace(d, wl):
    dbt = fa._tdesc(d["bt"]) if d["bt"] is not None else None
    n = fa.fa_varlen_workspace_bytes(fa._tdesc(d["q"]), fa._tdesc(d["k"]), fa._tdesc(d["v"]), wl.batch, dbt,
                                     wl.page_block_size)
    return torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")


def test_graph_split_decode():
    # 24 single-query sequences over page-32 caches of up to 3000 keys: keys split
    # into chunks, partials merged by the combine
    rng = np.random.Generator(np.random.PCG64(71))
    lk0 = rng.integers(2000, 3000, size=24, endpoint=True)
    wl = W.make_custom([1] * 24, lk0, 32, 8, 128, seed=72, page=32)
    d = to_dev(wl)
    out = torch.empty_like(d["q"])
    ws = _workspace(d, wl)
    g, (o, l) = _capture(lambda: _fwd(d, wl, out=out, ws=ws))

    def set_inputs(i):
        d["q"].copy_(W.normal_bf16(rng, tuple(d["q"].shape)).cuda())
        lk = rng.integers(1, lk0, endpoint=True)  # every sequence keeps its pages
        d["cu_k"].copy_(_cu(lk).cuda())

    _replay_and_check(g, (o, l), set_inputs, lambda: _fwd(d, wl), "split decode")


def test_graph_prefill_planner():
    # 20 packed sequences (more than a direct call takes), causal, new splits of
    # the 1200 query rows and 3000 key rows each replay
    rng = np.random.Generator(np.random.PCG64(73))
    lq0 = _split(rng, 1200, 20, lo=1)
    lk0 = lq0 + _split(rng, 1800, 20)
    wl = W.make_custom(lq0, lk0, 8, 2, 128, seed=74)
    d = to_dev(wl)
    out = torch.empty_like(d["q"])
    ws = _workspace(d, wl)
    g, (o, l) = _capture(lambda: _fwd(d, wl, out=out, ws=ws))

    def set_inputs(i):
        lq = _split(rng, 1200, 20, lo=1)
        lk = lq + _split(rng, 1800, 20)
        d["cu_q"].copy_(_cu(lq).cuda())
        d["cu_k"].copy_(_cu(lk).cuda())
        d["q"].copy_(W.normal_bf16(rng, tuple(d["q"].shape)).cuda())

    _replay_and_check(g, (o, l), set_inputs, lambda: _fwd(d, wl), "prefill")


def test_graph_direct_call():
    # 5 sequences, no key split: no planner; the grid covers any split of the 400 rows
    rng = np.random.Generator(np.random.PCG64(75))
    lq0 = _split(rng, 400, 5, lo=1)
    wl = W.make_custom(lq0, lq0 + 50, 8, 2, 64, seed=76, page=32, width=20)
    d = to_dev(wl)
    out = torch.empty_like(d["q"])
    ws = _workspace(d, wl)
    g, (o, l) = _capture(lambda: _fwd(d, wl, out=out, ws=ws))

    def set_inputs(i):
        lq = _split(rng, 400, 5)  # sequences with no query row too
        lk = np.minimum(lq + rng.integers(0, 60, size=5), (lq0 + 50 + 31) // 32 * 32)
        d["cu_q"].copy_(_cu(lq).cuda())
        d["cu_k"].copy_(_cu(lk).cuda())
        d["q"].copy_(W.normal_bf16(rng, tuple(d["q"].shape)).cuda())

    _replay_and_check(g, (o, l), set_inputs, lambda: _fwd(d, wl), "direct")


def test_graph_static_entry():
    rng = np.random.Generator(np.random.PCG64(77))
    lk0 = rng.integers(1500, 2500, size=16, endpoint=True)
    wl = W.make_custom([2] * 16, lk0, 16, 4, 128, seed=78, page=64)
    d = to_dev(wl)
    dq, dk, dv = fa._tdesc(d["q"]), fa._tdesc(d["k"]), fa._tdesc(d["v"])
    dbt = fa._tdesc(d["bt"])
    out = torch.empty_like(d["q"])
    lse = torch.empty((wl.num_heads, wl.q.shape[0]), dtype=torch.float32, device="cuda")

    def call():
        rc = fa.fa_varlen_fwd_static(dq, dk, dv, fa._tdesc(out), d["cu_q"].data_ptr(), d["cu_k"].data_ptr(),
                                     wl.batch, dbt, 64, wl.softmax_scale, -1, 0, lse.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
        assert rc == 0, fa.fa_last_error()
        return out, lse

    g, _ = _capture(call)

    def set_inputs(i):
        lk = rng.integers(2, lk0, endpoint=True)
        d["cu_k"].copy_(_cu(lk).cuda())
        d["q"].copy_(W.normal_bf16(rng, tuple(d["q"].shape)).cuda())

    _replay_and_check(g, (out, lse), set_inputs, lambda: _fwd(d, wl), "static entry")


def test_graph_append_then_attend():
    # one decode step: append each sequence's new K/V row into the pool, then
    # attend over the grown caches; replays reuse the same slots with new rows
    rng = np.random.Generator(np.random.PCG64(79))
    lk = rng.integers(100, 900, size=12, endpoint=True)
    wl = W.make_custom([1] * 12, lk, 16, 4, 128, seed=80, page=32, width=32)
    d = to_dev(wl)
    cu_new = _cu(np.ones(12, np.int64)).cuda()
    k_new = torch.empty((12, 4, 128), dtype=torch.bfloat16, device="cuda")
    v_new = torch.empty_like(k_new)
    out = torch.empty_like(d["q"])
    ws = _workspace(d, wl)
    pool0 = (d["k"].clone(), d["v"].clone())

    def step(kc, vc, o=None, w=None):
        fa.kv_append(k_new, v_new, cu_new, d["cu_k"], d["bt"], kc, vc)
        return fa.varlen_fwd(d["q"], kc, vc, d["cu_q"], d["cu_k"], block_table=d["bt"], page_block_size=32,
                             softmax_scale=wl.softmax_scale, window_left=-1, window_right=0, return_lse=True,
                             out=o, workspace=w)

    k_new.copy_(W.normal_bf16(rng, (12, 4, 128)).cuda())
    v_new.copy_(W.normal_bf16(rng, (12, 4, 128)).cuda())
    g, (o, l) = _capture(lambda: step(d["k"], d["v"], out, ws))

    def set_inputs(i):
        k_new.copy_(W.normal_bf16(rng, (12, 4, 128)).cuda())
        v_new.copy_(W.normal_bf16(rng, (12, 4, 128)).cuda())
        d["q"].copy_(W.normal_bf16(rng, tuple(d["q"].shape)).cuda())

    def eager():
        kc, vc = pool0[0].clone(), pool0[1].clone()
        o2, l2 = step(kc, vc)
        torch.cuda.synchronize()
        # the replay wrote the same rows into the captured pool
        assert _same(kc, d["k"]) and _same(vc, d["v"]), "append: pools differ"
        return o2, l2

    _replay_and_check(g, (o, l), set_inputs, eager, "append + attend")
