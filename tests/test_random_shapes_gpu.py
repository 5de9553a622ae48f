"""GPU parity on seeded random shapes (bar as in tests/test_parity_gpu.py).

A hundred and twenty small configurations drawn from one seeded generator,
each compared element by element with the fp64 oracle: batch 1-12, query
lengths 0-200 (some sequences empty), key counts below, equal to or above the
query count (some zero), GQA ratios 1-8, head dims from 8 to 512 (odd ones on
the element-wise path), packed or paged K/V with pages of 32-256 (NaN-poisoned
spare slots), windows unbounded, causal, sliding or two-sided, bf16 or fp16,
and the path chosen by the planner or forced.  Forty padded (B, S, H, D) calls
(batch-major or head-major views, Sq above or below Sk, Sk = 0 too) are compared
the same way, forty paged appends bit for bit against the oracle's pool, and
thirty more varlen draws with ALiBi slopes (per head or per sequence).
Every fourth varlen case runs a second time through the planner's work list
(FA_DIRECT=0) and must give the same bits.  The draws are fixed, so every run
checks the same cases; each case prints its parameters before it runs.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity_util import assert_close, run_hip, to_dev

pytestmark = pytest.mark.gpu

N_CASES = 120


def _draw(i):
    rng = np.random.Generator(np.random.PCG64(9000 + i))
    batch = int(rng.integers(1, 12, endpoint=True))
    lq = rng.integers(0, 200, size=batch, endpoint=True)
    lq[rng.random(batch) < 0.15] = 0
    mode = rng.integers(0, 3)
    if mode == 0:      # keys = queries (self-attention prefill)
        lk = lq.copy()
    elif mode == 1:    # a cached prefix before the queries
        lk = lq + rng.integers(0, 1500, size=batch, endpoint=True)
    else:              # unrelated key counts (rows with more queries than keys too)
        lk = rng.integers(0, 2500, size=batch, endpoint=True)
    Hk = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([8, 13, 40, 64, 80, 96, 128, 136, 200, 256, 320, 512]))
    page = int(rng.choice([0, 0, 32, 64, 128, 256]))
    win = int(rng.integers(0, 4))
    wl_, wr_ = [(-1, -1), (-1, 0), (int(rng.integers(0, 300)), 0),
                (int(rng.integers(0, 100)), int(rng.integers(0, 50)))][win]
    path = ["", "", "prefill", "decode"][int(rng.integers(0, 4))]
    scale = None if rng.random() < 0.7 else float(rng.uniform(0.02, 0.5))
    dtype = "f16" if rng.random() < 0.2 else "bf16"
    return dict(lq=lq.tolist(), lk=lk.tolist(), H=Hk * G, Hk=Hk, D=D, page=page, wl=wl_, wr=wr_,
                path=path, scale=scale, dtype=dtype, seed=9100 + i)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import varlen_flash_attention_fa_amd as fa
    fa.load()


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(oracle_mod, monkeypatch, i):
    c = _draw(i)
    print("case", i, c, flush=True)
    if c["path"]:
        monkeypatch.setenv("FA_FORCE_PATH", c["path"])
    else:
        monkeypatch.delenv("FA_FORCE_PATH", raising=False)
    wl = W.make_custom(c["lq"], c["lk"], c["H"], c["Hk"], c["D"], seed=c["seed"], page=c["page"],
                       window_left=c["wl"], window_right=c["wr"], scale=c["scale"], poison=c["page"] > 0,
                       dtype=c["dtype"])
    out, lse = run_hip(wl)
    ref_o, ref_l = oracle_mod.attention_workload(wl)
    assert_close(out, lse, ref_o, ref_l, what="random case %d" % i, n_keys=int(max([1] + c["lk"])))
    if i % 4 == 0:
        # the same call through the planner's work list (these small batches
        # otherwise run as direct calls when their keys are not split): same bits
        monkeypatch.setenv("FA_DIRECT", "0")
        out2, lse2 = run_hip(wl)
        monkeypatch.delenv("FA_DIRECT")
        assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "random case %d: planned" % i
        assert torch.equal(lse, lse2), "random case %d: planned lse" % i


# ------------------------------------------------------------ padded entry

N_PADDED = 40


def _draw_padded(i):
    rng = np.random.Generator(np.random.PCG64(9500 + i))
    B = int(rng.integers(1, 6, endpoint=True))
    Sq = int(rng.integers(1, 150, endpoint=True))
    Sk = int(rng.integers(0, 400, endpoint=True))
    Hk = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([8, 13, 64, 96, 128, 200, 256, 512]))
    win = int(rng.integers(0, 4))
    wl_, wr_ = [(-1, -1), (-1, 0), (int(rng.integers(0, 200)), 0),
                (int(rng.integers(0, 60)), int(rng.integers(0, 30)))][win]
    layout = ["bshd", "bhsd"][int(rng.integers(0, 2))]
    dtype = "f16" if rng.random() < 0.2 else "bf16"
    path = ["", "", "prefill", "decode"][int(rng.integers(0, 4))]
    return dict(B=B, Sq=Sq, Sk=Sk, H=Hk * G, Hk=Hk, D=D, wl=wl_, wr=wr_, layout=layout, dtype=dtype,
                path=path, seed=9600 + i)


def _upload(t, layout):
    """Keep the layout on the device: head-major views stay head-major views."""
    if layout == "bhsd":
        return t.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    return t.cuda()


@pytest.mark.parametrize("i", range(N_PADDED))
def test_random_padded(oracle_mod, monkeypatch, i):
    import varlen_flash_attention_fa_amd as fa
    from parity_util import MAX_ABS, MEAN_ABS, lse_bound
    c = _draw_padded(i)
    print("case", i, c, flush=True)
    if c["path"]:
        monkeypatch.setenv("FA_FORCE_PATH", c["path"])
    else:
        monkeypatch.delenv("FA_FORCE_PATH", raising=False)
    q, k, v = W.make_padded(c["B"], c["Sq"], c["Sk"], c["H"], c["Hk"], c["D"], seed=c["seed"],
                            layout=c["layout"], dtype=c["dtype"])
    scale = 1.0 / np.sqrt(c["D"])
    out, lse = fa.padded_fwd(_upload(q, c["layout"]), _upload(k, c["layout"]), _upload(v, c["layout"]),
                             softmax_scale=scale, window_left=c["wl"], window_right=c["wr"], return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.attention_padded(q, k, v, scale, c["wl"], c["wr"])
    o = out.float().cpu().double().numpy()
    l = lse.cpu().double().numpy()
    assert np.isfinite(o).all(), "non-finite output"
    err = np.abs(o - ref_o)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, "max %.3g mean %.3g" % (err.max(), err.mean())
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(l), fin), "lse -inf pattern"
    bound = lse_bound(out.dtype, max(1, c["Sk"]))
    assert np.abs(l[fin] - ref_l[fin]).max(initial=0.0) <= bound, "lse"


# ------------------------------------------------------------ paged append

N_APPEND = 40


def _draw_append(i):
    rng = np.random.Generator(np.random.PCG64(9700 + i))
    batch = int(rng.integers(1, 12, endpoint=True))
    lk = rng.integers(0, 3000, size=batch, endpoint=True)
    lnew = np.minimum(lk, rng.integers(0, 200, size=batch, endpoint=True))
    lnew[rng.random(batch) < 0.2] = 0
    Hk = int(rng.choice([1, 2, 3, 4, 8]))
    D = int(rng.choice([8, 13, 40, 64, 100, 128, 256, 512]))
    page = int(rng.choice([32, 64, 128, 256]))
    return dict(lnew=lnew.tolist(), lk=lk.tolist(), Hk=Hk, D=D, page=page, seed=9800 + i)


@pytest.mark.parametrize("i", range(N_APPEND))
def test_random_append_bit_exact(oracle_mod, i):
    import varlen_flash_attention_fa_amd as fa
    c = _draw_append(i)
    print("case", i, c, flush=True)
    wl, k_new, v_new, cu_new = W.make_append(c["lnew"], c["lk"], c["Hk"], c["D"], page=c["page"], seed=c["seed"])
    dev = "cuda"
    kp, vp = wl.k.to(dev), wl.v.to(dev)
    fa.kv_append(k_new.to(dev), v_new.to(dev), torch.from_numpy(np.ascontiguousarray(cu_new, np.int32)).to(dev),
                 torch.from_numpy(np.ascontiguousarray(wl.cu_seqlens_k, np.int32)).to(dev),
                 torch.from_numpy(np.ascontiguousarray(wl.block_table, np.int32)).to(dev), kp, vp)
    torch.cuda.synchronize()
    rk, rv = oracle_mod.kv_append(k_new, v_new, cu_new, wl.cu_seqlens_k, wl.block_table, wl.k, wl.v)
    gk = kp.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    gv = vp.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    assert int((gk != rk).sum()) == 0 and int((gv != rv).sum()) == 0, "pool differs from the oracle's"


# ------------------------------------------------------------------ ALiBi

N_ALIBI = 30


@pytest.mark.parametrize("i", range(N_ALIBI))
def test_random_alibi(oracle_mod, monkeypatch, i):
    # the varlen draws above, with per-head or per-sequence slopes (seeded uniform
    # draws in [0, 1), or the geometric sequence)
    import varlen_flash_attention_fa_amd as fa
    c = _draw(1000 + i)
    rng = np.random.Generator(np.random.PCG64(9900 + i))
    per_seq = bool(rng.random() < 0.5)
    geometric = bool(rng.random() < 0.3)
    slopes = W.alibi_slopes(c["H"], batch=len(c["lq"]) if per_seq else 0,
                            seed=None if geometric else 9950 + i)
    print("case", i, c, "per_seq", per_seq, "geometric", geometric, flush=True)
    if c["path"]:
        monkeypatch.setenv("FA_FORCE_PATH", c["path"])
    else:
        monkeypatch.delenv("FA_FORCE_PATH", raising=False)
    wl = W.make_custom(c["lq"], c["lk"], c["H"], c["Hk"], c["D"], seed=c["seed"], page=c["page"],
                       window_left=c["wl"], window_right=c["wr"], scale=c["scale"], poison=c["page"] > 0,
                       dtype=c["dtype"])
    d = to_dev(wl)
    out, lse = fa.varlen_fwd(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], block_table=d["bt"],
                             page_block_size=wl.page_block_size or None, softmax_scale=wl.softmax_scale,
                             window_left=wl.window_left, window_right=wl.window_right, return_lse=True,
                             alibi_slopes=torch.from_numpy(slopes).cuda())
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.attention_workload(wl, alibi_slopes=slopes)
    assert_close(out, lse, ref_o, ref_l, what="random alibi case %d" % i, n_keys=int(max([1] + c["lk"])))
