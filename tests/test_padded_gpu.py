"""GPU parity of the padded (batch-major, non-varlen) entry, fa_padded_fwd through the C ABI.

Same bar as the varlen forward: bf16 out within max |d| <= 2e-2 and mean
|d| <= 2e-3 of the fp64 oracle, lse within the bound of
parity_util.lse_bound.  Cases cover both kernel
paths (prefill rows > 64 per sequence and K/V head, decode otherwise), GQA/MQA,
windows, Sq > Sk, odd and large head dims, and head-major tensors passed as
(B, S, H, D) views (batch stride not S * token stride).  The two padded bench
workloads are checked in full (decode) or on sampled rows (prefill).
"""
import numpy as np
import pytest
import torch

import varlen_flash_attention_fa_amd as fa
import workloads as W
from parity_util import LSE_ABS, MAX_ABS, MEAN_ABS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()


def to_dev(t, layout):
    """Upload keeping the layout: head-major views stay head-major views on the device."""
    if layout == "bhsd":
        return t.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    return t.cuda()


def compare(out, lse, ref_o, ref_l, what, rows=None):
    o = out.float().cpu().double().numpy()
    l = lse.cpu().double().numpy()
    if rows is not None:   # rows: (b, i) pairs
        o = np.stack([o[b, i] for b, i in rows])
        ref_o = np.stack([ref_o[b, i] for b, i in rows])
        l = np.stack([l[b, :, i] for b, i in rows])
        ref_l = np.stack([ref_l[b, :, i] for b, i in rows])
    assert np.isfinite(o).all(), what + ": non-finite output"
    err = np.abs(o - ref_o)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, "%s: max %.3g mean %.3g" % (what, err.max(), err.mean())
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(l), fin), what + ": lse -inf pattern"
    assert np.abs(l[fin] - ref_l[fin]).max(initial=0.0) <= LSE_ABS, what + ": lse"


CASES = [
    # name, B, Sq, Sk, H, Hk, D, wl, wr, layout
    ("prefill-causal-gqa", 3, 150, 150, 8, 2, 128, -1, 0, "bshd"),
    ("prefill-bhsd-window", 2, 200, 260, 4, 4, 64, 50, 0, "bhsd"),
    ("prefill-d256", 2, 70, 90, 4, 2, 256, -1, 0, "bshd"),
    ("prefill-d512-mqa", 2, 40, 70, 4, 1, 512, -1, 0, "bhsd"),
    ("decode-q1", 9, 1, 1000, 32, 8, 128, -1, 0, "bshd"),
    ("decode-q4-bhsd", 5, 4, 2100, 16, 1, 256, -1, 0, "bhsd"),
    ("two-sided-sq-gt-sk", 2, 37, 20, 4, 2, 128, 7, 5, "bshd"),
    ("odd-d13", 2, 33, 40, 4, 2, 13, -1, 0, "bshd"),
    ("noncausal", 2, 64, 64, 4, 2, 80, -1, -1, "bhsd"),
]


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[c[0] for c in CASES])
def test_small_cases(oracle_mod, idx):
    name, B, Sq, Sk, H, Hk, D, wl, wr, layout = CASES[idx]
    print("case", name, flush=True)
    q, k, v = W.make_padded(B, Sq, Sk, H, Hk, D, seed=500 + idx, layout=layout)
    scale = 1.0 / np.sqrt(D)
    qd, kd, vd = to_dev(q, layout), to_dev(k, layout), to_dev(v, layout)
    out, lse = fa.padded_fwd(qd, kd, vd, softmax_scale=scale, window_left=wl, window_right=wr, return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.attention_padded(q, k, v, scale, wl, wr)
    compare(out, lse, ref_o, ref_l, name)


def test_strided_out_and_empty_keys(oracle_mod):
    """out as a head-major view; a call with Sk = 0 writes zeros and -inf."""
    B, Sq, Sk, H, Hk, D = 2, 20, 30, 4, 2, 64
    q, k, v = W.make_padded(B, Sq, Sk, H, Hk, D, seed=600)
    out = torch.full((B, H, Sq, D), 7.0, dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    res, lse = fa.padded_fwd(q.cuda(), k.cuda(), v.cuda(), softmax_scale=0.125, window_left=-1, window_right=0,
                             return_lse=True, out=out)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.attention_padded(q, k, v, 0.125, -1, 0)
    compare(res, lse, ref_o, ref_l, "strided out")
    ke = torch.zeros(B, 0, Hk, D, dtype=torch.bfloat16, device="cuda")
    o2, l2 = fa.padded_fwd(q.cuda(), ke, ke, softmax_scale=0.125, return_lse=True)
    torch.cuda.synchronize()
    assert not o2.float().abs().sum().item() and torch.isneginf(l2).all()


def test_decode_workload_full(oracle_mod):
    cfg = W.PADDED["p2"]
    q, k, v = W.make_padded(cfg["B"], cfg["Sq"], cfg["Sk"], cfg["num_heads"], cfg["num_heads_k"],
                            cfg["head_dim"], seed=cfg["seed"])
    scale = 1.0 / np.sqrt(cfg["head_dim"])
    out, lse = fa.padded_fwd(q.cuda(), k.cuda(), v.cuda(), softmax_scale=scale, window_left=cfg["window_left"],
                             window_right=cfg["window_right"], return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.attention_padded(q, k, v, scale, cfg["window_left"], cfg["window_right"])
    compare(out, lse, ref_o, ref_l, "p2")


def test_prefill_workload_sampled(oracle_mod):
    cfg = W.PADDED["p4"]
    B, Sq, Sk, H, Hk, D = (cfg[x] for x in ("B", "Sq", "Sk", "num_heads", "num_heads_k", "head_dim"))
    q, k, v = W.make_padded(B, Sq, Sk, H, Hk, D, seed=cfg["seed"])
    scale = 1.0 / np.sqrt(D)
    out, lse = fa.padded_fwd(q.cuda(), k.cuda(), v.cuda(), softmax_scale=scale, window_left=cfg["window_left"],
                             window_right=cfg["window_right"], return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(77))
    rows = [(b, i) for b in range(B) for i in (0, Sq - 1)]
    rows += [(int(b), int(i)) for b, i in zip(rng.integers(0, B, 24), rng.integers(0, Sq, 24))]
    sel = np.zeros(B * Sq, np.uint8)
    for b, i in rows:
        sel[b * Sq + i] = 1
    # rows of the equivalent varlen call (uniform offsets; pinned bit-exact on the CPU)
    o_flat, l_flat = oracle_mod.attention(q.reshape(B * Sq, H, D), k.reshape(B * Sk, Hk, D), v.reshape(B * Sk, Hk, D),
                                          np.arange(B + 1, dtype=np.int32) * Sq,
                                          np.arange(B + 1, dtype=np.int32) * Sk, softmax_scale=scale,
                                          window_left=cfg["window_left"], window_right=cfg["window_right"],
                                          token_sel=sel)
    ref_o = o_flat.reshape(B, Sq, H, D)
    ref_l = l_flat.reshape(H, B, Sq).transpose(1, 0, 2)
    compare(out, lse, ref_o, ref_l, "p4 sampled", rows=rows)
