"""GPU parity of the fp16 (IEEE binary16) instantiation through the C ABI.

Same output bar as bf16: out within max |d| <= 2e-2 and mean |d| <= 2e-3 of
the fp64 oracle on the same fp16 inputs.  lse within the fp16 bound derived in
parity_util.lse_bound (2^-11 rounding of the probabilities, their subnormal
range, fp32 sums): about 6.2e-4 at 4097 keys, where bf16 allows 3.9e-3.  The
append stays bit-exact.
Covers configuration 1, every small shape of the bf16 suite (both kernel paths,
head dims 13-512, paged and packed, windows), the full-size paged decode and
long-prefill workloads on sampled rows, the padded entry and the append.
"""
import numpy as np
import pytest
import torch

import varlen_flash_attention_fa_amd as fa
import workloads as W
from parity_util import assert_close, lse_bound, run_hip
from test_parity_gpu import SMALL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()


def check(oracle_mod, wl, what, rows=None):
    assert wl.q.dtype == torch.float16
    out, lse = run_hip(wl)
    assert out.dtype == torch.float16
    sel = None
    if rows is not None:
        sel = np.zeros(wl.q.shape[0], np.uint8)
        sel[rows] = 1
    ref_o, ref_l = oracle_mod.attention_workload(wl, token_sel=sel)
    return assert_close(out, lse, ref_o, ref_l, rows=rows, what=what,
                        n_keys=int(max([1] + list(wl.lens_k))))


def test_config1_f16(oracle_mod):
    check(oracle_mod, W.make_config("c1", dtype="f16"), "c1 f16")


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes_f16(oracle_mod, case):
    name, lq, lk, H, Hk, D, P, wl_, wr_ = case
    wl = W.make_custom(lq, lk, H, Hk, D, seed=700, page=P, window_left=wl_, window_right=wr_, dtype="f16")
    check(oracle_mod, wl, name + " f16")


def sampled_rows(wl, n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    cu = wl.cu_seqlens_q
    rows = set()
    for b in range(wl.batch):
        if cu[b + 1] > cu[b]:
            rows.update((int(cu[b]), int(cu[b + 1]) - 1))
    rows.update(int(x) for x in rng.integers(0, wl.q.shape[0], n))
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["c2", "c4"])
def test_full_size_f16_sampled(oracle_mod, name):
    wl = W.make_config(name, dtype="f16")
    print("f16 full size", name, flush=True)
    check(oracle_mod, wl, name + " f16", rows=sampled_rows(wl, 48, 5))


def test_padded_f16(oracle_mod):
    q, k, v = W.make_padded(3, 150, 170, 8, 2, 128, seed=701, layout="bhsd", dtype="f16")
    qd = q.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    kd = k.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    vd = v.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    out, lse = fa.padded_fwd(qd, kd, vd, softmax_scale=0.1, window_left=-1, window_right=0, return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.attention_padded(q, k, v, 0.1, -1, 0)
    o = out.float().cpu().double().numpy()
    err = np.abs(o - ref_o)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
    assert np.abs(lse.cpu().double().numpy() - ref_l).max() <= lse_bound("f16", 170)


def test_append_f16_bit_exact(oracle_mod):
    lnew, lk = [3, 1, 20, 0], [70, 33, 200, 9]
    wl = W.make_custom(lnew, lk, 4, 4, 64, seed=702, page=32, dtype="f16")
    k_new, cu_new = wl.q, wl.cu_seqlens_q
    v_new = -wl.q
    kp, vp = wl.k.cuda(), wl.v.cuda()
    fa.kv_append(k_new.cuda(), v_new.cuda(), torch.from_numpy(cu_new).cuda(),
                 torch.from_numpy(wl.cu_seqlens_k).cuda(), torch.from_numpy(wl.block_table).cuda(), kp, vp)
    torch.cuda.synchronize()
    rk, rv = oracle_mod.kv_append(k_new, v_new, cu_new, wl.cu_seqlens_k, wl.block_table, wl.k, wl.v)
    assert np.array_equal(kp.cpu().view(torch.int16).numpy().view(np.uint16), rk)
    assert np.array_equal(vp.cpu().view(torch.int16).numpy().view(np.uint16), rv)
