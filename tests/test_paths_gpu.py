"""GPU parity on kernel paths that the configuration workloads do not reach.

Each case compares the HIP path, through the C ABI, with the fp64 oracle to the
same bar as tests/test_parity_gpu.py (bf16 out max |d| <= 2e-2, mean |d| <=
2e-3, lse within parity_util.lse_bound).  Covered here:

* windows at the int32 limit: the window edges a - window_left and
  a + window_right + 1 must not wrap, so INT32_MAX behaves as "no limit"
  (rows with more queries than keys included, both kernel paths);
* the combine kernel with more than 64 key chunks per query row (forced and
  chosen by the planner), and items whose keys span several block-table
  segments (more than 255 pages);
* the planner with more than 1024 sequences (its carried scan) and more than
  2048 (offsets and spans read from global memory);
* page sizes 256 and 512;
* a negative softmax scale (applied as an exact sign flip of q).
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity_util import assert_close, run_hip

pytestmark = pytest.mark.gpu

I32_MAX = 2 ** 31 - 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import varlen_flash_attention_fa_amd as fa
    fa.load()


@pytest.fixture()
def force_env(monkeypatch):
    def set_(**kv):
        for k, v in kv.items():
            monkeypatch.setenv(k, str(v))
    return set_


def check(oracle_mod, wl, what):
    print("case", what, flush=True)
    out, lse = run_hip(wl)
    ref_o, ref_l = oracle_mod.attention_workload(wl)
    return assert_close(out, lse, ref_o, ref_l, what=what, n_keys=int(max([1] + list(wl.lens_k))))


# ------------------------------------------------------------ int32 windows

WINDOWS = [(I32_MAX, 0), (-1, I32_MAX), (I32_MAX, I32_MAX), (I32_MAX, 5), (3, I32_MAX),
           (I32_MAX - 1, I32_MAX - 1), (I32_MAX, -1)]


@pytest.mark.parametrize("path", ["prefill", "decode"])
@pytest.mark.parametrize("page", [0, 32])
@pytest.mark.parametrize("wl_,wr_", WINDOWS)
def test_int32_limit_windows(oracle_mod, force_env, path, page, wl_, wr_):
    # sequences 0, 2 and 4 have more queries than keys (rows before the first
    # key position), sequence 3 has no key at all
    force_env(FA_FORCE_PATH=path)
    lq, lk = [5, 40, 70, 3, 9], [3, 300, 200, 0, 1]
    wl = W.make_custom(lq, lk, 8, 2, 128, seed=31, page=page, window_left=wl_, window_right=wr_)
    check(oracle_mod, wl, "window (%d, %d) %s page %d" % (wl_, wr_, path, page))


def test_int32_limit_windows_equal_unbounded():
    # the same inputs with INT32_MAX and with -1 (no limit): identical bits
    lq, lk = [5, 40, 70], [3, 300, 200]
    wl = W.make_custom(lq, lk, 8, 2, 128, seed=32, page=32, window_left=-1, window_right=-1)
    ref, _ = run_hip(wl)
    wl.window_left, wl.window_right = I32_MAX, I32_MAX
    got, _ = run_hip(wl)
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))


# ----------------------------------------------- many chunks, many segments

def test_combine_over_64_chunks_forced(oracle_mod, force_env):
    # 512-key chunks over 40k keys: 79 partials per query row
    force_env(FA_FORCE_PATH="decode", FA_SPLIT_KEYS=512)
    wl = W.make_custom([1, 1, 3], [40000, 37, 33000], 8, 2, 128, seed=33, page=32)
    check(oracle_mod, wl, "79 chunks")


def test_combine_over_64_chunks_adaptive(oracle_mod):
    # two short-query sequences over 70k keys: the planner's chunk (512..2048
    # keys) leaves 35..137 chunks per row; the work list fills well under a
    # quarter of the GPU, so it takes the small end
    wl = W.make_custom([1, 2], [70000, 69000], 16, 2, 128, seed=34, page=64)
    check(oracle_mod, wl, "adaptive long decode")


def test_many_block_table_segments(oracle_mod, force_env):
    # 16384-key chunks over 32-key pages: every item spans three segments of at
    # most 255 pages of block ids staged in LDS
    force_env(FA_FORCE_PATH="decode", FA_SPLIT_KEYS=16384)
    wl = W.make_custom([1, 4], [40000, 9000], 8, 2, 128, seed=35, page=32)
    check(oracle_mod, wl, "segments decode")
    # prefill without a key split over 9k keys of 32-key pages: two segments
    force_env(FA_FORCE_PATH="prefill", FA_SPLIT_KEYS=0)
    wl = W.make_custom([150, 20], [9000, 8500], 8, 2, 128, seed=36, page=32, window_left=8300)
    check(oracle_mod, wl, "segments prefill")


# ------------------------------------------------------- large batch sizes

@pytest.mark.parametrize("batch", [1500, 3000])
def test_decode_large_batch(oracle_mod, batch):
    # > 1024 sequences: the planner's scan carries over blocks of 1024; > 2048:
    # spans and item offsets are read from global memory instead of LDS.  Some
    # caches are long enough to be split, so the combine's per-token chunk
    # counts are filled too.
    rng = np.random.Generator(np.random.PCG64(37 + batch))
    lk = rng.integers(1, 300, size=batch, endpoint=True)
    lk[::97] = rng.integers(1500, 3500, size=lk[::97].shape[0])
    wl = W.make_custom([1] * batch, lk.tolist(), 8, 2, 128, seed=38, page=32)
    check(oracle_mod, wl, "decode batch %d" % batch)


@pytest.mark.parametrize("batch", [1500, 3000])
def test_prefill_large_batch(oracle_mod, batch):
    rng = np.random.Generator(np.random.PCG64(39 + batch))
    lq = rng.integers(1, 40, size=batch, endpoint=True)
    lq[5] = 0
    lk = lq + rng.integers(0, 100, size=batch, endpoint=True)
    wl = W.make_custom(lq.tolist(), lk.tolist(), 8, 2, 64, seed=40, page=0)
    check(oracle_mod, wl, "prefill batch %d" % batch)


# --------------------------------------------------------- large page sizes

@pytest.mark.parametrize("page", [256, 512])
@pytest.mark.parametrize("path", ["prefill", "decode"])
def test_large_pages(oracle_mod, force_env, page, path):
    force_env(FA_FORCE_PATH=path)
    lq, lk = [1, 130, 4, 17], [2000, 900, 513, 17]
    wl = W.make_custom(lq, lk, 8, 2, 128, seed=41, page=page, poison=True, width=9)
    check(oracle_mod, wl, "page %d %s" % (page, path))


@pytest.mark.parametrize("page", [256, 512])
def test_large_pages_d512(oracle_mod, page):
    wl = W.make_custom([4, 4], [3000, 700], 16, 1, 512, seed=42, page=page)
    check(oracle_mod, wl, "page %d d512" % page)


# ------------------------------------------------------------ negative scale

@pytest.mark.parametrize("path", ["prefill", "decode"])
@pytest.mark.parametrize("scale", [-0.0883883461356163, -0.5])
def test_negative_scale(oracle_mod, force_env, path, scale):
    force_env(FA_FORCE_PATH=path)
    wl = W.make_custom([1, 77, 3], [300, 77, 1000], 8, 2, 128, seed=43, page=32, scale=scale)
    check(oracle_mod, wl, "scale %g %s" % (scale, path))
