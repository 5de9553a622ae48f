"""GPU parity on seeded random shapes (bar as in tests/test_parity_gpu.py).

A hundred and twenty small configurations drawn from one seeded generator,
each compared element by element with the fp64 oracle: batch 1-12, query
lengths 0-200 (some sequences empty), key counts below, equal to or above the
query count (some zero), GQA ratios 1-8, head dims from 8 to 512 (odd ones on
the element-wise path), packed or paged K/V with pages of 32-256 (NaN-poisoned
spare slots), windows unbounded, causal, sliding or two-sided, bf16 or fp16,
and the path chosen by the planner or forced.  The draw is fixed, so every run
checks the same cases; each case prints its parameters before it runs.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity_util import assert_close, run_hip

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
