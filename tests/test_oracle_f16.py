"""Pins for the oracle's fp16 (IEEE binary16) inputs.

The widening of both 16-bit types is checked exhaustively against numpy's and
torch's own conversions (every bit pattern); the fp16 attention is checked
against torch fp64 SDPA on the same fp16 inputs, and against the closed form of
a single visible key."""
import numpy as np
import pytest
import torch

import workloads as W
from test_oracle_pins import sdpa_reference


def test_widening_is_exact_for_every_bit_pattern(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f16 = oracle_mod.widen(bits, "f16")
    ref16 = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref16)
    assert np.array_equal(np.isnan(f16), nan)
    assert np.array_equal(f16[~nan], ref16[~nan])
    bf = oracle_mod.widen(bits, "bf16")
    refbf = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nanb = np.isnan(refbf)
    assert np.array_equal(np.isnan(bf), nanb)
    assert np.array_equal(bf[~nanb], refbf[~nanb])


CASES = [
    # lens_q, lens_k, H, Hk, D, page, wl, wr
    ([17, 64, 5], [17, 64, 5], 4, 2, 64, 0, -1, 0),
    ([1, 3, 2], [40, 130, 64], 8, 2, 32, 32, -1, 0),
    ([9, 30], [40, 30], 4, 4, 16, 0, 6, 3),
]


@pytest.mark.parametrize("case", CASES)
def test_f16_matches_torch_sdpa(oracle_mod, case):
    lq, lk, H, Hk, D, P, wl_, wr_ = case
    wl = W.make_custom(lq, lk, H, Hk, D, seed=31, page=P, window_left=wl_, window_right=wr_, dtype="f16")
    assert wl.q.dtype == torch.float16
    out, _ = oracle_mod.attention_workload(wl)
    ref, valid = sdpa_reference(wl)
    assert np.abs(out[valid] - ref[valid]).max() < 1e-12
    assert (out[~valid] == 0).all()


def test_f16_single_key_gives_v_exactly(oracle_mod):
    wl = W.make_custom([4], [9], 2, 1, 32, seed=32, window_left=0, window_right=0, dtype="f16")
    out, _ = oracle_mod.attention_workload(wl)
    # row i sees key i + Lk - Lq only
    keys = np.arange(4) + 9 - 4
    ref = wl.v[keys].double().repeat_interleave(2, dim=1).numpy()
    assert np.array_equal(out, ref)


def test_f16_values_outside_bf16_precision(oracle_mod):
    """Values bf16 cannot hold (11 significant bits) keep their fp16 meaning."""
    q = torch.tensor([[[1.0009765625, 0.0]]], dtype=torch.float16)   # 1 + 2^-10
    k = torch.tensor([[[3.0, 0.0]], [[2.0, 0.0]]], dtype=torch.float16)
    v = torch.tensor([[[1.0, 2049.0]], [[-1.0, 0.5]]], dtype=torch.float16)
    out, lse = oracle_mod.attention(q, k, v, np.array([0, 1], np.int32), np.array([0, 2], np.int32),
                                    softmax_scale=1.0, window_left=-1, window_right=-1)
    s = np.array([3.0, 2.0]) * (1 + 2.0 ** -10)
    p = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    ref = p[0] * np.array([1.0, 2048.0]) + p[1] * np.array([-1.0, 0.5])   # 2049 rounds to 2048 in fp16
    assert np.allclose(out[0, 0], ref, rtol=0, atol=1e-12)
    assert abs(lse[0, 0] - np.log(np.exp(s).sum())) < 1e-12
