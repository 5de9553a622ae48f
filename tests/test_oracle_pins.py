"""Pins for the fp64 oracle against facts fixed outside it.

Every check here compares the oracle with something other than itself:
closed forms (single visible key, uniform V, zero Q, two keys), torch's fp64
``scaled_dot_product_attention`` with masks built from ``torch.tril``/``triu``
(the textbook causal / band matrices), mpmath at 50 digits on tiny inputs, and
invariants the method must satisfy (paged == packed, block permutation, GQA ==
repeated K/V heads, batch == concatenation of single-sequence calls).

The mask reading being pinned: query row i of a sequence with Lq queries and Lk
keys sits at key position a = i + Lk - Lq (bottom-right alignment); key j is
visible iff j >= a - window_left (when window_left >= 0) and j <= a +
window_right (when window_right >= 0); causal is (-1, 0).  The pages name
window_len_left/right and softmax_scale as the constructor arguments of
FlashAttentionVarLen (page "paged flash-attn requires page_block_size",
section Example fix) without defining them further.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def bf16(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def lib_mask(Lq, Lk, wl, wr):
    """Visible-key matrix from textbook band routines (tril/triu offsets)."""
    m = torch.ones(Lq, Lk, dtype=torch.bool)
    if wr >= 0:
        m = m.tril(diagonal=Lk - Lq + wr)
    if wl >= 0:
        m = m.triu(diagonal=Lk - Lq - wl)
    return m


def sdpa_reference(wl):
    """torch fp64 SDPA per sequence with repeat_interleave'd K/V heads."""
    H, Hk = wl.num_heads, wl.num_heads_k
    G = H // Hk
    out = np.zeros((wl.q.shape[0], H, wl.head_dim))
    valid_rows = np.zeros((wl.q.shape[0],), dtype=bool)
    for b in range(wl.batch):
        q0, q1 = int(wl.cu_seqlens_q[b]), int(wl.cu_seqlens_q[b + 1])
        Lq, Lk = q1 - q0, int(wl.lens_k[b])
        if wl.paged:
            P = wl.page_block_size
            rows_k = [wl.k[wl.block_table[b, j // P], j % P] for j in range(Lk)]
            rows_v = [wl.v[wl.block_table[b, j // P], j % P] for j in range(Lk)]
            kb = torch.stack(rows_k) if Lk else torch.zeros(0, Hk, wl.head_dim)
            vb = torch.stack(rows_v) if Lk else torch.zeros(0, Hk, wl.head_dim)
        else:
            k0 = int(wl.cu_seqlens_k[b])
            kb, vb = wl.k[k0:k0 + Lk], wl.v[k0:k0 + Lk]
        if Lq == 0:
            continue
        mask = lib_mask(Lq, Lk, wl.window_left, wl.window_right)
        rows_ok = mask.any(dim=1)
        valid_rows[q0:q1] = rows_ok.numpy()
        if Lk == 0 or not rows_ok.any():
            continue
        qh = wl.q[q0:q1].double().permute(1, 0, 2)                    # H, Lq, D
        kh = kb.double().repeat_interleave(G, dim=1).permute(1, 0, 2)  # H, Lk, D
        vh = vb.double().repeat_interleave(G, dim=1).permute(1, 0, 2)
        o = torch.nn.functional.scaled_dot_product_attention(
            qh, kh, vh, attn_mask=mask, scale=float(wl.softmax_scale))
        o = o.permute(1, 0, 2).numpy()
        o[~rows_ok.numpy()] = 0.0
        out[q0:q1] = o
    return out, valid_rows


def run(oracle_mod, wl, **kw):
    return oracle_mod.attention_workload(wl, **kw)


# ----------------------------------------------------------------- closed forms

def test_single_visible_key_gives_v_exactly(oracle_mod):
    # window (0, 0) with Lq == Lk: row i sees exactly key i, so p = 1 and out = v_i
    wl = W.make_custom([7, 33, 1], [7, 33, 1], 4, 2, 24, seed=3, window_left=0, window_right=0)
    out, lse = run(oracle_mod, wl)
    G = 2
    v = wl.v.double().numpy()
    q = wl.q.double().numpy()
    k = wl.k.double().numpy()
    for t in range(wl.q.shape[0]):
        for h in range(4):
            assert np.array_equal(out[t, h], v[t, h // G])
            s = float(wl.softmax_scale) * float(np.dot(q[t, h], k[t, h // G]))
            assert lse[h, t] == pytest.approx(s, rel=1e-13, abs=1e-13)


def test_single_visible_key_paged_decode(oracle_mod):
    # decode row with window_left 0: only the newest key (position Lk-1) is visible
    wl = W.make_custom([1, 1, 1], [5, 64, 100], 2, 1, 16, seed=4, page=32, window_left=0,
                       window_right=0)
    out, _ = run(oracle_mod, wl)
    for b in range(3):
        Lk = int(wl.lens_k[b])
        blk, slot = wl.block_table[b, (Lk - 1) // 32], (Lk - 1) % 32
        for h in range(2):
            assert np.array_equal(out[b, h], wl.v[blk, slot, 0].double().numpy())


def test_uniform_v_gives_that_row(oracle_mod):
    wl = W.make_custom([9, 20], [30, 20], 4, 4, 32, seed=5, window_left=3, window_right=1)
    c = W.normal_bf16(np.random.Generator(np.random.PCG64(9)), (4, 32))
    wl.v[:] = c
    out, _ = run(oracle_mod, wl)
    _, valid = sdpa_reference(wl)
    assert valid.all()
    np.testing.assert_allclose(out, np.broadcast_to(c.double().numpy(), out.shape), rtol=1e-14,
                               atol=1e-14)


def test_zero_q_gives_mean_of_visible_rows(oracle_mod):
    wl = W.make_custom([12, 3, 40], [12, 19, 40], 6, 3, 8, seed=6, window_left=5, window_right=2)
    wl.q.zero_()
    out, lse = run(oracle_mod, wl)
    for b in range(wl.batch):
        q0, Lq, Lk = int(wl.cu_seqlens_q[b]), int(wl.lens_q[b]), int(wl.lens_k[b])
        k0 = int(wl.cu_seqlens_k[b])
        m = lib_mask(Lq, Lk, 5, 2).numpy()
        vb = wl.v[k0:k0 + Lk].double().numpy()
        for i in range(Lq):
            n = m[i].sum()
            for h in range(6):
                if n == 0:
                    assert np.all(out[q0 + i, h] == 0) and lse[h, q0 + i] == -np.inf
                    continue
                np.testing.assert_allclose(out[q0 + i, h], vb[m[i], h // 2].mean(axis=0),
                                           rtol=1e-13, atol=1e-14)
                assert lse[h, q0 + i] == pytest.approx(math.log(n), rel=1e-14)


def test_scale_zero_is_uniform_average(oracle_mod):
    wl = W.make_custom([10], [10], 2, 1, 16, seed=7, scale=0.0)
    out, _ = run(oracle_mod, wl)
    v = wl.v.double().numpy()
    for i in range(10):
        np.testing.assert_allclose(out[i, 0], v[: i + 1, 0].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_two_keys_logistic_closed_form(oracle_mod):
    wl = W.make_custom([1], [2], 1, 1, 8, seed=8, window_right=-1)
    out, lse = run(oracle_mod, wl)
    q = wl.q[0, 0].double().numpy()
    k = wl.k[:, 0].double().numpy()
    v = wl.v[:, 0].double().numpy()
    s0 = float(wl.softmax_scale) * q.dot(k[0])
    s1 = float(wl.softmax_scale) * q.dot(k[1])
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    np.testing.assert_allclose(out[0, 0], w0 * v[0] + w1 * v[1], rtol=1e-13, atol=1e-14)
    assert lse[0, 0] == pytest.approx(max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))), rel=1e-13)


def test_no_visible_key_rows_are_zero(oracle_mod):
    # Lq > Lk under causal: the first Lq-Lk rows see nothing; Lk = 0 sees nothing
    wl = W.make_custom([6, 3], [2, 0], 2, 1, 8, seed=9)
    out, lse = run(oracle_mod, wl)
    assert np.all(out[0:4] == 0) and np.all(lse[:, 0:4] == -np.inf)
    assert np.all(out[6:9] == 0) and np.all(lse[:, 6:9] == -np.inf)
    assert np.all(np.isfinite(lse[:, 4:6]))


# ----------------------------------------------------------- library routine

@pytest.mark.parametrize("case", [
    dict(lq=[17, 64, 5], lk=[17, 64, 5], H=4, Hk=2, D=64, wl=-1, wr=0),        # config 1 shape
    dict(lq=[1, 1, 1, 1], lk=[50, 7, 128, 1], H=8, Hk=2, D=32, wl=-1, wr=0),   # decode
    dict(lq=[5, 30, 9], lk=[40, 30, 70], H=6, Hk=3, D=40, wl=11, wr=0),        # chunked + window
    dict(lq=[20, 8], lk=[20, 30], H=2, Hk=2, D=16, wl=4, wr=3),               # two-sided window
    dict(lq=[9, 14], lk=[31, 14], H=4, Hk=1, D=24, wl=-1, wr=-1),             # no mask, MQA
    dict(lq=[12, 4], lk=[5, 0], H=2, Hk=1, D=8, wl=-1, wr=0),                 # Lq > Lk, empty
    dict(lq=[7, 19], lk=[30, 19], H=3, Hk=1, D=13, wl=5, wr=-1),              # odd head dim
])
@pytest.mark.parametrize("paged", [False, True])
def test_matches_torch_sdpa_fp64(oracle_mod, case, paged):
    wl = W.make_custom(case["lq"], case["lk"], case["H"], case["Hk"], case["D"], seed=11,
                       page=32 if paged else 0, window_left=case["wl"], window_right=case["wr"])
    out, _ = run(oracle_mod, wl)
    ref, valid = sdpa_reference(wl)
    np.testing.assert_allclose(out[valid], ref[valid], rtol=1e-12, atol=1e-13)
    assert np.all(out[~valid] == 0)


def test_config1_matches_torch_sdpa_fp64(oracle_mod):
    wl = W.make_config("c1")
    out, _ = run(oracle_mod, wl)
    ref, valid = sdpa_reference(wl)
    assert valid.all()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    # causal with Lq == Lk is the textbook lower-triangular mask
    for L in (17, 64, 5):
        assert torch.equal(lib_mask(L, L, -1, 0), torch.ones(L, L, dtype=torch.bool).tril())


# ------------------------------------------------------------ mask, one-hot

@pytest.mark.parametrize("Lq,Lk,wl_,wr_", [(5, 9, -1, 0), (9, 5, -1, 0), (8, 8, 2, 1),
                                          (3, 12, 4, -1), (7, 7, 0, 0), (6, 10, -1, -1),
                                          (4, 20, 3, 2),
                                          # windows at the int32 limit act as no limit,
                                          # also on rows before the first key (Lq > Lk)
                                          (9, 5, 2 ** 31 - 1, 0), (5, 9, -1, 2 ** 31 - 1),
                                          (9, 5, 2 ** 31 - 1, 2 ** 31 - 1), (9, 5, 3, 2 ** 31 - 2)])
def test_visible_set_equals_band_matrix(oracle_mod, Lq, Lk, wl_, wr_):
    # Q = 0 and V[j, d] = [j == d]: out[i, d] = 1/n_i exactly where key d is visible
    wl = W.make_custom([Lq], [Lk], 1, 1, Lk, seed=12, window_left=wl_, window_right=wr_)
    wl.q.zero_()
    wl.k.zero_()
    wl.v.copy_(torch.eye(Lk).to(torch.bfloat16).reshape(Lk, 1, Lk))
    out, _ = run(oracle_mod, wl)
    vis = out[:, 0, :] > 0
    assert np.array_equal(vis, lib_mask(Lq, Lk, wl_, wr_).numpy())


# ------------------------------------------------------ mpmath brute force

def test_mpmath_50_digits_tiny(oracle_mod):
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    wl = W.make_custom([3, 5], [6, 5], 2, 1, 4, seed=13, window_left=2, window_right=0, page=32)
    out, lse = run(oracle_mod, wl)
    for b in range(2):
        q0, Lq, Lk = int(wl.cu_seqlens_q[b]), int(wl.lens_q[b]), int(wl.lens_k[b])
        kb = [wl.k[wl.block_table[b, 0], j, 0].double().tolist() for j in range(Lk)]
        vb = [wl.v[wl.block_table[b, 0], j, 0].double().tolist() for j in range(Lk)]
        vis = lib_mask(Lq, Lk, 2, 0)
        for i in range(Lq):
            for h in range(2):
                qv = wl.q[q0 + i, h].double().tolist()
                js = [j for j in range(Lk) if vis[i, j]]
                sc = mpmath.mpf(float(wl.softmax_scale))
                e = {j: mpmath.exp(sc * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(c)
                                                    for a, c in zip(qv, kb[j]))) for j in js}
                z = mpmath.fsum(e.values())
                for d in range(4):
                    exact = mpmath.fsum(e[j] * mpmath.mpf(vb[j][d]) for j in js) / z
                    assert abs(out[q0 + i, h, d] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))
                assert abs(lse[h, q0 + i] - float(mpmath.log(z))) <= 1e-12


# --------------------------------------------------------------- invariants

def _to_packed(wl):
    """Same logical K/V as a paged workload, laid out as packed rank-3 rows."""
    P = wl.page_block_size
    ks, vs = [], []
    for b in range(wl.batch):
        for j in range(int(wl.lens_k[b])):
            ks.append(wl.k[wl.block_table[b, j // P], j % P])
            vs.append(wl.v[wl.block_table[b, j // P], j % P])
    return W.Workload(name="packed", seed=wl.seed, q=wl.q, k=torch.stack(ks), v=torch.stack(vs),
                      cu_seqlens_q=wl.cu_seqlens_q, cu_seqlens_k=wl.cu_seqlens_k,
                      block_table=None, page_block_size=0, softmax_scale=wl.softmax_scale,
                      window_left=wl.window_left, window_right=wl.window_right)


def test_paged_equals_packed_bit_exact(oracle_mod):
    wl = W.make_custom([3, 40, 1, 17], [70, 40, 33, 100], 8, 2, 32, seed=14, page=32,
                       window_left=20, window_right=0)
    o1, l1 = run(oracle_mod, wl)
    o2, l2 = run(oracle_mod, _to_packed(wl))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_block_permutation_invariance_bit_exact(oracle_mod):
    wl = W.make_custom([2, 9], [90, 70], 4, 2, 16, seed=15, page=32, spare=0.5)
    o1, l1 = run(oracle_mod, wl)
    rng = np.random.Generator(np.random.PCG64(99))
    nb = wl.k.shape[0]
    perm = rng.permutation(nb)             # new physical id of old block i is perm[i]
    k2 = torch.empty_like(wl.k)
    v2 = torch.empty_like(wl.v)
    k2[torch.from_numpy(perm)] = wl.k
    v2[torch.from_numpy(perm)] = wl.v
    bt2 = perm[wl.block_table].astype(np.int32)
    wl2 = W.Workload(name="perm", seed=0, q=wl.q, k=k2, v=v2, cu_seqlens_q=wl.cu_seqlens_q,
                     cu_seqlens_k=wl.cu_seqlens_k, block_table=bt2, page_block_size=32,
                     softmax_scale=wl.softmax_scale, window_left=-1, window_right=0)
    o2, l2 = run(oracle_mod, wl2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_gqa_equals_repeated_kv_heads_bit_exact(oracle_mod):
    wl = W.make_custom([5, 12], [5, 30], 8, 2, 16, seed=16, window_left=6, window_right=1)
    o1, l1 = run(oracle_mod, wl)
    wl2 = W.Workload(name="mha", seed=0, q=wl.q, k=wl.k.repeat_interleave(4, dim=1),
                     v=wl.v.repeat_interleave(4, dim=1), cu_seqlens_q=wl.cu_seqlens_q,
                     cu_seqlens_k=wl.cu_seqlens_k, block_table=None, page_block_size=0,
                     softmax_scale=wl.softmax_scale, window_left=6, window_right=1)
    o2, l2 = run(oracle_mod, wl2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_batch_equals_concatenated_single_calls_bit_exact(oracle_mod):
    wl = W.make_custom([4, 1, 9], [11, 6, 9], 4, 2, 8, seed=17, window_left=-1, window_right=0)
    o1, l1 = run(oracle_mod, wl)
    for b in range(3):
        q0, q1 = int(wl.cu_seqlens_q[b]), int(wl.cu_seqlens_q[b + 1])
        k0, k1 = int(wl.cu_seqlens_k[b]), int(wl.cu_seqlens_k[b + 1])
        one = W.Workload(name="one", seed=0, q=wl.q[q0:q1], k=wl.k[k0:k1], v=wl.v[k0:k1],
                         cu_seqlens_q=np.array([0, q1 - q0], np.int32),
                         cu_seqlens_k=np.array([0, k1 - k0], np.int32), block_table=None,
                         page_block_size=0, softmax_scale=wl.softmax_scale, window_left=-1,
                         window_right=0)
        o2, l2 = run(oracle_mod, one)
        assert np.array_equal(o1[q0:q1], o2) and np.array_equal(l1[:, q0:q1], l2)


def test_token_selection_matches_full_call(oracle_mod):
    wl = W.make_custom([6, 10], [20, 10], 2, 1, 8, seed=18)
    o1, l1 = run(oracle_mod, wl)
    sel = np.zeros(16, np.uint8)
    sel[[0, 5, 7, 15]] = 1
    o2, l2 = run(oracle_mod, wl, token_sel=sel)
    idx = np.flatnonzero(sel)
    assert np.array_equal(o1[idx], o2[idx]) and np.array_equal(l1[:, idx], l2[:, idx])
    assert np.isnan(o2[np.flatnonzero(sel == 0)]).all()


def test_thread_count_does_not_change_result(oracle_mod):
    wl = W.make_custom([30, 7], [64, 90], 4, 2, 32, seed=19, page=32)
    o1, l1 = run(oracle_mod, wl, nthreads=1)
    o2, l2 = run(oracle_mod, wl, nthreads=5)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_rejects_block_ids_outside_pool(oracle_mod):
    wl = W.make_custom([1], [40], 1, 1, 8, seed=20, page=32)
    wl.block_table[0, 1] = wl.k.shape[0]
    with pytest.raises(ValueError):
        run(oracle_mod, wl)
