// Host-only driver of the library's argument contract and launch planner, built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py (no GPU: every call here either fails a check
// or returns before any device work).  Each case states the status it must
// return; a mismatch, or any sanitizer report, fails the test.
#include <climits>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/fa_varlen.h"
#include "../../varlen_flash_attention_fa_amd/csrc/fa_internal.h"

namespace {

int g_bad = 0;

fa_tensor T(std::initializer_list<long long> shape, int32_t dtype = FA_DTYPE_BF16,
            std::initializer_list<long long> stride = {}, void* data = nullptr) {
    fa_tensor t;
    std::memset(&t, 0, sizeof t);
    t.data = data;
    t.dtype = dtype;
    t.rank = (int32_t)shape.size();
    int i = 0;
    for (long long s : shape) t.shape[i++ & 3] = s;
    if (stride.size()) {
        i = 0;
        for (long long s : stride) t.stride[i++ & 3] = s;
    } else {
        long long acc = 1;
        for (int d = t.rank - 1; d >= 0; --d) {
            t.stride[d & 3] = acc;
            acc *= t.shape[d & 3] > 0 ? t.shape[d & 3] : 1;
        }
    }
    return t;
}

void expect(const char* what, int got, int want) {
    if (got != want) {
        std::printf("MISMATCH %s: status %d, expected %d (%s)\n", what, got, want, fa_last_error());
        ++g_bad;
    }
}

}  // namespace

int main() {
    const int I = FA_DTYPE_I32, F16 = FA_DTYPE_F16, F32 = FA_DTYPE_F32;
    fa_tensor Q = T({86, 4, 64}), K3 = T({86, 2, 64}), KP = T({10, 32, 2, 64}), BT = T({3, 4}, I);

    // valid calls and each quoted check in order
    expect("valid packed", fa_varlen_check(&Q, &K3, &K3, &Q, 3, nullptr, 0, nullptr), FA_OK);
    expect("valid paged", fa_varlen_check(&Q, &KP, &KP, &Q, 3, &BT, 32, nullptr), FA_OK);
    fa_tensor q4 = T({2, 86, 4, 64});
    expect("rank3", fa_varlen_check(&q4, &K3, &K3, nullptr, 3, nullptr, 0, nullptr), FA_ERR_RANK);
    fa_tensor q0 = T({});
    expect("rank0", fa_varlen_check(&q0, &K3, &K3, nullptr, 3, nullptr, 0, nullptr), FA_ERR_RANK);
    fa_tensor qbad = Q;
    qbad.rank = 9;  // out of range: reported by the rank check, never indexed
    expect("rank9", fa_varlen_check(&qbad, &K3, &K3, nullptr, 3, nullptr, 0, nullptr), FA_ERR_RANK);
    qbad.rank = -3;
    expect("rank-3", fa_varlen_check(&qbad, &K3, &K3, nullptr, 3, nullptr, 0, nullptr), FA_ERR_RANK);
    expect("rank4 paged", fa_varlen_check(&Q, &K3, &K3, nullptr, 3, &BT, 32, nullptr), FA_ERR_RANK);
    fa_tensor qs = T({86, 4, 64}, FA_DTYPE_BF16, {512, 128, 2});
    expect("contig q", fa_varlen_check(&qs, &K3, &K3, nullptr, 3, nullptr, 0, nullptr), FA_ERR_CONTIGUOUS);
    fa_tensor kp2 = T({10, 32, 2, 32});
    expect("paged k/v", fa_varlen_check(&Q, &KP, &kp2, nullptr, 3, &BT, 32, nullptr), FA_ERR_SHAPE);
    expect("no page", fa_varlen_check(&Q, &KP, &KP, nullptr, 3, &BT, 0, nullptr), FA_ERR_PAGE_SIZE);
    expect("page mismatch", fa_varlen_check(&Q, &KP, &KP, nullptr, 3, &BT, 64, nullptr), FA_ERR_PAGE_SIZE);
    fa_tensor k48 = T({10, 48, 2, 64});
    expect("page %32", fa_varlen_check(&Q, &k48, &k48, nullptr, 3, &BT, 48, nullptr), FA_ERR_PAGE_SIZE);
    fa_tensor q520 = T({5, 2, 520}), k520 = T({4, 32, 1, 520});
    expect("head 520", fa_varlen_check(&q520, &k520, &k520, nullptr, 3, &BT, 32, nullptr), FA_ERR_HEAD_DIM);
    fa_tensor kbad = T({86, 2, 32});
    expect("packed k", fa_varlen_check(&Q, &kbad, &K3, nullptr, 3, nullptr, 0, nullptr), FA_ERR_SHAPE);
    // checks beyond the quoted ones
    fa_tensor qi = T({86, 4, 64}, I);
    expect("dtype", fa_varlen_check(&qi, &K3, &K3, nullptr, 3, nullptr, 0, nullptr), FA_ERR_DTYPE);
    fa_tensor qi4 = T({2, 86, 4, 64}, I);
    expect("rank before dtype", fa_varlen_check(&qi4, &K3, &K3, nullptr, 3, nullptr, 0, nullptr), FA_ERR_RANK);
    fa_tensor q3h = T({86, 3, 64});
    expect("heads", fa_varlen_check(&q3h, &K3, &K3, nullptr, 3, nullptr, 0, nullptr), FA_ERR_ARGUMENT);
    expect("batch<0", fa_varlen_check(&Q, &K3, &K3, nullptr, -1, nullptr, 0, nullptr), FA_ERR_ARGUMENT);
    fa_tensor neg = T({86, 2, 64}, FA_DTYPE_BF16, {-128, 64, 1});
    expect("neg stride", fa_varlen_check(&Q, &neg, &neg, nullptr, 3, nullptr, 0, nullptr), FA_ERR_SHAPE);
    fa_tensor big = T({1LL << 40, 4, 64});
    expect("huge total_q", fa_varlen_check(&big, &K3, &K3, nullptr, 3, nullptr, 0, nullptr), FA_ERR_ARGUMENT);
    fa_tensor btw = T({3, 1LL << 30}, I);
    expect("huge table", fa_varlen_check(&Q, &KP, &KP, nullptr, 3, &btw, 32, nullptr), FA_ERR_ARGUMENT);
    fa_tensor bts = T({3, 4}, I, {8, 2});
    expect("table stride", fa_varlen_check(&Q, &KP, &KP, nullptr, 3, &bts, 32, nullptr), FA_ERR_CONTIGUOUS);
    fa_tensor al = T({4}, F32), al2 = T({3, 4}, F32), alb = T({8}, F32), al3 = T({2, 2, 2}, F32);
    expect("alibi", fa_varlen_check(&Q, &K3, &K3, nullptr, 3, nullptr, 0, &al), FA_OK);
    expect("alibi2", fa_varlen_check(&Q, &K3, &K3, nullptr, 3, nullptr, 0, &al2), FA_OK);
    expect("alibi shape", fa_varlen_check(&Q, &K3, &K3, nullptr, 3, nullptr, 0, &alb), FA_ERR_SHAPE);
    expect("alibi rank", fa_varlen_check(&Q, &K3, &K3, nullptr, 3, nullptr, 0, &al3), FA_ERR_SHAPE);
    fa_tensor qf = T({86, 4, 64}, F16), kf = T({86, 2, 64}, F16);
    expect("f16", fa_varlen_check(&qf, &kf, &kf, &qf, 3, nullptr, 0, nullptr), FA_OK);
    expect("mixed", fa_varlen_check(&qf, &K3, &K3, nullptr, 3, nullptr, 0, nullptr), FA_ERR_DTYPE);
    expect("null", fa_varlen_check(nullptr, &K3, &K3, nullptr, 3, nullptr, 0, nullptr), FA_ERR_ARGUMENT);

    // planner through the workspace size, over the shapes of the five workloads
    // and limits (every head dim tier, forced paths, key splits)
    struct WS { long long tq, H, Hk, D, nb, P, batch, width; const char* what; } ws[] = {
        {86, 4, 2, 64, 0, 0, 3, 0, "c1"},
        {64, 32, 8, 128, 4600, 32, 64, 128, "c2"},
        {4104, 32, 8, 128, 1300, 64, 16, 136, "c3"},
        {65536, 64, 8, 128, 0, 0, 8, 0, "c4"},
        {128, 16, 16, 256, 5400, 128, 32, 256, "c5a"},
        {128, 16, 1, 512, 5400, 128, 32, 256, "c5b"},
        {3000, 8, 2, 128, 7000, 32, 3000, 120, "3000 seqs"},
        {73, 8, 2, 13, 700, 64, 2, 313, "short list, odd D"},
        {1, 1, 1, 1, 1, 32, 1, 1, "tiny"},
        {5, 16, 1, 512, 300000, 512, 2, 4000, "long decode, large page"},
    };
    for (const auto& w : ws) {
        fa_tensor q = T({w.tq, w.H, w.D});
        fa_tensor k = w.P ? T({w.nb, w.P, w.Hk, w.D}) : T({w.tq, w.Hk, w.D});
        fa_tensor bt = T({w.batch, w.width}, I);
        size_t bytes = 0;
        expect(w.what, fa_varlen_workspace_bytes(&q, &k, &k, (int32_t)w.batch, w.P ? &bt : nullptr, (int32_t)w.P,
                                                 &bytes), FA_OK);
        if (bytes == 0 || bytes % 256) {
            std::printf("MISMATCH %s: workspace %zu\n", w.what, bytes);
            ++g_bad;
        }
    }
    size_t pb = 0;
    fa_tensor QP = T({2, 5, 4, 64}), KP4 = T({2, 9, 2, 64});
    expect("padded ws", fa_padded_workspace_bytes(&QP, &KP4, &KP4, &pb), FA_OK);
    expect("padded check", fa_padded_check(&QP, &KP4, &KP4, &QP, nullptr), FA_OK);
    fa_tensor QPi = T({2, 5, 4, 64}, I);
    expect("padded dtype", fa_padded_check(&QPi, &KP4, &KP4, nullptr, nullptr), FA_ERR_DTYPE);
    expect("padded rank", fa_padded_check(&Q, &KP4, &KP4, nullptr, nullptr), FA_ERR_RANK);
    expect("ws null", fa_varlen_workspace_bytes(&Q, &K3, &K3, 3, nullptr, 0, nullptr), FA_ERR_ARGUMENT);

    // the forward's early returns and host-side device checks (no GPU here:
    // host pointers are not device memory, so nothing is launched)
    std::vector<uint16_t> host(86 * 4 * 64);
    std::vector<int32_t> cu = {0, 40, 80, 86};
    fa_tensor qh = T({86, 4, 64}, FA_DTYPE_BF16, {}, host.data());
    fa_tensor kh = T({86, 2, 64}, FA_DTYPE_BF16, {}, host.data());
    fa_tensor oh = T({86, 4, 64}, FA_DTYPE_BF16, {}, host.data());
    expect("fwd batch 0", fa_varlen_fwd(&qh, &kh, &kh, &oh, nullptr, nullptr, 0, nullptr, 0, 0.125f, -1, 0,
                                        nullptr, nullptr, nullptr, 0, nullptr), FA_OK);
    expect("fwd host ptrs", fa_varlen_fwd(&qh, &kh, &kh, &oh, cu.data(), cu.data(), 3, nullptr, 0, 0.125f,
                                          INT_MAX, INT_MAX, nullptr, nullptr, nullptr, 0, nullptr), FA_ERR_DEVICE);
    expect("fwd no out", fa_varlen_fwd(&qh, &kh, &kh, nullptr, cu.data(), cu.data(), 3, nullptr, 0, 0.125f, -1, 0,
                                       nullptr, nullptr, nullptr, 0, nullptr), FA_ERR_ARGUMENT);
    expect("static batch 0", fa_varlen_fwd_static(&qh, &kh, &kh, &oh, nullptr, nullptr, 0, nullptr, 0, 0.125f, -1,
                                                  0, nullptr, nullptr, nullptr), FA_OK);
    expect("static host ptrs", fa_varlen_fwd_static(&qh, &kh, &kh, &oh, cu.data(), cu.data(), 3, nullptr, 0, 0.125f,
                                                    -1, 0, nullptr, nullptr, nullptr), FA_ERR_DEVICE);
    expect("static contract", fa_varlen_fwd_static(&q4, &kh, &kh, &oh, cu.data(), cu.data(), 3, nullptr, 0, 0.125f,
                                                   -1, 0, nullptr, nullptr, nullptr), FA_ERR_RANK);
    fa_tensor QP0 = T({0, 5, 4, 64}), KP0 = T({0, 9, 2, 64});
    expect("padded empty", fa_padded_fwd(&QP0, &KP0, &KP0, &QP0, 0.1f, -1, 0, nullptr, nullptr, nullptr, 0,
                                         nullptr), FA_OK);

    // append contract
    fa_tensor KN = T({6, 2, 64}), KC = T({10, 32, 2, 64}), BT3 = T({3, 4}, I);
    expect("append ok", fa_kv_append_check(&KN, &KN, 3, &BT3, &KC, &KC, 32), FA_OK);
    fa_tensor KC48 = T({10, 48, 2, 64});
    expect("append page", fa_kv_append_check(&KN, &KN, 3, &BT3, &KC48, &KC48, 48), FA_ERR_PAGE_SIZE);
    expect("append rank", fa_kv_append_check(&KC, &KN, 3, &BT3, &KC, &KC, 32), FA_ERR_RANK);
    expect("append null", fa_kv_append_check(&KN, &KN, 3, nullptr, &KC, &KC, 32), FA_ERR_ARGUMENT);
    std::vector<int32_t> cun = {0, 2, 4, 6};
    expect("append host", fa_kv_append(&KN, &KN, cun.data(), cu.data(), 3, &BT3, &KC, &KC, 32, nullptr),
           FA_ERR_DEVICE);

    // direct calls (no planner): a few sequences, no key split, a bounded grid;
    // the grid's row tiles cover every split of total_q over the sequences
    struct DC { long long tq, H, Hk, D, max_lk, batch; bool paged; bool direct; long long tiles; const char* what; } dc[] = {
        {86, 4, 2, 64, 86, 3, false, true, 3, "c1: 3 sequences, decode path"},
        {64, 32, 8, 128, 4096, 64, true, false, 0, "c2: 64 sequences"},
        {4104, 32, 8, 128, 8704, 16, true, false, 0, "c3: 16 sequences, grid over 4096 units"},
        {1024, 8, 2, 128, 1500, 16, false, true, 32, "16 sequences, 1024 rows"},
        {1024, 8, 2, 128, 1500, 17, false, false, 0, "17 sequences"},
        {4, 32, 8, 128, 5000, 4, true, false, 0, "decode with a key split"},
        {4, 32, 8, 128, 512, 4, true, true, 1, "decode, one chunk"},
    };
    for (const auto& c : dc) {
        fa::Shapes sh;
        sh.total_q = c.tq; sh.H = c.H; sh.Hk = c.Hk; sh.D = c.D; sh.max_lk = c.max_lk; sh.batch = c.batch;
        sh.paged = c.paged;
        fa::Plan pl;
        expect(c.what, fa::make_plan(sh, &pl), FA_OK);
        if (pl.direct != c.direct || (c.direct && pl.direct_tiles != c.tiles) ||
            (pl.direct && pl.direct_tiles * pl.rows < c.tq * (c.H / c.Hk))) {
            std::printf("MISMATCH %s: direct %d tiles %lld (rows %d)\n", c.what, (int)pl.direct,
                        (long long)pl.direct_tiles, pl.rows);
            ++g_bad;
        }
    }
    {
        setenv("FA_DIRECT", "0", 1);  // keeps the planner for every call
        fa::Shapes sh;
        sh.total_q = 86; sh.H = 4; sh.Hk = 2; sh.D = 64; sh.max_lk = 86; sh.batch = 3; sh.paged = false;
        fa::Plan pl;
        expect("FA_DIRECT=0", fa::make_plan(sh, &pl), FA_OK);
        if (pl.direct) {
            std::printf("MISMATCH FA_DIRECT=0: direct\n");
            ++g_bad;
        }
        unsetenv("FA_DIRECT");
    }

    std::printf("contract driver: %d mismatches\n", g_bad);
    return g_bad ? 1 : 0;
}
