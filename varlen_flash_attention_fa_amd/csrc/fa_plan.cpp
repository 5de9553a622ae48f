// Host launch planner of the varlen forward: from the call's shapes alone
// (never the sequence lengths, which live on the device) it picks the kernel
// configuration (prefill or decode tiles), whether and how keys are split into
// chunks, an upper bound of the work list, and the workspace layout.  Plain
// host C++ that launches nothing and calls no HIP function, so it also builds
// with a host compiler (the sanitizer test of the contract and the planner).
#include <algorithm>
#include <climits>
#include <cstdlib>
#include <cstring>

#include "../../include/fa_varlen.h"
#include "fa_internal.h"

namespace fa {
namespace {

int env_int(const char* name, int dflt) {
    const char* s = std::getenv(name);
    if (!s || !*s) return dflt;
    return std::atoi(s);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

int make_plan(const Shapes& s, Plan* plan) {
    Plan P;
    std::memset(&P, 0, sizeof P);
    P.dp = s.D <= 64 ? 64 : s.D <= 128 ? 128 : s.D <= 256 ? 256 : 512;
    const int64_t G = s.H / s.Hk;
    const int64_t batch = std::max<int64_t>(1, s.batch);
    const int64_t rows_avg = (s.total_q * G + batch - 1) / batch;  // rows per (sequence, kv head)
    int kind = rows_avg <= 64 ? KIND_DECODE : KIND_PREFILL;
    const char* force = std::getenv("FA_FORCE_PATH");
    if (force && std::strcmp(force, "prefill") == 0) kind = KIND_PREFILL;
    if (force && std::strcmp(force, "decode") == 0) kind = KIND_DECODE;
    P.kind = kind;
    if (kind == KIND_PREFILL) {
        P.mr = P.dp <= 256 ? 32 : 16;
        P.wr = 4;
        P.bn = P.dp <= 128 ? 64 : 32;
        P.chunk = INT_MAX;
        P.chunk_min = INT_MAX;
        P.adapt = false;
        P.max_chunks = 1;
        // Only a work list too short to fill one round of resident workgroups
        // (a few row tiles over long key ranges) has its keys cut into chunks,
        // merged by the combine kernel: about 1536 work units in all, chunks of at
        // least 2048 keys.  Longer lists are balanced by the planner's
        // largest-first order alone; splitting them only adds partials and the
        // combine (a 16-sequence chunked prefill over 8k-key caches: 0.37 ms with
        // halves, 0.35 ms without).
        const int64_t rows = (int64_t)P.mr * P.wr;
        const int64_t items = ((s.total_q * G + rows - 1) / rows + s.batch) * s.Hk;
        int64_t chunk = 0;
        if (items < 512 && s.max_lk >= 8192)
            chunk = std::max<int64_t>(2048, (s.max_lk * items / 1536 + P.bn - 1) / P.bn * P.bn);
        chunk = env_int("FA_SPLIT_KEYS", (int)chunk);
        if (chunk > 0) {
            chunk = std::max<int64_t>(P.bn, (chunk + P.bn - 1) / P.bn * P.bn);
            const int64_t mc = (s.max_lk + chunk - 1) / chunk;
            if (mc > 4096) return FA_ERR_ARGUMENT;
            if (mc > 1) {
                P.chunk = (int)chunk;
                P.chunk_min = (int)chunk;
                P.max_chunks = (int)mc;
            }
        }
    } else {
        P.mr = 16;
        P.wr = rows_avg <= 16 ? 1 : 4;
        P.bn = 32;
        // base chunk; the planner may resize it from half to twice (a forced size
        // is kept)
        const int forced = env_int("FA_SPLIT_KEYS", 0);
        int chunk = forced > 0 ? forced : 1024;
        if (chunk < P.bn) chunk = P.bn;
        chunk = (chunk + P.bn - 1) / P.bn * P.bn;
        P.chunk = chunk;
        P.adapt = forced <= 0;
        P.chunk_min = P.adapt ? std::max(P.bn, (chunk / 2 + P.bn - 1) / P.bn * P.bn) : chunk;
        const int64_t mc = std::max<int64_t>(1, (s.max_lk + P.chunk_min - 1) / P.chunk_min);
        if (mc > 4096) return FA_ERR_ARGUMENT;
        P.max_chunks = (int)mc;
        if (P.max_chunks == 1) {
            P.chunk = P.chunk_min = INT_MAX;
            P.adapt = false;
        }
    }
    P.rows = P.mr * P.wr;
    const int64_t tiles = (s.total_q * G + P.rows - 1) / P.rows + s.batch;
    const int64_t items = tiles * P.max_chunks;
    if (items >= INT32_MAX / 2 || s.Hk > 65535) return FA_ERR_ARGUMENT;
    // runs of units per XCD: whole heads when Hk is a multiple of 8, else runs of
    // 8 units (neighbouring items of one head for Hk = 1)
    P.xcd_chunk = (s.Hk % 8 == 0) ? 1 : 8;
    // A call with a few sequences and no key split needs no work list: its
    // workgroups read their sequence's offsets themselves (a planner launch is
    // about as long as the attention of such a call).  The grid is sized for any
    // split of total_q over the sequences; workgroups past a sequence's row tiles exit.
    // FA_DIRECT=0 keeps the planner for every call.
    P.direct_tiles = (s.total_q * G + P.rows - 1) / P.rows;
    P.direct = P.max_chunks == 1 && s.batch > 0 && s.batch <= kDirectMaxBatch &&
               s.batch * P.direct_tiles * s.Hk <= 4096 && env_int("FA_DIRECT", 1) != 0;
    if ((items * s.Hk + 64) * 8 >= (int64_t)UINT32_MAX / 2) return FA_ERR_ARGUMENT;
    P.items_bound = items;
    // workspace: [split partials o][split partials lse][items][count][seq offsets]
    size_t off = 0;
    if (P.max_chunks > 1) {
        off += (size_t)P.max_chunks * (size_t)s.total_q * (size_t)s.H * (size_t)P.dp * 4u;
        off += (size_t)P.max_chunks * (size_t)s.total_q * (size_t)s.H * 4u;
    }
    off = align256(off);
    P.off_items = off;
    off = align256(off + (size_t)items * 32u);
    P.off_count = off;
    off = align256(off + 4u);
    P.off_seq = off;
    off = align256(off + (size_t)(s.batch + 1) * 4u);
    P.off_tok = off;
    if (P.max_chunks > 1) off = align256(off + (size_t)s.total_q * 4u);
    P.ws_bytes = off;
    *plan = P;
    return 0;
}

}  // namespace fa
