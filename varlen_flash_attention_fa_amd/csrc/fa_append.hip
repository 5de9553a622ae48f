// Paged K/V cache append for gfx950: scatter the new tokens' K and V rows into
// the pool blocks that each sequence's block table names.
//
// The new tokens of sequence b are its last Lnew_b keys: new token j sits at
// logical key position Lk_b - Lnew_b + j, the same bottom-right alignment the
// attention uses for its query rows, and logical position n of sequence b
// lives in block block_table[b][n / P], slot n % P (pages "flash-attn-varlen
// paged expects k/v tensors of rank 4" and "page_block_size ... does not match
// k shape", What it means).
//
// The work is a pure copy, bound by HBM: one lane moves one 16-byte unit of K
// and the same unit of V (8 bf16 of one head row), so a wave reads and writes
// 1 KiB of contiguous row data per tensor.  A workgroup covers one tile of
// units (no grid-stride loop: the grid covers all units).  Each lane first
// issues the loads of its new rows (their addresses need only the unit index);
// meanwhile one lane per token of the tile finds the token's sequence by a
// binary search over cu_seqlens_new (staged with cu_seqlens_k in LDS when the
// batch is small) and its block and slot from the block table, into LDS; then
// every lane stores its rows there.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "../../include/fa_varlen.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kAppendUnroll = 4;      // units per lane per tile
constexpr int kAppendMetaMax = 8;     // cu entries staged per lane: batch+1 <= 8 * 256 in LDS

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool LDS>
__device__ __forceinline__ int32_t meta(const int32_t* g, const int32_t* s, int i) {
    if constexpr (LDS) return s[i];
    else return g[i];
}

// META = entries of cu_seqlens_new / cu_seqlens_k that each lane stages in LDS
// (1 or 8); 0 = the lookup searches them in global memory (large batches).
template <bool VEC, int META>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(AppendParams p) {
    constexpr bool LDS = META > 0;
    constexpr int kTile = kAppendThreads * kAppendUnroll;  // units per workgroup
    extern __shared__ int32_t s_meta[];  // [batch+1] cu_new, then [batch+1] cu_k (LDS only)
    __shared__ int32_t s_blk[kTile];     // per token of the tile: block id (-1 = skip)
    __shared__ int32_t s_slot[kTile];    //                        slot in the block
    int32_t* s_cn = s_meta;
    int32_t* s_ck = s_meta + (p.batch + 1);
    // 0. sequence offsets first: loads complete in issue order, so loads issued
    //    after the row loads could only be waited for together with them
    int32_t m_cn[LDS ? META : 1], m_ck[LDS ? META : 1];
    if constexpr (LDS) {
#pragma unroll
        for (int m = 0; m < META; ++m) {
            const int i = min((int)threadIdx.x + m * kAppendThreads, p.batch);
            m_cn[m] = p.cu_new[i];
            m_ck[m] = p.cu_k[i];
        }
        __builtin_amdgcn_sched_barrier(0);  // keep them ahead of the row loads
    }
    constexpr int E = VEC ? 8 : 1;  // elements per unit
    using Unit = typename std::conditional<VEC, u32x4, uint16_t>::type;
    const uint32_t per_tok = (uint32_t)p.Hk * (uint32_t)p.upr;
    const uint32_t tile = blockIdx.x * (uint32_t)kTile;
    const uint32_t t_first = tile / per_tok;
    const uint32_t t_end = (min(tile + (uint32_t)kTile, p.units) - 1) / per_tok + 1;

    // 1. the source rows depend only on the unit index: issue their loads first,
    //    so they overlap the sequence lookup and the block-table read.  Lanes past
    //    the last unit load the last unit again (no branch around the loads, which
    //    would make the compiler wait for each one) and do not store it.
    Unit kv[kAppendUnroll], vv[kAppendUnroll];
#pragma unroll
    for (int u = 0; u < kAppendUnroll; ++u) {
        const uint32_t idx = min(tile + (uint32_t)(u * kAppendThreads) + threadIdx.x, p.units - 1);
        const uint32_t t = idx / per_tok;
        const uint32_t r = idx - t * per_tok;
        const uint32_t h = r / (uint32_t)p.upr;
        const uint32_t e = (r - h * (uint32_t)p.upr) * E;
        kv[u] = *reinterpret_cast<const Unit*>(p.k_new + (int64_t)t * p.kn_s0 + (int64_t)h * p.kn_s1 + e);
        vv[u] = *reinterpret_cast<const Unit*>(p.v_new + (int64_t)t * p.vn_s0 + (int64_t)h * p.vn_s1 + e);
    }
    // 2. sequence offsets into LDS (small batches)
    if constexpr (LDS) {
#pragma unroll
        for (int m = 0; m < META; ++m) {
            const int i = (int)threadIdx.x + m * kAppendThreads;
            if (i <= p.batch) {
                s_cn[i] = m_cn[m];
                s_ck[i] = m_ck[m];
            }
        }
        __syncthreads();
    }
    // 3. destination of each token of the tile, one lane per token.  A token that
    //    lies in no sequence, or whose position or block id falls outside the
    //    table or the pool, is skipped.
    const int64_t max_pos = (int64_t)p.bt_width * p.page;
    for (uint32_t i = threadIdx.x; i < t_end - t_first; i += kAppendThreads) {
        const uint32_t t = t_first + i;
        int32_t blk = -1, slot = 0;
        // last sequence whose first new token is <= t
        int lo = 0, hi = p.batch;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (meta<LDS>(p.cu_new, s_cn, mid) <= (int32_t)t) lo = mid;
            else hi = mid - 1;
        }
        const int b = lo;
        if (b < p.batch) {
            const int64_t n0 = meta<LDS>(p.cu_new, s_cn, b), n1 = meta<LDS>(p.cu_new, s_cn, b + 1);
            const int64_t lk = (int64_t)meta<LDS>(p.cu_k, s_ck, b + 1) - meta<LDS>(p.cu_k, s_ck, b);
            const int64_t pos = lk - (n1 - n0) + ((int64_t)t - n0);
            if ((int64_t)t >= n0 && (int64_t)t < n1 && pos >= 0 && pos < max_pos) {
                const int32_t id = p.bt[(int64_t)b * p.bt_s0 + pos / p.page];
                if (id >= 0 && id < p.num_blocks) {
                    blk = id;
                    slot = (int32_t)(pos % p.page);
                }
            }
        }
        s_blk[i] = blk;
        s_slot[i] = slot;
    }
    __syncthreads();
    // 4. stores
#pragma unroll
    for (int u = 0; u < kAppendUnroll; ++u) {
        const uint32_t idx = tile + (uint32_t)(u * kAppendThreads) + threadIdx.x;
        if (idx >= p.units) continue;
        const uint32_t t = idx / per_tok;
        const int64_t blk = s_blk[t - t_first];
        if (blk < 0) continue;
        const int64_t slot = s_slot[t - t_first];
        const uint32_t r = idx - t * per_tok;
        const uint32_t h = r / (uint32_t)p.upr;
        const int64_t e = (int64_t)(r - h * (uint32_t)p.upr) * E;
        *reinterpret_cast<Unit*>(p.k_cache + blk * p.kc_s0 + slot * p.kc_s1 + (int64_t)h * p.kc_s2 + e) = kv[u];
        *reinterpret_cast<Unit*>(p.v_cache + blk * p.vc_s0 + slot * p.vc_s1 + (int64_t)h * p.vc_s2 + e) = vv[u];
    }
}

template <bool VEC, int META>
hipError_t launch_append(const AppendParams& p, hipStream_t s) {
    const uint32_t per_wg = kAppendThreads * kAppendUnroll;
    const uint32_t grid = (p.units + per_wg - 1) / per_wg;
    const size_t lds = META > 0 ? 2u * (size_t)(p.batch + 1) * sizeof(int32_t) : 0;
    hipLaunchKernelGGL((kv_append_kernel<VEC, META>), dim3(grid), dim3(kAppendThreads), lds, s, p);
    return hipGetLastError();
}

template <bool VEC>
hipError_t launch_append_meta(const AppendParams& p, hipStream_t s) {
    if (p.batch + 1 <= kAppendThreads) return launch_append<VEC, 1>(p, s);
    if (p.batch + 1 <= kAppendMetaMax * kAppendThreads) return launch_append<VEC, kAppendMetaMax>(p, s);
    return launch_append<VEC, 0>(p, s);
}

thread_local hipError_t g_append_last = hipSuccess;  // per calling thread, like the error text

}  // namespace

int launch_kv_append(const AppendParams& p, void* stream, void* ev_start, void* ev_stop) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (p.units == 0) return 0;
    if (ev_start) e = hipEventRecord(static_cast<hipEvent_t>(ev_start), s);
    if (e == hipSuccess) e = p.vec ? launch_append_meta<true>(p, s) : launch_append_meta<false>(p, s);
    if (e == hipSuccess && ev_stop) e = hipEventRecord(static_cast<hipEvent_t>(ev_stop), s);
    g_append_last = e;
    return e == hipSuccess ? 0 : FA_ERR_HIP;
}

const char* last_append_error() { return hipGetErrorString(g_append_last); }

}  // namespace fa
