// gfx950 kernels of the varlen (paged) flash-attention forward, and the host
// planner that picks their launch shapes.
//
// What is computed (the operation named by candle's FlashAttentionVarLen
// forward; layouts from the pages "flash-attn-varlen expects input tensors of
// rank 3" and "flash-attn-varlen paged expects k/v tensors of rank 4",
// sections What it means): for sequence b, query row i, head h,
//   out[i,h,:] = softmax_j(scale * q[i,h,:] . k_b[j,h/G,:]) v_b[j,h/G,:]
// over the keys j visible to row i (window around a = i + Lk - Lq).  Paged
// K/V rows are found through block_table[b][j / P], slot j % P (page
// "page_block_size ... does not match k shape", section What it means).
//
// Work decomposition.  A work item is (sequence b, row tile, key chunk) for one
// K/V head hk (grid.y).  The rows of (b, hk) are the pairs (query i, head g in
// the group) numbered r = i*G + g, so one tile packs all G query heads that
// read the same K/V head and every K/V tile staged in LDS serves all of them.
// Each wave owns MR rows; the workgroup's WR waves share the K/V tiles.
//
// Per wave the scores are computed transposed, S^T = K Q^T, with bf16 (or fp16) MFMA
// (32x32x16 when MR = 32, 16x16x32 when MR = 16): every lane then holds a
// single query row, so row max / row sum are in-lane plus one or two
// cross-lane steps, and the O^T = V^T P^T product takes P straight from the
// score registers.  The rows of the K operand are fed in a permuted key order
// chosen so that the eight keys a lane holds in its score registers are
// exactly the eight keys it must supply as the B operand of the PV MFMA.
// V is transposed once while being staged into LDS.
//
// Online softmax in the log2 domain (scale * log2 e folded in, v_exp_f32),
// fp32 accumulation, P rounded to the input element type for the PV product,
// output rounded to it (round to nearest even).  Keys past a tile's end are zero-filled in LDS
// and masked, so stale or NaN memory is never read.
//
// Split-KV: when a sequence's keys are cut into several chunks, each item
// writes its normalized fp32 partial and log2-sum-exp to the workspace and a
// second kernel merges them (lse-weighted average).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/fa_varlen.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();

// Element types of q/k/v/out: bf16 and IEEE binary16 (fp16), both 16-bit, so
// every layout, copy and LDS pattern is shared; they differ in the MFMA
// instructions, the fp32 -> 16-bit rounding (nearest even) and the packed dot
// used for row sums.
struct EBf16 {
    typedef __bf16 e8 __attribute__((ext_vector_type(8)));
    typedef __bf16 e2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(e8, a), __builtin_bit_cast(e8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(e8, a), __builtin_bit_cast(e8, b), c, 0, 0, 0);
    }
    // two floats -> two bf16 in one v_cvt_pk_bf16_f32
    static __device__ __forceinline__ unsigned int pack2(float a, float b) {
        const f32x2 v = {a, b};
        return __builtin_bit_cast(unsigned int, __builtin_convertvector(v, e2));
    }
    static __device__ __forceinline__ unsigned short one(float a) {
        return __builtin_bit_cast(unsigned short, static_cast<__bf16>(a));
    }
    // acc + both halves of a packed pair (v_dot2_f32_bf16 with ones)
    static __device__ __forceinline__ float sum2(unsigned int pp, float acc) {
        const e2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(e2, pp), ones, acc, false);
    }
};
struct EF16 {
    typedef _Float16 e8 __attribute__((ext_vector_type(8)));
    typedef _Float16 e2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(e8, a), __builtin_bit_cast(e8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(e8, a), __builtin_bit_cast(e8, b), c, 0, 0, 0);
    }
    // two floats -> two fp16 in one v_cvt_pk_f16_f32
    static __device__ __forceinline__ unsigned int pack2(float a, float b) {
        const f32x2 v = {a, b};
        return __builtin_bit_cast(unsigned int, __builtin_convertvector(v, e2));
    }
    static __device__ __forceinline__ unsigned short one(float a) {
        return __builtin_bit_cast(unsigned short, static_cast<_Float16>(a));
    }
    static __device__ __forceinline__ float sum2(unsigned int pp, float acc) {
        const e2 ones = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(e2, pp), ones, acc, false);
    }
};

template <int MR, class E>
struct Mfma;
template <class E>
struct Mfma<32, E> {
    static constexpr int KSTEP = 16;  // contraction length per instruction
    static constexpr int NACC = 16;   // accumulators per lane
    typedef f32x16 acc_t;
    static __device__ __forceinline__ acc_t mma(u32x4 a, u32x4 b, acc_t c) { return E::mma32(a, b, c); }
};
template <class E>
struct Mfma<16, E> {
    static constexpr int KSTEP = 32;
    static constexpr int NACC = 4;
    typedef f32x4 acc_t;
    static __device__ __forceinline__ acc_t mma(u32x4 a, u32x4 b, acc_t c) { return E::mma16(a, b, c); }
};

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Eight bf16 at base[d0 .. d0+8), zero past D.  `vec` promises that base is
// 16-byte aligned whenever d0 is a multiple of 8 and that D % 8 == 0.
__device__ __forceinline__ u32x4 load8(const uint16_t* base, int d0, int D, bool vec) {
    if (vec) {
        if (d0 < D) return *reinterpret_cast<const u32x4*>(base + d0);
        return u32x4{0u, 0u, 0u, 0u};
    }
    unsigned int w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        unsigned int lo = (d0 + 2 * j < D) ? base[d0 + 2 * j] : 0u;
        unsigned int hi = (d0 + 2 * j + 1 < D) ? base[d0 + 2 * j + 1] : 0u;
        w[j] = lo | (hi << 16);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}


// Values of lanes l and l^32 (permlane32 swap) or l and l^16 (permlane16 swap),
// as a pair that is the same on both lanes: one VALU instruction instead of an
// LDS permute.
__device__ __forceinline__ float2 pair_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return float2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float2 pair_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return float2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float max_xor32(float x) { const float2 r = pair_xor32(x); return fmaxf(r.x, r.y); }
__device__ __forceinline__ float max_xor16(float x) { const float2 r = pair_xor16(x); return fmaxf(r.x, r.y); }
__device__ __forceinline__ float sum_xor32(float x) { const float2 r = pair_xor32(x); return r.x + r.y; }
__device__ __forceinline__ float sum_xor16(float x) { const float2 r = pair_xor16(x); return r.x + r.y; }

struct Item {
    int b, rt, c, nc, cl;  // cl: keys per chunk of this call
    int q0, Lq, k0, Lk;
};

// Key ranges are [lo, hi) in sequence-local key positions.
struct Range {
    int lo, hi;
};

// The window edges a - window_left and a + window_right + 1 are formed in 64
// bits: any int32 window is legal (INT32_MAX is a common "no limit"), and with
// a near 2^31 or below 0 (more queries than keys) the 32-bit sums would wrap.
// The clamped results lie in [0, Lk] and fit in int again.
__device__ __forceinline__ Range row_range(const FwdParams& p, int i, int Lq, int Lk) {
    const int64_t a = (int64_t)i + Lk - Lq;
    Range r;
    r.lo = p.window_left >= 0 ? (int)max((int64_t)0, min((int64_t)Lk, a - p.window_left)) : 0;
    r.hi = p.window_right >= 0 ? (int)min((int64_t)Lk, max((int64_t)0, a + p.window_right + 1)) : Lk;
    return r;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0, "vmcnt");
    constexpr int n = N > 63 ? 63 : N;
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// if source lane a points at four consecutive bf16 of row (key0 + a/4),
// columns d0 + 4*(a%4) .. +3, then lane i receives column d0 + i of rows
// key0 .. key0+3: a 4-key slice of V^T.
__device__ __forceinline__ u32x2 lds_read_tr16(const unsigned char* ptr) {
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(ptr));
    return __builtin_bit_cast(u32x2, r);
}

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ unsigned lds_u32(const unsigned char* p) {
    return (unsigned)(size_t)(const __attribute__((address_space(3))) unsigned char*)p;
}

// One 16-byte global -> LDS copy per lane (global_load_lds_dwordx4): lane l's
// data lands at LDS byte address lds + 16*l; lds (in M0) must be wave-uniform.
// Written as inline assembly so the compiler does not treat the copy as an LDS
// store: it would otherwise wait for every copy in flight before any later LDS
// read, which serialises loading the next tile with computing on this one.
// Completion is tracked by the kernel itself (vmcnt waits + barriers).  The
// instruction between the M0 write and the copy is the one wait state the copy
// needs after M0 is written.
__device__ __forceinline__ void copy16_to_lds(const uint16_t* gsrc, unsigned lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(gsrc), "s"(lds) : "m0");
}
// Same, with a wave-uniform 64-bit base and a per-lane 32-bit byte offset.  The
// base is first copied by a scalar move, so the copy never reads an SGPR that a
// vector instruction has just written.
__device__ __forceinline__ void copy16_to_lds_sv(const unsigned char* sbase, unsigned voff, unsigned lds) {
    unsigned long long tmp;
    asm volatile("s_mov_b32 m0, %2\n\ts_mov_b64 %0, %3\n\tglobal_load_lds_dwordx4 %1, %0"
                 : "=&s"(tmp) : "v"(voff), "s"(lds), "s"(sbase) : "m0");
}

constexpr int kPageCap = 256;

// The lane id laundered through an empty asm: values derived from it inside a
// loop are recomputed each iteration instead of being hoisted and kept live
// (keeps register pressure of the unrolled LDS address patterns down).
__device__ __forceinline__ int opaque_lane() {
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    return l;
}  // block-table entries staged in LDS per segment

// Row order of the K operand of the 32x32 S^T product: lane row rho holds key
// kappa(rho) (bits 2 and 3 swapped), so the 8 keys a lane holds in its score
// registers are the 8 it supplies as the B operand of O^T = V^T P^T.
__device__ __forceinline__ int kappa32(int rl) { return (rl & ~12) | ((rl & 4) << 1) | ((rl & 8) >> 1); }

// Sequence b's query rows [q0, q0+Lq) and key count Lk, clamped to the
// tensors the call was given: cu_seqlens contents are not validated, and a bad
// table must not make any kernel address outside q/out, k/v or the block table.
struct SeqSpan {
    int q0, Lq, k0, Lk;
};

__device__ __forceinline__ SeqSpan seq_span(const FwdParams& p, int b) {
    SeqSpan s;
    const bool uq = p.padded != 0;
    const int cq0 = uq ? b * p.uniform_q : p.cu_q[b];
    const int cq1 = uq ? cq0 + p.uniform_q : p.cu_q[b + 1];
    const int q0 = min(max(cq0, 0), p.total_q);
    const int q1 = min(max(cq1, q0), p.total_q);
    s.q0 = q0;
    s.Lq = q1 - q0;
    const bool uk = p.padded != 0;
    const int k0 = uk ? b * p.uniform_k : p.cu_k[b];
    int lk = max(0, (uk ? k0 + p.uniform_k : p.cu_k[b + 1]) - k0);
    if (p.bt) {
        s.k0 = 0;
        lk = p.num_blocks > 0 ? min(lk, p.max_lk) : 0;
    } else {
        s.k0 = min(max(k0, 0), p.max_lk);
        lk = min(lk, p.max_lk - s.k0);
    }
    s.Lk = lk;
    return s;
}

// ---------------------------------------------------------------- planner
//
// One workgroup turns cu_seqlens into the work list of the main kernel:
// sequence b owns ceil(Lq_b*G/R) row tiles times nc_b key chunks.  Items are
// written in decreasing order of estimated cost (visible keys x the workgroup's
// rows, in half-octave buckets); the main kernel's workgroup x handles item x, and
// workgroups are dispatched in index order, so the longest items start first
// and the short ones fill the tail.
constexpr int kPlanThreads = 1024;
constexpr int kCostBuckets = 128;
constexpr int kLdsSeqs = 2048;  // sequences whose spans and item offsets stay in LDS

__device__ __forceinline__ int seq_chunks(const FwdParams& p, int lk, int chunk) {
    return p.max_chunks > 1 ? min(p.max_chunks, max(1, ceil_div(lk, chunk))) : 1;
}

// Candidate chunk sizes for a decode call whose planner may resize the chunk:
// 1/2 .. 2 times the base size, rounded up to whole key tiles.
constexpr int kChunkCands = 9;
constexpr int kBaseCand = 4;  // the candidate equal to the base size
__device__ __forceinline__ int chunk_cand(const FwdParams& p, int k) {
    const int eighths = k <= 4 ? 4 + k : 2 * k;  // 4, 5, 6, 7, 8, 10, 12, 14, 16
    const int c = (int)((int64_t)p.chunk * eighths / 8);
    return max(p.chunk_min, (c + p.chunk_align - 1) / p.chunk_align * p.chunk_align);
}

__device__ __forceinline__ int cost_bucket(int64_t cost) {
    if (cost <= 0) return 0;
    const int lg = 63 - __builtin_clzll((unsigned long long)cost);
    const int half = lg >= 1 ? (int)((cost >> (lg - 1)) & 1) : 0;
    return min(kCostBuckets - 1, 1 + 2 * lg + half);
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const FwdParams p) {
    __shared__ int s_off_lds[kLdsSeqs + 1];
    __shared__ int4 s_span[kLdsSeqs];
    __shared__ int s_wsum[kPlanThreads / 64];
    __shared__ int s_hist[kCostBuckets];
    __shared__ int s_wcnt[kPlanThreads / 64][kCostBuckets];  // per-wave bucket counts of a chunk
    __shared__ unsigned s_cand[kChunkCands];
    __shared__ int s_chunk;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const bool cached = p.batch <= kLdsSeqs;
    int* off = cached ? s_off_lds : p.seq_off;
    const bool split = p.max_chunks > 1;
    const int R = p.rows;

    for (int i = tid; i < kCostBuckets; i += kPlanThreads) s_hist[i] = 0;
    for (int i = tid; i < kCostBuckets * (kPlanThreads / 64); i += kPlanThreads) (&s_wcnt[0][0])[i] = 0;

    // items per sequence -> exclusive offsets off[0..batch] (wave shuffles + one
    // LDS step per 1024 sequences); returns the item count.  The first call stages
    // the sequence spans in LDS (when they fit).
    auto offsets = [&](int ck, bool staged) {
        int carry = 0;
        for (int base = 0; base < p.batch; base += kPlanThreads) {
            const int b = base + tid;
            int cnt = 0;
            if (b < p.batch) {
                const SeqSpan sp = staged ? SeqSpan{s_span[b].x, s_span[b].y, s_span[b].z, s_span[b].w} : seq_span(p, b);
                if (cached && !staged) s_span[b] = make_int4(sp.q0, sp.Lq, sp.k0, sp.Lk);
                cnt = ceil_div(sp.Lq * p.G, R) * seq_chunks(p, sp.Lk, ck);
            }
            int x = cnt;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(x, o, 64);
                if (lane >= o) x += y;
            }
            if (lane == 63) s_wsum[wave] = x;
            __syncthreads();
            if (wave == 0) {
                int w = lane < kPlanThreads / 64 ? s_wsum[lane] : 0;
#pragma unroll
                for (int o = 1; o < kPlanThreads / 64; o <<= 1) {
                    const int y = __shfl_up(w, o, 64);
                    if (lane >= o) w += y;
                }
                if (lane < kPlanThreads / 64) s_wsum[lane] = w;
            }
            __syncthreads();
            const int incl = x + (wave > 0 ? s_wsum[wave - 1] : 0);
            if (b < p.batch) off[b] = carry + incl - cnt;
            carry += s_wsum[kPlanThreads / 64 - 1];
            __syncthreads();
        }
        return carry;
    };
    // Chunk size.  Work items of one call cost about the same, and the hardware
    // runs `slots` of them at a time, so the kernel takes about
    // ceil(items / slots) rounds of (chunk + per-item overhead).  The items are
    // counted with the base chunk first; only when they need more than one round,
    // or fill less than a quarter of one, are the candidates counted and the one
    // with the smallest such estimate taken (fewer keys per item can fill the
    // last round instead of leaving it nearly empty, more keys per item can save
    // a round, and a nearly empty round gains parallelism from smaller items).
    // A round that is at least a quarter full keeps the base chunk: a paged
    // decode batch at half a round ran 98 us with it against 100 us with the
    // candidate, and counting the candidates took 5 us of planner time.
    int chunk = p.chunk;
    int carry = offsets(chunk, false);
    const unsigned slots = (unsigned)max(1, p.slots);
    const unsigned base_units = (unsigned)carry * (unsigned)p.Hk;
    if (split && p.chunk_adapt && (base_units > slots || 4u * base_units < slots)) {
        // item counts of every candidate chunk in one pass over the sequences:
        // lane (j, k) of a wave counts candidate k over its share of the
        // sequences (seven per wave and round), and the partial counts meet in
        // LDS (one add per lane, no cross-lane chains); counts stay below 2^31 /
        // Hk, which the host checks at the smallest candidate
        if (tid < kChunkCands) s_cand[tid] = 0u;
        __syncthreads();
        constexpr int kSlots = 64 / kChunkCands;  // sequence slots per wave
        if (lane < kSlots * kChunkCands) {
            const int k = lane % kChunkCands;
            const int ck = chunk_cand(p, k);
            unsigned cnt = 0u;
            for (int b = wave * kSlots + lane / kChunkCands; b < p.batch; b += (kPlanThreads / 64) * kSlots) {
                const SeqSpan sp = cached ? SeqSpan{s_span[b].x, s_span[b].y, s_span[b].z, s_span[b].w} : seq_span(p, b);
                cnt += (unsigned)(ceil_div(sp.Lq * p.G, R) * seq_chunks(p, sp.Lk, ck));
            }
            if (cnt) atomicAdd(&s_cand[k], cnt);
        }
        __syncthreads();
        if (wave == 0) {  // one candidate per lane of the first 16
            unsigned long long key = ~0ull;  // (estimate, candidate) of this lane
            if (lane < kChunkCands) {
                const unsigned units = s_cand[lane] * (unsigned)p.Hk;
                const unsigned long long est = (unsigned long long)((units + slots - 1) / slots) *
                                               (unsigned long long)(chunk_cand(p, lane) + 2 * R + 64);
                key = (est << 4) | (unsigned long long)lane;
            }
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) {
                const unsigned long long y = __shfl_xor(key, o, 16);
                key = y < key ? y : key;
            }
            if (lane == 0) s_chunk = chunk_cand(p, (int)(key & 15));
        }
        __syncthreads();
        chunk = s_chunk;
        if (chunk != p.chunk) carry = offsets(chunk, cached);
    }
    const int total = min(carry, p.items_bound);
    if (tid == 0) {
        off[p.batch] = carry;
        *p.item_count = total;
    }
    __syncthreads();
    // split partials: chunks per token for the combine (0 = in no sequence); one
    // token per thread, its sequence found by a search over the query offsets
    if (split)
        for (int t = tid; t < p.total_q; t += kPlanThreads) {
            int lo = 0, hi = p.batch;  // last b whose first query row is <= t
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                const int q0 = cached ? s_span[mid].x : seq_span(p, mid).q0;
                if (q0 <= t) lo = mid; else hi = mid;
            }
            int nc = 0;
            if (p.batch > 0) {
                const SeqSpan sp = cached ? SeqSpan{s_span[lo].x, s_span[lo].y, s_span[lo].z, s_span[lo].w} : seq_span(p, lo);
                if (t >= sp.q0 && t < sp.q0 + sp.Lq) nc = seq_chunks(p, sp.Lk, chunk);
            }
            p.tok_nc[t] = nc;
        }

    // decode item i -> (b, rt, c, nc, cost bucket); the first pass counts
    // buckets, the second places each item in its bucket in item order (a stable
    // counting sort: sequence, row tile, chunk), so that the workgroups running
    // together on an XCD take neighbouring row tiles of one sequence and share
    // its K/V window in that XCD's L2.  When one round of threads holds every
    // item, the second pass keeps the first one's records instead of decoding again.
    const bool one_round = total <= kPlanThreads;
    int bucket = -1;
    int4 rec0 = {}, rec1 = {};
    for (int pass = 0; pass < 2; ++pass) {
        for (int base = 0; base < total; base += kPlanThreads) {
            const int i = base + tid;
            if (pass == 0 || !one_round) {
                bucket = -1;
                if (i < total) {
                    int lo = 0, hi = p.batch;  // last b with off[b] <= i
                    while (hi - lo > 1) {
                        const int mid = (lo + hi) >> 1;
                        if (off[mid] <= i) lo = mid; else hi = mid;
                    }
                    const int b = lo;
                    const SeqSpan sp = cached ? SeqSpan{s_span[b].x, s_span[b].y, s_span[b].z, s_span[b].w} : seq_span(p, b);
                    const int lq = sp.Lq, lk = sp.Lk;
                    const int nc = seq_chunks(p, lk, chunk);
                    const int local = i - off[b];
                    const int rt = local / nc, c = local % nc;
                    const int nrows = lq * p.G;
                    const int r0 = rt * R, r1 = min(nrows, r0 + R) - 1;
                    const Range a = row_range(p, r0 / p.G, lq, lk);
                    const Range z = row_range(p, r1 / p.G, lq, lk);
                    int kb = a.lo, ke = z.hi;
                    if (split) {
                        kb = max(kb, c * chunk);
                        ke = min(ke, (c + 1) * chunk);
                    }
                    // every wave of the workgroup computes all its rows for every key tile,
                    // so a partial row tile costs as much as a full one: the keys decide
                    // (rows only break ties)
                    const int nr = r1 - r0 + 1;
                    const int64_t cost = (int64_t)max(0, ke - kb) * R + nr;
                    bucket = cost_bucket(cost);
                    rec0 = make_int4(b, rt, c | (nc << 16), chunk);
                    rec1 = make_int4(sp.q0, sp.Lq, sp.k0, sp.Lk);
                }
            }
            if (pass == 0) {
                if (bucket >= 0) atomicAdd(&s_hist[bucket], 1);
                continue;
            }
            // rank among the earlier items of this wave with the same bucket (one
            // round per distinct bucket in the wave), and the wave's count per bucket
            int rank = 0;
            unsigned long long rem = __ballot(bucket >= 0);
            while (rem) {
                const int leader = __ffsll((long long)rem) - 1;
                const int v = __shfl(bucket, leader, 64);
                const unsigned long long m = __ballot(bucket == v);
                if (bucket == v) rank = __popcll(m & ((1ull << lane) - 1ull));
                if (lane == leader) s_wcnt[wave][v] = __popcll(m);
                rem &= ~m;
            }
            __syncthreads();
            // per bucket: each wave's counts become its first position (after the
            // earlier waves and rounds), and the bucket's next free position moves on
            if (tid < kCostBuckets) {
                int pos = s_hist[tid];
                for (int w = 0; w < kPlanThreads / 64; ++w) {
                    const int n = s_wcnt[w][tid];
                    s_wcnt[w][tid] = pos;
                    pos += n;
                }
                s_hist[tid] = pos;
            }
            __syncthreads();
            if (bucket >= 0) {
                const int pos = s_wcnt[wave][bucket] + rank;
                p.items[2 * pos] = rec0;
                p.items[2 * pos + 1] = rec1;
            }
            // this wave's row back to zero counts for the next round (only this
            // wave reads or writes its row until the next barrier)
            for (int k = lane; k < kCostBuckets; k += 64) s_wcnt[wave][k] = 0;
        }
        __syncthreads();
        if (pass == 0 && wave == 0) {  // bucket starts, most expensive first: one wave scan
            static_assert(kCostBuckets == 128, "two buckets per lane");
            const int k0 = kCostBuckets - 1 - 2 * lane;  // this lane's buckets k0, k0 - 1
            const int c0 = s_hist[k0], c1 = s_hist[k0 - 1];
            int x = c0 + c1;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(x, o, 64);
                if (lane >= o) x += y;
            }
            const int excl = x - c0 - c1;
            s_hist[k0] = excl;
            s_hist[k0 - 1] = excl + c0;
        }
        __syncthreads();
    }
}

// Main attention kernel.
//   DP: head dim padded to 64/128/256/512      MR: rows per wave (MFMA 32x32x16 or 16x16x32)
//   WR: waves per workgroup (they share K/V)    BN: keys per tile     NS: LDS pipeline stages
//   AL: the call has ALiBi slopes               DIRECT: no work list (a few sequences, no key split)
//
// K and V tiles live in LDS row-major ([key][d], DP*2 bytes per row) with the
// 16-byte chunks of row r stored at position (chunk ^ swizzle(r)), so that the
// MFMA operand reads below hit distinct banks.  Tiles start at multiples of BN;
// rows outside [kb, ke) are loaded from the nearest valid row and masked.
template <class E, int DP, int MR, int WR, int BN, int NS, bool AL, bool DIRECT>
// Waves per SIMD asked of the compiler: three for the D<=128 prefill kernels,
// with or without ALiBi (their 33 KiB of LDS allow three workgroups per CU; the
// staggered K/V copies would otherwise raise them to 181-193 registers and two
// waves; at 168 a few values that live across the tile loop spill, outside the
// loop, and the ALiBi one reloads two per tile); two for
// the other 4-wave D<=128 kernels and the 4-wave D256/D512 decode kernels (the
// D512 one would otherwise take 380 registers and keep one wave per SIMD where
// its 64 KiB of LDS allow two workgroups per CU).
__global__ __launch_bounds__(64 * WR) __attribute__((amdgpu_waves_per_eu(
    (WR == 4 && DP <= 128 && MR == 32) ? 3
    : ((WR == 4 && DP <= 128) || (WR == 4 && MR == 16 && NS == 1 && DP >= 256) || (WR == 1 && DP <= 128)) ? 2
    : 1, 8))) void
attn_fwd_kernel(const FwdParams p) {
    typedef Mfma<MR, E> M;
    typedef typename M::acc_t acc_t;
    constexpr int NT = 64 * WR;
    constexpr int R = MR * WR;
    constexpr int CH = DP / 8;            // 16-byte chunks per row
    constexpr int ROWB = DP * 2;          // bytes per LDS row
    constexpr int TILEB = BN * ROWB;      // bytes per K (or V) tile
    constexpr int NI = BN * CH / NT;      // 16-byte copies per thread per tensor per tile
    constexpr int NU = BN / 32;           // 32-key units per tile
    constexpr int NKS = DP / M::KSTEP;
    constexpr int NDB = DP / MR;
    constexpr int SWK = (CH < 16 ? CH : 16) - 1;
    constexpr int SWV = (CH < 16 ? CH : 16) - 1;
    constexpr int RPI = 64 / CH > 0 ? 64 / CH : 1;   // rows per 64-lane copy
    constexpr int CPD = MR / 8;           // 16-byte chunks per d-block of the PV product
    constexpr int NPAT = (NDB < (SWV + 1) / CPD) ? NDB : (SWV + 1) / CPD;  // V read XOR patterns
    // 16-byte chunk c of LDS row r sits at position c ^ swk(r) (K) or c ^ swv(r) (V).
    // Both maps are linear over the row bits, so swz(r0 + l) = swz(r0) ^ swz(l) when r0
    // is a multiple of a power of two above l.  With 32 rows per wave and >= 16 chunks
    // per row: the K rows 0..15 that one operand read touches take 16 distinct
    // positions, and rows r, r + 8 differ by 4 mod 8; the V rows 0..3 of a transposing
    // read land in distinct 64-byte quarters and distinct 32-byte eighths mod 128 bytes.
    // Either way the reads are free of bank conflicts whether the LDS serves 128 or 256
    // bytes per cycle.
    // With 16 rows per wave, one K operand read touches rows {0..3, 8..11, 16..19,
    // 24..27} (+ 4), which take 16 distinct positions; the V rows 0..3 and 8..11
    // of a transposing read take distinct 32-byte segments.  Rows of fewer than 16
    // chunks keep row & (chunks - 1) (K) and 2 row & (chunks - 1) (V).
    auto swk = [](int r) {
        if constexpr (MR == 32 && CH >= 16) return (r & 15) ^ ((r >> 1) & 4);
        else if constexpr (CH >= 16) return (r & 3) | ((r >> 1) & 12);
        else return r & SWK;
    };
    auto swv = [](int r) {
        if constexpr (MR == 32 && CH >= 16) return (0xCA60 >> (4 * (r & 3))) & 15;  // 0, 6, 10, 12
        else if constexpr (CH >= 16) return ((2 * r) & 6) | (r & 8);
        else return (2 * r) & SWV;
    };
    static_assert(BN % 32 == 0 && (BN * CH) % NT == 0 && CH <= 64 && 64 % CH == 0, "tile shape");

    __shared__ __attribute__((aligned(1024))) unsigned char smem[NS * 2 * TILEB];
    __shared__ int s_pages[kPageCap];
    // Per-lane LDS read offsets of the 32-row kernels with >= 16 chunks per row,
    // the same for every wave: the K operand base of S and the V read bases of the
    // NPAT XOR patterns of PV.  One LDS read per tile each replaces rebuilding them
    // from the lane id (about 13 and 16 VALU instructions per tile).
    constexpr bool LANE_TAB = MR == 32 && CH >= 16;
    __shared__ int s_lane_k[LANE_TAB ? 64 : 1];
    __shared__ int4 s_lane_v[LANE_TAB ? 64 : 1];
    // and each thread's per-lane offsets of its NI = 4 interior-tile K copies
    // ([0, NT)) and V copies ([NT, 2 NT)), read once per tile instead of rebuilt
    // (not with ALiBi: there the table's values spill inside the tile loop)
    constexpr bool CP_TAB = LANE_TAB && !AL;
    __shared__ int4 s_cp_off[CP_TAB ? 2 * NT : 1];
    const unsigned smem_lds = lds_u32(smem);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // Workgroups are dispatched round-robin over the 8 XCDs (each with its own
    // L2).  Work units (item, K/V head) are numbered head-fastest, in the
    // planner's order, and the XCD that receives dispatch slot j gets units in
    // runs of xcd_chunk: units that share K/V tiles (same head, neighbouring row
    // tiles of one sequence) run on the same L2.  With Hk a multiple of 8 and
    // runs of 1, every XCD serves whole K/V heads.
    const unsigned wg = blockIdx.x;
    const unsigned slot = wg >> 3, chunk = (unsigned)p.xcd_chunk;
    const unsigned unit = DIRECT ? wg : ((slot / chunk) * 8u + (wg & 7u)) * chunk + slot % chunk;
    const int hk = (int)(unit % (unsigned)p.Hk);
    const bool split = p.max_chunks > 1;
    const bool vec = p.vec != 0;
    const int D = p.D;
    const bool paged = p.bt != nullptr;
    const int P = p.page;

    // one workgroup per work item, in the planner's order (largest first);
    // workgroups past the end of the list exit.  Direct calls: the item is row
    // tile rt of sequence b, spans read here, and workgroups past the sequence's
    // row tiles exit.
    const int item_idx = (int)(unit / (unsigned)p.Hk);
    Item it;
    if constexpr (DIRECT) {
        const int b = item_idx / p.direct_tiles, rt = item_idx % p.direct_tiles;
        const SeqSpan sp = seq_span(p, b);
        if (rt >= ceil_div(sp.Lq * p.G, R)) return;
        it.b = b;
        it.rt = rt;
        it.c = 0;
        it.nc = 1;
        it.cl = INT_MAX;
        it.q0 = sp.q0;
        it.Lq = sp.Lq;
        it.k0 = sp.k0;
        it.Lk = sp.Lk;
    } else {
        if (item_idx >= *p.item_count) return;
        const int4 d = p.items[2 * item_idx];
        const int4 e = p.items[2 * item_idx + 1];
        it.b = d.x;
        it.rt = d.y;
        it.c = d.z & 0xffff;
        it.nc = d.z >> 16;
        it.cl = d.w;
        it.q0 = e.x;
        it.Lq = e.y;
        it.k0 = e.z;
        it.Lk = e.w;
    }
    const int Lq = it.Lq, Lk = it.Lk;
    const int nrows = Lq * p.G;
    const int32_t* bt_row = paged ? p.bt + (int64_t)it.b * p.bt_s0 : nullptr;
    // extra per-sequence offsets of padded (B, S, ...) k/v (zero for varlen)
    const int64_t kbx = (int64_t)it.b * p.k_bx, vbx = (int64_t)it.b * p.v_bx;

    // keys of this item: union of the tile rows' windows, cut to the chunk
    const int r_first = it.rt * R;
    const int r_last = min(nrows, r_first + R) - 1;
    const Range rf = row_range(p, r_first / p.G, Lq, Lk);
    const Range rl = row_range(p, r_last / p.G, Lq, Lk);
    int kb = rf.lo, ke = rl.hi;
    if (split) {
        kb = max(kb, it.c * it.cl);
        ke = min(ke, (it.c + 1) * it.cl);
    }

    // this lane's row
    const int rloc = lane % MR;
    const int kgrp = lane / MR;
    const int r = r_first + wave * MR + rloc;
    const bool row_ok = r < nrows;
    const int qi = row_ok ? r / p.G : 0;
    const int g = row_ok ? r % p.G : 0;
    const int h = hk * p.G + g;
    // (rows past the item keep the item's range: in-range bounds, whatever they
    // compute is never stored)
    int lo = kb, hi = ke;
    if (row_ok) {
        const Range rr = row_range(p, qi, Lq, Lk);
        lo = max(rr.lo, kb);
        hi = min(rr.hi, ke);
    }
    int w_lo = lo, w_hi = hi;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        w_lo = max(w_lo, __shfl_xor(w_lo, off, 64));
        w_hi = min(w_hi, __shfl_xor(w_hi, off, 64));
    }

    // Q^T operand: lane holds q[row][s*KSTEP + kgrp*8 .. +8) for every k-step s.
    // The softmax below needs a positive scale: a negative scale is applied as
    // an exact sign flip of q, a zero scale as q = 0 with scale 1 (uniform weights).
    float c2 = p.scale_log2;
    unsigned int qflip = 0u;
    bool qzero = false;
    if (c2 < 0.f) { qflip = 0x80008000u; c2 = -c2; }
    if (c2 == 0.f) { qzero = true; c2 = 1.f; }
    u32x4 qreg[NKS];
    {
        const uint16_t* qrow = p.q + (int64_t)(it.q0 + qi) * p.q_s0 + (int64_t)it.b * p.q_bx + (int64_t)h * p.q_s1;
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            u32x4 x = (row_ok && !qzero) ? load8(qrow, s * M::KSTEP + kgrp * 8, D, vec) : u32x4{0u, 0u, 0u, 0u};
            qreg[s] = x ^ u32x4{qflip, qflip, qflip, qflip};
        }
    }

    // ALiBi (AL: the call has slopes; a separate instantiation so the plain
    // kernel keeps its registers): this row's score for key n gets
    // al2 * |apos - n| (log2 units)
    float al2 = 0.f;
    if constexpr (AL) al2 = row_ok ? -p.alibi[(int64_t)it.b * p.alibi_sb + h] * 1.4426950408889634f : 0.f;
    const int apos = qi + Lk - Lq;

    acc_t o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < M::NACC; ++v) o[db][v] = 0.f;
    // running max (log2 domain) and sum of the rows; m_run is a reference
    // value that only moves when the tile max exceeds it by more than 8, so the
    // O rescale is rare and probabilities stay <= 2^8
    float m_run = kNegInf, l_run = 0.f;

    // copy i of this thread covers tile row (wave*NI + i)*RPI + lane/CH and
    // chunk position lane%CH (computed inside issue())
    const int nchv = (D + 7) / 8;  // chunks that hold real columns

    const int kb_al = (kb / BN) * BN;
    const int seg_keys = paged ? max(BN, ((kPageCap - 1) * P / BN) * BN) : INT_MAX;

    // Interior-tile copy bases without the per-tile part: this item's K/V head
    // (and, packed, its sequence's first key row), so a tile adds one 32 x 32-bit
    // row or page product.  Paged: the block stride in bytes.
    const unsigned char* kh = reinterpret_cast<const unsigned char*>(
        p.k + (paged ? (int64_t)hk * p.k_s2 : (int64_t)it.k0 * p.k_s0 + kbx + (int64_t)hk * p.k_s1));
    const unsigned char* vh = reinterpret_cast<const unsigned char*>(
        p.v + (paged ? (int64_t)hk * p.v_s2 : (int64_t)it.k0 * p.v_s0 + vbx + (int64_t)hk * p.v_s1));
    const uint64_t kblkb = (uint64_t)p.k_s0 * 2u, vblkb = (uint64_t)p.v_s0 * 2u;

    if constexpr (LANE_TAB) {
        static_assert(NPAT == 4, "four V read patterns in the lane table");
        if (threadIdx.x < 64) {
            const int ln = threadIdx.x;
            const int kr = kappa32(ln & 31);
            s_lane_k[ln] = kr * ROWB + (((ln >> 5) ^ swk(kr)) << 4);
            // V read base of rows r0 (and r0 + 4: same swizzle, one immediate 4 * ROWB on)
            const int g16 = ln >> 4, a16 = ln & 15;
            const int r0 = (g16 >> 1) * 8 + (a16 >> 2);
            const int c0 = (g16 & 1) * 2 + ((a16 >> 1) & 1);
            const int bx = r0 * ROWB + ((c0 ^ swv(r0)) << 4) + (a16 & 1) * 8;
            s_lane_v[ln] = int4{bx, bx ^ (CPD << 4), bx ^ ((2 * CPD) << 4), bx ^ ((3 * CPD) << 4)};
        }
        if constexpr (CP_TAB) {
            // the interior-tile copy offsets of issue() below, each copy's first row
            // included so that the four copies share one scalar base (only used when
            // its fast path is taken: row strides below 2^24, so every offset stays
            // below 2^28)
            static_assert(NI == 4, "four copies per tensor in the copy-offset table");
            constexpr int W = NI * RPI;
            const int lrow = lane / CH, lpos = lane % CH;
            const int xk = lpos ^ swk(lrow), xv = lpos ^ swv(lrow);
            const unsigned lk_off = __umul24((unsigned)lrow, (unsigned)p.k_rowb);
            const unsigned lv_off = __umul24((unsigned)lrow, (unsigned)p.v_rowb);
            int ko[NI], vo[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int r0 = wave * W + i * RPI;
                ko[i] = (int)(lk_off + (unsigned)(i * RPI) * (unsigned)p.k_rowb + ((unsigned)(xk ^ swk(r0)) << 4));
                vo[i] = (int)(lv_off + (unsigned)(i * RPI) * (unsigned)p.v_rowb + ((unsigned)(xv ^ swv(r0)) << 4));
            }
            s_cp_off[threadIdx.x] = int4{ko[0], ko[1], ko[2], ko[3]};
            s_cp_off[NT + threadIdx.x] = int4{vo[0], vo[1], vo[2], vo[3]};
        }
        __syncthreads();
    }
    int4 cp_k = {}, cp_v = {};  // this thread's copy offsets (table), loaded ahead of issue()

    // (an empty range, kb >= ke, runs no tile: its rows keep l = 0 and give 0)
    for (int seg0 = kb_al; kb < ke && seg0 < ke; seg0 = (seg_keys == INT_MAX ? ke : seg0 + seg_keys)) {
        const int seg1 = (seg_keys == INT_MAX) ? ke : min(ke, seg0 + seg_keys);
        int pg_first = 0;
        if (paged) {
            __syncthreads();  // previous segment's users of s_pages and tiles are done
            pg_first = seg0 / P;
            const int npg = (seg1 - 1) / P - pg_first + 1;
            for (int i = threadIdx.x; i < npg; i += NT)  // block ids clamped into the pool
                s_pages[i] = min(max(bt_row[pg_first + i], 0), p.num_blocks - 1);
            __syncthreads();
        }
        const int ntiles = (seg1 - seg0 + BN - 1) / BN;

        // page index and slot of the first key of the next tile whose K (index 0)
        // or V (index 1) copies are issued (paged); each tensor's tiles are issued
        // in increasing order, so both advance by BN per issued tile
        int nx_page[2] = {pg_first, pg_first}, nx_slot[2] = {0, 0};
        const int pg_last = paged ? (seg1 - 1) / P : 0;
        if (paged) nx_slot[0] = nx_slot[1] = seg0 - pg_first * P;
        // block id and slot of this wave's rows in the last K tile issued on the
        // fast path: V of the same tile, issued next, reuses them
        unsigned pg_c = 0;
        int ws_c = 0;

        // issue the copies of tile t of this segment into stage t % NS: which = 0
        // K only, 1 V only, 2 both
        auto issue = [&](int t, int which) __attribute__((always_inline)) {
            const int ts = seg0 + t * BN;
            unsigned char* kbuf = smem + (t % NS) * 2 * TILEB;
            unsigned char* vbuf = kbuf + TILEB;
            const int sx = which == 1 ? 1 : 0;
            const int t_page = nx_page[sx], t_slot = nx_slot[sx];
            if (paged) {  // P >= 32 and BN <= 64: at most two page steps
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    if (x == sx || which == 2) {
                        nx_slot[x] += BN;
                        if (nx_slot[x] >= P) { nx_slot[x] -= P; ++nx_page[x]; }
                        if (nx_slot[x] >= P) { nx_slot[x] -= P; ++nx_page[x]; }
                    }
                }
            }
            const unsigned ln = (unsigned)opaque_lane();  // unsigned: shifts, not signed division
            const int lrow = (int)(ln / CH);
            const int lpos = (int)(ln % CH);
            // Fast path for interior tiles: the W rows one wave copies lie in one page
            // (W divides 32, which divides P, and tiles start at multiples of BN), so
            // every copy address is a wave-uniform base (page, first row, head) plus a
            // per-lane offset (row within the copy, swizzled chunk).  The swizzle
            // splits as (lane part) ^ (uniform part) because each copy's first row is
            // a multiple of RPI.
            if (p.fast_copy && ts >= kb && ts + BN <= ke) {
                constexpr int W = NI * RPI;
                static_assert(32 % W == 0, "a wave's copy rows must stay inside one page");
                const int wv = __builtin_amdgcn_readfirstlane(wave);  // lets the compiler keep bases scalar
                // (block ids, slots and rows are non-negative; the fast path is only
                // taken when a row stride fits in 24 bits)
                const unsigned char *kw, *vw;
                if (paged) {
                    unsigned pg;
                    int ws;
                    if (which == 1) {
                        // V(t) alone follows K(t), which took this path too (same tile)
                        pg = pg_c;
                        ws = ws_c;
                    } else {
                        int wp = t_page;
                        ws = t_slot + wv * W;
                        if (ws >= P) { ws -= P; ++wp; }
                        if (ws >= P) { ws -= P; ++wp; }
                        pg = (unsigned)__builtin_amdgcn_readfirstlane(s_pages[wp - pg_first]);
                        pg_c = pg;
                        ws_c = ws;
                    }
                    kw = kh + pg * kblkb + (uint64_t)(unsigned)ws * (unsigned)p.k_rowb;
                    vw = vh + pg * vblkb + (uint64_t)(unsigned)ws * (unsigned)p.v_rowb;
                } else {
                    const unsigned row = (unsigned)(ts + wv * W);
                    kw = kh + (uint64_t)row * (unsigned)p.k_rowb;
                    vw = vh + (uint64_t)row * (unsigned)p.v_rowb;
                }
                const int xk = lpos ^ swk(lrow);
                const int xv = lpos ^ swv(lrow);
                // (24-bit products, full rate: lrow < 64 and row strides < 2^24 here)
                const unsigned lk_off = __umul24((unsigned)lrow, (unsigned)p.k_rowb);
                const unsigned lv_off = __umul24((unsigned)lrow, (unsigned)p.v_rowb);
                const int tk[4] = {cp_k.x, cp_k.y, cp_k.z, cp_k.w};
                const int tv[4] = {cp_v.x, cp_v.y, cp_v.z, cp_v.w};
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int r0 = wv * W + i * RPI;  // tile row of the copy's first lane row (uniform)
                    unsigned vk, vv;
                    if constexpr (CP_TAB) {
                        vk = (unsigned)tk[i];
                        vv = (unsigned)tv[i];
                    } else {
                        vk = lk_off + ((unsigned)(xk ^ swk(r0)) << 4);
                        vv = lv_off + ((unsigned)(xv ^ swv(r0)) << 4);
                    }
                    const unsigned dst = smem_lds + (unsigned)((t % NS) * 2 * TILEB + (wv * NI + i) * 1024);
                    // (table offsets hold the copy's first row; otherwise the base does)
                    const size_t krow = CP_TAB ? 0 : (size_t)(i * RPI) * p.k_rowb;
                    const size_t vrow = CP_TAB ? 0 : (size_t)(i * RPI) * p.v_rowb;
                    if (which != 1) copy16_to_lds_sv(kw + krow, vk, dst);
                    if (which != 0) copy16_to_lds_sv(vw + vrow, vv, dst + TILEB);
                }
                return;
            }
            // boundary tiles: per-lane rows clamped into [kb, ke); a tile spans at
            // most two pages
            int pg0 = 0, pg1 = 0, base0 = 0;
            if (paged) {
                pg0 = __builtin_amdgcn_readfirstlane(s_pages[t_page - pg_first]);
                pg1 = __builtin_amdgcn_readfirstlane(s_pages[min(t_page + 1, pg_last) - pg_first]);
                base0 = ts - t_slot;
            }
            if (vec) {
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int rr = (wave * NI + i) * RPI + lrow;
                    const int n = min(max(ts + rr, kb), ke - 1);
                    int64_t offk, offv;
                    if (paged) {
                        const int off = n - base0;
                        const int blk = off < P ? pg0 : pg1;
                        const int slot = off < P ? off : off - P;
                        offk = (int64_t)blk * p.k_s0 + (int64_t)slot * p.k_s1 + (int64_t)hk * p.k_s2;
                        offv = (int64_t)blk * p.v_s0 + (int64_t)slot * p.v_s1 + (int64_t)hk * p.v_s2;
                    } else {
                        offk = (int64_t)(it.k0 + n) * p.k_s0 + kbx + (int64_t)hk * p.k_s1;
                        offv = (int64_t)(it.k0 + n) * p.v_s0 + vbx + (int64_t)hk * p.v_s1;
                    }
                    int ck = lpos ^ swk(rr);
                    int cv = lpos ^ swv(rr);
                    ck = ck < nchv ? ck : 0;
                    cv = cv < nchv ? cv : 0;
                    const unsigned dst = smem_lds + (unsigned)__builtin_amdgcn_readfirstlane((t % NS) * 2 * TILEB + (wave * NI + i) * 1024);
                    if (which != 1) copy16_to_lds(p.k + offk + ck * 8, dst);
                    if (which != 0) copy16_to_lds(p.v + offv + cv * 8, dst + TILEB);
                }
            } else {
                // unaligned or odd head dim: element-wise loads, zero fill, plain LDS stores
#pragma unroll 1
                for (int i = 0; i < NI; ++i) {
                    const int rr = (wave * NI + i) * RPI + lrow;
                    const int n = ts + rr;
                    const bool ok = n >= kb && n < ke;
                    const int nc = min(max(n, kb), ke - 1);
                    const uint16_t *rowk, *rowv;
                    if (paged) {
                        const int off = nc - base0;
                        const int blk = off < P ? pg0 : pg1;
                        const int slot = off < P ? off : off - P;
                        rowk = p.k + (int64_t)blk * p.k_s0 + (int64_t)slot * p.k_s1 + (int64_t)hk * p.k_s2;
                        rowv = p.v + (int64_t)blk * p.v_s0 + (int64_t)slot * p.v_s1 + (int64_t)hk * p.v_s2;
                    } else {
                        rowk = p.k + (int64_t)(it.k0 + nc) * p.k_s0 + kbx + (int64_t)hk * p.k_s1;
                        rowv = p.v + (int64_t)(it.k0 + nc) * p.v_s0 + vbx + (int64_t)hk * p.v_s1;
                    }
                    const int ck = lpos ^ swk(rr);
                    const int cv = lpos ^ swv(rr);
                    const u32x4 zk = u32x4{0u, 0u, 0u, 0u};
                    if (which != 1) {
                        const u32x4 valk = ok ? load8(rowk, ck * 8, D, false) : zk;
                        *reinterpret_cast<u32x4*>(kbuf + rr * ROWB + lpos * 16) = valk;
                    }
                    if (which != 0) {
                        const u32x4 valv = ok ? load8(rowv, cv * 8, D, false) : zk;
                        *reinterpret_cast<u32x4*>(vbuf + rr * ROWB + lpos * 16) = valv;
                    }
                }
            }
        };

        // One stage (NS = 1), staggered: V(t) is copied while S(t) and the softmax
        // of tile t run, K(t+1) while the softmax and PV of tile t run; each
        // buffer is refilled once every wave is past its last read of it.
        // NS >= 2: whole tiles NS-1 ahead.
        if constexpr (CP_TAB) {
            cp_k = s_cp_off[threadIdx.x];
            cp_v = s_cp_off[NT + threadIdx.x];
        }
        if constexpr (NS == 1) {
            if (ntiles > 0) {
                __syncthreads();  // every wave is done with the previous segment's K tile
                issue(0, 0);
            }
        } else {
#pragma unroll
            for (int t = 0; t < NS - 1; ++t)
                if (t < ntiles) issue(t, 2);
        }

        for (int t = 0; t < ntiles; ++t) {
            int kb_lane = 0;  // this lane's K operand base (lane table), read before the waits
            if constexpr (LANE_TAB) kb_lane = s_lane_k[lane];
            if constexpr (CP_TAB) {
                cp_v = s_cp_off[NT + threadIdx.x];
                if constexpr (NS > 1) cp_k = s_cp_off[threadIdx.x];
            }
            if constexpr (NS == 1) {
                wait_vmcnt<0>();  // K(t) has landed (no other copy is in flight)
                __syncthreads();  // K(t) visible to every wave; every wave is done with V(t-1)
                issue(t, 1);
            } else {
                if (t + NS - 2 < ntiles) wait_vmcnt<(NS >= 2 ? (NS - 2) * 2 * NI : 0)>();
                else wait_vmcnt<0>();
                __syncthreads();  // tile t is in LDS for every wave; stage (t-1)%NS is free
                if (t + NS - 1 < ntiles) issue(t + NS - 1, 2);
            }

            const int n0 = seg0 + t * BN;
            const unsigned char* kbuf = smem + (t % NS) * 2 * TILEB;
            const unsigned char* vbuf = kbuf + TILEB;

            // ---- S^T = K Q^T for this wave's rows, one accumulator set per 32-key unit.
            // A lane's K operand rows: unit u adds 32 rows, which leaves the row
            // swizzle (row mod 16) unchanged, so one base address per 16-key half
            // serves every unit with a constant offset; k-step st is an XOR of the
            // chunk position.  The fragments of k-step st+1 are read before the MFMAs
            // of step st are issued, and two independent accumulator chains alternate
            // (two 32-key units or the two 16-key halves, or even and odd k-steps when
            // the tile has one 32x32 unit).
            constexpr int SPU = MR / 2;  // score values per lane per 32-key unit
            float sc[NU][SPU];
            if constexpr (MR == 32) {
                int kbase;
                if constexpr (LANE_TAB) {
                    kbase = kb_lane;
                } else {
                    const int ln = opaque_lane();
                    const int kr = kappa32(ln & 31);
                    kbase = kr * ROWB + (((ln >> 5) ^ swk(kr)) << 4);
                }
                auto kread = [&](int u, int st) {
                    return *reinterpret_cast<const u32x4*>(kbuf + (kbase ^ (st << 5)) + u * 32 * ROWB);
                };
                if constexpr (NU >= 2) {
                    acc_t sacc[NU];
                    u32x4 a[NU], nx[NU];
#pragma unroll
                    for (int u = 0; u < NU; ++u) {
                        sacc[u] = acc_t{};
                        a[u] = kread(u, 0);
                    }
#pragma unroll
                    for (int st = 0; st < NKS; ++st) {
                        if (st + 1 < NKS) {
#pragma unroll
                            for (int u = 0; u < NU; ++u) nx[u] = kread(u, st + 1);
                        }
#pragma unroll
                        for (int u = 0; u < NU; ++u) sacc[u] = M::mma(a[u], qreg[st], sacc[u]);
                        if (st + 1 < NKS) {
#pragma unroll
                            for (int u = 0; u < NU; ++u) a[u] = nx[u];
                        }
                        __builtin_amdgcn_sched_barrier(0);  // keep the step order
                    }
#pragma unroll
                    for (int u = 0; u < NU; ++u)
#pragma unroll
                        for (int v = 0; v < 16; ++v) sc[u][v] = sacc[u][v];
                } else {
                    acc_t s0 = {}, s1 = {};
                    u32x4 a0 = kread(0, 0), a1 = kread(0, 1);
#pragma unroll
                    for (int st = 0; st < NKS; st += 2) {
                        u32x4 n0, n1;
                        if (st + 2 < NKS) {
                            n0 = kread(0, st + 2);
                            n1 = kread(0, st + 3);
                        }
                        s0 = M::mma(a0, qreg[st], s0);
                        s1 = M::mma(a1, qreg[st + 1], s1);
                        if (st + 2 < NKS) {
                            a0 = n0;
                            a1 = n1;
                        }
                        __builtin_amdgcn_sched_barrier(0);  // keep the step order
                    }
#pragma unroll
                    for (int v = 0; v < 16; ++v) sc[0][v] = s0[v] + s1[v];
                }
            } else {
                // chunk st*4 + kgrp at position (st*4 + kgrp) ^ swz = base ^ (st << 6);
                // the two 16-key halves sb are the two chains
                const int ln = opaque_lane();
                const int rl = ln & 15;
                int kbase[2];
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    const int kr = (rl >> 2) * 8 + sb * 4 + (rl & 3);
                    kbase[sb] = kr * ROWB + (((ln >> 4) ^ swk(kr)) << 4);
                }
                auto kread = [&](int u, int sb, int st) {
                    return *reinterpret_cast<const u32x4*>(kbuf + (kbase[sb] ^ (st << 6)) + u * 32 * ROWB);
                };
#pragma unroll
                for (int u = 0; u < NU; ++u) {
                    acc_t sacc[2] = {acc_t{}, acc_t{}};
                    u32x4 a[2], nx[2];
#pragma unroll
                    for (int sb = 0; sb < 2; ++sb) a[sb] = kread(u, sb, 0);
#pragma unroll
                    for (int st = 0; st < NKS; ++st) {
                        if (st + 1 < NKS) {
#pragma unroll
                            for (int sb = 0; sb < 2; ++sb) nx[sb] = kread(u, sb, st + 1);
                        }
#pragma unroll
                        for (int sb = 0; sb < 2; ++sb) sacc[sb] = M::mma(a[sb], qreg[st], sacc[sb]);
                        if (st + 1 < NKS) {
#pragma unroll
                            for (int sb = 0; sb < 2; ++sb) a[sb] = nx[sb];
                        }
                        __builtin_amdgcn_sched_barrier(0);  // keep the step order
                    }
#pragma unroll
                    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                        for (int v = 0; v < 4; ++v) sc[u][sb * 4 + v] = sacc[sb][v];
                }
            }

            if constexpr (NS == 1) {
                if constexpr (CP_TAB) cp_k = s_cp_off[threadIdx.x];
                __syncthreads();  // every wave is done with K(t)
                if (t + 1 < ntiles) issue(t + 1, 0);
            }

            // ---- ALiBi (when slopes are given): scores become c2 * s + al2 * |apos - n|,
            // already scaled, so the rest of the tile uses the factor cc = 1
            float cc = c2;
            if constexpr (AL) {
#pragma unroll
                for (int u = 0; u < NU; ++u)
#pragma unroll
                    for (int e = 0; e < SPU; ++e) {
                        int key;
                        if constexpr (MR == 32) key = u * 32 + (e >> 3) * 16 + kgrp * 8 + (e & 7);
                        else key = u * 32 + kgrp * 8 + e;
                        const int dist = abs(apos - (n0 + key));
                        sc[u][e] = __builtin_fmaf(sc[u][e], c2, al2 * (float)dist);
                    }
                cc = 1.f;
            }

            // ---- mask, running max (raw scores; cc > 0 so the scaled max is cc * max)
            const bool need_mask = !(w_lo <= n0 && w_hi >= n0 + BN);
            float mx = kNegInf;
            if (need_mask) {
                // key n0 + 8 kgrp + c of score e against [lo, hi): the bounds are taken
                // relative to the lane's first key once, so each score compares its
                // compile-time c (lo and hi lie in [kb, ke], so nothing overflows)
                const int kl = n0 + kgrp * 8;
                const int dlo = lo - kl, dhi = hi - kl;
#pragma unroll
                for (int u = 0; u < NU; ++u)
#pragma unroll
                    for (int e = 0; e < SPU; ++e) {
                        int c;
                        if constexpr (MR == 32) c = u * 32 + (e >> 3) * 16 + (e & 7);
                        else c = u * 32 + e;
                        if (c < dlo || c >= dhi) sc[u][e] = kNegInf;
                    }
            }
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int e = 0; e < SPU; ++e) mx = fmaxf(mx, sc[u][e]);
            if constexpr (MR == 32) {
                mx = max_xor32(mx);
            } else {
                mx = max_xor32(max_xor16(mx));
            }
            mx *= cc;
            const bool grow = mx > m_run + 8.f;
            if (__ballot(grow)) {
                // rows that do not grow keep alpha = 1 (their m_run may still be -inf)
                const float m_new = grow ? mx : m_run;
                const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
                l_run *= alpha;
                m_run = m_new;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int v = 0; v < M::NACC; ++v) o[db][v] *= alpha;
            }
            const float nm = (m_run == kNegInf) ? 0.f : -m_run;
            float rs0 = 0.f, rs1 = 0.f;
            unsigned int pk[NU][SPU / 2];
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int e = 0; e < SPU; e += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][e], cc, nm));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][e + 1], cc, nm));
                    const unsigned int pp = E::pack2(p0, p1);
                    pk[u][e / 2] = pp;
                    // row sum of the bf16-rounded probabilities that feed the PV product
                    if ((e / 2) & 1) rs1 = E::sum2(pp, rs1);
                    else rs0 = E::sum2(pp, rs0);
                }
            float rs = rs0 + rs1;
            if constexpr (MR == 32) {
                rs = sum_xor32(rs);
            } else {
                rs = sum_xor32(sum_xor16(rs));
            }
            l_run += rs;

            int4 vx_lane = {};  // V read bases (lane table), read before the wait
            if constexpr (LANE_TAB) vx_lane = s_lane_v[lane];
            if constexpr (NS == 1) {
                // V(t) has landed: only K(t+1)'s NI copies per lane may still be in flight
                if (t + 1 < ntiles) wait_vmcnt<NI>();
                else wait_vmcnt<0>();
                __syncthreads();  // V(t) visible to every wave
            }

            // ---- O^T += V^T P^T, V^T slices by transposing LDS reads.  Per tile, the
            // lane's two read addresses (rows r0, r0 + 4) are built for the first 16
            // keys and each XOR pattern of the swizzled chunk bits; other 16-key
            // groups add whole rows (the swizzle depends on the row mod 16 only) and
            // d-blocks past the swizzled bits add a whole chunk group, both constants.
            {
                int vx[NPAT][2];
                if constexpr (LANE_TAB) {
                    const int vv[4] = {vx_lane.x, vx_lane.y, vx_lane.z, vx_lane.w};
#pragma unroll
                    for (int pat = 0; pat < NPAT; ++pat) {
                        vx[pat][0] = vv[pat];
                        vx[pat][1] = vv[pat] + 4 * ROWB;
                    }
                } else {
                    const int ln = opaque_lane();
                    const int g16 = ln >> 4, a16 = ln & 15;
                    const int r0 = (MR == 32) ? (g16 >> 1) * 8 + (a16 >> 2) : g16 * 8 + (a16 >> 2);
                    const int c0 = (MR == 32) ? (g16 & 1) * 2 + ((a16 >> 1) & 1) : (a16 >> 1) & 1;
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int rr = r0 + 4 * h2;
                        const int bx = rr * ROWB + ((c0 ^ swv(rr)) << 4) + (a16 & 1) * 8;
#pragma unroll
                        for (int pat = 0; pat < NPAT; ++pat) vx[pat][h2] = bx ^ ((pat * CPD) << 4);
                    }
                }
                if constexpr (MR == 32) {
                    // MFMA i: unit i / (2 NDB), 16-key half (i / NDB) % 2, d-block i % NDB;
                    // fragments read PF MFMAs ahead (one MFMA is shorter than an LDS read)
                    constexpr int NMF = NU * 2 * NDB, PF = 3;
                    auto vread = [&](int i) {
                        const int u = i / (2 * NDB), ts = (i / NDB) % 2, db = i % NDB;
                        const int off = (u * 32 + ts * 16) * ROWB + (db / NPAT) * (NPAT * CPD * 16);
                        const u32x2 lo2 = lds_read_tr16(vbuf + vx[db % NPAT][0] + off);
                        const u32x2 hi2 = lds_read_tr16(vbuf + vx[db % NPAT][1] + off);
                        return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
                    };
                    u32x4 a[PF];
#pragma unroll
                    for (int i = 0; i < PF - 1; ++i) a[i] = vread(i);
#pragma unroll
                    for (int i = 0; i < NMF; ++i) {
                        if (i + PF - 1 < NMF) a[(i + PF - 1) % PF] = vread(i + PF - 1);
                        const int u = i / (2 * NDB), ts = (i / NDB) % 2, db = i % NDB;
                        const u32x4 b = u32x4{pk[u][ts * 4 + 0], pk[u][ts * 4 + 1], pk[u][ts * 4 + 2],
                                              pk[u][ts * 4 + 3]};
                        o[db] = M::mma(a[i % PF], b, o[db]);
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < NU; ++u) {
                        const u32x4 b = u32x4{pk[u][0], pk[u][1], pk[u][2], pk[u][3]};
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            const int off = u * 32 * ROWB + (db / NPAT) * (NPAT * CPD * 16);
                            const u32x2 lo2 = lds_read_tr16(vbuf + vx[db % NPAT][0] + off);
                            const u32x2 hi2 = lds_read_tr16(vbuf + vx[db % NPAT][1] + off);
                            const u32x4 a = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
                            o[db] = M::mma(a, b, o[db]);
                        }
                    }
                }
            }
        }
    }

    // ---- epilogue.  The lane's row, head and column group are rebuilt from the
    // lane id: kept from the prologue, they (and 64-bit products of them) lived
    // across the tile loop and spilled.
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const float lse2 = l_run > 0.f ? m_run + __builtin_amdgcn_logf(l_run) : kNegInf;
    const int lane_e = opaque_lane();
    const int kgrp_e = lane_e / MR;
    const int r_e = r_first + wave * MR + lane_e % MR;
    const bool row_ok_e = r_e < nrows;
    const int tq = it.q0 + (row_ok_e ? r_e / p.G : 0);
    const int h_e = hk * p.G + (row_ok_e ? r_e % p.G : 0);
    if (split && it.nc > 1) {
        if (row_ok_e) {
            float* po = p.part_o + (((int64_t)it.c * p.total_q + tq) * p.H + h_e) * DP;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int v4 = 0; v4 < M::NACC; v4 += 4) {
                    int d;
                    if constexpr (MR == 32) d = db * 32 + (v4 >> 2) * 8 + kgrp_e * 4;
                    else d = db * 16 + kgrp_e * 4;
                    f32x4 val = {o[db][v4] * inv, o[db][v4 + 1] * inv, o[db][v4 + 2] * inv,
                                 o[db][v4 + 3] * inv};
                    *reinterpret_cast<f32x4*>(po + d) = val;
                }
            if (kgrp_e == 0) p.part_lse[((int64_t)it.c * p.total_q + tq) * p.H + h_e] = lse2;
        }
    } else if (row_ok_e) {
        uint16_t* orow = p.out + (int64_t)tq * p.o_s0 + (int64_t)it.b * p.o_bx + (int64_t)h_e * p.o_s1;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int v4 = 0; v4 < M::NACC; v4 += 4) {
                int d;
                if constexpr (MR == 32) d = db * 32 + (v4 >> 2) * 8 + kgrp_e * 4;
                else d = db * 16 + kgrp_e * 4;
                if (d >= D) continue;
                const float x0 = o[db][v4] * inv, x1 = o[db][v4 + 1] * inv;
                const float x2 = o[db][v4 + 2] * inv, x3 = o[db][v4 + 3] * inv;
                if (vec) {
                    *reinterpret_cast<u32x2*>(orow + d) = u32x2{E::pack2(x0, x1), E::pack2(x2, x3)};
                } else {
                    const float xs[4] = {x0, x1, x2, x3};
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (d + j < D) orow[d + j] = E::one(xs[j]);
                }
            }
        if (p.lse && kgrp_e == 0) p.lse[(int64_t)h_e * p.lse_sh + tq + (int64_t)it.b * p.lse_bx] = lse2 * 0.6931471805599453f;
    }
}

// Merge split partials: one wave per (token, head).  Lane c holds chunk c's
// weight 2^(lse_c - max); the partial rows are then accumulated four chunks at a
// time so that several loads are in flight (a chunk-by-chunk loop waits twice
// per chunk).
template <class E, int DP>
__global__ __launch_bounds__(256) void combine_kernel(const FwdParams p) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x;
    const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
    if (h >= p.H) return;
    // chunks of this token's sequence (planner), 0 if none; never more than the
    // call's bound, so no value can index past the partials.  The first 64 chunk
    // LSEs and the first group's partial rows are loaded beside the count (every
    // slot below the bound is inside the partials buffer) and what lies past the
    // count is masked after: the start is one load deep instead of three.
    constexpr int PER = DP / 64;
    constexpr int U = 4;  // chunks per group of loads
    const float* pl = p.part_lse + (int64_t)t * p.H + h;
    const int64_t cstride_l = (int64_t)p.total_q * p.H;
    const float* po = p.part_o + ((int64_t)t * p.H + h) * DP + lane;
    const int64_t cstride_o = (int64_t)p.total_q * p.H * DP;
    const float lsp = lane < p.max_chunks ? pl[lane * cstride_l] : kNegInf;
    float x0[U][PER];
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
        for (int e = 0; e < PER; ++e) x0[q][e] = po[(int64_t)min(q, p.max_chunks - 1) * cstride_o + e * 64];
    const int nc = min(p.tok_nc[t], p.max_chunks);
    if (nc <= 1) return;
    const int64_t b = p.padded ? t / p.uniform_q : 0;  // only padded calls have per-sequence offsets
    float* lse = p.lse ? p.lse + (int64_t)h * p.lse_sh + t + b * p.lse_bx : nullptr;
    const float l0 = lane < nc ? lsp : kNegInf;  // the first 64 chunks
    float M = l0;
    for (int c = lane + 64; c < nc; c += 64) M = fmaxf(M, pl[c * cstride_l]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    uint16_t* orow = p.out + (int64_t)t * p.o_s0 + b * p.o_bx + (int64_t)h * p.o_s1;
    const int D = p.D;
    if (M == kNegInf) {  // no chunk saw a key
        for (int d = lane; d < D; d += 64) orow[d] = 0;
        if (lse && lane == 0) *lse = kNegInf;
        return;
    }
    float acc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = 0.f;
    float wsum = 0.f;
    for (int c0 = 0; c0 < nc; c0 += 64) {
        const int c = c0 + lane;
        const float lc = c0 == 0 ? l0 : (c < nc ? pl[c * cstride_l] : kNegInf);
        const float wl = c < nc ? __builtin_amdgcn_exp2f(lc - M) : 0.f;  // lane c's chunk weight
        wsum += wl;
        const int n = min(64, nc - c0);
        for (int j = 0; j < n; j += U) {
            float w[U], x[U][PER];
            const bool first = c0 == 0 && j == 0;  // rows already loaded
#pragma unroll
            for (int q = 0; q < U; ++q) {
                const int jj = min(j + q, n - 1);  // a short last group repeats a chunk with weight 0
                w[q] = j + q < n ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), jj)) : 0.f;
                if (first) {
#pragma unroll
                    for (int e = 0; e < PER; ++e) x[q][e] = x0[q][e];
                } else {
#pragma unroll
                    for (int e = 0; e < PER; ++e) x[q][e] = po[(int64_t)(c0 + jj) * cstride_o + e * 64];
                }
            }
#pragma unroll
            for (int q = 0; q < U; ++q)
#pragma unroll
                for (int e = 0; e < PER; ++e) acc[e] += w[q] != 0.f ? w[q] * x[q][e] : 0.f;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off, 64);
    const float inv = 1.f / wsum;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int d = j * 64 + lane;
        if (d < D) orow[d] = E::one(acc[j] * inv);
    }
    if (lse && lane == 0) *lse = (M + __builtin_amdgcn_logf(wsum)) * 0.6931471805599453f;
}

thread_local hipError_t g_last = hipSuccess;  // per calling thread, like the error text

// With `slots` set, report how many workgroups of the kernel the launch would
// use can be resident on the whole GPU at once instead of launching it.
template <class E, int DP, int MR, int WR, int BN, int NS>
hipError_t launch_attn(const Plan& plan, const FwdParams& p, hipStream_t s, int* slots = nullptr) {
    if (slots) {
        // resident workgroups per CU, one cache per kernel (with and without ALiBi:
        // their register counts differ); the same on every CU of this target
        // (atomics: concurrent callers may fill it; they store the same value)
        static std::atomic<int> per_cu_of[2] = {{-1}, {-1}};
        std::atomic<int>& cache = per_cu_of[p.alibi ? 1 : 0];
        int per_cu = cache.load(std::memory_order_relaxed);
        if (per_cu < 0) {
            int nb = 0;
            const void* fn = p.alibi ? reinterpret_cast<const void*>(&attn_fwd_kernel<E, DP, MR, WR, BN, NS, true, false>)
                                     : reinterpret_cast<const void*>(&attn_fwd_kernel<E, DP, MR, WR, BN, NS, false, false>);
            hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, 64 * WR, 0);
            if (e != hipSuccess) return e;
            per_cu = nb;
            cache.store(nb, std::memory_order_relaxed);
        }
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        static std::atomic<int> cus_of[64] = {};  // compute units per device id
        int cus = (dev >= 0 && dev < 64) ? cus_of[dev].load(std::memory_order_relaxed) : 0;
        if (cus <= 0) {
            e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
            if (e != hipSuccess) return e;
            if (dev >= 0 && dev < 64) cus_of[dev].store(cus, std::memory_order_relaxed);
        }
        *slots = std::max(1, per_cu * cus);
        return hipSuccess;
    }
    // one workgroup per (item, K/V head) unit, padded to whole runs on all 8 XCDs;
    // direct calls: one per (sequence, row tile, K/V head)
    const int64_t units = plan.items_bound * (int64_t)p.Hk;
    const int64_t run = 8 * (int64_t)p.xcd_chunk;
    if (plan.direct) {
        const dim3 grid((unsigned)((int64_t)p.batch * plan.direct_tiles * p.Hk));
        if (p.alibi) hipLaunchKernelGGL((attn_fwd_kernel<E, DP, MR, WR, BN, NS, true, true>), grid, dim3(64 * WR), 0, s, p);
        else hipLaunchKernelGGL((attn_fwd_kernel<E, DP, MR, WR, BN, NS, false, true>), grid, dim3(64 * WR), 0, s, p);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((units + run - 1) / run * run));
    if (p.alibi) hipLaunchKernelGGL((attn_fwd_kernel<E, DP, MR, WR, BN, NS, true, false>), grid, dim3(64 * WR), 0, s, p);
    else hipLaunchKernelGGL((attn_fwd_kernel<E, DP, MR, WR, BN, NS, false, false>), grid, dim3(64 * WR), 0, s, p);
    return hipGetLastError();
}

template <class E, int DP>
hipError_t launch_combine(const FwdParams& p, hipStream_t s) {
    dim3 grid((unsigned)p.total_q, (unsigned)((p.H + 3) / 4));
    hipLaunchKernelGGL((combine_kernel<E, DP>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

template <class E, int DP>
hipError_t launch_dp(const Plan& plan, const FwdParams& p, hipStream_t s, int* slots) {
    // one LDS stage here too: it frees registers and LDS for 3 resident workgroups
    // per CU, which beat a prefetching second stage (+6-8% on long prefill)
    if (plan.kind == KIND_PREFILL) {
        if constexpr (DP <= 128) return launch_attn<E, DP, 32, 4, 64, 1>(plan, p, s, slots);
        else if constexpr (DP == 256) return launch_attn<E, DP, 32, 4, 32, 2>(plan, p, s, slots);
        else return launch_attn<E, DP, 16, 4, 32, 2>(plan, p, s, slots);
    }
    // decode: 16 rows per wave, keys split over work items, one LDS stage: HBM
    // latency is hidden by the number of resident workgroups (LDS-limited),
    // which beats deeper per-wave pipelines on this path (a second stage: paged
    // decode -9%, MQA head dim 512 -11%), except for one-wave head dim 256 (the
    // spec-decode batch: +1.5%, 2 workgroups of 64 KiB per CU)
    if (plan.wr == 1) {
        if constexpr (DP == 256) return launch_attn<E, DP, 16, 1, 32, 2>(plan, p, s, slots);
        else return launch_attn<E, DP, 16, 1, 32, 1>(plan, p, s, slots);
    }
    return launch_attn<E, DP, 16, 4, 32, 1>(plan, p, s, slots);
}

template <class E>
hipError_t launch_main(const Plan& plan, const FwdParams& p, hipStream_t s, int* slots = nullptr) {
    switch (plan.dp) {
        case 64: return launch_dp<E, 64>(plan, p, s, slots);
        case 128: return launch_dp<E, 128>(plan, p, s, slots);
        case 256: return launch_dp<E, 256>(plan, p, s, slots);
        default: return launch_dp<E, 512>(plan, p, s, slots);
    }
}

template <class E>
hipError_t launch_merge(const Plan& plan, const FwdParams& p, hipStream_t s) {
    switch (plan.dp) {
        case 64: return launch_combine<E, 64>(p, s);
        case 128: return launch_combine<E, 128>(p, s);
        case 256: return launch_combine<E, 256>(p, s);
        default: return launch_combine<E, 512>(p, s);
    }
}

}  // namespace

const char* last_hip_error() { return hipGetErrorString(g_last); }

// ---------------------------------------------------------- static scratch
//
// Scratch of the allocation-free entry (fa_varlen_fwd_static): one array per
// GPU in the library's code object, so a call that uses it allocates nothing.
// In host code the name `scratch` is a host-side stand-in, not a device
// address; the device address of each GPU's copy is looked up once, with that
// GPU current, by hipGetSymbolAddress, and only that address ever reaches a
// kernel.  Nothing in it has to start at zero: the planner writes the work
// list, its count, the offsets and the per-token chunk counts before any
// kernel reads them, and every split item writes its partials (rows without a
// visible key included) before the combine reads them.
namespace {

static __device__ __align__(256) unsigned char scratch[FA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

int static_scratch(void* stream, void** ptr, size_t* bytes) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last = e;
        return FA_ERR_HIP;
    }
    if (stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
        if (e != hipSuccess) {
            g_last = e;
            return FA_ERR_HIP;
        }
        if (sdev != dev) return FA_ERR_DEVICE;
    }
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_DEVICE;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) {
                g_last = e != hipSuccess ? e : hipErrorInvalidSymbol;
                return FA_ERR_HIP;
            }
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    *bytes = (size_t)FA_STATIC_SCRATCH_BYTES;
    return 0;
}

int launch_fwd(const Plan& plan, const FwdParams& p_in, void* stream, void* ev_start, void* ev_stop) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    FwdParams p = p_in;
    p.rows = plan.rows;
    p.items_bound = (int32_t)plan.items_bound;
    p.xcd_chunk = plan.xcd_chunk;
    p.chunk = plan.chunk;
    p.chunk_min = plan.chunk_min;
    p.chunk_align = plan.bn;
    p.chunk_adapt = plan.adapt ? 1 : 0;
    p.direct_tiles = (int32_t)plan.direct_tiles;
    hipError_t e = hipSuccess;
    if (plan.adapt) {
        int slots = 0;
        e = p.f16 ? launch_main<EF16>(plan, p, s, &slots) : launch_main<EBf16>(plan, p, s, &slots);
        p.slots = slots;
    }
    if (e == hipSuccess && !plan.direct) {
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, p);
        e = hipGetLastError();
    }
    if (e == hipSuccess && ev_start) e = hipEventRecord(static_cast<hipEvent_t>(ev_start), s);
    if (e == hipSuccess) e = p.f16 ? launch_main<EF16>(plan, p, s) : launch_main<EBf16>(plan, p, s);
    if (e == hipSuccess && ev_stop) e = hipEventRecord(static_cast<hipEvent_t>(ev_stop), s);
    if (e == hipSuccess && plan.max_chunks > 1)
        e = p.f16 ? launch_merge<EF16>(plan, p, s) : launch_merge<EBf16>(plan, p, s);
    g_last = e;
    return e == hipSuccess ? 0 : FA_ERR_HIP;
}

}  // namespace fa
