// Internal interface between the host front end (fa_api.cpp) and the kernels
// (fa_fwd.hip).  Not installed; the public ABI is include/fa_varlen.h.
#pragma once

#include <hip/hip_runtime.h>  // int4 and the runtime types; host-only users build it with -D__HIP_PLATFORM_AMD__
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Everything a kernel launch needs.  Strides are in elements.
struct FwdParams {
    const uint16_t* q;      // bf16 or fp16 bits
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* out;
    float* lse;             // [H][total_q] natural log, or nullptr
    const int32_t* cu_q;
    const int32_t* cu_k;
    const int32_t* bt;      // block table, nullptr = non-paged
    float* part_o;          // split partials [chunk][total_q][H][DP] (fp32, normalized)
    float* part_lse;        // [chunk][total_q][H] log2-domain
    int64_t q_s0, q_s1;     // token, head
    int64_t k_s0, k_s1, k_s2;  // paged: block, slot, head; non-paged: token, head, -
    int64_t v_s0, v_s1, v_s2;
    int64_t o_s0, o_s1;
    int64_t bt_s0;
    int32_t batch, H, Hk, G, D, page;
    int32_t total_q;
    int32_t max_lk;         // paged: block_table width * page; non-paged: total_k
    int32_t num_blocks;     // paged pool size (block ids are clamped into it)
    int32_t window_left, window_right;
    int32_t chunk;          // keys per split (split only if max_chunks > 1); the planner may shrink it
    int32_t chunk_min;      // smallest chunk the workspace allows (decode: chunk / 2)
    int32_t chunk_align;    // chunk sizes are multiples of this (the key tile)
    int32_t chunk_adapt;    // 1 = the planner picks the chunk from the sequence lengths
    int32_t slots;          // workgroups of the main kernel resident at once (whole GPU)
    int32_t max_chunks;
    int32_t rows;           // rows per work item (MFMA rows per wave * waves)
    int32_t items_bound;    // upper bound of the number of work items per K/V head
    int32_t xcd_chunk;      // work units per run on one XCD (grid remap)
    int4* items;            // work list: per item {b, rt, c | nc<<16, 0}, {q0, Lq, k0, Lk}
    int32_t* item_count;    // number of work items (per K/V head)
    int32_t* seq_off;       // [batch+1] item offsets when they do not fit in LDS
    int32_t* tok_nc;        // [total_q] chunks of each token's sequence (split only)
    // Direct calls (a few sequences, no key split) run no planner: workgroup
    // (b * direct_tiles + rt) * Hk + hk takes row tile rt of sequence b from the
    // offsets itself, and exits when the sequence has fewer row tiles.
    int32_t direct_tiles;   // row tiles of the longest possible sequence
    int32_t f16;            // element type of q/k/v/out: 0 = bf16, 1 = fp16
    const float* alibi;     // ALiBi slopes or nullptr: slope of (sequence b, head h) at alibi[b * alibi_sb + h]
    int64_t alibi_sb;
    int32_t vec;            // 1 = 16-byte vector loads are legal for q/k/v/out
    int32_t fast_copy;      // 1 = interior K/V tiles may use uniform-base + lane-offset copies
    int32_t k_rowb, v_rowb; // bytes between consecutive key rows (paged: slot stride; packed: token stride)
    float scale_log2;       // softmax_scale * log2(e)
    // Padded (B, S, H, D) calls: every sequence has uniform_q queries and
    // uniform_k keys (the offsets are b * uniform_*; no cu_seqlens arrays), and
    // row t of sequence b sits at t * s0 + b * *_bx, the extra per-sequence
    // offset of a batch stride that is not S * s0.  Varlen calls: all zero.
    int32_t padded, uniform_q, uniform_k;
    int64_t q_bx, k_bx, v_bx, o_bx;
    // lse element of (token t of sequence b, head h): h * lse_sh + t + b * lse_bx
    // (varlen: lse_sh = total_q, lse_bx = 0; padded (B, H, Sq): Sq and (H - 1) * Sq)
    int64_t lse_sh, lse_bx;
};

enum Kind { KIND_PREFILL = 0, KIND_DECODE = 1 };

struct Plan {
    int kind;       // Kind
    int dp;         // padded head dim: 64/128/256/512
    int mr;         // MFMA rows per wave (16 or 32)
    int wr;         // waves per workgroup (each owns mr rows)
    int bn;         // keys per LDS tile
    int rows;       // rows per workgroup = mr * wr
    int chunk;      // keys per split (base size)
    int chunk_min;  // smallest chunk the planner may pick (workspace is sized for it)
    bool adapt;     // planner picks the chunk
    int max_chunks; // upper bound of splits per sequence
    int64_t items_bound;  // upper bound of work items per K/V head
    int xcd_chunk;        // work units per run on one XCD
    bool direct;          // no planner: the grid covers (sequence, row tile, K/V head) directly
    int64_t direct_tiles; // row tiles per sequence in that grid (the longest possible sequence's)
    size_t off_items, off_count, off_seq, off_tok;  // workspace layout (bytes)
    size_t ws_bytes;
};

// Largest batch that runs without the planner (when no key split is needed).
constexpr int kDirectMaxBatch = 16;

// Shapes the planner needs (host values only).
struct Shapes {
    int64_t total_q, H, Hk, D;
    int64_t max_lk;     // upper bound of any sequence's key count
    int64_t batch;
    bool paged;
};

// Paged K/V append: new token rows scattered into pool blocks.  Strides in elements.
struct AppendParams {
    const uint16_t* k_new;   // [total_new][Hk][D] bf16 bits (strided tokens/heads)
    const uint16_t* v_new;
    uint16_t* k_cache;       // [num_blocks][page][Hk][D]
    uint16_t* v_cache;
    const int32_t* cu_new;   // [batch+1]
    const int32_t* cu_k;     // [batch+1] key counts after the append
    const int32_t* bt;       // [batch][bt_width]
    int64_t kn_s0, kn_s1, vn_s0, vn_s1;
    int64_t kc_s0, kc_s1, kc_s2, vc_s0, vc_s1, vc_s2;
    int64_t bt_s0;
    int32_t batch, Hk, D, page, bt_width, num_blocks;
    int32_t vec;             // 1: a unit is 8 elements (16 bytes); 0: one element
    int32_t upr;             // units per head row: D/8 or D
    uint32_t units;          // total_new * Hk * upr (< 2^31)
};

int make_plan(const Shapes& s, Plan* plan);   // 0 or an fa_status code

// Device scratch of the allocation-free entry: FA_STATIC_SCRATCH_BYTES per GPU,
// a __device__ array of the library's code object.  Writes the calling
// thread's current device's copy of it to *ptr (its size to *bytes); the
// stream, when given, must belong to that device.  0, FA_ERR_DEVICE or
// FA_ERR_HIP.
int static_scratch(void* stream, void** ptr, size_t* bytes);
// 0 or FA_ERR_HIP.  ev_start/ev_stop (hipEvent_t or null) bracket the main kernel.
int launch_fwd(const Plan& plan, const FwdParams& p, void* stream, void* ev_start, void* ev_stop);
const char* last_hip_error();
// 0 or FA_ERR_HIP.  ev_start/ev_stop (hipEvent_t or null) bracket the append kernel.
int launch_kv_append(const AppendParams& p, void* stream, void* ev_start, void* ev_stop);
const char* last_append_error();

}  // namespace fa
