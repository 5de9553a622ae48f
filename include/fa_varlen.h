/*
 * fa_varlen.h -- C ABI of the MI355X (gfx950) varlen flash-attention forward.
 *
 * The forward pass of softmax attention over sequences packed back to back
 * ("varlen"), with grouped-query heads, a softmax scale, a left/right key
 * window around the bottom-right aligned diagonal, and an optional paged K/V
 * cache read through a per-sequence block table; the same forward over padded
 * (batch, seqlen, heads, head_dim) tensors; and the append that writes new
 * tokens' K/V into a paged cache.
 *
 * The operation and its argument contract are those of candle's
 * FlashAttentionVarLen forward (huggingface/candle, candle-flash-attn), as the
 * error-explainer pages for it describe:
 *   - page "flash-attn-varlen expects input tensors of rank 3", sections
 *     What it means and Source: q is rank 3 (total_q, num_heads, head_dim);
 *     without a block table k and v are rank 3 too;
 *   - page "flash-attn-varlen paged expects k/v tensors of rank 4", sections
 *     What it means and Source: with a block table, k and v are rank-4 pools
 *     (num_blocks, page_block_size, num_heads_k, head_dim); the last dim of
 *     q, k and v must be contiguous;
 *   - page "paged flash-attn requires page_block_size", section Source: v must
 *     have k's shape, k's head size must be q's, a page size must be given;
 *   - page "page_block_size ... does not match k shape", section What it
 *     means: the page size argument must equal k's dim 1;
 *   - page "paged flash-attn requires page_block_size to be a multiple of 32",
 *     section Source: the page size must be a multiple of 32, the head size at
 *     most 512, and without paging k/v must be (total_k, num_heads_k, head_dim).
 * The checks run in that order and the error texts are kept identical to the
 * quoted ones, because callers match on them.
 *
 * Ownership: the caller owns every buffer (inputs, out, softmax_lse,
 * workspace) and the stream.  The library allocates and frees nothing, keeps
 * no state between calls other than the thread-local error text (and the
 * fixed scratch array of fa_varlen_fwd_static, part of its code object), and
 * never synchronizes the device: fa_varlen_fwd only enqueues kernels on `stream`.
 * A call can therefore be captured into a HIP graph (no memset or copy nodes
 * either); the kernels read the offsets and the block table when they run, so
 * a replay with new contents in the same buffers computes the new lengths, as
 * long as the tensor shapes are those of the captured call: the host sizes
 * the grids from batch, total_q and the longest possible key range (k's rows,
 * or the block-table width times the page size).  FA_VALIDATE=1 (below)
 * synchronizes, so it cannot be captured.
 *
 * Errors: every function returns FA_OK (0) or one of the FA_ERR_* codes; the
 * text of the last error on the calling thread is returned by fa_last_error().
 * On an error nothing is launched and no output is touched.  The contents of
 * the offset arrays and the block table are not checked by default: the
 * kernels clamp them into the tensors they were given, so a bad table gives
 * wrong values but no access outside the buffers.  With FA_VALIDATE=1 in the
 * environment, fa_varlen_fwd (and fa_varlen_fwd_static) and fa_kv_append first
 * copy those arrays to the host on `stream`, wait for the copy (the only
 * synchronizing path of the library, meant for debugging) and return
 * FA_ERR_ARGUMENT, launching nothing, for offsets that decrease or leave
 * [0, rows], a sequence with more keys than its block-table row holds, or a
 * block id outside the pool among the pages its keys (appended rows) use.
 * Faults inside the kernels surface at the caller's next synchronization, as
 * with any asynchronous device work.
 */
#ifndef FA_VARLEN_H
#define FA_VARLEN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types: q/k/v/out (and the append's rows and pools) are all bf16 or
 * all IEEE binary16 (fp16) -- the candle wrapper is generic over the element
 * type (page "flash-attn-varlen paged expects k/v tensors of rank 4", Source);
 * block tables are int32 */
enum fa_dtype { FA_DTYPE_BF16 = 1, FA_DTYPE_I32 = 2, FA_DTYPE_F16 = 3, FA_DTYPE_F32 = 4 };

/* status codes */
enum fa_status {
    FA_OK = 0,
    FA_ERR_RANK = 1,         /* q/k/v/out/block_table rank */
    FA_ERR_CONTIGUOUS = 2,   /* last dim not contiguous */
    FA_ERR_SHAPE = 3,        /* shapes disagree */
    FA_ERR_PAGE_SIZE = 4,    /* page_block_size missing, mismatched or not a multiple of 32 */
    FA_ERR_HEAD_DIM = 5,     /* head_dim > 512 or < 1 */
    FA_ERR_DTYPE = 6,        /* tensors not all bf16 or all fp16 / block_table not int32 */
    FA_ERR_ARGUMENT = 7,     /* null pointer, negative batch, heads not divisible, size limits */
    FA_ERR_WORKSPACE = 8,    /* workspace missing or smaller than fa_varlen_workspace_bytes() */
    FA_ERR_DEVICE = 9,       /* a pointer is not device memory */
    FA_ERR_HIP = 10          /* the HIP runtime refused a launch */
};

/*
 * A strided view.  `data` is the address of element (0, ..., 0) with any view
 * offset already applied (candle's start_offset); strides are in elements.
 * Only shape[0..rank) and stride[0..rank) are read.
 */
typedef struct fa_tensor {
    void*   data;
    int32_t dtype;     /* enum fa_dtype */
    int32_t rank;      /* 0..4 */
    int64_t shape[4];
    int64_t stride[4];
} fa_tensor;

/*
 * fa_varlen_check -- the shape/stride/dtype contract alone.  Pure host code:
 * no pointer is dereferenced and no HIP call is made, so it runs without a GPU.
 *
 *   q            (total_q, num_heads, head_dim) bf16 or fp16, last dim contiguous
 *   k, v         paged: (num_blocks, page_block_size, num_heads_k, head_dim)
 *                non-paged: (total_k, num_heads_k, head_dim); same dtype as q, last dim contiguous
 *   out          same shape and dtype as q, last dim contiguous (may be NULL here)
 *   batch        number of sequences (>= 0)
 *   block_table  NULL = non-paged; else int32 (batch, max_blocks_per_seq), last dim contiguous
 *   page_block_size  0 = not given; must equal k.shape[1] and be a multiple of 32 when paged;
 *                ignored without a block table
 *   alibi_slopes NULL, or fp32 (num_heads) or (batch, num_heads), last dim contiguous
 *                (the shape the pages' "shape mismatch alibi_slopes {:?}, expected {:?}"
 *                error guards: page "page_block_size ... does not match k shape",
 *                Related errors)
 * Returns FA_OK or the first failing check's code (text in fa_last_error()).
 */
int fa_varlen_check(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                    const fa_tensor* out, int32_t batch, const fa_tensor* block_table,
                    int32_t page_block_size, const fa_tensor* alibi_slopes);

/*
 * fa_varlen_workspace_bytes -- device scratch that fa_varlen_fwd needs for the
 * same arguments (split-KV partial outputs).  Runs fa_varlen_check first.
 * Depends on shapes only (never on sequence lengths, which live on the device).
 * Writes 0 when the call needs no workspace.
 */
int fa_varlen_workspace_bytes(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                              int32_t batch, const fa_tensor* block_table,
                              int32_t page_block_size, size_t* bytes);

/*
 * fa_varlen_fwd -- enqueue the forward pass on `stream` (a hipStream_t; NULL =
 * the null stream).
 *
 *   cu_seqlens_q, cu_seqlens_k  device int32 arrays of batch+1 cumulative lengths,
 *       starting at 0.  Sequence b owns query rows [cu_q[b], cu_q[b+1]) of q/out
 *       and Lk_b = cu_k[b+1] - cu_k[b] keys: non-paged, rows [cu_k[b], cu_k[b+1])
 *       of k/v; paged, logical key j lives in pool block block_table[b][j / P],
 *       slot j % P (P = page_block_size).  Rows of out past cu_q[batch] are not
 *       written.  Contents are the caller's promise (monotone offsets, block ids
 *       inside the pool, Lk_b <= max_blocks_per_seq * P), checked only with
 *       FA_VALIDATE=1 (above).
 *   softmax_scale  multiplies q.k before the softmax.
 *   window_left, window_right  query row i of a sequence sits at key position
 *       a = i + Lk - Lq; key j is visible iff j >= a - window_left (when
 *       window_left >= 0) and j <= a + window_right (when window_right >= 0).
 *       Negative = unbounded; causal is (-1, 0).  Any int32 value is legal: a
 *       window at least as long as every distance (INT32_MAX, say) sees every
 *       key on its side, as a negative one does.  Query head h reads key/value
 *       head h / (num_heads / num_heads_k).  A row that sees no key gets out = 0.
 *   alibi_slopes  NULL, or device fp32 slopes as for fa_varlen_check: the scaled
 *       score of key j for query row i of head h gets -slope * |a - j| added
 *       (slope = alibi[h], or alibi[b][h] for per-sequence slopes).
 *   softmax_lse  NULL, or device fp32 [num_heads][total_q]: natural-log
 *       sum of exp of the scaled scores per row (-inf for a row that sees no key).
 *   workspace, workspace_bytes  device scratch of at least
 *       fa_varlen_workspace_bytes(); may be NULL when that is 0.
 * The call is asynchronous; out must not alias q, k or v.
 */
int fa_varlen_fwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                  const fa_tensor* out, const int32_t* cu_seqlens_q,
                  const int32_t* cu_seqlens_k, int32_t batch, const fa_tensor* block_table,
                  int32_t page_block_size, float softmax_scale, int32_t window_left,
                  int32_t window_right, const fa_tensor* alibi_slopes, float* softmax_lse,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_varlen_fwd_static -- fa_varlen_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, results, checks and errors as
 * fa_varlen_fwd, without the workspace: the scratch comes from a fixed
 * FA_STATIC_SCRATCH_BYTES array that the library's code object holds on each
 * GPU it runs on (from the first load of the library until the process ends).
 * The call allocates and frees nothing.
 *
 *   Limit: a call whose fa_varlen_workspace_bytes() exceeds
 *       FA_STATIC_SCRATCH_BYTES is rejected with FA_ERR_WORKSPACE (nothing is
 *       launched); use fa_varlen_fwd with a workspace for it.
 *   stream: must belong to the calling thread's current device (else
 *       FA_ERR_DEVICE), whose copy of the scratch is used.
 *   Sharing: every call on one GPU uses that GPU's one scratch, which keeps the
 *       last call's contents (no call relies on them: all of it is written
 *       before it is read).  Calls whose kernels can overlap on one GPU (other
 *       streams, other threads) race on it; serialize them, for instance on one
 *       stream.
 */
#define FA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

int fa_varlen_fwd_static(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                         const fa_tensor* out, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_k, int32_t batch, const fa_tensor* block_table,
                         int32_t page_block_size, float softmax_scale, int32_t window_left,
                         int32_t window_right, const fa_tensor* alibi_slopes, float* softmax_lse,
                         void* stream);

/*
 * Padded (non-varlen) entry: the same forward over batch-major tensors in which
 * every sequence has the same length, the layout the pages send callers to
 * when they hold (B, S, H, D) tensors instead of packed ones (page
 * "flash-attn-varlen expects input tensors of rank 3", Solutions and When it
 * happens: padded batch attention goes to the non-varlen FlashAttention).  It
 * computes exactly what fa_varlen_fwd computes with cu_seqlens_q = b * Sq and
 * cu_seqlens_k = b * Sk (no cu arrays are needed).
 *
 *   q, out   (B, Sq, H, D) bf16 or fp16 (one dtype for q, k, v and out), last
 *            dim contiguous, any other strides (for instance a (B, H, S, D)
 *            tensor viewed as (B, S, H, D)).
 *   k, v     (B, Sk, Hk, D), last dim contiguous, same shape; H % Hk == 0;
 *            1 <= D <= 512; B*Sq*H and B*Sk below 2^31.
 *   softmax_scale, window_left, window_right, alibi_slopes  as for
 *            fa_varlen_fwd (query row i sits at key position i + Sk - Sq; per-
 *            sequence slopes are (B, H)).
 *   softmax_lse  NULL or device fp32 (B, H, Sq), natural log.
 *   workspace    at least fa_padded_workspace_bytes() bytes (may be NULL if 0).
 * Errors, ownership and asynchrony as for fa_varlen_fwd; fa_padded_check runs
 * the contract alone without a GPU.
 */
int fa_padded_check(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* out,
                    const fa_tensor* alibi_slopes);

int fa_padded_workspace_bytes(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, size_t* bytes);

int fa_padded_fwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* out,
                  float softmax_scale, int32_t window_left, int32_t window_right,
                  const fa_tensor* alibi_slopes, float* softmax_lse, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * fa_kv_append_check -- the contract of fa_kv_append alone (host code, no GPU
 * needed, no pointer dereferenced).  Returns FA_OK or the first failing check.
 */
int fa_kv_append_check(const fa_tensor* k_new, const fa_tensor* v_new, int32_t batch,
                       const fa_tensor* block_table, const fa_tensor* k_cache,
                       const fa_tensor* v_cache, int32_t page_block_size);

/*
 * fa_kv_append -- enqueue on `stream` the write that fills a paged K/V cache
 * before a paged fa_varlen_fwd reads it: each new token's K and V rows are
 * scattered into the pool block and slot that its sequence's block table names.
 * Addressing is the paged read's (pages "flash-attn-varlen paged expects k/v
 * tensors of rank 4" and "page_block_size ... does not match k shape", What it
 * means: logical key n of sequence b is block block_table[b][n / P], slot n % P).
 *
 *   k_new, v_new   (total_new, num_heads_k, head_dim) bf16 or fp16, last dim contiguous,
 *                  same shape; read only.
 *   cu_seqlens_new device int32 [batch+1], cumulative new-token counts from 0:
 *                  sequence b owns rows [cu_new[b], cu_new[b+1]) of k_new/v_new.
 *   cu_seqlens_k   device int32 [batch+1], cumulative key counts AFTER the append
 *                  (the array the following fa_varlen_fwd takes).  The new tokens
 *                  are each sequence's last keys: new token j of sequence b goes to
 *                  logical position Lk_b - Lnew_b + j.
 *   block_table    int32 (batch, max_blocks), last dim contiguous.
 *   k_cache, v_cache  (num_blocks, page_block_size, num_heads_k, head_dim), dtype of k_new,
 *                  last dim contiguous, same shape; written in place.
 *   page_block_size  must equal k_cache.shape[1] and be a multiple of 32; the
 *                  head size is at most 512 (the paged forward's rules and texts).
 * Every other element of the pools is left untouched.  A token whose position
 * falls outside [0, max_blocks * P), whose block id falls outside the pool, or
 * that lies in no sequence's range, is skipped (nothing is written for it).
 * Overlapping targets (two tokens mapped to one slot) leave either one's row.
 * Ownership and errors as for fa_varlen_fwd; the call is asynchronous and
 * allocates nothing.  total_new * num_heads_k * head_dim must be below 2^31.
 */
int fa_kv_append(const fa_tensor* k_new, const fa_tensor* v_new, const int32_t* cu_seqlens_new,
                 const int32_t* cu_seqlens_k, int32_t batch, const fa_tensor* block_table,
                 const fa_tensor* k_cache, const fa_tensor* v_cache, int32_t page_block_size,
                 void* stream);

/*
 * fa_varlen_set_kernel_events -- measurement hook for benchmarks.  With both
 * arguments non-NULL (hipEvent_t handles created by the caller), every later
 * fa_varlen_fwd / fa_padded_fwd (fa_kv_append) on this thread records
 * `start_event` immediately before and `stop_event` immediately after its main
 * attention kernel (its append kernel), on the call's stream, so the caller can read
 * that kernel's duration with hipEventElapsedTime.  NULL, NULL turns it off.  The events stay owned by the
 * caller.  Always returns FA_OK.
 */
int fa_varlen_set_kernel_events(void* start_event, void* stop_event);

/* Text of the last non-zero status returned on this thread ("" if none). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_VARLEN_H */
