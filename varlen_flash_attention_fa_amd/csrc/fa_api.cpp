// Host front end of the C ABI: argument contract, planning, device checks.
//
// The contract checks follow candle's FlashAttentionVarLen forward as the
// error-explainer pages quote it (pages "flash-attn-varlen expects input
// tensors of rank 3" and "flash-attn-varlen paged expects k/v tensors of rank
// 4", section Source: ranks then last-dim contiguity; pages "paged flash-attn
// requires page_block_size" and "... to be a multiple of 32", section Source:
// the paged shape chain and the non-paged k/v shape check).  The order of the
// checks and the message texts are kept identical because callers match on
// them.  Checks the pages do not show (dtypes, out, block table shape, head
// divisibility, workspace) come after and carry their own texts.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/fa_varlen.h"
#include "fa_internal.h"

namespace {

bool is_elem16(int32_t dt) { return dt == FA_DTYPE_BF16 || dt == FA_DTYPE_F16; }

thread_local std::string g_err;
thread_local void* g_ev_start = nullptr;
thread_local void* g_ev_stop = nullptr;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

// Rust-style debug list: [a, b, c]
std::string dims(const fa_tensor* t, bool strides) {
    std::string s = "[";
    for (int i = 0; i < t->rank && i < 4; ++i) {
        if (i) s += ", ";
        s += std::to_string(strides ? t->stride[i] : t->shape[i]);
    }
    return s + "]";
}

bool same_dims(const fa_tensor* a, const fa_tensor* b) {
    if (a->rank != b->rank) return false;
    for (int i = 0; i < a->rank; ++i)
        if (a->shape[i] != b->shape[i]) return false;
    return true;
}

// ALiBi slopes: fp32, (num_heads) or (batch, num_heads), last dim contiguous.  The
// shape text is the one the pages list among the related errors (page
// "page_block_size ... does not match k shape", Related errors).
int alibi_check(const fa_tensor* al, int64_t batch, int64_t num_heads) {
    if (!al) return FA_OK;
    if (al->rank < 0 || al->rank > 4) return fail(FA_ERR_RANK, "tensor rank must be in 0..4 (got %d)", (int)al->rank);
    if (al->dtype != FA_DTYPE_F32)
        return fail(FA_ERR_DTYPE, "alibi_slopes must be f32 (dtype code %d)", (int)al->dtype);
    const bool ok1 = al->rank == 1 && al->shape[0] == num_heads;
    const bool ok2 = al->rank == 2 && al->shape[0] == batch && al->shape[1] == num_heads;
    if (!ok1 && !ok2) {
        const std::string exp = al->rank == 2 ? "[" + std::to_string(batch) + ", " + std::to_string(num_heads) + "]"
                                              : "[" + std::to_string(num_heads) + "]";
        return fail(FA_ERR_SHAPE, "shape mismatch alibi_slopes %s, expected %s", dims(al, false).c_str(), exp.c_str());
    }
    if (al->stride[al->rank - 1] != 1 && al->shape[al->rank - 1] > 1)
        return fail(FA_ERR_CONTIGUOUS, "alibi_slopes last dimension must be contiguous");
    if (al->rank == 2 && al->stride[0] < 0) return fail(FA_ERR_SHAPE, "negative alibi_slopes stride");
    return FA_OK;
}

int check_impl(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* out,
               int32_t batch, const fa_tensor* bt, int32_t page_block_size, const fa_tensor* alibi) {
    if (!q || !k || !v) return fail(FA_ERR_ARGUMENT, "q, k and v descriptors must not be NULL");

    // the rank checks come first and index nothing; every later check reads
    // shape/stride entries below the rank they establish (3, or 4 for paged k/v)
    const bool paged = bt != nullptr;
    const int q_rank = q->rank, k_rank = k->rank, v_rank = v->rank;
    if (q_rank != 3 || (!paged && k_rank != 3) || (!paged && v_rank != 3))
        return fail(FA_ERR_RANK, "flash-attn-varlen expects input tensors of rank 3 (q: %d, k: %d, v: %d",
                    q_rank, k_rank, v_rank);
    if (paged && (k_rank != 4 || v_rank != 4))
        return fail(FA_ERR_RANK, "flash-attn-varlen paged expects k/v tensors of rank 4 (k: %d, v: %d)",
                    k_rank, v_rank);
    if (q->stride[q_rank - 1] != 1)
        return fail(FA_ERR_CONTIGUOUS, "the last dim of q must be contiguous %s", dims(q, true).c_str());
    if (k->stride[k_rank - 1] != 1)
        return fail(FA_ERR_CONTIGUOUS, "the last dim of k must be contiguous %s", dims(k, true).c_str());
    if (v->stride[v_rank - 1] != 1)
        return fail(FA_ERR_CONTIGUOUS, "the last dim of v must be contiguous %s", dims(v, true).c_str());

    const int64_t total_q = q->shape[0], num_heads = q->shape[1], head_size = q->shape[2];
    int64_t num_heads_k;
    if (paged) {
        const int64_t page = k->shape[1];
        num_heads_k = k->shape[2];
        if (!same_dims(k, v))
            return fail(FA_ERR_SHAPE, "shape mismatch k %s and v %s", dims(k, false).c_str(),
                        dims(v, false).c_str());
        if (k->shape[3] != head_size)
            return fail(FA_ERR_SHAPE, "shape mismatch q %s and k %s", dims(q, false).c_str(),
                        dims(k, false).c_str());
        if (page_block_size <= 0) return fail(FA_ERR_PAGE_SIZE, "paged flash-attn requires page_block_size");
        if ((int64_t)page_block_size != page)
            return fail(FA_ERR_PAGE_SIZE, "page_block_size %d does not match k shape %s",
                        (int)page_block_size, dims(k, false).c_str());
        if (page % 32 != 0)
            return fail(FA_ERR_PAGE_SIZE,
                        "paged flash-attn requires page_block_size to be a multiple of 32 (got %lld)",
                        (long long)page);
        if (head_size > 512)
            return fail(FA_ERR_HEAD_DIM, "paged flash-attn supports head sizes up to 512 (got %lld)",
                        (long long)head_size);
    } else {
        num_heads_k = k->shape[1];
        const int64_t total_k = k->shape[0];
        if (!(k->shape[0] == total_k && k->shape[1] == num_heads_k && k->shape[2] == head_size))
            return fail(FA_ERR_SHAPE, "shape mismatch q %s and k %s", dims(q, false).c_str(),
                        dims(k, false).c_str());
        if (!(v->shape[0] == total_k && v->shape[1] == num_heads_k && v->shape[2] == head_size))
            return fail(FA_ERR_SHAPE, "shape mismatch q %s and v %s", dims(q, false).c_str(),
                        dims(v, false).c_str());
    }

    // ---- checks beyond the quoted ones
    if (!is_elem16(q->dtype) || k->dtype != q->dtype || v->dtype != q->dtype)
        return fail(FA_ERR_DTYPE, "flash-attn-varlen takes bf16 or f16 q/k/v of one dtype (dtype codes q: %d, k: %d, v: %d)",
                    (int)q->dtype, (int)k->dtype, (int)v->dtype);
    if (head_size < 1 || head_size > 512)
        return fail(FA_ERR_HEAD_DIM, "flash-attn-varlen supports head sizes 1..512 (got %lld)",
                    (long long)head_size);
    if (num_heads < 1 || num_heads_k < 1 || num_heads % num_heads_k != 0)
        return fail(FA_ERR_ARGUMENT,
                    "number of heads in q (%lld) must be a positive multiple of the number of heads in k/v (%lld)",
                    (long long)num_heads, (long long)num_heads_k);
    if (batch < 0) return fail(FA_ERR_ARGUMENT, "batch must be >= 0 (got %d)", (int)batch);
    if (total_q < 0 || total_q * num_heads >= INT32_MAX)
        return fail(FA_ERR_ARGUMENT, "total_q * num_heads must be below 2^31 (got %lld * %lld)",
                    (long long)total_q, (long long)num_heads);
    for (const fa_tensor* t : {q, k, v})
        for (int i = 0; i < t->rank; ++i)
            if (t->shape[i] < 0 || t->stride[i] < 0)
                return fail(FA_ERR_SHAPE, "negative shape or stride %s / %s", dims(t, false).c_str(),
                            dims(t, true).c_str());
    if (out) {
        if (out->dtype != q->dtype)
            return fail(FA_ERR_DTYPE, "out must have the dtype of q (dtype codes %d and %d)", (int)out->dtype,
                        (int)q->dtype);
        if (!same_dims(out, q))
            return fail(FA_ERR_SHAPE, "out must have the shape of q %s (got %s)", dims(q, false).c_str(),
                        dims(out, false).c_str());
        if (out->stride[2] != 1)
            return fail(FA_ERR_CONTIGUOUS, "the last dim of out must be contiguous %s",
                        dims(out, true).c_str());
    }
    if (paged) {
        if (bt->dtype != FA_DTYPE_I32)
            return fail(FA_ERR_DTYPE, "block_table must be int32 (dtype code %d)", (int)bt->dtype);
        if (bt->rank != 2 || bt->shape[0] != batch || bt->shape[1] < 0)
            return fail(FA_ERR_SHAPE, "block_table must have shape (batch=%d, max_blocks) (got %s)",
                        (int)batch, dims(bt, false).c_str());
        if (bt->stride[1] != 1 && bt->shape[1] > 1)
            return fail(FA_ERR_CONTIGUOUS, "block_table last dimension must be contiguous");
        if (bt->shape[1] * (int64_t)page_block_size >= INT32_MAX)
            return fail(FA_ERR_ARGUMENT, "max_blocks * page_block_size must be below 2^31");
        if (k->shape[0] >= INT32_MAX) return fail(FA_ERR_ARGUMENT, "num_blocks must be below 2^31");
    } else if (k->shape[0] >= INT32_MAX) {
        return fail(FA_ERR_ARGUMENT, "total_k must be below 2^31");
    }
    return alibi_check(alibi, batch, num_heads);
}

// Contract of the paged K/V append.  Its page and head-size rules are the ones
// the pages state for the paged pools the forward reads (pages "paged
// flash-attn requires page_block_size", "page_block_size ... does not match k
// shape" and "... to be a multiple of 32"), with the same texts.
int append_check_impl(const fa_tensor* k_new, const fa_tensor* v_new, int32_t batch, const fa_tensor* bt,
                      const fa_tensor* k_cache, const fa_tensor* v_cache, int32_t page_block_size) {
    if (!k_new || !v_new || !k_cache || !v_cache || !bt)
        return fail(FA_ERR_ARGUMENT, "k_new, v_new, block_table, k_cache and v_cache descriptors must not be NULL");
    for (const fa_tensor* t : {k_new, v_new, k_cache, v_cache, bt})
        if (t->rank < 0 || t->rank > 4)
            return fail(FA_ERR_RANK, "tensor rank must be in 0..4 (got %d)", (int)t->rank);
    for (const fa_tensor* t : {k_new, v_new, k_cache, v_cache})
        if (!is_elem16(t->dtype) || t->dtype != k_new->dtype)
            return fail(FA_ERR_DTYPE, "kv append takes bf16 or f16 k_new/v_new/k_cache/v_cache of one dtype (dtype code %d)",
                        (int)t->dtype);
    if (k_new->rank != 3 || v_new->rank != 3 || k_cache->rank != 4 || v_cache->rank != 4)
        return fail(FA_ERR_RANK,
                    "kv append expects k_new/v_new of rank 3 and k_cache/v_cache of rank 4 (got %d, %d, %d, %d)",
                    (int)k_new->rank, (int)v_new->rank, (int)k_cache->rank, (int)v_cache->rank);
    if (k_new->stride[2] != 1)
        return fail(FA_ERR_CONTIGUOUS, "the last dim of k_new must be contiguous %s", dims(k_new, true).c_str());
    if (v_new->stride[2] != 1)
        return fail(FA_ERR_CONTIGUOUS, "the last dim of v_new must be contiguous %s", dims(v_new, true).c_str());
    if (k_cache->stride[3] != 1)
        return fail(FA_ERR_CONTIGUOUS, "the last dim of k must be contiguous %s", dims(k_cache, true).c_str());
    if (v_cache->stride[3] != 1)
        return fail(FA_ERR_CONTIGUOUS, "the last dim of v must be contiguous %s", dims(v_cache, true).c_str());
    for (const fa_tensor* t : {k_new, v_new, k_cache, v_cache, bt})
        for (int i = 0; i < t->rank; ++i)
            if (t->shape[i] < 0 || t->stride[i] < 0)
                return fail(FA_ERR_SHAPE, "negative shape or stride %s / %s", dims(t, false).c_str(),
                            dims(t, true).c_str());
    if (!same_dims(k_cache, v_cache))
        return fail(FA_ERR_SHAPE, "shape mismatch k %s and v %s", dims(k_cache, false).c_str(),
                    dims(v_cache, false).c_str());
    if (!same_dims(k_new, v_new))
        return fail(FA_ERR_SHAPE, "shape mismatch k_new %s and v_new %s", dims(k_new, false).c_str(),
                    dims(v_new, false).c_str());
    if (k_new->shape[1] != k_cache->shape[2] || k_new->shape[2] != k_cache->shape[3])
        return fail(FA_ERR_SHAPE, "shape mismatch k_new %s and k %s", dims(k_new, false).c_str(),
                    dims(k_cache, false).c_str());
    const int64_t page = k_cache->shape[1], head_size = k_cache->shape[3];
    if (page_block_size <= 0) return fail(FA_ERR_PAGE_SIZE, "paged flash-attn requires page_block_size");
    if ((int64_t)page_block_size != page)
        return fail(FA_ERR_PAGE_SIZE, "page_block_size %d does not match k shape %s", (int)page_block_size,
                    dims(k_cache, false).c_str());
    if (page % 32 != 0)
        return fail(FA_ERR_PAGE_SIZE, "paged flash-attn requires page_block_size to be a multiple of 32 (got %lld)",
                    (long long)page);
    if (head_size > 512)
        return fail(FA_ERR_HEAD_DIM, "paged flash-attn supports head sizes up to 512 (got %lld)",
                    (long long)head_size);
    if (head_size < 1 || k_new->shape[1] < 1)
        return fail(FA_ERR_HEAD_DIM, "kv append needs head_dim >= 1 and num_heads_k >= 1 (got %lld, %lld)",
                    (long long)head_size, (long long)k_new->shape[1]);
    if (batch < 0) return fail(FA_ERR_ARGUMENT, "batch must be >= 0 (got %d)", (int)batch);
    if (bt->dtype != FA_DTYPE_I32)
        return fail(FA_ERR_DTYPE, "block_table must be int32 (dtype code %d)", (int)bt->dtype);
    if (bt->rank != 2 || bt->shape[0] != batch)
        return fail(FA_ERR_SHAPE, "block_table must have shape (batch=%d, max_blocks) (got %s)", (int)batch,
                    dims(bt, false).c_str());
    if (bt->stride[1] != 1 && bt->shape[1] > 1)
        return fail(FA_ERR_CONTIGUOUS, "block_table last dimension must be contiguous");
    if (bt->shape[1] * page >= INT32_MAX)
        return fail(FA_ERR_ARGUMENT, "max_blocks * page_block_size must be below 2^31");
    if (k_cache->shape[0] >= INT32_MAX) return fail(FA_ERR_ARGUMENT, "num_blocks must be below 2^31");
    if (k_new->shape[0] * k_new->shape[1] * head_size >= INT32_MAX)
        return fail(FA_ERR_ARGUMENT, "total_new * num_heads_k * head_dim must be below 2^31");
    return FA_OK;
}

fa::Shapes shapes_of(const fa_tensor* q, const fa_tensor* k, int32_t batch, const fa_tensor* bt,
                     int32_t page_block_size) {
    fa::Shapes s;
    s.total_q = q->shape[0];
    s.H = q->shape[1];
    s.D = q->shape[2];
    s.paged = bt != nullptr;
    s.Hk = s.paged ? k->shape[2] : k->shape[1];
    s.max_lk = s.paged ? bt->shape[1] * (int64_t)page_block_size : k->shape[0];
    s.batch = batch;
    return s;
}

bool is_device_ptr(const void* p) {
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Launch-time values that differ between the varlen and the padded entry.
struct Extra {
    int32_t padded = 0, uniform_q = 0, uniform_k = 0;
    int64_t q_bx = 0, k_bx = 0, v_bx = 0, o_bx = 0;
    int64_t lse_sh = 0, lse_bx = 0;
    bool vec_ok = true;   // alignment of the strides the 3-d views do not show
    bool static_ws = false;  // the workspace is the library's own device array
    fa::Shapes shapes{};
};

// Contract of the padded (non-varlen) entry: q/out (B, Sq, H, D), k/v (B, Sk, Hk, D).
int padded_check_impl(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* out,
                      const fa_tensor* alibi) {
    if (!q || !k || !v) return fail(FA_ERR_ARGUMENT, "q, k and v descriptors must not be NULL");
    // rank, then last-dim contiguity, then shapes, then dtypes: the varlen entry's order
    if (q->rank != 4 || k->rank != 4 || v->rank != 4)
        return fail(FA_ERR_RANK, "flash-attn expects (batch, seqlen, heads, head_dim) tensors of rank 4 (q: %d, k: %d, v: %d)",
                    (int)q->rank, (int)k->rank, (int)v->rank);
    if (q->stride[3] != 1)
        return fail(FA_ERR_CONTIGUOUS, "the last dim of q must be contiguous %s", dims(q, true).c_str());
    if (k->stride[3] != 1)
        return fail(FA_ERR_CONTIGUOUS, "the last dim of k must be contiguous %s", dims(k, true).c_str());
    if (v->stride[3] != 1)
        return fail(FA_ERR_CONTIGUOUS, "the last dim of v must be contiguous %s", dims(v, true).c_str());
    for (const fa_tensor* t : {q, k, v})
        for (int i = 0; i < 4; ++i)
            if (t->shape[i] < 0 || t->stride[i] < 0)
                return fail(FA_ERR_SHAPE, "negative shape or stride %s / %s", dims(t, false).c_str(),
                            dims(t, true).c_str());
    if (!same_dims(k, v))
        return fail(FA_ERR_SHAPE, "shape mismatch k %s and v %s", dims(k, false).c_str(), dims(v, false).c_str());
    if (k->shape[0] != q->shape[0] || k->shape[3] != q->shape[3])
        return fail(FA_ERR_SHAPE, "shape mismatch q %s and k %s", dims(q, false).c_str(), dims(k, false).c_str());
    if (!is_elem16(q->dtype) || k->dtype != q->dtype || v->dtype != q->dtype)
        return fail(FA_ERR_DTYPE, "flash-attn takes bf16 or f16 q/k/v of one dtype (dtype codes q: %d, k: %d, v: %d)",
                    (int)q->dtype, (int)k->dtype, (int)v->dtype);
    const int64_t B = q->shape[0], Sq = q->shape[1], H = q->shape[2], D = q->shape[3];
    const int64_t Sk = k->shape[1], Hk = k->shape[2];
    if (D < 1 || D > 512)
        return fail(FA_ERR_HEAD_DIM, "flash-attn supports head sizes 1..512 (got %lld)", (long long)D);
    if (H < 1 || Hk < 1 || H % Hk != 0)
        return fail(FA_ERR_ARGUMENT,
                    "number of heads in q (%lld) must be a positive multiple of the number of heads in k/v (%lld)",
                    (long long)H, (long long)Hk);
    if (B * Sq * H >= INT32_MAX || B * Sk >= INT32_MAX || B >= INT32_MAX)
        return fail(FA_ERR_ARGUMENT, "batch * seqlen_q * heads and batch * seqlen_k must be below 2^31");
    if (out) {
        if (out->dtype != q->dtype)
            return fail(FA_ERR_DTYPE, "out must have the dtype of q (dtype codes %d and %d)", (int)out->dtype,
                        (int)q->dtype);
        if (!same_dims(out, q))
            return fail(FA_ERR_SHAPE, "out must have the shape of q %s (got %s)", dims(q, false).c_str(),
                        dims(out, false).c_str());
        if (out->stride[3] != 1)
            return fail(FA_ERR_CONTIGUOUS, "the last dim of out must be contiguous %s", dims(out, true).c_str());
        for (int i = 0; i < 4; ++i)
            if (out->stride[i] < 0)
                return fail(FA_ERR_SHAPE, "negative shape or stride %s / %s", dims(out, false).c_str(),
                            dims(out, true).c_str());
    }
    return alibi_check(alibi, B, H);
}

fa::Shapes padded_shapes(const fa_tensor* q, const fa_tensor* k) {
    fa::Shapes s;
    s.total_q = q->shape[0] * q->shape[1];
    s.H = q->shape[2];
    s.D = q->shape[3];
    s.Hk = k->shape[2];
    s.max_lk = k->shape[1];  // every sequence has seqlen_k keys
    s.batch = q->shape[0];
    s.paged = false;
    return s;
}

// ------------------------------------------------------------ FA_VALIDATE
//
// The fast path trusts the contents of the offsets and the block table: the
// kernels only clamp them into the tensors they were given (a bad table gives
// wrong values, never an access outside the buffers).  With FA_VALIDATE=1 in
// the environment, the forward and the append first copy those arrays to the
// host on the call's stream, wait for them (the library's one synchronizing
// path, for debugging) and reject what the contract forbids, launching nothing.

bool validate_on() {
    const char* e = std::getenv("FA_VALIDATE");
    return e && std::strcmp(e, "1") == 0;
}

int copy_to_host(std::vector<int32_t>* dst, const int32_t* src, size_t n, void* stream) {
    dst->assign(n, 0);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(dst->data(), src, n * sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "FA_VALIDATE: copying the metadata failed: %s", hipGetErrorString(e));
    return FA_OK;
}

// offsets: non-decreasing, within [0, limit] (limit < 0: no upper bound)
int check_offsets(const std::vector<int32_t>& cu, const char* name, int64_t limit) {
    for (size_t b = 0; b < cu.size(); ++b) {
        const bool bad = cu[b] < 0 || (limit >= 0 && cu[b] > limit) || (b > 0 && cu[b] < cu[b - 1]);
        if (bad && b == 0)
            return fail(FA_ERR_ARGUMENT, "FA_VALIDATE: %s must be non-decreasing within [0, %lld] (entry 0 is %d)",
                        name, (long long)(limit >= 0 ? limit : INT32_MAX), cu[0]);
        if (bad)
            return fail(FA_ERR_ARGUMENT, "FA_VALIDATE: %s must be non-decreasing within [0, %lld] (entry %zu is %d after %d)",
                        name, (long long)(limit >= 0 ? limit : INT32_MAX), b, cu[b], cu[b - 1]);
    }
    return FA_OK;
}

// the block ids of keys [j0, j1) of sequence b lie in [0, num_blocks)
int check_pages(const std::vector<int32_t>& tab, int64_t row_stride, int32_t b, int64_t j0, int64_t j1, int32_t P,
                int64_t num_blocks) {
    if (j1 <= j0) return FA_OK;
    for (int64_t pg = j0 / P; pg <= (j1 - 1) / P; ++pg) {
        const int32_t id = tab[(size_t)(b * row_stride + pg)];
        if (id < 0 || id >= num_blocks)
            return fail(FA_ERR_ARGUMENT, "FA_VALIDATE: block_table[%d][%lld] = %d is outside the pool of %lld blocks",
                        b, (long long)pg, id, (long long)num_blocks);
    }
    return FA_OK;
}

int copy_table(std::vector<int32_t>* dst, const fa_tensor* bt, int32_t batch, void* stream) {
    const size_t n = batch > 0 ? (size_t)(batch - 1) * (size_t)bt->stride[0] + (size_t)bt->shape[1] : 0;
    return copy_to_host(dst, static_cast<const int32_t*>(bt->data), n, stream);
}

// forward: offsets within q (and, packed, within k); paged, every sequence's keys
// within the table's width and their block ids inside the pool
int validate_fwd(const fa_tensor* q, const fa_tensor* k, const int32_t* cu_q, const int32_t* cu_k, int32_t batch,
                 const fa_tensor* bt, int32_t P, void* stream) {
    std::vector<int32_t> hq, hk, tab;
    int rc = copy_to_host(&hq, cu_q, (size_t)batch + 1, stream);
    if (!rc) rc = copy_to_host(&hk, cu_k, (size_t)batch + 1, stream);
    if (!rc) rc = check_offsets(hq, "cu_seqlens_q", q->shape[0]);
    if (!rc) rc = check_offsets(hk, "cu_seqlens_k", bt ? -1 : k->shape[0]);
    if (rc || !bt) return rc;
    rc = copy_table(&tab, bt, batch, stream);
    const int64_t cap = bt->shape[1] * (int64_t)P;
    for (int32_t b = 0; !rc && b < batch; ++b) {
        const int64_t lk = (int64_t)hk[b + 1] - hk[b];
        if (lk > cap)
            return fail(FA_ERR_ARGUMENT, "FA_VALIDATE: sequence %d has %lld keys, more than %lld pages of %d",
                        b, (long long)lk, (long long)bt->shape[1], P);
        rc = check_pages(tab, bt->stride[0], b, 0, lk, P, k->shape[0]);
    }
    return rc;
}

// append: new rows within k_new, each sequence's new rows at the end of its keys,
// its keys within the table's width, the pages they land in inside the pool
int validate_append(int64_t total_new, const int32_t* cu_new, const int32_t* cu_k, int32_t batch,
                    const fa_tensor* bt, int32_t P, int64_t num_blocks, void* stream) {
    std::vector<int32_t> hn, hk, tab;
    int rc = copy_to_host(&hn, cu_new, (size_t)batch + 1, stream);
    if (!rc) rc = copy_to_host(&hk, cu_k, (size_t)batch + 1, stream);
    if (!rc) rc = check_offsets(hn, "cu_seqlens_new", total_new);
    if (!rc) rc = check_offsets(hk, "cu_seqlens_k", -1);
    if (!rc) rc = copy_table(&tab, bt, batch, stream);
    const int64_t cap = bt->shape[1] * (int64_t)P;
    for (int32_t b = 0; !rc && b < batch; ++b) {
        const int64_t lk = (int64_t)hk[b + 1] - hk[b], ln = (int64_t)hn[b + 1] - hn[b];
        if (ln > lk)
            return fail(FA_ERR_ARGUMENT, "FA_VALIDATE: sequence %d appends %lld rows but has %lld keys after the append",
                        b, (long long)ln, (long long)lk);
        if (lk > cap)
            return fail(FA_ERR_ARGUMENT, "FA_VALIDATE: sequence %d has %lld keys, more than %lld pages of %d",
                        b, (long long)lk, (long long)bt->shape[1], P);
        rc = check_pages(tab, bt->stride[0], b, lk - ln, lk, P, num_blocks);
    }
    return rc;
}

// Device checks, plan, parameters and launch shared by both entries.  q/k/v/out
// are rank-3 (token, head, dim) views (paged k/v: rank 4); cu arrays are only
// read when the call is varlen.
int run_fwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* out,
            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch, const fa_tensor* block_table,
            int32_t page_block_size, float softmax_scale, int32_t window_left, int32_t window_right,
            const fa_tensor* alibi, float* softmax_lse, void* workspace, size_t workspace_bytes, void* stream,
            const Extra& ex) {
    const bool paged = block_table != nullptr;
    const int64_t total_q = q->shape[0];
    if (paged && (!block_table->data || !is_device_ptr(block_table->data)))
        return fail(FA_ERR_DEVICE, "block_table must be a cuda tensor");
    if (!q->data || !is_device_ptr(q->data)) return fail(FA_ERR_DEVICE, "q must be a cuda tensor");
    // k/v without any row are never read (every sequence then has no key)
    const bool kv_empty = k->shape[0] == 0;
    if (!kv_empty && (!k->data || !is_device_ptr(k->data))) return fail(FA_ERR_DEVICE, "k must be a cuda tensor");
    if (!kv_empty && (!v->data || !is_device_ptr(v->data))) return fail(FA_ERR_DEVICE, "v must be a cuda tensor");
    if (!out->data || !is_device_ptr(out->data)) return fail(FA_ERR_DEVICE, "out must be a cuda tensor");
    if (softmax_lse && !is_device_ptr(softmax_lse))
        return fail(FA_ERR_DEVICE, "softmax_lse must be a cuda tensor");
    if (alibi && (!alibi->data || !is_device_ptr(alibi->data)))
        return fail(FA_ERR_DEVICE, "alibi_slopes must be a cuda tensor");
    int rc = FA_OK;
    if (!ex.padded && validate_on()) {
        rc = validate_fwd(q, k, cu_seqlens_q, cu_seqlens_k, batch, block_table, page_block_size, stream);
        if (rc) return rc;
    }

    fa::Plan plan;
    rc = fa::make_plan(ex.shapes, &plan);
    if (rc) return fail(rc, "no launch plan for these shapes");
    if (plan.ws_bytes) {
        if (!workspace || workspace_bytes < plan.ws_bytes)
            return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", plan.ws_bytes,
                        workspace ? workspace_bytes : (size_t)0);
        if (!aligned16(workspace)) return fail(FA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
        if (!ex.static_ws && !is_device_ptr(workspace)) return fail(FA_ERR_DEVICE, "workspace must be a cuda tensor");
    }

    fa::FwdParams p;
    std::memset(&p, 0, sizeof p);
    p.q = static_cast<const uint16_t*>(q->data);
    p.k = static_cast<const uint16_t*>(k->data);
    p.v = static_cast<const uint16_t*>(v->data);
    p.out = static_cast<uint16_t*>(out->data);
    p.lse = softmax_lse;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.q_s0 = q->stride[0];
    p.q_s1 = q->stride[1];
    p.o_s0 = out->stride[0];
    p.o_s1 = out->stride[1];
    if (paged) {
        p.bt = static_cast<const int32_t*>(block_table->data);
        p.bt_s0 = block_table->stride[0];
        p.page = page_block_size;
        p.k_s0 = k->stride[0]; p.k_s1 = k->stride[1]; p.k_s2 = k->stride[2];
        p.v_s0 = v->stride[0]; p.v_s1 = v->stride[1]; p.v_s2 = v->stride[2];
    } else {
        p.bt = nullptr;
        p.page = 0;
        p.k_s0 = k->stride[0]; p.k_s1 = k->stride[1]; p.k_s2 = 0;
        p.v_s0 = v->stride[0]; p.v_s1 = v->stride[1]; p.v_s2 = 0;
    }
    p.batch = batch;
    p.max_lk = (int32_t)(paged ? block_table->shape[1] * (int64_t)page_block_size : k->shape[0]);
    p.num_blocks = (int32_t)(paged ? k->shape[0] : 0);
    p.H = (int32_t)q->shape[1];
    p.Hk = (int32_t)(paged ? k->shape[2] : k->shape[1]);
    p.G = p.H / p.Hk;
    p.D = (int32_t)q->shape[2];
    p.total_q = (int32_t)total_q;
    p.window_left = window_left < 0 ? -1 : window_left;
    p.window_right = window_right < 0 ? -1 : window_right;
    p.chunk = plan.chunk;
    p.max_chunks = plan.max_chunks;
    p.scale_log2 = softmax_scale * 1.4426950408889634f;
    p.f16 = q->dtype == FA_DTYPE_F16 ? 1 : 0;
    p.alibi = alibi ? static_cast<const float*>(alibi->data) : nullptr;
    p.alibi_sb = (alibi && alibi->rank == 2) ? alibi->stride[0] : 0;
    p.padded = ex.padded;
    p.uniform_q = ex.uniform_q;
    p.uniform_k = ex.uniform_k;
    p.q_bx = ex.q_bx;
    p.k_bx = ex.k_bx;
    p.v_bx = ex.v_bx;
    p.o_bx = ex.o_bx;
    p.lse_sh = ex.lse_sh;
    p.lse_bx = ex.lse_bx;
    {
        unsigned char* ws = static_cast<unsigned char*>(workspace);
        if (plan.max_chunks > 1) {
            const size_t n_o = (size_t)plan.max_chunks * (size_t)total_q * (size_t)p.H * (size_t)plan.dp;
            p.part_o = reinterpret_cast<float*>(ws);
            p.part_lse = p.part_o + n_o;
        }
        p.items = reinterpret_cast<int4*>(ws + plan.off_items);
        p.item_count = reinterpret_cast<int32_t*>(ws + plan.off_count);
        p.seq_off = reinterpret_cast<int32_t*>(ws + plan.off_seq);
        p.tok_nc = reinterpret_cast<int32_t*>(ws + plan.off_tok);
    }
    // 16-byte vector access is legal when every row start is 16-byte aligned
    bool vec = (p.D % 8 == 0) && ex.vec_ok;
    for (const fa_tensor* t : {q, k, v, out}) {
        if (t->shape[0] == 0) continue;  // never read
        vec = vec && aligned16(t->data);
        for (int i = 0; i + 1 < t->rank; ++i) vec = vec && (t->stride[i] % 8 == 0);
    }
    p.vec = vec ? 1 : 0;
    // the uniform-base copy path needs the padded head dim to be the real one and
    // the per-lane byte offsets (up to 8 rows) to fit in 32 bits
    {
        const int dp = p.D <= 64 ? 64 : p.D <= 128 ? 128 : p.D <= 256 ? 256 : 512;
        const int64_t krow = 2 * (paged ? k->stride[1] : k->stride[0]);
        const int64_t vrow = 2 * (paged ? v->stride[1] : v->stride[0]);
        p.k_rowb = (int32_t)std::min<int64_t>(krow, INT32_MAX);
        p.v_rowb = (int32_t)std::min<int64_t>(vrow, INT32_MAX);
        p.fast_copy = (vec && p.D == dp && 128 * krow + 2 * dp < INT32_MAX && 128 * vrow + 2 * dp < INT32_MAX) ? 1 : 0;
    }

    rc = fa::launch_fwd(plan, p, stream, g_ev_start, g_ev_stop);
    if (rc) return fail(rc, "kernel launch failed: %s", fa::last_hip_error());
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_varlen_check(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* out,
                    int32_t batch, const fa_tensor* block_table, int32_t page_block_size,
                    const fa_tensor* alibi_slopes) {
    return check_impl(q, k, v, out, batch, block_table, page_block_size, alibi_slopes);
}

int fa_varlen_workspace_bytes(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, int32_t batch,
                              const fa_tensor* block_table, int32_t page_block_size, size_t* bytes) {
    if (!bytes) return fail(FA_ERR_ARGUMENT, "bytes must not be NULL");
    int rc = check_impl(q, k, v, nullptr, batch, block_table, page_block_size, nullptr);
    if (rc) return rc;
    fa::Plan plan;
    rc = fa::make_plan(shapes_of(q, k, batch, block_table, page_block_size), &plan);
    if (rc) return fail(rc, "no launch plan for these shapes");
    *bytes = plan.ws_bytes;
    return FA_OK;
}

int fa_varlen_fwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* out,
                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                  const fa_tensor* block_table, int32_t page_block_size, float softmax_scale,
                  int32_t window_left, int32_t window_right, const fa_tensor* alibi_slopes,
                  float* softmax_lse, void* workspace, size_t workspace_bytes, void* stream) {
    if (!out) return fail(FA_ERR_ARGUMENT, "out descriptor must not be NULL");
    int rc = check_impl(q, k, v, out, batch, block_table, page_block_size, alibi_slopes);
    if (rc) return rc;
    if (batch == 0 || q->shape[0] == 0) return FA_OK;  // nothing to compute, nothing written
    if (!cu_seqlens_q || !is_device_ptr(cu_seqlens_q))
        return fail(FA_ERR_DEVICE, "seqlens_q must be a cuda tensor");
    if (!cu_seqlens_k || !is_device_ptr(cu_seqlens_k))
        return fail(FA_ERR_DEVICE, "seqlens_k must be a cuda tensor");
    Extra ex;
    ex.lse_sh = q->shape[0];
    ex.shapes = shapes_of(q, k, batch, block_table, page_block_size);
    return run_fwd(q, k, v, out, cu_seqlens_q, cu_seqlens_k, batch, block_table, page_block_size, softmax_scale,
                   window_left, window_right, alibi_slopes, softmax_lse, workspace, workspace_bytes, stream, ex);
}

int fa_varlen_fwd_static(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* out,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                         const fa_tensor* block_table, int32_t page_block_size, float softmax_scale,
                         int32_t window_left, int32_t window_right, const fa_tensor* alibi_slopes,
                         float* softmax_lse, void* stream) {
    if (!out) return fail(FA_ERR_ARGUMENT, "out descriptor must not be NULL");
    int rc = check_impl(q, k, v, out, batch, block_table, page_block_size, alibi_slopes);
    if (rc) return rc;
    if (batch == 0 || q->shape[0] == 0) return FA_OK;  // nothing to compute, nothing written
    if (!cu_seqlens_q || !is_device_ptr(cu_seqlens_q))
        return fail(FA_ERR_DEVICE, "seqlens_q must be a cuda tensor");
    if (!cu_seqlens_k || !is_device_ptr(cu_seqlens_k))
        return fail(FA_ERR_DEVICE, "seqlens_k must be a cuda tensor");
    Extra ex;
    ex.lse_sh = q->shape[0];
    ex.shapes = shapes_of(q, k, batch, block_table, page_block_size);
    ex.static_ws = true;
    fa::Plan plan;
    rc = fa::make_plan(ex.shapes, &plan);
    if (rc) return fail(rc, "no launch plan for these shapes");
    if (plan.ws_bytes > FA_STATIC_SCRATCH_BYTES)
        return fail(FA_ERR_WORKSPACE,
                    "fa_varlen_fwd_static: these shapes need %zu bytes of scratch, more than the %zu of the "
                    "static scratch; call fa_varlen_fwd with a workspace instead",
                    plan.ws_bytes, (size_t)FA_STATIC_SCRATCH_BYTES);
    void* ws = nullptr;
    size_t ws_bytes = 0;
    rc = fa::static_scratch(stream, &ws, &ws_bytes);
    if (rc == FA_ERR_DEVICE) return fail(rc, "the stream does not belong to the current device");
    if (rc) return fail(rc, "static scratch lookup failed: %s", fa::last_hip_error());
    return run_fwd(q, k, v, out, cu_seqlens_q, cu_seqlens_k, batch, block_table, page_block_size, softmax_scale,
                   window_left, window_right, alibi_slopes, softmax_lse, ws, ws_bytes, stream, ex);
}

int fa_padded_check(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* out,
                    const fa_tensor* alibi_slopes) {
    return padded_check_impl(q, k, v, out, alibi_slopes);
}

int fa_padded_workspace_bytes(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, size_t* bytes) {
    if (!bytes) return fail(FA_ERR_ARGUMENT, "bytes must not be NULL");
    int rc = padded_check_impl(q, k, v, nullptr, nullptr);
    if (rc) return rc;
    fa::Plan plan;
    rc = fa::make_plan(padded_shapes(q, k), &plan);
    if (rc) return fail(rc, "no launch plan for these shapes");
    *bytes = plan.ws_bytes;
    return FA_OK;
}

int fa_padded_fwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* out,
                  float softmax_scale, int32_t window_left, int32_t window_right, const fa_tensor* alibi_slopes,
                  float* softmax_lse, void* workspace, size_t workspace_bytes, void* stream) {
    if (!out) return fail(FA_ERR_ARGUMENT, "out descriptor must not be NULL");
    int rc = padded_check_impl(q, k, v, out, alibi_slopes);
    if (rc) return rc;
    const int64_t B = q->shape[0], Sq = q->shape[1], Sk = k->shape[1];
    if (B == 0 || Sq == 0) return FA_OK;
    // the same operation over (B*S, heads, head_dim) views: row t of sequence b
    // sits at t * token_stride + b * (batch_stride - S * token_stride)
    fa_tensor q3, k3, v3, o3;
    auto flat = [](const fa_tensor* t4, fa_tensor* t3) {
        *t3 = *t4;
        t3->rank = 3;
        t3->shape[0] = t4->shape[0] * t4->shape[1];
        t3->shape[1] = t4->shape[2];
        t3->shape[2] = t4->shape[3];
        t3->stride[0] = t4->stride[1];
        t3->stride[1] = t4->stride[2];
        t3->stride[2] = t4->stride[3];
        t3->shape[3] = t3->stride[3] = 0;
    };
    flat(q, &q3);
    flat(k, &k3);
    flat(v, &v3);
    flat(out, &o3);
    Extra ex;
    ex.padded = 1;
    ex.uniform_q = (int32_t)Sq;
    ex.uniform_k = (int32_t)Sk;
    ex.q_bx = q->stride[0] - Sq * q->stride[1];
    ex.k_bx = k->stride[0] - Sk * k->stride[1];
    ex.v_bx = v->stride[0] - Sk * v->stride[1];
    ex.o_bx = out->stride[0] - Sq * out->stride[1];
    ex.lse_sh = Sq;                           // softmax_lse is (B, H, Sq)
    ex.lse_bx = (q->shape[2] - 1) * Sq;
    ex.vec_ok = q->stride[0] % 8 == 0 && k->stride[0] % 8 == 0 && v->stride[0] % 8 == 0 &&
                out->stride[0] % 8 == 0;
    ex.shapes = padded_shapes(q, k);
    return run_fwd(&q3, &k3, &v3, &o3, nullptr, nullptr, (int32_t)B, nullptr, 0, softmax_scale, window_left,
                   window_right, alibi_slopes, softmax_lse, workspace, workspace_bytes, stream, ex);
}

int fa_kv_append_check(const fa_tensor* k_new, const fa_tensor* v_new, int32_t batch,
                       const fa_tensor* block_table, const fa_tensor* k_cache, const fa_tensor* v_cache,
                       int32_t page_block_size) {
    return append_check_impl(k_new, v_new, batch, block_table, k_cache, v_cache, page_block_size);
}

int fa_kv_append(const fa_tensor* k_new, const fa_tensor* v_new, const int32_t* cu_seqlens_new,
                 const int32_t* cu_seqlens_k, int32_t batch, const fa_tensor* block_table,
                 const fa_tensor* k_cache, const fa_tensor* v_cache, int32_t page_block_size, void* stream) {
    int rc = append_check_impl(k_new, v_new, batch, block_table, k_cache, v_cache, page_block_size);
    if (rc) return rc;
    const int64_t total_new = k_new->shape[0];
    if (batch == 0 || total_new == 0) return FA_OK;  // nothing to write

    if (!cu_seqlens_new || !is_device_ptr(cu_seqlens_new))
        return fail(FA_ERR_DEVICE, "seqlens_new must be a cuda tensor");
    if (!cu_seqlens_k || !is_device_ptr(cu_seqlens_k))
        return fail(FA_ERR_DEVICE, "seqlens_k must be a cuda tensor");
    if (!block_table->data || !is_device_ptr(block_table->data))
        return fail(FA_ERR_DEVICE, "block_table must be a cuda tensor");
    if (!k_new->data || !is_device_ptr(k_new->data)) return fail(FA_ERR_DEVICE, "k_new must be a cuda tensor");
    if (!v_new->data || !is_device_ptr(v_new->data)) return fail(FA_ERR_DEVICE, "v_new must be a cuda tensor");
    if (!k_cache->data || !is_device_ptr(k_cache->data)) return fail(FA_ERR_DEVICE, "k must be a cuda tensor");
    if (!v_cache->data || !is_device_ptr(v_cache->data)) return fail(FA_ERR_DEVICE, "v must be a cuda tensor");
    if (validate_on()) {
        rc = validate_append(total_new, cu_seqlens_new, cu_seqlens_k, batch, block_table, page_block_size,
                             k_cache->shape[0], stream);
        if (rc) return rc;
    }

    fa::AppendParams p;
    std::memset(&p, 0, sizeof p);
    p.k_new = static_cast<const uint16_t*>(k_new->data);
    p.v_new = static_cast<const uint16_t*>(v_new->data);
    p.k_cache = static_cast<uint16_t*>(k_cache->data);
    p.v_cache = static_cast<uint16_t*>(v_cache->data);
    p.cu_new = cu_seqlens_new;
    p.cu_k = cu_seqlens_k;
    p.bt = static_cast<const int32_t*>(block_table->data);
    p.kn_s0 = k_new->stride[0]; p.kn_s1 = k_new->stride[1];
    p.vn_s0 = v_new->stride[0]; p.vn_s1 = v_new->stride[1];
    p.kc_s0 = k_cache->stride[0]; p.kc_s1 = k_cache->stride[1]; p.kc_s2 = k_cache->stride[2];
    p.vc_s0 = v_cache->stride[0]; p.vc_s1 = v_cache->stride[1]; p.vc_s2 = v_cache->stride[2];
    p.bt_s0 = block_table->stride[0];
    p.batch = batch;
    p.Hk = (int32_t)k_new->shape[1];
    p.D = (int32_t)k_new->shape[2];
    p.page = page_block_size;
    p.bt_width = (int32_t)block_table->shape[1];
    p.num_blocks = (int32_t)k_cache->shape[0];
    bool vec = (p.D % 8 == 0);
    for (const fa_tensor* t : {k_new, v_new, k_cache, v_cache}) {
        vec = vec && aligned16(t->data);
        for (int i = 0; i + 1 < t->rank; ++i) vec = vec && (t->stride[i] % 8 == 0);
    }
    p.vec = vec ? 1 : 0;
    p.upr = vec ? p.D / 8 : p.D;
    p.units = (uint32_t)(total_new * p.Hk * p.upr);
    rc = fa::launch_kv_append(p, stream, g_ev_start, g_ev_stop);
    if (rc) return fail(rc, "kernel launch failed: %s", fa::last_append_error());
    return FA_OK;
}

int fa_varlen_set_kernel_events(void* start_event, void* stop_event) {
    if (start_event && stop_event) {
        g_ev_start = start_event;
        g_ev_stop = stop_event;
    } else {
        g_ev_start = g_ev_stop = nullptr;
    }
    return FA_OK;
}

const char* fa_last_error(void) { return g_err.c_str(); }

}  // extern "C"
