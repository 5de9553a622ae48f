/*
 * fa_oracle.c -- fp64 reference for the varlen (paged) softmax-attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the test suite, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no source with the HIP library.
 *
 * What it computes is the plain definition, written out:
 *
 *   For sequence b with Lq = cu_q[b+1]-cu_q[b] queries and Lk = cu_k[b+1]-cu_k[b]
 *   keys, query head h reads key/value head hk = h / (num_heads / num_heads_k).
 *   Query row i is aligned to key position a = i + Lk - Lq (bottom-right), and
 *   key j is visible to it iff 0 <= j < Lk and
 *       (window_left  < 0 or j >= a - window_left) and
 *       (window_right < 0 or j <= a + window_right).
 *   s_j = scale * sum_d q[i][h][d] * k_b[j][hk][d]  -  slope_bh * |a - j|
 *         (the ALiBi term only when slopes are given; slope_bh = alibi[b][h] or
 *         alibi[h]: the pages name the alibi_slopes argument through its shape
 *         error, page "page_block_size ... does not match k shape", Related
 *         errors; the linear distance penalty is the plainest reading, taken
 *         with the same bottom-right alignment a as the window)
 *   out[i][h][:] = sum_j softmax(s)_j * v_b[j][hk][:]   (0 if no key is visible)
 *   lse[h][i]    = log(sum_j exp(s_j))                  (-inf if no key is visible)
 *
 * Sources for each part (pages of the huggingface/candle error explainers):
 *  - packed layouts q (total_q, num_heads, head_dim) and k/v
 *    (total_k, num_heads_k, head_dim): page "flash-attn-varlen expects input
 *    tensors of rank 3", sections What it means and Solutions, and the dims3
 *    destructuring in section Source of page "paged flash-attn requires
 *    page_block_size to be a multiple of 32";
 *  - the paged pool (num_blocks, page_block_size, num_heads_k, head_dim) read
 *    through a per-sequence block table: page "flash-attn-varlen paged expects
 *    k/v tensors of rank 4", section What it means, and page
 *    "page_block_size ... does not match k shape", section What it means;
 *  - softmax_scale, window_len_left and window_len_right as the attention
 *    parameters: page "paged flash-attn requires page_block_size", section
 *    Example fix.
 * The pages name these parameters but do not spell out the mask; the reading
 * used here is the flash-attention window around the bottom-right aligned
 * diagonal, with causal = (window_left < 0, window_right = 0), and GQA heads
 * grouped contiguously.
 *
 * Numerics: inputs are bf16 or IEEE binary16 (fp16) widened exactly to double
 * (the element type the candle wrapper is generic over: page "flash-attn-varlen
 * paged expects k/v tensors of rank 4", section Source); every sum is a plain
 * left-to-right double sum; the softmax is the two-pass stable form (max, then
 * exp and sum).  Work items (sequence, head) are spread over POSIX threads.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE 754 binary16: sign, 5-bit exponent (bias 15), 10-bit fraction. */
static double f16_to_double(uint16_t h) {
    const int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-14 / 1024 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Test hook: widen n 16-bit values (dtype 0 = bf16, 1 = fp16) to double. */
void fa_oracle_widen(const uint16_t *in, int64_t n, int dtype, double *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = dtype ? f16_to_double(in[i]) : bf16_to_double(in[i]);
}

typedef struct {
    const uint16_t *q, *k, *v;
    int f16;               /* element type: 0 = bf16, 1 = fp16 */
    int64_t total_q;
    int num_heads, num_heads_k, head_dim;
    int64_t kv_rows;       /* total_k (non-paged) or num_blocks (paged) */
    int page;              /* 0 = non-paged */
    const int32_t *cu_q, *cu_k;
    int batch;
    const int32_t *block_table;
    int bt_width;
    double scale;
    const double *alibi;   /* NULL, or slopes: alibi[b * alibi_sb + h] */
    int64_t alibi_sb;
    int window_left, window_right;
    const uint8_t *token_sel;
    double *out, *lse;
    int64_t next_item;     /* shared work counter */
    int error;             /* first error seen (block id out of range) */
} job_t;

/* Element offset of logical key/value row j of sequence b, head hk, d = 0.
 * Returns -1 when the block table sends the row outside the pool. */
static int64_t kv_row_offset(const job_t *J, int b, int64_t j, int hk) {
    int64_t row;
    if (J->page == 0) {
        row = (int64_t)J->cu_k[b] + j;
        if (row < 0 || row >= J->kv_rows) return -1;
    } else {
        int64_t slot = j / J->page;
        if (slot >= J->bt_width) return -1;
        int64_t blk = J->block_table[(int64_t)b * J->bt_width + slot];
        if (blk < 0 || blk >= J->kv_rows) return -1;
        row = blk * J->page + j % J->page;
    }
    return (row * J->num_heads_k + hk) * J->head_dim;
}

static int key_visible(const job_t *J, int64_t i, int64_t j, int64_t Lq, int64_t Lk) {
    int64_t a = i + Lk - Lq;
    if (j < 0 || j >= Lk) return 0;
    if (J->window_left >= 0 && j < a - J->window_left) return 0;
    if (J->window_right >= 0 && j > a + J->window_right) return 0;
    return 1;
}

static void run_item(job_t *J, int b, int h, double *s, int64_t *koff) {
    const int D = J->head_dim;
    const int group = J->num_heads / J->num_heads_k;
    const int hk = h / group;
    const int64_t q0 = J->cu_q[b];
    const int64_t Lq = (int64_t)J->cu_q[b + 1] - J->cu_q[b];
    const int64_t Lk = (int64_t)J->cu_k[b + 1] - J->cu_k[b];

    /* logical K_b / V_b rows: gathered once per item, independent of queries */
    for (int64_t j = 0; j < Lk; ++j) {
        koff[j] = kv_row_offset(J, b, j, hk);
        if (koff[j] < 0) { __atomic_store_n(&J->error, 1, __ATOMIC_RELAXED); return; }
    }
    for (int64_t i = 0; i < Lq; ++i) {
        const int64_t t = q0 + i;
        if (J->token_sel && !J->token_sel[t]) continue;
        const uint16_t *qrow = J->q + (t * J->num_heads + h) * D;
        double *orow = J->out + (t * J->num_heads + h) * D;
        double m = -INFINITY;
        int64_t n_visible = 0;
        for (int64_t j = 0; j < Lk; ++j) {
            if (!key_visible(J, i, j, Lq, Lk)) continue;
            const uint16_t *krow = J->k + koff[j];
            double dot = 0.0;
            if (J->f16)
                for (int d = 0; d < D; ++d) dot += f16_to_double(qrow[d]) * f16_to_double(krow[d]);
            else
                for (int d = 0; d < D; ++d) dot += bf16_to_double(qrow[d]) * bf16_to_double(krow[d]);
            s[j] = J->scale * dot;
            if (J->alibi) s[j] -= J->alibi[(int64_t)b * J->alibi_sb + h] * fabs((double)(i + Lk - Lq - j));
            if (s[j] > m) m = s[j];
            ++n_visible;
        }
        for (int d = 0; d < D; ++d) orow[d] = 0.0;
        if (n_visible == 0) {
            J->lse[(int64_t)h * J->total_q + t] = -INFINITY;
            continue;
        }
        double l = 0.0;
        for (int64_t j = 0; j < Lk; ++j) {
            if (!key_visible(J, i, j, Lq, Lk)) continue;
            double p = exp(s[j] - m);
            l += p;
            const uint16_t *vrow = J->v + koff[j];
            if (J->f16)
                for (int d = 0; d < D; ++d) orow[d] += p * f16_to_double(vrow[d]);
            else
                for (int d = 0; d < D; ++d) orow[d] += p * bf16_to_double(vrow[d]);
        }
        for (int d = 0; d < D; ++d) orow[d] /= l;
        J->lse[(int64_t)h * J->total_q + t] = m + log(l);
    }
}

static void *worker(void *arg) {
    job_t *J = (job_t *)arg;
    int64_t maxLk = 1;
    for (int b = 0; b < J->batch; ++b) {
        int64_t Lk = (int64_t)J->cu_k[b + 1] - J->cu_k[b];
        if (Lk > maxLk) maxLk = Lk;
    }
    double *s = (double *)malloc(sizeof(double) * (size_t)maxLk);
    int64_t *koff = (int64_t *)malloc(sizeof(int64_t) * (size_t)maxLk);
    if (!s || !koff) { __atomic_store_n(&J->error, 2, __ATOMIC_RELAXED); free(s); free(koff); return NULL; }
    const int64_t n_items = (int64_t)J->batch * J->num_heads;
    for (;;) {
        int64_t it = __atomic_fetch_add(&J->next_item, 1, __ATOMIC_RELAXED);
        if (it >= n_items) break;
        run_item(J, (int)(it / J->num_heads), (int)(it % J->num_heads), s, koff);
    }
    free(s);
    free(koff);
    return NULL;
}

/*
 * All arrays are host memory, contiguous, row-major:
 *   q    [total_q][num_heads][head_dim]           bf16 (dtype 0) or fp16 (dtype 1) bits
 *   k, v [kv_rows][num_heads_k][head_dim]          (page == 0)
 *        [kv_rows][page][num_heads_k][head_dim]    (page  > 0, kv_rows = num_blocks)
 *   cu_q, cu_k [batch+1]  int32 cumulative lengths
 *   block_table [batch][bt_width] int32 (page > 0 only)
 *   token_sel   [total_q] or NULL: rows with 0 are skipped (left untouched)
 *   out  [total_q][num_heads][head_dim] double;  lse [num_heads][total_q] double
 *   alibi  NULL or ALiBi slopes, slope of (sequence b, head h) at alibi[b * alibi_sb + h]
 *          (alibi_sb = 0: one slope per head for every sequence)
 * Returns 0, or -1 for bad arguments, -2 for a block id / row outside the pool,
 * -3 when memory runs out.
 */
int fa_oracle_attention_t(const uint16_t *q, int64_t total_q, int num_heads, int head_dim,
                          const uint16_t *k, const uint16_t *v, int64_t kv_rows, int page,
                          int num_heads_k, const int32_t *cu_q, const int32_t *cu_k, int batch,
                          const int32_t *block_table, int bt_width, double scale,
                          int window_left, int window_right, const uint8_t *token_sel,
                          double *out, double *lse, int nthreads, int dtype,
                          const double *alibi, int64_t alibi_sb) {
    if (num_heads <= 0 || num_heads_k <= 0 || head_dim <= 0 || batch < 0) return -1;
    if (num_heads % num_heads_k != 0) return -1;
    if (page < 0 || (page > 0 && !block_table)) return -1;
    if (batch > 0 && ((int64_t)cu_q[batch] > total_q)) return -1;
    for (int b = 0; b < batch; ++b)
        if (cu_q[b + 1] < cu_q[b] || cu_k[b + 1] < cu_k[b]) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    if (dtype != 0 && dtype != 1) return -1;
    J.q = q; J.k = k; J.v = v; J.total_q = total_q; J.f16 = dtype;
    J.num_heads = num_heads; J.num_heads_k = num_heads_k; J.head_dim = head_dim;
    J.kv_rows = kv_rows; J.page = page; J.cu_q = cu_q; J.cu_k = cu_k; J.batch = batch;
    J.block_table = block_table; J.bt_width = bt_width; J.scale = scale;
    J.window_left = window_left; J.window_right = window_right; J.token_sel = token_sel;
    J.alibi = alibi; J.alibi_sb = alibi_sb;
    J.out = out; J.lse = lse;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[started], NULL, worker, &J) == 0) ++started;
    worker(&J);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    if (J.error == 1) return -2;
    if (J.error == 2) return -3;
    return 0;
}

/* bf16 entry (dtype 0). */
int fa_oracle_attention(const uint16_t *q, int64_t total_q, int num_heads, int head_dim,
                        const uint16_t *k, const uint16_t *v, int64_t kv_rows, int page,
                        int num_heads_k, const int32_t *cu_q, const int32_t *cu_k, int batch,
                        const int32_t *block_table, int bt_width, double scale,
                        int window_left, int window_right, const uint8_t *token_sel,
                        double *out, double *lse, int nthreads) {
    return fa_oracle_attention_t(q, total_q, num_heads, head_dim, k, v, kv_rows, page, num_heads_k, cu_q,
                                 cu_k, batch, block_table, bt_width, scale, window_left, window_right,
                                 token_sel, out, lse, nthreads, 0, NULL, 0);
}

/*
 * Paged K/V cache append (the write that precedes paged attention): the new
 * tokens of sequence b are its last Lnew_b keys, i.e. new token j sits at
 * logical key position  pos = Lk_b - Lnew_b + j  with  Lk_b = cu_k[b+1]-cu_k[b]
 * (lengths after the append) and  Lnew_b = cu_new[b+1]-cu_new[b];  it is
 * written to block block_table[b][pos / page], slot pos % page, for every K/V
 * head.  Same block-table addressing as the attention's paged reads (page
 * "flash-attn-varlen paged expects k/v tensors of rank 4", What it means;
 * page "page_block_size ... does not match k shape", What it means).
 *
 *   k_new, v_new [total_new][Hk][D] bf16 bits;  k_pool, v_pool
 *   [num_blocks][page][Hk][D] bf16 bits, updated in place.
 * Returns 0, -1 for bad arguments, -2 when a position or block id falls
 * outside the table or the pool (nothing is written for that token).
 */
int fa_oracle_kv_append(const uint16_t *k_new, const uint16_t *v_new, int64_t total_new, int num_heads_k,
                        int head_dim, const int32_t *cu_new, const int32_t *cu_k, int batch,
                        const int32_t *block_table, int bt_width, int page, int64_t num_blocks,
                        uint16_t *k_pool, uint16_t *v_pool) {
    if (batch < 0 || page <= 0 || num_heads_k <= 0 || head_dim <= 0) return -1;
    const int64_t row = (int64_t)num_heads_k * head_dim;
    int rc = 0;
    for (int b = 0; b < batch; ++b) {
        const int64_t n0 = cu_new[b], lnew = (int64_t)cu_new[b + 1] - cu_new[b];
        const int64_t lk = (int64_t)cu_k[b + 1] - cu_k[b];
        for (int64_t j = 0; j < lnew; ++j) {
            const int64_t pos = lk - lnew + j;
            if (n0 + j < 0 || n0 + j >= total_new || pos < 0 || pos / page >= bt_width) { rc = -2; continue; }
            const int64_t blk = block_table[(int64_t)b * bt_width + pos / page];
            if (blk < 0 || blk >= num_blocks) { rc = -2; continue; }
            const int64_t dst = (blk * page + pos % page) * row;
            memcpy(k_pool + dst, k_new + (n0 + j) * row, (size_t)row * sizeof(uint16_t));
            memcpy(v_pool + dst, v_new + (n0 + j) * row, (size_t)row * sizeof(uint16_t));
        }
    }
    return rc;
}
