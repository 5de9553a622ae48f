/* Host driver of the fp64 oracle (oracle/fa_oracle.c), built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_host_sanitizers.py.  It runs the oracle's entry points over
 * packed and paged layouts, windows (including int32-limit ones and rows with
 * more queries than keys), empty sequences, row selection, ALiBi slopes, both
 * 16-bit element types, several threads and the append's skip rules, and
 * checks the return codes and that every computed value is finite; any
 * sanitizer report fails the test.  It shares nothing with the HIP library. */
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int fa_oracle_attention_t(const uint16_t *q, int64_t total_q, int num_heads, int head_dim,
                          const uint16_t *k, const uint16_t *v, int64_t kv_rows, int page,
                          int num_heads_k, const int32_t *cu_q, const int32_t *cu_k, int batch,
                          const int32_t *block_table, int bt_width, double scale,
                          int window_left, int window_right, const uint8_t *token_sel,
                          double *out, double *lse, int nthreads, int dtype,
                          const double *alibi, int64_t alibi_sb);
int fa_oracle_kv_append(const uint16_t *k_new, const uint16_t *v_new, int64_t total_new, int num_heads_k,
                        int head_dim, const int32_t *cu_new, const int32_t *cu_k, int batch,
                        const int32_t *block_table, int bt_width, int page, int64_t num_blocks,
                        uint16_t *k_pool, uint16_t *v_pool);
void fa_oracle_widen(const uint16_t *in, int64_t n, int dtype, double *out);

static int bad = 0;
static uint64_t rng = 88172645463325252ull;

static uint16_t rnd16(int dtype) {
    /* a small finite value of either type: sign, exponent near 1, random mantissa */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    uint16_t sign = (uint16_t)((rng >> 20) & 1) << 15;
    if (dtype == 0) return (uint16_t)(sign | (uint16_t)((126 + (rng >> 40) % 3) << 7) | (uint16_t)(rng & 0x7f));
    return (uint16_t)(sign | (uint16_t)((14 + (rng >> 40) % 3) << 10) | (uint16_t)(rng & 0x3ff));
}

static void fill(uint16_t *x, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) x[i] = rnd16(dtype);
}

/* one call; paged when page > 0 (every sequence's pages at consecutive ids) */
static void run_case(const char *what, int batch, const int *lq, const int *lk, int H, int Hk, int D, int page,
                     int wl, int wr, int dtype, int use_alibi, int use_sel, int threads) {
    int32_t *cu_q = calloc(batch + 1, 4), *cu_k = calloc(batch + 1, 4);
    int width = 1, need = 0;
    for (int b = 0; b < batch; ++b) {
        cu_q[b + 1] = cu_q[b] + lq[b];
        cu_k[b + 1] = cu_k[b] + lk[b];
        int p = page ? (lk[b] + page - 1) / page : 0;
        if (p > width) width = p;
        need += p;
    }
    const int64_t tq = cu_q[batch], tk = cu_k[batch];
    const int64_t rows = page ? (int64_t)(need + 1) * page : (tk > 0 ? tk : 1);
    uint16_t *q = malloc(sizeof(uint16_t) * (size_t)(tq * H * D + 1));
    uint16_t *k = malloc(sizeof(uint16_t) * (size_t)(rows * Hk * D));
    uint16_t *v = malloc(sizeof(uint16_t) * (size_t)(rows * Hk * D));
    fill(q, tq * H * D, dtype);
    fill(k, rows * Hk * D, dtype);
    fill(v, rows * Hk * D, dtype);
    int32_t *bt = NULL;
    if (page) {
        bt = malloc(sizeof(int32_t) * (size_t)(batch * width));
        int id = need;  /* last ids first, so blocks are not in table order */
        for (int b = 0; b < batch; ++b)
            for (int j = 0; j < width; ++j)
                bt[b * width + j] = j < (lk[b] + page - 1) / page ? --id : -1;
    }
    double *al = NULL;
    if (use_alibi) {
        al = malloc(sizeof(double) * (size_t)(batch * H));
        for (int i = 0; i < batch * H; ++i) al[i] = 0.05 * (i % 7 + 1);
    }
    uint8_t *sel = NULL;
    if (use_sel) {
        sel = malloc((size_t)tq + 1);
        for (int64_t t = 0; t < tq; ++t) sel[t] = (uint8_t)(t % 3 == 0);
    }
    double *out = malloc(sizeof(double) * (size_t)(tq * H * D + 1));
    double *lse = malloc(sizeof(double) * (size_t)(tq * H + 1));
    for (int64_t i = 0; i < tq * H * D; ++i) out[i] = NAN;
    for (int64_t i = 0; i < tq * H; ++i) lse[i] = NAN;
    int rc = fa_oracle_attention_t(q, tq, H, D, k, v, rows / (page ? page : 1), page, Hk, cu_q, cu_k, batch, bt,
                                   width, 1.0 / sqrt((double)D), wl, wr, sel, out, lse, threads, dtype, al,
                                   use_alibi == 2 ? H : 0);
    if (rc != 0) {
        printf("MISMATCH %s: oracle returned %d\n", what, rc);
        ++bad;
    }
    for (int64_t t = 0; t < tq; ++t) {
        if (sel && !sel[t]) continue;
        for (int h = 0; h < H; ++h) {
            if (isnan(lse[(int64_t)h * tq + t])) { printf("MISMATCH %s: lse not written\n", what); ++bad; t = tq; break; }
            for (int d = 0; d < D; ++d)
                if (!isfinite(out[(t * H + h) * D + d])) { printf("MISMATCH %s: out\n", what); ++bad; t = tq; h = H; break; }
        }
    }
    free(cu_q); free(cu_k); free(q); free(k); free(v); free(bt); free(al); free(sel); free(out); free(lse);
}

int main(void) {
    const int lq1[] = {17, 64, 5}, lk1[] = {17, 64, 5};
    run_case("c1 shape", 3, lq1, lk1, 4, 2, 64, 0, -1, 0, 0, 0, 0, 1);
    const int lq2[] = {1, 1, 1, 1}, lk2[] = {50, 7, 128, 1};
    run_case("decode paged", 4, lq2, lk2, 8, 2, 32, 32, -1, 0, 0, 0, 0, 4);
    const int lq3[] = {12, 4, 0, 9}, lk3[] = {5, 0, 3, 9};
    run_case("Lq > Lk, empty", 4, lq3, lk3, 2, 1, 8, 32, -1, 0, 0, 0, 0, 3);
    run_case("int32 windows", 4, lq3, lk3, 2, 1, 8, 0, INT_MAX, INT_MAX, 0, 0, 0, 2);
    run_case("int32 left", 4, lq3, lk3, 2, 1, 8, 32, INT_MAX, 0, 1, 0, 0, 2);
    run_case("int32 right", 4, lq3, lk3, 2, 1, 8, 0, 3, INT_MAX - 1, 0, 0, 0, 2);
    const int lq4[] = {30, 8}, lk4[] = {40, 30};
    run_case("two-sided", 2, lq4, lk4, 4, 2, 13, 64, 4, 3, 0, 0, 1, 2);
    run_case("alibi per head f16", 2, lq4, lk4, 4, 4, 24, 0, -1, -1, 1, 1, 0, 2);
    run_case("alibi per seq", 2, lq4, lk4, 4, 1, 40, 32, 7, 0, 0, 2, 1, 5);
    const int lq5[] = {4, 4}, lk5[] = {300, 1100};
    run_case("mqa d512", 2, lq5, lk5, 16, 1, 512, 128, -1, 0, 0, 0, 0, 8);

    /* argument rejection */
    int32_t cu[] = {0, 5, 3};
    uint16_t x[64] = {0};
    double o[64], l[8];
    if (fa_oracle_attention_t(x, 5, 1, 4, x, x, 8, 0, 1, cu, cu, 2, NULL, 0, 1.0, -1, 0, NULL, o, l, 1, 0,
                              NULL, 0) != -1) { printf("MISMATCH decreasing offsets accepted\n"); ++bad; }
    int32_t cuq[] = {0, 1}, cuk[] = {0, 9};
    int32_t bt1[] = {7};
    if (fa_oracle_attention_t(x, 1, 1, 4, x, x, 2, 32, 1, cuq, cuk, 1, bt1, 1, 1.0, -1, 0, NULL, o, l, 1, 0,
                              NULL, 0) != -2) { printf("MISMATCH block id outside the pool accepted\n"); ++bad; }

    /* append: in-table positions written, out-of-table ones skipped (-2) */
    {
        const int Hk = 2, D = 16, P = 32, nb = 6, width = 3;
        uint16_t *kp = calloc((size_t)nb * P * Hk * D, 2), *vp = calloc((size_t)nb * P * Hk * D, 2);
        uint16_t kn[5 * 2 * 16], vn[5 * 2 * 16];
        fill(kn, 5 * Hk * D, 0);
        fill(vn, 5 * Hk * D, 0);
        int32_t cu_new[] = {0, 2, 5}, cu_kk[] = {0, 40, 140};
        int32_t bt[] = {3, 1, -1, 0, 9, 2};
        int rc = fa_oracle_kv_append(kn, vn, 5, Hk, D, cu_new, cu_kk, 2, bt, width, P, nb, kp, vp);
        if (rc != -2) { printf("MISMATCH append skip code %d\n", rc); ++bad; }
        free(kp); free(vp);
    }

    /* widening of every bit pattern of both types */
    uint16_t *all = malloc(65536 * 2);
    double *w = malloc(65536 * sizeof(double));
    for (int i = 0; i < 65536; ++i) all[i] = (uint16_t)i;
    fa_oracle_widen(all, 65536, 0, w);
    fa_oracle_widen(all, 65536, 1, w);
    free(all); free(w);

    printf("oracle driver: %d mismatches\n", bad);
    return bad ? 1 : 0;
}
