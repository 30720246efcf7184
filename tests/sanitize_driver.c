/*
 * Host-only driver that runs every entry point of the C oracle (oracle/oracle.c)
 * and of the input generator (synth/gen.c) on small shapes, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py).
 * It covers fp32 and bf16 inputs, ragged and empty rows, N above the row
 * length, subsets of (b, i) pairs, the Atop-N calibration / stale step and the
 * SparQ-style scorer; any out-of-bounds access, use after free, leak or
 * undefined operation aborts the run. It also checks a few invariants of the
 * results (softmax weights summing to 1, sorted -1-padded index lists) so a
 * silently wrong build fails too.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* synth/gen.c */
void synth_draws(uint64_t seed, uint64_t stream, uint64_t offset, int64_t count, uint64_t* out);
void synth_fill_normal(uint64_t seed, uint64_t stream, int64_t rows, int d,
                       const double* row_scale, int dtype, void* out);
int synth_heavy_rows(uint64_t seed, uint64_t stream, int B, int h, int64_t S_max,
                     const int32_t* lens, const int32_t* count, double factor, double* row_scale);
void synth_lengths(uint64_t seed, uint64_t stream, int B, int32_t lo, int32_t hi, int32_t* lens);

/* oracle/oracle.c */
int oracle_topn_attn(const void* q, const void* k, const void* v, const int32_t* lens, int B,
                     int h_q, int h_k, int h_v, int d, int64_t S_max, int dtype, int N,
                     const int64_t* pairs, int64_t npairs, double* out, int32_t* idx,
                     double* sel, double* tN, double* psum, int nthreads);
int oracle_dense_attn(const void* q, const void* k, const void* v, const int32_t* lens, int B,
                      int h_q, int h_k, int h_v, int d, int64_t S_max, int dtype,
                      const int64_t* pairs, int64_t npairs, double* out, int nthreads);
int oracle_logits(const void* q, const void* k, const int32_t* lens, int B, int h_q, int h_k,
                  int d, int64_t S_max, int dtype, const int64_t* pairs, int64_t npairs,
                  double* scores, int nthreads);
int oracle_attend_given(const void* q, const void* k, const void* v, const int32_t* lens, int B,
                        int h_q, int h_k, int h_v, int d, int64_t S_max, int dtype, int N,
                        const int64_t* pairs, int64_t npairs, const int32_t* idx, double* out,
                        double* psum, int nthreads);
int oracle_atopn_calibrate(const void* q, const void* k, const int32_t* lens, int B, int h_q,
                           int h_k, int d, int64_t S_max, int dtype, int N,
                           const int64_t* pairs, int64_t npairs, double* tau, double* lse,
                           int nthreads);
int oracle_atopn_attn(const void* q, const void* k, const void* v, const int32_t* lens, int B,
                      int h_q, int h_k, int h_v, int d, int64_t S_max, int dtype, int N,
                      const double* tau, const int64_t* pairs, int64_t npairs, double* out,
                      int32_t* idx, double* sel, int64_t* above, double* theta, double* psum,
                      int nthreads);
int oracle_sparq_attn(const void* q, const void* k, const void* v, const int32_t* lens, int B,
                      int h_q, int h_k, int h_v, int d, int64_t S_max, int dtype, int N, int r,
                      int l, const double* vmean, const int64_t* pairs, int64_t npairs,
                      double* out, int32_t* idx, double* alpha, double* tau, double* zthr,
                      int32_t* dims, double* zhat, int nthreads);

static int failures = 0;
#define EXPECT(c, ...)                                        \
    do {                                                      \
        if (!(c)) {                                           \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                     \
            fprintf(stderr, "\n");                            \
            ++failures;                                       \
        }                                                     \
    } while (0)

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

/* index list of one pair: first n ascending and in [0, L), the rest -1 */
static void check_list(const int32_t* idx, int N, int64_t n, int64_t L, const char* what) {
    for (int r = 0; r < N; ++r) {
        if (r < n) {
            EXPECT(idx[r] >= 0 && idx[r] < L, "%s: slot %d = %d outside [0, %lld)", what, r,
                   idx[r], (long long)L);
            if (r > 0) EXPECT(idx[r] > idx[r - 1], "%s: slot %d not ascending", what, r);
        } else {
            EXPECT(idx[r] == -1, "%s: slot %d = %d past the kept count", what, r, idx[r]);
        }
    }
}

static void run_shape(int B, int h_q, int h_k, int h_v, int d, int64_t S, int N, int dtype,
                      const int32_t* lens_in, uint64_t seed) {
    const size_t es = dtype ? 2 : 4;
    const int64_t rows = (int64_t)B * h_q;
    int32_t* lens = (int32_t*)xmalloc(sizeof(int32_t) * B);
    if (lens_in) memcpy(lens, lens_in, sizeof(int32_t) * B);
    else synth_lengths(seed, 4, B, (int32_t)(S / 2), (int32_t)S, lens);
    double* scale = (double*)xmalloc(sizeof(double) * (size_t)(B * h_k * S));
    for (int64_t j = 0; j < B * h_k * S; ++j) scale[j] = 1.0;
    int32_t* cnt = (int32_t*)xmalloc(sizeof(int32_t) * B);
    for (int b = 0; b < B; ++b) cnt[b] = lens[b] / 8;
    EXPECT(synth_heavy_rows(seed, 3, B, h_k, S, lens, cnt, 3.0, scale) == 0, "heavy rows");
    void* q = xmalloc(es * (size_t)(rows * d));
    void* k = xmalloc(es * (size_t)(B * h_k * S * d));
    void* v = xmalloc(es * (size_t)(B * h_v * S * d));
    synth_fill_normal(seed, 0, rows, d, NULL, dtype, q);
    synth_fill_normal(seed, 1, (int64_t)B * h_k * S, d, scale, dtype, k);
    synth_fill_normal(seed, 2, (int64_t)B * h_v * S, d, NULL, dtype, v);
    uint64_t draws[16];
    synth_draws(seed, 5, 7, 16, draws);

    double* out = (double*)xmalloc(sizeof(double) * (size_t)(rows * d));
    int32_t* idx = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)(rows * 2 * N));
    double* sel = (double*)xmalloc(sizeof(double) * (size_t)(rows * 2 * N));
    double* tN = (double*)xmalloc(sizeof(double) * (size_t)rows);
    double* psum = (double*)xmalloc(sizeof(double) * (size_t)rows);
    EXPECT(oracle_topn_attn(q, k, v, lens, B, h_q, h_k, h_v, d, S, dtype, N, NULL, 0, out, idx,
                            sel, tN, psum, 2) > 0, "topn");
    for (int64_t j = 0; j < rows; ++j) {
        const int64_t L = lens[j / h_q], n = L < N ? L : N;
        check_list(idx + j * N, N, n, L, "topn");
        if (n > 0) EXPECT(fabs(psum[j] - 1.0) < 1e-12, "topn psum %.17g", psum[j]);
    }
    /* the same rows again through an explicit pair list, and Eq. 7 on the kept sets */
    int64_t* pairs = (int64_t*)xmalloc(sizeof(int64_t) * 2 * (size_t)rows);
    for (int64_t j = 0; j < rows; ++j) {
        pairs[2 * j] = j / h_q;
        pairs[2 * j + 1] = j % h_q;
    }
    double* out2 = (double*)xmalloc(sizeof(double) * (size_t)(rows * d));
    double* ps2 = (double*)xmalloc(sizeof(double) * (size_t)rows);
    EXPECT(oracle_attend_given(q, k, v, lens, B, h_q, h_k, h_v, d, S, dtype, N, pairs, rows, idx,
                               out2, ps2, 2) > 0, "attend_given");
    for (int64_t j = 0; j < rows * d; ++j)
        EXPECT(fabs(out2[j] - out[j]) < 1e-12, "attend_given differs at %lld", (long long)j);
    EXPECT(oracle_dense_attn(q, k, v, lens, B, h_q, h_k, h_v, d, S, dtype, pairs, rows, out2, 2) > 0,
           "dense");
    double* sc = (double*)xmalloc(sizeof(double) * (size_t)(rows * S));
    EXPECT(oracle_logits(q, k, lens, B, h_q, h_k, d, S, dtype, NULL, 0, sc, 2) > 0, "logits");
    double* tau = (double*)xmalloc(sizeof(double) * (size_t)rows);
    double* lse = (double*)xmalloc(sizeof(double) * (size_t)rows);
    EXPECT(oracle_atopn_calibrate(q, k, lens, B, h_q, h_k, d, S, dtype, N, NULL, 0, tau, lse, 2) > 0,
           "calibrate");
    int64_t* above = (int64_t*)xmalloc(sizeof(int64_t) * (size_t)rows);
    double* theta = (double*)xmalloc(sizeof(double) * (size_t)rows);
    EXPECT(oracle_atopn_attn(q, k, v, lens, B, h_q, h_k, h_v, d, S, dtype, N, tau, NULL, 0, out,
                             idx, sel, above, theta, psum, 2) > 0, "atopn");
    for (int64_t j = 0; j < rows; ++j) {
        const int64_t L = lens[j / h_q];
        const int64_t n = above[j] < 2 * N ? above[j] : 2 * N;
        check_list(idx + j * 2 * N, 2 * N, n, L, "atopn");
    }
    const int r = d / 4, l = N / 4;
    double* vmean = (double*)xmalloc(sizeof(double) * (size_t)(B * h_v * d));
    for (int64_t j = 0; j < B * h_v * d; ++j) vmean[j] = 0.01 * (double)(j % 7);
    double* alpha = (double*)xmalloc(sizeof(double) * (size_t)rows);
    double* zthr = (double*)xmalloc(sizeof(double) * (size_t)rows);
    int32_t* dims = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)(rows * r));
    EXPECT(oracle_sparq_attn(q, k, v, lens, B, h_q, h_k, h_v, d, S, dtype, N, r, l, vmean, NULL, 0,
                             out, idx, alpha, tau, zthr, dims, sc, 2) > 0, "sparq");
    for (int64_t j = 0; j < rows; ++j) {
        const int64_t L = lens[j / h_q];
        const int64_t n = L < N ? L : N;
        check_list(idx + j * N, N, n, L, "sparq");
        EXPECT(alpha[j] >= 0.0 && alpha[j] <= 1.0 + 1e-12, "sparq alpha %.17g", alpha[j]);
    }
    /* bad arguments are refused, not read */
    EXPECT(oracle_topn_attn(q, k, v, lens, B, h_q, h_k, h_v, d, S, dtype, 0, NULL, 0, out, idx,
                            sel, tN, psum, 1) == -1, "N = 0 refused");
    free(vmean); free(alpha); free(zthr); free(dims);
    free(above); free(theta); free(tau); free(lse); free(sc);
    free(out2); free(ps2); free(pairs);
    free(out); free(idx); free(sel); free(tN); free(psum);
    free(q); free(k); free(v); free(scale); free(cnt); free(lens);
}

int main(void) {
    const int32_t edge[4] = {1, 0, 37, 64};
    run_shape(4, 4, 1, 2, 64, 64, 16, 0, edge, 11);        /* fp32; L = 0, 1, < N, = S */
    run_shape(2, 8, 2, 4, 128, 300, 40, 1, NULL, 12);      /* bf16, ragged */
    run_shape(1, 6, 2, 3, 64, 129, 200, 1, NULL, 13);      /* N > L: every position kept */
    run_shape(2, 12, 1, 2, 128, 520, 64, 1, NULL, 14);     /* the Qwen head layout */
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("sanitized oracle and generator: all entry points ran clean\n");
    return 0;
}
