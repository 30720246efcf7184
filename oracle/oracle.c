/*
 * CPU oracle for single-token decode attention under Sparse Asymmetric
 * Group-Query Attention (SAGA) with top-N selection.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code with the HIP
 * path: it is a plain, slow, fp64 restatement of the definitions below.
 *
 * Source: "More Value per Key: Asymmetric Sparse Attention for Faster LLM
 * Decoding" (arXiv 2610.04753):
 *   - scaled dot-product attention, §2.1 Eqs. 2-4;
 *   - decode with a KV cache (one query row), §2.2 Eq. 5;
 *   - top-N attention: keep the N largest logits of the row, mask the rest
 *     before the softmax, §2.5 Eq. 6;
 *   - attention over the gathered entries, softmax(A[i]) V[i], §3.1 Eq. 7;
 *   - SAGA: separate key and value head counts h_k <= h_v, §3.2;
 *   - query head blocks: contiguous blocks of g = h_q / h_kv query heads share
 *     one key (value) head, App. B Eq. 29 -- so query head i uses key head
 *     i / (h_q / h_k) and value head i / (h_q / h_v).
 *
 * Readings where the pages leave a step open (all exact, no approximation):
 *   - the threshold is fresh at every step, so exactly N_eff = min(N, L)
 *     entries are kept (the pages' threshold reuse over n steps is a
 *     different, history-dependent selector);
 *   - ranking is on the scaled logits; equal logits are ordered by lower
 *     position first; -0.0 equals +0.0 (fp64 comparison);
 *   - N > L keeps all L entries; unused output slots hold index -1 and
 *     score -inf;
 *   - positions t >= L (= seq_lens[b]) are never read.
 *
 * Precision: inputs are the stored fp32 / bf16 values decoded exactly; all
 * arithmetic is fp64 with the host libm exp().
 *
 * Atop-N with a stale threshold (§3.1, App. C.1), the two functions at the
 * end of this file. Readings where the pages leave a step open:
 *   - calibration keeps tau = the N_eff-th largest probability of the exact
 *     softmax over all L positions (probability space, per (b, i));
 *   - a later step keeps the positions whose probability reaches tau,
 *     p_t = exp(z_t - LSE(z)) >= tau (compared here in probability space,
 *     computed exactly as tau was); in logit space that is
 *     z_t >= log(tau) + LSE(z), the pages' approximate max logit only
 *     stabilising the sum; ">=" (not ">") so that the calibration step's own
 *     inputs give back exactly its top-N set;
 *   - at most 2N positions are kept, the first 2N in ascending position (the
 *     pages drop the excess in the order of an atomic counter);
 *   - no position reaching tau: the output is 0 (a softmax over an empty set
 *     is undefined).
 *
 * SparQ-style approximate scoring in front of the same selector ("SparQ
 * Attention: Bandwidth-Efficient LLM Inference", Steps 1-3 with the GQA
 * modifications), the last function of this file; its readings are listed
 * in its own comment.
 *
 * Parity pins live in tests/test_oracle_pins.py, tests/test_oracle_atopn_pins.py
 * and tests/test_oracle_sparq_pins.py (closed forms, library
 * reductions, brute force); every function below is pinned there.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

typedef struct {
    const void* q;         /* [B][h_q][d] */
    const void* k;         /* [B][h_k][S_max][d] */
    const void* v;         /* [B][h_v][S_max][d] */
    const int32_t* lens;   /* [B] */
    int B, h_q, h_k, h_v, d;
    int64_t S_max;
    int dtype;
} problem_t;

/* Decode one stored element to fp64 exactly. */
static double elem(const void* base, int dtype, int64_t i) {
    if (dtype == ORACLE_F32) return (double)((const float*)base)[i];
    uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int64_t seq_len(const problem_t* P, int b) {
    int64_t L = P->lens[b];
    if (L < 0) L = 0;
    if (L > P->S_max) L = P->S_max;
    return L;
}

/* Head mapping of App. B (contiguous query-head blocks). */
static int key_head(const problem_t* P, int i) { return i / (P->h_q / P->h_k); }
static int value_head(const problem_t* P, int i) { return i / (P->h_q / P->h_v); }

/* Scaled logit of Eq. 2 for query (b, i) and cached position t. */
static double logit(const problem_t* P, int b, int i, int64_t t) {
    int d = P->d;
    int kh = key_head(P, i);
    int64_t qo = ((int64_t)b * P->h_q + i) * d;
    int64_t ko = (((int64_t)b * P->h_k + kh) * P->S_max + t) * d;
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += elem(P->q, P->dtype, qo + c) * elem(P->k, P->dtype, ko + c);
    return acc / sqrt((double)d);
}

typedef struct { double s; int64_t t; } scored_t;

/* Order of Eq. 6 with the tie rule: larger logit first, then lower position. */
static int by_logit_desc(const void* a, const void* b) {
    const scored_t* x = (const scored_t*)a;
    const scored_t* y = (const scored_t*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->t > y->t) - (x->t < y->t);
}

static int by_pos(const void* a, const void* b) {
    const scored_t* x = (const scored_t*)a;
    const scored_t* y = (const scored_t*)b;
    return (x->t > y->t) - (x->t < y->t);
}

/*
 * Steps 4-5 (Eq. 7): softmax over the given entries (sorted by position),
 * then the weighted sum of their value rows, summed in ascending position.
 * Writes out[d] and returns sum(p) through psum.
 */
static void attend(const problem_t* P, int b, int i, const scored_t* sel, int64_t n,
                   double* out, double* psum) {
    int d = P->d;
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    *psum = 0.0;
    if (n <= 0) return;
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) if (sel[j].s > m) m = sel[j].s;
    double z = 0.0;
    for (int64_t j = 0; j < n; ++j) z += exp(sel[j].s - m);
    int vh = value_head(P, i);
    for (int64_t j = 0; j < n; ++j) {
        double p = exp(sel[j].s - m) / z;
        *psum += p;
        int64_t vo = (((int64_t)b * P->h_v + vh) * P->S_max + sel[j].t) * d;
        for (int c = 0; c < d; ++c) out[c] += p * elem(P->v, P->dtype, vo + c);
    }
}

static int check(const problem_t* P) {
    if (P->B < 1 || P->h_q < 1 || P->h_k < 1 || P->h_v < 1 || P->d < 1 || P->S_max < 1) return -1;
    if (P->h_q % P->h_k || P->h_q % P->h_v) return -1;
    if (P->dtype != ORACLE_F32 && P->dtype != ORACLE_BF16) return -1;
    return 0;
}

static void pair_of(const problem_t* P, const int64_t* pairs, int64_t j, int* b, int* i) {
    if (pairs) { *b = (int)pairs[2 * j]; *i = (int)pairs[2 * j + 1]; }
    else { *b = (int)(j / P->h_q); *i = (int)(j % P->h_q); }
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * Top-N decode attention (Eqs. 2, 6, 7) for `npairs` (b, i) pairs (pairs ==
 * NULL: all B*h_q pairs in b-major order). Per pair:
 *   out[d]        attention output
 *   idx[N]        kept positions in ascending order, -1 padded
 *   sel[N]        their logits, -inf padded
 *   tN            the N_eff-th largest logit (NaN if L = 0)
 *   psum          sum of the softmax weights
 * Returns the thread count used, or -1 on bad arguments.
 */
int oracle_topn_attn(const void* q, const void* k, const void* v, const int32_t* lens,
                     int B, int h_q, int h_k, int h_v, int d, int64_t S_max, int dtype, int N,
                     const int64_t* pairs, int64_t npairs,
                     double* out, int32_t* idx, double* sel, double* tN, double* psum,
                     int nthreads) {
    problem_t P = {q, k, v, lens, B, h_q, h_k, h_v, d, S_max, dtype};
    if (check(&P) || N < 1) return -1;
    if (!pairs) npairs = (int64_t)B * h_q;
    int used = set_threads(nthreads);
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t j = 0; j < npairs; ++j) {
        int b, i;
        pair_of(&P, pairs, j, &b, &i);
        if (b < 0 || b >= B || i < 0 || i >= h_q) { bad = 1; continue; }
        int64_t L = seq_len(&P, b);
        int64_t n = L < N ? L : N;
        scored_t* all = (scored_t*)malloc(sizeof(scored_t) * (size_t)(L > 0 ? L : 1));
        if (!all) { bad = 1; continue; }
        for (int64_t t = 0; t < L; ++t) { all[t].s = logit(&P, b, i, t); all[t].t = t; }
        qsort(all, (size_t)L, sizeof(scored_t), by_logit_desc);
        tN[j] = n > 0 ? all[n - 1].s : NAN;
        qsort(all, (size_t)n, sizeof(scored_t), by_pos);
        for (int64_t r = 0; r < N; ++r) {
            idx[j * N + r] = r < n ? (int32_t)all[r].t : -1;
            sel[j * N + r] = r < n ? all[r].s : -INFINITY;
        }
        attend(&P, b, i, all, n, out + j * d, psum + j);
        free(all);
    }
    return bad ? -1 : used;
}

/*
 * Full decode attention (Eqs. 2-5) over all L positions: no selection step.
 * Same pair convention as oracle_topn_attn. Returns threads used or -1.
 */
int oracle_dense_attn(const void* q, const void* k, const void* v, const int32_t* lens,
                      int B, int h_q, int h_k, int h_v, int d, int64_t S_max, int dtype,
                      const int64_t* pairs, int64_t npairs, double* out, int nthreads) {
    problem_t P = {q, k, v, lens, B, h_q, h_k, h_v, d, S_max, dtype};
    if (check(&P)) return -1;
    if (!pairs) npairs = (int64_t)B * h_q;
    int used = set_threads(nthreads);
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t j = 0; j < npairs; ++j) {
        int b, i;
        pair_of(&P, pairs, j, &b, &i);
        if (b < 0 || b >= B || i < 0 || i >= h_q) { bad = 1; continue; }
        int64_t L = seq_len(&P, b);
        scored_t* all = (scored_t*)malloc(sizeof(scored_t) * (size_t)(L > 0 ? L : 1));
        if (!all) { bad = 1; continue; }
        for (int64_t t = 0; t < L; ++t) { all[t].s = logit(&P, b, i, t); all[t].t = t; }
        double ps;
        attend(&P, b, i, all, L, out + j * d, &ps);
        free(all);
    }
    return bad ? -1 : used;
}

/*
 * Scaled logits (Eq. 2) for each pair at every position: scores[npairs][S_max],
 * NaN at t >= L. Returns threads used or -1.
 */
int oracle_logits(const void* q, const void* k, const int32_t* lens,
                  int B, int h_q, int h_k, int d, int64_t S_max, int dtype,
                  const int64_t* pairs, int64_t npairs, double* scores, int nthreads) {
    problem_t P = {q, k, NULL, lens, B, h_q, h_k, h_k, d, S_max, dtype};
    if (check(&P)) return -1;
    if (!pairs) npairs = (int64_t)B * h_q;
    int used = set_threads(nthreads);
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t j = 0; j < npairs; ++j) {
        int b, i;
        pair_of(&P, pairs, j, &b, &i);
        if (b < 0 || b >= B || i < 0 || i >= h_q) { bad = 1; continue; }
        int64_t L = seq_len(&P, b);
        for (int64_t t = 0; t < S_max; ++t)
            scores[j * S_max + t] = t < L ? logit(&P, b, i, t) : NAN;
    }
    return bad ? -1 : used;
}

/*
 * Eq. 7 on a caller-supplied index set: idx[npairs][N] (entries < 0 are
 * ignored; entries must be distinct positions < L). Logits are recomputed
 * here. Returns threads used, or -1 on bad arguments / out-of-range indices.
 */
int oracle_attend_given(const void* q, const void* k, const void* v, const int32_t* lens,
                        int B, int h_q, int h_k, int h_v, int d, int64_t S_max, int dtype,
                        int N, const int64_t* pairs, int64_t npairs, const int32_t* idx,
                        double* out, double* psum, int nthreads) {
    problem_t P = {q, k, v, lens, B, h_q, h_k, h_v, d, S_max, dtype};
    if (check(&P) || N < 1) return -1;
    if (!pairs) npairs = (int64_t)B * h_q;
    int used = set_threads(nthreads);
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t j = 0; j < npairs; ++j) {
        int b, i;
        pair_of(&P, pairs, j, &b, &i);
        if (b < 0 || b >= B || i < 0 || i >= h_q) { bad = 1; continue; }
        int64_t L = seq_len(&P, b);
        scored_t* sel = (scored_t*)malloc(sizeof(scored_t) * (size_t)N);
        if (!sel) { bad = 1; continue; }
        int64_t n = 0;
        for (int r = 0; r < N; ++r) {
            int64_t t = idx[j * N + r];
            if (t < 0) continue;
            if (t >= L) { bad = 1; continue; }
            sel[n].t = t;
            sel[n].s = logit(&P, b, i, t);
            ++n;
        }
        qsort(sel, (size_t)n, sizeof(scored_t), by_pos);
        for (int64_t r = 1; r < n; ++r) if (sel[r].t == sel[r - 1].t) bad = 1;
        attend(&P, b, i, sel, n, out + j * d, psum + j);
        free(sel);
    }
    return bad ? -1 : used;
}

/* log sum_t exp(z_t) over the row, stabilised by its largest logit. */
static double log_sum_exp(const scored_t* all, int64_t L) {
    double m = -INFINITY;
    for (int64_t t = 0; t < L; ++t) if (all[t].s > m) m = all[t].s;
    double z = 0.0;
    for (int64_t t = 0; t < L; ++t) z += exp(all[t].s - m);
    return m + log(z);
}

/*
 * Atop-N calibration step (App. C.1): the exact softmax probabilities of the
 * row and the N_eff-th largest of them, tau[j] (NaN if L = 0); lse[j] is the
 * row's log-sum-exp of the logits. Same pair convention as oracle_topn_attn.
 * Returns threads used or -1.
 */
int oracle_atopn_calibrate(const void* q, const void* k, const int32_t* lens,
                           int B, int h_q, int h_k, int d, int64_t S_max, int dtype, int N,
                           const int64_t* pairs, int64_t npairs, double* tau, double* lse,
                           int nthreads) {
    problem_t P = {q, k, NULL, lens, B, h_q, h_k, h_k, d, S_max, dtype};
    if (check(&P) || N < 1) return -1;
    if (!pairs) npairs = (int64_t)B * h_q;
    int used = set_threads(nthreads);
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t j = 0; j < npairs; ++j) {
        int b, i;
        pair_of(&P, pairs, j, &b, &i);
        if (b < 0 || b >= B || i < 0 || i >= h_q) { bad = 1; continue; }
        int64_t L = seq_len(&P, b);
        if (L <= 0) { tau[j] = NAN; lse[j] = NAN; continue; }
        scored_t* all = (scored_t*)malloc(sizeof(scored_t) * (size_t)L);
        if (!all) { bad = 1; continue; }
        for (int64_t t = 0; t < L; ++t) { all[t].s = logit(&P, b, i, t); all[t].t = t; }
        const double z = log_sum_exp(all, L);
        qsort(all, (size_t)L, sizeof(scored_t), by_logit_desc);
        const int64_t n = L < N ? L : N;
        tau[j] = exp(all[n - 1].s - z);
        lse[j] = z;
        free(all);
    }
    return bad ? -1 : used;
}

/*
 * Atop-N step with the stale thresholds tau[npairs] (§3.1, App. C.1): keep
 * the positions t < L with exp(z_t - LSE(z)) >= tau, in ascending position,
 * at most the first 2N of them; then Eq. 7 over the kept entries (out = 0
 * when none is kept). Per pair:
 *   out[d]; idx[2N] kept positions (-1 pad); sel[2N] their logits (-inf pad);
 *   above[j] = count of positions reaching tau (before the 2N cap);
 *   theta[j] = log(tau) + LSE(z), the same threshold in logit space;
 *   psum[j] = sum of the softmax weights (0 when none is kept).
 * Returns threads used or -1.
 */
int oracle_atopn_attn(const void* q, const void* k, const void* v, const int32_t* lens,
                      int B, int h_q, int h_k, int h_v, int d, int64_t S_max, int dtype, int N,
                      const double* tau, const int64_t* pairs, int64_t npairs,
                      double* out, int32_t* idx, double* sel, int64_t* above, double* theta,
                      double* psum, int nthreads) {
    problem_t P = {q, k, v, lens, B, h_q, h_k, h_v, d, S_max, dtype};
    if (check(&P) || N < 1) return -1;
    if (!pairs) npairs = (int64_t)B * h_q;
    const int64_t cap = 2 * (int64_t)N;
    int used = set_threads(nthreads);
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t j = 0; j < npairs; ++j) {
        int b, i;
        pair_of(&P, pairs, j, &b, &i);
        if (b < 0 || b >= B || i < 0 || i >= h_q) { bad = 1; continue; }
        int64_t L = seq_len(&P, b);
        scored_t* all = (scored_t*)malloc(sizeof(scored_t) * (size_t)(L > 0 ? L : 1));
        if (!all) { bad = 1; continue; }
        for (int64_t t = 0; t < L; ++t) { all[t].s = logit(&P, b, i, t); all[t].t = t; }
        const double z = L > 0 ? log_sum_exp(all, L) : NAN;
        theta[j] = log(tau[j]) + z;
        int64_t n = 0, cnt = 0;
        for (int64_t t = 0; t < L; ++t) {       /* ascending position */
            if (!(exp(all[t].s - z) >= tau[j])) continue;
            ++cnt;
            if (n < cap) all[n++] = all[t];     /* n <= t: in-place compaction */
        }
        above[j] = cnt;
        for (int64_t r = 0; r < cap; ++r) {
            idx[j * cap + r] = r < n ? (int32_t)all[r].t : -1;
            sel[j * cap + r] = r < n ? all[r].s : -INFINITY;
        }
        attend(&P, b, i, all, n, out + j * d, psum + j);
        free(all);
    }
    return bad ? -1 : used;
}

/*
 * SparQ-style approximate scoring feeding the top-N selector ("SparQ
 * Attention: Bandwidth-Efficient LLM Inference", Steps 1-3 with the GQA
 * modifications), on the SAGA head layout. Per pair (b, i), key head kh:
 *   Step 1  u[c] = sum over the g_k query heads of the key head of |q[c]|;
 *           dims = the r largest u[c] (equal values: lower c first);
 *           tau = sqrt(d * sum_{c in dims} |q_i[c]| / sum_c |q_i[c]|);
 *           zhat_t = sum_{c in dims} q_i[c] K[t][c] / tau (zhat = 0 when
 *           the query has no mass on dims);
 *           shat = softmax(zhat) over all L positions.
 *   Step 2  the last l_eff = min(l, L) positions are always kept (local
 *           window); of the first L' = L - l_eff positions the N - l with the
 *           largest zhat are kept (equal values: lower position first).
 *           Then the exact Eq. 7 attention (logits q.K / sqrt(d)) over the
 *           kept set gives y3.
 *   Step 3  alpha = sum of shat over the kept set; out = alpha y3 +
 *           (1 - alpha) vmean[b][vh] when vmean is given, else out = y3.
 * Requires 0 <= l <= N and 1 <= r <= d. L = 0 keeps nothing: out = 0,
 * alpha = 0. Per pair outputs: out[d], idx[N] (ascending, -1 pad),
 * alpha, tau (0 when zhat = 0), zthr = the smallest kept zhat of the scored
 * (non-local) part (NaN if none), dims[r] (ascending), and, when zhat is not
 * NULL, zhat[S_max] (NaN past L). vmean is [B][h_v][d] (fp64) or NULL.
 * Returns threads used or -1.
 */
int oracle_sparq_attn(const void* q, const void* k, const void* v, const int32_t* lens,
                      int B, int h_q, int h_k, int h_v, int d, int64_t S_max, int dtype, int N,
                      int r, int l, const double* vmean, const int64_t* pairs, int64_t npairs,
                      double* out, int32_t* idx, double* alpha, double* tau, double* zthr,
                      int32_t* dims, double* zhat, int nthreads) {
    problem_t P = {q, k, v, lens, B, h_q, h_k, h_v, d, S_max, dtype};
    if (check(&P) || N < 1 || r < 1 || r > d || l < 0 || l > N) return -1;
    if (!pairs) npairs = (int64_t)B * h_q;
    const int g = h_q / h_k;
    int used = set_threads(nthreads);
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t j = 0; j < npairs; ++j) {
        int b, i;
        pair_of(&P, pairs, j, &b, &i);
        if (b < 0 || b >= B || i < 0 || i >= h_q) { bad = 1; continue; }
        const int kh = key_head(&P, i), vh = value_head(&P, i);
        const int64_t L = seq_len(&P, b);
        scored_t* all = (scored_t*)malloc(sizeof(scored_t) * (size_t)(L > 0 ? L : 1));
        scored_t* u = (scored_t*)malloc(sizeof(scored_t) * (size_t)d);
        char* in_dims = (char*)calloc((size_t)d, 1);
        if (!all || !u || !in_dims) { bad = 1; free(all); free(u); free(in_dims); continue; }
        /* Step 1: the group's query-magnitude ranking and the r kept dims */
        for (int c = 0; c < d; ++c) {
            double s = 0.0;
            for (int jj = kh * g; jj < (kh + 1) * g; ++jj)
                s += fabs(elem(q, dtype, ((int64_t)b * h_q + jj) * d + c));
            u[c].s = s;
            u[c].t = c;
        }
        qsort(u, (size_t)d, sizeof(scored_t), by_logit_desc);
        for (int e = 0; e < r; ++e) in_dims[u[e].t] = 1;
        for (int c = 0, e = 0; c < d; ++c) if (in_dims[c]) dims[j * r + e++] = c;
        const int64_t qo = ((int64_t)b * h_q + i) * d;
        double num = 0.0, den = 0.0;
        for (int c = 0; c < d; ++c) {
            const double a = fabs(elem(q, dtype, qo + c));
            den += a;
            if (in_dims[c]) num += a;
        }
        const double tq = num > 0.0 ? sqrt((double)d * num / den) : 0.0;
        tau[j] = tq;
        for (int64_t t = 0; t < L; ++t) {
            double acc = 0.0;
            if (num > 0.0) {
                const int64_t ko = (((int64_t)b * h_k + kh) * S_max + t) * d;
                for (int c = 0; c < d; ++c)
                    if (in_dims[c]) acc += elem(q, dtype, qo + c) * elem(k, dtype, ko + c);
                acc /= tq;
            }
            all[t].s = acc;
            all[t].t = t;
        }
        if (zhat)
            for (int64_t t = 0; t < S_max; ++t) zhat[j * S_max + t] = t < L ? all[t].s : NAN;
        const double lse = L > 0 ? log_sum_exp(all, L) : NAN;
        /* Step 2: local window, then the top N - l of the scored prefix */
        const int64_t lw = L < l ? L : l;
        const int64_t Lp = L - lw;
        const int64_t ns = (int64_t)(N - l) < Lp ? (int64_t)(N - l) : Lp;
        qsort(all, (size_t)Lp, sizeof(scored_t), by_logit_desc);
        zthr[j] = ns > 0 ? all[ns - 1].s : NAN;
        int64_t n = 0;
        for (int64_t e = 0; e < ns; ++e) all[n++] = all[e];
        for (int64_t t = Lp; t < L; ++t) {   /* zhat of the local positions, for alpha */
            double acc = 0.0;
            if (num > 0.0) {
                const int64_t ko = (((int64_t)b * h_k + kh) * S_max + t) * d;
                for (int c = 0; c < d; ++c)
                    if (in_dims[c]) acc += elem(q, dtype, qo + c) * elem(k, dtype, ko + c);
                acc /= tq;
            }
            all[n].s = acc;
            all[n].t = t;
            ++n;
        }
        qsort(all, (size_t)n, sizeof(scored_t), by_pos);
        double a = 0.0;
        for (int64_t e = 0; e < n; ++e) a += exp(all[e].s - lse);
        alpha[j] = a;
        for (int64_t e = 0; e < N; ++e) idx[j * N + e] = e < n ? (int32_t)all[e].t : -1;
        /* exact logits of the kept set, then Eq. 7 */
        for (int64_t e = 0; e < n; ++e) all[e].s = logit(&P, b, i, all[e].t);
        double psum;
        attend(&P, b, i, all, n, out + j * d, &psum);
        if (vmean && n > 0)   /* Step 3: mean value reallocation */
            for (int c = 0; c < d; ++c)
                out[j * d + c] = a * out[j * d + c] +
                                 (1.0 - a) * vmean[((int64_t)b * h_v + vh) * d + c];
        free(all);
        free(u);
        free(in_dims);
    }
    return bad ? -1 : used;
}
