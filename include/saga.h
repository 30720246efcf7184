/*
 * libsaga -- single-token decode attention under Sparse Asymmetric
 * Group-Query Attention (SAGA) with top-N selection, for AMD MI355X (gfx950).
 *
 * Method: "More Value per Key: Asymmetric Sparse Attention for Faster LLM
 * Decoding" (arXiv 2610.04753).
 *   - Query head i of h_q uses key head i / (h_q / h_k) and value head
 *     i / (h_q / h_v): contiguous query-head blocks (App. B, Eq. 29), with the
 *     key and value head counts decoupled, h_k <= h_v (§3.2).
 *   - Logits s_t = <q, K_t> / sqrt(d) over the cached positions (§2.1 Eq. 2,
 *     §2.2 Eq. 5).
 *   - Keep the N largest logits of the row (§2.5 Eq. 6); the threshold is the
 *     N-th largest value, found fresh at every call (§3.1), so exactly
 *     N_eff = min(N, L) positions are kept, equal logits going to the lower
 *     position.
 *   - Softmax over the kept logits only, then the weighted sum of the kept
 *     value rows (§3.1 Eq. 7; App. C.1).
 *
 * The decode call never writes the full logit matrix to memory: the K-scan
 * keeps each chunk's logits on chip and publishes only the keys at or above
 * a per-chunk cutoff; the selector proves the union's N-th key exact from the
 * cutoffs, or recomputes that head's logits when it cannot.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are device pointers owned by the caller. The
 *     library never allocates, frees or synchronises inside these calls; it
 *     enqueues kernels on `stream` and returns. It keeps no state between
 *     calls, so a call sequence can be captured in a HIP graph.
 *   - Layouts (row-major, innermost dimension last, elements of `dtype`):
 *       q        [B][h_q][d]
 *       k_cache  [B][h_k][S_max][d]
 *       v_cache  [B][h_v][S_max][d]
 *       seq_lens int32 [B]        cached length L_b of batch row b
 *       out      float32 [B][h_q][d]
 *     q, k_cache and v_cache must be 16-byte aligned.
 *   - Preconditions the host cannot check without a sync: 0 <= seq_lens[b]
 *     <= S_max (kernels clamp to this range for memory safety; L_b = 0 gives
 *     out = 0 and no kept index). Positions t >= L_b are never read.
 *   - Scalar arguments are checked on the host before any HIP call; a bad
 *     argument returns an error status and enqueues nothing.
 *   - Results are deterministic: the same inputs give bitwise-equal outputs.
 */
#ifndef SAGA_H
#define SAGA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SAGA_OK = 0,
    SAGA_ERR_INVALID_ARG = -1,  /* null pointer, non-positive size, head counts that do not
                                   divide h_q, h_k > h_v, unknown dtype, misaligned tensor */
    SAGA_ERR_UNSUPPORTED = -2,  /* head dimension d other than 64 or 128; h_q / h_v > 64 */
    SAGA_ERR_WORKSPACE = -3,    /* workspace null or smaller than the size functions return */
    SAGA_ERR_HIP = -4,          /* a kernel launch failed (hipGetLastError) */
    SAGA_ERR_TOO_LARGE = -5     /* saga_decode_attn_noalloc: the shape needs more scratch than
                                   saga_noalloc_scratch_bytes() */
} saga_status;

typedef enum {
    SAGA_F32 = 0,   /* IEEE float32 inputs */
    SAGA_BF16 = 1   /* bfloat16 inputs (stored as 16-bit patterns) */
} saga_dtype;

/*
 * Bytes of device workspace saga_decode_attn needs for these sizes. Host only,
 * no HIP call; returns 0 when the arguments are invalid. The workspace holds
 * the fp32 logit rows, the kept index/logit lists and the per-split partial
 * sums; it needs no initialisation and is fully rewritten by every call.
 */
size_t saga_workspace_size(int B, int h_q, int h_k, int h_v, int d, int N, int64_t S_max,
                           saga_dtype dtype);

/*
 * SAGA decode attention with top-N selection (§3.1 Eq. 7 on the §2.5 Eq. 6
 * set, §3.2 head counts).
 *   q, k_cache, v_cache, seq_lens, out : as in the layouts above.
 *   B, h_q, h_k, h_v, d : batch, query/key/value head counts, head dimension.
 *                         h_q % h_k == 0, h_q % h_v == 0, h_k <= h_v, d in {64, 128}.
 *   N        : positions kept per query head (N >= 1; N >= L_b keeps all L_b).
 *   stream   : HIP stream the kernels are enqueued on (0 = null stream).
 *   S_max    : capacity (stride) of the sequence axis of the caches.
 *   dtype    : element type of q, k_cache and v_cache.
 *   workspace, workspace_bytes : device scratch of at least saga_workspace_size(...) bytes,
 *              256-byte aligned, not used by anything else while the call runs.
 *   idx_out  : optional (may be NULL) int32 [B][h_q][N]: the kept positions of each query
 *              head in ascending order; slots past N_eff = min(N, L_b) hold -1.
 */
saga_status saga_decode_attn(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* seq_lens, float* out,
                             int B, int h_q, int h_k, int h_v, int d, int N, hipStream_t stream,
                             int64_t S_max, saga_dtype dtype,
                             void* workspace, size_t workspace_bytes, int32_t* idx_out);

/*
 * saga_decode_attn with phase timing for benchmarks: identical work and
 * results, and records events[i] on `stream` for i < n_events (0..4) at phase
 * boundary i: 0 the start and 1 the end of the K-scan kernel (with its
 * per-chunk candidate extraction; on the top-M path both are stamped by that
 * dispatch itself, so 1 - 0 is the kernel's run time, without launch
 * latency), 2 after top-N selection, 3 after the value gather (the end of the
 * call). On the top-M path selection and gather are one dispatch, so 2 and 3
 * are both recorded after it. The events are created by the caller (timing
 * enabled); a null event
 * or n_events outside 0..4 gives SAGA_ERR_INVALID_ARG.
 */
saga_status saga_decode_attn_timed(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* seq_lens, float* out,
                                   int B, int h_q, int h_k, int h_v, int d, int N,
                                   hipStream_t stream, int64_t S_max, saga_dtype dtype,
                                   void* workspace, size_t workspace_bytes, int32_t* idx_out,
                                   hipEvent_t* events, int n_events);

/*
 * saga_decode_attn for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments and results as saga_decode_attn, without the
 * workspace: the scratch memory is a static device array of the library,
 * saga_noalloc_scratch_bytes() bytes (128 MiB), one per GPU, held by every
 * GPU the library runs on until the process ends. The call allocates
 * nothing (no hipMalloc, no hipFree, no allocating library routine); on its
 * first use on a device it looks up the array's device address once. The
 * kernels run on the device of `stream` (the current device for the null
 * stream).
 *   - A shape whose saga_workspace_size exceeds saga_noalloc_scratch_bytes()
 *     returns SAGA_ERR_TOO_LARGE and enqueues nothing.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (the decode path rewrites everything it reads, so
 *     nothing needs clearing). Calls that overlap in time on one GPU (on
 *     different streams, or from different host threads without ordering)
 *     race on the array: the caller must serialise them.
 * Other errors as for saga_decode_attn.
 */
size_t saga_noalloc_scratch_bytes(void);

saga_status saga_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* seq_lens, float* out,
                                     int B, int h_q, int h_k, int h_v, int d, int N,
                                     hipStream_t stream, int64_t S_max, saga_dtype dtype,
                                     int32_t* idx_out);

/*
 * Bytes of device workspace saga_dense_attn needs (host only; 0 on invalid
 * arguments): one (max logit, weight sum, weighted value sum[d]) fp32 partial
 * per (b, query head) and chunk of cached positions; logits never go to
 * memory. The chunk is 1024, 512 or 256 positions (256 when h_q / h_k > 16):
 * among those leaving at most 128 chunks per row, the longest that gives at
 * least 256 (b, key head, chunk) items, else the shortest; so the size
 * depends on B and h_k as well as S_max.
 */
size_t saga_dense_workspace_size(int B, int h_q, int h_k, int h_v, int d, int64_t S_max,
                                 saga_dtype dtype);

/*
 * Full (dense) decode attention over all L_b cached positions (§2.1 Eqs. 2-4,
 * §2.2 Eq. 5): the GQA baseline when h_k == h_v and "SAGA full" when h_k < h_v
 * (§5.1). Arguments as for saga_decode_attn, without N and idx_out. Two
 * kernels on `stream`: the fused per-chunk pass (K rows, softmax, V rows)
 * and the log-sum-exp merge of the chunks. A row with L_b = 0 gets out = 0.
 */
saga_status saga_dense_attn(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, float* out,
                            int B, int h_q, int h_k, int h_v, int d, hipStream_t stream,
                            int64_t S_max, saga_dtype dtype,
                            void* workspace, size_t workspace_bytes);

/*
 * Atop-N, the pages' production selector with a stale threshold ("More Value
 * per Key" §3.1, App. C.1). A calibration step (every n steps in the pages,
 * n = 32) is the exact top-N step and also records, per (b, query head), tau
 * = the N_eff-th largest attention probability of the row. The steps in
 * between keep the positions whose probability reaches tau,
 * p_t = exp(z_t - LSE(z)) >= tau (compared as z_t >= log(tau) + LSE), at most
 * the first 2N in position order (the pages drop the excess in the order of
 * an atomic counter), and attend over them (Eq. 7); a row keeping none gets
 * out = 0. tau is state owned by the caller: device memory, fp32
 * [B][h_q], written by saga_atopn_calibrate and read by saga_atopn_attn.
 *
 * Both take the saga_decode_attn arguments plus tau, and need a workspace of
 * saga_atopn_workspace_size bytes (the decode workspace with 2N kept slots
 * per row). Supported for h_q / h_k <= 16 and S_max <= 512 Ki (the top-M
 * K-scan path); other shapes give SAGA_ERR_UNSUPPORTED. Errors as for
 * saga_decode_attn; a null tau is SAGA_ERR_INVALID_ARG.
 */
size_t saga_atopn_workspace_size(int B, int h_q, int h_k, int h_v, int d, int N,
                                 int64_t S_max, saga_dtype dtype);

/* Calibration: the exact top-N step (same out and idx_out [B][h_q][N] as
 * saga_decode_attn) plus tau. Rows with L_b = 0 get tau = NaN. */
saga_status saga_atopn_calibrate(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* seq_lens, float* out, int B, int h_q, int h_k,
                                 int h_v, int d, int N, hipStream_t stream, int64_t S_max,
                                 saga_dtype dtype, void* workspace, size_t workspace_bytes,
                                 float* tau, int32_t* idx_out);

/* Stale-threshold step. idx_out (nullable): [B][h_q][2N] kept positions in
 * ascending order, -1 padded. count_out (nullable): int32 [B][h_q], the
 * positions reaching the threshold before the 2N cap. tau = 0 keeps every
 * position (up to the cap); tau = NaN keeps none. */
saga_status saga_atopn_attn(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, float* out, int B, int h_q, int h_k,
                            int h_v, int d, int N, hipStream_t stream, int64_t S_max,
                            saga_dtype dtype, void* workspace, size_t workspace_bytes,
                            const float* tau, int32_t* idx_out, int32_t* count_out);

/*
 * SparQ-style approximate scoring in front of the top-N selector ("SparQ
 * Attention: Bandwidth-Efficient LLM Inference", Steps 1-3 with the GQA
 * modifications), on the SAGA head layout. Per (b, key head): the r dims
 * with the largest sum of |q| over the key head's g query heads (equal sums:
 * lower dim first). Per (b, query head i):
 *   - approximate logits over those dims only, zhat_t = <q_i, K_t>_dims / tau
 *     with tau = sqrt(d |q_i on dims|_1 / |q_i|_1) (all 0 when q_i has no
 *     mass on the dims), read from kt_cache;
 *   - the last min(local, L_b) positions are always kept; of the first
 *     L_b - min(local, L_b) positions the N - local with the largest zhat
 *     (equal values: lower position first);
 *   - exact attention (Eq. 7, logits q.K / sqrt(d) from k_cache) over the
 *     kept set gives y3;
 *   - alpha = sum over the kept set of softmax(zhat) (normalised over all L_b
 *     positions); out = alpha y3 + (1 - alpha) v_mean[b][vh] when v_mean is
 *     given, else out = y3. The pages keep the running value mean across
 *     steps and drop this mix for GQA models.
 *
 * Arguments as for saga_decode_attn, plus:
 *   kt_cache  device, the cache dtype, [B][h_k][d][S_max]: the same keys as
 *             k_cache, S-contiguous (the pages' second copy of K); only the r
 *             kept dims of each key head are read, rows t < L_b.
 *   r         1 <= r <= d.        local  0 <= local <= N.
 *   v_mean    nullable, device fp32 [B][h_v][d].
 *   idx_out   nullable, int32 [B][h_q][N]: the kept positions, ascending, -1 pad.
 *   alpha_out nullable, fp32 [B][h_q].
 *   dims_out  nullable, int32 [B][h_k][r]: the kept dims, ascending.
 * Two dispatches on `stream`: the scan of the kept columns into candidate
 * lists (each of its workgroups derives the dims and temperatures of the rows
 * it scans), then one dispatch per row for selection, exact rescoring and the
 * value gather. The workspace is
 * saga_sparq_workspace_size bytes (256-byte aligned). A row with L_b = 0
 * gets out = 0 and alpha = 0. SAGA_ERR_INVALID_ARG: a null required pointer,
 * r or local out of range, q / k_cache / kt_cache / v_cache not 16-byte
 * aligned, v_mean not 4-byte aligned, and the saga_decode_attn checks.
 * SAGA_ERR_UNSUPPORTED: h_q / h_k > 16, S_max > 512 Ki, N > 4096, or S_max
 * not a multiple of 16 bytes' worth of elements (8 bf16, 4 fp32).
 */
size_t saga_sparq_workspace_size(int B, int h_q, int h_k, int h_v, int d, int N, int r,
                                 int64_t S_max, saga_dtype dtype);

saga_status saga_sparq_attn(const void* q, const void* k_cache, const void* kt_cache,
                            const void* v_cache, const int32_t* seq_lens, float* out, int B,
                            int h_q, int h_k, int h_v, int d, int N, int r, int local,
                            const float* v_mean, hipStream_t stream, int64_t S_max,
                            saga_dtype dtype, void* workspace, size_t workspace_bytes,
                            int32_t* idx_out, float* alpha_out, int32_t* dims_out);

/*
 * GQA -> SAGA key-head merge ("More Value per Key", §4: Eqs. 13-17, Lemma 4.1,
 * Theorem 4.2; proof in App. A; strategies of App. B.1, Eq. 35). An offline
 * tool, not a decode call: it turns one attention module of a GQA teacher
 * with h_kt = 2 h_k^S key heads into h_k^S merged key heads.
 *
 * Inputs (device, bf16 only, 16-byte aligned, linear-layer storage
 * [out features][in features]):
 *   x   [L][D]         hidden states of L calibration tokens
 *   wq  [h_q * d][D]   query projection; query head j uses teacher key head
 *                      j / (h_q / h_kt) (contiguous blocks, App. B Eq. 29)
 *   wk  [h_kt * d][D]  teacher key projection
 * Outputs (device, caller-owned):
 *   merged_k  float32 [h_kt / 2][d][D]  merged key head i (storage layout)
 *             for matched pair i: M(a, b) = (W_a S_a + W_b S_b)(S_a + S_b)^+
 *             (Eq. 15) for SAGA_MERGE_LOGIT, the average (W_a + W_b) / 2 for
 *             the other two strategies
 *   sigma     int32 [h_kt]  the pairing: merged head i = teacher heads
 *             (sigma[2i], sigma[2i+1]), sigma[2i] < sigma[2i+1], pairs by
 *             increasing first head (App. B's sigma; feed it to
 *             saga_merge_permute)
 *   pair_w    nullable float64 [h_kt][h_kt]  weights the matching ran on:
 *             w(a, b) of Eq. 16 (LOGIT), ||X W_a - X W_b||_F^2 of Eq. 35
 *             (KEY), zeros (SEQUENTIAL); diagonal 0
 *   objective nullable float64 [1]  Eq. 14's objective for the returned
 *             pairing and merges (for LOGIT its minimum, Theorem 4.2)
 *   stats     nullable float32 [h_kt*d*d + (h_kt*d)^2]  S_r = sum over the
 *             query heads j of key head r of (X W_Q^j)^T (X W_Q^j) (Eq. 21),
 *             then H = (X W_K)^T (X W_K)
 * strategy: SAGA_MERGE_LOGIT = the §4 method (minimum-weight perfect matching
 * on Eq. 16, merges by Eq. 15); SAGA_MERGE_KEY = matching on Eq. 35 and
 * averaged pairs; SAGA_MERGE_SEQUENTIAL = pairs (0,1), (2,3), ... averaged.
 * The pseudo-inverse treats eigenvalues of S_a + S_b at or below
 * 2^-23 d lambda_max as zero (the resolution of fp32-accumulated statistics);
 * equal-weight matchings resolve to the lowest partner of the lowest head.
 * Arithmetic: X^T X on bf16 MFMA with fp32 accumulation, the statistics in
 * fp32, the per-pair algebra and the matching in fp64.
 * Limits: D and d multiples of 16, 16 <= d <= 128, h_kt even with
 * 2 <= h_kt <= 24, h_q a multiple of h_kt, L >= 1, D <= 46340; otherwise
 * SAGA_ERR_UNSUPPORTED (dtype other than SAGA_BF16 too). Null required
 * pointers, bad strategy or misaligned inputs: SAGA_ERR_INVALID_ARG; a
 * workspace below saga_key_merge_workspace_size: SAGA_ERR_WORKSPACE.
 * saga_key_merge_workspace_size returns 0 for unsupported shapes.
 */
typedef enum {
    SAGA_MERGE_LOGIT = 0,
    SAGA_MERGE_KEY = 1,
    SAGA_MERGE_SEQUENTIAL = 2
} saga_merge_strategy;

size_t saga_key_merge_workspace_size(int64_t L, int D, int h_q, int h_kt, int d);

saga_status saga_key_merge(const void* x, const void* wq, const void* wk, int64_t L, int D,
                           int h_q, int h_kt, int d, saga_merge_strategy strategy,
                           saga_dtype dtype, float* merged_k, int32_t* sigma, double* pair_w,
                           double* objective, float* stats, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * saga_key_merge with up to 5 events recorded on `stream` after the phases:
 * [0] X^T X partial products (one dispatch), [1] their reduction to X^T X,
 * [2] statistics S and H, [3] per-pair closed forms and weights, [4]
 * matching and merged projections. n_events outside 0..5 (or events null
 * with n_events > 0): SAGA_ERR_INVALID_ARG.
 */
saga_status saga_key_merge_timed(const void* x, const void* wq, const void* wk, int64_t L,
                                 int D, int h_q, int h_kt, int d,
                                 saga_merge_strategy strategy, saga_dtype dtype,
                                 float* merged_k, int32_t* sigma, double* pair_w,
                                 double* objective, float* stats, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream,
                                 hipEvent_t* events, int n_events);

/*
 * App. B's induced permutations (Eqs. 28-34) for a pairing sigma (device
 * int32 [h_kt], a permutation of 0 .. h_kt - 1, e.g. from saga_key_merge):
 *   wv_out head block i  = wv head block sigma[i]          ([h_kt*d][D])
 *   wq_out head block k  = wq head block pi_Q(k)           ([h_q*d][D])
 *   wo_out column block k = wo column block pi_Q(k)        ([D][h_q*d])
 * with pi_Q(k) = sigma[k / g] g + k % g, g = h_q / h_kt. A copy in `dtype`
 * (bf16 or float32); outputs must not overlap the inputs. D * esize and
 * d * esize must be multiples of 16 bytes (else SAGA_ERR_UNSUPPORTED);
 * pointers 16-byte aligned (else SAGA_ERR_INVALID_ARG). sigma is read on the
 * device and must hold a permutation (not checked).
 */
saga_status saga_merge_permute(const int32_t* sigma, const void* wq, const void* wv,
                               const void* wo, int D, int h_q, int h_kt, int d,
                               saga_dtype dtype, void* wq_out, void* wv_out, void* wo_out,
                               hipStream_t stream);

/*
 * The K-scan step alone (§2.1 Eq. 2 with the App. B key-head map): writes the
 * fp32 logits scores[B][h_q][S_max] for t < L_b; entries t >= L_b are left
 * untouched. Same argument rules as saga_decode_attn (h_v is not involved).
 */
saga_status saga_debug_scores(const void* q, const void* k_cache, const int32_t* seq_lens,
                              float* scores, int B, int h_q, int h_k, int d, hipStream_t stream,
                              int64_t S_max, saga_dtype dtype);

/*
 * Diagnostic for tests: after a saga_decode_attn call on `stream` with the same
 * sizes and workspace, copies to host_flags[B*h_q] (host memory), per query
 * head: 0 when its kept set was settled from the chunk candidate lists, 2 when
 * some chunks' lists could not prove the top-N exact and those chunks' logits
 * were recomputed, 1 when all of its logits were recomputed (too many such
 * chunks, more than half the row). Synchronises `stream`. Heads recompute
 * only when their largest logits crowd into a few chunks (attention sinks, a
 * recency window); the result is exact either way.
 */
saga_status saga_debug_fallback_rows(const void* workspace, size_t workspace_bytes, int B,
                                     int h_q, int h_k, int h_v, int d, int N, int64_t S_max,
                                     saga_dtype dtype, int32_t* host_flags, hipStream_t stream);

/*
 * Bandwidth ceilings of the decode step's two memory access patterns, for
 * benchmarks (they compute nothing of the method):
 *   saga_debug_stream_read reads every byte of the device buffer `buf`
 *   (bytes > 0, a multiple of 16, buf 16-byte aligned) once, sequentially,
 *   as the K-scan reads the key cache; sink is a device uint32 that is never
 *   written for real data.
 *   saga_debug_gather_rows reads the value rows listed per (b, query head)
 *   in idx int32 [B][h_q][N] (positions in [0, S_max); negative entries are
 *   skipped) from v_cache [B][h_v][S_max][d], with the
 *   decode path's gather loop and workgroup placement, and writes their mean
 *   to out fp32 [B][h_q][d] (0 for an empty list): the value gather without
 *   selection or softmax.
 * Same argument checks as saga_decode_attn where they apply.
 */
saga_status saga_debug_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                                   hipStream_t stream);

saga_status saga_debug_gather_rows(const void* v_cache, const int32_t* idx, float* out, int B,
                                   int h_q, int h_v, int d, int N, hipStream_t stream,
                                   int64_t S_max, saga_dtype dtype);

/* Static English text for a status code (never NULL). */
const char* saga_status_string(saga_status s);

#ifdef __cplusplus
}
#endif

#endif /* SAGA_H */
