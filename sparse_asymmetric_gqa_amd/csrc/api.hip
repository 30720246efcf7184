// C ABI of libsaga: argument checks, workspace layout and the launch sequence.
//
// saga_decode_attn enqueues, on the caller's stream and without allocating:
//   K-scan (logits, Eq. 2) -> top-N select (Eq. 6) -> sparse PV (Eq. 7).
// saga_dense_attn enqueues the fused dense pass -> chunk merge (Eqs. 2-4).
#include "saga.h"
#include "saga_internal.h"

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

namespace saga {

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

Workspace carve(void* base, int B, int h_q, int h_k, int d, int N, int64_t S_max,
                bool dense, int chunk, int nsplit, SparqWs* sq) {
    Workspace w{};
    w.chunk = chunk;
    w.nsplit = nsplit;
    char* p = static_cast<char*>(base);
    size_t off = 0;
    const size_t rows = (size_t)B * (size_t)h_q;
    auto take = [&](size_t bytes) -> char* {
        char* r = p ? p + off : nullptr;
        off += align256(bytes);
        return r;
    };
    if (!dense) {
        w.scores = reinterpret_cast<float*>(
            take(rows * (size_t)score_stride(S_max) * sizeof(float)));
        const size_t nch = (size_t)num_chunks(S_max, chunk);
        w.cand = reinterpret_cast<uint2*>(take(rows * nch * (size_t)chunk * sizeof(uint2)));
        w.cand_meta = reinterpret_cast<uint4*>(take(rows * nch * sizeof(uint4)));
        w.cand_stat = reinterpret_cast<float2*>(take(rows * nch * sizeof(float2)));
        w.row_flag = reinterpret_cast<int32_t*>(take(rows * sizeof(int32_t)));
        w.sel_idx = reinterpret_cast<int32_t*>(take(rows * (size_t)N * sizeof(int32_t)));
        w.sel_val = reinterpret_cast<float*>(take(rows * (size_t)N * sizeof(float)));
        w.row_max = reinterpret_cast<float*>(take(rows * sizeof(float)));
        w.row_cnt = reinterpret_cast<int32_t*>(take(rows * sizeof(int32_t)));
        if (nsplit > 1) {
            w.split_part = reinterpret_cast<float*>(
                take(rows * (size_t)nsplit * (size_t)d * sizeof(float)));
            w.split_cnt = reinterpret_cast<int32_t*>(take(rows * sizeof(int32_t)));
        }
        if (sq) sq->qm = reinterpret_cast<float*>(take(rows * (size_t)d * sizeof(float)));
    } else {
        const size_t nsplit = (size_t)dense_nsplit(B, h_k, S_max, h_q / h_k);
        w.part = reinterpret_cast<float*>(take(rows * nsplit * (size_t)(d + 2) * sizeof(float)));
    }
    w.bytes = off;
    return w;
}

bool use_union_path(int h_q, int h_k, int64_t S_max) {
    return h_q / h_k <= 16 && num_chunks(S_max) <= max_union_chunks();
}

// The decode workspace of saga_decode_attn: K-scan chunk and value-gather
// split chosen from the shape (the same choice at sizing and at launch).
Workspace carve_decode(void* base, int B, int h_q, int h_k, int d, int N, int64_t S_max) {
    const bool u = use_union_path(h_q, h_k, S_max);
    return carve(base, B, h_q, h_k, d, N, S_max, false,
                 u ? topm_chunk(B, h_k, S_max) : kScanChunk, u ? gather_split(B, h_q) : 1);
}

// The Atop-N workspace: the decode one with 2N kept slots per row.
Workspace carve_atopn(void* base, int B, int h_q, int h_k, int d, int N, int64_t S_max) {
    return carve(base, B, h_q, h_k, d, 2 * N, S_max, false, topm_chunk(B, h_k, S_max),
                 gather_split(B, h_q));
}

}  // namespace saga

namespace {

using saga::kMaxHeadGroup;
using saga::kScanChunk;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Scalar checks shared by all entry points (no HIP call).
saga_status check_shape(int B, int h_q, int h_k, int h_v, int d, int64_t S_max, int dtype) {
    if (B < 1 || h_q < 1 || h_k < 1 || h_v < 1 || S_max < 1) return SAGA_ERR_INVALID_ARG;
    if (h_q % h_k != 0 || h_q % h_v != 0 || h_k > h_v) return SAGA_ERR_INVALID_ARG;
    if (dtype != SAGA_F32 && dtype != SAGA_BF16) return SAGA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return SAGA_ERR_UNSUPPORTED;
    if (h_q / h_k > kMaxHeadGroup || h_q / h_v > kMaxHeadGroup) return SAGA_ERR_UNSUPPORTED;
    // index arithmetic inside the kernels is 32-bit over rows and positions
    if (S_max > (int64_t)INT32_MAX / 2 || (int64_t)B * h_q > (int64_t)INT32_MAX / 64)
        return SAGA_ERR_UNSUPPORTED;
    return SAGA_OK;
}

// A failed launch maps to SAGA_ERR_HIP; with SAGA_DEBUG set in the environment the
// failing step and HIP's error text are also written to stderr.
// hipGetLastError reports the last error of any HIP runtime call on this thread;
// clear one left pending by unrelated earlier calls so that a failure reported
// here belongs to our own launches.
void clear_stale_error() { (void)hipGetLastError(); }

saga_status from_hip(hipError_t e, const char* step) {
    if (e == hipSuccess) return SAGA_OK;
    if (getenv("SAGA_DEBUG")) fprintf(stderr, "libsaga: %s: %s\n", step, hipGetErrorString(e));
    return SAGA_ERR_HIP;
}

}  // namespace

extern "C" {

size_t saga_workspace_size(int B, int h_q, int h_k, int h_v, int d, int N, int64_t S_max,
                           saga_dtype dtype) {
    if (check_shape(B, h_q, h_k, h_v, d, S_max, dtype) != SAGA_OK || N < 1) return 0;
    return saga::carve_decode(nullptr, B, h_q, h_k, d, N, S_max).bytes;
}

size_t saga_dense_workspace_size(int B, int h_q, int h_k, int h_v, int d, int64_t S_max,
                                 saga_dtype dtype) {
    if (check_shape(B, h_q, h_k, h_v, d, S_max, dtype) != SAGA_OK) return 0;
    return saga::carve(nullptr, B, h_q, h_k, d, 1, S_max, true, kScanChunk, 1).bytes;
}

}  // extern "C"

namespace {

// Records events[i] (i < n_events) at phase boundary i of the decode sequence.
struct PhaseMarks {
    hipEvent_t* ev;
    int n;
    saga_status mark(int i, hipStream_t st) const {
        if (i >= n) return SAGA_OK;
        return from_hip(hipEventRecord(ev[i], st), "event record");
    }
};

saga_status decode(const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* seq_lens, float* out, int B, int h_q, int h_k, int h_v, int d,
                   int N, hipStream_t stream, int64_t S_max, saga_dtype dtype, void* workspace,
                   size_t workspace_bytes, int32_t* idx_out, PhaseMarks pm) {
    if (!q || !k_cache || !v_cache || !seq_lens || !out) return SAGA_ERR_INVALID_ARG;
    saga_status s = check_shape(B, h_q, h_k, h_v, d, S_max, dtype);
    if (s != SAGA_OK) return s;
    if (N < 1) return SAGA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return SAGA_ERR_INVALID_ARG;
    const saga::Workspace need = saga::carve_decode(nullptr, B, h_q, h_k, d, N, S_max);
    if (!workspace || workspace_bytes < need.bytes || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return SAGA_ERR_WORKSPACE;
    const saga::Workspace w = saga::carve_decode(workspace, B, h_q, h_k, d, N, S_max);
    const bool bf16 = dtype == SAGA_BF16;
    const int64_t ss = saga::score_stride(S_max);

    clear_stale_error();
    if (saga::use_union_path(h_q, h_k, S_max)) {
        // events 0 and 1 carry the K-scan dispatch's own start and end
        // the K-scan clears the split counters the fused select + gather uses
        const saga::TopmOut tm{w.cand, w.cand_meta, N, nullptr, w.chunk,
                               w.nsplit > 1 ? w.split_cnt : nullptr, B * h_q};
        s = from_hip(saga::launch_kscan_topm(q, k_cache, seq_lens, tm, B, h_q, h_k, d, S_max,
                                             bf16, stream, pm.n > 0 ? pm.ev[0] : nullptr,
                                             pm.n > 1 ? pm.ev[1] : nullptr),
                     "kscan_topm");
        if (s != SAGA_OK) return s;
        // selection and value gather in one dispatch: the kept lists stay in LDS
        s = from_hip(saga::launch_select_pv(tm, seq_lens, B, h_q, h_k, h_v, d, N, S_max,
                                            w.sel_idx, w.sel_val, w.row_max, w.row_cnt, idx_out,
                                            w.row_flag, q, k_cache, v_cache, w.scores, ss, out,
                                            bf16, w.nsplit, w.split_part, w.split_cnt, nullptr,
                                            stream),
                     "select_pv");
        if (s != SAGA_OK) return s;
        if ((s = pm.mark(2, stream)) != SAGA_OK) return s;
        return pm.mark(3, stream);
    } else {
        if ((s = pm.mark(0, stream)) != SAGA_OK) return s;
        s = from_hip(saga::launch_kscan(q, k_cache, seq_lens, w.scores, ss, B, h_q, h_k, d,
                                        S_max, bf16, stream), "kscan");
        if (s != SAGA_OK) return s;
        if ((s = pm.mark(1, stream)) != SAGA_OK) return s;
        s = from_hip(saga::launch_select(w.scores, ss, seq_lens, B, h_q, N, S_max, w.sel_idx,
                                         w.sel_val, w.row_max, w.row_cnt, idx_out, stream),
                     "select");
        if (s != SAGA_OK) return s;
    }
    if ((s = pm.mark(2, stream)) != SAGA_OK) return s;
    s = from_hip(saga::launch_pv_sparse(v_cache, w.sel_idx, w.sel_val, w.row_max, w.row_cnt,
                                        out, B, h_q, h_v, d, N, S_max, bf16, stream), "pv_sparse");
    if (s != SAGA_OK) return s;
    return pm.mark(3, stream);
}

// ---- the no-allocation decode entry: a static device scratch buffer ----------
// One array per GPU, part of the library's device code object (each GPU the
// library runs on holds it until the process ends). Host code never passes
// the array's name to a kernel: the name is a host-side stand-in. Its device
// address is looked up once per device, with that device current, and kept.
constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::once_flag g_scratch_once[saga::kMaxDevices];
void* g_scratch_ptr[saga::kMaxDevices];

// Device address of this device's scratch array (null on failure).
void* scratch_address(int dev) {
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        int cur = -1;
        bool switched = false;
        if (hipGetDevice(&cur) == hipSuccess && cur != dev)
            switched = hipSetDevice(dev) == hipSuccess;
        if (cur == dev || switched) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) p = nullptr;
            if (switched) (void)hipSetDevice(cur);
        }
        g_scratch_ptr[dev] = p;
    });
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

saga_status saga_decode_attn(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* seq_lens, float* out,
                             int B, int h_q, int h_k, int h_v, int d, int N, hipStream_t stream,
                             int64_t S_max, saga_dtype dtype,
                             void* workspace, size_t workspace_bytes, int32_t* idx_out) {
    return decode(q, k_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d, N, stream, S_max,
                  dtype, workspace, workspace_bytes, idx_out, PhaseMarks{nullptr, 0});
}

saga_status saga_decode_attn_timed(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* seq_lens, float* out,
                                   int B, int h_q, int h_k, int h_v, int d, int N,
                                   hipStream_t stream, int64_t S_max, saga_dtype dtype,
                                   void* workspace, size_t workspace_bytes, int32_t* idx_out,
                                   hipEvent_t* events, int n_events) {
    if (n_events < 0 || n_events > 4 || (n_events > 0 && !events)) return SAGA_ERR_INVALID_ARG;
    for (int i = 0; i < n_events; ++i)
        if (!events[i]) return SAGA_ERR_INVALID_ARG;
    return decode(q, k_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d, N, stream, S_max,
                  dtype, workspace, workspace_bytes, idx_out, PhaseMarks{events, n_events});
}

size_t saga_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

saga_status saga_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* seq_lens, float* out, int B, int h_q, int h_k,
                                     int h_v, int d, int N, hipStream_t stream, int64_t S_max,
                                     saga_dtype dtype, int32_t* idx_out) {
    if (!q || !k_cache || !v_cache || !seq_lens || !out) return SAGA_ERR_INVALID_ARG;
    saga_status s = check_shape(B, h_q, h_k, h_v, d, S_max, dtype);
    if (s != SAGA_OK) return s;
    if (N < 1) return SAGA_ERR_INVALID_ARG;
    const size_t need = saga::carve_decode(nullptr, B, h_q, h_k, d, N, S_max).bytes;
    if (need > kNoAllocScratchBytes) return SAGA_ERR_TOO_LARGE;
    // the device the kernels run on: the stream's, else the current one
    int dev = -1;
    if (stream) {
        if (hipStreamGetDevice(stream, &dev) != hipSuccess) return SAGA_ERR_HIP;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return SAGA_ERR_HIP;
    }
    if (dev < 0 || dev >= saga::kMaxDevices) return SAGA_ERR_UNSUPPORTED;
    void* ws = scratch_address(dev);
    if (!ws) return SAGA_ERR_HIP;
    return decode(q, k_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d, N, stream, S_max,
                  dtype, ws, kNoAllocScratchBytes, idx_out, PhaseMarks{nullptr, 0});
}

saga_status saga_dense_attn(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, float* out,
                            int B, int h_q, int h_k, int h_v, int d, hipStream_t stream,
                            int64_t S_max, saga_dtype dtype,
                            void* workspace, size_t workspace_bytes) {
    if (!q || !k_cache || !v_cache || !seq_lens || !out) return SAGA_ERR_INVALID_ARG;
    saga_status s = check_shape(B, h_q, h_k, h_v, d, S_max, dtype);
    if (s != SAGA_OK) return s;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return SAGA_ERR_INVALID_ARG;
    const saga::Workspace need = saga::carve(nullptr, B, h_q, h_k, d, 1, S_max, true, kScanChunk, 1);
    if (!workspace || workspace_bytes < need.bytes || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return SAGA_ERR_WORKSPACE;
    const saga::Workspace w = saga::carve(workspace, B, h_q, h_k, d, 1, S_max, true, kScanChunk, 1);
    const bool bf16 = dtype == SAGA_BF16;

    clear_stale_error();
    return from_hip(saga::launch_dense_attn(q, k_cache, v_cache, seq_lens, w.part, out, B, h_q,
                                            h_k, h_v, d, S_max, bf16, stream),
                    "dense_attn");
}

size_t saga_atopn_workspace_size(int B, int h_q, int h_k, int h_v, int d, int N,
                                int64_t S_max, saga_dtype dtype) {
    if (check_shape(B, h_q, h_k, h_v, d, S_max, dtype) != SAGA_OK || N < 1 || N > (1 << 29))
        return 0;
    // the decode workspace with kept lists of 2N slots per row
    return saga::carve_atopn(nullptr, B, h_q, h_k, d, N, S_max).bytes;
}

}  // extern "C"

namespace {

// Shared argument checks and workspace carve of the two Atop-N entry points.
saga_status atopn_prepare(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* seq_lens, const float* out, int B, int h_q, int h_k,
                          int h_v, int d, int N, int64_t S_max, saga_dtype dtype, void* workspace,
                          size_t workspace_bytes, const float* tau, saga::Workspace& w) {
    if (!q || !k_cache || !v_cache || !seq_lens || !out || !tau) return SAGA_ERR_INVALID_ARG;
    saga_status s = check_shape(B, h_q, h_k, h_v, d, S_max, dtype);
    if (s != SAGA_OK) return s;
    if (N < 1 || N > (1 << 29)) return SAGA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return SAGA_ERR_INVALID_ARG;
    if (!saga::use_union_path(h_q, h_k, S_max)) return SAGA_ERR_UNSUPPORTED;
    const saga::Workspace need = saga::carve_atopn(nullptr, B, h_q, h_k, d, N, S_max);
    if (!workspace || workspace_bytes < need.bytes ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return SAGA_ERR_WORKSPACE;
    w = saga::carve_atopn(workspace, B, h_q, h_k, d, N, S_max);
    return SAGA_OK;
}

}  // namespace

extern "C" {

saga_status saga_atopn_calibrate(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* seq_lens, float* out, int B, int h_q, int h_k,
                                 int h_v, int d, int N, hipStream_t stream, int64_t S_max,
                                 saga_dtype dtype, void* workspace, size_t workspace_bytes,
                                 float* tau, int32_t* idx_out) {
    saga::Workspace w;
    saga_status s = atopn_prepare(q, k_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d, N,
                                  S_max, dtype, workspace, workspace_bytes, tau, w);
    if (s != SAGA_OK) return s;
    const bool bf16 = dtype == SAGA_BF16;
    const int64_t ss = saga::score_stride(S_max);
    clear_stale_error();
    // the exact top-N step (the decode call's two kernels, with its chunk size
    // and split), the K-scan also writing per-chunk softmax statistics and the
    // fused select + gather also tau
    const saga::TopmOut tm{w.cand, w.cand_meta, N, w.cand_stat, w.chunk,
                           w.nsplit > 1 ? w.split_cnt : nullptr, B * h_q};
    s = from_hip(saga::launch_kscan_topm(q, k_cache, seq_lens, tm, B, h_q, h_k, d, S_max, bf16,
                                         stream), "kscan_topm");
    if (s != SAGA_OK) return s;
    return from_hip(saga::launch_select_pv(tm, seq_lens, B, h_q, h_k, h_v, d, N, S_max,
                                           w.sel_idx, w.sel_val, w.row_max, w.row_cnt, idx_out,
                                           w.row_flag, q, k_cache, v_cache, w.scores, ss, out,
                                           bf16, w.nsplit, w.split_part, w.split_cnt, tau,
                                           stream),
                    "select_pv");
}

saga_status saga_atopn_attn(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, float* out, int B, int h_q, int h_k,
                            int h_v, int d, int N, hipStream_t stream, int64_t S_max,
                            saga_dtype dtype, void* workspace, size_t workspace_bytes,
                            const float* tau, int32_t* idx_out, int32_t* count_out) {
    saga::Workspace w;
    saga_status s = atopn_prepare(q, k_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d, N,
                                  S_max, dtype, workspace, workspace_bytes, tau, w);
    if (s != SAGA_OK) return s;
    const bool bf16 = dtype == SAGA_BF16;
    const int64_t ss = saga::score_stride(S_max);
    const int cap = 2 * N;
    clear_stale_error();
    // candidate lists sized for 1.5 N kept entries (a drifted query keeps
    // more than the N of its calibration; the completeness check sends a row
    // whose lists do not cover the threshold to the recompute), with chunk
    // statistics; the K-scan also clears the split counters
    const saga::TopmOut tm{w.cand, w.cand_meta, N + N / 2, w.cand_stat, w.chunk,
                           w.nsplit > 1 ? w.split_cnt : nullptr, B * h_q};
    s = from_hip(saga::launch_kscan_topm(q, k_cache, seq_lens, tm, B, h_q, h_k, d, S_max, bf16,
                                         stream), "kscan_topm");
    if (s != SAGA_OK) return s;
    return from_hip(saga::launch_select_thresh(tm, seq_lens, tau, B, h_q, h_k, h_v, d, cap, S_max,
                                               w.sel_idx, w.sel_val, idx_out, count_out,
                                               w.row_flag, q, k_cache, v_cache, w.scores, ss,
                                               out, bf16, w.nsplit, w.split_part, w.split_cnt,
                                               stream),
                    "select_thresh");
}

size_t saga_sparq_workspace_size(int B, int h_q, int h_k, int h_v, int d, int N, int r,
                                 int64_t S_max, saga_dtype dtype) {
    if (check_shape(B, h_q, h_k, h_v, d, S_max, dtype) != SAGA_OK) return 0;
    if (N < 1 || N > (1 << 29) || r < 1 || r > d) return 0;
    saga::SparqWs sw{};
    return saga::carve(nullptr, B, h_q, h_k, d, N, S_max, false, kScanChunk, 1, &sw).bytes;
}

saga_status saga_sparq_attn(const void* q, const void* k_cache, const void* kt_cache,
                            const void* v_cache, const int32_t* seq_lens, float* out, int B,
                            int h_q, int h_k, int h_v, int d, int N, int r, int local,
                            const float* v_mean, hipStream_t stream, int64_t S_max,
                            saga_dtype dtype, void* workspace, size_t workspace_bytes,
                            int32_t* idx_out, float* alpha_out, int32_t* dims_out) {
    if (!q || !k_cache || !kt_cache || !v_cache || !seq_lens || !out) return SAGA_ERR_INVALID_ARG;
    saga_status s = check_shape(B, h_q, h_k, h_v, d, S_max, dtype);
    if (s != SAGA_OK) return s;
    if (N < 1 || N > (1 << 29) || r < 1 || r > d || local < 0 || local > N)
        return SAGA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(kt_cache) || !aligned16(v_cache) ||
        (reinterpret_cast<uintptr_t>(v_mean) & 3u))
        return SAGA_ERR_INVALID_ARG;
    const int esize = dtype == SAGA_BF16 ? 2 : 4;
    // the scan reads 16-byte pieces of the S-contiguous copy's rows
    if (!saga::use_union_path(h_q, h_k, S_max) || !saga::sparq_select_fits(N) ||
        S_max % (16 / esize) != 0)
        return SAGA_ERR_UNSUPPORTED;
    saga::SparqWs sw{};
    const saga::Workspace need = saga::carve(nullptr, B, h_q, h_k, d, N, S_max, false, kScanChunk, 1, &sw);
    if (!workspace || workspace_bytes < need.bytes || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return SAGA_ERR_WORKSPACE;
    const saga::Workspace w = saga::carve(workspace, B, h_q, h_k, d, N, S_max, false, kScanChunk, 1, &sw);
    const bool bf16 = dtype == SAGA_BF16;
    clear_stale_error();
    // Step 1 on the kept dims into candidate lists with chunk statistics (the
    // window is ranked by nobody), then Steps 2-3 in one dispatch per row
    const saga::TopmOut tm{w.cand, w.cand_meta, N - local, w.cand_stat, kScanChunk, nullptr, 0};
    s = from_hip(saga::launch_sparq_scan(q, kt_cache, seq_lens, tm, sw, B, h_q, h_k, d, r, local,
                                         S_max, bf16, dims_out, stream),
                 "sparq_scan");
    if (s != SAGA_OK) return s;
    return from_hip(saga::launch_select_sparq(tm, sw, seq_lens, B, h_q, h_k, h_v, d, N, local,
                                              S_max, w.sel_idx, w.sel_val, w.row_max, w.row_cnt,
                                              idx_out, w.row_flag, q, k_cache, v_cache, w.scores,
                                              saga::score_stride(S_max), v_mean, out, alpha_out,
                                              bf16, stream),
                    "select_sparq");
}

saga_status saga_debug_scores(const void* q, const void* k_cache, const int32_t* seq_lens,
                              float* scores, int B, int h_q, int h_k, int d, hipStream_t stream,
                              int64_t S_max, saga_dtype dtype) {
    if (!q || !k_cache || !seq_lens || !scores) return SAGA_ERR_INVALID_ARG;
    saga_status s = check_shape(B, h_q, h_k, h_k, d, S_max, dtype);
    if (s != SAGA_OK) return s;
    if (!aligned16(q) || !aligned16(k_cache)) return SAGA_ERR_INVALID_ARG;
    clear_stale_error();
    return from_hip(saga::launch_kscan(q, k_cache, seq_lens, scores, S_max, B, h_q, h_k, d,
                                       S_max, dtype == SAGA_BF16, stream), "kscan");
}

saga_status saga_debug_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                                  hipStream_t stream) {
    if (!buf || !sink || bytes < 16 || (bytes & 15) || !aligned16(buf))
        return SAGA_ERR_INVALID_ARG;
    clear_stale_error();
    return from_hip(saga::launch_stream_read(buf, bytes, sink, stream), "stream_read");
}

saga_status saga_debug_gather_rows(const void* v_cache, const int32_t* idx, float* out, int B,
                                   int h_q, int h_v, int d, int N, hipStream_t stream,
                                   int64_t S_max, saga_dtype dtype) {
    if (!v_cache || !idx || !out || N < 1) return SAGA_ERR_INVALID_ARG;
    saga_status s = check_shape(B, h_q, h_v, h_v, d, S_max, dtype);
    if (s != SAGA_OK) return s;
    if (!aligned16(v_cache)) return SAGA_ERR_INVALID_ARG;
    clear_stale_error();
    return from_hip(saga::launch_gather_rows(v_cache, idx, out, B, h_q, h_v, d, N, S_max,
                                             dtype == SAGA_BF16, stream), "gather_rows");
}

saga_status saga_debug_fallback_rows(const void* workspace, size_t workspace_bytes, int B,
                                     int h_q, int h_k, int h_v, int d, int N, int64_t S_max,
                                     saga_dtype dtype, int32_t* host_flags, hipStream_t stream) {
    if (!workspace || !host_flags) return SAGA_ERR_INVALID_ARG;
    saga_status s = check_shape(B, h_q, h_k, h_v, d, S_max, dtype);
    if (s != SAGA_OK) return s;
    if (N < 1) return SAGA_ERR_INVALID_ARG;
    const saga::Workspace need = saga::carve_decode(nullptr, B, h_q, h_k, d, N, S_max);
    if (workspace_bytes < need.bytes) return SAGA_ERR_WORKSPACE;
    const size_t rows = (size_t)B * (size_t)h_q;
    if (!saga::use_union_path(h_q, h_k, S_max)) {
        for (size_t r = 0; r < rows; ++r) host_flags[r] = 0;
        return SAGA_OK;
    }
    const saga::Workspace w =
        saga::carve_decode(const_cast<void*>(workspace), B, h_q, h_k, d, N, S_max);
    clear_stale_error();
    if (hipMemcpyAsync(host_flags, w.row_flag, rows * sizeof(int32_t), hipMemcpyDeviceToHost,
                       stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return SAGA_ERR_HIP;
    return SAGA_OK;
}

const char* saga_status_string(saga_status s) {
    switch (s) {
        case SAGA_OK: return "ok";
        case SAGA_ERR_INVALID_ARG: return "invalid argument";
        case SAGA_ERR_UNSUPPORTED: return "unsupported shape (d must be 64 or 128; head groups <= 64)";
        case SAGA_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
        case SAGA_ERR_HIP: return "HIP launch failure";
        case SAGA_ERR_TOO_LARGE:
            return "the shape needs more scratch than the static buffer of saga_decode_attn_noalloc";
    }
    return "unknown status";
}

}  // extern "C"
