// Internal declarations shared by the libsaga translation units (HIP, gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace saga {

// ---- launch geometry (also used by the workspace-size functions) ----------
#ifndef SAGA_KSCAN_CHUNK
#define SAGA_KSCAN_CHUNK 1024
#endif
constexpr int kScanChunk = SAGA_KSCAN_CHUNK;   // positions per K-scan workgroup
constexpr int kPvEntries = 2048;     // kept entries staged per block of the sparse PV
constexpr int kSelectThreads = 1024; // threads of one select workgroup
constexpr int kMaxHeadGroup = 64;    // largest h_q / h_k and h_q / h_v supported
constexpr int kMaxDevices = 64;      // device ordinals the host-side caches cover

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Row stride (floats) of the logit workspace: padded so rows start 64-byte aligned.
inline int64_t score_stride(int64_t S_max) { return round_up(S_max, 16); }

struct Workspace {
    float* scores;      // [B][h_q][score_stride]  logits (decode: wide key groups, fallback rows)
    uint2* cand;        // candidate pool: B*h_k*nchunk items x g*chunk entries
    uint4* cand_meta;   // [B][h_q][nchunk]  {pool offset lo, count, cutoff, pool offset hi}
    float2* cand_stat;  // [B][h_q][nchunk]  {max logit, sum exp(logit - max)} (Atop-N)
    int32_t* row_flag;  // [B][h_q]   1 if the row took the dense fallback in the last call
    int32_t* sel_idx;   // [B][h_q][N]
    float* sel_val;     // [B][h_q][N]
    float* row_max;     // [B][h_q]   largest kept logit
    int32_t* row_cnt;   // [B][h_q]   N_eff
    float* part;        // dense: [B][h_q][nchunk][d + 2]  (m, l, acc[d]) per chunk
    float* split_part;  // [B][h_q][nsplit][d]  value-gather partial sums (nsplit > 1)
    int32_t* split_cnt; // [B][h_q]   parts of a row finished (nsplit > 1)
    int chunk;          // positions per K-scan work item
    int nsplit;         // value-gather workgroups per (b, i) row
    size_t bytes;
};

// SparQ-style scoring state per call (written by the scan's set-up kernel):
struct SparqWs {
    float* qm;         // [B*h_q][d]    q / tau on the kept dims, 0 elsewhere (written by the scan)
};

inline int num_chunks(int64_t S_max, int chunk = kScanChunk) {
    return (int)((S_max + chunk - 1) / chunk);
}

// Positions per work item of the top-M K-scan: 1024 when that gives at
// least 256 items (one per CU); else 512 where that does, with rows of at
// most 256 chunks (the union select's fast path); else 256 for rows of up to
// 64 Ki positions, 512 up to 128 Ki. Shorter items fill the CUs of a short
// call; 512 rather than 256 keeps the candidate lists shorter where it can.
inline int topm_chunk(int B, int h_k, int64_t S_max) {
    const int64_t rows = (int64_t)B * h_k;
    if (rows * num_chunks(S_max) >= 256) return kScanChunk;
    if (S_max <= 256 * 512 && rows * num_chunks(S_max, 512) >= 256) return 512;
    if (S_max <= 256 * 256) return 256;
    return S_max <= 256 * 512 ? 512 : kScanChunk;
}

// Workgroups per (b, i) row of the fused select + value gather: rows are
// split along their kept list when there are too few of them to occupy the
// CUs (each part gathers a slice; the last part to finish merges the sums).
constexpr int kMaxSplit = 8;
inline int gather_split(int B, int h_q) {
    const int rows = B * h_q;
    const int p = rows >= 256 ? 1 : 256 / rows;
    return p < kMaxSplit ? p : kMaxSplit;
}

// Whether saga_decode_attn takes the top-M K-scan + union select path.
bool use_union_path(int h_q, int h_k, int64_t S_max);
int max_union_chunks();

// Carve the decode workspace (dense == false) or the dense one out of `base`
// (base may be null to only compute the size), for K-scan items of `chunk`
// positions and `nsplit` value-gather parts per row. With sq, the SparQ state
// follows the decode part.
Workspace carve(void* base, int B, int h_q, int h_k, int d, int N, int64_t S_max, bool dense,
                int chunk, int nsplit, SparqWs* sq = nullptr);

// The decode workspace (chunk and split from the shape) and the Atop-N one
// (2N kept slots per row).
Workspace carve_decode(void* base, int B, int h_q, int h_k, int d, int N, int64_t S_max);
Workspace carve_atopn(void* base, int B, int h_q, int h_k, int d, int N, int64_t S_max);

// Dense attention: positions per work item for a call's shape (B rows of h_k
// key heads, key groups of g query heads), and chunks (partials) per (b, i)
// row.
int dense_chunk(int B, int h_k, int64_t S_max, int g);
int dense_nsplit(int B, int h_k, int64_t S_max, int g);   // ceil(S_max / dense_chunk(...))

// Candidate lists published by the top-M K-scan. The workgroup that takes
// work items [w0, w1) packs the lists of their heads, in any order, from pool
// entry w0 * g * chunk on (the items' regions bound the total). For slot
// (b*h_q + i, chunk): meta = {off_lo, cnt, cut, off_hi} with the list at
// cand[off, off + cnt) = (position, key) ascending in position, off the 64-bit
// absolute pool index, and cut = the chunk's cutoff key (every key of the
// chunk left out is below it).
struct TopmOut {
    uint2* cand;
    uint4* meta;       // [B*h_q][nchunk]
    int N;             // the M of each chunk's list is sized for this N
    float2* stat;      // nullable: [B*h_q][nchunk] {max logit, sum of exp(logit - max)}
    int chunk;         // positions per work item (kScanChunk, 512 or 256)
    int32_t* zero;     // nullable: nzero ints the K-scan clears before anything else
    int nzero;
};

// ---- host-side launch caches (launch.hip; thread-safe, per current device) ----
int cu_count();
// Resident workgroups per CU of `kern` at this block size and dynamic LDS.
int blocks_per_cu(const void* kern, int threads, size_t lds);
// Opts `kern` in to `lds` bytes of dynamic LDS (> 64 KiB) once per device.
hipError_t allow_dynamic_lds(const void* kern, size_t lds);

// ---- launchers (defined next to their kernels) ------------------------------
// All return hipGetLastError() after enqueueing.
hipError_t launch_kscan(const void* q, const void* k, const int32_t* lens, float* scores,
                        int64_t s_stride, int B, int h_q, int h_k, int d, int64_t S_max,
                        bool bf16, hipStream_t st);

// K-scan in top-M mode (h_q / h_k <= 16): candidate lists instead of logits.
// ev0 / ev1 (nullable) are stamped with the kernel's own start and end.
hipError_t launch_kscan_topm(const void* q, const void* k, const int32_t* lens, const TopmOut& tm,
                             int B, int h_q, int h_k, int d, int64_t S_max, bool bf16,
                             hipStream_t st, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

hipError_t launch_select(const float* scores, int64_t s_stride, const int32_t* lens, int B,
                         int h_q, int N, int64_t S_max, int32_t* sel_idx, float* sel_val,
                         float* row_max, int32_t* row_cnt, int32_t* idx_out, hipStream_t st);



// Atop-N stale-threshold selection fused with the value gather (lists from
// launch_kscan_topm with stat): keeps the positions with logit >= log(tau) +
// LSE, the first cap in position order, and writes out[B*h_q][d] (0 for a
// row keeping none). idx_out (nullable) [B*h_q][cap]; count_out (nullable)
// gets the count before the cap; sel_idx / sel_val [B*h_q][cap] serve rows
// that recompute their logits. nsplit, split_part, split_cnt as for
// launch_select_pv (tm.zero clears split_cnt).
hipError_t launch_select_thresh(const TopmOut& tm, const int32_t* lens, const float* tau, int B,
                                int h_q, int h_k, int h_v, int d, int cap, int64_t S_max,
                                int32_t* sel_idx, float* sel_val, int32_t* idx_out,
                                int32_t* count_out, int32_t* row_flag, const void* q,
                                const void* k, const void* v, float* scores, int64_t s_stride,
                                float* out, bool bf16, int nsplit, float* split_part,
                                int32_t* split_cnt, hipStream_t st);



// Union select fused with the value gather: writes out[B][h_q][d] directly
// (sel_idx / sel_val only for rows the general code takes). With tau (and
// tm.stat from the K-scan) also the Atop-N calibration tau [B*h_q].
hipError_t launch_select_pv(const TopmOut& tm, const int32_t* lens, int B, int h_q, int h_k,
                            int h_v, int d, int N, int64_t S_max, int32_t* sel_idx,
                            float* sel_val, float* row_max, int32_t* row_cnt, int32_t* idx_out,
                            int32_t* row_flag, const void* q, const void* k, const void* v,
                            float* scores, int64_t s_stride, float* out, bool bf16, int nsplit,
                            float* split_part, int32_t* split_cnt, float* tau, hipStream_t st);

// SparQ-style scoring (h_q / h_k <= 16): the set-up kernel (dims, 1 / tau,
// qm, the scan operand; dims_out nullable [B*h_k][r]) and the scan of the r
// kept columns of kt [B][h_k][d][S_max] into candidate lists (tm.N = N - local,
// tm.stat required); positions of the last `local` are left out of the lists.
hipError_t launch_sparq_scan(const void* q, const void* kt, const int32_t* lens, const TopmOut& tm,
                             const SparqWs& sw, int B, int h_q, int h_k, int d, int r, int local,
                             int64_t S_max, bool bf16, int32_t* dims_out, hipStream_t st);

// Union select over the SparQ candidate lists, the window appended, exact
// rescoring of the kept rows, the value gather and Step 3's mix with vmean
// (nullable [B][h_v][d]) into out; alpha_out (nullable) [B*h_q].
hipError_t launch_select_sparq(const TopmOut& tm, const SparqWs& sw, const int32_t* lens, int B,
                               int h_q, int h_k, int h_v, int d, int N, int local, int64_t S_max,
                               int32_t* sel_idx, float* sel_val, float* row_max, int32_t* row_cnt,
                               int32_t* idx_out, int32_t* row_flag, const void* q, const void* k,
                               const void* v, float* scores, int64_t s_stride, const float* vmean,
                               float* out, float* alpha_out, bool bf16, hipStream_t st);
// Whether launch_select_sparq can stage N kept entries in LDS.
bool sparq_select_fits(int N);

hipError_t launch_pv_sparse(const void* v, const int32_t* sel_idx, const float* sel_val,
                            const float* row_max, const int32_t* row_cnt, float* out, int B,
                            int h_q, int h_v, int d, int N, int64_t S_max, bool bf16,
                            hipStream_t st);

// Bandwidth ceilings (ceiling.hip): a sequential read of `bytes` (a multiple of
// 16; sink: device uint32, written only in the impossible case), and a plain
// gather of the value rows listed in idx [B*h_q][N] into out [B*h_q][d].
hipError_t launch_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t st);
hipError_t launch_gather_rows(const void* v, const int32_t* idx, float* out, int B, int h_q,
                              int h_v, int d, int N, int64_t S_max, bool bf16, hipStream_t st);

// Dense attention (every position, Eqs. 2-4): fused K stream, chunk softmax
// and V stream into part [B][h_q][nchunk][d + 2], then the log-sum-exp merge
// of the chunks into out[B][h_q][d].
hipError_t launch_dense_attn(const void* q, const void* k, const void* v, const int32_t* lens,
                             float* part, float* out, int B, int h_q, int h_k, int h_v, int d,
                             int64_t S_max, bool bf16, hipStream_t st);

}  // namespace saga

// ---- device helpers ---------------------------------------------------------
#ifdef __HIPCC__
namespace saga {
namespace dev {

typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline int64_t clamp_len(int32_t L, int64_t S_max) {
    int64_t x = L;
    return x < 0 ? 0 : (x > S_max ? S_max : x);
}

// Order-preserving map fp32 -> uint32 (larger float <=> larger key); -0.0 is
// folded onto +0.0 first so the two compare equal.
__device__ inline uint32_t float_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float key_float(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// popcount of the bits of a 64-lane mask that belong to lanes below this one
__device__ inline uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ inline uint64_t ballot(bool p) { return __ballot(p); }

// Inclusive prefix sum over the 64 lanes of a wave: row_shr DPP steps inside
// each row of 16 lanes, then the row totals (read from lanes 15, 31, 47) are
// added to the later rows. `total` receives the sum over all lanes.
__device__ inline uint32_t wave_incl_scan(uint32_t v, uint32_t& total) {
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane(x, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane(x, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane(x, 47);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane(x, 63);
    total = r0 + r1 + r2 + r3;
    const int row = (int)(threadIdx.x & 63) >> 4;
    const uint32_t add = (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
    return (uint32_t)x + add;
}

// Sum over the 64 lanes of a wave (uniform result).
__device__ inline uint32_t wave_sum(uint32_t v) {
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
    return (uint32_t)__builtin_amdgcn_readlane(x, 15) + (uint32_t)__builtin_amdgcn_readlane(x, 31) +
           (uint32_t)__builtin_amdgcn_readlane(x, 47) + (uint32_t)__builtin_amdgcn_readlane(x, 63);
}


// 16 bytes of a value row -> EPL fp32 values
template <typename T> struct Row16;
template <> struct Row16<uint16_t> {
    static constexpr int EPL = 8;
    __device__ static inline void cvt(const u32x4& r, float* f) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            f[2 * c] = __uint_as_float(r[c] << 16);
            f[2 * c + 1] = __uint_as_float(r[c] & 0xFFFF0000u);
        }
    }
};
template <> struct Row16<float> {
    static constexpr int EPL = 4;
    __device__ static inline void cvt(const u32x4& r, float* f) {
#pragma unroll
        for (int c = 0; c < 4; ++c) f[c] = __uint_as_float(r[c]);
    }
};

// Maximum over the wave of an unsigned value (uniform result). DPP row
// shifts build each 16-lane row's running maximum; lanes without a source
// keep 0, the identity.
__device__ inline uint32_t wave_umax(uint32_t v) {
    // lanes without a source keep 0, the identity of an unsigned maximum
    int x = (int)v, y;
    y = __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false); x = (uint32_t)y > (uint32_t)x ? y : x;
    y = __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false); x = (uint32_t)y > (uint32_t)x ? y : x;
    y = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false); x = (uint32_t)y > (uint32_t)x ? y : x;
    y = __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false); x = (uint32_t)y > (uint32_t)x ? y : x;
    uint32_t r = (uint32_t)__builtin_amdgcn_readlane(x, 15);
    uint32_t t = (uint32_t)__builtin_amdgcn_readlane(x, 31); r = t > r ? t : r;
    t = (uint32_t)__builtin_amdgcn_readlane(x, 47); r = t > r ? t : r;
    t = (uint32_t)__builtin_amdgcn_readlane(x, 63); r = t > r ? t : r;
    return r;
}

// Sum over the wave of a float (uniform result; same DPP pattern, +0.0 for
// lanes without a source).
__device__ inline float wave_fsum(float v) {
    float x = v;
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, false));
    return (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15)) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31))) +
           (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47)) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63)));
}

// Logical workgroup id from the hardware one: hardware ids are dealt to the
// 8 XCDs round-robin, so give XCD x the contiguous logical range [x Q,
// (x + 1) Q), Q = ceil(total / 8). A permutation of [0, total) when total is
// a multiple of 8 (grids are rounded up to that, or keep the identity).
__device__ inline int xcd_logical(int hw, int total) {
    const int q = (total + 7) >> 3;
    return (hw & 7) * q + (hw >> 3);
}

}  // namespace dev
}  // namespace saga
#endif
