// Softmax weights + value gather (PV) in splits, and the log-sum-exp merge.
//
// "More Value per Key" §3.1 Eq. 7: O = softmax(A[i]) V[i] -- only the kept
// value rows are read (App. C.1: gather, then a batched product), and each
// query head uses value head i / (h_q / h_v) (§3.2, App. B Eq. 29).
//
// Sparse path: one workgroup per (b, i) row, walking its kept list in blocks
// of kPvEntries. Per block its 256 threads stage positions and weights
// exp(s - m) in LDS (m = the row's largest kept logit), then every wave
// streams its share of value rows with 16-byte loads, LPR lanes per row, all
// rows of a wave in flight at once; the block sums stay in registers and the
// row ends with out = acc / l, so no merge pass is needed. The g_v heads that
// share a value head are mapped to the same XCD at neighbouring times so value
// rows they have in common are served from that XCD's L2.
//
// Dense path (full attention over all L_b rows, §2.1 Eqs. 2-4): one
// workgroup per (b, value head, group of <= 8 query heads, block of
// kDenseRows positions); every value row of the block is read once and
// applied to all heads of the group; partials carry their own max.
//
// Merge: out = sum_s acc_s e^{m_s - M} / sum_s l_s e^{m_s - M}, M = max m_s.
#include "saga_internal.h"

namespace saga {
using namespace dev;

namespace {

constexpr int kPvThreads = 256;
constexpr int kPvWaves = kPvThreads / 64;
constexpr int kDenseHeads = 8;

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

// logical workgroup id from the hardware one: hardware ids are dealt to the 8
// XCDs round-robin, so give XCD x the contiguous logical range [x*Q, (x+1)*Q).
__device__ inline int xcd_logical(int hw, int total) {
    const int q = (total + 7) >> 3;
    return (hw & 7) * q + (hw >> 3);
}

template <typename T, int DH>
__global__ __launch_bounds__(kPvThreads) void pv_sparse(
    const T* __restrict__ v, const int32_t* __restrict__ sel_idx, const float* __restrict__ sel_val,
    const float* __restrict__ row_max, const int32_t* __restrict__ row_cnt,
    float* __restrict__ out, int h_q, int h_v, int N, int64_t S_max, int total) {
    using R = Row16<T>;
    constexpr int EPL = R::EPL;
    constexpr int LPR = DH / EPL;          // lanes per value row
    constexpr int RPI = 64 / LPR;          // rows per wave instruction
    constexpr int STEP = kPvWaves * RPI;   // rows per workgroup step
    constexpr int PER = kPvEntries / STEP; // rows per row-group and block
    constexpr int UNR = PER < 16 ? PER : 16;
    __shared__ int32_t s_pos[kPvEntries];
    __shared__ float s_w[kPvEntries];
    __shared__ float s_red[kPvWaves][DH];
    __shared__ float s_l[kPvWaves];

    const int lid = xcd_logical((int)blockIdx.x, total);
    if (lid >= total) return;
    const int row = lid;                     // = b*h_q + i; the g_v heads of a value head are adjacent
    const int b = row / h_q;
    const int i = row - b * h_q;
    const int g_v = h_q / h_v;
    const int vh = i / g_v;
    const int cnt = row_cnt[row];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    float* o = out + (int64_t)row * DH;
    if (cnt <= 0) {   // no kept entry (L_b = 0): out = 0
        for (int c = tid; c < DH; c += kPvThreads) o[c] = 0.f;
        return;
    }
    const float m = row_max[row];
    const T* vb = v + (int64_t)(b * h_v + vh) * S_max * DH;
    const int rg = lane / LPR;
    const int sub = lane - rg * LPR;
    const int first = wave * RPI + rg;
    float acc[EPL];
#pragma unroll
    for (int c = 0; c < EPL; ++c) acc[c] = 0.f;
    float lsum = 0.f;   // thread tid's share of l, blocks in order
#pragma unroll 1
    for (int e0 = 0; e0 < cnt; e0 += kPvEntries) {
        const int ne = cnt - e0 < kPvEntries ? cnt - e0 : kPvEntries;
        {
            const int e = tid;
            float w = 0.f;
            int32_t pos = 0;
            if (e < ne) {
                pos = sel_idx[(int64_t)row * N + e0 + e];
                // kept positions lie in [0, L_b); clamp anyway so a bad list cannot leave the cache
                pos = pos < 0 ? 0 : (pos >= S_max ? (int32_t)(S_max - 1) : pos);
                w = __expf(sel_val[(int64_t)row * N + e0 + e] - m);
            }
            s_pos[e] = pos;
            s_w[e] = w;
            lsum += w;
        }
        __syncthreads();
#pragma unroll 1
        for (int k0 = 0; k0 < PER; k0 += UNR) {
            u32x4 raw[UNR];
            float wt[UNR];
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                const int e = first + (k0 + k) * STEP;
                wt[k] = s_w[e];   // 0 past ne
                raw[k] = *reinterpret_cast<const u32x4*>(vb + (int64_t)s_pos[e] * DH + sub * EPL);
            }
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                float f[EPL];
                R::cvt(raw[k], f);
#pragma unroll
                for (int c = 0; c < EPL; ++c) acc[c] += wt[k] * f[c];
            }
        }
        __syncthreads();   // the block's LDS lists are reused by the next block
    }
    // l: thread shares summed over lanes, then waves (fixed order)
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off, 64);
    if (lane == 0) s_l[wave] = lsum;
    // acc: reduce over the row-groups of the wave, then over waves
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
        for (int c = 0; c < EPL; ++c) acc[c] += __shfl_xor(acc[c], off, 64);
    if (rg == 0)
#pragma unroll
        for (int c = 0; c < EPL; ++c) s_red[wave][sub * EPL + c] = acc[c];
    __syncthreads();
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kPvWaves; ++w) l += s_l[w];
    for (int c = tid; c < DH; c += kPvThreads) {
        float sacc = 0.f;
#pragma unroll
        for (int w = 0; w < kPvWaves; ++w) sacc += s_red[w][c];
        o[c] = sacc / l;   // l >= 1: the largest kept logit has weight 1
    }
}

template <typename T, int DH>
__global__ __launch_bounds__(kPvThreads) void pv_dense(
    const T* __restrict__ v, const float* __restrict__ scores, int64_t s_stride,
    const int32_t* __restrict__ lens, float* __restrict__ part, int h_q, int h_v, int nsplit,
    int64_t S_max, int ngrp) {
    using R = Row16<T>;
    constexpr int EPL = R::EPL;
    constexpr int LPR = DH / EPL;
    constexpr int RPI = 64 / LPR;
    constexpr int STEP = kPvWaves * RPI;
    constexpr int UNR = 4;
    constexpr int HR = kDenseHeads;
    static_assert(HR * kDenseRows >= kPvWaves * HR * DH, "reduction buffer must fit");
    __shared__ float s_w[HR][kDenseRows];
    __shared__ float s_m[HR];
    __shared__ float s_l[HR];

    const int split = blockIdx.x;
    const int hg = blockIdx.y % ngrp;
    const int bvh = blockIdx.y / ngrp;
    const int b = bvh / h_v;
    const int vh = bvh - b * h_v;
    const int g_v = h_q / h_v;
    const int u0 = hg * HR;
    const int nh = g_v - u0 < HR ? g_v - u0 : HR;
    const int64_t L = clamp_len(lens[b], S_max);
    const int64_t p0 = (int64_t)split * kDenseRows;
    if (p0 >= L) return;
    const int cnt = (int)(L - p0 < kDenseRows ? L - p0 : kDenseRows);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int row0 = b * h_q + vh * g_v + u0;   // first query head of the group

    for (int u = 0; u < nh; ++u)
        for (int r = tid; r < cnt; r += kPvThreads)
            s_w[u][r] = scores[(int64_t)(row0 + u) * s_stride + p0 + r];
    __syncthreads();
    // per-head max and weights; wave w handles heads w, w + 4
    for (int u = wave; u < nh; u += kPvWaves) {
        float mx = -__builtin_inff();
        for (int r = lane; r < cnt; r += 64) mx = fmaxf(mx, s_w[u][r]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        float l = 0.f;
        for (int r = lane; r < cnt; r += 64) {
            const float w = __expf(s_w[u][r] - mx);
            s_w[u][r] = w;
            l += w;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
        if (lane == 0) {
            s_m[u] = mx;
            s_l[u] = l;
        }
    }
    __syncthreads();

    const int rg = lane / LPR;
    const int sub = lane - rg * LPR;
    const T* vb = v + ((int64_t)(b * h_v + vh) * S_max + p0) * DH + sub * EPL;
    float acc[HR][EPL];
#pragma unroll
    for (int u = 0; u < HR; ++u)
#pragma unroll
        for (int c = 0; c < EPL; ++c) acc[u][c] = 0.f;
    const int first = wave * RPI + rg;
#pragma unroll 1
    for (int r0 = 0; r0 < cnt; r0 += STEP * UNR) {
        u32x4 raw[UNR];
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            int r = r0 + first + k * STEP;
            r = r < cnt ? r : cnt - 1;
            raw[k] = *reinterpret_cast<const u32x4*>(vb + (int64_t)r * DH);
        }
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            const int r = r0 + first + k * STEP;
            if (r < cnt) {
                float f[EPL];
                R::cvt(raw[k], f);
#pragma unroll
                for (int u = 0; u < HR; ++u) {
                    if (u < nh) {
                        const float w = s_w[u][r];
#pragma unroll
                        for (int c = 0; c < EPL; ++c) acc[u][c] += w * f[c];
                    }
                }
            }
        }
    }
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
        for (int u = 0; u < HR; ++u)
#pragma unroll
            for (int c = 0; c < EPL; ++c) acc[u][c] += __shfl_xor(acc[u][c], o, 64);
    __syncthreads();   // s_w is reused below as the cross-wave reduction buffer
    float* red = &s_w[0][0];   // [kPvWaves][HR][DH]
    if (rg == 0)
#pragma unroll
        for (int u = 0; u < HR; ++u)
#pragma unroll
            for (int c = 0; c < EPL; ++c) red[(wave * HR + u) * DH + sub * EPL + c] = acc[u][c];
    __syncthreads();
    for (int x = tid; x < nh * DH; x += kPvThreads) {
        const int u = x / DH;
        const int c = x - u * DH;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kPvWaves; ++w) s += red[(w * HR + u) * DH + c];
        float* dst = part + ((int64_t)(row0 + u) * nsplit + split) * (DH + 2);
        dst[2 + c] = s;
        if (c == 0) {
            dst[0] = s_m[u];
            dst[1] = s_l[u];
        }
    }
}

template <int DH>
__global__ __launch_bounds__(DH) void lse_merge(const float* __restrict__ part, int nsplit,
                                               int unit, const int32_t* __restrict__ row_cnt,
                                               const int32_t* __restrict__ lens, int64_t S_max,
                                               float* __restrict__ out, int h_q) {
    const int row = blockIdx.x;
    const int c = threadIdx.x;
    const int64_t count = row_cnt ? (int64_t)row_cnt[row] : clamp_len(lens[row / h_q], S_max);
    int64_t ns = (count + unit - 1) / unit;
    if (ns > nsplit) ns = nsplit;
    const float* p = part + (int64_t)row * nsplit * (DH + 2);
    float M = -__builtin_inff();
    for (int s = 0; s < ns; ++s)
        if (p[s * (DH + 2) + 1] > 0.f) M = fmaxf(M, p[s * (DH + 2)]);
    float num = 0.f, den = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float* q = p + s * (DH + 2);
        if (q[1] > 0.f) {
            const float f = __expf(q[0] - M);
            den += q[1] * f;
            num += q[2 + c] * f;
        }
    }
    out[(int64_t)row * DH + c] = den > 0.f ? num / den : 0.f;
}

}  // namespace

int sparse_nsplit(int N) { return (N + kPvEntries - 1) / kPvEntries; }
int dense_nsplit(int64_t S_max) { return (int)((S_max + kDenseRows - 1) / kDenseRows); }

hipError_t launch_pv_sparse(const void* v, const int32_t* sel_idx, const float* sel_val,
                            const float* row_max, const int32_t* row_cnt, float* out, int B,
                            int h_q, int h_v, int d, int N, int64_t S_max, bool bf16,
                            hipStream_t st) {
    const int total = B * h_q;
    const unsigned grid = (unsigned)(((total + 7) / 8) * 8);
#define SAGA_PV(T, D)                                                                        \
    hipLaunchKernelGGL((pv_sparse<T, D>), dim3(grid), dim3(kPvThreads), 0, st, (const T*)v,   \
                       sel_idx, sel_val, row_max, row_cnt, out, h_q, h_v, N, S_max, total)
    if (bf16) {
        if (d == 64) SAGA_PV(uint16_t, 64); else SAGA_PV(uint16_t, 128);
    } else {
        if (d == 64) SAGA_PV(float, 64); else SAGA_PV(float, 128);
    }
#undef SAGA_PV
    return hipGetLastError();
}

hipError_t launch_pv_dense(const void* v, const float* scores, int64_t s_stride,
                           const int32_t* lens, float* part, int B, int h_q, int h_v, int d,
                           int64_t S_max, bool bf16, hipStream_t st) {
    const int nsplit = dense_nsplit(S_max);
    const int g_v = h_q / h_v;
    const int ngrp = (g_v + kDenseHeads - 1) / kDenseHeads;
    dim3 grid((unsigned)nsplit, (unsigned)(B * h_v * ngrp));
#define SAGA_PVD(T, D)                                                                        \
    hipLaunchKernelGGL((pv_dense<T, D>), grid, dim3(kPvThreads), 0, st, (const T*)v, scores,  \
                       s_stride, lens, part, h_q, h_v, nsplit, S_max, ngrp)
    if (bf16) {
        if (d == 64) SAGA_PVD(uint16_t, 64); else SAGA_PVD(uint16_t, 128);
    } else {
        if (d == 64) SAGA_PVD(float, 64); else SAGA_PVD(float, 128);
    }
#undef SAGA_PVD
    return hipGetLastError();
}

hipError_t launch_merge(const float* part, int nsplit, int unit, const int32_t* row_cnt,
                        const int32_t* lens, int64_t S_max, float* out, int B, int h_q, int d,
                        hipStream_t st) {
    if (d == 64)
        hipLaunchKernelGGL((lse_merge<64>), dim3((unsigned)(B * h_q)), dim3(64), 0, st, part,
                           nsplit, unit, row_cnt, lens, S_max, out, h_q);
    else
        hipLaunchKernelGGL((lse_merge<128>), dim3((unsigned)(B * h_q)), dim3(128), 0, st, part,
                           nsplit, unit, row_cnt, lens, S_max, out, h_q);
    return hipGetLastError();
}

}  // namespace saga
