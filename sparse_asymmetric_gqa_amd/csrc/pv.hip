// Softmax weights + value gather (PV) over the kept entries.
//
// "More Value per Key" §3.1 Eq. 7: O = softmax(A[i]) V[i] -- only the kept
// value rows are read (App. C.1: gather, then a batched product), and each
// query head uses value head i / (h_q / h_v) (§3.2, App. B Eq. 29).
//
// One workgroup per (b, i) row, walking its kept list in blocks of
// kPvEntries (a whole list of up to 2048 is one block). Per block its 256
// threads stage positions and weights exp(s - m) in LDS (m = the row's
// largest kept logit), then every wave streams its share of value rows with
// 16-byte loads, LPR lanes per row, in batches of 8 rows per lane that are
// double-buffered (the next batch is in flight while one is summed); the sums
// stay in registers and the row ends with out = acc / l, so no merge pass is
// needed. The g_v heads that
// share a value head are mapped to the same XCD at neighbouring times so value
// rows they have in common are served from that XCD's L2.
#include "saga_internal.h"

namespace saga {
using namespace dev;

namespace {

constexpr int kPvThreads = 256;
constexpr int kPvWaves = kPvThreads / 64;

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
    constexpr int UNR = 8;                 // row steps per batch (one load each per lane)
    constexpr int BATCH = STEP * UNR;
    static_assert(kPvEntries % BATCH == 0, "a block is whole batches");
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
        // the block's positions and weights exp(s - m) into LDS; entries past
        // ne read row 0 with weight 0
        for (int e = tid; e < kPvEntries; e += kPvThreads) {
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
        // value rows in batches of UNR steps, double-buffered: batch j + 1 is
        // requested before batch j is used
        const int nb = (ne + BATCH - 1) / BATCH;
        u32x4 ra[UNR], rb[UNR];
        auto issue = [&](u32x4 (&dst)[UNR], int j) {
            j = j < nb ? j : nb - 1;   // past the last batch: re-read it (never used)
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                const int e = j * BATCH + first + k * STEP;
                dst[k] = *reinterpret_cast<const u32x4*>(vb + (int64_t)s_pos[e] * DH + sub * EPL);
            }
        };
        auto use = [&](const u32x4 (&src)[UNR], int j) {
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                const float wt = s_w[j * BATCH + first + k * STEP];   // 0 past ne
                float f[EPL];
                R::cvt(src[k], f);
#pragma unroll
                for (int c = 0; c < EPL; ++c) acc[c] += wt * f[c];
            }
        };
        issue(ra, 0);
#pragma unroll 1
        for (int j = 0; j < nb; j += 2) {
            issue(rb, j + 1);
            use(ra, j);
            issue(ra, j + 2);
            if (j + 1 < nb) use(rb, j + 1);   // uniform
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

}  // namespace


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

}  // namespace saga
