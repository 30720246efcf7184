// Softmax weights + value gather (PV) over the kept entries.
//
// "More Value per Key" §3.1 Eq. 7: O = softmax(A[i]) V[i] -- only the kept
// value rows are read (App. C.1: gather, then a batched product), and each
// query head uses value head i / (h_q / h_v) (§3.2, App. B Eq. 29).
//
// One workgroup per (b, i) row, walking its kept list in blocks of
// kPvEntries (a whole list of up to 2048 is one block). Per block its 256
// threads stage positions and weights exp(s - m) in LDS (m = the row's
// largest kept logit), then stream the value rows (gather.h); the sums stay
// in registers and the row ends with out = acc / l, so no merge pass is
// needed. The g_v heads that
// share a value head are mapped to the same XCD at neighbouring times so value
// rows they have in common are served from that XCD's L2.
#include "gather.h"

namespace saga {
using namespace dev;

namespace {

constexpr int kPvThreads = 256;


template <typename T, int DH>
__global__ __launch_bounds__(kPvThreads) void pv_sparse(
    const T* __restrict__ v, const int32_t* __restrict__ sel_idx, const float* __restrict__ sel_val,
    const float* __restrict__ row_max, const int32_t* __restrict__ row_cnt,
    float* __restrict__ out, int h_q, int h_v, int N, int64_t S_max, int total) {
    using G = Gather<T, DH>;
    static_assert(kPvThreads == kGatherThreads, "one gather workgroup per row");
    static_assert(kPvEntries % G::BATCH == 0, "a block is whole batches");
    __shared__ int32_t s_pos[kPvEntries];
    __shared__ float s_w[kPvEntries];
    __shared__ float s_red[G::NW * DH + G::NW];

    const int lid = xcd_logical((int)blockIdx.x, total);
    if (lid >= total) return;
    const int row = lid;                     // = b*h_q + i; the g_v heads of a value head are adjacent
    const int b = row / h_q;
    const int i = row - b * h_q;
    const int g_v = h_q / h_v;
    const int vh = i / g_v;
    const int cnt = row_cnt[row];
    const int tid = threadIdx.x;
    float* o = out + (int64_t)row * DH;
    if (cnt <= 0) {   // no kept entry (L_b = 0): out = 0
        for (int c = tid; c < DH; c += kPvThreads) o[c] = 0.f;
        return;
    }
    const float m = row_max[row];
    const T* vb = v + (int64_t)(b * h_v + vh) * S_max * DH;
    float acc[G::EPL];
#pragma unroll
    for (int c = 0; c < G::EPL; ++c) acc[c] = 0.f;
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
        G::run(vb, s_pos, s_w, ne, acc);
        __syncthreads();   // the block's LDS lists are reused by the next block
    }
    G::finish(acc, lsum, s_red, o);
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
