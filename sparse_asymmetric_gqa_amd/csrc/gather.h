// Weighted sum of gathered value rows by one 256-thread workgroup ("More
// Value per Key" §3.1 Eq. 7: O = softmax(A[i]) V[i], only the kept value rows
// are read). Shared by the sparse value gather and the fused select + gather.
//
// The kept positions and their softmax weights sit in LDS. Every wave streams
// its share of the rows with 16-byte loads, LPR lanes per row, in batches of
// 8 rows per lane that are double-buffered (the next batch is in flight while
// one is summed). The sums stay in registers; finish() reduces them over the
// row groups and waves and writes out = acc / l.
#ifndef SAGA_GATHER_H
#define SAGA_GATHER_H
#include "saga_internal.h"

namespace saga {
namespace {
using namespace dev;

constexpr int kGatherThreads = 256;

// logical workgroup id from the hardware one: hardware ids are dealt to the 8
// XCDs round-robin, so give XCD x the contiguous logical range [x*Q, (x+1)*Q).
__device__ inline int xcd_logical(int hw, int total) {
    const int q = (total + 7) >> 3;
    return (hw & 7) * q + (hw >> 3);
}

template <typename T, int DH>
struct Gather {
    using R = Row16<T>;
    static constexpr int NW = kGatherThreads / 64;
    static constexpr int EPL = R::EPL;          // values per lane per row
    static constexpr int LPR = DH / EPL;        // lanes per value row
    static constexpr int RPI = 64 / LPR;        // rows per wave instruction
    static constexpr int STEP = NW * RPI;       // rows per workgroup step
    static constexpr int UNR = 8;               // row steps per batch
    static constexpr int BATCH = STEP * UNR;    // entries per batch (<= 256)

    // acc += sum over entries e < n of w[e] * V[pos[e]] (this lane's columns).
    // pos / w are LDS arrays readable up to the next multiple of BATCH, with
    // weight 0 (and a row < L) past n. vb points at the value head's row 0.
    __device__ static void run(const T* __restrict__ vb, const int32_t* pos, const float* w,
                               int n, float (&acc)[EPL]) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int rg = lane / LPR;
        const int sub = lane - rg * LPR;
        const int first = wave * RPI + rg;
        const int nb = (n + BATCH - 1) / BATCH;
        if (nb == 0) return;   // uniform
        u32x4 ra[UNR], rb[UNR];
        auto issue = [&](u32x4 (&dst)[UNR], int j) {
            j = j < nb ? j : nb - 1;   // past the last batch: re-read it (never used)
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                const int e = j * BATCH + first + k * STEP;
                dst[k] = *reinterpret_cast<const u32x4*>(vb + (int64_t)pos[e] * DH + sub * EPL);
            }
        };
        auto use = [&](const u32x4 (&src)[UNR], int j) {
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                const float wt = w[j * BATCH + first + k * STEP];   // 0 past n
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
    }

    // out[c] = (sum of acc over the workgroup)[c] / l; lsum is each thread's
    // share of l (summed in a fixed order). red: LDS [NW][DH] + [NW] floats.
    // With vm (nullable, [DH]): out[c] = alpha (sum / l) + (1 - alpha) vm[c].
    __device__ static void finish(float (&acc)[EPL], float lsum, float* red, float* o,
                                  float alpha = 1.f, const float* vm = nullptr) {
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int rg = lane / LPR;
        const int sub = lane - rg * LPR;
        float* s_red = red;             // [NW][DH]
        float* s_l = red + NW * DH;     // [NW]
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off, 64);
        if (lane == 0) s_l[wave] = lsum;
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
            for (int c = 0; c < EPL; ++c) acc[c] += __shfl_xor(acc[c], off, 64);
        if (rg == 0)
#pragma unroll
            for (int c = 0; c < EPL; ++c) s_red[wave * DH + sub * EPL + c] = acc[c];
        __syncthreads();
        float l = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) l += s_l[w];
        for (int c = tid; c < DH; c += kGatherThreads) {
            float sacc = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) sacc += s_red[w * DH + c];
            const float y = sacc / l;   // l >= 1: the largest kept logit has weight 1
            o[c] = vm ? alpha * y + (1.f - alpha) * vm[c] : y;
        }
    }
};

// Dot products of gathered key rows with two query vectors, in the lane layout
// of Gather: for each entry e < n of the LDS list pos, za[e] = <qa, K[pos[e]]>
// (written to LDS by the row's first lane) and zb = <qb, K[pos[e]]>. Each lane
// holds its EPL columns of qa and qb; the row's LPR lanes sum their partial
// dots by butterfly. Accumulates, per thread, se += exp(zb - shift) and
// mz = max(mz, za) over the entries whose first lane it is.
template <typename T, int DH>
struct KeyDots {
    using G = Gather<T, DH>;
    using R = typename G::R;
    static constexpr int EPL = G::EPL, LPR = G::LPR, STEP = G::STEP, UNR = G::UNR,
                         BATCH = G::BATCH, RPI = G::RPI, NW = G::NW;
    __device__ static void run(const T* __restrict__ kb, const int32_t* pos, int n,
                               const float (&qa)[EPL], const float (&qb)[EPL], float* za,
                               float shift, float& se, float& mz) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int rg = lane / LPR;
        const int sub = lane - rg * LPR;
        const int first = wave * RPI + rg;
        const int nb = (n + BATCH - 1) / BATCH;
        if (nb == 0) return;   // uniform
        u32x4 ra[UNR], rb[UNR];
        auto issue = [&](u32x4 (&dst)[UNR], int j) {
            j = j < nb ? j : nb - 1;   // past the last batch: re-read it (never used)
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                const int e = j * BATCH + first + k * STEP;
                dst[k] = *reinterpret_cast<const u32x4*>(kb + (int64_t)pos[e] * DH + sub * EPL);
            }
        };
        auto use = [&](const u32x4 (&src)[UNR], int j) {
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                const int e = j * BATCH + first + k * STEP;
                float f[EPL];
                R::cvt(src[k], f);
                float da = 0.f, db = 0.f;
#pragma unroll
                for (int c = 0; c < EPL; ++c) {
                    da = fmaf(qa[c], f[c], da);
                    db = fmaf(qb[c], f[c], db);
                }
#pragma unroll
                for (int off = 1; off < LPR; off <<= 1) {
                    da += __shfl_xor(da, off, 64);
                    db += __shfl_xor(db, off, 64);
                }
                if (sub == 0 && e < n) {
                    za[e] = da;
                    se += __expf(db - shift);
                    mz = fmaxf(mz, da);
                }
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
    }
};

}  // namespace
}  // namespace saga
#endif
