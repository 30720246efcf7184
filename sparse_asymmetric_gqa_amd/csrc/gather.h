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
        // Whole pairs of batches per iteration, both summed unconditionally,
        // and scheduling barriers between the phases: a batch's loads are then
        // issued before the other batch's sums (a conditional sum lets the
        // compiler move its loads down into it, and every batch would wait
        // for all loads in flight). An odd last batch is summed after the loop.
        issue(ra, 0);
#pragma unroll 1
        for (int j = 0; j + 1 < nb; j += 2) {
            issue(rb, j + 1);
            __builtin_amdgcn_sched_barrier(0);
            use(ra, j);
            __builtin_amdgcn_sched_barrier(0);
            issue(ra, j + 2);
            __builtin_amdgcn_sched_barrier(0);
            use(rb, j + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (nb & 1) use(ra, nb - 1);   // uniform
    }

    // Sums of acc over the workgroup, written to dst[0 .. DH) (global memory,
    // not yet divided by l) with device-scope stores, which write through the
    // XCD's L2: one part of a row whose kept list is gathered by several
    // workgroups. red: LDS [NW][DH] floats.
    __device__ static void partial(float (&acc)[EPL], float* red, float* dst) {
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int rg = lane / LPR;
        const int sub = lane - rg * LPR;
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
            for (int c = 0; c < EPL; ++c) acc[c] += __shfl_xor(acc[c], off, 64);
        if (rg == 0)
#pragma unroll
            for (int c = 0; c < EPL; ++c) red[wave * DH + sub * EPL + c] = acc[c];
        __syncthreads();
        for (int c = tid; c < DH; c += kGatherThreads) {
            float sacc = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) sacc += red[w * DH + c];
            __hip_atomic_store(dst + c, sacc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // The row's output from its nparts (1 .. kMaxSplit) partial sums src[p][DH] (written by
    // other workgroups with device-scope stores, read here with device-scope
    // loads, which do not hit a stale line of this XCD's L2), added in part
    // order: out[c] = (sum_p src[p][c]) / l, with l reduced from the threads'
    // shares lsum as in finish(). red: LDS [NW] floats.
    __device__ static void merge(float lsum, float* red, const float* src, int nparts, float* o) {
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off, 64);
        if (lane == 0) red[wave] = lsum;
        __syncthreads();
        float l = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) l += red[w];
        for (int c = tid; c < DH; c += kGatherThreads) {
            // all parts are requested before the first is added, so the row
            // waits for one memory round trip rather than one per part; part
            // indices past nparts re-read the last part and are not added
            float v[kMaxSplit];
#pragma unroll
            for (int p = 0; p < kMaxSplit; ++p)
                v[p] = __hip_atomic_load(src + (p < nparts ? p : nparts - 1) * DH + c,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            float sacc = 0.f;
#pragma unroll
            for (int p = 0; p < kMaxSplit; ++p)
                if (p < nparts) sacc += v[p];
            o[c] = sacc / l;
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

// The value gather of one row whose kept list is staged in LDS: positions
// st_idx and softmax weights st_w for entries [0, n), zero weights (position
// 0) on [n, nst), nst a multiple of Gather::BATCH. With nsplit == 1 the
// workgroup gathers the whole list and writes o = sum / l. With nsplit > 1
// it is part `part` of the row: it gathers the slice of whole batches
// [part * per, (part + 1) * per) of the list, stores its partial sums in
// split_part [row][nsplit][DH], and the part that finishes last (counted in
// split_cnt[row], which starts at 0) adds the partials in part order and
// writes o, so the bits do not depend on which part that is. l is summed from
// the staged weights slot by slot in every part. red: LDS [NW][DH] + [NW]
// floats; bcast: one LDS word. Every thread of the workgroup calls this.
// The parts hand over through device-scope accesses only: the partial sums
// are stored at device scope and every store has completed (vmcnt 0) before
// the part's counter increment is issued; the last part reads them at device
// scope after its increment returned. (An agent-scope fence would also write
// back and invalidate the whole L2 of the XCD, which costs every workgroup
// on it far more than these few hundred bytes.)
template <typename T, int DH>
__device__ __forceinline__ void gather_staged(const T* __restrict__ vb, const int32_t* st_idx, const float* st_w,
                              int n, int nst, float* red, uint32_t* bcast, int row, int part,
                              int nsplit, float* __restrict__ split_part,
                              int32_t* __restrict__ split_cnt, float* __restrict__ o) {
    using G = Gather<T, DH>;
    const int tid = threadIdx.x;
    float lsum = 0.f;
    for (int j = tid; j < nst; j += kGatherThreads) lsum += st_w[j];
    float acc[G::EPL];
#pragma unroll
    for (int c = 0; c < G::EPL; ++c) acc[c] = 0.f;
    if (nsplit == 1) {
        G::run(vb, st_idx, st_w, n, acc);
        G::finish(acc, lsum, red, o);
        return;
    }
    // whole batches per part, so that the gather's reads past a slice stay
    // inside the staged, zero-weighted entries
    const int per = ((n + nsplit - 1) / nsplit + G::BATCH - 1) / G::BATCH * G::BATCH;
    const int e_lo = part * per < n ? part * per : n;
    const int e_hi = e_lo + per < n ? e_lo + per : n;
    G::run(vb, st_idx + e_lo, st_w + e_lo, e_hi - e_lo, acc);
    G::partial(acc, red, split_part + ((int64_t)row * nsplit + part) * DH);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's stores have completed
    __syncthreads();                      // ... and every other thread's
    if (tid == 0)
        *bcast = (uint32_t)__hip_atomic_fetch_add(split_cnt + row, 1, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*bcast == (uint32_t)(nsplit - 1))   // uniform: the last part merges
        G::merge(lsum, red, split_part + (int64_t)row * nsplit * DH, nsplit, o);
}

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
        issue(ra, 0);   // pairs of batches, phases in order, as in Gather::run
#pragma unroll 1
        for (int j = 0; j + 1 < nb; j += 2) {
            issue(rb, j + 1);
            __builtin_amdgcn_sched_barrier(0);
            use(ra, j);
            __builtin_amdgcn_sched_barrier(0);
            issue(ra, j + 2);
            __builtin_amdgcn_sched_barrier(0);
            use(rb, j + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (nb & 1) use(ra, nb - 1);   // uniform
    }
};

}  // namespace
}  // namespace saga
#endif
