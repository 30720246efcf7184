// K-scan: logits s[b, i, t] = <q[b, i], K[b, kh(i), t]> / sqrt(d) for t < L_b.
//
// Eq. 2 of "More Value per Key" (§2.1) for one decode query row (§2.2 Eq. 5);
// query head i uses key head i / (h_q / h_k) (App. B Eq. 29, §3.2).
//
// The g = h_q / h_k query heads that share a key head form the N side of a
// 16x16 matrix-core tile, 16 cached positions the M side and the head
// dimension the K side, so every K row is read from HBM exactly once per call
// and reused for all g heads inside the MFMA.
//
// Memory access: a tile is 16 K rows. Lane l owns row l % 16 and, for each
// 16-byte vector v of the tile, bytes [64 v + 16 (l / 16), +16) of that row:
// one wave instruction reads 64 contiguous bytes of each of 16 rows.
//   bf16: vector v = d-elements [32 v + 8 (l/16), +8) = one 16x16x32 MFMA step
//   fp32: vector v = d-elements [16 v + 4 (l/16), +4) = four 16x16x4 steps
// The query operand uses the same lane -> d mapping, so the contraction
// covers every d exactly once whatever order the hardware sums in.
//
// Work is split into (b, key head, 1024-position chunk) items, walked by
// persistent workgroups. A streaming wave keeps NS = 2 register stages of K
// tiles in flight, consumed in rotation with no
// register copies; the last round of an item already loads the next item's
// first stages.
//
// Two kernels:
//   kscan       -- fp32 logits to a [B][h_q][stride] array (the dense baseline,
//                  the debug entry point, and key groups wider than 16 heads);
//                  four streaming waves per workgroup.
//   kscan_topm  -- the decode path: logits never leave the chip. One
//                  workgroup per CU with two roles. Four producer waves
//                  stream item t and write its logits as order-preserving keys
//                  into one of two LDS buffers; meanwhile eight consumer waves
//                  take item t-1 from the other buffer and, per query head,
//                  find a cutoff key with M <= count(key >= cutoff) (M from N
//                  and L_b) and publish every key at or above it as a
//                  position-sorted (position, key) list, with the cutoff.
//                  Every key left out is below its chunk's cutoff, which is
//                  what lets the selector prove its union result exact. The
//                  two roles meet at one barrier per item, so candidate
//                  extraction overlaps the K stream instead of stalling it.
//                  The lists are packed into the workgroup's pool range and
//                  staged in the LDS left over by the key buffers; they are
//                  written out after the last item, so list stores do not
//                  compete with the K stream.
#include "topm.h"

#include <hip/hip_ext.h>

namespace saga {
using namespace dev;

namespace {


// ---- dense mode: fp32 logits ------------------------------------------------------

template <typename T, int DH, int NHT>
__global__ __launch_bounds__(256) void kscan(const T* __restrict__ q, const T* __restrict__ k,
                                             const int32_t* __restrict__ lens,
                                             float* __restrict__ scores, int64_t s_stride,
                                             int h_q, int h_k, int64_t S_max, int nchunk,
                                             int nwork, float scale, bool vst) {
    using S = Streamer<T, DH, NHT>;
    constexpr int NS = S::NS;
    const int g = h_q / h_k;
    const int lane = threadIdx.x & 63;
    S sm(threadIdx.x >> 6, lane);

    auto len_of = [&](int b) { return lens[b]; };
    Item<T> it;
    int w = next_item<T, DH>(blockIdx.x, gridDim.x, nwork, nchunk, h_k, S_max, len_of, k, it);
    if (w >= nwork) return;
    sm.load_q(q + (int64_t)(it.b * h_q + it.kh * g) * DH, g);
#pragma unroll
    for (int s = 0; s < NS; ++s) sm.load(s, it, s);

    auto sink = [&](int ht, int r0, int off, f32x4 acc) {
        const int n = ht * 16 + sm.r16;
        float* dst = scores + (int64_t)(it.b * h_q + it.kh * g + n) * s_stride + it.c0 + off;
        if (vst && r0 + 16 <= it.n) {
            if (n < g) *reinterpret_cast<f32x4*>(dst) = acc;
        } else if (r0 < it.n) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n < g && off + e < it.n) dst[e] = acc[e];
        }
    };
#pragma unroll 1
    while (true) {
        // stages cover the chunk's rows, rounded up to a multiple of NS
        int nst = (it.n + S::STAGE - 1) / S::STAGE;
        nst = (nst + NS - 1) / NS * NS;
        // Loads are unconditional: past the chunk the rows clamp to its last row
        // (a cache hit), and straight-line loads keep the wait counts exact. The
        // first round is peeled off the loop: it is the one that waits for the
        // item's query loads, so the loop header only ever waits for one stage.
        auto round = [&](int st) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
                sm.consume(s, st + s, scale, sink, [&] { sm.load(s, it, st + s + NS); });
        };
        int st = 0;
        if (nst > NS) {
            round(0);
            st = NS;
        }
#pragma unroll 1
        for (; st < nst - NS; st += NS) round(st);
        Item<T> nx;
        const int wn = next_item<T, DH>(w + gridDim.x, gridDim.x, nwork, nchunk, h_k, S_max,
                                        len_of, k, nx);
        if (wn >= nwork) nx = it;   // re-read this item's rows; never consumed
        asm volatile("" : "+s"(st));   // keep the last round's offsets out of loop-invariant registers
#pragma unroll
        for (int s = 0; s < NS; ++s) sm.consume(s, st + s, scale, sink, [&] { sm.load(s, nx, s); });
        if (wn >= nwork) break;
        sm.load_q(q + (int64_t)(nx.b * h_q + nx.kh * g) * DH, g);
        w = wn;
        it = nx;
    }
}

// ---- top-M mode: producer / consumer workgroup --------------------------------------

// LDS layout of kscan_topm (32-bit words):
//   keys [2][g][kKeyRow]     double-buffered key rows of the current items
//   warm [g]                  previous cutoff per head
//   cursor, used, pad [4]     list cursor and end of the staged lists
//   flo [g], flo_tag [g]      lowest cutoff of the row's earlier chunks per head, its row tag
//   meta_stg [kMetaStage] uint4, meta_slot [kMetaStage]   staged metadata
//   xtile [kWaves][16 rows]   producers' transpose buffers (bf16 only)
//   stg  [..]                 staged candidate lists (uint2), the rest of the LDS
template <typename T>
constexpr bool topm_xp() { return sizeof(T) == 2; }
template <typename T, int DH, int C>
__host__ __device__ constexpr size_t topm_lds_words(int g) {
    // every area starts 16-byte aligned
    return (size_t)2 * g * key_row<C>() + ((3 * g + 4 + 3) & ~3) + 5 * kMetaStage +
           (topm_xp<T>() ? (size_t)kWaves * 16 * DH * sizeof(T) / 4 : 0);
}

template <typename T, int DH, int C>
__global__ __launch_bounds__(kTopmThreads, 1) void kscan_topm(
        const T* __restrict__ q, const T* __restrict__ k, const int32_t* __restrict__ lens,
        int h_q, int h_k, int64_t S_max, int nchunk, int nwork, float scale, TopmOut tm,
        uint32_t lds_bytes) {
    using S = Streamer<T, DH, 1, topm_xp<T>()>;
    constexpr int KR = key_row<C>();
    constexpr int NS = S::NS;
    extern __shared__ uint32_t lds[];
    const int g = h_q / h_k;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // wave-uniform
    const bool producer = wave < kWaves;
    uint32_t* keys = lds;
    uint32_t* warm = lds + 2 * g * KR;
    uint32_t* cursor = warm + g;   // cursor[0]: next free entry, cursor[1]: end of staged lists
    uint32_t* flo = cursor + 4;    // flo[g], then flo_tag[g]
    uint32_t* meta_words = lds + 2 * g * KR + ((3 * g + 4 + 3) & ~3);
    uint32_t* xtile_words = meta_words + 5 * kMetaStage;
    const uint32_t fixed_words = (uint32_t)topm_lds_words<T, DH, C>(g);

    // counters the next kernel of the call relies on starting at zero
    if (tm.zero && blockIdx.x == 0)
        for (int j = (int)threadIdx.x; j < tm.nzero; j += kTopmThreads) tm.zero[j] = 0;
    // The workgroup takes a contiguous range of items (consecutive chunks of a
    // row), so that each head's previous cutoff is a good first guess. Ranges
    // are dealt XCD-blocked: the workgroups of one XCD take consecutive ranges,
    // i.e. whole rows of the batch, and the fused select places those rows on
    // the same XCD (its lists are then read from that XCD's L2); a row's
    // costly chunks (a recency window with a long list) are spread over all
    // XCDs instead of landing on the same two.
    const int per = (nwork + gridDim.x - 1) / gridDim.x;
    const int wr = gridDim.x % 8 == 0 ? xcd_logical((int)blockIdx.x, (int)gridDim.x)
                                      : (int)blockIdx.x;
    const int wbeg = wr * per;
    const int wend = wbeg + per < nwork ? wbeg + per : nwork;
    if (wbeg >= wend) return;   // uniform over the workgroup
    // The workgroup's pool range is the regions of its items (g C entries
    // each); its lists are packed from the start of that range.
    ListSink sink;
    sink.base = (uint64_t)wbeg * g * C;
    sink.pool = tm.cand + sink.base;
    sink.stg = reinterpret_cast<uint2*>(lds + fixed_words);
    sink.cap = ((lds_bytes / 4 - fixed_words) / 2) & ~1u;
    sink.cursor = cursor;
    sink.used = cursor + 1;
    sink.meta_stg = reinterpret_cast<uint4*>(meta_words);
    sink.meta_slot = meta_words + 4 * kMetaStage;
    auto len_of = [&](int b) { return lens[b]; };   // uniform index: a scalar load

    Item<T> cur;
    int w = next_item<T, DH, C>(wbeg, 1, wend, nchunk, h_k, S_max, len_of, k, cur);
    if (w >= wend) return;   // uniform over the workgroup
    S sm(wave, lane,
         reinterpret_cast<u32x4*>(xtile_words) + (wave < kWaves ? wave : 0) * (S::TILE_BYTES / 16));
    // producers: the next item's query operand is prefetched into bqn while
    // the current item streams
    u32x4 bqn[S::NV];
    auto qrow = [&](const Item<T>& it) { return q + (int64_t)(it.b * h_q + it.kh * g) * DH; };
    if (producer) {
        sm.load_q(qrow(cur), g);
#pragma unroll
        for (int s = 0; s < NS; ++s) sm.load(s, cur, s);
    } else {
        for (int n = wave - kWaves; n < g; n += kConsumers)
            if (lane == 0) {
                warm[n] = 0u;
                flo[g + n] = 0u;   // no row yet
            }
        if (threadIdx.x == 64 * kWaves) cursor[0] = cursor[1] = 0u;
    }
    lds_barrier();

    Item<T> prev = cur;
    bool have_prev = false;
    int t = 0;
#pragma unroll 1
    while (true) {
        const bool have_cur = w < wend;
        if (!have_cur && !have_prev) break;   // uniform
        Item<T> nx = cur;
        const int wn = have_cur ? next_item<T, DH, C>(w + 1, 1, wend, nchunk, h_k, S_max, len_of, k,
                                                   nx)
                                : wend;
        if (producer && have_cur) {
            {
                uint32_t* kbuf = keys + (t & 1) * g * KR;
                {
                    const int n = sm.r16;   // next item's query operand (nx == cur after the last)
#pragma unroll
                    for (int v = 0; v < S::NV; ++v)
                        bqn[v] = n < g ? *reinterpret_cast<const u32x4*>(
                                             qrow(nx) + (int64_t)n * DH + v * 4 * S::EV +
                                             sm.grp * S::EV)
                                       : u32x4{0u, 0u, 0u, 0u};
                }
                // keys of positions past the chunk are 0, below every real key;
                // rem is opaque to the optimiser so that the per-stage offsets
                // are not hoisted out of the item loop (they would be spilled)
                auto sink = [&](int, int, int off, f32x4 acc) {
                    int rem = cur.n - off;
                    asm volatile("" : "+v"(rem));
                    if (sm.r16 < g) {
                        u32x4 kv;
#pragma unroll
                        for (int e = 0; e < 4; ++e) kv[e] = (e < rem) ? float_key(acc[e]) : 0u;
                        *reinterpret_cast<u32x4*>(&kbuf[sm.r16 * KR + off]) = kv;
                    }
                };
                // Every stage of the chunk runs, so each key row is fully
                // rewritten; rows past the chunk clamp to its last row (cache
                // hits). The first round is peeled off the loop (it waits for
                // the query operand); the last round loads the next item.
                constexpr int nst = C / S::STAGE;
                static_assert(nst % NS == 0 && nst >= 2 * NS, "chunk must span >= 2 rounds");
                auto round = [&](int st) {
#pragma unroll
                    for (int s = 0; s < NS; ++s)
                        sm.consume(s, st + s, scale, sink,
                                   [&] { sm.load(s, cur, st + s + NS); });
                };
                round(0);
                int st = NS;
#pragma unroll 1
                for (; st < nst - NS; st += NS) round(st);
                asm volatile("" : "+s"(st));
                // after the last item nx == cur: these re-reads are never consumed
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    sm.consume(s, st + s, scale, sink, [&] { sm.load(s, nx, s); });
#pragma unroll
                for (int v = 0; v < S::NV; ++v) sm.bq[0][v] = bqn[v];
            }
        }
        // The consumers extract the previous item's heads while it streams; the
        // last item, with nothing left to stream, is shared by all waves.
        if (have_prev && (!producer || !have_cur)) {
            // M: 1.5 times the chunk's expected share of the row's top N, plus
            // a margin (a heuristic: any M gives exact results, M only sets
            // how often the selector has to recompute a head)
            const float share = (float)tm.N * (float)C / (float)prev.L;
            const uint32_t M = share >= (float)(C / 2)
                                   ? (uint32_t)C
                                   : (uint32_t)__builtin_ceilf(1.5f * share) + 16u;
            uint32_t* kbuf = keys + ((t + 1) & 1) * g * KR;
            const int first = have_cur ? wave - kWaves : wave;
            const int step = have_cur ? kConsumers : kWaves + kConsumers;
#pragma unroll 1
            for (int n = first; n < g; n += step)
                extract<T, C>(prev, n, M, kbuf + n * KR, warm, sink, t - 1, lane, g, h_q,
                        nchunk, tm, prev.L, flo);
        }
        lds_barrier();   // keys of item t are complete; buffer (t - 1) & 1 is free again
        prev = cur;
        have_prev = have_cur;
        if (have_cur) {
            w = wn;
            cur = nx;
        }
        ++t;
    }
    // all lists are published: write the staged ones out (16-byte stores;
    // entries past a list's end are the alignment pads of its allocation)
    const uint32_t used = (sink.used[0] + 1u) & ~1u;
    const u32x4* s4 = reinterpret_cast<const u32x4*>(sink.stg);
    u32x4* d4 = reinterpret_cast<u32x4*>(sink.pool);
    for (uint32_t j = threadIdx.x; j < used / 2; j += kTopmThreads) d4[j] = s4[j];
    // and the staged metadata records (items 0 .. t-2 of this workgroup)
    const int nmeta = (t - 1) * g < kMetaStage ? (t - 1) * g : kMetaStage;
    for (int e = (int)threadIdx.x; e < nmeta; e += kTopmThreads)
        tm.meta[sink.meta_slot[e]] = sink.meta_stg[e];
}

template <typename T, int DH>
hipError_t go_dense(int nht, const void* q, const void* k, const int32_t* lens, float* scores,
                    int64_t s_stride, int B, int h_q, int h_k, int64_t S_max, bool vst,
                    hipStream_t st) {
    const int nchunk = (int)((S_max + kScanChunk - 1) / kScanChunk);
    const int nwork = B * h_k * nchunk;
    const float scale = (float)(1.0 / __builtin_sqrt((double)DH));
#define SAGA_KS(NH)                                                                            \
    {                                                                                          \
        auto kern = &kscan<T, DH, NH>;                                                         \
        const int grid = resident_grid(kern, 256, 0, nwork);                                   \
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, (const T*)q,         \
                           (const T*)k, lens, scores, s_stride, h_q, h_k, S_max, nchunk,       \
                           nwork, scale, vst);                                                 \
    }
    if (nht <= 1) SAGA_KS(1)
    else if (nht <= 2) SAGA_KS(2)
    else SAGA_KS(4)
#undef SAGA_KS
    return hipGetLastError();
}

template <typename T, int DH, int C>
hipError_t go_topm(const void* q, const void* k, const int32_t* lens, const TopmOut& tm, int B,
                   int h_q, int h_k, int64_t S_max, hipStream_t st, hipEvent_t ev0,
                   hipEvent_t ev1) {
    const int nchunk = (int)((S_max + C - 1) / C);
    const int nwork = B * h_k * nchunk;
    const float scale = (float)(1.0 / __builtin_sqrt((double)DH));
    auto kern = &kscan_topm<T, DH, C>;
    // the whole LDS: the key buffers, and the rest stages candidate lists
    const size_t lds = kTopmLdsBytes;
    static_assert(topm_lds_words<T, DH, C>(16) * 4 + 8 * 1024 <= kTopmLdsBytes,
                  "staging area too small");
    {   // allow > 64 KiB of dynamic LDS
        const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), lds);
        if (e != hipSuccess) return e;
    }
    const int grid = resident_grid(kern, kTopmThreads, lds, nwork);
    if (ev0 || ev1)   // events stamped with the dispatch's own start and end
        hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kTopmThreads), lds, st, ev0, ev1, 0,
                              (const T*)q, (const T*)k, lens, h_q, h_k, S_max, nchunk, nwork,
                              scale, tm, (uint32_t)lds);
    else
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kTopmThreads), lds, st, (const T*)q,
                           (const T*)k, lens, h_q, h_k, S_max, nchunk, nwork, scale, tm,
                           (uint32_t)lds);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kscan(const void* q, const void* k, const int32_t* lens, float* scores,
                        int64_t s_stride, int B, int h_q, int h_k, int d, int64_t S_max,
                        bool bf16, hipStream_t st) {
    const int nht = (h_q / h_k + 15) / 16;   // 16-head tiles: 1, 2 or 4 (g <= 64)
    const bool vst = (s_stride % 4 == 0) && ((reinterpret_cast<uintptr_t>(scores) & 15) == 0);
    if (bf16)
        return d == 64 ? go_dense<uint16_t, 64>(nht, q, k, lens, scores, s_stride, B, h_q, h_k, S_max, vst, st)
                       : go_dense<uint16_t, 128>(nht, q, k, lens, scores, s_stride, B, h_q, h_k, S_max, vst, st);
    return d == 64 ? go_dense<float, 64>(nht, q, k, lens, scores, s_stride, B, h_q, h_k, S_max, vst, st)
                   : go_dense<float, 128>(nht, q, k, lens, scores, s_stride, B, h_q, h_k, S_max, vst, st);
}

hipError_t launch_kscan_topm(const void* q, const void* k, const int32_t* lens, const TopmOut& tm,
                             int B, int h_q, int h_k, int d, int64_t S_max, bool bf16,
                             hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
#define SAGA_TM(T, D)                                                                       \
    (tm.chunk == 256   ? go_topm<T, D, 256>(q, k, lens, tm, B, h_q, h_k, S_max, st, ev0, ev1)  \
     : tm.chunk == 512 ? go_topm<T, D, 512>(q, k, lens, tm, B, h_q, h_k, S_max, st, ev0, ev1)  \
                       : go_topm<T, D, kScanChunk>(q, k, lens, tm, B, h_q, h_k, S_max, st, ev0, ev1))
    if (tm.chunk != 256 && tm.chunk != 512 && tm.chunk != kScanChunk) return hipErrorInvalidValue;
    if (bf16) return d == 64 ? SAGA_TM(uint16_t, 64) : SAGA_TM(uint16_t, 128);
    return d == 64 ? SAGA_TM(float, 64) : SAGA_TM(float, 128);
#undef SAGA_TM
}

}  // namespace saga
