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
// Pipeline: two register stages of kTilesPerStage tiles each are in flight
// per wave (ping-pong, no register copies), so a wave never waits for the
// loads it has just issued. Workgroups loop over (key head, chunk) work items
// so their start-up cost is paid once per workgroup, not once per chunk.
//
// Two output modes:
//   dense  -- fp32 logits to a [B][h_q][stride] array (the dense baseline, the
//             debug entry point, and key groups wider than one 16-head tile);
//   top-M  -- logits stay on chip: as order-preserving keys in LDS, then for
//             each query head a cutoff key with M <= count(key >= cutoff) (M
//             from N and L_b) is found by bisection over the key bits, and every
//             key at or above it is published as a position-sorted (position,
//             key) list, with the cutoff. Every key left out is below its
//             chunk's cutoff, which is what lets the selector prove its union
//             result exact.
//
// Work items are software-pipelined: the next item's query and first K stages
// are loaded before the current item's candidates are published, and the
// LDS-reuse barriers wait on LDS only, so no wave ever waits for its own
// global stores to drain.
#include "saga_internal.h"

namespace saga {
using namespace dev;

namespace {

#ifndef SAGA_KSCAN_U
#define SAGA_KSCAN_U 1
#endif
#ifndef SAGA_KSCAN_NT
#define SAGA_KSCAN_NT 1
#endif
constexpr int kWaves = 4;
constexpr int kTilesPerStage = SAGA_KSCAN_U;

// K rows are read exactly once per call: mark the loads non-temporal.
template <typename V>
__device__ inline V load_stream(const V* p) {
#if SAGA_KSCAN_NT
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

template <typename T> struct Mfma;
template <> struct Mfma<uint16_t> {
    __device__ static inline f32x4 step(const u32x4& a, const u32x4& b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    __device__ static inline f32x4 step(const u32x4& a, const u32x4& b, f32x4 c) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[j]), __uint_as_float(b[j]),
                                                     c, 0, 0, 0);
        return c;
    }
};

// LDS-only barrier: orders LDS accesses of the workgroup without waiting for
// outstanding global stores (a __syncthreads() would also drain those).
__device__ inline void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt / expcnt left as they are
    __builtin_amdgcn_s_barrier();
}

struct Item {
    int bkh, b, kh, chunk;
    int64_t L, c0, c1;
};

template <typename T, int DH, int NHT, bool TOPM>
__global__ __launch_bounds__(256, (TOPM && sizeof(T) == 2) ? 3 : 1) void kscan(const T* __restrict__ q, const T* __restrict__ k,
                                             const int32_t* __restrict__ lens,
                                             float* __restrict__ scores, int64_t s_stride,
                                             int h_q, int h_k, int64_t S_max, int nchunk,
                                             int nwork, float scale, bool vst, TopmOut tm) {
    extern __shared__ uint32_t lds_keys[];   // top-M: [g][kScanChunk] keys of the chunk
    constexpr int NV = DH * (int)sizeof(T) / 64;   // 16-byte vectors per lane per tile
    constexpr int EV = 16 / (int)sizeof(T);        // elements per vector
    constexpr int U = kTilesPerStage;
    constexpr int STAGE = kWaves * U * 16;         // positions per stage of the workgroup
    const int g = h_q / h_k;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15;
    const int grp = lane >> 4;

    // first work item at or after w whose chunk starts inside its row
    auto next_item = [&](int w, Item& it) -> int {
        for (; w < nwork; w += gridDim.x) {
            it.bkh = w / nchunk;
            it.chunk = w - it.bkh * nchunk;
            it.b = it.bkh / h_k;
            it.kh = it.bkh - it.b * h_k;
            it.L = clamp_len(lens[it.b], S_max);
            it.c0 = (int64_t)it.chunk * kScanChunk;
            if (it.c0 < it.L) {
                it.c1 = it.c0 + kScanChunk < it.L ? it.c0 + kScanChunk : it.L;
                return w;
            }
        }
        return nwork;
    };

    u32x4 bq[NHT][NV];
    u32x4 A[U][NV], Bv[U][NV];
    auto load_q = [&](const Item& it) {
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
            const int n = ht * 16 + r16;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                bq[ht][v] = u32x4{0u, 0u, 0u, 0u};
                if (n < g)
                    bq[ht][v] = *reinterpret_cast<const u32x4*>(
                        q + (int64_t)(it.b * h_q + it.kh * g + n) * DH + v * 4 * EV + grp * EV);
            }
        }
    };
    auto load = [&](u32x4 (&dst)[U][NV], const Item& it, int st) {
        const T* kb = k + (int64_t)it.bkh * S_max * DH + grp * EV;
        const int64_t last = it.c1 - 1;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t row = it.c0 + 16 * (int64_t)(wave + kWaves * (u + U * st)) + r16;
            row = row < last ? row : last;
            const T* src = kb + row * DH;
#pragma unroll
            for (int v = 0; v < NV; ++v)
                dst[u][v] = load_stream(reinterpret_cast<const u32x4*>(src + v * 4 * EV));
        }
    };
    auto consume = [&](const u32x4 (&src)[U][NV], const Item& it, int st) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t0 = it.c0 + 16 * (int64_t)(wave + kWaves * (u + U * st));
            const int64_t p = t0 + 4 * grp;
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int v = 0; v < NV; ++v) acc = Mfma<T>::step(src[u][v], bq[ht][v], acc);
                acc = acc * scale;
                const int n = ht * 16 + r16;
                if (TOPM) {
                    // keys of positions past the chunk are 0, below every real key
                    const int off = (int)(p - it.c0);
                    if (n < g && off < kScanChunk) {
                        u32x4 kv;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            kv[e] = (p + e < it.c1) ? float_key(acc[e]) : 0u;
                        *reinterpret_cast<u32x4*>(&lds_keys[n * kScanChunk + off]) = kv;
                    }
                } else {
                    float* dst = scores + (int64_t)(it.b * h_q + it.kh * g + n) * s_stride + p;
                    if (vst && t0 + 16 <= it.c1) {
                        if (n < g) *reinterpret_cast<f32x4*>(dst) = acc;
                    } else if (t0 < it.c1) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n < g && p + e < it.c1) dst[e] = acc[e];
                    }
                }
            }
        }
    };

    // Candidate extraction for one head (TOPM): the wave reads the head's keys
    // (position lane + 64 e, conflict-free) into registers and finds a cutoff by
    // MSB-first bisection on the key: count(key >= x) comes from ballots and
    // scalar popcounts, so the search needs no LDS traffic and no atomics. It
    // stops at the first prefix with M <= count <= M + M/8 (or at 20 bits). Every
    // key >= cutoff is then staged in the head's LDS row in ascending position
    // order and written out with 16-byte stores.
    auto extract = [&](const Item& it, int n, uint32_t M) {
        const int nvalid = (int)(it.c1 - it.c0);
        uint32_t* row = &lds_keys[n * kScanChunk];
        uint32_t kk[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int j = lane + 64 * e;
            kk[e] = j < nvalid ? row[j] : 0u;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // keys are in registers before the row is reused
        uint32_t cut = 0;   // publish everything when the chunk holds <= M keys
        if ((uint32_t)nvalid > M) {
            const uint32_t hi = M + (M >> 3);
            uint32_t prefix = 0;
#pragma unroll 1
            for (int bit = 31; bit >= 12; --bit) {
                const uint32_t x = prefix | (1u << bit);
                uint32_t cnt = 0;
#pragma unroll
                for (int e = 0; e < 16; ++e) cnt += (uint32_t)__popcll(ballot(kk[e] >= x));
                if (cnt >= M) {
                    prefix = x;
                    if (cnt <= hi) break;
                }
            }
            cut = prefix;
        }
        const int64_t slot = ((int64_t)(it.b * h_q + it.kh * g + n) * nchunk + it.chunk);
        uint2* dst = tm.cand + slot * kScanChunk;
        uint2* stage = reinterpret_cast<uint2*>(row);   // 512 entries
        uint32_t base = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const bool keep = kk[e] != 0u && kk[e] >= cut;
            const uint64_t m = ballot(keep);
            if (keep) {
                const uint32_t at = base + lanes_below(m);
                const uint2 v = make_uint2((uint32_t)(it.c0 + lane + 64 * e), kk[e]);
                if (at < kScanChunk / 2) stage[at] = v; else dst[at] = v;
            }
            base += (uint32_t)__popcll(m);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        const uint32_t staged = base < kScanChunk / 2 ? base : kScanChunk / 2;
        for (uint32_t j = 2 * lane; j < staged; j += 128) {
            u32x4 v2;
            const uint2 a0 = stage[j];
            const uint2 a1 = j + 1 < staged ? stage[j + 1] : make_uint2(0u, 0u);
            v2[0] = a0.x; v2[1] = a0.y; v2[2] = a1.x; v2[3] = a1.y;
            *reinterpret_cast<u32x4*>(dst + j) = v2;   // dst + j is 16-byte aligned (j even)
        }
        if (lane == 0) {
            tm.cnt[slot] = (int32_t)base;
            tm.cut[slot] = cut;
        }
    };

    Item it;
    int w = next_item(blockIdx.x, it);
    if (w >= nwork) return;
    load_q(it);
    load(A, it, 0);
    load(Bv, it, 1);
#pragma unroll 1
    while (true) {
        // stages cover [c0, c1); an even count keeps the ping-pong loop simple
        int nst = (int)((it.c1 - it.c0 + STAGE - 1) / STAGE);
        nst += nst & 1;
#pragma unroll 1
        for (int st = 0; st < nst; st += 2) {
            // unconditional: past the chunk the rows clamp to its last row (a
            // cache hit), and straight-line loads keep the wait counts exact
            consume(A, it, st);
            load(A, it, st + 2);
            consume(Bv, it, st + 1);
            load(Bv, it, st + 3);
        }
        // issue the next item's loads before this item's publishing stores, so
        // that waiting for them never waits for the stores
        Item nx;
        const int wn = next_item(w + gridDim.x, nx);
        if (wn < nwork) {
            load_q(nx);
            load(A, nx, 0);
            load(Bv, nx, 1);
        }
        if (TOPM) {
            lds_barrier();   // all keys of the chunk are in LDS
            int64_t expct = ((int64_t)tm.N * kScanChunk + it.L - 1) / it.L;
            int64_t M64 = 2 * expct + 32;   // twice the chunk's expected share, plus a margin
            const uint32_t M = (uint32_t)(M64 < kScanChunk ? M64 : kScanChunk);
#pragma unroll 1
            for (int n = wave; n < g; n += kWaves) extract(it, n, M);
            lds_barrier();   // LDS is rewritten by the next item
        }
        if (wn >= nwork) break;
        w = wn;
        it = nx;
    }
}

int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Persistent grid: as many workgroups as can be resident at once (so none of
// them waits for another to finish all of its work before starting), at most
// one per work item. Residency per CU is queried once per kernel and LDS size.
template <typename K>
int resident_grid(K kern, size_t lds, int nwork) {
    static int cached_lds[8] = {-1, -1, -1, -1, -1, -1, -1, -1};
    static int cached_blocks[8] = {0};
    int per_cu = 0;
    for (int i = 0; i < 8; ++i)
        if (cached_lds[i] == (int)lds) per_cu = cached_blocks[i];
    if (per_cu == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, lds) != hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        for (int i = 0; i < 8; ++i)
            if (cached_lds[i] < 0) {
                cached_lds[i] = (int)lds;
                cached_blocks[i] = per_cu;
                break;
            }
    }
    const int grid = cu_count() * per_cu;
    return grid < nwork ? grid : nwork;
}

template <typename T, int DH>
hipError_t go(int nht, const void* q, const void* k, const int32_t* lens, float* scores,
              int64_t s_stride, int B, int h_q, int h_k, int64_t S_max, bool vst,
              const TopmOut* tm, hipStream_t st) {
    const int nchunk = (int)((S_max + kScanChunk - 1) / kScanChunk);
    const int nwork = B * h_k * nchunk;
    const float scale = (float)(1.0 / __builtin_sqrt((double)DH));
    const TopmOut none{};
    if (tm) {
        // top-M mode: one 16-head tile (g <= 16), keys of the chunk in LDS
        auto kern = &kscan<T, DH, 1, true>;
        const size_t lds = (size_t)(h_q / h_k) * kScanChunk * sizeof(uint32_t);
        static bool attr_set = false;   // one per instantiation: allow > 64 KiB of dynamic LDS
        if (!attr_set) {
            if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)(16 * kScanChunk * sizeof(uint32_t))) != hipSuccess)
                return hipGetLastError();
            attr_set = true;
        }
        const int grid = resident_grid(kern, lds, nwork);
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, st, (const T*)q,
                           (const T*)k, lens, nullptr, 0, h_q, h_k, S_max, nchunk, nwork, scale,
                           false, *tm);
        return hipGetLastError();
    }
#define SAGA_KS(NH)                                                                            \
    {                                                                                          \
        auto kern = &kscan<T, DH, NH, false>;                                                  \
        const int grid = resident_grid(kern, 0, nwork);                                        \
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, (const T*)q,         \
                           (const T*)k, lens, scores, s_stride, h_q, h_k, S_max, nchunk,       \
                           nwork, scale, vst, none);                                           \
    }
    if (nht <= 1) SAGA_KS(1)
    else if (nht <= 2) SAGA_KS(2)
    else SAGA_KS(4)
#undef SAGA_KS
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kscan(const void* q, const void* k, const int32_t* lens, float* scores,
                        int64_t s_stride, int B, int h_q, int h_k, int d, int64_t S_max,
                        bool bf16, hipStream_t st) {
    const int nht = (h_q / h_k + 15) / 16;   // 16-head tiles: 1, 2 or 4 (g <= 64)
    const bool vst = (s_stride % 4 == 0) && ((reinterpret_cast<uintptr_t>(scores) & 15) == 0);
    if (bf16)
        return d == 64 ? go<uint16_t, 64>(nht, q, k, lens, scores, s_stride, B, h_q, h_k, S_max, vst, nullptr, st)
                       : go<uint16_t, 128>(nht, q, k, lens, scores, s_stride, B, h_q, h_k, S_max, vst, nullptr, st);
    return d == 64 ? go<float, 64>(nht, q, k, lens, scores, s_stride, B, h_q, h_k, S_max, vst, nullptr, st)
                   : go<float, 128>(nht, q, k, lens, scores, s_stride, B, h_q, h_k, S_max, vst, nullptr, st);
}

hipError_t launch_kscan_topm(const void* q, const void* k, const int32_t* lens, const TopmOut& tm,
                             int B, int h_q, int h_k, int d, int64_t S_max, bool bf16,
                             hipStream_t st) {
    if (bf16)
        return d == 64 ? go<uint16_t, 64>(1, q, k, lens, nullptr, 0, B, h_q, h_k, S_max, false, &tm, st)
                       : go<uint16_t, 128>(1, q, k, lens, nullptr, 0, B, h_q, h_k, S_max, false, &tm, st);
    return d == 64 ? go<float, 64>(1, q, k, lens, nullptr, 0, B, h_q, h_k, S_max, false, &tm, st)
                   : go<float, 128>(1, q, k, lens, nullptr, 0, B, h_q, h_k, S_max, false, &tm, st);
}

}  // namespace saga
