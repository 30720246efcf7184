// K streaming shared by the K-scan kernels and the fused dense kernel: the
// matrix-core step, the LDS-only barrier, work items and the streaming wave
// (Streamer). Included by one translation unit each; everything here has
// internal linkage.
//
// The g = h_q / h_k query heads that share a key head form the N side of a
// 16x16 matrix-core tile, 16 cached positions the M side and the head
// dimension the K side ("More Value per Key" §2.1 Eq. 2, App. B Eq. 29), so
// every K row is read from HBM once and reused for all g heads.
#ifndef SAGA_KSTREAM_H
#define SAGA_KSTREAM_H
#include "saga_internal.h"

namespace saga {
namespace {
using namespace dev;

#ifndef SAGA_KSCAN_U
#define SAGA_KSCAN_U 1
#endif
#ifndef SAGA_KSCAN_NT
#define SAGA_KSCAN_NT 1
#endif
constexpr int kWaves = 4;          // streaming waves per workgroup
constexpr int kTilesPerStage = SAGA_KSCAN_U;
// Register stages in flight per streaming wave. Two measured faster than four
// on the top-M K-scan (more loads in flight only raised their latency).
__host__ __device__ constexpr int stages_for(int) { return 2; }

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
// outstanding global loads or stores (a __syncthreads() would also drain those).
__device__ inline void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt / expcnt left as they are
    __builtin_amdgcn_s_barrier();
}

// One (b, key head, chunk) work item. Positions fit in int: S_max is capped on
// the host at INT32_MAX / 2.
template <typename T>
struct Item {
    const T* kb;       // K row c0 of this (b, kh)
    int bkh, b, kh, chunk;
    int L, c0, n;      // cached length, first position, positions in the chunk
};

// First work item at or after w (stepping by `step`) whose chunk of C
// positions starts inside its row; returns nwork when there is none.
template <typename T, int DH, int C = kScanChunk, typename LenOf>
__device__ inline int next_item(int w, int step, int nwork, int nchunk, int h_k, int64_t S_max,
                                LenOf&& len_of, const T* __restrict__ k, Item<T>& it) {
    for (; w < nwork; w += step) {
        it.bkh = w / nchunk;
        it.chunk = w - it.bkh * nchunk;
        it.b = it.bkh / h_k;
        it.kh = it.bkh - it.b * h_k;
        it.L = (int)clamp_len(len_of(it.b), S_max);
        it.c0 = it.chunk * C;
        if (it.c0 < it.L) {
            it.n = it.L - it.c0 < C ? it.L - it.c0 : C;
            it.kb = k + ((int64_t)it.bkh * S_max + it.c0) * DH;
            return w;
        }
    }
    return nwork;
}

// The streaming side shared by both kernels: wave `sw` (0..kWaves-1) of the
// streaming group loads and multiplies tiles 16 * (sw + kWaves * (u + U * st))
// of an item, st = stage index.
//
// XP = false: each lane loads its MFMA operand straight from HBM (lane l: row
// l % 16, 16-byte chunk 4 v + l / 16 of it), so one load instruction covers
// 64 bytes of each of 16 rows.
// XP = true: loads are row-coalesced -- instruction v covers RPI whole rows,
// lane l taking 16-byte chunk l % CPR of row RPI v + l / CPR -- and the tile
// is transposed into the MFMA layout through a per-wave LDS buffer of 16 rows.
// Slot (r, c) of that buffer is r CPR + (c ^ h(r)): with h(r) = r (CPR >= 16)
// or (r / 2) % 8 (CPR = 8), both the row-wise writes and the column-wise
// MFMA reads touch 16 distinct 16-byte bank groups per 16 lanes. Row-coalesced
// loads read HBM faster (6.9 vs 6.1 TB/s in a plain read test).
template <typename T, int DH, int NHT, bool XP = false>
struct Streamer {
    static constexpr int NV = DH * (int)sizeof(T) / 64;   // 16-byte vectors per lane per tile
    static constexpr int EV = 16 / (int)sizeof(T);        // elements per vector
    static constexpr int U = kTilesPerStage;
    static constexpr int NS = stages_for(NV);
    static constexpr int STAGE = kWaves * U * 16;         // positions per stage
    static constexpr int RB = DH * (int)sizeof(T);        // bytes per K row
    static constexpr int CPR = RB / 16;                   // 16-byte chunks per row
    static constexpr int RPI = 64 / CPR;                  // rows per coalesced instruction
    static constexpr int TILE_BYTES = 16 * RB;            // LDS transpose buffer per wave
    static_assert(!XP || (CPR >= 8 && CPR <= 32), "row layout not supported");

    int sw, r16, grp;
    u32x4 bq[NHT][NV];
    u32x4 buf[NS][U][NV];
    u32x4* tile;   // XP: this wave's LDS transpose buffer (16 rows)

    __device__ Streamer(int sw_, int lane, u32x4* tile_ = nullptr)
        : sw(sw_), r16(lane & 15), grp(lane >> 4), tile(tile_) {}

    __device__ static inline int slot(int r, int c) {
        const int h = CPR >= 16 ? r : ((r >> 1) & 7);
        return r * CPR + (c ^ h);
    }

    // Query operand from a [g][DH] array (global or LDS); heads >= g are 0.
    __device__ inline void load_q(const T* qrow0, int g) {
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
            const int n = ht * 16 + r16;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                bq[ht][v] = u32x4{0u, 0u, 0u, 0u};
                if (n < g)
                    bq[ht][v] = *reinterpret_cast<const u32x4*>(qrow0 + (int64_t)n * DH +
                                                                 v * 4 * EV + grp * EV);
            }
        }
    }
    // 32-bit byte offsets from the item's uniform base (at most one chunk of rows)
    __device__ inline void load(int s, const Item<T>& it, int st) {
        const char* kb = reinterpret_cast<const char*>(it.kb);
        const int last = it.n - 1;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r0 = 16 * (sw + kWaves * (u + U * st));
            if (XP) {
                const int lane = grp * 16 + r16;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    int row = r0 + RPI * v + lane / CPR;
                    row = row < last ? row : last;
                    buf[s][u][v] = load_stream(reinterpret_cast<const u32x4*>(
                        kb + (uint32_t)row * RB + (uint32_t)(lane % CPR) * 16));
                }
            } else {
                int row = r0 + r16;
                row = row < last ? row : last;
                const uint32_t off = (uint32_t)(row * DH + grp * EV) * (uint32_t)sizeof(T);
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    buf[s][u][v] = load_stream(reinterpret_cast<const u32x4*>(
                        kb + off + v * 4 * EV * (int)sizeof(T)));
            }
        }
    }
    // Tile u of stage buffer s: acc[e] = scaled logit of head ht*16 + r16 at
    // chunk offset r0 + 4 grp + e, handed to sink(ht, r0, off, acc) with
    // off = r0 + 4 grp (the tile's first row r0 = 16 (sw + kWaves (u + U st))).
    // refill() reloads stage buffer s; it is called as soon as the buffer's
    // registers are free (after the LDS write with XP, after the MFMAs
    // without), so the next loads are issued before this stage's MFMAs.
    template <typename Sink, typename Refill>
    __device__ inline void consume(int s, int st, float scale, Sink&& sink, Refill&& refill) {
        static_assert(!XP || U == 1, "the transpose buffer holds one tile");
        if (XP) {
            const int r0 = 16 * (sw + kWaves * (U * st));
            // row-major 16-byte chunks in, MFMA operand layout out (the wave's
            // LDS operations complete in order)
            const int lane = grp * 16 + r16;
#pragma unroll
            for (int v = 0; v < NV; ++v)
                tile[slot(RPI * v + lane / CPR, lane % CPR)] = buf[s][0][v];
            refill();
            u32x4 a[NV];
#pragma unroll
            for (int v = 0; v < NV; ++v) a[v] = tile[slot(r16, 4 * v + grp)];
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int v = 0; v < NV; ++v) acc = Mfma<T>::step(a[v], bq[ht][v], acc);
                sink(ht, r0, r0 + 4 * grp, acc * scale);
            }
            return;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r0 = 16 * (sw + kWaves * (u + U * st));
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int v = 0; v < NV; ++v) acc = Mfma<T>::step(buf[s][u][v], bq[ht][v], acc);
                sink(ht, r0, r0 + 4 * grp, acc * scale);
            }
        }
        refill();
    }
};

}  // namespace
}  // namespace saga
#endif
