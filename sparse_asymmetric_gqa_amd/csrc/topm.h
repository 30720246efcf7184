// Top-M candidate extraction shared by the K-scan kernels that keep logits
// on chip (kscan_topm, sparq_topm): the consumer side of the producer /
// consumer workgroup, its list sink, and the persistent-grid helpers.
#ifndef SAGA_TOPM_H
#define SAGA_TOPM_H
#include "kstream.h"

namespace saga {
using namespace dev;

namespace {

constexpr int kConsumers = 8;      // extracting waves of kscan_topm
constexpr int kTopmThreads = 64 * (kWaves + kConsumers);
// Candidates of one head staged in its own LDS row before the global write:
// entries [0, stage_max) hold data, [stage_max, stage_max + 64) are per-lane
// sinks for the branch-free writes of entries that are not kept.
template <int C> constexpr uint32_t stage_max() { return C / 2 - 64; }
// Words per head key row in LDS: one 16-byte slot beyond the chunk, so that
// the 16 heads written by one 16-lane store start in distinct bank groups
// (rows exactly 4 KiB apart would put all 16 lanes on one bank).
template <int C> constexpr int key_row() { return C + 4; }
constexpr int kKeyRow = key_row<kScanChunk>();
constexpr size_t kTopmLdsBytes = 160 * 1024;   // LDS of a gfx950 CU: one workgroup per CU

// Candidate extraction of head n of item `it` by one consumer wave, from the
// head's key row in LDS (every offset of the row was written for this item, 0
// past the chunk's end). Lane l takes offsets [KPL l, KPL l + KPL), KPL = C / 64,
// so lane order is position order. The cutoff is a key with M <= count(key >= cutoff) <=
// M + M/4 where one is found within a bracket of 2^12, else the largest probed
// key with count >= M. The search starts from the cutoff this wave found for
// the same head on its previous item (the workgroup walks consecutive chunks
// of a row, so that is usually close), gallops away from it and bisects;
// without a previous cutoff it bisects the whole key range. Counts are
// scalar popcounts of per-key lane masks. Positions at or after
// local_from (a window the caller keeps anyway) count in the chunk statistics
// but are left out of the ranking and of the list.
// The keys at or above the cutoff are then written in position order: a
// prefix scan of the per-lane counts gives each lane its first slot.
// Destination of the candidate lists of one workgroup: the workgroup's pool
// range (entries from `base`), filled in order through an LDS cursor; the
// first `cap` entries are staged in LDS (`stg`) and written out once, at the
// end of the kernel, so that no list store competes with the K stream.
struct ListSink {
    uint2* pool;        // global: the workgroup's range
    uint64_t base;      // its first entry (absolute index into the pool)
    uint2* stg;         // LDS staging of entries [0, cap)
    uint32_t cap;
    uint32_t* cursor;   // LDS: next free entry (relative to base)
    uint32_t* used;     // LDS: end of the staged lists
    uint4* meta_stg;    // LDS: metadata records of the first kMetaStage (item, head) pairs
    uint32_t* meta_slot;   // LDS: their slots
};
constexpr int kMetaStage = 256;

//
// Row floor (flo != nullptr): flo[n] holds the lowest cutoff of the earlier
// chunks of the same (b, key head) row that this workgroup extracted, tagged
// in flo_tag[n] = 1 + b h_q + kh g (flo_tag = flo + g). A chunk whose cutoff
// lies above that floor publishes every key down to the floor instead: a
// chunk that holds more of the row's top keys than its M suggest (a recency
// window, a block of sinks) then needs no recompute in the selector, while a
// chunk like its neighbours gains only the few keys between the two cutoffs.
// Any cutoff keeps the result exact: every key left out is still below the
// cutoff the chunk publishes.
template <typename T, int C = kScanChunk>
__device__ inline void extract(const Item<T>& it, int n, uint32_t M, uint32_t* row,
                               uint32_t* warm, const ListSink& sink, int local, int lane, int g,
                               int h_q, int nchunk, const TopmOut& tm, int local_from,
                               uint32_t* flo = nullptr) {
    constexpr int KPL = C / 64;   // keys per lane
    static_assert(KPL % 4 == 0, "lanes read whole 16-byte key groups");
    constexpr uint32_t kStageMax = stage_max<C>();
    uint32_t kk[KPL];
#pragma unroll
    for (int j = 0; j < KPL / 4; ++j) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(row + KPL * lane + 4 * j);
#pragma unroll
        for (int c = 0; c < 4; ++c) kk[4 * j + c] = v[c];
    }
    const uint32_t guess = warm[n];
    __builtin_amdgcn_s_waitcnt(0xc07f);   // keys are in registers before the row is reused
    if (tm.stat) {   // uniform
        // the chunk's softmax statistics for this head: its largest logit and
        // the sum of exp(logit - largest); empty slots hold key 0, below
        // every real key, and are left out of the sum
        uint32_t kx = 0;
#pragma unroll
        for (int e = 0; e < KPL; ++e) kx = kk[e] > kx ? kk[e] : kx;
        const float mx = key_float(wave_umax(kx));
        float se = 0.f;
#pragma unroll
        for (int e = 0; e < KPL; ++e) se += kk[e] != 0u ? __expf(key_float(kk[e]) - mx) : 0.f;
        se = wave_fsum(se);
        if (lane == 0)
            tm.stat[(int64_t)(it.b * h_q + it.kh * g + n) * nchunk + it.chunk] = make_float2(mx, se);
    }
    if (local_from < it.c0 + it.n) {   // uniform: positions from local_from on are not ranked
#pragma unroll
        for (int e = 0; e < KPL; ++e)
            if (it.c0 + KPL * lane + e >= local_from) kk[e] = 0u;
    }
    // count over the wave of keys >= x: one compare per key into a lane mask
    // and its scalar popcount (no per-lane sums to reduce across lanes)
    auto count_ge = [&](uint32_t x) -> uint32_t {
        uint32_t c = 0u;
#pragma unroll
        for (int e = 0; e < KPL; ++e) c += (uint32_t)__builtin_popcountll(__ballot(kk[e] >= x));
        return __builtin_amdgcn_readfirstlane(c);
    };
    uint32_t cut = 0;   // publish everything when the chunk holds <= M keys
    if ((uint32_t)it.n > M) {
        const uint32_t hi = M + (M >> 2);
        // Invariant of the search: count(key >= a) >= M (a = 0 counts every
        // slot) and count(key >= z) < M (z = 2^32, as a 64-bit bound).
        uint32_t a = 0;
        uint64_t z = 1ull << 32;
        bool done = false;
        if (guess != 0u) {
            // gallop from the previous cutoff in steps that double from 2^18
            // (about 3 % of the value for an fp32 logit) until the count
            // crosses M, then bisect between the last two probes
            uint32_t c = count_ge(guess);
            if (c >= M && c <= hi) {
                cut = guess;
                done = true;
            } else if (c > hi) {
                a = guess;
                uint64_t step = 1ull << 18;
#pragma unroll 1
                while (true) {
                    const uint64_t x = (uint64_t)a + step;
                    if (x >= z) break;
                    c = count_ge((uint32_t)x);
                    if (c < M) { z = x; break; }
                    a = (uint32_t)x;
                    if (c <= hi) { cut = a; done = true; break; }
                    step <<= 1;
                }
            } else {
                z = guess;
                uint64_t step = 1ull << 18;
#pragma unroll 1
                while (true) {
                    if ((uint64_t)a + step >= z) break;
                    const uint32_t x = (uint32_t)(z - step);
                    c = count_ge(x);
                    if (c >= M) {
                        a = x;
                        if (c <= hi) { cut = a; done = true; }
                        break;
                    }
                    z = x;
                    step <<= 1;
                }
            }
        }
        if (!done) {
            // bisection of [a, z) down to a width of 2^12
#pragma unroll 1
            while (z - a > (1ull << 12)) {
                const uint32_t x = (uint32_t)(a + ((z - a) >> 1));
                const uint32_t c = count_ge(x);
                if (c >= M) {
                    a = x;
                    if (c <= hi) break;
                } else {
                    z = x;
                }
            }
            cut = a;
        }
        if (lane == 0) warm[n] = cut;
    }
    uint32_t pub = cut;   // the published cutoff
    if (flo && cut != 0u) {   // uniform
        uint32_t* flo_tag = flo + g;
        const uint32_t tag = 1u + (uint32_t)(it.b * h_q + it.kh * g);
        const bool same = flo_tag[n] == tag;
        const uint32_t fl = flo[n];
        if (same && fl < cut) pub = fl;
        __builtin_amdgcn_s_waitcnt(0xc07f);   // every lane has read flo before lane 0 writes it
        if (lane == 0) {
            flo[n] = same && fl < cut ? fl : cut;
            flo_tag[n] = tag;
        }
    }
    const uint32_t lo = pub > 1u ? pub : 1u;   // key 0 marks an empty slot
    uint32_t kc = 0;
#pragma unroll
    for (int e = 0; e < KPL; ++e) kc += kk[e] >= lo ? 1u : 0u;
    uint32_t total;
    const uint32_t first = wave_incl_scan(kc, total) - kc;
    const int64_t slot = ((int64_t)(it.b * h_q + it.kh * g + n) * nchunk + it.chunk);
    // the list goes to the next free (16-byte aligned) place of the
    // workgroup's range: staged in LDS while it fits, else stored directly
    uint32_t off = 0;
    if (lane == 0) off = atomicAdd(sink.cursor, (total + 1u) & ~1u);
    off = __builtin_amdgcn_readfirstlane(off);
    const bool staged_lds = off + total <= sink.cap;
    if (staged_lds && lane == 0) atomicMax(sink.used, off + total);
    // The destination is LDS or global memory (uniformly): typed pointers
    // for each, so that no store becomes a flat store (whose completion the
    // waits below would otherwise have to cover).
    typedef uint32_t v2u __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    typedef __attribute__((address_space(3))) v2u lds_v2u;
    typedef __attribute__((address_space(1))) u32x4 glb_u32x4;
    typedef __attribute__((address_space(1))) v2u glb_v2u;
    lds_v2u* dst_l = (lds_v2u*)(sink.stg + off);
    glb_v2u* dst_g = (glb_v2u*)(sink.pool + off);
    uint32_t pos0 = (uint32_t)(it.c0 + KPL * lane);
    asm volatile("" : "+v"(pos0));   // positions are formed at each store, not held in registers
    if (total <= kStageMax) {
        uint2* stage = reinterpret_cast<uint2*>(row);
        uint32_t at = first;
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
            const uint32_t keep = kk[e] >= lo ? 1u : 0u;
            stage[keep ? at : kStageMax + lane] = make_uint2(pos0 + e, kk[e]);
            at += keep;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        for (uint32_t j = 2 * lane; j < total; j += 128) {
            u32x4 v2;
            const uint2 a0 = stage[j];
            const uint2 a1 = j + 1 < total ? stage[j + 1] : make_uint2(0u, 0u);
            v2[0] = a0.x; v2[1] = a0.y; v2[2] = a1.x; v2[3] = a1.y;
            // dst + j is 16-byte aligned (j even)
            if (staged_lds) *(lds_u32x4*)(dst_l + j) = v2;
            else *(glb_u32x4*)(dst_g + j) = v2;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // the head's row is reused as soon as this returns
    } else {
        uint32_t at = first;
        if (staged_lds) {
#pragma unroll
            for (int e = 0; e < KPL; ++e)
                if (kk[e] >= lo) dst_l[at++] = v2u{pos0 + e, kk[e]};
        } else {
#pragma unroll
            for (int e = 0; e < KPL; ++e)
                if (kk[e] >= lo) dst_g[at++] = v2u{pos0 + e, kk[e]};
        }
    }
    if (lane == 0) {
        const uint64_t abs_off = sink.base + off;
        const uint4 m = make_uint4((uint32_t)abs_off, total, pub, (uint32_t)(abs_off >> 32));
        const int e = local * g + n;   // staged while it fits, like the lists
        if (e < kMetaStage) {
            sink.meta_stg[e] = m;
            sink.meta_slot[e] = (uint32_t)slot;
        } else {
            tm.meta[slot] = m;
        }
    }
}

// Persistent grid: as many workgroups as can be resident at once (so none of
// them waits for another to finish all of its work before starting), at most
// one per work item.
template <typename K>
int resident_grid(K kern, int threads, size_t lds, int nwork) {
    const int grid = cu_count() * blocks_per_cu(reinterpret_cast<const void*>(kern), threads, lds);
    return grid < nwork ? grid : nwork;
}

}  // namespace
}  // namespace saga
#endif
