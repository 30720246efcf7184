// Top-N selection per query head: threshold select + compaction.
//
// "More Value per Key" §2.5 Eq. 6 keeps the N largest logits of the row;
// §3.1 and App. C.1 find them by comparing every logit with the N-th largest
// value instead of sorting. Here that threshold is found exactly for the
// current logits (a fresh threshold at every call), and equal logits at the
// threshold are taken in ascending position until exactly N_eff = min(N, L)
// entries are kept.
//
// Core (one workgroup per (b, i) row):
//   1. keys (order-preserving uint32 images of the fp32 logits, -0 == +0)
//      are held in registers, KPT per lane per tile;
//   2. the key T of rank N_eff from the top and the number of ties at T to
//      keep: by MSB-first bisection with ballot-popcount counts when the keys
//      fit one register tile, else by three LDS histogram rounds over
//      12/10/10-bit digits (re-reading the keys per round);
//   3. compaction in ascending position order: wave ballots + mbcnt give each
//      kept element its slot, a scan over the waves orders the waves.
// Rows longer than one register tile are processed tile by tile, re-reading
// the keys from memory in each round.
//
// Sources of keys:
//   dense  -- fp32 logits of every position (kscan dense mode);
//   union  -- the candidate lists the top-M K-scan published per chunk. The
//             union's key of rank N_eff, T, is the true one when every chunk
//             cutoff is <= T (all keys a chunk left out are below its cutoff,
//             hence below T, so exactly the keys >= T are all present). When
//             that check fails the workgroup recomputes its head's logits and
//             selects on them densely, so the result is always exact.
#include "saga_internal.h"

namespace saga {
using namespace dev;

namespace {

constexpr int kUnionThreads = 256;
constexpr int kUnionKPT = 16;
constexpr int kMaxChunks = 4096;

__device__ inline uint32_t wave_sum(uint32_t x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

__device__ inline uint32_t wave_max(uint32_t x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t y = __shfl_xor(x, o, 64);
        x = y > x ? y : x;
    }
    return x;
}

// Exclusive prefix (over lanes below) and total of a per-lane count in [0, 7].
__device__ inline void wave_scan_small(uint32_t x, uint32_t& pre, uint32_t& tot) {
    const uint64_t b0 = ballot(x & 1u), b1 = ballot(x & 2u), b2 = ballot(x & 4u);
    pre = lanes_below(b0) + 2u * lanes_below(b1) + 4u * lanes_below(b2);
    tot = (uint32_t)__popcll(b0) + 2u * (uint32_t)__popcll(b1) + 4u * (uint32_t)__popcll(b2);
}

struct SelShared {
    uint32_t hist[4096];
    uint32_t wtot[2 * 16];
    uint32_t bc[4];
};

// Keys of every position of a dense fp32 logit row. Group of 4: lane l holds
// positions tile*CAP + w*SEG + 256*j4 + 4l + c (c = 0..3) in slots 4*j4 + c.
template <int KPT, int NW>
struct DenseSrc {
    static constexpr int GROUP = 4;
    static constexpr int SEG = KPT * 64;
    static constexpr int CAP = NW * SEG;
    const float* srow;
    int64_t n;   // positions
    __device__ void load(int tile, uint32_t (&key)[KPT], int32_t (&)[KPT]) const {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
        for (int j4 = 0; j4 < KPT / 4; ++j4) {
            const int64_t p = (int64_t)tile * CAP + wave * SEG + j4 * 256 + 4 * lane;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            // rows are padded to a multiple of 16 floats, so p < n keeps p + 3 in the row
            if (p < n) v = *reinterpret_cast<const f32x4*>(srow + p);
#pragma unroll
            for (int c = 0; c < 4; ++c) key[j4 * 4 + c] = (p + c < n) ? float_key(v[c]) : 0u;
        }
    }
    __device__ int32_t position(int tile, int slot, const int32_t (&)[KPT]) const {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        return (int32_t)((int64_t)tile * CAP + wave * SEG + (slot / 4) * 256 + 4 * lane + slot % 4);
    }
};

// Candidate lists of one row: chunk k holds cnt_k entries at base + coff[k]
// (coff in LDS, 64-bit pool offsets); pref[] (LDS) is the exclusive prefix of
// the counts. Element j of the union (chunk-major, so ascending in position)
// sits in slot s of lane l of wave w with j = tile*CAP + w*SEG + 64 s + l.
template <int KPT, int NW>
struct UnionSrc {
    static constexpr int GROUP = 1;
    static constexpr int SEG = KPT * 64;
    static constexpr int CAP = NW * SEG;
    const uint2* base;
    const int64_t* coff;   // LDS, nch entries
    const int32_t* pref;   // LDS, nch + 1 entries
    int nch;
    int64_t n;             // total candidates
    __device__ void load(int tile, uint32_t (&key)[KPT], int32_t (&pos)[KPT]) const {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int64_t j0 = (int64_t)tile * CAP + wave * SEG + lane;
        // chunk of the lane's first element: largest k with pref[k] <= j0 (binary search);
        // the lane's later slots only move forward from there
        int kc = 0;
        if (j0 < n) {
            int hi = nch;
            while (hi - kc > 1) {
                const int mid = (kc + hi) >> 1;
                if (pref[mid] <= j0) kc = mid; else hi = mid;
            }
        }
#pragma unroll
        for (int s = 0; s < KPT; ++s) {
            const int64_t j = j0 + 64 * s;
            key[s] = 0u;
            pos[s] = -1;
            if (j < n) {
                while (pref[kc + 1] <= j) ++kc;
                const uint2 e = base[coff[kc] + (j - pref[kc])];
                pos[s] = (int32_t)e.x;
                key[s] = e.y;
            }
        }
    }
    __device__ int32_t position(int, int slot, const int32_t (&pos)[KPT]) const { return pos[slot]; }
};

// Radix rounds: T = key of rank n_eff (from the top) among the source's keys,
// krem = how many keys equal to T are kept, kmax = the largest key.
template <int NT, int KPT, class Src>
__device__ void find_threshold(const Src& src, int ntiles, uint32_t n_eff, uint32_t (&key)[KPT],
                               int32_t (&pos)[KPT], SelShared& sh, uint32_t& T, uint32_t& krem,
                               uint32_t& kmax) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool resident = ntiles == 1;
    uint32_t prefix = 0;
    krem = n_eff;
    kmax = 0;
    if (resident) src.load(0, key, pos);
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int bits = pass == 0 ? 12 : 10;
        const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
        const int nb = 1 << bits;
        for (int i = tid; i < nb; i += NT) sh.hist[i] = 0u;
        __syncthreads();
#pragma unroll 1
        for (int tile = 0; tile < ntiles; ++tile) {
            if (!resident) src.load(tile, key, pos);
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                const uint32_t kk = key[j];
                if (pass == 0) kmax = kk > kmax ? kk : kmax;
                const bool match = pass == 0 ? kk != 0u : (kk >> (shift + bits)) == prefix;
                if (match) atomicAdd(&sh.hist[(kk >> shift) & (uint32_t)(nb - 1)], 1u);
            }
        }
        __syncthreads();
        const int bpt = nb / NT;   // bins per thread
        uint32_t mine = 0;
        for (int i = 0; i < bpt; ++i) mine += sh.hist[tid * bpt + i];
        uint32_t suf = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_down(suf, o, 64);
            if (lane + o < 64) suf += y;
        }
        if (lane == 0) sh.wtot[wave] = suf;
        __syncthreads();
        uint32_t above = suf - mine;
        for (int w = wave + 1; w < NW; ++w) above += sh.wtot[w];
        for (int i = bpt - 1; i >= 0; --i) {
            const uint32_t c = sh.hist[tid * bpt + i];
            if (above < krem && above + c >= krem) {
                sh.bc[0] = (uint32_t)(tid * bpt + i);
                sh.bc[1] = above;
            }
            above += c;
        }
        __syncthreads();
        krem -= sh.bc[1];
        prefix = (prefix << bits) | sh.bc[0];
        __syncthreads();
    }
    T = prefix;
    kmax = wave_max(kmax);
    if (lane == 0) sh.wtot[wave] = kmax;
    __syncthreads();
    uint32_t m = 0;
    for (int w = 0; w < NW; ++w) m = sh.wtot[w] > m ? sh.wtot[w] : m;
    kmax = m;
    __syncthreads();
}

// Same result as find_threshold for keys already resident in registers (one
// tile), without LDS atomics: MSB-first bisection for the largest key x with
// count(key >= x) >= n_eff, where each count is a sum of wave ballot
// popcounts (scalar unit) and one LDS slot per wave, double-buffered so each
// bit costs a single barrier.
template <int NT, int KPT>
__device__ void find_threshold_bisect(uint32_t n_eff, const uint32_t (&key)[KPT], SelShared& sh,
                                      uint32_t& T, uint32_t& krem, uint32_t& kmax) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) m = key[j] > m ? key[j] : m;
    m = wave_max(m);
    uint32_t prefix = 0;
#pragma unroll 1
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t x = prefix | (1u << bit);
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) c += (uint32_t)__popcll(ballot(key[j] >= x));
        uint32_t* slot = sh.wtot + (bit & 1) * NW;
        if (lane == 0) slot[wave] = c;
        __syncthreads();
        uint32_t tot = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) tot += slot[w];
        if (tot >= n_eff) prefix = x;
    }
    T = prefix;
    uint32_t gt = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) gt += (uint32_t)__popcll(ballot(key[j] > T));
    if (lane == 0) {
        sh.wtot[2 * NW + wave] = gt;
        sh.wtot[3 * NW + wave] = m;
    }
    __syncthreads();
    uint32_t g = 0, mx = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        g += sh.wtot[2 * NW + w];
        mx = sh.wtot[3 * NW + w] > mx ? sh.wtot[3 * NW + w] : mx;
    }
    krem = n_eff - g;
    kmax = mx;
    __syncthreads();
}

// Keep keys > T and the first krem keys == T, in ascending position order.
template <int NT, int KPT, class Src>
__device__ void compact(const Src& src, int ntiles, uint32_t T, uint32_t krem, uint32_t n_eff,
                        uint32_t (&key)[KPT], int32_t (&pos)[KPT], SelShared& sh, int32_t* oi,
                        float* ov, int32_t* ou) {
    constexpr int NW = NT / 64;
    constexpr int G = Src::GROUP;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool resident = ntiles == 1;
    uint32_t base = 0, eq_tile = 0;
#pragma unroll 1
    for (int tile = 0; tile < ntiles; ++tile) {
        if (!resident) src.load(tile, key, pos);
        uint32_t cg = 0, ce = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            cg += key[j] > T;
            ce += key[j] == T;
        }
        cg = wave_sum(cg);
        ce = wave_sum(ce);
        if (lane == 0) {
            sh.wtot[wave] = cg;
            sh.wtot[NW + wave] = ce;
        }
        __syncthreads();
        uint32_t eqb = eq_tile, selb = 0, my_eqb = 0, my_selb = 0;
        for (int w = 0; w < NW; ++w) {
            if (w == wave) {
                my_eqb = eqb;
                my_selb = selb;
            }
            const uint32_t ew = sh.wtot[NW + w];
            const uint32_t room = krem > eqb ? krem - eqb : 0u;
            selb += sh.wtot[w] + (ew < room ? ew : room);
            eqb += ew;
        }
        uint32_t req = my_eqb;
        uint32_t rsel = base + my_selb;
#pragma unroll
        for (int g0 = 0; g0 < KPT / G; ++g0) {
            uint32_t ecnt = 0;
#pragma unroll
            for (int c = 0; c < G; ++c) ecnt += key[g0 * G + c] == T;
            uint32_t epre, etot;
            wave_scan_small(ecnt, epre, etot);
            uint32_t er = req + epre;
            bool keep[G];
            uint32_t scnt = 0;
#pragma unroll
            for (int c = 0; c < G; ++c) {
                const uint32_t kk = key[g0 * G + c];
                const bool eq = kk == T;
                keep[c] = kk > T || (eq && er < krem);
                er += eq;
                scnt += keep[c];
            }
            uint32_t spre, stot;
            wave_scan_small(scnt, spre, stot);
            uint32_t slot = rsel + spre;
#pragma unroll
            for (int c = 0; c < G; ++c) {
                // slot < n_eff holds by construction; the test keeps stores in bounds
                if (keep[c] && slot < n_eff) {
                    const int32_t p = src.position(tile, g0 * G + c, pos);
                    oi[slot] = p;
                    ov[slot] = key_float(key[g0 * G + c]);
                    if (ou) ou[slot] = p;
                    ++slot;
                }
            }
            req += etot;
            rsel += stot;
        }
        base += selb;
        eq_tile = eqb;
        __syncthreads();
    }
}

// ---- dense select: one 1024-thread workgroup per row ------------------------------
template <int KPT>
__global__ __launch_bounds__(kSelectThreads) void select_dense(
    const float* __restrict__ scores, int64_t s_stride, const int32_t* __restrict__ lens,
    int h_q, int N, int64_t S_max, int32_t* __restrict__ sel_idx, float* __restrict__ sel_val,
    float* __restrict__ row_max, int32_t* __restrict__ row_cnt, int32_t* __restrict__ idx_out) {
    constexpr int NT = kSelectThreads;
    __shared__ SelShared sh;
    const int row = blockIdx.x;
    const int b = row / h_q;
    const int64_t L = clamp_len(lens[b], S_max);
    const int n_eff = (int)((int64_t)N < L ? (int64_t)N : L);
    int32_t* oi = sel_idx + (int64_t)row * N;
    float* ov = sel_val + (int64_t)row * N;
    int32_t* ou = idx_out ? idx_out + (int64_t)row * N : nullptr;
    for (int s = n_eff + threadIdx.x; s < N; s += NT) {
        oi[s] = -1;
        ov[s] = -__builtin_inff();
        if (ou) ou[s] = -1;
    }
    if (n_eff == 0) {
        if (threadIdx.x == 0) {
            row_max[row] = -__builtin_inff();
            row_cnt[row] = 0;
        }
        return;
    }
    using Src = DenseSrc<KPT, NT / 64>;
    const Src src{scores + (int64_t)row * s_stride, L};
    const int ntiles = (int)((L + Src::CAP - 1) / Src::CAP);
    uint32_t key[KPT];
    int32_t pos[KPT];
    uint32_t T, krem, kmax;
    find_threshold<NT, KPT>(src, ntiles, (uint32_t)n_eff, key, pos, sh, T, krem, kmax);
    if (threadIdx.x == 0) {
        row_max[row] = key_float(kmax);
        row_cnt[row] = n_eff;
    }
    compact<NT, KPT>(src, ntiles, T, krem, (uint32_t)n_eff, key, pos, sh, oi, ov, ou);
}

// ---- union select over the top-M candidate lists ----------------------------------
// Fallback logits of one head, VALU, written to a dense row: lane-parallel over
// positions, q staged in LDS as fp32.
template <typename T, int DH>
__device__ void head_logits(const T* __restrict__ q, const T* __restrict__ k, int b, int i,
                            int h_q, int h_k, int64_t S_max, int64_t L, float scale,
                            float* __restrict__ out, float* qs) {
    const int g = h_q / h_k;
    const int kh = i / g;
    const T* qr = q + (int64_t)(b * h_q + i) * DH;
    for (int c = threadIdx.x; c < DH; c += kUnionThreads) {
        if (sizeof(T) == 2) qs[c] = __uint_as_float((uint32_t)((const uint16_t*)qr)[c] << 16);
        else qs[c] = ((const float*)qr)[c];
    }
    __syncthreads();
    const T* kb = k + (int64_t)(b * h_k + kh) * S_max * DH;
    for (int64_t t = threadIdx.x; t < L; t += kUnionThreads) {
        const T* kr = kb + t * DH;
        float acc = 0.f;
        for (int c0 = 0; c0 < DH; c0 += 16 / (int)sizeof(T)) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(kr + c0);
            if (sizeof(T) == 2) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc = fmaf(qs[c0 + 2 * e], __uint_as_float(v[e] << 16), acc);
                    acc = fmaf(qs[c0 + 2 * e + 1], __uint_as_float(v[e] & 0xFFFF0000u), acc);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = fmaf(qs[c0 + e], __uint_as_float(v[e]), acc);
            }
        }
        out[t] = acc * scale;
    }
    __syncthreads();
}

template <typename T, int DH>
__global__ __launch_bounds__(kUnionThreads) void select_union(
    const uint2* __restrict__ cand, const uint4* __restrict__ cand_meta,
    const int32_t* __restrict__ lens, int h_q, int h_k,
    int N, int64_t S_max, int nchunk, int32_t* __restrict__ sel_idx, float* __restrict__ sel_val,
    float* __restrict__ row_max, int32_t* __restrict__ row_cnt, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ row_flag, const T* __restrict__ q, const T* __restrict__ k,
    float* __restrict__ scores, int64_t s_stride, float scale) {
    constexpr int NT = kUnionThreads;
    constexpr int NW = NT / 64;
    constexpr int KPT = kUnionKPT;
    __shared__ SelShared sh;
    __shared__ int32_t pref[kMaxChunks + 1];
    __shared__ int64_t coff[kMaxChunks];
    __shared__ uint32_t bad;
    const int row = blockIdx.x;
    const int b = row / h_q;
    const int i = row - b * h_q;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t L = clamp_len(lens[b], S_max);
    const int n_eff = (int)((int64_t)N < L ? (int64_t)N : L);
    int32_t* oi = sel_idx + (int64_t)row * N;
    float* ov = sel_val + (int64_t)row * N;
    int32_t* ou = idx_out ? idx_out + (int64_t)row * N : nullptr;
    for (int s = n_eff + tid; s < N; s += NT) {
        oi[s] = -1;
        ov[s] = -__builtin_inff();
        if (ou) ou[s] = -1;
    }
    if (n_eff == 0) {
        if (tid == 0) {
            row_max[row] = -__builtin_inff();
            row_cnt[row] = 0;
            row_flag[row] = 0;
        }
        return;
    }
    const int nch = (int)((L + kScanChunk - 1) / kScanChunk);
    const uint4* meta = cand_meta + (int64_t)row * nchunk;
    const int g = h_q / h_k;
    // pool region of this row's chunk c: item (b*h_k + kh)*nchunk + c
    const int64_t item0 = (int64_t)(b * h_k + i / g) * nchunk;

    // exclusive prefix of the chunk counts: each thread sums a contiguous run
    const int per = (nch + NT - 1) / NT;
    int32_t run = 0;
    for (int c = tid * per; c < nch && c < (tid + 1) * per; ++c) {
        const uint4 m = meta[c];
        coff[c] = (item0 + c) * g * kScanChunk + m.x;
        run += (int32_t)m.y;
    }
    int32_t incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) sh.wtot[wave] = (uint32_t)incl;
    if (tid == 0) bad = 0u;
    __syncthreads();
    int32_t off = incl - run;
    for (int w = 0; w < wave; ++w) off += (int32_t)sh.wtot[w];
    for (int c = tid * per; c < nch && c < (tid + 1) * per; ++c) {
        pref[c] = off;
        off += (int32_t)meta[c].y;
    }
    if (tid == NT - 1) pref[nch] = off;   // last thread's running sum = total
    __syncthreads();
    const int64_t total = pref[nch];
    __syncthreads();

    uint32_t key[KPT];
    int32_t pos[KPT];
    uint32_t thr = 0, krem = 0, kmax = 0;
    bool ok = total >= n_eff;
    if (ok) {
        using Src = UnionSrc<KPT, NW>;
        const Src src{cand, coff, pref, nch, total};
        const int ntiles = (int)((total + Src::CAP - 1) / Src::CAP);
        if (ntiles == 1) {
            src.load(0, key, pos);
            find_threshold_bisect<NT, KPT>((uint32_t)n_eff, key, sh, thr, krem, kmax);
        } else {
            find_threshold<NT, KPT>(src, ntiles, (uint32_t)n_eff, key, pos, sh, thr, krem, kmax);
        }
        // exact iff every chunk's cutoff is <= the union's threshold key
        for (int c = tid; c < nch; c += NT)
            if (meta[c].z > thr) bad = 1u;
        __syncthreads();
        ok = bad == 0u;
        if (ok) compact<NT, KPT>(src, ntiles, thr, krem, (uint32_t)n_eff, key, pos, sh, oi, ov, ou);
    }
    if (!ok) {
        // dense fallback: this head's logits over all L positions, then a full select
        float* srow = scores + (int64_t)row * s_stride;
        head_logits<T, DH>(q, k, b, i, h_q, h_k, S_max, L, scale, srow,
                           reinterpret_cast<float*>(sh.hist));
        using Src = DenseSrc<KPT, NW>;
        const Src src{srow, L};
        const int ntiles = (int)((L + Src::CAP - 1) / Src::CAP);
        if (ntiles == 1) {
            src.load(0, key, pos);
            find_threshold_bisect<NT, KPT>((uint32_t)n_eff, key, sh, thr, krem, kmax);
        } else {
            find_threshold<NT, KPT>(src, ntiles, (uint32_t)n_eff, key, pos, sh, thr, krem, kmax);
        }
        compact<NT, KPT>(src, ntiles, thr, krem, (uint32_t)n_eff, key, pos, sh, oi, ov, ou);
    }
    if (tid == 0) {
        row_max[row] = key_float(kmax);
        row_cnt[row] = n_eff;
        row_flag[row] = ok ? 0 : 1;
    }
}

template <int KPT>
hipError_t go_dense(const float* scores, int64_t s_stride, const int32_t* lens, int B, int h_q,
                    int N, int64_t S_max, int32_t* sel_idx, float* sel_val, float* row_max,
                    int32_t* row_cnt, int32_t* idx_out, hipStream_t st) {
    hipLaunchKernelGGL((select_dense<KPT>), dim3((unsigned)(B * h_q)), dim3(kSelectThreads), 0, st,
                       scores, s_stride, lens, h_q, N, S_max, sel_idx, sel_val, row_max, row_cnt,
                       idx_out);
    return hipGetLastError();
}

}  // namespace

int max_union_chunks() { return kMaxChunks; }

hipError_t launch_select(const float* scores, int64_t s_stride, const int32_t* lens, int B,
                         int h_q, int N, int64_t S_max, int32_t* sel_idx, float* sel_val,
                         float* row_max, int32_t* row_cnt, int32_t* idx_out, hipStream_t st) {
    const int64_t per = (int64_t)kSelectThreads;
    if (S_max <= 4 * per)
        return go_dense<4>(scores, s_stride, lens, B, h_q, N, S_max, sel_idx, sel_val, row_max, row_cnt, idx_out, st);
    if (S_max <= 8 * per)
        return go_dense<8>(scores, s_stride, lens, B, h_q, N, S_max, sel_idx, sel_val, row_max, row_cnt, idx_out, st);
    if (S_max <= 16 * per)
        return go_dense<16>(scores, s_stride, lens, B, h_q, N, S_max, sel_idx, sel_val, row_max, row_cnt, idx_out, st);
    return go_dense<32>(scores, s_stride, lens, B, h_q, N, S_max, sel_idx, sel_val, row_max, row_cnt, idx_out, st);
}

hipError_t launch_select_union(const TopmOut& tm, const int32_t* lens, int B, int h_q, int h_k,
                               int d, int N, int64_t S_max, int32_t* sel_idx, float* sel_val,
                               float* row_max, int32_t* row_cnt, int32_t* idx_out,
                               int32_t* row_flag, const void* q, const void* k, float* scores,
                               int64_t s_stride, bool bf16, hipStream_t st) {
    const int nchunk = (int)((S_max + kScanChunk - 1) / kScanChunk);
    const float scale = (float)(1.0 / __builtin_sqrt((double)d));
#define SAGA_SU(T, D)                                                                            \
    hipLaunchKernelGGL((select_union<T, D>), dim3((unsigned)(B * h_q)), dim3(kUnionThreads), 0,   \
                       st, tm.cand, tm.meta, lens, h_q, h_k, N, S_max, nchunk, sel_idx,           \
                       sel_val, row_max, row_cnt, idx_out, row_flag, (const T*)q, (const T*)k,    \
                       scores, s_stride, scale)
    if (bf16) {
        if (d == 64) SAGA_SU(uint16_t, 64); else SAGA_SU(uint16_t, 128);
    } else {
        if (d == 64) SAGA_SU(float, 64); else SAGA_SU(float, 128);
    }
#undef SAGA_SU
    return hipGetLastError();
}

}  // namespace saga
