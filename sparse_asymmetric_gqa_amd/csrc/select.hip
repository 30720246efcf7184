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
//             hence below T, so exactly the keys >= T are all present). One
//             workgroup per row: rows of at most 256 chunks whose lists fit
//             the registers settle with a histogram descent (select_union);
//             the rest take the general code (union_row), which also
//             recomputes the head's logits and selects on them densely when
//             the check fails, so the result is always exact.
#include "gather.h"

namespace saga {
using namespace dev;

namespace {

constexpr int kUnionThreads = 256;
constexpr int kUnionKPT = 16;
constexpr int kMaxChunks = 512;   // chunks per row on the union path (S_max <= 512 Ki)

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

// The key of rank `need` (from the top) among the keys the 256 threads hold
// in registers, by histogram descent: each pass spreads the keys of the
// current range [lo, hi] over 256 LDS bins with shared-memory atomics, every
// wave scans all bins itself (4 per lane, a DPP prefix) and picks the bin
// holding rank `need`, so a pass costs one barrier and narrows the range by
// 8 bits. Requires every key above hi to be absent and at least `need` keys
// in [lo, hi]. Returns a T with count(key >= T) >= need > count(key > T)
// when the final bin is a single key value, or the lower end of a bin with
// count(key >= T) == need exactly. hist: 3 x 256 LDS words (rotated, so a
// pass clears the bins read two passes earlier).
template <int KPT>
__device__ uint32_t descend(const uint32_t (&key)[KPT], uint32_t need, uint32_t lo, uint32_t hi,
                            uint32_t* hist) {
    const int tid = threadIdx.x, lane = tid & 63;
    hist[tid] = 0u;
    __syncthreads();
#pragma unroll 1
    for (int pass = 0;; ++pass) {
        uint32_t* h = hist + 256 * (pass % 3);
        hist[256 * ((pass + 1) % 3) + tid] = 0u;   // last read two passes ago
        const uint32_t span = hi - lo;
        const int nb = span ? 32 - __clz((int)span) : 0;
        const int shift = nb > 8 ? nb - 8 : 0;
#pragma unroll
        for (int s = 0; s < KPT; ++s)
            if (key[s] >= lo && key[s] <= hi)
                __hip_atomic_fetch_add(h + ((key[s] - lo) >> shift), 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
        __syncthreads();
        // lane l holds bins 255-4l (top) down to 252-4l; every wave scans all
        const uint4 hv = reinterpret_cast<const uint4*>(h)[63 - lane];
        const uint32_t lsum = (hv.x + hv.y) + (hv.z + hv.w);
        uint32_t total;
        const uint32_t incl = wave_incl_scan(lsum, total);   // keys in bins >= 252-4l
        const uint32_t above0 = incl - lsum;
        const uint64_t hit = ballot(incl >= need && above0 < need);
        const int hl = (int)__builtin_ctzll(hit);   // exactly one lane
        uint32_t bin = 255u - 4u * (uint32_t)lane, above = above0, inbin = hv.w;
        if (above + hv.w < need) {
            above += hv.w; bin -= 1u; inbin = hv.z;
            if (above + hv.z < need) {
                above += hv.z; bin -= 1u; inbin = hv.y;
                if (above + hv.y < need) { above += hv.y; bin -= 1u; inbin = hv.x; }
            }
        }
        bin = (uint32_t)__builtin_amdgcn_readlane((int)bin, hl);
        above = (uint32_t)__builtin_amdgcn_readlane((int)above, hl);
        inbin = (uint32_t)__builtin_amdgcn_readlane((int)inbin, hl);
        need -= above;
        lo += bin << shift;
        const uint32_t wmask = (1u << shift) - 1u;
        hi = hi - lo <= wmask ? hi : lo + wmask;
        if (inbin == need || shift == 0) {   // keys >= lo are exactly need, or one key value
            __syncthreads();   // every wave has read this pass's bins
            return lo;
        }
    }
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

// Load of a value another thread of this workgroup stored to global memory
// before a barrier: a relaxed atomic of workgroup scope, so that it is a
// vector load (never the scalar data cache, which vector stores do not
// update) and needs no device-wide fence.
template <typename V>
__device__ inline V wg_load(const V* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Scaled logit of one cached key row against the query staged in LDS as fp32.
template <typename T, int DH>
__device__ inline float row_logit(const T* __restrict__ kr, const float* qs, float scale) {
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
    return acc * scale;
}

// ---- union select over the top-M candidate lists ----------------------------------
// Fallback logits of one head, VALU, written to a dense row: lane-parallel over
// positions, q staged in LDS as fp32.
// With qf (fp32 [DH], nullable) the query is taken from qf instead of q.
template <typename T, int DH>
__device__ void head_logits(const T* __restrict__ q, const T* __restrict__ k, int b, int i,
                            int h_q, int h_k, int64_t S_max, int64_t L, float scale,
                            float* __restrict__ out, float* qs, const float* qf = nullptr) {
    const int g = h_q / h_k;
    const int kh = i / g;
    const T* qr = q + (int64_t)(b * h_q + i) * DH;
    for (int c = threadIdx.x; c < DH; c += kUnionThreads) {
        if (qf) qs[c] = qf[c];
        else if (sizeof(T) == 2) qs[c] = __uint_as_float((uint32_t)((const uint16_t*)qr)[c] << 16);
        else qs[c] = ((const float*)qr)[c];
    }
    __syncthreads();
    const T* kb = k + (int64_t)(b * h_k + kh) * S_max * DH;
    for (int64_t t = threadIdx.x; t < L; t += kUnionThreads) out[t] = row_logit<T, DH>(kb + t * DH, qs, scale);
    __syncthreads();
}

// LDS of the general code of the union select (and of the stale-threshold
// select's recompute).
struct UnionShared {
    SelShared sh;
    int32_t pref[kMaxChunks + 1];
    int64_t coff[kMaxChunks];
    int32_t roff[kMaxChunks + 1];   // chunk-local recompute: a chunk's place in the row's region, or -1
    uint32_t bad;
};


// Builds in us.pref / us.coff the union of one row's chunk candidate lists,
// with every chunk whose cutoff is above `lim` replaced by all of its keys,
// recomputed for this head (query qf when given, else the row's q with
// `scale`) into the row's region of the logit workspace (srow, as (position,
// key) pairs in ascending position). Returns the union's size, or -1 when
// those chunks do not fit the region (half the row's positions); sets
// `recomputed` when some chunk was replaced. lim = 0xFFFFFFFF keeps every
// list. Every thread of the workgroup calls this; LDS: us.
template <typename T, int DH>
__device__ __attribute__((noinline)) int64_t build_union(UnionShared& us, const uint2* __restrict__ cand,
                               const uint4* __restrict__ meta, int nch, int chunk, int64_t L,
                               uint32_t lim, const T* __restrict__ q, const T* __restrict__ k,
                               const float* qf, float scale, float* srow, int64_t s_stride,
                               int b, int i, int h_q, int h_k, int64_t S_max, bool& recomputed) {
    constexpr int NT = kUnionThreads;
    SelShared& sh = us.sh;
    int32_t* pref = us.pref;
    int64_t* coff = us.coff;
    int32_t* roff = us.roff;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Exclusive prefix over the chunks of cnt(c) into dst[0 .. nch] (dst[nch]
    // = the total): each thread sums a contiguous run of chunks.
    const int per = (nch + NT - 1) / NT;
    auto prefix = [&](auto&& cnt, int32_t* dst) -> int64_t {
        int32_t run = 0;
        for (int c = tid * per; c < nch && c < (tid + 1) * per; ++c) run += cnt(c);
        int32_t incl = run;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int32_t y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
        }
        if (lane == 63) sh.wtot[wave] = (uint32_t)incl;
        __syncthreads();
        int32_t off = incl - run;
        for (int w = 0; w < wave; ++w) off += (int32_t)sh.wtot[w];
        for (int c = tid * per; c < nch && c < (tid + 1) * per; ++c) {
            dst[c] = off;
            off += cnt(c);
        }
        if (tid == NT - 1) dst[nch] = off;   // last thread's running sum = total
        __syncthreads();
        const int64_t tot = dst[nch];
        __syncthreads();
        return tot;
    };
    auto clen = [&](int c) -> int32_t {
        const int64_t c0 = (int64_t)c * chunk;
        return (int32_t)((L - c0) < chunk ? (L - c0) : chunk);
    };
    auto fails = [&](int c) -> bool { return meta[c].z > lim; };
    recomputed = false;
    int64_t nre = 0;
    if (lim != 0xFFFFFFFFu) {   // uniform
        nre = prefix([&](int c) { return fails(c) ? clen(c) : 0; }, roff);
        if (nre > s_stride / 2) return -1;
        // from here on roff[c] < 0 marks a chunk that keeps its list (LDS, so
        // the loops below read no chunk record from memory)
        for (int c = tid; c < nch; c += NT)
            if (!fails(c)) roff[c] = -1;
        __syncthreads();
    }
    auto redo = [&](int c) -> bool { return nre > 0 && roff[c] >= 0; };
    uint2* region = reinterpret_cast<uint2*>(srow);
    if (nre > 0) {   // uniform
        recomputed = true;
        float* qs = reinterpret_cast<float*>(sh.hist);   // the query as fp32 in LDS
        const T* qr = q + (int64_t)(b * h_q + i) * DH;
        for (int c = tid; c < DH; c += NT) {
            if (qf) qs[c] = qf[c];
            else if (sizeof(T) == 2) qs[c] = __uint_as_float((uint32_t)((const uint16_t*)qr)[c] << 16);
            else qs[c] = ((const float*)qr)[c];
        }
        __syncthreads();
        const float sc = qf ? 1.f : scale;
        const T* kb = k + (int64_t)(b * h_k + i / (h_q / h_k)) * S_max * DH;
        // Coalesced: LPR lanes share a key row, each taking one 16-byte piece
        // and its slice of the query, and a butterfly over them gives the dot
        // product; UNR rows per lane group are in flight at once.
        constexpr int EPL = 16 / (int)sizeof(T);   // elements per piece
        constexpr int LPR = DH / EPL;              // lanes per row
        constexpr int RPW = 64 / LPR;              // rows per wave instruction
        constexpr int UNR = 8;
        constexpr int STEP = (NT / 64) * RPW;      // rows per workgroup step
        const int rg = lane / LPR, sub = lane - rg * LPR;
        float qv[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) qv[e] = qs[sub * EPL + e] * sc;
#pragma unroll 1
        for (int c = 0; c < nch; ++c) {
            if (roff[c] < 0) continue;   // uniform (LDS)
            const int64_t c0 = (int64_t)c * chunk;
            const int32_t n = clen(c);
            uint2* dst = region + roff[c];
            const T* kc = kb + c0 * DH + sub * EPL;
#pragma unroll 1
            for (int base = wave * RPW; base < n; base += STEP * UNR) {   // uniform per wave
                const int r0 = base + rg;
                u32x4 v[UNR];
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    int r = r0 + u * STEP;
                    r = r < n ? r : n - 1;   // past the chunk: re-read its last row (unused)
                    v[u] = *reinterpret_cast<const u32x4*>(kc + (int64_t)r * DH);
                }
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    float f[EPL];
                    Row16<T>::cvt(v[u], f);
                    float acc = 0.f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc = fmaf(qv[e], f[e], acc);
#pragma unroll
                    for (int o = 1; o < LPR; o <<= 1) acc += __shfl_xor(acc, o, 64);
                    const int r = r0 + u * STEP;
                    if (sub == 0 && r < n)
                        dst[r] = make_uint2((uint32_t)(c0 + r), float_key(acc));
                }
            }
        }
        __syncthreads();   // the region's stores, before any thread reads them
    }
    const int64_t rbase = (int64_t)(region - cand);
    for (int c = tid; c < nch; c += NT) {
        const uint4 m = meta[c];
        coff[c] = redo(c) ? rbase + roff[c] : (int64_t)(((uint64_t)m.w << 32) | m.x);
    }
    return prefix([&](int c) { return redo(c) ? clen(c) : (int32_t)meta[c].y; }, pref);
}

// ---- union select, general code (one workgroup per row) ----------------------------
// The union select over any number of candidates (register tiles) and the
// cutoff check. When the check fails, the chunks whose cutoff lies above the
// union's key of rank N_eff are recomputed (build_union) and the select runs
// again on the completed union: a chunk whose cutoff is at or below that key
// (a lower bound of the true one, since the union is a subset of all keys) is
// complete for the true threshold, as every key it left out is below its
// cutoff; the recomputed chunks are complete by construction, so the second
// result is exact. When the union held fewer than N_eff keys there is no
// bound and every chunk that left keys out is recomputed. When too many
// chunks would be recomputed, all of the head's logits are. row_flag: 0
// settled from the lists, 2 some chunks recomputed, 1 all logits recomputed.
template <typename T, int DH>
__device__ __attribute__((noinline)) void union_row(
    int row, UnionShared& us, const uint2* __restrict__ cand, const uint4* __restrict__ cand_meta,
    const int32_t* __restrict__ lens, int h_q, int h_k,
    int N, int64_t S_max, int nchunk, int32_t* __restrict__ sel_idx, float* __restrict__ sel_val,
    float* __restrict__ row_max, int32_t* __restrict__ row_cnt, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ row_flag, const T* __restrict__ q, const T* __restrict__ k,
    float* __restrict__ scores, int64_t s_stride, float scale, int64_t L, int n_eff,
    const float* qf, int chunk, uint32_t& kmax_out) {
    constexpr int NT = kUnionThreads;
    constexpr int NW = NT / 64;
    constexpr int KPT = kUnionKPT;
    SelShared& sh = us.sh;
    uint32_t& bad = us.bad;
    kmax_out = 0u;
    const int b = row / h_q;
    const int i = row - b * h_q;
    const int tid = threadIdx.x;
    (void)lens;
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
    const int nch = (int)((L + chunk - 1) / chunk);
    const uint4* meta = cand_meta + (int64_t)row * nchunk;
    float* srow = scores + (int64_t)row * s_stride;
    uint32_t thr = 0, krem = 0, kmax = 0;
    // select over the union built from `lim`; false (nothing written) when
    // the union holds fewer than N_eff keys or does not fit. The key registers
    // live inside, so that nothing large is live across the union's build.
    auto select = [&](uint32_t lim, bool check, bool& recomputed) -> bool {
        const int64_t total = build_union<T, DH>(us, cand, meta, nch, chunk, L, lim, q, k, qf,
                                                 scale, srow, s_stride, b, i, h_q, h_k, S_max,
                                                 recomputed);
        if (total < n_eff) {   // uniform (also -1: too many chunks to recompute)
            thr = 0u;
            return false;
        }
        uint32_t key[KPT];
        int32_t pos[KPT];
        using Src = UnionSrc<KPT, NW>;
        const Src src{cand, us.coff, us.pref, nch, total};
        const int ntiles = (int)((total + Src::CAP - 1) / Src::CAP);
        if (ntiles == 1) {
            // the union in registers: histogram descent for its key of rank
            // N_eff, then T = the smallest key at or above that bound and
            // krem = N_eff - count(key > T)
            src.load(0, key, pos);
            const int wave = tid >> 6, lane = tid & 63;
            uint32_t mx = 0;
#pragma unroll
            for (int j = 0; j < KPT; ++j) mx = key[j] > mx ? key[j] : mx;
            mx = wave_umax(mx);
            if (lane == 0) sh.wtot[wave] = mx;
            __syncthreads();
            kmax = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) kmax = sh.wtot[w] > kmax ? sh.wtot[w] : kmax;
            __syncthreads();
            const uint32_t tb = descend<KPT>(key, (uint32_t)n_eff, 1u, kmax, sh.hist);
            uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
            for (int j = 0; j < KPT; ++j) mn = key[j] >= tb && key[j] < mn ? key[j] : mn;
            mn = ~wave_umax(~mn);
            if (lane == 0) sh.wtot[wave] = mn;
            __syncthreads();
            thr = 0xFFFFFFFFu;
#pragma unroll
            for (int w = 0; w < NW; ++w) thr = sh.wtot[w] < thr ? sh.wtot[w] : thr;
            __syncthreads();
            uint32_t gt = 0;
#pragma unroll
            for (int j = 0; j < KPT; ++j) gt += key[j] > thr ? 1u : 0u;
            gt = wave_sum(gt);
            if (lane == 0) sh.wtot[wave] = gt;
            __syncthreads();
            gt = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) gt += sh.wtot[w];
            krem = (uint32_t)n_eff - gt;
            __syncthreads();
        } else {
            find_threshold<NT, KPT>(src, ntiles, (uint32_t)n_eff, key, pos, sh, thr, krem, kmax);
        }
        if (check) {   // exact iff every chunk's cutoff is <= the union's threshold key
            if (tid == 0) bad = 0u;
            __syncthreads();
            for (int c = tid; c < nch; c += NT)
                if (meta[c].z > thr) bad = 1u;
            __syncthreads();
            if (bad != 0u) return false;
        }
        compact<NT, KPT>(src, ntiles, thr, krem, (uint32_t)n_eff, key, pos, sh, oi, ov, ou);
        return true;
    };
    // first the lists as published, with the cutoff check; then, if that
    // fails, the union completed for thr (the union's key of rank N_eff, or 0
    // when there was none), which needs no check
    bool rec = false;
    bool ok = false;
    int flag = 0;
#pragma unroll 1
    for (int attempt = 0; attempt < 2 && !ok; ++attempt) {
        ok = select(attempt == 0 ? 0xFFFFFFFFu : thr, attempt == 0, rec);
        if (attempt == 1) flag = ok ? 2 : 1;
    }
    if (!ok) {
        // dense fallback: this head's logits over all L positions, then a full select
        head_logits<T, DH>(q, k, b, i, h_q, h_k, S_max, L, qf ? 1.f : scale, srow,
                           reinterpret_cast<float*>(sh.hist), qf);
        uint32_t key[KPT];
        int32_t pos[KPT];
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
    kmax_out = kmax;   // uniform
    if (tid == 0) {
        row_max[row] = key_float(kmax);
        row_cnt[row] = n_eff;
        row_flag[row] = flag;
    }
}

// LSE of a row from its chunks' {max, sum exp(z - max)}: M + log sum_c s_c
// e^(m_c - M), M = max_c m_c. Also the largest chunk cutoff. Uniform results.
struct RowStats {
    float M, lse;
    uint32_t maxcut;
};
__device__ inline RowStats row_stats(const float2* __restrict__ stat, const uint4* __restrict__ meta,
                                     int nch, uint4* red, float* redf) {
    constexpr int NT = kUnionThreads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t km = 0, cm = 0;
    for (int c = tid; c < nch; c += NT) {
        const uint32_t kx = float_key(stat[c].x);
        km = kx > km ? kx : km;
        const uint32_t cu = meta[c].z;
        cm = cu > cm ? cu : cm;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t y = (uint32_t)__shfl_xor((int)km, o, 64);
        const uint32_t z = (uint32_t)__shfl_xor((int)cm, o, 64);
        km = y > km ? y : km;
        cm = z > cm ? z : cm;
    }
    if (lane == 0) red[wave] = make_uint4(km, cm, 0u, 0u);
    __syncthreads();
    km = 0;
    cm = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        km = red[w].x > km ? red[w].x : km;
        cm = red[w].y > cm ? red[w].y : cm;
    }
    RowStats r;
    r.M = key_float(km);
    r.maxcut = cm;
    float se = 0.f;
    for (int c = tid; c < nch; c += NT) {
        const float2 st = stat[c];
        se += st.y * __expf(st.x - r.M);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) se += __shfl_xor(se, o, 64);
    if (lane == 0) redf[wave] = se;
    __syncthreads();
    float S = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) S += redf[w];
    r.lse = r.M + __logf(S);
    return r;
}

// Atop-N calibration of one row (all threads of the workgroup): tau = exp(T -
// LSE) with T the smallest kept logit, LSE from the row's chunk statistics;
// NaN when nothing is kept. Written by thread 0 when `write`.
__device__ inline void calib_tau(const float2* __restrict__ stat, const uint4* __restrict__ meta,
                                 int nch, float T, bool any, uint4* red, float* redf, float* tau,
                                 bool write) {
    float t = __builtin_nanf("");
    if (any) {   // uniform
        const RowStats rs = row_stats(stat, meta, nch, red, redf);
        t = __expf(T - rs.lse);
    }
    if (write && threadIdx.x == 0) *tau = t;
}

// ---- union select, one workgroup per row -------------------------------------------
// Fast path, for rows of at most 256 chunks whose union of lists holds at most
// 256 KPT entries: thread t takes entries [KPT t, KPT t + KPT) of the lists
// laid end to end (load_union_fast), read with 16-byte loads straight from the
// lists the chunks' records point at. Thread order is therefore position
// order. The union's key of
// rank N_eff, T, is searched in [max chunk cutoff, max key]: the count of keys
// at or above the lower end being >= N_eff is exactly the proof that every
// chunk cutoff is <= T, so the result is exact. The search is a histogram
// descent: each pass spreads the keys of the current range over 256 LDS bins
// (shared-memory atomics), and every wave then scans the 256 bins itself to
// pick the bin holding rank N_eff, so a pass costs one barrier and narrows
// the range by 8 bits (at most four passes); it stops early as soon as the
// keys at or above a bin's lower end are exactly N_eff. Compaction is one
// workgroup prefix scan of the packed (above T, equal to T) counts: equal keys
// at T are taken in position order. The kept entries are staged in LDS and
// written with 16-byte stores. Rows the fast path cannot take (a union larger
// than 256 KPT, or the proof failing) go through union_row in the same workgroup:
// the multi-tile union select, or the dense recompute.
// One wave's copy of a row's union layout for the fast path: where chunk c's
// list starts in the pool (even; bit 0 set when its length is odd) and the
// exclusive prefix of the lengths rounded up to even. Each wave builds its own
// copy, so no workgroup barrier is needed before the list loads.
struct WaveUnion {
    int64_t coff[kUnionThreads];
    uint32_t pref[kUnionThreads + 1];
};
struct FastShared {
    uint32_t hist[3][kUnionThreads];       // one bin per thread, three in rotation
    uint4 red[kUnionThreads / 64];         // wave maxima: max key, max cutoff, overflow
    uint32_t scan[kUnionThreads / 64];     // wave totals of the compaction scan
    WaveUnion wu[kUnionThreads / 64];
};

// Chunk records of a row, requested at kernel start before the row length is
// known: lane l holds chunks [l cpl, l cpl + cpl), cpl = ceil(nchunk / 64)
// (at most 4: the fast path takes rows of at most 256 chunks).
struct ChunkRecs {
    uint4 m[4];
    int cpl;
};
template <class Rec>
__device__ inline ChunkRecs load_chunk_recs(const Rec* __restrict__ rec, int nchunk, int lane) {
    ChunkRecs r;
    r.cpl = (nchunk + 63) >> 6;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = lane * r.cpl + j;
        r.m[j] = make_uint4(0u, 0u, 0u, 0u);
        if (j < r.cpl && c < nchunk) r.m[j] = rec[c];
    }
    return r;
}

// Fast-path load of a row's union of chunk lists (nch <= 256 chunks): thread
// t takes entries [KPT t, KPT t + KPT) of the lists laid end to end in chunk
// order, so thread order is position order and any split of the union among
// the chunks fits as long as the union holds at most 256 KPT entries (a chunk
// that published its whole list, a recency window say, included). Lists
// start at even pool entries and are allocated in whole pairs: with the
// lengths rounded up to even every pair below is one aligned 16-byte load
// inside the list's allocation; the pad entry of an odd list and every slot
// past the union read as key 0 (below every real key). Returns the union's
// size (uniform); maxcut = the largest chunk cutoff. wu: this wave's LDS.
template <int KPT>
__device__ inline uint32_t load_union_fast(const uint2* __restrict__ cand, const ChunkRecs& cr,
                                           int nch, WaveUnion& wu, uint32_t& maxcut,
                                           uint32_t (&key)[KPT], int32_t (&pos)[KPT]) {
    const int tid = threadIdx.x, lane = tid & 63;
    uint32_t run = 0, mc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = lane * cr.cpl + j;
        if (j < cr.cpl && c < nch) {
            run += (cr.m[j].y + 1u) & ~1u;
            mc = cr.m[j].z > mc ? cr.m[j].z : mc;
        }
    }
    uint32_t tot;
    uint32_t at = wave_incl_scan(run, tot) - run;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = lane * cr.cpl + j;
        if (j < cr.cpl && c < nch) {
            wu.pref[c] = at;
            wu.coff[c] = (int64_t)(((uint64_t)cr.m[j].w << 32) | cr.m[j].x) | (int64_t)(cr.m[j].y & 1u);
            at += (cr.m[j].y + 1u) & ~1u;
        }
    }
    if (lane == 0) wu.pref[nch] = tot;
    maxcut = wave_umax(mc);
    // this wave's LDS stores are complete before its lanes read each other's
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const uint32_t e0 = (uint32_t)(KPT * tid);
    int c = 0;
    if (e0 < tot) {   // the last chunk whose range starts at or before e0
        int hi = nch;
        while (hi - c > 1) {
            const int mid = (c + hi) >> 1;
            if (wu.pref[mid] <= e0) c = mid; else hi = mid;
        }
    }
    uint4 ev[KPT / 2];
    uint32_t vm = 0;   // bit s: slot s holds an entry
#pragma unroll
    for (int p = 0; p < KPT / 2; ++p) {
        const uint32_t j = e0 + 2u * (uint32_t)p;
        const uint4* a = reinterpret_cast<const uint4*>(cand);   // past the union: unused
        if (j < tot) {
            while (wu.pref[c + 1] <= j) ++c;
            const int64_t cw = wu.coff[c];
            const uint32_t off = j - wu.pref[c];
            const uint32_t tl = wu.pref[c + 1] - wu.pref[c] - (uint32_t)(cw & 1);
            a = reinterpret_cast<const uint4*>(cand + ((cw & ~(int64_t)1) + off));
            vm |= (off < tl ? 1u : 0u) << (2 * p);
            vm |= (off + 1u < tl ? 1u : 0u) << (2 * p + 1);
        }
        ev[p] = *a;
    }
#pragma unroll
    for (int s = 0; s < KPT; ++s) {
        const uint4 e = ev[s >> 1];
        pos[s] = (int32_t)((s & 1) ? e.z : e.x);
        key[s] = (vm >> s) & 1u ? ((s & 1) ? e.w : e.y) : 0u;
    }
    return tot;
}
// The fast path's output staging (indices, then logits) follows FastShared.
__host__ __device__ constexpr size_t select_stage_offset() {
    return (sizeof(FastShared) + 15) & ~(size_t)15;
}


// Four workgroups per CU (<= 128 VGPRs): the general code spills at this
// bound, which only costs the rare rows that need it. Dynamic LDS:
// max(sizeof(UnionShared), select_stage_offset() + 8 nst) bytes, nst >= the
// kept entries of any fast-path row, a multiple of 4.
//
// SparQ-style inputs of the select (MODE 2; empty for the other modes, so
// they carry no extra kernel arguments).
template <int MODE> struct SqArg {};
// The fused decode step (MODE 1) as an Atop-N calibration step: with tau set,
// the row's tau = exp(T - LSE) is written as well, T the smallest kept logit
// and LSE the log-sum-exp of all logits from the chunk statistics.
template <> struct SqArg<1> {
    const float2* stat;     // nullable [rows][nchunk] chunk softmax statistics
    float* tau;             // nullable [rows]
};
template <> struct SqArg<2> {
    const float* qm;        // [rows][DH] q / tau on the kept dims (the approximate logits)
    const float2* stat;     // [rows][nchunk] chunk softmax statistics of those logits
    int local;              // window: the last min(local, L) positions are always kept
    const float* vmean;     // nullable [B][h_v][DH] running value means (Step 3)
    float* alpha_out;       // nullable [rows]
};
template <int MODE> __device__ inline int sq_local(const SqArg<MODE>&) { return 0; }
__device__ inline int sq_local(const SqArg<2>& a) { return a.local; }
template <int MODE> __device__ inline const float* sq_qm(const SqArg<MODE>&, int, int) { return nullptr; }
__device__ inline const float* sq_qm(const SqArg<2>& a, int row, int dh) {
    return a.qm + (int64_t)row * dh;
}

// MODE 1 (fused): the workgroup forms the softmax weights of the kept entries
// and gathers their value rows (gather.h), writing out[row] directly: the
// kept list never leaves LDS on the fast path (sel_idx / sel_val are not
// written; idx_out is, when given). Rows are then mapped XCD-aware so the
// g_v query heads of a value head share that XCD's L2. Rows of the general
// code write their list to memory first and read it back after a fence.
// Dynamic LDS with FUSE adds the gather's reduction area after the staging:
// nst a multiple of 256 and max(sizeof(UnionShared), select_stage_offset() +
// 8 nst + 4 (4 DH + 4)) bytes. With nsplit > 1 (few rows) each row has
// nsplit workgroups: all of them run the same selection, each gathers its
// slice of the kept list (whole gather batches, in position order) and
// stores its partial sums in split_part [rows][nsplit][DH]; the part that
// finishes last (split_cnt, cleared by the K-scan of the same call) adds
// the partials in part order and writes the row, so the result does not
// depend on which part finishes last. Rows of the general code are done
// whole by part 0.
// MODE 2 (SparQ): the candidates rank approximate logits over the first
// L - min(local, L) positions, N - local of them are kept and the window is
// appended; the kept key rows are then gathered to rescore them exactly
// (logits q.K / sqrt(d), and the approximate ones for alpha, the approximate
// softmax mass of the kept set over the row's log-sum-exp from the chunk
// statistics), and the value gather mixes in vmean with weight 1 - alpha. The
// whole kept list (N entries) is staged in LDS: nst >= N.
template <typename T, int DH, int KPT, int MODE>
__global__ __launch_bounds__(kUnionThreads, 4) void select_union(
    const uint2* __restrict__ cand, const uint4* __restrict__ cand_meta,
    const int32_t* __restrict__ lens, int h_q, int h_k, int N, int64_t S_max, int nchunk, int nst,
    int32_t* __restrict__ sel_idx, float* __restrict__ sel_val, float* __restrict__ row_max,
    int32_t* __restrict__ row_cnt, int32_t* __restrict__ idx_out, int32_t* __restrict__ row_flag,
    const T* __restrict__ q, const T* __restrict__ k, float* __restrict__ scores,
    int64_t s_stride, float scale, const T* __restrict__ v, float* __restrict__ out, int h_v,
    int rows, SqArg<MODE> sq, int chunk, int nsplit, float* __restrict__ split_part,
    int32_t* __restrict__ split_cnt) {
    static_assert(KPT % 2 == 0, "entries are loaded in pairs");
    constexpr bool FUSE = MODE == 1;
    constexpr bool SPQ = MODE == 2;
    constexpr int NT = kUnionThreads;
    using G = Gather<T, DH>;
    static_assert(MODE == 1 || MODE == 2, "fused decode / calibration, or SparQ");
    static_assert(NT == kGatherThreads, "one gather workgroup per row");
    extern __shared__ __attribute__((aligned(16))) unsigned char sel_lds[];
    FastShared& F = *reinterpret_cast<FastShared*>(sel_lds);
    UnionShared& U = *reinterpret_cast<UnionShared*>(sel_lds);
    // the nsplit parts of a row are adjacent logical workgroups
    const int lid = xcd_logical((int)blockIdx.x, rows * nsplit);
    if (lid >= rows * nsplit) return;   // the grid is rounded up to whole XCD shares
    const int row = lid / nsplit;
    const int part = lid - row * nsplit;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = row / h_q;
    // the row's chunk records, requested together with the length (no second
    // round trip before the list loads): lane l's chunks, and this thread's
    // chunk in the per-chunk layout of a full-length row
    const ChunkRecs crec = load_chunk_recs(cand_meta + (int64_t)row * nchunk, nchunk, lane);
    const int tpc_full = nchunk <= NT ? NT / nchunk : 1;
    const int c_full = tid / tpc_full < nchunk ? tid / tpc_full : nchunk - 1;
    const uint4 m_full = cand_meta[(int64_t)row * nchunk + c_full];
    const int64_t Lrow = clamp_len(lens[b], S_max);
    // ranked positions [0, L) and the count kept from them (SparQ: the window is not ranked)
    const int local = sq_local(sq);
    const int64_t L = SPQ ? Lrow - (local < Lrow ? local : Lrow) : Lrow;
    const int n_rank = SPQ ? N - local : N;
    const int n_eff = (int)((int64_t)n_rank < L ? (int64_t)n_rank : L);
    const int nch = (int)((L + chunk - 1) / chunk);
    // fused gather: the value head's rows, the staged lists and the reduction area
    const T* vb = v + (int64_t)(b * h_v + (row - b * h_q) / (h_q / h_v)) * S_max * DH;
    int32_t* g_pos = reinterpret_cast<int32_t*>(sel_lds + select_stage_offset());
    float* g_w = reinterpret_cast<float*>(g_pos + nst);
    float* g_red = g_w + nst;
    auto general = [&] {
        uint32_t gkmax = 0u;
        union_row<T, DH>(row, U, cand, cand_meta, lens, h_q, h_k, N, S_max, nchunk, sel_idx,
                         sel_val, row_max, row_cnt, SPQ ? nullptr : idx_out, row_flag, q, k,
                         scores, s_stride, scale, L, n_eff, sq_qm(sq, row, DH), chunk, gkmax);
        if constexpr (FUSE) {
            // the list union_row wrote, read back in blocks of nst entries by the
            // same workgroup: its waves share one CU's caches, so completed
            // stores and the barrier's workgroup-scope release / acquire order
            // these global accesses (a device-scope fence would also write back
            // and invalidate the XCD's whole L2, which every other workgroup on
            // it pays for). The count and the row max come from registers, so
            // every address below is bounded by the row's N slots whatever the
            // memory holds.
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's stores have completed
            __syncthreads();
            float* o = out + (int64_t)row * DH;
            const int cnt = n_eff;   // union_row keeps exactly N_eff <= N
            if (cnt <= 0) {   // no kept entry (L_b = 0): out = 0
                for (int c = tid; c < DH; c += NT) o[c] = 0.f;
                if (sq.tau && tid == 0) sq.tau[row] = __builtin_nanf("");
                return;
            }
            const float mrow = key_float(gkmax);
            if (sq.tau) {   // uniform: T is the smallest of the kept logits
                uint32_t mk = 0xFFFFFFFFu;
                for (int e = tid; e < cnt; e += NT)
                    mk = min(mk, float_key(wg_load(sel_val + (int64_t)row * N + e)));
                mk = ~wave_umax(~mk);
                if (lane == 0) F.scan[wave] = mk;
                __syncthreads();
                mk = 0xFFFFFFFFu;
#pragma unroll
                for (int w = 0; w < NT / 64; ++w) mk = min(mk, F.scan[w]);
                __syncthreads();
                calib_tau(sq.stat + (int64_t)row * nchunk, cand_meta + (int64_t)row * nchunk, nch,
                          key_float(mk), true, F.red, reinterpret_cast<float*>(F.scan),
                          sq.tau + row, true);
            }
            float acc[G::EPL];
#pragma unroll
            for (int c = 0; c < G::EPL; ++c) acc[c] = 0.f;
            float lsum = 0.f;
#pragma unroll 1
            for (int e0 = 0; e0 < cnt; e0 += nst) {
                const int ne = cnt - e0 < nst ? cnt - e0 : nst;
                for (int e = tid; e < nst; e += NT) {
                    int32_t pos = 0;
                    float w = 0.f;
                    if (e < ne) {
                        pos = wg_load(sel_idx + (int64_t)row * N + e0 + e);
                        pos = pos < 0 ? 0 : (pos >= S_max ? (int32_t)(S_max - 1) : pos);
                        w = __expf(wg_load(sel_val + (int64_t)row * N + e0 + e) - mrow);
                    }
                    g_pos[e] = pos;
                    g_w[e] = w;
                    lsum += w;
                }
                __syncthreads();
                G::run(vb, g_pos, g_w, ne, acc);
                __syncthreads();
            }
            G::finish(acc, lsum, g_red, o);
        }
    };
    // The fast path returns false, with every thread past a barrier, when the
    // row needs the general code; that call sits outside it so the fast path's
    // register arrays are dead across it.
    auto fast = [&]() -> bool {
        int32_t* ou = idx_out ? idx_out + (int64_t)row * N : nullptr;
        int32_t* st_idx = reinterpret_cast<int32_t*>(sel_lds + select_stage_offset());
        float* st_val = reinterpret_cast<float*>(st_idx + nst);

        F.hist[0][tid] = 0u;
        // this thread's KPT entries of the union, in position order: when every
        // chunk's list fits the runs of its tpc = 256 / chunks threads (the
        // usual case), thread t takes a run of P consecutive entries of chunk
        // t / tpc (P even, so runs start on 16-byte boundaries); otherwise the
        // lists are laid end to end (load_union_fast)
        uint32_t key[KPT];
        int32_t pos[KPT];
        uint32_t wcut, wo;
        const int tpc = NT / nch;
        uint32_t lmax = 0;
    #pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int cj = lane * crec.cpl + j;
            if (j < crec.cpl && cj < nch) lmax = crec.m[j].y > lmax ? crec.m[j].y : lmax;
        }
        lmax = wave_umax(lmax);
        if (((((lmax + (uint32_t)tpc - 1u) / (uint32_t)tpc) + 1u) & ~1u) <= (uint32_t)KPT) {
            const int c = tid / tpc;
            const int sub = tid - c * tpc;
            const bool cv = c < nch;
            const uint4 m = nch == nchunk ? m_full : cand_meta[(int64_t)row * nchunk + (cv ? c : nch - 1)];
            const uint32_t cnt = cv ? m.y : 0u;
            const uint32_t P = (((cnt + (uint32_t)tpc - 1u) / (uint32_t)tpc) + 1u) & ~1u;
            const uint32_t j0 = (uint32_t)sub * P;
            const uint32_t mine = cnt > j0 ? (cnt - j0 < P ? cnt - j0 : P) : 0u;
            const uint32_t npair = (mine + 1u) >> 1;
            // pairs past the run re-read its last pair (an empty run reads the
            // pool's first pair), so every load is unconditional and in bounds
            const uint4* run = reinterpret_cast<const uint4*>(cand + ((((uint64_t)m.w << 32) | m.x) + j0));
            uint4 ev[KPT / 2];
    #pragma unroll
            for (int p = 0; p < KPT / 2; ++p) {
                const uint4* a = npair ? run + ((uint32_t)p < npair ? (uint32_t)p : npair - 1u)
                                       : reinterpret_cast<const uint4*>(cand);
                ev[p] = *a;
            }
    #pragma unroll
            for (int s = 0; s < KPT; ++s) {
                const uint4 e = ev[s >> 1];
                pos[s] = (int32_t)((s & 1) ? e.z : e.x);
                key[s] = (uint32_t)s < mine ? ((s & 1) ? e.w : e.y) : 0u;
            }
            wcut = wave_umax(cv ? m.z : 0u);
            wo = 0u;
        } else {
            const uint32_t utot = load_union_fast<KPT>(cand, crec, nch, F.wu[wave], wcut, key, pos);
            wo = utot > (uint32_t)(NT * KPT) ? 1u : 0u;   // does not fit
        }
        uint32_t kmax = 0;
    #pragma unroll
        for (int s = 0; s < KPT; ++s) kmax = key[s] > kmax ? key[s] : kmax;
        {
            const uint32_t wk = wave_umax(kmax);
            if (lane == 0) F.red[wave] = make_uint4(wk, wcut, wo, 0u);
        }
        __syncthreads();
        uint32_t maxcut = 0, ovf = 0;
        kmax = 0;
    #pragma unroll
        for (int w = 0; w < NT / 64; ++w) {
            const uint4 r = F.red[w];
            kmax = r.x > kmax ? r.x : kmax;
            maxcut = r.y > maxcut ? r.y : maxcut;
            ovf |= r.z;
        }
        uint32_t lo = maxcut > 1u ? maxcut : 1u;
        uint32_t hi = kmax;
        if (ovf != 0u || hi < lo) {   // uniform; hi < lo: no key reaches the largest cutoff
            __syncthreads();
            return false;
        }

        // histogram descent for T
        uint32_t need = (uint32_t)n_eff, Tk = 0;
    #pragma unroll 1
        for (int pass = 0;; ++pass) {
            uint32_t* h = F.hist[pass % 3];
            F.hist[(pass + 1) % 3][tid] = 0u;   // last read two passes ago
            const uint32_t span = hi - lo;
            const int nb = span ? 32 - __clz((int)span) : 0;
            const int shift = nb > 8 ? nb - 8 : 0;
    #pragma unroll
            for (int s = 0; s < KPT; ++s)
                if (key[s] >= lo && key[s] <= hi)
                    __hip_atomic_fetch_add(h + ((key[s] - lo) >> shift), 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
            __syncthreads();
            // lane l holds bins 255-4l (top) down to 252-4l; every wave scans all
            const uint4 hv = reinterpret_cast<const uint4*>(h)[63 - lane];
            const uint32_t lsum = (hv.x + hv.y) + (hv.z + hv.w);
            uint32_t total;
            const uint32_t incl = wave_incl_scan(lsum, total);   // keys in bins >= 252-4l
            if (pass == 0 && total < need) {   // uniform: the proof fails
                __syncthreads();
                return false;
            }
            const uint32_t above0 = incl - lsum;
            const uint64_t hit = ballot(incl >= need && above0 < need);
            const int hl = (int)__builtin_ctzll(hit);   // exactly one lane
            uint32_t bin = 255u - 4u * (uint32_t)lane, above = above0, inbin = hv.w;
            if (above + hv.w < need) {
                above += hv.w; bin -= 1u; inbin = hv.z;
                if (above + hv.z < need) {
                    above += hv.z; bin -= 1u; inbin = hv.y;
                    if (above + hv.y < need) { above += hv.y; bin -= 1u; inbin = hv.x; }
                }
            }
            bin = (uint32_t)__builtin_amdgcn_readlane((int)bin, hl);
            above = (uint32_t)__builtin_amdgcn_readlane((int)above, hl);
            inbin = (uint32_t)__builtin_amdgcn_readlane((int)inbin, hl);
            need -= above;
            lo += bin << shift;
            const uint32_t wmask = (1u << shift) - 1u;
            hi = hi - lo <= wmask ? hi : lo + wmask;
            if (inbin == need || shift == 0) {   // keys >= lo are exactly N_eff, or the bin is one key
                Tk = lo;
                break;
            }
        }

        // compaction: keys > T, then the first krem keys == T in position order
        uint32_t ngt = 0, neq = 0;
    #pragma unroll
        for (int s = 0; s < KPT; ++s) {
            ngt += key[s] > Tk ? 1u : 0u;
            neq += key[s] == Tk ? 1u : 0u;
        }
        const uint32_t packed = ngt | (neq << 16);   // each sum <= 256 KPT < 2^16
        uint32_t wtot;
        const uint32_t pincl = wave_incl_scan(packed, wtot);
        if (lane == 0) F.scan[wave] = wtot;
        __syncthreads();
        uint32_t before = pincl - packed, tot = 0;
    #pragma unroll
        for (int w = 0; w < NT / 64; ++w) {
            const uint32_t x = F.scan[w];
            before += w < wave ? x : 0u;
            tot += x;
        }
        const uint32_t krem = (uint32_t)n_eff - (tot & 0xFFFFu);
        uint32_t eq_seen = before >> 16;
        uint32_t slot = (before & 0xFFFFu) + (eq_seen < krem ? eq_seen : krem);
        // fused gather: the staged value is already the softmax weight
        // exp(logit - row max), and the slots past N_eff are cleared here
        const float mrow = key_float(kmax);
        uint32_t kmin = 0xFFFFFFFFu;   // the smallest kept key (Tk may lie below every key)
    #pragma unroll
        for (int s = 0; s < KPT; ++s) {
            const bool eq = key[s] == Tk;
            const bool keep = key[s] > Tk || (eq && eq_seen < krem);
            eq_seen += eq ? 1u : 0u;
            kmin = keep && key[s] < kmin ? key[s] : kmin;
            if (keep) {   // slot < N_eff by construction
                st_idx[slot] = pos[s];
                if constexpr (FUSE) {
                    st_val[slot] = __expf(key_float(key[s]) - mrow);
                } else {
                    st_val[slot] = key_float(key[s]);
                }
            }
            slot += keep ? 1u : 0u;
        }
        if constexpr (FUSE)
            for (int j = n_eff + tid; j < nst; j += NT) {
                st_idx[j] = 0;
                st_val[j] = 0.f;
            }
        __syncthreads();
        if (tid == 0 && part == 0) {
            row_max[row] = key_float(kmax);
            row_cnt[row] = n_eff;
            row_flag[row] = 0;
        }
        if constexpr (FUSE) {
            if (sq.tau) {   // uniform: T, the N_eff-th largest logit, is the smallest kept one
                const uint32_t wm = ~wave_umax(~kmin);
                if (lane == 0) F.scan[wave] = wm;
                __syncthreads();
                uint32_t mk = 0xFFFFFFFFu;
    #pragma unroll
                for (int w = 0; w < NT / 64; ++w) mk = min(mk, F.scan[w]);
                // row_stats writes F.scan only after its first barrier
                calib_tau(sq.stat + (int64_t)row * nchunk, cand_meta + (int64_t)row * nchunk,
                          nch, key_float(mk), true, F.red, reinterpret_cast<float*>(F.scan),
                          sq.tau + row, part == 0);
            }
            // weights of the staged entries in place; the gather reads positions
            // and weights up to nst (weight 0, row 0 past n_eff)
            if (ou && part == 0)
                for (int j = tid; j < N; j += NT) ou[j] = j < n_eff ? st_idx[j] : -1;
            // the weights summed slot by slot (the order the unfused value
            // gather uses, so both give the same bits); nst is whole batches
            gather_staged<T, DH>(vb, st_idx, st_val, n_eff, nst, g_red, &F.scan[0], row, part,
                                 nsplit, split_part, split_cnt, out + (int64_t)row * DH);
            return true;
        }
        return true;   // SparQ: the list stays staged for the tail
    };
    if constexpr (!SPQ) {
        // no kept entry, too many chunks, or no proof: the general code, whole
        // row in part 0 (the decision is the same in every part of the row)
        if (n_eff == 0 || nch > NT || crec.cpl > 4 || !fast())
            if (part == 0) general();
        return;
    } else {
        int32_t* st_idx = g_pos;
        float* st_val = g_w;
        if (n_eff == 0 && tid == 0) {   // nothing ranked (only the window, or L_b = 0)
            row_max[row] = -__builtin_inff();
            row_cnt[row] = 0;
            row_flag[row] = 0;
        }
        if (n_eff > 0 && (nch > NT || crec.cpl > 4 || !fast())) {
            // the general code writes the list; this workgroup reads it back into
            // the stage (completed stores and the barrier order the global
            // accesses within it; n_eff bounds the reads)
            general();
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
            __syncthreads();
            for (int e = tid; e < n_eff; e += NT) {
                int32_t p = wg_load(sel_idx + (int64_t)row * N + e);
                st_idx[e] = p < 0 ? 0 : (p >= L ? (int32_t)(L - 1) : p);
            }
        }
        // the window follows the ranked entries (all below L); pad with row 0
        const int n = n_eff + (int)(Lrow - L);
        for (int e = n_eff + tid; e < nst; e += NT) st_idx[e] = e < n ? (int32_t)(L + (e - n_eff)) : 0;
        __syncthreads();
        if (idx_out)
            for (int e = tid; e < N; e += NT) idx_out[(int64_t)row * N + e] = e < n ? st_idx[e] : -1;
        float* o = out + (int64_t)row * DH;
        if (n == 0) {   // L_b = 0: nothing kept
            for (int c = tid; c < DH; c += NT) o[c] = 0.f;
            if (sq.alpha_out && tid == 0) sq.alpha_out[row] = 0.f;
            return;
        }
        // log-sum-exp of the approximate logits over all L_b positions
        float* sred = g_red + 4 * DH + 4;   // [4] uint4 + [4] + [8] floats past the gather's area
        const int nchr = (int)((Lrow + chunk - 1) / chunk);
        const RowStats rs = row_stats(sq.stat + (int64_t)row * nchunk,
                                      cand_meta + (int64_t)row * nchunk, nchr,
                                      reinterpret_cast<uint4*>(sred), sred + 16);
        // exact logits of the kept rows, and alpha from their approximate ones
        using KD = KeyDots<T, DH>;
        const int i = row - b * h_q;
        const T* kb = k + (int64_t)(b * h_k + i / (h_q / h_k)) * S_max * DH;
        float qa[G::EPL], qb[G::EPL];
        {
            const int sub = lane % G::LPR;
            const T* qr = q + (int64_t)row * DH + sub * G::EPL;
            const float* qmr = sq.qm + (int64_t)row * DH + sub * G::EPL;
#pragma unroll
            for (int c = 0; c < G::EPL; ++c) {
                float x;
                if constexpr (sizeof(T) == 2)
                    x = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(qr)[c] << 16);
                else
                    x = reinterpret_cast<const float*>(qr)[c];
                qa[c] = x * scale;
                qb[c] = qmr[c];
            }
        }
        float se = 0.f, mz = -__builtin_inff();
        KD::run(kb, st_idx, n, qa, qb, st_val, rs.lse, se, mz);
        se = wave_fsum(se);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mz = fmaxf(mz, __shfl_xor(mz, off, 64));
        if (lane == 0) {
            sred[20 + wave] = se;
            sred[24 + wave] = mz;
        }
        __syncthreads();
        float alpha = 0.f, zmax = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) {
            alpha += sred[20 + w];
            zmax = fmaxf(zmax, sred[24 + w]);
        }
        float lsum = 0.f;
        for (int e = tid; e < nst; e += NT) {
            const float wgt = e < n ? __expf(st_val[e] - zmax) : 0.f;
            st_val[e] = wgt;
            lsum += wgt;
        }
        __syncthreads();
        float acc[G::EPL];
#pragma unroll
        for (int c = 0; c < G::EPL; ++c) acc[c] = 0.f;
        G::run(vb, st_idx, st_val, n, acc);
        const int vh = i / (h_q / h_v);
        G::finish(acc, lsum, g_red, o, alpha,
                  sq.vmean ? sq.vmean + (int64_t)(b * h_v + vh) * DH : nullptr);
        if (sq.alpha_out && tid == 0) sq.alpha_out[row] = alpha;
    }
}

// ---- Atop-N: stale-threshold selection and calibration ---------------------------
// "More Value per Key" §3.1 and App. C.1: a calibration step keeps, per
// head, the N-th largest attention probability tau; later steps keep every
// position whose probability reaches tau -- logit z >= log(tau) + LSE(z), the
// log-sum-exp of the row's logits -- at most 2N of them (the first 2N in
// position order here), and attend over those.


struct ThreshShared {
    uint4 red[kUnionThreads / 64];
    float redf[kUnionThreads / 64];
    uint32_t scan[kUnionThreads / 64];
    WaveUnion wu[kUnionThreads / 64];
};
__host__ __device__ constexpr size_t thresh_stage_offset() {
    return (sizeof(ThreshShared) + 15) & ~(size_t)15;
}

// Stale-threshold selection fused with the value gather, one workgroup per
// (b, i) row (nsplit per row when there are few rows, as for the exact
// step). cap = 2N kept slots per row. Fast path: the row's chunk lists are
// complete for the threshold (every chunk cutoff <= theta: every key a chunk
// left out is below its cutoff), at most 256 chunks, and runs of at most KPT
// entries per thread (the layout of select_union): the keys >= theta are
// counted and slotted by one workgroup prefix scan in position order, the
// first cap staged in LDS as positions and softmax weights (shifted by the
// largest kept logit), and gathered (gather_staged). Otherwise part 0
// recomputes the chunks whose cutoff lies above theta (row_flag = 2; all of
// the head's logits when too many do, row_flag = 1), applies the same rule,
// writes the list to sel_idx / sel_val [rows][cap], reads it back into the
// staging and gathers it alone. count_out = positions reaching
// the threshold before the cap; a row keeping none gets out = 0. idx_out
// (nullable) [rows][cap]: the kept positions, -1 padded.
// Dynamic LDS: max(sizeof(UnionShared), thresh_stage_offset() + 8 nst +
// 4 (4 DH + 4)) bytes, nst = cap rounded up to 256.
template <typename T, int DH, int KPT>
__global__ __launch_bounds__(kUnionThreads, 4) void select_thresh(
    const uint2* __restrict__ cand, const uint4* __restrict__ cand_meta,
    const float2* __restrict__ cand_stat, const int32_t* __restrict__ lens,
    const float* __restrict__ tau, int h_q, int h_k, int h_v, int cap, int nst, int64_t S_max,
    int nchunk, int chunk, int32_t* __restrict__ sel_idx, float* __restrict__ sel_val,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ count_out,
    int32_t* __restrict__ row_flag, const T* __restrict__ q, const T* __restrict__ k,
    float* __restrict__ scores, int64_t s_stride, float scale, const T* __restrict__ v,
    float* __restrict__ out, int rows, int nsplit, float* __restrict__ split_part,
    int32_t* __restrict__ split_cnt) {
    static_assert(KPT % 2 == 0, "entries are loaded in pairs");
    constexpr int NT = kUnionThreads;
    static_assert(NT == kGatherThreads, "one gather workgroup per row");
    extern __shared__ __attribute__((aligned(16))) unsigned char thr_lds[];
    ThreshShared& F = *reinterpret_cast<ThreshShared*>(thr_lds);
    UnionShared& U = *reinterpret_cast<UnionShared*>(thr_lds);
    int32_t* st_idx = reinterpret_cast<int32_t*>(thr_lds + thresh_stage_offset());
    float* st_w = reinterpret_cast<float*>(st_idx + nst);
    float* g_red = st_w + nst;
    const int lid = xcd_logical((int)blockIdx.x, rows * nsplit);
    if (lid >= rows * nsplit) return;   // the grid is rounded up to whole XCD shares
    const int row = lid / nsplit;
    const int part = lid - row * nsplit;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = row / h_q;
    const int i = row - b * h_q;
    // the row's chunk records and statistics, requested together with the
    // length (lane l: chunks [l cpl, l cpl + cpl))
    const ChunkRecs crec = load_chunk_recs(cand_meta + (int64_t)row * nchunk, nchunk, lane);
    const int tpc_full = nchunk <= NT ? NT / nchunk : 1;
    const int c_full = tid / tpc_full < nchunk ? tid / tpc_full : nchunk - 1;
    const uint4 m_full = cand_meta[(int64_t)row * nchunk + c_full];
    float2 cst[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = lane * crec.cpl + j;
        cst[j] = make_float2(0.f, 0.f);
        if (j < crec.cpl && c < nchunk) cst[j] = cand_stat[(int64_t)row * nchunk + c];
    }
    const int64_t L = clamp_len(lens[b], S_max);
    const int nch = (int)((L + chunk - 1) / chunk);
    const T* vb = v + (int64_t)(b * h_v + i / (h_q / h_v)) * S_max * DH;
    float* o = out + (int64_t)row * DH;
    int32_t* ou = idx_out ? idx_out + (int64_t)row * cap : nullptr;
    // the row's records, by part 0: kept positions (staged, nk of them),
    // the count before the cap, the recompute flag
    auto records = [&](int nk, int64_t total, int flag) {
        if (part != 0) return;
        if (ou)
            for (int j = tid; j < cap; j += NT) ou[j] = j < nk ? st_idx[j] : -1;
        if (tid == 0) {
            if (count_out) count_out[row] = (int32_t)(total < 0x7FFFFFFF ? total : 0x7FFFFFFF);
            row_flag[row] = flag;
        }
    };
    // staged logits [0, nk) -> weights exp(z - largest staged logit); the
    // rest of the staging (up to nst) zero-weighted at position 0
    auto weigh = [&](int nk) {
        uint32_t mk = 0;
        for (int j = tid; j < nk; j += NT) mk = max(mk, float_key(st_w[j]));
        mk = wave_umax(mk);
        if (lane == 0) F.scan[wave] = mk;
        __syncthreads();
        mk = 0;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) mk = max(mk, F.scan[w]);
        const float m = key_float(mk);
        for (int j = tid; j < nst; j += NT) {
            if (j < nk) {
                st_w[j] = __expf(st_w[j] - m);
            } else {
                st_idx[j] = 0;
                st_w[j] = 0.f;
            }
        }
        __syncthreads();
    };
    if (L == 0) {
        records(0, 0, 0);
        if (part == 0)
            for (int c = tid; c < DH; c += NT) o[c] = 0.f;
        return;
    }
    const uint4* meta = cand_meta + (int64_t)row * nchunk;
    const float2* stat = cand_stat + (int64_t)row * nchunk;
    const float t = tau[row];
    if (nch <= NT && crec.cpl <= 4) {
        // Fast path, rows of at most 256 chunks whose union fits 256 KPT
        // entries: the union loaded as in select_union (per-chunk runs when
        // every list fits them, else laid end to end), and the row's largest
        // cutoff and LSE formed by every wave alike from the chunk records and
        // statistics its lanes hold, so no workgroup barrier comes before the
        // count.
        uint32_t key[KPT];
        int32_t pos[KPT];
        uint32_t mc = 0, lmax = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int cj = lane * crec.cpl + j;
            if (j < crec.cpl && cj < nch) {
                mc = crec.m[j].z > mc ? crec.m[j].z : mc;
                lmax = crec.m[j].y > lmax ? crec.m[j].y : lmax;
            }
        }
        const uint32_t maxcut = wave_umax(mc);
        lmax = wave_umax(lmax);
        const int tpc = NT / nch;
        bool fits = true;
        if (((((lmax + (uint32_t)tpc - 1u) / (uint32_t)tpc) + 1u) & ~1u) <= (uint32_t)KPT) {
            const int c = tid / tpc;
            const int sub = tid - c * tpc;
            const bool cv = c < nch;
            const uint4 m = nch == nchunk ? m_full : meta[cv ? c : nch - 1];
            const uint32_t cnt = cv ? m.y : 0u;
            const uint32_t P = (((cnt + (uint32_t)tpc - 1u) / (uint32_t)tpc) + 1u) & ~1u;
            const uint32_t j0 = (uint32_t)sub * P;
            const uint32_t mine = cnt > j0 ? (cnt - j0 < P ? cnt - j0 : P) : 0u;
            const uint32_t npair = (mine + 1u) >> 1;
            const uint4* run = reinterpret_cast<const uint4*>(cand + ((((uint64_t)m.w << 32) | m.x) + j0));
            uint4 ev[KPT / 2];
#pragma unroll
            for (int p2 = 0; p2 < KPT / 2; ++p2) {
                const uint4* a = npair ? run + ((uint32_t)p2 < npair ? (uint32_t)p2 : npair - 1u)
                                       : reinterpret_cast<const uint4*>(cand);
                ev[p2] = *a;
            }
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const uint4 x = ev[e >> 1];
                pos[e] = (int32_t)((e & 1) ? x.z : x.x);
                key[e] = (uint32_t)e < mine ? ((e & 1) ? x.w : x.y) : 0u;
            }
        } else {
            uint32_t mc2;
            fits = load_union_fast<KPT>(cand, crec, nch, F.wu[wave], mc2, key, pos) <=
                   (uint32_t)(NT * KPT);
        }
        uint32_t kx = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = lane * crec.cpl + j;
            if (j < crec.cpl && c < nch) {
                const uint32_t kc = float_key(cst[j].x);
                kx = kc > kx ? kc : kx;
            }
        }
        const float M = key_float(wave_umax(kx));
        float se = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = lane * crec.cpl + j;
            if (j < crec.cpl && c < nch) se += cst[j].y * __expf(cst[j].x - M);
        }
        const float S = wave_fsum(se);
        // theta = log(tau) + LSE; tau = 0 keeps every position, NaN keeps none
        const float theta = t == t ? __logf(t) + (M + __logf(S)) : __builtin_inff();
        const uint32_t tk = float_key(theta);
        const uint32_t lo = tk > 1u ? tk : 1u;   // key 0 marks an empty slot
        if (fits && maxcut <= tk) {   // uniform: fits, complete for theta
            uint32_t ng = 0;
#pragma unroll
            for (int e = 0; e < KPT; ++e) ng += key[e] >= lo ? 1u : 0u;
            uint32_t wt;
            const uint32_t incl = wave_incl_scan(ng, wt);
            if (lane == 0) F.scan[wave] = wt;
            __syncthreads();
            uint32_t before = incl - ng, total = 0;
#pragma unroll
            for (int w = 0; w < NT / 64; ++w) {
                before += w < wave ? F.scan[w] : 0u;
                total += F.scan[w];
            }
            uint32_t slot = before;
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const bool keep = key[e] >= lo;
                if (keep && slot < (uint32_t)cap) {
                    st_idx[slot] = pos[e];
                    st_w[slot] = key_float(key[e]);
                }
                slot += keep ? 1u : 0u;
            }
            __syncthreads();   // every wave has read F.scan and staged its entries
            const int kept = (int)(total < (uint32_t)cap ? total : (uint32_t)cap);
            records(kept, total, 0);
            if (kept == 0) {   // uniform: nothing reaches the threshold
                if (part == 0)
                    for (int cc = tid; cc < DH; cc += NT) o[cc] = 0.f;
                return;
            }
            weigh(kept);
            gather_staged<T, DH>(vb, st_idx, st_w, kept, nst, g_red, &F.scan[0], row, part,
                                 nsplit, split_part, split_cnt, o);
            return;
        }
    }
    // general: part 0 completes the row's union for theta -- every chunk
    // whose cutoff lies above it recomputed whole (build_union; all of the
    // head's logits when too many are) -- and applies the same rule; the
    // other parts have nothing to do
    if (part != 0) return;
    const RowStats rs = row_stats(stat, meta, nch, F.red, F.redf);
    const float theta = t == t ? __logf(t) + rs.lse : __builtin_inff();
    const uint32_t tk = float_key(theta);
    const uint32_t lo = tk > 1u ? tk : 1u;
    __syncthreads();
    constexpr int KG = kUnionKPT;
    constexpr int NW = NT / 64;
    SelShared& sh = U.sh;
    int32_t* oi = sel_idx + (int64_t)row * cap;
    float* ov = sel_val + (int64_t)row * cap;
    float* srow = scores + (int64_t)row * s_stride;
    uint32_t gk[KG];
    int32_t gp[KG];
    int64_t total = 0;
    // keys >= lo over a source, counted, then the first cap compacted in
    // position order (keys > lo - 1)
    auto apply = [&](const auto& src, int ntiles) {
#pragma unroll 1
        for (int tile = 0; tile < ntiles; ++tile) {
            src.load(tile, gk, gp);
            uint32_t cc = 0;
#pragma unroll
            for (int e = 0; e < KG; ++e) cc += gk[e] >= lo ? 1u : 0u;
            cc = wave_sum(cc);
            if (lane == 0) sh.wtot[wave] = cc;
            __syncthreads();
#pragma unroll
            for (int w = 0; w < NW; ++w) total += sh.wtot[w];
            __syncthreads();
        }
        compact<NT, KG>(src, ntiles, lo - 1u, 0u, (uint32_t)cap, gk, gp, sh, oi, ov, nullptr);
    };
    bool rec = false;
    const int64_t nu = build_union<T, DH>(U, cand, meta, nch, chunk, L, tk, q, k, nullptr, scale,
                                          srow, s_stride, b, i, h_q, h_k, S_max, rec);
    int flag = 2;
    if (nu >= 0) {   // uniform
        using Src = UnionSrc<KG, NW>;
        apply(Src{cand, U.coff, U.pref, nch, nu}, (int)((nu + Src::CAP - 1) / Src::CAP));
    } else {
        flag = 1;
        head_logits<T, DH>(q, k, b, i, h_q, h_k, S_max, L, scale, srow,
                           reinterpret_cast<float*>(sh.hist));
        using Src = DenseSrc<KG, NW>;
        apply(Src{srow, L}, (int)((L + Src::CAP - 1) / Src::CAP));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the compacted list's stores completed
    __syncthreads();
    const int kept = (int)(total < cap ? total : cap);   // from registers: bounds the reads
    // the list back into the staging (cap <= nst) for the gather
    for (int j = tid; j < kept; j += NT) {
        int32_t pp = wg_load(oi + j);
        st_idx[j] = pp < 0 ? 0 : (pp >= L ? (int32_t)(L - 1) : pp);
        st_w[j] = wg_load(ov + j);
    }
    __syncthreads();
    records(kept, total, flag);
    if (kept == 0) {
        for (int cc = tid; cc < DH; cc += NT) o[cc] = 0.f;
        return;
    }
    weigh(kept);
    gather_staged<T, DH>(vb, st_idx, st_w, kept, nst, g_red, &F.scan[0], row, 0, 1, nullptr,
                         nullptr, o);
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

namespace {

// Kept entries the SparQ select stages in LDS at most.
constexpr int kSparqMaxN = 4096;

template <int MODE>
hipError_t go_select_union(const TopmOut& tm, const int32_t* lens, int B, int h_q, int h_k, int d,
                           int N, int64_t S_max, int32_t* sel_idx, float* sel_val,
                           float* row_max, int32_t* row_cnt, int32_t* idx_out, int32_t* row_flag,
                           const void* q, const void* k, float* scores, int64_t s_stride,
                           bool bf16, const void* v, float* out, int h_v,
                           const SqArg<MODE>& sq, int nsplit, float* split_part,
                           int32_t* split_cnt, hipStream_t st) {
    const int chunk = tm.chunk;
    const int nchunk = (int)((S_max + chunk - 1) / chunk);
    const int rows = B * h_q;
    const float scale = (float)(1.0 / __builtin_sqrt((double)d));
    // Register slots per thread for the fast path: the longest run, an even
    // ceil(per_chunk / tpc) with tpc = floor(256 / chunks) threads per chunk
    // and up to per_chunk = 1.25 (1.5 share + 16) keys in a full chunk's list
    // (share = N * 1024 / L, N the ranked count); rows with longer runs take
    // the general code.
    int n_rank = N;
    if constexpr (MODE == 2) n_rank = N - sq.local;
    const double share = (double)n_rank * chunk / (double)S_max;
    int64_t per_chunk = (int64_t)(1.25 * (1.5 * share + 16.0)) + 1;
    per_chunk = per_chunk < chunk ? per_chunk : chunk;
    const int64_t tpc = nchunk <= kUnionThreads ? kUnionThreads / nchunk : 1;
    const int64_t slots = (((per_chunk + tpc - 1) / tpc) + 1) & ~(int64_t)1;
    // staged kept entries: N_eff <= N, and <= the 256 KPT keys in registers
    // (the gathers read them in whole batches: a multiple of 256); SparQ
    // stages the whole list, window included
    auto nst_for = [&](int kpt) -> int {
        if (MODE == 2) return (int)round_up(N, 256);
        int64_t nst = (int64_t)N < (int64_t)kUnionThreads * kpt ? (int64_t)N : (int64_t)kUnionThreads * kpt;
        return (int)((nst + 255) & ~(int64_t)255);
    };
    auto lds_for = [&](int kpt) -> size_t {
        size_t fast = select_stage_offset() + (size_t)nst_for(kpt) * 8;
        fast += (size_t)(4 * d + 4) * sizeof(float);
        if (MODE == 2) fast += 32 * sizeof(float);
        return fast > sizeof(UnionShared) ? fast : sizeof(UnionShared);
    };
    if (MODE != 1) nsplit = 1;
    const unsigned grid = (unsigned)(((rows * nsplit + 7) / 8) * 8);
#define SAGA_SU(T, D, KPT)                                                                       \
    hipLaunchKernelGGL((select_union<T, D, KPT, MODE>), dim3(grid), dim3(kUnionThreads),          \
                       (unsigned)lds_for(KPT), st, tm.cand, tm.meta, lens, h_q, h_k, N, S_max,     \
                       nchunk, nst_for(KPT), sel_idx, sel_val, row_max, row_cnt, idx_out, row_flag, \
                       (const T*)q, (const T*)k, scores, s_stride, scale, (const T*)v, out, h_v,   \
                       rows, sq, chunk, nsplit, split_part, split_cnt)
#define SAGA_SU_K(T, D)                                                                          \
    if (slots <= 8) SAGA_SU(T, D, 8);                                                            \
    else if (slots <= 16) SAGA_SU(T, D, 16);                                                     \
    else SAGA_SU(T, D, 32);
    if (bf16) {
        if (d == 64) { SAGA_SU_K(uint16_t, 64) } else { SAGA_SU_K(uint16_t, 128) }
    } else {
        if (d == 64) { SAGA_SU_K(float, 64) } else { SAGA_SU_K(float, 128) }
    }
#undef SAGA_SU_K
#undef SAGA_SU
    return hipGetLastError();
}

}  // namespace

hipError_t launch_select_pv(const TopmOut& tm, const int32_t* lens, int B, int h_q, int h_k,
                            int h_v, int d, int N, int64_t S_max, int32_t* sel_idx,
                            float* sel_val, float* row_max, int32_t* row_cnt, int32_t* idx_out,
                            int32_t* row_flag, const void* q, const void* k, const void* v,
                            float* scores, int64_t s_stride, float* out, bool bf16, int nsplit,
                            float* split_part, int32_t* split_cnt, float* tau, hipStream_t st) {
    const SqArg<1> cal{tau ? tm.stat : nullptr, tm.stat ? tau : nullptr};
    return go_select_union<1>(tm, lens, B, h_q, h_k, d, N, S_max, sel_idx, sel_val, row_max,
                              row_cnt, idx_out, row_flag, q, k, scores, s_stride, bf16, v, out,
                              h_v, cal, nsplit, split_part, split_cnt, st);
}

bool sparq_select_fits(int N) { return N >= 1 && N <= kSparqMaxN; }

hipError_t launch_select_sparq(const TopmOut& tm, const SparqWs& sw, const int32_t* lens, int B,
                               int h_q, int h_k, int h_v, int d, int N, int local, int64_t S_max,
                               int32_t* sel_idx, float* sel_val, float* row_max, int32_t* row_cnt,
                               int32_t* idx_out, int32_t* row_flag, const void* q, const void* k,
                               const void* v, float* scores, int64_t s_stride, const float* vmean,
                               float* out, float* alpha_out, bool bf16, hipStream_t st) {
    const SqArg<2> sq{sw.qm, tm.stat, local, vmean, alpha_out};
    return go_select_union<2>(tm, lens, B, h_q, h_k, d, N, S_max, sel_idx, sel_val, row_max,
                              row_cnt, idx_out, row_flag, q, k, scores, s_stride, bf16, v, out,
                              h_v, sq, 1, nullptr, nullptr, st);
}

hipError_t launch_select_thresh(const TopmOut& tm, const int32_t* lens, const float* tau, int B,
                                int h_q, int h_k, int h_v, int d, int cap, int64_t S_max,
                                int32_t* sel_idx, float* sel_val, int32_t* idx_out,
                                int32_t* count_out, int32_t* row_flag, const void* q,
                                const void* k, const void* v, float* scores, int64_t s_stride,
                                float* out, bool bf16, int nsplit, float* split_part,
                                int32_t* split_cnt, hipStream_t st) {
    const int chunk = tm.chunk;
    const int nchunk = (int)((S_max + chunk - 1) / chunk);
    const int rows = B * h_q;
    const float scale = (float)(1.0 / __builtin_sqrt((double)d));
    // registers per thread: as for the union select, the lists sized for tm.N
    const double share = (double)tm.N * chunk / (double)S_max;
    int64_t per_chunk = (int64_t)(1.25 * (1.5 * share + 16.0)) + 1;
    per_chunk = per_chunk < chunk ? per_chunk : chunk;
    const int64_t tpc = nchunk <= kUnionThreads ? kUnionThreads / nchunk : 1;
    const int64_t slots = (((per_chunk + tpc - 1) / tpc) + 1) & ~(int64_t)1;
    const int nst = (int)round_up(cap, 256);
    size_t lds = thresh_stage_offset() + (size_t)nst * 8 + (size_t)(4 * d + 4) * sizeof(float);
    lds = lds > sizeof(UnionShared) ? lds : sizeof(UnionShared);
    const unsigned grid = (unsigned)(((rows * nsplit + 7) / 8) * 8);
#define SAGA_ST(T, D, KPT)                                                                       \
    {                                                                                            \
        auto kern = &select_thresh<T, D, KPT>;                                                   \
        if (lds > 64 * 1024) {                                                                   \
            const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), lds);    \
            if (e != hipSuccess) return e;                                                       \
        }                                                                                        \
        hipLaunchKernelGGL(kern, dim3(grid), dim3(kUnionThreads), (unsigned)lds, st, tm.cand,    \
                           tm.meta, tm.stat, lens, tau, h_q, h_k, h_v, cap, nst, S_max, nchunk,  \
                           chunk, sel_idx, sel_val, idx_out, count_out, row_flag, (const T*)q,   \
                           (const T*)k, scores, s_stride, scale, (const T*)v, out, rows, nsplit, \
                           split_part, split_cnt);                                               \
    }
#define SAGA_ST_K(T, D)                                                                          \
    if (slots <= 8) SAGA_ST(T, D, 8)                                                             \
    else if (slots <= 16) SAGA_ST(T, D, 16)                                                      \
    else SAGA_ST(T, D, 32)
    if (bf16) {
        if (d == 64) { SAGA_ST_K(uint16_t, 64) } else { SAGA_ST_K(uint16_t, 128) }
    } else {
        if (d == 64) { SAGA_ST_K(float, 64) } else { SAGA_ST_K(float, 128) }
    }
#undef SAGA_ST_K
#undef SAGA_ST
    return hipGetLastError();
}


}  // namespace saga
