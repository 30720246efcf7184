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
//             hence below T, so exactly the keys >= T are all present). A
//             wave per row settles the common case with all keys in
//             registers; rows it cannot settle go to a workgroup per row,
//             which recomputes the head's logits and selects on them densely
//             when the check fails, so the result is always exact.
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

// ---- union select, one wave per row (the common case) -------------------------------
// Each wave takes one (b, i) row and holds the union of its chunks' candidate
// lists in registers, lane-major: with P = ceil(total / 64), lane l holds
// union elements [l P, l P + P) in slots 0..P-1 (the union is chunk-major,
// so this is ascending position, lane by lane). The union's key of rank
// N_eff, T, is found by bisection of the key range [max cutoff, max key]:
// the count at the lower end being >= N_eff is exactly the proof that every
// chunk cutoff is <= T, so the result is exact. Compaction needs only two
// wave prefix scans (ties kept in position order, then output slots). Rows
// that cannot be settled here -- count(key >= max cutoff) < N_eff, more
// candidates than 64 KPT, or more than kFastChunks chunks -- are flagged
// (row_flag = 2) for the workgroup kernel below.
constexpr int kFastChunks = 128;       // chunk lists per row described in LDS
constexpr int kFastBracket = 512;      // keys left in the bracket before packing

// LDS of one wave: the union (element-major, 64 KPT entries), reused for the
// bracket keys and then for the staged output (n_eff <= 32 KPT pairs).
template <int KPT>
struct FastWaveLds {
    uint2 uni[64 * KPT];
    uint32_t pref[kFastChunks + 1];
    uint32_t coff[kFastChunks];
};

template <int KPT, int NWV>
__global__ __launch_bounds__(64 * NWV) void select_union_fast(
    const uint2* __restrict__ cand, const uint4* __restrict__ cand_meta,
    const int32_t* __restrict__ lens, int rows, int h_q, int h_k, int N, int64_t S_max,
    int nchunk, int32_t* __restrict__ sel_idx, float* __restrict__ sel_val,
    float* __restrict__ row_max, int32_t* __restrict__ row_cnt, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ row_flag) {
    __shared__ FastWaveLds<KPT> lds_all[NWV];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // wave-uniform
    FastWaveLds<KPT>& W = lds_all[wave];
    const int row = blockIdx.x * NWV + wave;
    if (row >= rows) return;   // no workgroup barriers below
    const int b = row / h_q;
    const int i = row - b * h_q;
    const int64_t L = clamp_len(lens[b], S_max);
    const int n_eff = (int)((int64_t)N < L ? (int64_t)N : L);
    int32_t* oi = sel_idx + (int64_t)row * N;
    float* ov = sel_val + (int64_t)row * N;
    int32_t* ou = idx_out ? idx_out + (int64_t)row * N : nullptr;
    for (int s = n_eff + lane; s < N; s += 64) {
        oi[s] = -1;
        ov[s] = -__builtin_inff();
        if (ou) ou[s] = -1;
    }
    if (n_eff == 0) {
        if (lane == 0) {
            row_max[row] = -__builtin_inff();
            row_cnt[row] = 0;
            row_flag[row] = 0;
        }
        return;
    }
    const int nch = (int)((L + kScanChunk - 1) / kScanChunk);
    if (nch > kFastChunks) {
        if (lane == 0) row_flag[row] = 2;
        return;
    }
    // chunk lists: prefix of the counts and pool offsets (relative to the
    // row's first item region) in this wave's LDS, largest cutoff
    uint32_t* pref = W.pref;
    uint32_t* coff = W.coff;
    const uint4* meta = cand_meta + (int64_t)row * nchunk;
    const int g = h_q / h_k;
    const uint2* pool = cand + (int64_t)(b * h_k + i / g) * nchunk * g * kScanChunk;
    uint32_t carry = 0, maxcut = 0;
    for (int c0 = 0; c0 < nch; c0 += 64) {
        const int c = c0 + lane;
        uint4 m = make_uint4(0u, 0u, 0u, 0u);
        if (c < nch) m = meta[c];
        uint32_t tot;
        const uint32_t incl = wave_incl_scan(m.y, tot);
        if (c < nch) {
            pref[c] = carry + incl - m.y;
            coff[c] = (uint32_t)c * g * kScanChunk + m.x;
        }
        carry += tot;
        maxcut = m.z > maxcut ? m.z : maxcut;
    }
    if (lane == 0) pref[nch] = carry;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t y = (uint32_t)__shfl_xor((int)maxcut, o, 64);
        maxcut = y > maxcut ? y : maxcut;
    }
    maxcut = (uint32_t)__builtin_amdgcn_readfirstlane((int)maxcut);   // equal in every lane
    const uint32_t total = carry;
    if (total < (uint32_t)n_eff || total > 64u * KPT) {
        if (lane == 0) row_flag[row] = 2;
        return;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // this wave's LDS writes are visible to it

    // The union, element-major (element j = lane + 64 t): coalesced loads,
    // all issued before any is waited for (unconditional; slots past the
    // union read entry 0 of the row's pool and are discarded), then written to
    // LDS in union order.
    const uint32_t P = (total + 63) / 64;
    {
        uint2 ev[KPT];
        uint32_t kc = 0, cur = pref[0], nxt = pref[1], base = coff[0];
#pragma unroll
        for (int t = 0; t < KPT; ++t) {
            const uint32_t j = (uint32_t)(lane + 64 * t);
            const bool valid = j < total;
            if (valid && j >= nxt) {   // chunk of element j (LDS only)
                do {
                    ++kc;
                } while (pref[kc + 1] <= j);
                cur = pref[kc];
                nxt = pref[kc + 1];
                base = coff[kc];
            }
            ev[t] = pool[valid ? base + (j - cur) : 0u];
        }
#pragma unroll
        for (int t = 0; t < KPT; ++t)
            if ((uint32_t)t < P) W.uni[lane + 64 * t] = ev[t];
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // this wave's LDS writes are visible to it
    // (position, key) lane-major: lane l holds elements [l P, l P + P) in
    // slots 0..P-1 (ascending position); empty slots hold key 0, below every
    // real key
    const uint32_t j0 = (uint32_t)lane * P;
    const uint32_t jend = j0 + P < total ? j0 + P : total;
    uint32_t key[KPT];
    int32_t pos[KPT];
#pragma unroll
    for (int s = 0; s < KPT; ++s) {
        const uint32_t j = j0 + (uint32_t)s;
        const bool valid = j < jend;
        const uint2 v = W.uni[valid ? j : 0u];
        pos[s] = valid ? (int32_t)v.x : -1;
        key[s] = valid ? v.y : 0u;
    }
    uint32_t kmax = 0;
#pragma unroll
    for (int s = 0; s < KPT; ++s) kmax = key[s] > kmax ? key[s] : kmax;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t y = (uint32_t)__shfl_xor((int)kmax, o, 64);
        kmax = y > kmax ? y : kmax;
    }
    kmax = (uint32_t)__builtin_amdgcn_readfirstlane((int)kmax);   // equal in every lane
    // per-lane count of keys >= x (independent partial sums for latency)
    auto lane_ge = [&](uint32_t x) -> uint32_t {
        uint32_t c[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
        for (int s = 0; s < KPT; ++s) c[s & 7] += key[s] >= x ? 1u : 0u;
        return ((c[0] + c[1]) + (c[2] + c[3])) + ((c[4] + c[5]) + (c[6] + c[7]));
    };
    auto wave_min = [&](uint32_t m) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const uint32_t y = (uint32_t)__shfl_xor((int)m, o, 64);
            m = y < m ? y : m;
        }
        return (uint32_t)__builtin_amdgcn_readfirstlane((int)m);   // equal in every lane
    };
    // T: the largest x with count(key >= x) >= n_eff, searched in [a, z) with
    // count(>= a) >= n_eff > count(>= z). Phase 1 bisects over every register
    // slot until at most kFastBracket keys lie in the bracket; those are then
    // packed through LDS into 8 registers per lane, and phase 2 bisects there.
    uint32_t a = maxcut > 1u ? maxcut : 1u;
    uint32_t la = lane_ge(a);
    uint32_t ca = wave_sum(la);
    if (ca < (uint32_t)n_eff) {
        // some chunk's cutoff is above the union's N_eff-th key: not provable here
        if (lane == 0) row_flag[row] = 2;
        return;
    }
    uint64_t z = (uint64_t)kmax + 1;
    uint32_t lz = 0, cz = 0;   // lane / wave counts of keys >= z
    bool found = false;
#pragma unroll 1
    while (z - a > 1 && ca - cz > (uint32_t)kFastBracket) {
        const uint32_t mid = (uint32_t)(a + ((z - a) >> 1));
        const uint32_t lc = lane_ge(mid);
        const uint32_t c = wave_sum(lc);
        if (c == (uint32_t)n_eff) {
            // exactly n_eff keys are >= mid: T is the smallest of them
            uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
            for (int s = 0; s < KPT; ++s)
                if (key[s] >= mid && key[s] < mn) mn = key[s];
            a = wave_min(mn);
            found = true;
            break;
        }
        if (c > (uint32_t)n_eff) {
            a = mid;
            la = lc;
            ca = c;
        } else {
            z = mid;
            lz = lc;
            cz = c;
        }
    }
    if (!found && z - a > 1) {
        // pack the keys in [a, z) (lane by lane) into this wave's LDS area
        uint32_t* bkt = reinterpret_cast<uint32_t*>(W.uni);   // the union is in registers now
        const uint32_t nin = la - lz;
        uint32_t ntot;
        uint32_t at = wave_incl_scan(nin, ntot) - nin;
#pragma unroll
        for (int s = 0; s < KPT; ++s) {
            const bool in = key[s] >= a && (uint64_t)key[s] < z;
            if (in) bkt[at] = key[s];
            at += in ? 1u : 0u;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // this wave's LDS writes are visible to it
        uint32_t kb[kFastBracket / 64];
#pragma unroll
        for (int j = 0; j < kFastBracket / 64; ++j) {
            const uint32_t e = (uint32_t)(lane + 64 * j);
            kb[j] = e < ntot ? bkt[e] : 0u;   // 0 < a: never counted
        }
        // cz stays the count above the bracket at the time of the packing:
        // kb keeps the keys that a lower z leaves above it
#pragma unroll 1
        while (z - a > 1) {
            const uint32_t mid = (uint32_t)(a + ((z - a) >> 1));
            uint32_t lc = 0;
#pragma unroll
            for (int j = 0; j < kFastBracket / 64; ++j) lc += kb[j] >= mid ? 1u : 0u;
            const uint32_t c = cz + wave_sum(lc);
            if (c == (uint32_t)n_eff) {
                uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
                for (int j = 0; j < kFastBracket / 64; ++j)
                    if (kb[j] >= mid && kb[j] < mn) mn = kb[j];
                a = wave_min(mn);
                break;
            }
            if (c > (uint32_t)n_eff) a = mid; else z = mid;
        }
    }
    const uint32_t T = a;

    // Compaction. Keys > T are kept; of the keys == T, the first krem in
    // position order, krem = n_eff - count(> T). Lane-major order is
    // position order, so a scan of the per-lane tie counts ranks the ties and
    // a scan of the per-lane kept counts gives each lane its first output
    // slot. The kept (index, logit) pairs are staged in LDS when they fit and
    // written out with 16-byte stores; otherwise they are stored directly.
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int s = 0; s < KPT; ++s) {
        ngt += key[s] > T ? 1u : 0u;
        neq += key[s] == T ? 1u : 0u;
    }
    uint32_t tot_gt, tot_eq;
    (void)wave_incl_scan(ngt, tot_gt);
    const uint32_t eq_base = wave_incl_scan(neq, tot_eq) - neq;
    const uint32_t krem = (uint32_t)n_eff - tot_gt;
    const uint32_t eq_keep = krem > eq_base ? (krem - eq_base < neq ? krem - eq_base : neq) : 0u;
    const uint32_t nkeep = ngt + eq_keep;
    uint32_t tot_keep;
    uint32_t slot = wave_incl_scan(nkeep, tot_keep) - nkeep;
    const bool staged = n_eff <= 32 * KPT;   // two words per kept entry fit the union area
    int32_t* st_idx = reinterpret_cast<int32_t*>(W.uni);
    float* st_val = reinterpret_cast<float*>(W.uni) + 32 * KPT;
    uint32_t eq_seen = 0;
#pragma unroll
    for (int s = 0; s < KPT; ++s) {
        const bool eq = key[s] == T;
        const bool keep = key[s] > T || (eq && eq_seen < eq_keep);
        eq_seen += eq ? 1u : 0u;
        if (keep && slot < (uint32_t)n_eff) {   // holds by construction; keeps stores in bounds
            if (staged) {
                st_idx[slot] = pos[s];
                st_val[slot] = key_float(key[s]);
            } else {
                oi[slot] = pos[s];
                ov[slot] = key_float(key[s]);
                if (ou) ou[slot] = pos[s];
            }
        }
        slot += keep ? 1u : 0u;
    }
    if (staged) {
        __builtin_amdgcn_s_waitcnt(0xc07f);   // this wave's LDS writes are visible to it
        // 16-byte stores where the rows start 16-byte aligned, else 4-byte ones
        const bool v4 = (((uintptr_t)oi | (uintptr_t)ov | (uintptr_t)ou) & 15u) == 0;
        const int n4 = v4 ? n_eff / 4 : 0;
        for (int j = lane; j < n4; j += 64) {
            const int4 vi = reinterpret_cast<const int4*>(st_idx)[j];
            reinterpret_cast<int4*>(oi)[j] = vi;
            reinterpret_cast<float4*>(ov)[j] = reinterpret_cast<const float4*>(st_val)[j];
            if (ou) reinterpret_cast<int4*>(ou)[j] = vi;
        }
        for (int j = 4 * n4 + lane; j < n_eff; j += 64) {
            oi[j] = st_idx[j];
            ov[j] = st_val[j];
            if (ou) ou[j] = st_idx[j];
        }
    }
    if (lane == 0) {
        row_max[row] = key_float(kmax);
        row_cnt[row] = n_eff;
        row_flag[row] = 0;
    }
}

// ---- union select, one workgroup per row (deferred rows) ---------------------------
// Rows the wave kernel flagged: the union select over any number of
// candidates (register tiles), the cutoff check, and the dense fallback that
// recomputes the head's logits when the check fails. row_flag becomes 0
// (settled from the candidates) or 1 (dense fallback).
struct UnionShared {
    SelShared sh;
    int32_t pref[kMaxChunks + 1];
    int64_t coff[kMaxChunks];
    uint32_t bad;
};

template <typename T, int DH>
__device__ void union_row(
    int row, UnionShared& us, const uint2* __restrict__ cand, const uint4* __restrict__ cand_meta,
    const int32_t* __restrict__ lens, int h_q, int h_k,
    int N, int64_t S_max, int nchunk, int32_t* __restrict__ sel_idx, float* __restrict__ sel_val,
    float* __restrict__ row_max, int32_t* __restrict__ row_cnt, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ row_flag, const T* __restrict__ q, const T* __restrict__ k,
    float* __restrict__ scores, int64_t s_stride, float scale) {
    constexpr int NT = kUnionThreads;
    constexpr int NW = NT / 64;
    constexpr int KPT = kUnionKPT;
    SelShared& sh = us.sh;
    int32_t* pref = us.pref;
    int64_t* coff = us.coff;
    uint32_t& bad = us.bad;
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

template <typename T, int DH>
__global__ __launch_bounds__(kUnionThreads) void select_union(
    const uint2* __restrict__ cand, const uint4* __restrict__ cand_meta,
    const int32_t* __restrict__ lens, int rows, int h_q, int h_k, int N, int64_t S_max,
    int nchunk, int32_t* __restrict__ sel_idx, float* __restrict__ sel_val,
    float* __restrict__ row_max, int32_t* __restrict__ row_cnt, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ row_flag, const T* __restrict__ q, const T* __restrict__ k,
    float* __restrict__ scores, int64_t s_stride, float scale) {
    __shared__ UnionShared us;
    __shared__ uint32_t nflag;
    __shared__ int32_t flagged[kUnionThreads];
    // The rows of this workgroup are blockIdx.x + r * gridDim.x; their flags
    // are read in parallel, kUnionThreads rows per round, and only the flagged
    // ones are processed.
#pragma unroll 1
    for (int r0 = blockIdx.x; r0 < rows; r0 += gridDim.x * kUnionThreads) {
        if (threadIdx.x == 0) nflag = 0u;
        __syncthreads();
        const int rr = r0 + (int)threadIdx.x * gridDim.x;
        if (rr < rows && row_flag[rr] != 0) flagged[atomicAdd(&nflag, 1u)] = rr;
        __syncthreads();
        const uint32_t nf = nflag;
#pragma unroll 1
        for (uint32_t f = 0; f < nf; ++f) {
            union_row<T, DH>(flagged[f], us, cand, cand_meta, lens, h_q, h_k, N, S_max, nchunk,
                             sel_idx, sel_val, row_max, row_cnt, idx_out, row_flag, q, k, scores,
                             s_stride, scale);
            __syncthreads();   // shared state is reused by the next row
        }
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
    const int rows = B * h_q;
    const float scale = (float)(1.0 / __builtin_sqrt((double)d));
    // Register slots per lane for the wave kernel: ceil(union size / 64), the
    // union holding up to 1.25 M = 1.25 (1.5 share + 16) keys per full chunk
    // (share = N * 1024 / L); rows with a larger union are deferred.
    const double share = (double)N * kScanChunk / (double)S_max;
    int64_t per_chunk = (int64_t)(1.25 * (1.5 * share + 16.0)) + 1;
    per_chunk = per_chunk < kScanChunk ? per_chunk : kScanChunk;
    const int64_t slots = ((int64_t)nchunk * per_chunk + 63) / 64;
#define SAGA_SF(KPT, NWV)                                                                        \
    hipLaunchKernelGGL((select_union_fast<KPT, NWV>), dim3((unsigned)((rows + NWV - 1) / NWV)), \
                       dim3(64 * NWV), 0, st, tm.cand, tm.meta, lens, rows, h_q, h_k, N, S_max,   \
                       nchunk, sel_idx, sel_val, row_max, row_cnt, idx_out, row_flag)
    // LDS per wave: 512 KPT bytes of union + 1 KiB of chunk data
    if (slots <= 16) SAGA_SF(16, 4);
    else if (slots <= 32) SAGA_SF(32, 4);
    else if (slots <= 48) SAGA_SF(48, 4);
    else if (slots <= 64) SAGA_SF(64, 2);
    else if (slots <= 96) SAGA_SF(96, 2);
    else SAGA_SF(128, 1);
#undef SAGA_SF
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // deferred rows: a persistent pass that skips the settled ones
    const unsigned grid = (unsigned)(rows < 256 ? rows : 256);
#define SAGA_SU(T, D)                                                                            \
    hipLaunchKernelGGL((select_union<T, D>), dim3(grid), dim3(kUnionThreads), 0, st, tm.cand,    \
                       tm.meta, lens, rows, h_q, h_k, N, S_max, nchunk, sel_idx, sel_val,         \
                       row_max, row_cnt, idx_out, row_flag, (const T*)q, (const T*)k, scores,     \
                       s_stride, scale)
    if (bf16) {
        if (d == 64) SAGA_SU(uint16_t, 64); else SAGA_SU(uint16_t, 128);
    } else {
        if (d == 64) SAGA_SU(float, 64); else SAGA_SU(float, 128);
    }
#undef SAGA_SU
    return hipGetLastError();
}

}  // namespace saga
