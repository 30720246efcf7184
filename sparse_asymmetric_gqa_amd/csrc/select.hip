// Top-N selection per query head: threshold select + compaction.
//
// "More Value per Key" §2.5 Eq. 6 keeps the N largest logits of the row;
// §3.1 and App. C.1 find them by comparing every logit with the N-th largest
// value instead of sorting. Here that threshold is found exactly for the
// current logits (a fresh threshold at every call), and equal logits at the
// threshold are taken in ascending position until exactly N_eff = min(N, L)
// entries are kept.
//
// One 1024-thread workgroup per (b, i) row:
//   1. logits -> order-preserving uint32 keys held in registers (-0 == +0);
//   2. three LDS histogram rounds over 12/10/10-bit digits narrow the key of
//      rank N_eff from the top down to a single value T and the number of
//      ties at T that must be kept;
//   3. compaction in ascending position order: wave ballots + mbcnt give each
//      kept element its slot, a 16-entry scan across waves orders the waves.
// Rows longer than one register tile (16 waves x 64 lanes x KPT) are
// processed tile by tile, re-reading the logits from memory in each round.
#include "saga_internal.h"

namespace saga {
using namespace dev;

namespace {

constexpr int kNW = kSelectThreads / 64;

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

template <int KPT>
__global__ __launch_bounds__(kSelectThreads) void select_topn(
    const float* __restrict__ scores, int64_t s_stride, const int32_t* __restrict__ lens,
    int h_q, int N, int64_t S_max, int32_t* __restrict__ sel_idx, float* __restrict__ sel_val,
    float* __restrict__ row_max, int32_t* __restrict__ row_cnt, int32_t* __restrict__ idx_out) {
    static_assert(KPT % 4 == 0, "KPT must be a multiple of 4");
    constexpr int SEG = KPT * 64;       // positions of one wave in one tile
    constexpr int CAP = kNW * SEG;      // positions of one tile
    __shared__ uint32_t hist[4096];
    __shared__ uint32_t wtot[2 * kNW];
    __shared__ uint32_t bc[4];

    const int row = blockIdx.x;
    const int b = row / h_q;
    const int64_t L = clamp_len(lens[b], S_max);
    const int n_eff = (int)((int64_t)N < L ? (int64_t)N : L);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const float* srow = scores + (int64_t)row * s_stride;
    int32_t* oi = sel_idx + (int64_t)row * N;
    float* ov = sel_val + (int64_t)row * N;
    int32_t* ou = idx_out ? idx_out + (int64_t)row * N : nullptr;

    // slots past N_eff: index -1, logit -inf
    for (int s = n_eff + tid; s < N; s += kSelectThreads) {
        oi[s] = -1;
        ov[s] = -__builtin_inff();
        if (ou) ou[s] = -1;
    }
    if (n_eff == 0) {
        if (tid == 0) {
            row_max[row] = -__builtin_inff();
            row_cnt[row] = 0;
        }
        return;
    }

    const int ntiles = (int)((L + CAP - 1) / CAP);
    const bool resident = ntiles == 1;
    uint32_t key[KPT];
    auto load_tile = [&](int tile) {
#pragma unroll
        for (int j4 = 0; j4 < KPT / 4; ++j4) {
            const int64_t p = (int64_t)tile * CAP + wave * SEG + j4 * 256 + 4 * lane;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            // rows are padded to a multiple of 16 floats, so p < L keeps p + 3 in the row
            if (p < L) v = *reinterpret_cast<const f32x4*>(srow + p);
#pragma unroll
            for (int c = 0; c < 4; ++c) key[j4 * 4 + c] = (p + c < L) ? float_key(v[c]) : 0u;
        }
    };

    // ---- radix rounds: find T = key of rank n_eff from the top ------------------
    uint32_t prefix = 0;
    uint32_t krem = (uint32_t)n_eff;   // rank still to locate, counted from the top
    uint32_t tie_cnt = 0;
    uint32_t kmax = 0;
    if (resident) load_tile(0);
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int bits = pass == 0 ? 12 : 10;
        const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
        const int nb = 1 << bits;
        for (int i = tid; i < nb; i += kSelectThreads) hist[i] = 0u;
        __syncthreads();
#pragma unroll 1
        for (int tile = 0; tile < ntiles; ++tile) {
            if (!resident) load_tile(tile);
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                const uint32_t kk = key[j];
                if (pass == 0) kmax = kk > kmax ? kk : kmax;
                const bool match = pass == 0 ? kk != 0u : (kk >> (shift + bits)) == prefix;
                if (match) atomicAdd(&hist[(kk >> shift) & (uint32_t)(nb - 1)], 1u);
            }
        }
        __syncthreads();
        // suffix sums over bins: count of keys in bins above this thread's bins
        const int bpt = nb / kSelectThreads;   // 4 or 1 bins per thread
        uint32_t mine = 0;
        for (int i = 0; i < bpt; ++i) mine += hist[tid * bpt + i];
        uint32_t suf = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_down(suf, o, 64);
            if (lane + o < 64) suf += y;
        }
        if (lane == 0) wtot[wave] = suf;
        __syncthreads();
        uint32_t above = suf - mine;
        for (int w = wave + 1; w < kNW; ++w) above += wtot[w];
        for (int i = bpt - 1; i >= 0; --i) {
            const uint32_t c = hist[tid * bpt + i];
            if (above < krem && above + c >= krem) {
                bc[0] = (uint32_t)(tid * bpt + i);
                bc[1] = above;
                bc[2] = c;
            }
            above += c;
        }
        __syncthreads();
        const uint32_t digit = bc[0];
        krem -= bc[1];
        tie_cnt = bc[2];
        prefix = (prefix << bits) | digit;
        __syncthreads();
    }
    const uint32_t T = prefix;     // full key of the N_eff-th largest logit
    (void)tie_cnt;                 // keys equal to T; krem of them are kept

    // ---- row max (largest kept logit) -------------------------------------------
    kmax = wave_max(kmax);
    if (lane == 0) wtot[wave] = kmax;
    __syncthreads();
    if (tid == 0) {
        uint32_t m = 0;
        for (int w = 0; w < kNW; ++w) m = wtot[w] > m ? wtot[w] : m;
        row_max[row] = key_float(m);
        row_cnt[row] = n_eff;
    }
    __syncthreads();

    // ---- compaction in ascending position order -----------------------------------
    uint32_t base = 0;        // kept entries in earlier tiles
    uint32_t eq_tile = 0;     // keys == T in earlier tiles
#pragma unroll 1
    for (int tile = 0; tile < ntiles; ++tile) {
        if (!resident) load_tile(tile);
        uint32_t cg = 0, ce = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            cg += key[j] > T;
            ce += key[j] == T;
        }
        cg = wave_sum(cg);
        ce = wave_sum(ce);
        if (lane == 0) {
            wtot[wave] = cg;
            wtot[kNW + wave] = ce;
        }
        __syncthreads();
        uint32_t eqb = eq_tile, selb = 0, my_eqb = 0, my_selb = 0;
        for (int w = 0; w < kNW; ++w) {
            if (w == wave) {
                my_eqb = eqb;
                my_selb = selb;
            }
            const uint32_t ew = wtot[kNW + w];
            const uint32_t room = krem > eqb ? krem - eqb : 0u;
            selb += wtot[w] + (ew < room ? ew : room);
            eqb += ew;
        }
        uint32_t req = my_eqb;
        uint32_t rsel = base + my_selb;
#pragma unroll
        for (int j4 = 0; j4 < KPT / 4; ++j4) {
            uint32_t ecnt = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) ecnt += key[j4 * 4 + c] == T;
            uint32_t epre, etot;
            wave_scan_small(ecnt, epre, etot);
            uint32_t er = req + epre;
            bool keep[4];
            uint32_t scnt = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t kk = key[j4 * 4 + c];
                const bool eq = kk == T;
                keep[c] = kk > T || (eq && er < krem);
                er += eq;
                scnt += keep[c];
            }
            uint32_t spre, stot;
            wave_scan_small(scnt, spre, stot);
            uint32_t slot = rsel + spre;
            const int64_t p0 = (int64_t)tile * CAP + wave * SEG + j4 * 256 + 4 * lane;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                // slot < n_eff holds by construction; the test keeps stores in bounds
                if (keep[c] && slot < (uint32_t)n_eff) {
                    oi[slot] = (int32_t)(p0 + c);
                    ov[slot] = key_float(key[j4 * 4 + c]);
                    if (ou) ou[slot] = (int32_t)(p0 + c);
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

template <int KPT>
hipError_t go(const float* scores, int64_t s_stride, const int32_t* lens, int B, int h_q, int N,
              int64_t S_max, int32_t* sel_idx, float* sel_val, float* row_max, int32_t* row_cnt,
              int32_t* idx_out, hipStream_t st) {
    hipLaunchKernelGGL((select_topn<KPT>), dim3((unsigned)(B * h_q)), dim3(kSelectThreads), 0, st,
                       scores, s_stride, lens, h_q, N, S_max, sel_idx, sel_val, row_max, row_cnt,
                       idx_out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const float* scores, int64_t s_stride, const int32_t* lens, int B,
                         int h_q, int N, int64_t S_max, int32_t* sel_idx, float* sel_val,
                         float* row_max, int32_t* row_cnt, int32_t* idx_out, hipStream_t st) {
    const int64_t per = (int64_t)kSelectThreads;
    if (S_max <= 4 * per)
        return go<4>(scores, s_stride, lens, B, h_q, N, S_max, sel_idx, sel_val, row_max, row_cnt, idx_out, st);
    if (S_max <= 8 * per)
        return go<8>(scores, s_stride, lens, B, h_q, N, S_max, sel_idx, sel_val, row_max, row_cnt, idx_out, st);
    if (S_max <= 16 * per)
        return go<16>(scores, s_stride, lens, B, h_q, N, S_max, sel_idx, sel_val, row_max, row_cnt, idx_out, st);
    return go<32>(scores, s_stride, lens, B, h_q, N, S_max, sel_idx, sel_val, row_max, row_cnt, idx_out, st);
}

}  // namespace saga
