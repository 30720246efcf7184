// SparQ-style approximate scoring on the SAGA key heads ("SparQ Attention:
// Bandwidth-Efficient LLM Inference", Step 1 with its GQA modification),
// feeding the top-M candidate lists of the exact path's selector.
//
// The set-up of Step 1, per (b, key head) row: u[c] = sum over the key
// head's g query heads of |q[c]| (fp32, heads in order); the r dims of
// largest u (equal sums: lower dim first), ascending, -1 padded to
// RP = round_up(r, 16); per query head the inverse temperature
// 1 / tau = sqrt(|q|_1 / (d |q on dims|_1)), 0 when the head has no mass on
// the dims (its approximate scores are then all 0); qm = q / tau on the dims
// and 0 elsewhere (used by the selector to rescore kept rows); and the scan's
// matrix-core operand per 16-dim slice and lane. Each producer wave of the
// scan computes it for the rows it streams (sq_row_setup), so no dispatch
// precedes the scan.
//
// sparq_topm: the producer / consumer workgroup of kscan_topm with the same
// consumers (topm.h), but the producers stream only the r kept columns of the
// key head, from a second, S-contiguous copy of the key cache
// Kt [B][h_k][d][S_max]: a column is a contiguous run of positions, so the
// S r elements of Step 1 are read as whole 512-byte row segments (the four
// producer waves take adjacent 64-position pieces of the same 256 positions).
// Each wave takes 16-dim x 64-position sub-tiles: row-coalesced 16-byte
// loads into registers (four sub-tiles in flight, one per 64-position step of
// the wave's share of the chunk), then through a 16-row LDS tile whose
// transposing reads hand each lane 4 consecutive dims of one position -- the
// A operand of a 16x16x16 bf16 MFMA (positions x dims) against the query
// operand (dims x heads). fp32 caches use 16x16x4 f32 steps with plain LDS
// reads. The logits are scaled by 1 / tau per head and written to the chunk's
// key rows as order-preserving keys, which the consumer waves turn into
// candidate lists exactly as for the exact path. Positions of the local
// window are ranked by nobody: the consumers count them in the chunk's
// softmax statistics and then drop them (the selector keeps them anyway).
#include "topm.h"

#include <type_traits>

namespace saga {
using namespace dev;

namespace {

// Consumer waves of the scan's workgroup (after the kWaves producers). The
// stream of r columns is short, so an item's time is the consumers'
// extraction: a chain of dependent LDS and wave-reduction steps that leaves
// the SIMDs about half idle at three waves each. Where the producers fit in
// 128 registers (bf16, r <= 32) a fourth wave per SIMD runs twelve
// consumers, one per query head of a 12-head group and item; other shapes
// keep the eight of kscan_topm.
template <typename T, int KT>
constexpr int sq_consumers() { return sizeof(T) == 2 && KT <= 2 ? 12 : kConsumers; }
template <typename T, int KT>
constexpr int sq_threads() { return 64 * (kWaves + sq_consumers<T, KT>()); }

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- Step 1 set-up -----------------------------------------------------------------
// Query operand of the scan for slice kt and lane l: element e is the query of
// head l % 16 at dim dims[16 kt + 4 (l / 16) + e] (0 for heads >= g and pad dims).
template <typename T> struct SqOp;
template <> struct SqOp<uint16_t> { using Q = u32x2; };
template <> struct SqOp<float> { using Q = u32x4; };

// Step 1 set-up of one (b, key head) row, computed by one producer wave of the
// scan on its own (no workgroup barrier, so the consumers never wait for it).
// With c = lane + 64 i the lane's dims:
//   u[c] = sum over the g query heads, in head order, of |q[c]| (fp32);
//   dims = the r dims of largest u (equal sums: lower dim first), ascending,
//          -1 padded to RP, into the wave's table dtab (which holds u first);
//   1 / tau per head = sqrt(|q|_1 / (d |q on dims|_1)), 0 when the head has no
//          mass on the dims (its approximate scores are then all 0): per-lane
//          sums over the lane's dims in order, reduced over the wave, into
//          itab (0 for heads >= g);
//   qk   = the scan's query operand per 16-dim slice.
// `writer` (the workgroup that scans the row's first chunk) also writes
// qm = q / tau on the dims and 0 elsewhere (the selector rescores kept rows
// with it) and, when asked, the dims in dims_out [r].
// A call of its own (it runs once per row), so the item loop's registers are
// not shared with it; its pointers carry their address spaces, since a
// called function cannot infer them (it would use flat accesses).
typedef __attribute__((address_space(3))) int32_t lds_i32;
typedef __attribute__((address_space(3))) float lds_f32;
template <typename T> using glb = __attribute__((address_space(1))) T;
template <typename T, int DH, int KT>
__device__ __noinline__ void sq_row_setup(const glb<T>* __restrict__ qg, int g, int r, int RP,
                                          int lane, lds_i32* dtab, lds_f32* itab,
                                          typename SqOp<T>::Q (&qk)[KT], bool writer,
                                          glb<float>* __restrict__ qm_out,
                                          glb<int32_t>* __restrict__ dims_out) {
    constexpr int CPL = DH / 64;   // dims per lane
    constexpr int GM = 16;         // g <= 16 query heads per key head
    auto qval = [&](int j, int c) -> float {
        if constexpr (sizeof(T) == 2)
            return __uint_as_float((uint32_t)qg[(int64_t)j * DH + c] << 16);
        else
            return qg[(int64_t)j * DH + c];
    };
    // the g query rows at the lane's dims, all requested before the first use
    // (bf16: a lane's dims packed in one register, its raw bits). The loads
    // are unconditional (rows past g re-read row g - 1 and are zeroed after):
    // a load whose register another path zeroes is waited for on the spot.
    uint32_t qp[GM];
    float qf[GM][CPL];
#pragma unroll
    for (int j = 0; j < GM; ++j) {
        const int jj = j < g ? j : g - 1;
        if constexpr (sizeof(T) == 2) {
            const uint32_t lo = (uint32_t)qg[(int64_t)jj * DH + lane];
            const uint32_t hi = CPL == 2 ? (uint32_t)qg[(int64_t)jj * DH + lane + 64] : 0u;
            qp[j] = lo | (hi << 16);
        } else {
#pragma unroll
            for (int i = 0; i < CPL; ++i) qf[j][i] = qval(jj, lane + 64 * i);
        }
    }
#pragma unroll
    for (int j = 0; j < GM; ++j) {
        if (j < g) continue;   // uniform
        qp[j] = 0u;
#pragma unroll
        for (int i = 0; i < CPL; ++i) qf[j][i] = 0.f;
    }
    auto qv = [&](int j, int i) -> float {
        if constexpr (sizeof(T) == 2)
            return __uint_as_float(i == 0 ? qp[j] << 16 : qp[j] & 0xFFFF0000u);
        else
            return qf[j][i];
    };
    float u[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        u[i] = 0.f;
#pragma unroll
        for (int j = 0; j < GM; ++j)
            if (j < g) u[i] += fabsf(qv(j, i));   // uniform; heads in order
    }
    // The kept dims: with K the r-th largest of the d sums (order-preserving
    // keys, found bit by bit from the top: the largest K with at least r sums
    // at or above it), every dim above K and the first r - count(above K)
    // dims equal to K in dim order -- exactly the dims whose rank (larger
    // sums, or equal sums at lower dims) is below r.
    uint32_t ku[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) ku[i] = float_key(u[i]);
    auto count_ge = [&](uint32_t x) -> uint32_t {
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < CPL; ++i) c += (uint32_t)__builtin_popcountll(ballot(ku[i] >= x));
        return c;
    };
    uint32_t kth = 0u;
#pragma unroll 4
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = kth | (1u << bit);
        if (count_ge(cand) >= (uint32_t)r) kth = cand;   // uniform
    }
    uint32_t n_gt = 0;
#pragma unroll
    for (int i = 0; i < CPL; ++i) n_gt += (uint32_t)__builtin_popcountll(ballot(ku[i] > kth));
    const uint32_t n_eq = (uint32_t)r - n_gt;   // ties kept, lowest dims first
    bool keep[CPL];
    uint64_t km[CPL];
    uint32_t eq_before = 0;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const uint64_t me = ballot(ku[i] == kth);
        keep[i] = ku[i] > kth || (ku[i] == kth && eq_before + lanes_below(me) < n_eq);
        eq_before += (uint32_t)__builtin_popcountll(me);
        km[i] = ballot(keep[i]);
    }
    // ascending list of the kept dims: a kept dim's place is the number of
    // kept dims below it
    for (int e = r + lane; e < RP; e += 64) dtab[e] = -1;
    uint32_t below = 0;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        if (keep[i]) {
            const uint32_t at = below + lanes_below(km[i]);
            dtab[at] = c;
            if (writer && dims_out) dims_out[at] = c;
        }
        below += (uint32_t)__builtin_popcountll(km[i]);
    }
    // per head: 1 / tau. The lane's partial sums of every head first, then
    // their wave sums for all heads together (wave_fsum's tree and order, so
    // the bits are the same), then each head's 1 / tau in lane j; heads past
    // g have no mass and get 0
    float xd[GM], xn[GM];
#pragma unroll
    for (int j = 0; j < GM; ++j) {
        float den = 0.f, num = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const float a = fabsf(qv(j, i));
            den += a;
            num += keep[i] ? a : 0.f;
        }
        xd[j] = den;
        xn[j] = num;
    }
    auto dpp_step = [&](float (&x)[GM], auto ctrl) {
#pragma unroll
        for (int j = 0; j < GM; ++j)
            x[j] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[j]),
                                                               decltype(ctrl)::value, 0xf, 0xf,
                                                               false));
    };
    dpp_step(xd, std::integral_constant<int, 0x111>{});
    dpp_step(xn, std::integral_constant<int, 0x111>{});
    dpp_step(xd, std::integral_constant<int, 0x112>{});
    dpp_step(xn, std::integral_constant<int, 0x112>{});
    dpp_step(xd, std::integral_constant<int, 0x114>{});
    dpp_step(xn, std::integral_constant<int, 0x114>{});
    dpp_step(xd, std::integral_constant<int, 0x118>{});
    dpp_step(xn, std::integral_constant<int, 0x118>{});
    auto total = [](float x) {
        return (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15)) +
                __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31))) +
               (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47)) +
                __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63)));
    };
    float myden = 0.f, mynum = 0.f;
#pragma unroll
    for (int j = 0; j < GM; ++j) {
        const float dj = total(xd[j]), nj = total(xn[j]);
        myden = lane == j ? dj : myden;
        mynum = lane == j ? nj : mynum;
    }
    const float myinv = mynum > 0.f ? sqrtf(myden / ((float)DH * mynum)) : 0.f;
    if (lane < GM) itab[lane] = myinv;
    if (writer)   // qm from the workgroup that writes it
#pragma unroll
        for (int j = 0; j < GM; ++j) {
            const float inv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myinv), j));
            if (j < g)   // uniform
#pragma unroll
                for (int i = 0; i < CPL; ++i)
                    qm_out[(int64_t)j * DH + lane + 64 * i] = keep[i] ? qv(j, i) * inv : 0.f;
        }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // the dims are in the table before they are read back
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // the scan's query operand, one slice of 16 dims at a time
    const int hd = lane & 15, G = lane >> 4;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = dtab[16 * kt + 4 * G + e];
            const float xl = qval(hd < g ? hd : 0, c >= 0 ? c : 0);   // in bounds, unconditional
            const float x = (hd < g && c >= 0) ? xl : 0.f;
            // the cache's own values: back to its type exactly
            w[e] = sizeof(T) == 2 ? (__float_as_uint(x) >> 16) : __float_as_uint(x);
        }
        if constexpr (sizeof(T) == 2) {
            qk[kt][0] = w[0] | (w[1] << 16);
            qk[kt][1] = w[2] | (w[3] << 16);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) qk[kt][e] = w[e];
        }
    }
}

// ---- the scan --------------------------------------------------------------------
// A sub-tile: 16 dims x 64 positions, rows of RB bytes in the wave's LDS tile.
// 16-byte unit u of row r is stored at unit u ^ swz(r): for bf16 the four rows
// of a transposing read (r = 4G + j) and the four 16-lane groups (G) land in
// distinct units; for fp32 the four groups of a 32-bit read do.
template <typename T>
struct SqTile {
    static constexpr int RB = 64 * (int)sizeof(T);   // bytes per row: 128 / 256
    static constexpr int NL = RB / 64;                // 16-byte loads per lane: 2 / 4
    static constexpr int BYTES = 16 * RB;
    __device__ static inline int swz(int r) {
        return sizeof(T) == 2 ? 2 * ((r ^ (r >> 2)) & 3) : 4 * ((r >> 2) & 3);
    }
};

// acc += (positions 16 nb .. + 15 of the tile) x (its 16 dims) . (query operand)
template <typename T> struct SqMma;
template <> struct SqMma<uint16_t> {
    using TL = SqTile<uint16_t>;
    __device__ static inline f32x4 block(const char* tile, int nb, int lane, u32x2 qo, f32x4 acc) {
        const int G = lane >> 4, i = lane & 15, a = i & 3, j = i >> 2;
        const int row = 4 * G + j;
        const int unit = 2 * nb + (a >> 1);
        // lane a + 4 j of the group addresses row 4 G + j, positions 16 nb + 4 a .. + 3;
        // lane i receives position 16 nb + i of rows 4 G .. 4 G + 3
        const v4s t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4s*)(tile + row * TL::RB + ((unit ^ TL::swz(row)) << 4) + 8 * (a & 1)));
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t, __builtin_bit_cast(v4s, qo), acc, 0, 0,
                                                         0);
    }
};
template <> struct SqMma<float> {
    using TL = SqTile<float>;
    __device__ static inline f32x4 block(const char* tile, int nb, int lane, u32x4 qo, f32x4 acc) {
        const int G = lane >> 4, i = lane & 15;
        const int unit = 4 * nb + (i >> 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 4 * G + j;   // dim 16 kt + 4 G + j, position 16 nb + i
            const float a = *reinterpret_cast<const float*>(
                tile + row * TL::RB + ((unit ^ TL::swz(row)) << 4) + 4 * (i & 3));
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, __uint_as_float(qo[j]), acc, 0, 0, 0);
        }
        return acc;
    }
};

// LDS layout of sparq_topm (32-bit words): as kscan_topm's, with each
// producer wave's tile and dims table in place of the transpose buffers:
//   keys [2][g][kKeyRow], warm [g] + cursor/used/pad, meta staging,
//   per producer wave: tile [SqTile::BYTES / 4], dims [DH], 1 / tau [16];
//   then list staging.
template <typename T, int DH>
__host__ __device__ constexpr size_t sq_lds_words(int g) {
    return (size_t)2 * g * kKeyRow + ((g + 4 + 3) & ~3) + 5 * kMetaStage +
           (size_t)kWaves * (SqTile<T>::BYTES / 4 + DH + 16);
}

// KT = RP / 16 slices of 16 dims per item, a template parameter so that the
// item's sub-tiles form straight-line code: the compiler then counts the
// loads in flight exactly instead of waiting for all of them at a loop head.
template <typename T, int DH, int KT>
__global__ __launch_bounds__((sq_threads<T, KT>()), 1) void sparq_topm(
        const T* __restrict__ kt, const int32_t* __restrict__ lens, int h_q, int h_k,
        int64_t S_max, int nchunk, int nwork, int RP, int local,
        const T* __restrict__ q, int r, float* __restrict__ qm, int32_t* __restrict__ dims_out,
        TopmOut tm, uint32_t lds_bytes) {
    using TL = SqTile<T>;
    using Q = typename SqOp<T>::Q;
    constexpr int NC = sq_consumers<T, KT>();
    constexpr int NTH = sq_threads<T, KT>();
    constexpr int NL = TL::NL;
    extern __shared__ uint32_t lds[];
    const int g = h_q / h_k;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // wave-uniform
    const bool producer = wave < kWaves;
    uint32_t* keys = lds;
    uint32_t* warm = lds + 2 * g * kKeyRow;
    uint32_t* cursor = warm + g;
    uint32_t* meta_words = lds + 2 * g * kKeyRow + ((g + 4 + 3) & ~3);
    uint32_t* wave_words = meta_words + 5 * kMetaStage;
    const uint32_t fixed_words = (uint32_t)sq_lds_words<T, DH>(g);
    char* tile =
        reinterpret_cast<char*>(wave_words + (producer ? wave : 0) * (TL::BYTES / 4 + DH + 16));
    int32_t* dtab = reinterpret_cast<int32_t*>(tile + TL::BYTES);
    float* itab = reinterpret_cast<float*>(dtab + DH);   // 1 / tau of the row's heads

    const int per = (nwork + gridDim.x - 1) / gridDim.x;
    // ranges dealt XCD-blocked, as in kscan_topm
    const int wr = gridDim.x % 8 == 0 ? xcd_logical((int)blockIdx.x, (int)gridDim.x)
                                      : (int)blockIdx.x;
    const int wbeg = wr * per;
    const int wend = wbeg + per < nwork ? wbeg + per : nwork;
    if (wbeg >= wend) return;   // uniform over the workgroup
    if (producer && wave == 0) {
        // The row whose chunk 0 is item bkh nchunk of this range has its
        // set-up outputs (qm, the dims) written by this workgroup. A row with
        // no positions (L_b = 0) has no item to scan, so its outputs are
        // written here, the tables being rewritten before any item uses them.
        for (int bkh = (wbeg + nchunk - 1) / nchunk; bkh * nchunk < wend; ++bkh) {
            const int b = bkh / h_k;
            if (clamp_len(lens[b], S_max) > 0) continue;   // uniform
            const int64_t qrow = (int64_t)(b * h_q + (bkh - b * h_k) * g) * DH;
            Q qs[KT];
            sq_row_setup<T, DH, KT>((const glb<T>*)(q + qrow), g, r, RP, lane, (lds_i32*)dtab,
                                    (lds_f32*)itab, qs, true, (glb<float>*)(qm + qrow),
                                    (glb<int32_t>*)(dims_out ? dims_out + (int64_t)bkh * r
                                                             : nullptr));
        }
    }
    ListSink sink;
    sink.base = (uint64_t)wbeg * g * kScanChunk;
    sink.pool = tm.cand + sink.base;
    sink.stg = reinterpret_cast<uint2*>(lds + fixed_words);
    sink.cap = ((lds_bytes / 4 - fixed_words) / 2) & ~1u;
    sink.cursor = cursor;
    sink.used = cursor + 1;
    sink.meta_stg = reinterpret_cast<uint4*>(meta_words);
    sink.meta_slot = meta_words + 4 * kMetaStage;
    auto len_of = [&](int b) { return lens[b]; };

    Item<T> cur;
    int w = next_item<T, DH>(wbeg, 1, wend, nchunk, h_k, S_max, len_of, kt, cur);
    if (w >= wend) return;   // uniform over the workgroup
    if (!producer) {
        for (int n = wave - kWaves; n < g; n += NC)
            if (lane == 0) warm[n] = 0u;
        if (threadIdx.x == 64 * kWaves) cursor[0] = cursor[1] = 0u;
    }

    // producer state: four sub-tiles in flight (one per 64-position step) and
    // their accumulators, declared per row (so they are not live across the
    // row's set-up), and the query operand of the row.
    // Loads are unconditional (pieces past L or of pad dims read an in-bounds
    // address) and masked when written to the tile: a load whose destination
    // could also be written by another path would make the compiler wait for
    // it on the spot.
    Q qk[KT];         // the row's query operand, one per slice
    const int hd = lane & 15;
    auto ktb = [&](const Item<T>& it) { return kt + (int64_t)it.bkh * DH * S_max; };
    auto load = [&](u32x4 (&dst)[NL], uint32_t& valid, const Item<T>& it, int slice, int st) {
        const int row = lane >> 2;
        const int dim = dtab[16 * slice + row];
        const int p0 = it.c0 + 256 * st + 64 * wave;
        const T* base = ktb(it) + (int64_t)(dim < 0 ? 0 : dim) * S_max;
        uint32_t m = 0;
#pragma unroll
        for (int h = 0; h < NL; ++h) {
            const int pos = p0 + (64 * h + 16 * (lane & 3)) / (int)sizeof(T);
            // a 16-byte piece starting before L stays inside the row (S_max is a
            // multiple of the piece); pad dims and pieces past L count as zero
            const bool ok = dim >= 0 && pos < it.L;
            m |= ok ? 1u << h : 0u;
            dst[h] = *reinterpret_cast<const u32x4*>(base + (ok ? pos : 0));
        }
        valid = m;
    };
    lds_barrier();

    // The two roles run separate loops with one barrier per item each (so the
    // compiler can count the producers' loads in flight without the
    // consumers' stores in the way): after producer item t and consumer
    // iteration t, the keys of item t are complete and buffer t & 1 holds them;
    // consumer iteration t extracts item t - 1.
    auto extract_item = [&](const Item<T>& it, int tt, int first, int step) {
        const float share = (float)tm.N * (float)kScanChunk / (float)it.L;
        const uint32_t M = share >= (float)(kScanChunk / 2)
                               ? (uint32_t)kScanChunk
                               : (uint32_t)__builtin_ceilf(1.5f * share) + 16u;
        uint32_t* kbuf = keys + (tt & 1) * g * kKeyRow;
        const int lw = local < it.L ? local : it.L;
#pragma unroll 1
        for (int n = first; n < g; n += step)
            extract(it, n, M, kbuf + n * kKeyRow, warm, sink, tt, lane, g, h_q, nchunk, tm,
                    it.L - lw);
    };
    Item<T> last = cur;
    int t = 0;
    if (producer) {
        // outer loop: one key row (b, kh) at a time; the workgroup's items are
        // consecutive chunks, so a row change is rare and its drain cheap
#pragma unroll 1
        while (w < wend) {
            const int row = cur.bkh;
            // the row's Step 1 set-up (dims and 1 / tau into this wave's tables,
            // the query operand), then the first item's first slice; the row's
            // first chunk is scanned by exactly one workgroup, whose wave 0
            // writes qm and the dims
            const int64_t qrow = (int64_t)(cur.b * h_q + cur.kh * g) * DH;
            sq_row_setup<T, DH, KT>((const glb<T>*)(q + qrow), g, r, RP, lane, (lds_i32*)dtab,
                                    (lds_f32*)itab, qk, cur.chunk == 0 && wave == 0,
                                    (glb<float>*)(qm + qrow),
                                    (glb<int32_t>*)(dims_out ? dims_out + (int64_t)row * r
                                                             : nullptr));
            u32x4 sr[4][NL];
            uint32_t vm[4];   // valid pieces of each stage
            f32x4 acc[4][4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) acc[s][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) load(sr[s], vm[s], cur, 0, s);
            // inner loop: the row's items; each one's last slice loads the next's first
#pragma unroll 1
            while (true) {
                Item<T> nx = cur;
                const int wn = next_item<T, DH>(w + 1, 1, wend, nchunk, h_k, S_max, len_of, kt, nx);
                const bool chain = wn < wend && nx.bkh == row;
#pragma unroll
                for (int sl = 0; sl < KT; ++sl) {
                    const bool lastsl = sl + 1 == KT;
                    // refills: the next slice, else the chained item's first slice,
                    // else (nothing follows in this row) a re-read that is never used
                    const Item<T>& ri = (lastsl && chain) ? nx : cur;
                    const int rsl = lastsl ? 0 : sl + 1;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
#pragma unroll
                        for (int h = 0; h < NL; ++h) {
                            const int r16 = lane >> 2, u = 4 * h + (lane & 3);
                            *reinterpret_cast<u32x4*>(tile + r16 * TL::RB +
                                                      ((u ^ TL::swz(r16)) << 4)) =
                                ((vm[s] >> h) & 1u) ? sr[s][h] : u32x4{0u, 0u, 0u, 0u};
                        }
                        load(sr[s], vm[s], ri, rsl, s);
#pragma unroll
                        for (int nb = 0; nb < 4; ++nb)
                            acc[s][nb] = SqMma<T>::block(tile, nb, lane, qk[sl], acc[s][nb]);
                    }
                }
                // keys of the chunk: position 256 s + 64 wave + 16 nb + 4 (lane / 16) + e,
                // head lane % 16
                uint32_t* kbuf = keys + (t & 1) * g * kKeyRow;
                if (hd < g) {
                    const float inv = itab[hd];
#pragma unroll
                    for (int s = 0; s < 4; ++s)
#pragma unroll
                        for (int nb = 0; nb < 4; ++nb) {
                            const int o = 256 * s + 64 * wave + 16 * nb + 4 * (lane >> 4);
                            int rem = cur.n - o;
                            asm volatile("" : "+v"(rem));
                            u32x4 kv;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                kv[e] = e < rem ? float_key(acc[s][nb][e] * inv) : 0u;
                            *reinterpret_cast<u32x4*>(&kbuf[hd * kKeyRow + o]) = kv;
                        }
                }
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) acc[s][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
                lds_barrier();   // keys of item t are complete
                last = cur;
                cur = nx;
                w = wn;
                ++t;
                if (!chain) break;   // the workgroup's items end, or a new row follows
            }
        }
    } else {
        Item<T> prev = cur;
#pragma unroll 1
        while (w < wend) {
            Item<T> nx = cur;
            const int wn = next_item<T, DH>(w + 1, 1, wend, nchunk, h_k, S_max, len_of, kt, nx);
            if (t > 0) extract_item(prev, t - 1, wave - kWaves, NC);
            lds_barrier();   // keys of item t are complete; buffer (t - 1) & 1 is free again
            prev = cur;
            last = cur;
            cur = nx;
            w = wn;
            ++t;
        }
    }
    // the last item, shared by all waves
    extract_item(last, t - 1, wave, kWaves + NC);
    lds_barrier();
    const uint32_t used = (sink.used[0] + 1u) & ~1u;
    const u32x4* s4 = reinterpret_cast<const u32x4*>(sink.stg);
    u32x4* d4 = reinterpret_cast<u32x4*>(sink.pool);
    for (uint32_t j = threadIdx.x; j < used / 2; j += NTH) d4[j] = s4[j];
    const int nmeta = t * g < kMetaStage ? t * g : kMetaStage;   // items 0 .. t-1
    for (int e = (int)threadIdx.x; e < nmeta; e += NTH)
        tm.meta[sink.meta_slot[e]] = sink.meta_stg[e];
}

template <typename T, int DH, int KT>
hipError_t go_sparq_scan(const void* q, const void* kt, const int32_t* lens, const TopmOut& tm,
                         const SparqWs& sw, int h_q, int h_k, int64_t S_max, int nchunk, int nwork,
                         int r, int RP, int local, int32_t* dims_out, hipStream_t st) {
    auto kern = &sparq_topm<T, DH, KT>;
    const size_t lds = kTopmLdsBytes;
    static_assert(sq_lds_words<T, DH>(16) * 4 + 8 * 1024 <= kTopmLdsBytes, "staging area too small");
    {   // allow > 64 KiB of dynamic LDS
        const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), lds);
        if (e != hipSuccess) return e;
    }
    constexpr int nth = sq_threads<T, KT>();
    const int grid = resident_grid(kern, nth, lds, nwork);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(nth), lds, st, (const T*)kt, lens,
                       h_q, h_k, S_max, nchunk, nwork, RP, local, (const T*)q, r, sw.qm,
                       dims_out, tm, (uint32_t)lds);
    return hipGetLastError();
}

template <typename T, int DH>
hipError_t go_sparq(const void* q, const void* kt, const int32_t* lens, const TopmOut& tm,
                    const SparqWs& sw, int B, int h_q, int h_k, int r, int local, int64_t S_max,
                    int32_t* dims_out, hipStream_t st) {
    const int nchunk = (int)((S_max + kScanChunk - 1) / kScanChunk);
    const int nwork = B * h_k * nchunk;
    const int RP = (int)round_up(r, 16);
#define SAGA_SQ(KT)                                                                                \
    case KT:                                                                                       \
        return go_sparq_scan<T, DH, (KT <= DH / 16 ? KT : DH / 16)>(                               \
            q, kt, lens, tm, sw, h_q, h_k, S_max, nchunk, nwork, r, RP, local, dims_out, st);
    switch (RP / 16) {
        SAGA_SQ(1) SAGA_SQ(2) SAGA_SQ(3) SAGA_SQ(4) SAGA_SQ(5) SAGA_SQ(6) SAGA_SQ(7) SAGA_SQ(8)
        default: return hipErrorInvalidValue;
    }
#undef SAGA_SQ
}

}  // namespace

hipError_t launch_sparq_scan(const void* q, const void* kt, const int32_t* lens, const TopmOut& tm,
                             const SparqWs& sw, int B, int h_q, int h_k, int d, int r, int local,
                             int64_t S_max, bool bf16, int32_t* dims_out, hipStream_t st) {
    if (bf16)
        return d == 64 ? go_sparq<uint16_t, 64>(q, kt, lens, tm, sw, B, h_q, h_k, r, local, S_max, dims_out, st)
                       : go_sparq<uint16_t, 128>(q, kt, lens, tm, sw, B, h_q, h_k, r, local, S_max, dims_out, st);
    return d == 64 ? go_sparq<float, 64>(q, kt, lens, tm, sw, B, h_q, h_k, r, local, S_max, dims_out, st)
                   : go_sparq<float, 128>(q, kt, lens, tm, sw, B, h_q, h_k, r, local, S_max, dims_out, st);
}

}  // namespace saga
