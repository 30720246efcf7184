// GQA -> SAGA key-head merge on MI355X (gfx950).
//
// "More Value per Key: Asymmetric Sparse Attention for Faster LLM Decoding",
// §4 (Eqs. 13-18, Lemma 4.1, Theorem 4.2), App. A (Eqs. 19-27), App. B
// (induced permutations, Eqs. 28-34; B.1 merge strategies, Eq. 35).
//
// The merge needs, per teacher key head r, S_r = sum_{j in Q_r} (X W_Q^j)^T
// (X W_Q^j) and the realized-key Gram H = (X W_K)^T (X W_K). Both are
// contractions of C = X^T X with the projections, so the path is
//   1. syrk_partial / syrk_reduce: C = X^T X (bf16 MFMA, fp32 accumulation;
//      upper-triangle 256 x 256 tiles, token range split over workgroups,
//      partials summed in a fixed order);
//   2. nt_bf16x3: F = W C for all query and key heads (bf16 MFMA on C split
//      into three bf16 parts, fp32 accuracy); nt_gemm: S and H from F (fp32
//      MFMA);
//   3. merge_pairs: per pair (a, b), in fp64, Y = P^+ S_a and Z = P^+ S_b for
//      P = S_a + S_b (the transposes of the coefficients of Eq. 15: M(a, b) =
//      W_a Y^T + W_b Z^T). A pair whose P is clearly regular (every
//      eigenvalue well above the pseudo-inverse cutoff, from the Frobenius
//      norms of P and its inverse, or else a power-iteration estimate) takes
//      P^+ = P^{-1} by Gauss-Jordan elimination; any other pair is
//      diagonalised by cyclic Jacobi rotations held in LDS, whose recorded
//      rotations are replayed to apply P^+. The pair weight of Eq. 16
//      follows from the identity
//        L_{a,b}(M(a, b)) = <Z Delta, S_a Z> + <Y Delta, S_b Y>,
//      Delta = (X W_a - X W_b)^T (X W_a - X W_b) (App. A's trace form with
//      Y^T + Z^T = P P^+ substituted);
//   4. matching: minimum-weight perfect matching (Theorem 4.2) by dynamic
//      programming over head subsets, one launch per subset size;
//   5. merge_apply: the merged projections of the matched pairs.
// saga_merge_permute applies App. B's head permutations to W_Q, W_V, W_O.
#include "saga.h"
#include "saga_internal.h"

#include <stdint.h>

#include <type_traits>

namespace saga {
namespace {
using namespace dev;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- sizes -----------------------------------------------------------------
constexpr int kSyrkThreads = 512;    // 8 waves: 2 (rows) x 4 (columns) of 128 x 64
constexpr int kBlk = 256;            // C tile edge (features)
constexpr int kStageTok = 32;        // tokens per LDS stage
constexpr int kRowBytes = kBlk * 2;  // one token's 256 features in bf16
constexpr int kStageBytes = kStageTok * kRowBytes;         // one operand of one stage
constexpr int kTargetCus = 256;      // MI355X compute units: splits fill one wave of them
constexpr int kNtThreads = 256;
constexpr int kPairThreads = 512;
constexpr int kMaxSweeps = 24;       // Jacobi sweeps recorded per pair
constexpr int kMaxHeads = 24;        // teacher key heads the subset DP takes (2^24 states)

__host__ __device__ inline int n_blocks(int D) { return (D + kBlk - 1) / kBlk; }
__host__ __device__ inline int n_tiles(int D) { return n_blocks(D) * (n_blocks(D) + 1) / 2; }
inline int n_splits(int64_t L, int D) {
    const int nt = n_tiles(D);
    int64_t s = kTargetCus / nt;
    if (s < 1) s = 1;
    const int64_t stages = (L + kStageTok - 1) / kStageTok;
    if (s > stages) s = stages > 0 ? stages : 1;
    return (int)s;
}
inline int64_t split_len(int64_t L, int ns) {
    return round_up((L + ns - 1) / ns, kStageTok);
}

// logical workgroup id from the hardware one (total a multiple of 8): the
// hardware deals ids to the 8 XCDs round-robin, so XCD x gets the contiguous
// logical range [x total / 8, (x + 1) total / 8) and the workgroups that share
// a token range share that XCD's L2.
__device__ inline int xcd_logical(int hw, int total) {
    return (hw & 7) * (total >> 3) + (hw >> 3);
}

// ---- 1. C = X^T X ------------------------------------------------------------
// On gfx950 the 32x32x16 bf16 MFMA does twice the work of the 16x16x32 one in
// the same issue time (measured: 2.4 against 1.3 PFLOP/s on independent
// chains), so the Gram tiles are built from 32 x 32 blocks.
//
// XOR swizzle of the 16-byte units of a staged token row: the transposing
// reads of the two 16-lane groups served together cover the same 4
// consecutive rows x 64 bytes (two adjacent 16-feature blocks); rotating the
// units by 4 per row puts the 16 row-unit pairs on distinct banks.
__device__ inline int unit_swz(int row) { return 4 * (row & 3); }

// The operand of one 32x32x16 MFMA: lane l holds features 32 nb + (l % 32) of
// the 8 consecutive tokens (rows) kbase + 8 (l / 32) .. + 7 (A and B use the
// same token order, so the product is X^T X whatever the order within k).
// Each 16-lane group reads 4 rows x 16 features per transposing read: group
// G takes feature block 2 nb + (G & 1) and token half G >> 1.
__device__ inline v8bf syrk_frag(const char* buf, int kbase, int nb32, int lane) {
    const int G = lane >> 4, i = lane & 15, a = i & 3, j = i >> 2;
    const int unit = 2 * (2 * nb32 + (G & 1)) + (a >> 1);
    const int r0 = kbase + 8 * (G >> 1) + j, r1 = r0 + 4;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4s*)(buf + r0 * kRowBytes + ((unit ^ unit_swz(r0)) << 4) + 8 * (a & 1)));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4s*)(buf + r1 * kRowBytes + ((unit ^ unit_swz(r1)) << 4) + 8 * (a & 1)));
    const v8s t = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(v8bf, t);
}

__device__ inline void tile_of(int t, int nb, int& bi, int& bj) {
    bi = 0;
    while (t >= nb - bi) {
        t -= nb - bi;
        ++bi;
    }
    bj = bi + t;
}

// Stage buffers of the Gram tiles: 4 stages x 2 operands of [32 tokens][256
// features] bf16, each its own LDS object so that the compiler can tell the
// direct-to-LDS loads of one stage from the fragment reads of another.
__shared__ __attribute__((aligned(16))) char sy0a[kStageBytes], sy0b[kStageBytes],
    sy1a[kStageBytes], sy1b[kStageBytes], sy2a[kStageBytes], sy2b[kStageBytes],
    sy3a[kStageBytes], sy3b[kStageBytes];
template <int P>
__device__ inline char* sy_buf(int op) {
    if constexpr (P == 0) return op ? sy0b : sy0a;
    if constexpr (P == 1) return op ? sy1b : sy1a;
    if constexpr (P == 2) return op ? sy2b : sy2a;
    return op ? sy3b : sy3a;
}

// Wait until at most n (0, 2, 4 or 8) of this wave's vector-memory operations
// are outstanding, finish its LDS operations, then meet the workgroup. The
// wait counts follow the load pipeline below; a plain __syncthreads would
// wait for every load in flight.
__device__ inline void sy_sync(int n) {
    if (n >= 8)
        asm volatile("s_waitcnt vmcnt(8)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if (n >= 4)
        asm volatile("s_waitcnt vmcnt(4)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if (n >= 2)
        asm volatile("s_waitcnt vmcnt(2)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One workgroup: tile (bi <= bj) of C over the tokens of one split. The 8
// waves hold 128 x 64 of the 256 x 256 tile each, as 4 x 2 blocks of 32 x 32.
// Token stages of 32 rows stream into four LDS stage buffers with
// direct-to-LDS loads issued three stages ahead, so about 96 KB per CU are in
// flight from the MALL or HBM while the MFMAs work on the current stage. A
// stage with tokens past the split or features past D (only the last stage
// of a split, or every stage of a tile at a ragged edge) is loaded through
// registers instead, with the missing values set to zero, one stage ahead.
// A diagonal tile stages its rows once per operand as well, so that every
// fragment read names a single stage buffer (a read through a pointer that
// may name either would make the compiler wait for every load in flight).
// Partials are written in MFMA fragment order:
// [split][tile][wave][4 x 2 blocks][4 quarters][64 lanes] x f32x4.
__global__ __launch_bounds__(kSyrkThreads, 1) void syrk_partial(
        const uint16_t* __restrict__ x, int64_t L, int D, int ntile, int nsplit,
        int64_t slen, int grid_total, f32x4* __restrict__ part) {
    const int total = ntile * nsplit;
    const int logical = xcd_logical(blockIdx.x, grid_total);
    if (logical >= total) return;
    const int split = logical / ntile, tile = logical - split * ntile;
    const int nb = n_blocks(D);
    int bi, bj;
    tile_of(tile, nb, bi, bj);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int64_t t_beg = (int64_t)split * slen;
    int64_t t_end = t_beg + slen;
    if (t_end > L) t_end = L;
    const int64_t ntok = t_end > t_beg ? t_end - t_beg : 0;
    const int nstage = (int)((ntok + kStageTok - 1) / kStageTok);
    // stages [0, nfull) are whole and take the direct path
    const bool cols_whole = (bi + 1) * kBlk <= D && (bj + 1) * kBlk <= D;
    const int nfull = cols_whole ? (int)(ntok / kStageTok) : 0;
    constexpr int per_stage = 4;      // direct loads per wave per stage
    const uint16_t* src[2] = {x + (int64_t)bi * kBlk, x + (int64_t)bj * kBlk};

    // direct loads: wave w moves row pairs 2 w and 2 w + 1 of each operand;
    // lane l fills 16-byte slot l % 32 of row 2 pr + l / 32, which holds the
    // row's unit (slot ^ unit_swz(row))
    auto issue = [&](int s, auto P) {
        constexpr int p = decltype(P)::value;
#pragma unroll
        for (int op = 0; op < 2; ++op) {
            char* base = sy_buf<p>(op);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int pr = 2 * wave + h, row = 2 * pr + (lane >> 5);
                const int un = (lane & 31) ^ unit_swz(row);
                const uint16_t* g = src[op] + (t_beg + (int64_t)s * kStageTok + row) * D + un * 8;
                __builtin_amdgcn_global_load_lds(
                    (__attribute__((address_space(1))) void*)g,
                    (__attribute__((address_space(3))) void*)(base + pr * 1024), 16, 0, 0);
            }
        }
    };
    // register path: unit u = tid + 512 h of a stage, row u / 32, unit u % 32
    auto copy_stage = [&](int s, auto P) {
        constexpr int p = decltype(P)::value;
        constexpr int kUnits = kStageTok * 32 / kSyrkThreads;
        u32x4 reg[2][kUnits];
#pragma unroll
        for (int op = 0; op < 2; ++op) {
#pragma unroll
            for (int h = 0; h < kUnits; ++h) {
                const int u = tid + kSyrkThreads * h, row = u >> 5, un = u & 31;
                const int64_t tok = t_beg + (int64_t)s * kStageTok + row;
                const int col = (op ? bj : bi) * kBlk + un * 8;
                const bool ok = tok < t_end && col < D;
                const uint16_t* g = ok ? src[op] + tok * D + un * 8 : x;
                reg[op][h] = *reinterpret_cast<const u32x4*>(g);
                if (!ok) reg[op][h] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int op = 0; op < 2; ++op) {
            char* base = sy_buf<p>(op);
#pragma unroll
            for (int h = 0; h < kUnits; ++h) {
                const int u = tid + kSyrkThreads * h, row = u >> 5, un = u & 31;
                *reinterpret_cast<u32x4*>(base + row * kRowBytes + ((un ^ unit_swz(row)) << 4)) =
                    reg[op][h];
            }
        }
    };
    // direct loads of this wave issued after stage t's: those of stages t + 1
    // and t + 2 that exist
    auto after = [&](int t) {
        int n = nfull - (t + 1);
        n = n < 0 ? 0 : n > 2 ? 2 : n;
        return n * per_stage;
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    if (0 < nfull) issue(0, I0{});
    if (1 < nfull) issue(1, I1{});
    if (2 < nfull) issue(2, I2{});
    if (nstage > 0 && nfull == 0) copy_stage(0, I0{});
    sy_sync(after(0));

    auto step = [&](int s, auto P) {
        constexpr int p = decltype(P)::value;
        const char* abuf = sy_buf<p>(0);
        const char* bbuf = sy_buf<p>(1);
#pragma unroll
        for (int kk = 0; kk < kStageTok / 16; ++kk) {
            v8bf bf[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) bf[j] = syrk_frag(bbuf, 16 * kk, wn * 2 + j, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const v8bf af = syrk_frag(abuf, 16 * kk, wm * 4 + i, lane);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[j], acc[i][j], 0,
                                                                        0, 0);
            }
            // the loads of stage s + 3 go out once this stage's first
            // fragments are read
            if (kk == 0 && s + 3 < nfull)
                issue(s + 3, std::integral_constant<int, (p + 3) & 3>{});
        }
        if (s + 1 < nstage && s + 1 >= nfull)
            copy_stage(s + 1, std::integral_constant<int, (p + 1) & 3>{});
        sy_sync(after(s + 1));
    };
    for (int s = 0; s < nstage; s += 4) {
        step(s, I0{});
        if (s + 1 < nstage) step(s + 1, I1{});
        if (s + 2 < nstage) step(s + 2, I2{});
        if (s + 3 < nstage) step(s + 3, I3{});
    }
    f32x4* out = part + (((int64_t)split * ntile + tile) * 8 + wave) * 32 * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                out[((i * 2 + j) * 4 + q) * 64 + lane] =
                    f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                          acc[i][j][4 * q + 3]};
}

// bf16 nearest-even of an fp32 value, as bits and as the value it stands for
__device__ inline uint16_t bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ inline float bf16_val(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// C[D][D] (both triangles) = sum over splits of the partials, in split order,
// stored as three bf16 matrices Cs[0] + Cs[1] + Cs[2] = C: each part is the
// rounding of what the previous parts leave, so the three carry C's 24-bit
// significand (the residues are exact in fp32).
__global__ __launch_bounds__(256) void syrk_reduce(const f32x4* __restrict__ part, int D,
                                                   int ntile, int nsplit,
                                                   uint16_t* __restrict__ Cs) {
    const int64_t slots = (int64_t)ntile * 8 * 32 * 64;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= slots) return;
    f32x4 s = part[idx];
    for (int k = 1; k < nsplit; ++k) s += part[idx + k * slots];
    // 32 x 32 accumulator layout: quarter q of lane l holds rows
    // 8 q + 4 (l / 32) .. + 3 of column l % 32
    const int lane = (int)(idx & 63), q = (int)((idx >> 6) & 3), blk = (int)((idx >> 8) & 7);
    const int wave = (int)((idx >> 11) & 7), tile = (int)(idx >> 14);
    int bi, bj;
    tile_of(tile, n_blocks(D), bi, bj);
    const int i = blk >> 1, j = blk & 1;
    const int row0 = bi * kBlk + (wave & 1) * 128 + 32 * i + 8 * q + 4 * (lane >> 5);
    const int col = bj * kBlk + (wave >> 1) * 64 + 32 * j + (lane & 31);
    if (col >= D) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int row = row0 + e;
        if (row >= D) break;
        float r = s[e];
        const int64_t dd = (int64_t)D * D;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            const uint16_t hb = bf16_bits(r);
            Cs[q * dd + (int64_t)row * D + col] = hb;
            if (bi != bj) Cs[q * dd + (int64_t)col * D + row] = hb;
            r -= bf16_val(hb);
        }
    }
}

// ---- 2. out[z] = sum_p A_p B_p^T (fp32 MFMA) -----------------------------------
// F[m][n] = sum_k A[m][k] (B0 + B1 + B2)[n][k] on bf16 MFMA (16x16x32, fp32
// accumulation): A bf16 [M][K] (the projections: rows m < M0 of A0, then
// rows of A1, so that query and key heads share one launch), B the three bf16 parts of
// C [N][K]. Products of bf16 values are exact in fp32, so F carries fp32
// accuracy. Workgroup tile 128 x 128 (8 waves of 64 x 32), k steps of 32
// staged through LDS (double-buffered; rows of 32 elements with the 16-byte
// units XOR-swizzled by row / 4, so the 16-lane groups of a fragment read
// hit distinct banks). M, N and K are multiples of 16.
constexpr int kF3Threads = 512;
constexpr int kF3Tile = 128;
constexpr int kF3RowB = 64;                                 // 32 bf16 per staged row
constexpr int kF3Stage = 4 * kF3Tile * kF3RowB;             // A + three B parts: 32 KB
constexpr int kF3Lds = 2 * kF3Stage;

__device__ inline int f3_swz(int row, int unit) { return unit ^ ((row >> 2) & 3); }

__global__ __launch_bounds__(kF3Threads) void nt_bf16x3(const uint16_t* __restrict__ A0,
                                                        const uint16_t* __restrict__ A1, int M0,
                                                        const uint16_t* __restrict__ Bs, int M,
                                                        int N, int K, float* __restrict__ F) {
    extern __shared__ __attribute__((aligned(16))) char smem3[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m0 = blockIdx.y * kF3Tile, n0 = blockIdx.x * kF3Tile;
    const int wm = (wave & 1) * 64, wn = (wave >> 1) * 32;
    // loader: unit u = tid + 512 h, h < 4: matrix u / 512 (0 = A, 1..3 = B parts),
    // row (u / 4) % 128, 16-byte unit u % 4 of the 32-element k step
    constexpr int NU = 4 * kF3Tile * 4 / kF3Threads;
    const int64_t nk = (int64_t)N * K;
    // this thread's units: fixed rows and matrices, k advancing by 32 per step
    const uint16_t* src[NU];
    bool rok[NU];
    int uoff[NU], ukk[NU];
#pragma unroll
    for (int h = 0; h < NU; ++h) {
        const int u = tid + kF3Threads * h, mat = u >> 9, row = (u >> 2) & 127, un = u & 3;
        const int grow = (mat == 0 ? m0 : n0) + row;
        rok[h] = grow < (mat == 0 ? M : N);
        const int r = rok[h] ? grow : 0;
        src[h] = mat == 0 ? (r < M0 ? A0 + (int64_t)r * K : A1 + (int64_t)(r - M0) * K)
                          : Bs + (mat - 1) * nk + (int64_t)r * K;
        ukk[h] = un * 8;
        uoff[h] = (mat * kF3Tile + row) * kF3RowB + (f3_swz(row, un) << 4);
    }
    u32x4 reg[NU];
    const int nstep = (K + 31) / 32;
    auto load = [&](int st) {
#pragma unroll
        for (int h = 0; h < NU; ++h) {
            const int k = 32 * st + ukk[h];
            const bool ok = rok[h] && k < K;
            reg[h] = *reinterpret_cast<const u32x4*>(src[h] + (ok ? k : 0));
            if (!ok) reg[h] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int h = 0; h < NU; ++h)
            *reinterpret_cast<u32x4*>(smem3 + buf * kF3Stage + uoff[h]) = reg[h];
    };
    // fragment: rows r0 + (lane % 16), k = 8 (lane / 16) .. + 7 of the staged step
    auto frag = [&](const char* base, int mat, int r0) {
        const int row = r0 + (lane & 15), un = lane >> 4;
        const u32x4 v = *reinterpret_cast<const u32x4*>(base + (mat * kF3Tile + row) * kF3RowB +
                                                        (f3_swz(row, un) << 4));
        return __builtin_bit_cast(v8bf, v);
    };
    f32x4 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    load(0);
    store(0);
    __syncthreads();
    for (int s = 0; s < nstep; ++s) {
        const bool more = s + 1 < nstep;
        if (more) load(s + 1);
        const char* base = smem3 + (s & 1) * kF3Stage;
        v8bf af[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = frag(base, 0, wm + 16 * i);
#pragma unroll
        for (int q = 1; q <= 3; ++q)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const v8bf bf = frag(base, q, wn + 16 * j);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf, acc[i][j], 0,
                                                                        0, 0);
            }
        if (more) store((s + 1) & 1);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn + 16 * j + (lane & 15);
            const int rb = m0 + wm + 16 * i + 4 * (lane >> 4);
            if (col >= N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (rb + e < M) F[(int64_t)(rb + e) * N + col] = acc[i][j][e];
        }
}

// out[z][i][j] = sum_{p < nsum} sum_k A[a0 + z*azs + p*aps + i][k] * B[b0 + ...][k],
// A bf16 or f32, B f32, rows of length K (K % 16 == 0, M and N multiples of 16).
struct NtJob {
    const void* A;
    const float* B;
    float* out;
    int64_t lda, ldb, ldo;         // row strides (elements)
    int64_t a_zs, b_zs, o_zs;      // batch strides: rows of A and B, elements of out
    int64_t a_ps, b_ps;            // rows per sum term
    int M, N, K, nsum;
    int kspl;                      // K splits: block z = batch * kspl + split, each
                                   // split writing its own output (partials)
};

template <typename TA>
__device__ inline f32x4 load4(const TA* p);
template <>
__device__ inline f32x4 load4<float>(const float* p) {
    return *reinterpret_cast<const f32x4*>(p);
}
template <>
__device__ inline f32x4 load4<uint16_t>(const uint16_t* p) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u),
                 __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xffff0000u)};
}

// 64 x 64 output tile per workgroup, 32 x 32 per wave (2 x 2 blocks of 16).
template <typename TA>
__global__ __launch_bounds__(kNtThreads) void nt_gemm(NtJob job) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int z = blockIdx.z / job.kspl, ks = blockIdx.z - z * job.kspl;
    const int kper = job.K / job.kspl, kbeg = ks * kper;
    const int i0 = blockIdx.y * 64 + (wave & 1) * 32, j0 = blockIdx.x * 64 + (wave >> 1) * 32;
    const TA* A = static_cast<const TA*>(job.A) + z * job.a_zs * job.lda + kbeg;
    const float* B = job.B + z * job.b_zs * job.ldb + kbeg;
    const int G = lane >> 4, r = lane & 15;
    bool rok[2], cok[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        rok[b] = i0 + 16 * b < job.M;
        cok[b] = j0 + 16 * b < job.N;
    }
    f32x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < job.nsum; ++p) {
        const TA* ap[2];
        const float* bp[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            ap[b] = A + (p * job.a_ps + (rok[b] ? i0 + 16 * b + r : 0)) * job.lda + 4 * G;
            bp[b] = B + (p * job.b_ps + (cok[b] ? j0 + 16 * b + r : 0)) * job.ldb + 4 * G;
        }
        f32x4 av[2], bv[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            av[b] = load4<TA>(ap[b]);
            bv[b] = load4<float>(bp[b]);
        }
        for (int k = 0; k < kper; k += 16) {
            f32x4 an[2], bn[2];
            const bool more = k + 16 < kper;
            if (more) {
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    an[b] = load4<TA>(ap[b] + k + 16);
                    bn[b] = load4<float>(bp[b] + k + 16);
                }
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a][s], bv[b][s],
                                                                         acc[a][b], 0, 0, 0);
            if (more) {
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    av[b] = an[b];
                    bv[b] = bn[b];
                }
            }
        }
    }
    float* o = job.out + (int64_t)blockIdx.z * job.o_zs;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            if (!rok[a] || !cok[b]) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[(int64_t)(i0 + 16 * a + 4 * G + e) * job.ldo + j0 + 16 * b + r] = acc[a][b][e];
        }
}

// out[r][e] = sum_{t < nt} part[r * nt + t][e], in t order
__global__ __launch_bounds__(256) void sum_parts(const float* __restrict__ part, int nt,
                                                 int64_t E, int R, float* __restrict__ out) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= E * R) return;
    const int64_t r = idx / E, e = idx - r * E;
    float s = 0.f;
    for (int t = 0; t < nt; ++t) s += part[(r * nt + t) * E + e];
    out[idx] = s;
}

// ---- 3. per-pair algebra (fp64) ------------------------------------------------
struct PairOut {
    double w_logit;   // Eq. 16
    double w_key;     // Eq. 35: tr(Delta)
    double l_avg;     // Eq. 13 at the average of the two heads: tr(Delta P) / 4
    double sweeps;    // Jacobi sweeps run
    double gj;        // 1: P inverted by Gauss-Jordan (Y, Z formed by pair_yz)
};

__device__ inline void pair_of_index(int p, int n, int& a, int& b) {
    a = 0;
    while (p >= n - 1 - a) {
        p -= n - 1 - a;
        ++a;
    }
    b = a + 1 + p;
}

// round r (0 .. d-2) of the cyclic tournament on d players: pair k
__device__ inline void tourney(int r, int k, int d, int& p, int& q) {
    const int m = d - 1;
    int u, v;
    if (k == 0) {
        u = r;
        v = m;
    } else {
        u = (r + k) % m;
        v = (r - k + m) % m;
    }
    p = u < v ? u : v;
    q = u < v ? v : u;
}

__device__ inline double block_sum(double v, double* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    double s = 0.0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
    return s;
}

struct PairArgs {
    const float* S;      // [n][d][d]
    const float* H;      // [n d][n d]
    double* Y;           // [npairs][d][d]  P^+ S_a
    double* Z;           // [npairs][d][d]  P^+ S_b
    double* Dl;          // [npairs][d][d]  Delta
    double* Pinv;        // [npairs][d][d]  P^{-1} (Gauss-Jordan path)
    double* part;        // [npairs][2 tiles]  loss partials per (term, output tile)
    double2* rec;        // [npairs][kMaxSweeps][d - 1][d / 2]  (c, s)
    PairOut* out;        // [npairs]
    int n, d, strategy;
};

// Delta(k, j) of pair (a, b) from the realized-key Gram
__device__ inline double delta_at(const float* H, int hd, int a, int b, int d, int k, int j) {
    const int64_t ra = (int64_t)(a * d + k) * hd, rb = (int64_t)(b * d + k) * hd;
    return ((double)H[ra + a * d + j] - (double)H[ra + b * d + j]) -
           ((double)H[rb + a * d + j] - (double)H[rb + b * d + j]);
}

// Replay the recorded rotations on the d x d matrix in LDS (row stride d + 1):
// forward applies J^T from the left in recording order, backward applies J
// from the left in reverse order. cs is a double-buffered staging area.
__device__ void replay(double* Ym, int d, const double2* rec, int nrounds, bool forward,
                       double2* cs) {
    const int np = d / 2, tid = threadIdx.x;
    auto round_at = [&](int i) { return forward ? i : nrounds - 1 - i; };
    if (nrounds == 0) return;
    if (tid < np) cs[tid] = rec[(int64_t)round_at(0) * np + tid];
    __syncthreads();
    for (int i = 0; i < nrounds; ++i) {
        double2 nx = double2{1.0, 0.0};
        if (i + 1 < nrounds && tid < np) nx = rec[(int64_t)round_at(i + 1) * np + tid];
        const int rr = round_at(i) % (d - 1);
        const double2* cur = cs + (i & 1) * 64;
        for (int idx = tid; idx < np * d; idx += kPairThreads) {
            const int k = idx / d, col = idx - k * d;
            int p, q;
            tourney(rr, k, d, p, q);
            const double c = cur[k].x, s = cur[k].y;
            const double yp = Ym[p * (d + 1) + col], yq = Ym[q * (d + 1) + col];
            if (forward) {
                Ym[p * (d + 1) + col] = c * yp - s * yq;
                Ym[q * (d + 1) + col] = s * yp + c * yq;
            } else {
                Ym[p * (d + 1) + col] = c * yp + s * yq;
                Ym[q * (d + 1) + col] = -s * yp + c * yq;
            }
        }
        if (i + 1 < nrounds && tid < np) cs[((i + 1) & 1) * 64 + tid] = nx;
        __syncthreads();
    }
}

// Two sums over the workgroup at once (one pair of barriers).
__device__ inline void block_sum2(double& x, double& y, double* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        x += __shfl_xor(x, o);
        y += __shfl_xor(y, o);
    }
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
        red[2 * w] = x;
        red[2 * w + 1] = y;
    }
    __syncthreads();
    x = y = 0.0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) {
        x += red[2 * i];
        y += red[2 * i + 1];
    }
}

// Largest eigenvalue of the symmetric d x d matrix in LDS (row stride ld) by
// power iteration from a fixed start vector (4 threads per row); the estimate
// is the Rayleigh quotient of the last iterate.
__device__ double power_max(const double* Am, int d, int ld, double* v, double* w,
                            double* red, int iters) {
    const int tid = threadIdx.x, row = tid >> 2, q = tid & 3;
    if (tid < d) v[tid] = 1.0 + 0.125 * (tid % 5);
    __syncthreads();
    double nv = block_sum(tid < d ? v[tid] * v[tid] : 0.0, red);
    double rq = 0.0;
    for (int it = 0; it < iters; ++it) {
        double y = 0.0;
        if (row < d) {
            const double* r_ = Am + row * ld;
#pragma unroll 8
            for (int j = q; j < d; j += 4) y += r_[j] * v[j];
        }
        y += __shfl_xor(y, 1);
        y += __shfl_xor(y, 2);
        const bool own = q == 0 && row < d;
        double vy = own ? v[row] * y : 0.0, yy = own ? y * y : 0.0;
        if (own) w[row] = y;
        block_sum2(vy, yy, red);
        rq = vy / nv;
        if (!(yy > 0.0) || !isfinite(yy)) return yy == 0.0 ? 0.0 : rq;
        const double sc = 1.0 / sqrt(yy);
        if (tid < d) v[tid] = w[tid] * sc;
        nv = 1.0;
        __syncthreads();
    }
    return rq;
}

// In-place Gauss-Jordan inversion of the symmetric positive definite d x d
// matrix in LDS (no pivoting), eliminating 4 x 4 pivot blocks K:
//   A_KK <- A_KK^{-1} =: Pi,            A_KJ <- Pi A_KJ,
//   A_IJ <- A_IJ - A_IK Pi A_KJ,        A_IK <- -A_IK Pi      (I, J outside K),
// which is four scalar steps at once (A[i][j] -= A[i][k] A[k][j] / A[k][k],
// row k scaled by 1 / A[k][k], column k by -1 / A[k][k], pivot inverted) and
// meets the same pivots, the Schur-complement diagonals. Every thread
// inverts the 4 x 4 block itself by those scalar steps. Thread (rb, cb)
// keeps the 4 x 8 block at rows 4 rb, columns 8 cb in registers for the
// whole elimination; the column block [d][4] and the row block [4][d] of K
// are broadcast through LDS, alternating between two halves of fcol and rowk
// ([2][4 d] each) so that one barrier per block step suffices: a thread
// writes step t + 2's half only after the barrier of step t + 1, which every
// thread passes after its reads of step t.
// Returns the smallest pivot (<= 0 or NaN: not positive definite).
__device__ double gj_invert(double* Am, int d, int ld, double* fcol, double* rowk) {
    const int tid = threadIdx.x, rb = tid >> 4, cb = tid & 15;
    const int r0 = 4 * rb, c0 = 8 * cb;
    const bool act = r0 < d && c0 < d;   // d is a multiple of 16: blocks are whole
    double v[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) v[r][c] = act ? Am[(r0 + r) * ld + c0 + c] : 0.0;
    double minpiv = INFINITY;
    for (int kb = 0; kb < d / 4; ++kb) {
        const int k0 = 4 * kb;
        const bool hi = kb & 1;   // uniform: K is columns 4 .. 7 of its thread column
        double* fc = fcol + (kb & 1) * 4 * d;   // [d][4]
        double* rk = rowk + (kb & 1) * 4 * d;   // [4][d]
        const bool colk = act && (kb >> 1) == cb, rowkk = act && kb == rb;
        // (the halves of v are named by constant indices in separate branches:
        // an index chosen at run time would put v in scratch memory)
        if (colk && hi) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int m = 0; m < 4; ++m) fc[(r0 + r) * 4 + m] = v[r][4 + m];
        } else if (colk) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int m = 0; m < 4; ++m) fc[(r0 + r) * 4 + m] = v[r][m];
        }
        if (rowkk) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int c = 0; c < 8; ++c) rk[m * d + c0 + c] = v[m][c];
        }
        __syncthreads();
        double f[4][4];
        if (act) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int m = 0; m < 4; ++m) f[r][m] = fc[(r0 + r) * 4 + m];
        }
        // Pi = A_KK^{-1} by four scalar Gauss-Jordan steps
        double pi[4][4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int n = 0; n < 4; ++n) pi[m][n] = rk[m * d + k0 + n];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const double pk = pi[q][q];
            minpiv = fmin(minpiv, pk);
            const double ip = 1.0 / pk;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i == q) continue;
                const double fi = pi[i][q] * ip;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (j != q) pi[i][j] -= fi * pi[q][j];
                pi[i][q] = -fi;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (j != q) pi[q][j] *= ip;
            pi[q][q] = ip;
        }
        if (act) {
            // by halves of the thread's 8 columns: rj <- Pi A_KJ, then
            // A_IJ -= A_IK (Pi A_KJ); rows of K take Pi A_KJ
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                double rj[4][4];
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int c = 0; c < 4; ++c) rj[m][c] = rk[m * d + c0 + 4 * h + c];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    double t[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        t[m] = pi[m][0] * rj[0][c] + pi[m][1] * rj[1][c] + pi[m][2] * rj[2][c] +
                               pi[m][3] * rj[3][c];
#pragma unroll
                    for (int m = 0; m < 4; ++m) rj[m][c] = t[m];
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        v[r][4 * h + c] -= f[r][0] * rj[0][c] + f[r][1] * rj[1][c] +
                                           f[r][2] * rj[2][c] + f[r][3] * rj[3][c];
                if (rowkk)
#pragma unroll
                    for (int m = 0; m < 4; ++m)
#pragma unroll
                        for (int c = 0; c < 4; ++c) v[m][4 * h + c] = rj[m][c];
            }
            if (colk) {   // A_IK <- -A_IK Pi, and A_KK <- Pi in the rows of K
                double e[4][4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        e[r][m] = rowkk ? pi[r][m]
                                        : -(f[r][0] * pi[0][m] + f[r][1] * pi[1][m] +
                                            f[r][2] * pi[2][m] + f[r][3] * pi[3][m]);
                if (hi) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int m = 0; m < 4; ++m) v[r][4 + m] = e[r][m];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int m = 0; m < 4; ++m) v[r][m] = e[r][m];
                }
            }
        }
    }
    if (act)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c) Am[(r0 + r) * ld + c0 + c] = v[r][c];
    __syncthreads();
    return minpiv;
}

__device__ inline double ldd(const double* p) { return *p; }
__device__ inline double ldd(const float* p) { return (double)*p; }

// Workgroup GEMM over d x d row-major matrices in global memory, one 64 x 64
// output tile (ti, tj) per call: C1 = A1 B1 (and C2 = A2 B2 when DUAL). Each thread holds 4
// rows x 2 columns of a tile; 16-wide k panels are double-buffered in LDS
// (pan: 2 x (DUAL ? 4 : 2) panels of [16][68] doubles, A panels stored
// k-major) while the next panel is loaded into registers. DUAL returns this
// thread's share of sum(C1 .* C2); otherwise C1 is stored to out and 0 returned.
constexpr int kPanLd = 68;
constexpr int kPanWords = 16 * kPanLd;
template <bool DUAL, typename TA1, typename TB1, typename TA2, typename TB2>
__device__ double tile_gemm(int d, int ti, int tj, const TA1* A1, const TB1* B1, const TA2* A2,
                            const TB2* B2, double* out, double* pan) {
    constexpr int NP = DUAL ? 4 : 2;
    const int tid = threadIdx.x, tr = (tid >> 5) * 4, tc = (tid & 31) * 2;
    // this thread's two elements of every panel: A (row ar, k ak), B (k bk, col bc)
    const int ar0 = tid >> 4, ak = tid & 15, ar1 = ar0 + 32;
    const int bk0 = tid >> 6, bc = tid & 63, bk1 = bk0 + 8;
    const int npan = d / 16;
    double dot = 0.0;
    {
            double acc1[4][2], acc2[4][2];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 2; ++c) acc1[r][c] = acc2[r][c] = 0.0;
            const bool a0 = ti + ar0 < d, a1 = ti + ar1 < d, bb = tj + bc < d;
            const int64_t ra0 = (int64_t)(a0 ? ti + ar0 : 0) * d + ak;
            const int64_t ra1 = (int64_t)(a1 ? ti + ar1 : 0) * d + ak;
            const int64_t rb0 = (int64_t)bk0 * d + (bb ? tj + bc : 0);
            const int64_t rb1 = (int64_t)bk1 * d + (bb ? tj + bc : 0);
            double x0, x1, y0, y1, u0 = 0, u1 = 0, w0 = 0, w1 = 0;
            x0 = ldd(A1 + ra0);
            x1 = ldd(A1 + ra1);
            y0 = ldd(B1 + rb0);
            y1 = ldd(B1 + rb1);
            if constexpr (DUAL) {
                u0 = ldd(A2 + ra0);
                u1 = ldd(A2 + ra1);
                w0 = ldd(B2 + rb0);
                w1 = ldd(B2 + rb1);
            }
            for (int p = 0; p < npan; ++p) {
                double* base = pan + (p & 1) * NP * kPanWords;
                base[ak * kPanLd + ar0] = a0 ? x0 : 0.0;
                base[ak * kPanLd + ar1] = a1 ? x1 : 0.0;
                base[kPanWords + bk0 * kPanLd + bc] = bb ? y0 : 0.0;
                base[kPanWords + bk1 * kPanLd + bc] = bb ? y1 : 0.0;
                if constexpr (DUAL) {
                    base[2 * kPanWords + ak * kPanLd + ar0] = a0 ? u0 : 0.0;
                    base[2 * kPanWords + ak * kPanLd + ar1] = a1 ? u1 : 0.0;
                    base[3 * kPanWords + bk0 * kPanLd + bc] = bb ? w0 : 0.0;
                    base[3 * kPanWords + bk1 * kPanLd + bc] = bb ? w1 : 0.0;
                }
                __syncthreads();
                if (p + 1 < npan) {   // next panel in flight while this one is used
                    const int64_t ko = (int64_t)16 * (p + 1), kr = ko * d;
                    x0 = ldd(A1 + ra0 + ko);
                    x1 = ldd(A1 + ra1 + ko);
                    y0 = ldd(B1 + rb0 + kr);
                    y1 = ldd(B1 + rb1 + kr);
                    if constexpr (DUAL) {
                        u0 = ldd(A2 + ra0 + ko);
                        u1 = ldd(A2 + ra1 + ko);
                        w0 = ldd(B2 + rb0 + kr);
                        w1 = ldd(B2 + rb1 + kr);
                    }
                }
#pragma unroll
                for (int kk = 0; kk < 16; ++kk) {
                    const double* ap = base + kk * kPanLd + tr;
                    const double* bp = base + kPanWords + kk * kPanLd + tc;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int c = 0; c < 2; ++c) acc1[r][c] += ap[r] * bp[c];
                    if constexpr (DUAL) {
                        const double* ap2 = base + 2 * kPanWords + kk * kPanLd + tr;
                        const double* bp2 = base + 3 * kPanWords + kk * kPanLd + tc;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
#pragma unroll
                            for (int c = 0; c < 2; ++c) acc2[r][c] += ap2[r] * bp2[c];
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int i = ti + tr + r, jj = tj + tc + c;
                    if (i < d && jj < d) {
                        if constexpr (DUAL)
                            dot += acc1[r][c] * acc2[r][c];
                        else
                            out[(int64_t)i * d + jj] = acc1[r][c];
                    }
                }
        }
    return dot;
}

// doubles of the matrix region: the Jacobi matrix, or the GEMM panels
__host__ __device__ inline int pair_matrix_words(int d) {
    const int jac = d * (d + 1), gem = 2 * 4 * kPanWords;
    return jac > gem ? jac : gem;
}

// P^+ S_a into Y and P^+ S_b into Z through the eigen-decomposition of
// P = S_a + S_b: cyclic Jacobi rotations on the matrix in LDS (a round rotates
// d / 2 disjoint index pairs), each round's rotations recorded in rec, then
// replayed on S_a (and on I when eigenvalues fall at or below the cutoff
// 2^-23 d lambda_max, to form P P^+). Returns the sweeps run.
__device__ int jacobi_pinv(double* Am, int d, const float* Sa, const float* Sb, double* Y,
                           double* Z, double2* rec, double2* cs, double* lam, double* red,
                           int* flag) {
    const int np = d / 2, ld = d + 1, tid = threadIdx.x;
    for (int idx = tid; idx < d * d; idx += kPairThreads) {
        const int i = idx / d, j = idx - i * d;
        Am[i * ld + j] = (double)Sa[idx] + (double)Sb[idx];
    }
    __syncthreads();
    // cyclic Jacobi (rotations zero one off-diagonal pair each; a round
    // rotates d / 2 disjoint pairs at once)
    int sweeps = 0;
    for (; sweeps < kMaxSweeps; ++sweeps) {
        double off = 0.0, dia = 0.0;
        for (int idx = tid; idx < d * d; idx += kPairThreads) {
            const int i = idx / d, j = idx - i * d;
            const double v = Am[i * ld + j];
            if (i == j)
                dia += v * v;
            else
                off += v * v;
        }
        off = block_sum(off, red);
        dia = block_sum(dia, red);
        // off-diagonal norm at the rounding level of a d x d fp64 matrix: done
        if (!(off > (double)d * d * 0x1p-104 * (off + dia))) break;
        for (int r = 0; r < d - 1; ++r) {
            if (tid < np) {
                int p, q;
                tourney(r, tid, d, p, q);
                const double apq = Am[p * ld + q];
                double c = 1.0, s = 0.0;
                if (apq != 0.0) {
                    const double tau = (Am[q * ld + q] - Am[p * ld + p]) / (2.0 * apq);
                    const double at = fabs(tau);
                    double t = at > 1e150 ? 0.5 / at : 1.0 / (at + sqrt(1.0 + tau * tau));
                    if (tau < 0.0) t = -t;
                    c = 1.0 / sqrt(1.0 + t * t);
                    s = t * c;
                }
                cs[tid] = double2{c, s};
                rec[((int64_t)sweeps * (d - 1) + r) * np + tid] = double2{c, s};
            }
            __syncthreads();
            for (int blk = tid; blk < np * np; blk += kPairThreads) {
                const int k = blk / np, l = blk - k * np;
                int pk, qk, pl, ql;
                tourney(r, k, d, pk, qk);
                tourney(r, l, d, pl, ql);
                const double ck = cs[k].x, sk = cs[k].y, cl = cs[l].x, sl = cs[l].y;
                const double x00 = Am[pk * ld + pl], x01 = Am[pk * ld + ql];
                const double x10 = Am[qk * ld + pl], x11 = Am[qk * ld + ql];
                const double y00 = ck * x00 - sk * x10, y01 = ck * x01 - sk * x11;
                const double y10 = sk * x00 + ck * x10, y11 = sk * x01 + ck * x11;
                double z00 = cl * y00 - sl * y01, z01 = sl * y00 + cl * y01;
                double z10 = cl * y10 - sl * y11, z11 = sl * y10 + cl * y11;
                if (k == l) z01 = z10 = 0.0;
                Am[pk * ld + pl] = z00;
                Am[pk * ld + ql] = z01;
                Am[qk * ld + pl] = z10;
                Am[qk * ld + ql] = z11;
            }
            __syncthreads();
        }
    }
    // eigenvalues, cutoff (2^-23 d lambda_max), reciprocals
    double lmax = 0.0;
    for (int i = 0; i < d; ++i) lmax = fmax(lmax, Am[i * ld + i]);
    const double cut = 0x1p-23 * d * lmax;
    __syncthreads();
    if (tid == 0) *flag = 0;
    __syncthreads();
    if (tid < d) {
        const double l = Am[tid * ld + tid];
        lam[tid] = l > cut ? 1.0 / l : 0.0;
        if (!(l > cut)) atomicOr(flag, 1);
    }
    __syncthreads();
    const bool trunc = *flag != 0;
    const int nrounds = sweeps * (d - 1);

    // Y = P^+ S_a = V Lambda^+ V^T S_a
    for (int pass = 0; pass < (trunc ? 2 : 1); ++pass) {
        for (int idx = tid; idx < d * d; idx += kPairThreads) {
            const int i = idx / d, j = idx - i * d;
            Am[i * ld + j] = pass == 0 ? (double)Sa[idx] : (i == j ? 1.0 : 0.0);
        }
        __syncthreads();
        replay(Am, d, rec, nrounds, true, cs);
        for (int idx = tid; idx < d * d; idx += kPairThreads) {
            const int i = idx / d, j = idx - i * d;
            // pass 1 forms P P^+ = V diag(lambda > cut) V^T
            Am[i * ld + j] *= pass == 0 ? lam[i] : (lam[i] != 0.0 ? 1.0 : 0.0);
        }
        __syncthreads();
        replay(Am, d, rec, nrounds, false, cs);
        for (int idx = tid; idx < d * d; idx += kPairThreads) {
            const int i = idx / d, j = idx - i * d;
            if (pass == 0)
                Y[idx] = Am[i * ld + j];
            else
                Z[idx] = Am[i * ld + j];
        }
        __syncthreads();
    }
    // Z = P^+ S_b = P P^+ - Y  (P P^+ = I without truncation)
    for (int idx = tid; idx < d * d; idx += kPairThreads) {
        const int i = idx / d, j = idx - i * d;
        const double e = trunc ? Z[idx] : (i == j ? 1.0 : 0.0);
        Z[idx] = e - Y[idx];
    }
    return sweeps;
}

// One workgroup per pair (a, b), a < b.
__global__ __launch_bounds__(kPairThreads) void merge_pairs(PairArgs pa) {
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    const int d = pa.d, np = d / 2, ld = d + 1, tid = threadIdx.x;
    const int pidx = blockIdx.x;
    int a, b;
    pair_of_index(pidx, pa.n, a, b);
    double* Am = reinterpret_cast<double*>(smem_raw);   // [d][d + 1], later GEMM panels
    double2* cs = reinterpret_cast<double2*>(Am + pair_matrix_words(d));   // [2][64]
    double* lam = reinterpret_cast<double*>(cs + 128);       // [d]
    double* va = lam + 128;                                   // [2][4][128] power-iteration
    double* vb = va + 1024;                                   // vectors, Gauss-Jordan buffers
    double* red = vb + 1024;                                  // [16]
    int* flag = reinterpret_cast<int*>(red + 16);
    const int hd = pa.n * d;
    const float* Sa = pa.S + (int64_t)a * d * d;
    const float* Sb = pa.S + (int64_t)b * d * d;
    double* Y = pa.Y + (int64_t)pidx * d * d;
    double* Z = pa.Z + (int64_t)pidx * d * d;
    double* Dl = pa.Dl + (int64_t)pidx * d * d;

    // Delta to global, P into LDS; tr(Delta), tr(Delta P), ||P||_F^2
    double t1 = 0.0, t2 = 0.0, t3 = 0.0;
    for (int idx = tid; idx < d * d; idx += kPairThreads) {
        const int i = idx / d, j = idx - i * d;
        const double P = (double)Sa[idx] + (double)Sb[idx];
        const double dl = delta_at(pa.H, hd, a, b, d, i, j);
        Am[i * ld + j] = P;
        Dl[idx] = dl;
        t2 += dl * P;
        t3 += P * P;
        if (i == j) t1 += dl;
    }
    block_sum2(t1, t2, red);
    const double trd = t1, trdp = t2;
    const double pf2 = block_sum(t3, red);

    if (pa.strategy != 0) {
        for (int idx = tid; idx < d * d; idx += kPairThreads) {
            const int i = idx / d, j = idx - i * d;
            Y[idx] = Z[idx] = i == j ? 0.5 : 0.0;
        }
        if (tid == 0) pa.out[pidx] = PairOut{0.0, trd, 0.25 * trdp, 0.0};
        return;
    }

    // Positive definite P with every eigenvalue well above the pseudo-inverse
    // cutoff 2^-23 d lambda_max: P^+ = P^{-1}, by Gauss-Jordan. The Frobenius
    // norms of P and P^{-1} bound the extreme eigenvalues; only when those
    // bounds do not settle it are the eigenvalues estimated by power
    // iteration. When P is not clearly regular, the eigen-decomposition
    // decides which eigenvalues count as zero.
    const double minpiv = gj_invert(Am, d, ld, va, vb);
    double q2 = 0.0;
    for (int idx = tid; idx < d * d; idx += kPairThreads) {
        const int i = idx / d, j = idx - i * d;
        const double v = Am[i * ld + j];
        q2 += v * v;
    }
    const double pinv_f = sqrt(block_sum(q2, red));
    double* Pi = pa.Pinv + (int64_t)pidx * d * d;
    bool regular = minpiv > 0.0 && isfinite(pinv_f) && pinv_f > 0.0 && pf2 > 0.0;
    // lambda_min >= 1 / ||P^{-1}||_F and lambda_max <= ||P||_F: that settles it
    // unless the conditioning is within a factor of about d of the cutoff
    if (regular && !(1.0 / pinv_f > 4.0 * 0x1p-23 * d * sqrt(pf2))) {
        // estimate both extreme eigenvalues: power iteration on P^{-1}, then
        // on P reloaded from the statistics (P^{-1} waits in global memory)
        const double linv = power_max(Am, d, ld, va, vb, red, 40);   // 1 / lambda_min
        for (int idx = tid; idx < d * d; idx += kPairThreads) {
            const int i = idx / d, j = idx - i * d;
            Pi[idx] = Am[i * ld + j];
            Am[i * ld + j] = (double)Sa[idx] + (double)Sb[idx];
        }
        __syncthreads();
        const double lmax_p = power_max(Am, d, ld, va, vb, red, 40);
        regular = isfinite(linv) && linv > 0.0 && 1.0 / linv > 4.0 * 0x1p-23 * d * lmax_p;
        for (int idx = tid; idx < d * d; idx += kPairThreads) {
            const int i = idx / d, j = idx - i * d;
            Am[i * ld + j] = Pi[idx];
        }
        __syncthreads();
    }
    int sweeps = 0;
    if (regular) {   // Y = P^{-1} S_a and Z = I - Y follow, tile by tile, in pair_yz
        for (int idx = tid; idx < d * d; idx += kPairThreads) {
            const int i = idx / d, j = idx - i * d;
            Pi[idx] = Am[i * ld + j];
        }
    } else {
        sweeps = jacobi_pinv(Am, d, Sa, Sb, Y, Z, pa.rec + (int64_t)pidx * kMaxSweeps * (d - 1) * np,
                             cs, lam, red, flag);
    }
    if (tid == 0) pa.out[pidx] = PairOut{0.0, trd, 0.25 * trdp, (double)sweeps, regular ? 1.0 : 0.0};
}

// Tile-parallel stages of the pair algebra: one 64 x 64 output tile per
// workgroup. pair_yz forms Y = P^{-1} S_a and Z = I - Y for the pairs that
// took the Gauss-Jordan path; pair_loss evaluates the two terms of
// w = <Z Delta, S_a Z> + <Y Delta, S_b Y> per tile into `part`, summed in a
// fixed order by match_weights.
__global__ __launch_bounds__(kPairThreads) void pair_yz(PairArgs pa) {
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    const int pidx = blockIdx.x, d = pa.d, nt = (d + 63) / 64;
    if (pa.strategy != 0 || pa.out[pidx].gj == 0.0) return;   // uniform
    int a, b;
    pair_of_index(pidx, pa.n, a, b);
    const int ti = (blockIdx.y / nt) * 64, tj = (blockIdx.y % nt) * 64;
    double* Y = pa.Y + (int64_t)pidx * d * d;
    double* Z = pa.Z + (int64_t)pidx * d * d;
    tile_gemm<false>(d, ti, tj, pa.Pinv + (int64_t)pidx * d * d, pa.S + (int64_t)a * d * d,
                     pa.Pinv, pa.S, Y, reinterpret_cast<double*>(smem_raw));
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += kPairThreads) {
        const int i = ti + (e >> 6), j = tj + (e & 63);
        if (i < d && j < d) Z[(int64_t)i * d + j] = (i == j ? 1.0 : 0.0) - Y[(int64_t)i * d + j];
    }
}

__global__ __launch_bounds__(kPairThreads) void pair_loss(PairArgs pa) {
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    const int pidx = blockIdx.x, d = pa.d, nt = (d + 63) / 64, t2 = nt * nt;
    if (pa.strategy != 0) return;
    int a, b;
    pair_of_index(pidx, pa.n, a, b);
    const int term = blockIdx.y / t2, tile = blockIdx.y % t2;
    const int ti = (tile / nt) * 64, tj = (tile % nt) * 64;
    const double* Y = pa.Y + (int64_t)pidx * d * d;
    const double* Z = pa.Z + (int64_t)pidx * d * d;
    const double* Dl = pa.Dl + (int64_t)pidx * d * d;
    const double* L1 = term == 0 ? Z : Y;
    const float* Sm = pa.S + (int64_t)(term == 0 ? a : b) * d * d;
    double* pan = reinterpret_cast<double*>(smem_raw);
    double dot = tile_gemm<true>(d, ti, tj, L1, Dl, Sm, L1, nullptr, pan);
    dot = block_sum(dot, pan + 8 * kPanWords);
    if (threadIdx.x == 0) pa.part[(int64_t)pidx * 2 * t2 + blockIdx.y] = dot;
}

// ---- 4. matching ----------------------------------------------------------------
struct MatchWs {
    double* w;        // [n][n] weights the matching runs on
    double* dp;       // [2^n]
    int8_t* ch;       // [2^n]  partner of the lowest head of the mask
    int32_t* pairs;   // [n]    matched pairs (a, b) by increasing a
};

__global__ __launch_bounds__(256) void match_weights(PairOut* po, const double* part, int t2,
                                                     int n, int strategy, MatchWs m) {
    const int np = n * (n - 1) / 2;
    if (strategy == 0) {
        for (int p = threadIdx.x; p < np; p += 256) {
            double w = 0.0;
            for (int y = 0; y < 2 * t2; ++y) w += part[(int64_t)p * 2 * t2 + y];
            po[p].w_logit = w;
        }
        __syncthreads();
    }
    for (int p = threadIdx.x; p < np; p += 256) {
        int a, b;
        pair_of_index(p, n, a, b);
        const double v = strategy == 0 ? po[p].w_logit : (strategy == 1 ? po[p].w_key : 0.0);
        m.w[a * n + b] = v;
        m.w[b * n + a] = v;
    }
    for (int i = threadIdx.x; i < n; i += 256) m.w[i * n + i] = 0.0;
    if (threadIdx.x == 0) m.dp[0] = 0.0;
}

__global__ __launch_bounds__(256) void match_layer(int n, int pop, MatchWs m) {
    const int64_t mask = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (mask >= ((int64_t)1 << n) || __popcll((uint64_t)mask) != pop) return;
    const int i = __ffsll((unsigned long long)mask) - 1;
    double best = 0.0;
    int bj = -1;
    for (int j = i + 1; j < n; ++j) {
        if (!((mask >> j) & 1)) continue;
        const double v = m.w[i * n + j] + m.dp[mask ^ ((int64_t)1 << i) ^ ((int64_t)1 << j)];
        if (bj < 0 || v < best) {
            best = v;
            bj = j;
        }
    }
    m.dp[mask] = best;
    m.ch[mask] = (int8_t)bj;
}

__global__ void match_finish(const PairOut* po, int n, int strategy, MatchWs m,
                             int32_t* __restrict__ sigma, double* __restrict__ pair_w,
                             double* __restrict__ objective) {
    if (pair_w)
        for (int e = threadIdx.x; e < n * n; e += blockDim.x) pair_w[e] = m.w[e];
    if (threadIdx.x != 0) return;
    int64_t mask = ((int64_t)1 << n) - 1;
    double obj = 0.0;
    for (int i = 0; i < n / 2; ++i) {
        int a, b;
        if (strategy == 2) {
            a = 2 * i;
            b = 2 * i + 1;
        } else {
            a = __ffsll((unsigned long long)mask) - 1;
            b = m.ch[mask];
            mask ^= ((int64_t)1 << a) | ((int64_t)1 << b);
        }
        m.pairs[2 * i] = a;
        m.pairs[2 * i + 1] = b;
        sigma[2 * i] = a;
        sigma[2 * i + 1] = b;
        const int p = a * n - a * (a + 1) / 2 + (b - a - 1);
        obj += strategy == 0 ? po[p].w_logit : po[p].l_avg;
    }
    if (objective) *objective = obj;
}

// ---- 5. merged projections ----------------------------------------------------
// merged[i][c][k] = sum_e Y[c][e] Wk[a d + e][k] + Z[c][e] Wk[b d + e][k]
__global__ __launch_bounds__(256) void merge_apply(const uint16_t* __restrict__ wk,
                                                   const double* __restrict__ Y,
                                                   const double* __restrict__ Z,
                                                   const int32_t* __restrict__ pairs, int n,
                                                   int d, int D, float* __restrict__ merged) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    const int c = blockIdx.y, i = blockIdx.z;
    if (k >= D) return;
    const int a = pairs[2 * i], b = pairs[2 * i + 1];
    const int p = a * n - a * (a + 1) / 2 + (b - a - 1);
    const double* y = Y + ((int64_t)p * d + c) * d;
    const double* z = Z + ((int64_t)p * d + c) * d;
    const uint16_t* wa = wk + (int64_t)a * d * D + k;
    const uint16_t* wb = wk + (int64_t)b * d * D + k;
    double s = 0.0;
    for (int e = 0; e < d; ++e) {
        const double va = (double)__uint_as_float((uint32_t)wa[(int64_t)e * D] << 16);
        const double vb = (double)__uint_as_float((uint32_t)wb[(int64_t)e * D] << 16);
        s += y[e] * va + z[e] * vb;
    }
    merged[((int64_t)i * d + c) * D + k] = (float)s;
}

// ---- App. B: induced permutations ------------------------------------------------
// Copies in 16-byte units: W_Q's head blocks and W_V's head blocks (rows of
// D elements), W_O's column blocks (d elements inside each of its D rows).
__global__ __launch_bounds__(256) void merge_permute(const int32_t* __restrict__ sigma,
                                                     const u32x4* __restrict__ wq,
                                                     const u32x4* __restrict__ wv,
                                                     const u32x4* __restrict__ wo,
                                                     int D, int h_q, int h_kt, int d, int esize,
                                                     u32x4* __restrict__ wq_o,
                                                     u32x4* __restrict__ wv_o,
                                                     u32x4* __restrict__ wo_o) {
    const int g = h_q / h_kt;
    const int64_t urow = (int64_t)D * esize / 16;           // units per W_Q / W_V row
    const int64_t uhead = (int64_t)d * esize / 16;          // units per head block of W_O rows
    const int64_t nq = (int64_t)h_q * d * urow, nv = (int64_t)h_kt * d * urow;
    const int64_t no = (int64_t)D * h_q * uhead;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx < nq) {
        const int64_t row = idx / urow, u = idx - row * urow;
        const int kq = (int)(row / d), e = (int)(row - (int64_t)kq * d);
        const int src = sigma[kq / g] * g + kq % g;
        wq_o[idx] = wq[((int64_t)src * d + e) * urow + u];
    } else if (idx < nq + nv) {
        const int64_t t = idx - nq;
        const int64_t row = t / urow, u = t - row * urow;
        const int kv = (int)(row / d), e = (int)(row - (int64_t)kv * d);
        wv_o[t] = wv[((int64_t)sigma[kv] * d + e) * urow + u];
    } else if (idx < nq + nv + no) {
        const int64_t t = idx - nq - nv;
        const int64_t per_row = (int64_t)h_q * uhead;
        const int64_t row = t / per_row, rem = t - row * per_row;
        const int kq = (int)(rem / uhead);
        const int64_t u = rem - (int64_t)kq * uhead;
        const int src = sigma[kq / g] * g + kq % g;
        wo_o[t] = wo[row * per_row + (int64_t)src * uhead + u];
    }
}

}  // namespace

// ---- host side -------------------------------------------------------------------
struct MergeWs {
    f32x4* part;
    uint16_t* Cs;      // X^T X as three bf16 parts [3][D][D]
    float *F, *S, *H, *part_s, *part_h;
    double *Y, *Z, *Dl, *Pinv, *lpart;
    double2* rec;
    PairOut* po;
    MatchWs m;
    size_t bytes;
};

// K splits giving about 256 workgroups for `tiles` output tiles (K / splits a
// multiple of 16)
static int k_splits(int K, int tiles) {
    int s = (256 + tiles - 1) / tiles;
    while (s > 1 && (K % s || (K / s) % 16 || K / s < 64)) --s;
    return s;
}

static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

static MergeWs carve_merge(void* base, int64_t L, int D, int h_q, int h_kt, int d) {
    MergeWs w{};
    char* p = static_cast<char*>(base);
    size_t off = 0;
    auto take = [&](size_t bytes) -> char* {
        char* r = p ? p + off : nullptr;
        off += al256(bytes);
        return r;
    };
    const int nt = n_tiles(D), ns = n_splits(L, D);
    const size_t np = (size_t)h_kt * (h_kt - 1) / 2;
    w.part = reinterpret_cast<f32x4*>(take((size_t)ns * nt * 8 * 32 * 64 * sizeof(f32x4)));
    w.Cs = reinterpret_cast<uint16_t*>(take((size_t)3 * D * D * 2));
    w.F = reinterpret_cast<float*>(take((size_t)(h_q + h_kt) * d * D * 4));
    w.S = reinterpret_cast<float*>(take((size_t)h_kt * d * d * 4));
    w.H = reinterpret_cast<float*>(take((size_t)h_kt * d * h_kt * d * 4));
    {
        const int tq = ((d + 63) / 64) * ((d + 63) / 64), hk = h_kt * d;
        const int th = ((hk + 63) / 64) * ((hk + 63) / 64);
        w.part_s = reinterpret_cast<float*>(take((size_t)h_q * k_splits(D, h_q * tq) * d * d * 4));
        w.part_h = reinterpret_cast<float*>(take((size_t)k_splits(D, th) * hk * hk * 4));
    }
    w.Y = reinterpret_cast<double*>(take(np * d * d * 8));
    w.Z = reinterpret_cast<double*>(take(np * d * d * 8));
    w.Dl = reinterpret_cast<double*>(take(np * d * d * 8));
    w.Pinv = reinterpret_cast<double*>(take(np * d * d * 8));
    w.lpart = reinterpret_cast<double*>(take(np * 2 * (size_t)((d + 63) / 64) * ((d + 63) / 64) * 8));
    w.rec = reinterpret_cast<double2*>(take(np * kMaxSweeps * (d - 1) * (d / 2) * 16));
    w.po = reinterpret_cast<PairOut*>(take(np * sizeof(PairOut)));
    w.m.w = reinterpret_cast<double*>(take((size_t)h_kt * h_kt * 8));
    w.m.dp = reinterpret_cast<double*>(take(((size_t)1 << h_kt) * 8));
    w.m.ch = reinterpret_cast<int8_t*>(take((size_t)1 << h_kt));
    w.m.pairs = reinterpret_cast<int32_t*>(take((size_t)h_kt * 4));
    w.bytes = off;
    return w;
}

static size_t pair_lds(int d) {
    return (size_t)pair_matrix_words(d) * 8 + 128 * 16 + (128 + 2048) * 8 + 16 * 8 + 16;
}

static bool merge_shape_ok(int64_t L, int D, int h_q, int h_kt, int d) {
    return L >= 1 && D >= 16 && D % 16 == 0 && d >= 16 && d <= 128 && d % 16 == 0 &&
           h_kt >= 2 && h_kt % 2 == 0 && h_kt <= kMaxHeads && h_q >= h_kt && h_q % h_kt == 0 &&
           (int64_t)D * D <= ((int64_t)1 << 31);
}

static NtJob nt_job(const void* A, const float* B, float* out, int64_t lda, int64_t ldb,
                    int64_t ldo, int M, int N, int K) {
    NtJob j{};
    j.A = A;
    j.B = B;
    j.out = out;
    j.lda = lda;
    j.ldb = ldb;
    j.ldo = ldo;
    j.M = M;
    j.N = N;
    j.K = K;
    j.nsum = 1;
    j.kspl = 1;
    return j;
}

static void launch_nt(const NtJob& j, int nz, hipStream_t st) {
    dim3 grid((j.N + 63) / 64, (j.M + 63) / 64, nz);
    hipLaunchKernelGGL(nt_gemm<uint16_t>, grid, dim3(kNtThreads), 0, st, j);
}

}  // namespace saga

using namespace saga;

extern "C" size_t saga_key_merge_workspace_size(int64_t L, int D, int h_q, int h_kt, int d) {
    if (!merge_shape_ok(L, D, h_q, h_kt, d)) return 0;
    return carve_merge(nullptr, L, D, h_q, h_kt, d).bytes;
}

static saga_status key_merge_impl(const void* x, const void* wq, const void* wk, int64_t L,
                                  int D, int h_q, int h_kt, int d, int strategy, int dtype,
                                  float* merged, int32_t* sigma, double* pair_w,
                                  double* objective, float* stats, void* workspace,
                                  size_t workspace_bytes, hipStream_t st, hipEvent_t* ev,
                                  int nev) {
    if (!x || !wq || !wk || !merged || !sigma) return SAGA_ERR_INVALID_ARG;
    if (strategy < 0 || strategy > 2 || nev < 0 || nev > 5 || (nev > 0 && !ev))
        return SAGA_ERR_INVALID_ARG;
    if (L < 1 || D < 1 || d < 1 || h_q < 1 || h_kt < 2 || h_kt % 2 || h_q % h_kt)
        return SAGA_ERR_INVALID_ARG;
    if (dtype != SAGA_BF16 || !merge_shape_ok(L, D, h_q, h_kt, d)) return SAGA_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(wq) |
         reinterpret_cast<uintptr_t>(wk)) & 15)
        return SAGA_ERR_INVALID_ARG;
    const MergeWs probe = carve_merge(nullptr, L, D, h_q, h_kt, d);
    if (!workspace || workspace_bytes < probe.bytes) return SAGA_ERR_WORKSPACE;
    MergeWs w = carve_merge(workspace, L, D, h_q, h_kt, d);
    // dynamic LDS beyond 64 KiB, opted in once per device (thread-safe)
    if (allow_dynamic_lds(reinterpret_cast<const void*>(nt_bf16x3), kF3Lds) != hipSuccess ||
        allow_dynamic_lds(reinterpret_cast<const void*>(pair_loss), 8 * kPanWords * 8 + 16 * 8) !=
            hipSuccess ||
        allow_dynamic_lds(reinterpret_cast<const void*>(merge_pairs), pair_lds(128)) != hipSuccess)
        return SAGA_ERR_HIP;
    bool ok = true;
    auto mark = [&](int i) {
        if (i < nev) ok = hipEventRecord(ev[i], st) == hipSuccess && ok;
    };
    // 1. C = X^T X
    const int nt = n_tiles(D), ns = n_splits(L, D);
    const int total = nt * ns, grid = (int)round_up(total, 8);
    hipLaunchKernelGGL(syrk_partial, dim3(grid), dim3(kSyrkThreads), 0, st,
                       static_cast<const uint16_t*>(x), L, D, nt, ns, split_len(L, ns), grid,
                       w.part);
    mark(0);
    const int64_t slots = (int64_t)nt * 8 * 32 * 64;
    hipLaunchKernelGGL(syrk_reduce, dim3((unsigned)((slots + 255) / 256)), dim3(256), 0, st,
                       w.part, D, nt, ns, w.Cs);
    mark(1);
    // 2. F = [W_Q; W_K] C, then S and H
    const int g = h_q / h_kt;
    float* Fq = w.F;
    float* Fk = w.F + (int64_t)h_q * d * D;
    // F = [W_Q; W_K] C in one launch, bf16 MFMA on the three parts of C
    const int mrows = (h_q + h_kt) * d;
    hipLaunchKernelGGL(nt_bf16x3, dim3((D + kF3Tile - 1) / kF3Tile, (mrows + kF3Tile - 1) / kF3Tile),
                       dim3(kF3Threads), kF3Lds, st, static_cast<const uint16_t*>(wq),
                       static_cast<const uint16_t*>(wk), h_q * d, w.Cs, mrows, D, D, w.F);
    // S: one output per (query head, K split), summed per key head in a fixed order
    const int tq = ((d + 63) / 64) * ((d + 63) / 64);
    const int ks_s = k_splits(D, h_q * tq);
    NtJob js = nt_job(wq, Fq, w.part_s, D, D, d, d, d, D);
    js.a_zs = js.b_zs = d;
    js.o_zs = (int64_t)d * d;
    js.kspl = ks_s;
    launch_nt(js, h_q * ks_s, st);
    hipLaunchKernelGGL(sum_parts, dim3((unsigned)(((int64_t)h_kt * d * d + 255) / 256)), dim3(256),
                       0, st, w.part_s, g * ks_s, (int64_t)d * d, h_kt, w.S);
    const int hk = h_kt * d, th = ((hk + 63) / 64) * ((hk + 63) / 64);
    const int ks_h = k_splits(D, th);
    NtJob jh = nt_job(wk, Fk, w.part_h, D, D, hk, hk, hk, D);
    jh.o_zs = (int64_t)hk * hk;
    jh.kspl = ks_h;
    launch_nt(jh, ks_h, st);
    hipLaunchKernelGGL(sum_parts, dim3((unsigned)(((int64_t)hk * hk + 255) / 256)), dim3(256), 0,
                       st, w.part_h, ks_h, (int64_t)hk * hk, 1, w.H);
    if (stats) {
        ok = hipMemcpyAsync(stats, w.S, (size_t)h_kt * d * d * 4, hipMemcpyDeviceToDevice,
                            st) == hipSuccess && ok;
        ok = hipMemcpyAsync(stats + (size_t)h_kt * d * d, w.H, (size_t)h_kt * d * h_kt * d * 4,
                            hipMemcpyDeviceToDevice, st) == hipSuccess && ok;
    }
    mark(2);
    // 3. pairs
    PairArgs pa{w.S, w.H, w.Y, w.Z, w.Dl, w.Pinv, w.lpart, w.rec, w.po, h_kt, d, strategy};
    const int npairs = h_kt * (h_kt - 1) / 2;
    const int t2 = ((d + 63) / 64) * ((d + 63) / 64);
    hipLaunchKernelGGL(merge_pairs, dim3(npairs), dim3(kPairThreads), pair_lds(d), st, pa);
    hipLaunchKernelGGL(pair_yz, dim3(npairs, t2), dim3(kPairThreads), 4 * kPanWords * 8, st, pa);
    hipLaunchKernelGGL(pair_loss, dim3(npairs, 2 * t2), dim3(kPairThreads),
                       8 * kPanWords * 8 + 16 * 8, st, pa);
    mark(3);
    // 4. matching, 5. merged projections
    hipLaunchKernelGGL(match_weights, dim3(1), dim3(256), 0, st, w.po, w.lpart, t2, h_kt, strategy,
                       w.m);
    if (strategy != 2) {
        const unsigned mb = (unsigned)((((int64_t)1 << h_kt) + 255) / 256);
        for (int k = 1; k <= h_kt / 2; ++k)
            hipLaunchKernelGGL(match_layer, dim3(mb), dim3(256), 0, st, h_kt, 2 * k, w.m);
    }
    hipLaunchKernelGGL(match_finish, dim3(1), dim3(256), 0, st, w.po, h_kt, strategy, w.m, sigma,
                       pair_w, objective);
    hipLaunchKernelGGL(merge_apply, dim3((D + 255) / 256, d, h_kt / 2), dim3(256), 0, st,
                       static_cast<const uint16_t*>(wk), w.Y, w.Z, w.m.pairs, h_kt, d, D, merged);
    mark(4);
    return hipGetLastError() == hipSuccess && ok ? SAGA_OK : SAGA_ERR_HIP;
}

extern "C" saga_status saga_key_merge(const void* x, const void* wq, const void* wk, int64_t L,
                                      int D, int h_q, int h_kt, int d,
                                      saga_merge_strategy strategy, saga_dtype dtype,
                                      float* merged_k, int32_t* sigma, double* pair_w,
                                      double* objective, float* stats, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    return key_merge_impl(x, wq, wk, L, D, h_q, h_kt, d, (int)strategy, (int)dtype, merged_k,
                          sigma, pair_w, objective, stats, workspace, workspace_bytes, stream,
                          nullptr, 0);
}

extern "C" saga_status saga_key_merge_timed(const void* x, const void* wq, const void* wk,
                                            int64_t L, int D, int h_q, int h_kt, int d,
                                            saga_merge_strategy strategy, saga_dtype dtype,
                                            float* merged_k,
                                            int32_t* sigma, double* pair_w, double* objective,
                                            float* stats, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream,
                                            hipEvent_t* events, int n_events) {
    return key_merge_impl(x, wq, wk, L, D, h_q, h_kt, d, (int)strategy, (int)dtype, merged_k,
                          sigma, pair_w, objective, stats, workspace, workspace_bytes, stream,
                          events, n_events);
}

extern "C" saga_status saga_merge_permute(const int32_t* sigma, const void* wq, const void* wv,
                                          const void* wo, int D, int h_q, int h_kt, int d,
                                          saga_dtype dtype, void* wq_out, void* wv_out,
                                          void* wo_out,
                                          hipStream_t stream) {
    if (!sigma || !wq || !wv || !wo || !wq_out || !wv_out || !wo_out) return SAGA_ERR_INVALID_ARG;
    if (D < 1 || d < 1 || h_q < 1 || h_kt < 1 || h_q % h_kt) return SAGA_ERR_INVALID_ARG;
    if (dtype != SAGA_BF16 && dtype != SAGA_F32) return SAGA_ERR_INVALID_ARG;
    const int esize = dtype == SAGA_BF16 ? 2 : 4;
    if (((int64_t)D * esize) % 16 || ((int64_t)d * esize) % 16) return SAGA_ERR_UNSUPPORTED;
    const uintptr_t al = reinterpret_cast<uintptr_t>(wq) | reinterpret_cast<uintptr_t>(wv) |
                         reinterpret_cast<uintptr_t>(wo) | reinterpret_cast<uintptr_t>(wq_out) |
                         reinterpret_cast<uintptr_t>(wv_out) | reinterpret_cast<uintptr_t>(wo_out);
    if (al & 15) return SAGA_ERR_INVALID_ARG;
    const int64_t units = ((int64_t)h_q * d * D * 2 + (int64_t)h_kt * d * D) * esize / 16;
    hipLaunchKernelGGL(merge_permute, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream,
                       sigma, static_cast<const u32x4*>(wq), static_cast<const u32x4*>(wv),
                       static_cast<const u32x4*>(wo), D, h_q, h_kt, d, esize,
                       static_cast<u32x4*>(wq_out), static_cast<u32x4*>(wv_out),
                       static_cast<u32x4*>(wo_out));
    return hipGetLastError() == hipSuccess ? SAGA_OK : SAGA_ERR_HIP;
}
