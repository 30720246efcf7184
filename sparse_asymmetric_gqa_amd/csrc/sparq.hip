// SparQ-style approximate scoring on the SAGA key heads ("SparQ Attention:
// Bandwidth-Efficient LLM Inference", Step 1 with its GQA modification),
// feeding the top-M candidate lists of the exact path's selector.
//
// sparq_prep, one wave per (b, key head):
//   u[c] = sum over the key head's g query heads of |q[c]| (fp32, heads in
//   order); the r dims of largest u (equal sums: lower dim first), ascending,
//   -1 padded to RP = round_up(r, 16); per query head the inverse temperature
//   1 / tau = sqrt(|q|_1 / (d |q on dims|_1)), 0 when the head has no mass on
//   the dims (its approximate scores are then all 0); qm = q / tau on the
//   dims and 0 elsewhere (used by the selector to rescore kept rows); and the
//   scan's matrix-core operand per 16-dim slice and lane.
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

namespace saga {
using namespace dev;

namespace {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline float elem_f(const uint16_t* p, int64_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
}
__device__ inline float elem_f(const float* p, int64_t i) { return p[i]; }

// ---- Step 1 set-up -----------------------------------------------------------------
// Query operand of the scan for slice kt and lane l: element e is the query of
// head l % 16 at dim dims[16 kt + 4 (l / 16) + e] (0 for heads >= g and pad dims).
template <typename T> struct SqOp;
template <> struct SqOp<uint16_t> { using Q = u32x2; };
template <> struct SqOp<float> { using Q = u32x4; };

template <typename T, int DH>
__global__ __launch_bounds__(64) void sparq_prep(const T* __restrict__ q, int h_q, int h_k, int r,
                                                 int RP, int32_t* __restrict__ dims,
                                                 typename SqOp<T>::Q* __restrict__ qop,
                                                 float* __restrict__ inv_tau,
                                                 float* __restrict__ qm,
                                                 int32_t* __restrict__ dims_out) {
    constexpr int NH = DH / 64;   // dims per lane
    __shared__ float us[DH];
    __shared__ int32_t sd[DH];
    const int bkh = blockIdx.x;
    const int b = bkh / h_k, kh = bkh - (bkh / h_k) * h_k;
    const int g = h_q / h_k;
    const int lane = threadIdx.x;
    const T* qg = q + (int64_t)(b * h_q + kh * g) * DH;
    float u[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        float s = 0.f;
        for (int j = 0; j < g; ++j) s += fabsf(elem_f(qg, (int64_t)j * DH + lane + 64 * h));
        u[h] = s;
        us[lane + 64 * h] = s;
    }
    __syncthreads();
    // rank of dim c: dims with a larger sum, or an equal sum and a lower index
    bool keep[NH];
    uint64_t bal[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int c = lane + 64 * h;
        int rank = 0;
        for (int c2 = 0; c2 < DH; ++c2) {
            const float v = us[c2];
            rank += (v > u[h] || (v == u[h] && c2 < c)) ? 1 : 0;
        }
        keep[h] = rank < r;
        bal[h] = ballot(keep[h]);
    }
    for (int e = r + lane; e < RP; e += 64) sd[e] = -1;
    int before = 0;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int c = lane + 64 * h;
        if (keep[h]) {
            const int at = before + (int)lanes_below(bal[h]);
            sd[at] = c;
            if (dims_out) dims_out[(int64_t)bkh * r + at] = c;
        }
        before += __popcll(bal[h]);
    }
    __syncthreads();
    for (int e = lane; e < RP; e += 64) dims[(int64_t)bkh * RP + e] = sd[e];
    // per head: inverse temperature and the masked, scaled query
    for (int j = 0; j < g; ++j) {
        float num = 0.f, den = 0.f, qv[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            qv[h] = elem_f(qg, (int64_t)j * DH + lane + 64 * h);
            const float a = fabsf(qv[h]);
            den += a;
            num += keep[h] ? a : 0.f;
        }
        num = wave_fsum(num);
        den = wave_fsum(den);
        const float inv = num > 0.f ? sqrtf(den / ((float)DH * num)) : 0.f;
        const int i = b * h_q + kh * g + j;
        if (lane == 0) inv_tau[i] = inv;
#pragma unroll
        for (int h = 0; h < NH; ++h) qm[(int64_t)i * DH + lane + 64 * h] = keep[h] ? qv[h] * inv : 0.f;
    }
    // the scan's query operand, one slice of 16 dims at a time
    const int hd = lane & 15, G = lane >> 4;
    for (int kt = 0; kt < RP / 16; ++kt) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = sd[16 * kt + 4 * G + e];
            if (sizeof(T) == 2) {
                w[e] = (hd < g && c >= 0)
                           ? (uint32_t)reinterpret_cast<const uint16_t*>(qg)[(int64_t)hd * DH + c]
                           : 0u;
            } else {
                w[e] = (hd < g && c >= 0)
                           ? __float_as_uint(reinterpret_cast<const float*>(qg)[(int64_t)hd * DH + c])
                           : 0u;
            }
        }
        typename SqOp<T>::Q o;
        if constexpr (sizeof(T) == 2) {
            o[0] = w[0] | (w[1] << 16);
            o[1] = w[2] | (w[3] << 16);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = w[e];
        }
        qop[((int64_t)bkh * (DH / 16) + kt) * 64 + lane] = o;
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
//   keys [2][g][kScanChunk], warm [g] + cursor/used/pad, meta staging,
//   per producer wave: tile [SqTile::BYTES / 4], dims [DH]; then list staging.
template <typename T, int DH>
__host__ __device__ constexpr size_t sq_lds_words(int g) {
    return (size_t)2 * g * kScanChunk + ((g + 4 + 3) & ~3) + 5 * kMetaStage +
           (size_t)kWaves * (SqTile<T>::BYTES / 4 + DH);
}

template <typename T, int DH>
__global__ __launch_bounds__(kTopmThreads, 1) void sparq_topm(
        const T* __restrict__ kt, const int32_t* __restrict__ lens, int h_q, int h_k,
        int64_t S_max, int nchunk, int nwork, int RP, int local,
        const int32_t* __restrict__ dims, const typename SqOp<T>::Q* __restrict__ qop,
        const float* __restrict__ inv_tau, TopmOut tm, uint32_t lds_bytes) {
    using TL = SqTile<T>;
    using Q = typename SqOp<T>::Q;
    constexpr int NL = TL::NL;
    constexpr int KTM = DH / 16;
    extern __shared__ uint32_t lds[];
    const int g = h_q / h_k;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // wave-uniform
    const bool producer = wave < kWaves;
    const int KT = RP / 16;
    uint32_t* keys = lds;
    uint32_t* warm = lds + 2 * g * kScanChunk;
    uint32_t* cursor = warm + g;
    uint32_t* meta_words = lds + 2 * g * kScanChunk + ((g + 4 + 3) & ~3);
    uint32_t* wave_words = meta_words + 5 * kMetaStage;
    const uint32_t fixed_words = (uint32_t)sq_lds_words<T, DH>(g);
    char* tile = reinterpret_cast<char*>(wave_words + (producer ? wave : 0) * (TL::BYTES / 4 + DH));
    int32_t* dtab = reinterpret_cast<int32_t*>(tile + TL::BYTES);

    const int per = (nwork + gridDim.x - 1) / gridDim.x;
    const int wbeg = blockIdx.x * per;
    const int wend = wbeg + per < nwork ? wbeg + per : nwork;
    if (wbeg >= wend) return;   // uniform over the workgroup
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
        for (int n = wave - kWaves; n < g; n += kConsumers)
            if (lane == 0) warm[n] = 0u;
        if (threadIdx.x == 64 * kWaves) cursor[0] = cursor[1] = 0u;
    }

    // producer state: four sub-tiles in flight (one per 64-position step),
    // their accumulators, and the query operand of the current slice
    u32x4 sr[4][NL];
    f32x4 acc[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[s][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    Q qc{}, q0{};   // current slice's query operand; the row's first slice's
    float inv = 0.f;
    int row_loaded = -1;   // (b, kh) whose dims are in dtab
    const int hd = lane & 15;
    auto ktb = [&](const Item<T>& it) { return kt + (int64_t)it.bkh * DH * S_max; };
    auto load = [&](u32x4 (&dst)[NL], const Item<T>& it, int slice, int st) {
        const int row = lane >> 2;
        const int dim = dtab[16 * slice + row];
        const int p0 = it.c0 + 256 * st + 64 * wave;
        const T* base = ktb(it) + (int64_t)(dim < 0 ? 0 : dim) * S_max;
#pragma unroll
        for (int h = 0; h < NL; ++h) {
            const int pos = p0 + (64 * h + 16 * (lane & 3)) / (int)sizeof(T);
            // a 16-byte piece starting before L stays inside the row (S_max is a
            // multiple of the piece); pad dims and pieces past L are zero
            dst[h] = (dim >= 0 && pos < it.L) ? *reinterpret_cast<const u32x4*>(base + pos)
                                              : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto qop_of = [&](const Item<T>& it, int slice) {
        return qop[((int64_t)it.bkh * KTM + slice) * 64 + lane];
    };
    lds_barrier();

    Item<T> prev = cur;
    bool have_prev = false;
    int t = 0;
#pragma unroll 1
    while (true) {
        const bool have_cur = w < wend;
        if (!have_cur && !have_prev) break;   // uniform
        Item<T> nx = cur;
        const int wn = have_cur ? next_item<T, DH>(w + 1, 1, wend, nchunk, h_k, S_max, len_of, kt,
                                                   nx)
                                : wend;
        if (producer && have_cur) {
            if (cur.bkh != row_loaded) {
                // a new key row: its dims into this wave's table, then the first slice
                for (int c = lane; c < RP; c += 64) dtab[c] = dims[(int64_t)cur.bkh * RP + c];
                inv = hd < g ? inv_tau[cur.b * h_q + cur.kh * g + hd] : 0.f;
                q0 = qop_of(cur, 0);
                qc = q0;
#pragma unroll
                for (int s = 0; s < 4; ++s) load(sr[s], cur, 0, s);
                row_loaded = cur.bkh;
            }
            // the next item of the same row is loaded by the last slice's refills
            const bool chain = wn < wend && nx.bkh == cur.bkh;
#pragma unroll 1
            for (int sl = 0; sl < KT; ++sl) {
                const bool last = sl + 1 == KT;
                // the next slice's operand is loaded before this slice's refills, so
                // waiting for those refills covers it; a chained item of the same
                // row starts again from q0
                const Q qn = !last ? qop_of(cur, sl + 1) : (chain ? q0 : qc);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
#pragma unroll
                    for (int h = 0; h < NL; ++h) {
                        const int r16 = lane >> 2, u = 4 * h + (lane & 3);
                        *reinterpret_cast<u32x4*>(tile + r16 * TL::RB + ((u ^ TL::swz(r16)) << 4)) =
                            sr[s][h];
                    }
                    if (!last) load(sr[s], cur, sl + 1, s);
                    else if (chain) load(sr[s], nx, 0, s);
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) acc[s][nb] = SqMma<T>::block(tile, nb, lane, qc, acc[s][nb]);
                }
                qc = qn;
            }
            // keys of the chunk: position 256 s + 64 wave + 16 nb + 4 (lane / 16) + e, head lane % 16
            uint32_t* kbuf = keys + (t & 1) * g * kScanChunk;
            if (hd < g) {
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
                        *reinterpret_cast<u32x4*>(&kbuf[hd * kScanChunk + o]) = kv;
                    }
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) acc[s][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (have_prev && (!producer || !have_cur)) {
            const float share = (float)tm.N * (float)kScanChunk / (float)prev.L;
            const uint32_t M = share >= (float)(kScanChunk / 2)
                                   ? (uint32_t)kScanChunk
                                   : (uint32_t)__builtin_ceilf(1.5f * share) + 16u;
            uint32_t* kbuf = keys + ((t + 1) & 1) * g * kScanChunk;
            const int first = have_cur ? wave - kWaves : wave;
            const int step = have_cur ? kConsumers : kWaves + kConsumers;
            const int lw = local < prev.L ? local : prev.L;
#pragma unroll 1
            for (int n = first; n < g; n += step)
                extract(prev, n, M, kbuf + n * kScanChunk, warm, sink, t - 1, lane, g, h_q,
                        nchunk, tm, prev.L - lw);
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
    const uint32_t used = (sink.used[0] + 1u) & ~1u;
    const u32x4* s4 = reinterpret_cast<const u32x4*>(sink.stg);
    u32x4* d4 = reinterpret_cast<u32x4*>(sink.pool);
    for (uint32_t j = threadIdx.x; j < used / 2; j += kTopmThreads) d4[j] = s4[j];
    const int nmeta = (t - 1) * g < kMetaStage ? (t - 1) * g : kMetaStage;
    for (int e = (int)threadIdx.x; e < nmeta; e += kTopmThreads)
        tm.meta[sink.meta_slot[e]] = sink.meta_stg[e];
}

template <typename T, int DH>
hipError_t go_sparq(const void* q, const void* kt, const int32_t* lens, const TopmOut& tm,
                    const SparqWs& sw, int B, int h_q, int h_k, int r, int local, int64_t S_max,
                    int32_t* dims_out, hipStream_t st) {
    const int nchunk = (int)((S_max + kScanChunk - 1) / kScanChunk);
    const int nwork = B * h_k * nchunk;
    const int RP = (int)round_up(r, 16);
    hipLaunchKernelGGL((sparq_prep<T, DH>), dim3((unsigned)(B * h_k)), dim3(64), 0, st,
                       (const T*)q, h_q, h_k, r, RP, sw.dims,
                       reinterpret_cast<typename SqOp<T>::Q*>(sw.qop), sw.inv_tau, sw.qm,
                       dims_out);
    auto kern = &sparq_topm<T, DH>;
    const size_t lds = kTopmLdsBytes;
    static_assert(sq_lds_words<T, DH>(16) * 4 + 8 * 1024 <= kTopmLdsBytes, "staging area too small");
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return hipGetLastError();
        attr_set = true;
    }
    const int grid = resident_grid(kern, kTopmThreads, lds, nwork);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kTopmThreads), lds, st, (const T*)kt, lens,
                       h_q, h_k, S_max, nchunk, nwork, RP, local, sw.dims,
                       reinterpret_cast<const typename SqOp<T>::Q*>(sw.qop), sw.inv_tau, tm,
                       (uint32_t)lds);
    return hipGetLastError();
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
