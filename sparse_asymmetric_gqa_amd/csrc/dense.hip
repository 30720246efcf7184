// Dense attention over every cached position: the full-attention baseline
// that top-N attention is measured against ("More Value per Key" §2.1 Eqs.
// 2-4; §3.2 and Table 5 compare GQA and SAGA with and without top-N).
//
// One fused pass per (b, key head, chunk of C positions) work item, one
// workgroup each:
//   1. K stream: the item's logits for the g query heads of the key head, on
//      the matrix cores (the K-scan's streaming waves), into LDS only;
//   2. per head: m = largest logit of the chunk, p = exp(s - m) in place,
//      l = sum of p;
//   3. V stream: for every value head the group's query heads use (one for
//      GQA, h_v / h_k for SAGA), acc[d] = sum_t p_t V[t][d], up to 8 query
//      heads per pass over the rows. bf16: on the matrix cores, P (heads x
//      positions, as bf16 hi + lo parts, so the weights keep ~16 bits) times
//      V (positions x d); the V operand needs positions contiguous per lane,
//      so each wave stages 32-row tiles of V in LDS and reads them back with
//      the gfx950 transposing LDS read. fp32: fp32 FMAs on the vector ALUs;
//   4. the partial (m, l, acc[d]) of each head and chunk goes to the
//      workspace.
// A log-sum-exp merge over the chunks then gives out = sum acc e^(m - M) /
// sum l e^(m - M). Logits never leave the chip, so the bytes moved are the K
// and V rows once each, plus the partials (d + 2 floats per head and chunk).
#include "kstream.h"

namespace saga {

namespace {

constexpr int kDenseThreads = 64 * kWaves;
constexpr int kDenseMaxHeadsPerPass = 8;   // query heads accumulated per pass over V

// Positions per work item (the chunk's logits of 16 NHT heads stay in LDS).
// Key groups of up to 16 heads take a chunk of 1024, 512 or 256 positions:
// among those that leave at most kDenseMaxParts partials per row for the
// merge (one workgroup per row reads them), the
// longest that still gives one work item per CU, else the shortest. Longer
// items move the same bytes with less per-item set-up; short calls need
// enough items to occupy the CUs. Wider groups take 256.
constexpr int kDenseMinItems = 256;   // the CUs of an MI355X
constexpr int kDenseMaxParts = 128;

template <typename T, int DH>
constexpr bool dense_xp() { return sizeof(T) == 2; }

// LDS: logits / weights [g][C] floats, then a buffer shared by the K
// stream's transpose tiles (bf16) and the cross-wave reduction of step 3.
template <typename T, int DH>
constexpr size_t dense_aux_bytes() {
    constexpr size_t red = (size_t)kWaves * kDenseMaxHeadsPerPass * DH * sizeof(float);
    constexpr size_t xt = dense_xp<T, DH>() ? (size_t)kWaves * 16 * DH * sizeof(T) : 0;
    constexpr size_t vt = sizeof(T) == 2 ? (size_t)kWaves * 32 * 128 : 0;   // V tiles
    constexpr size_t m = red > xt ? red : xt;
    return m > vt ? m : vt;
}
// Logit rows are padded to C + 32 floats: after the softmax, a head's bf16
// weight rows (hi and lo parts, C + 32 entries each) take exactly the bytes
// of its own logit row, and rows of neighbouring heads start in different
// LDS banks.
__host__ __device__ constexpr int dense_row_stride(int C) { return C + 32; }
__host__ __device__ inline size_t dense_logit_bytes(int g, int C) {
    return (size_t)g * dense_row_stride(C) * sizeof(float);
}

// bf16 round-to-nearest-even of a finite float
__device__ inline uint32_t bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// Step 3 on the matrix cores (bf16 V). Weights are in LDS as bf16 rows
// whi / wlo = base + h * (row_bytes) [+ lo_off], positions contiguous. Wave
// `wave` takes the 32-row blocks kb = wave, wave + 4, ... of the chunk; per
// block the 4 or 8 row-coalesced 16-byte loads per lane (32 rows x DH) go
// through the wave's 4 KB LDS tile one 128-byte half-row at a time. In the
// tile, row r (128 bytes) keeps 32-byte block c at (c ^ sw(r)) * 32 with
// sw(r) = ((r >> 1) ^ (r >> 3)) & 3, so the row-wise writes and the
// transposing reads (16 lanes: 4 rows x 32 bytes) spread over the banks. The
// transposing read hands lane i of a 16-lane group element i % 4 of the
// 8-byte pieces addressed by lanes i / 4 + 4 j: with lane a + 4 j addressing
// row j, columns 4 a .. 4 a + 3 of a 16-column block, lane i receives that
// block's column i for 4 consecutive rows -- the MFMA B operand layout
// (lane l: positions 8 (l / 16) .. + 7 of column l % 16) after two reads.
template <int DH>
struct PvTile {
    static constexpr int NHALF = DH / 64;   // 128-byte halves of a bf16 row
    static constexpr int NT = DH / 16;      // 16-column output tiles
    static __device__ inline int sw(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
};


__device__ inline float wave_fmax(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

template <typename T, int DH, int NHT, int C>
__global__ __launch_bounds__(kDenseThreads) void dense_attn(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ lens, float* __restrict__ part, int h_q, int h_k, int h_v,
    int64_t S_max, int nchunk, float scale) {
    constexpr bool XP = dense_xp<T, DH>();
    using S = Streamer<T, DH, NHT, XP>;
    constexpr int NS = S::NS;
    constexpr int nst = C / S::STAGE;
    static_assert(C % S::STAGE == 0 && nst % NS == 0 && nst >= 2 * NS,
                  "a chunk must span at least two rounds of stages");
    extern __shared__ __attribute__((aligned(16))) unsigned char dense_lds[];

    const int g = h_q / h_k;
    const int item = blockIdx.x;
    const int bkh = item / nchunk;
    const int chunk = item - bkh * nchunk;
    const int b = bkh / h_k;
    const int kh = bkh - b * h_k;
    const int64_t L = clamp_len(lens[b], S_max);
    const int64_t c0 = (int64_t)chunk * C;
    if (c0 >= L) return;   // uniform: the chunk starts past the row's end
    const int n = (int)(L - c0 < C ? L - c0 : C);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int SR = dense_row_stride(C);
    float* sc = reinterpret_cast<float*>(dense_lds);   // [g][SR]
    unsigned char* aux = dense_lds + dense_logit_bytes(g, C);

    // ---- 1. logits of the chunk into LDS (rows past n: -inf, weight 0)
    {
        Item<T> it;
        it.kb = k + ((int64_t)bkh * S_max + c0) * DH;
        it.n = n;
        S sm(wave, lane, XP ? reinterpret_cast<u32x4*>(aux) + wave * (S::TILE_BYTES / 16) : nullptr);
        sm.load_q(q + (int64_t)(b * h_q + kh * g) * DH, g);
#pragma unroll
        for (int s = 0; s < NS; ++s) sm.load(s, it, s);
        auto sink = [&](int ht, int, int off, f32x4 acc) {
            const int h = ht * 16 + sm.r16;
            if (h < g) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = off + e < n ? acc[e] : -__builtin_inff();
                *reinterpret_cast<f32x4*>(&sc[h * SR + off]) = x;
            }
        };
        // loads are unconditional (rows past the chunk clamp to its last row)
#pragma unroll 1
        for (int st = 0; st < nst - NS; st += NS)
#pragma unroll
            for (int s = 0; s < NS; ++s)
                sm.consume(s, st + s, scale, sink, [&] { sm.load(s, it, st + s + NS); });
#pragma unroll
        for (int s = 0; s < NS; ++s) sm.consume(s, nst - NS + s, scale, sink, [] {});
    }
    __syncthreads();

    if constexpr (sizeof(T) == 2) {
        // ---- steps 2 and 3 on the matrix cores
        using PT = PvTile<DH>;
        constexpr int NHALF = PT::NHALF;
        constexpr int NT = PT::NT;
        constexpr int NL = 4 * NHALF;                 // 16-byte loads per lane per block
        constexpr int HPM = kDenseMaxHeadsPerPass;
        const int g_v = h_q / h_v;
        const int i0 = kh * g;                        // first query head of the key head
        const int vlo = i0 / g_v;
        const int ng = (g_v + HPM - 1) / HPM;         // head groups per value head
        const int np = ((i0 + g - 1) / g_v - vlo + 1) * ng;
        const int nkb = (n + 31) / 32;                // 32-row blocks of the chunk
        const int nkw = wave < nkb ? (nkb - wave + kWaves - 1) / kWaves : 0;   // this wave's
        const int total = np * nkw;
        const int lr = lane >> 3;                     // loads: row 8 v + lr, chunk lc of a half
        const int lc = lane & 7;
        const char* vbase = reinterpret_cast<const char*>(v + ((int64_t)b * h_v * S_max + c0) * DH);
        u32x4 raw[NL];
        // block f of this wave (pass f / nkw, block wave + 4 (f % nkw)); past
        // the last one it re-reads that one, and rows past n clamp to n - 1
        auto issue = [&](int f) {
            f = f < total ? f : total - 1;
            const int pi = f / nkw;
            const int vh = vlo + pi / ng;
            const int t0 = 32 * (wave + kWaves * (f - pi * nkw));
            const char* vb = vbase + (int64_t)vh * S_max * DH * 2;
#pragma unroll
            for (int hh = 0; hh < NHALF; ++hh)
#pragma unroll
                for (int vv = 0; vv < 4; ++vv) {
                    int r = t0 + 8 * vv + lr;
                    r = r < n ? r : n - 1;
                    raw[hh * 4 + vv] = load_stream(reinterpret_cast<const u32x4*>(
                        vb + (int64_t)r * (DH * 2) + hh * 128 + lc * 16));
                }
        };
        if (total > 0) issue(0);   // uniform over the wave

        // ---- 2. softmax statistics; the weights replace the logits in place
        // as bf16 rows hi = rne(p), lo = rne(p - hi) (hi at bytes [0, 2 SR)
        // of the head's row, lo at [2 SR, 4 SR)); a wave owns whole rows
        const int64_t rec_stride = (int64_t)nchunk * (DH + 2);   // next head's record
        float* rec0 = part + ((int64_t)(b * h_q + kh * g) * nchunk + chunk) * (DH + 2);
        constexpr int PR = C / 128;                   // position pairs per lane
        for (int u = wave; u < g; u += kWaves) {
            float* srow = sc + u * SR;
            float2 x[PR];
#pragma unroll
            for (int j = 0; j < PR; ++j) x[j] = *reinterpret_cast<const float2*>(srow + 128 * j + 2 * lane);
            float mx = -__builtin_inff();
#pragma unroll
            for (int j = 0; j < PR; ++j) mx = fmaxf(mx, fmaxf(x[j].x, x[j].y));
            mx = wave_fmax(mx);   // finite: row 0 of the chunk is live
            float l = 0.f;
            uint32_t whi[PR], wlo[PR];
#pragma unroll
            for (int j = 0; j < PR; ++j) {
                const float p0 = __expf(x[j].x - mx);
                const float p1 = __expf(x[j].y - mx);
                l += p0 + p1;
                const uint32_t h0 = bf16_rne(p0), h1 = bf16_rne(p1);
                const uint32_t l0 = bf16_rne(p0 - __uint_as_float(h0 << 16));
                const uint32_t l1 = bf16_rne(p1 - __uint_as_float(h1 << 16));
                whi[j] = h0 | (h1 << 16);
                wlo[j] = l0 | (l1 << 16);
            }
            l = wave_fsum(l);
            uint32_t* wrow = reinterpret_cast<uint32_t*>(srow);
#pragma unroll
            for (int j = 0; j < PR; ++j) {
                wrow[64 * j + lane] = whi[j];
                wrow[SR / 2 + 64 * j + lane] = wlo[j];
            }
            if (lane == 0) {
                rec0[u * rec_stride] = mx;
                rec0[u * rec_stride + 1] = l;
            }
        }
        __syncthreads();

        // ---- 3. P (heads x positions) times V (positions x d) per pass
        unsigned char* tile = aux + wave * 4096;
        float* red = reinterpret_cast<float*>(aux);   // [kWaves][HPM][DH]
        const int q4 = lane >> 4;
        const int i16 = lane & 15;
        const int ta = i16 & 3;                       // transposing read: row tj, piece ta
        const int tj = i16 >> 2;
        int f = 0;
        for (int pi = 0; pi < np; ++pi) {
            const int vh = vlo + pi / ng;
            const int ulo = (vh * g_v > i0 ? vh * g_v : i0) - i0;
            const int uhi = ((vh + 1) * g_v < i0 + g ? (vh + 1) * g_v : i0 + g) - i0;
            const int u0 = ulo + (pi % ng) * HPM;
            const int nh = uhi - u0 < HPM ? uhi - u0 : HPM;   // <= 0: an empty group
            // A operand rows: heads u0 + lane % 16 (clamped to the array; rows
            // of other heads produce outputs that are never written)
            const int hu = u0 + i16 < g - 1 ? u0 + i16 : g - 1;
            const char* wr = reinterpret_cast<const char*>(sc + hu * SR) + 16 * q4;
            f32x4 acc[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
            for (int i = 0; i < nkw; ++i, ++f) {
                const int t0 = 32 * (wave + kWaves * i);
                const u32x4 ahi = *reinterpret_cast<const u32x4*>(wr + 2 * t0);
                const u32x4 alo = *reinterpret_cast<const u32x4*>(wr + 2 * SR + 2 * t0);
#pragma unroll
                for (int hh = 0; hh < NHALF; ++hh) {
#pragma unroll
                    for (int vv = 0; vv < 4; ++vv) {
                        const int r = 8 * vv + lr;
                        *reinterpret_cast<u32x4*>(tile + r * 128 + (((lc >> 1) ^ PT::sw(r)) << 5) +
                                                  ((lc & 1) << 4)) = raw[hh * 4 + vv];
                    }
                    if (hh == NHALF - 1) issue(f + 1);   // the registers are free
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        u32x4 bop;
#pragma unroll
                        for (int hr = 0; hr < 2; ++hr) {
                            const int r = 8 * q4 + 4 * hr + tj;
                            // generic -> LDS address space (the tile is in LDS)
                            const v4s t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                (lds_v4s*)(tile + r * 128 + ((c ^ PT::sw(r)) << 5) + (ta << 3)));
                            bop[2 * hr] = (uint32_t)(uint16_t)t[0] | ((uint32_t)(uint16_t)t[1] << 16);
                            bop[2 * hr + 1] = (uint32_t)(uint16_t)t[2] | ((uint32_t)(uint16_t)t[3] << 16);
                        }
                        acc[hh * 4 + c] = Mfma<uint16_t>::step(ahi, bop, acc[hh * 4 + c]);
                        acc[hh * 4 + c] = Mfma<uint16_t>::step(alo, bop, acc[hh * 4 + c]);
                    }
                }
            }
            // lane: out[head u0 + 4 q4 + e][column 16 nt + i16] of its rows
            __syncthreads();   // every wave is done with its tile (red overlays them)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * q4 + e < HPM) red[(wave * HPM + 4 * q4 + e) * DH + 16 * nt + i16] = acc[nt][e];
            __syncthreads();
            for (int x = tid; x < nh * DH; x += kDenseThreads) {
                const int u = x / DH;
                const int c = x - u * DH;
                float sum = 0.f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) sum += red[(w * HPM + u) * DH + c];
                rec0[(u0 + u) * rec_stride + 2 + c] = sum;
            }
            __syncthreads();   // red is rewritten by the next pass's tiles
        }
    } else {
        // ---- value-row geometry of step 3. The passes are (value head, group of
        // <= HP of its query heads); each pass walks the chunk's rows in batches
        // of UNR row steps. Batches are double-buffered across passes: batch f+1
        // is requested before batch f is used, and the first batch before step 2.
        constexpr int HP = kDenseMaxHeadsPerPass;   // heads per pass (unused ones idle)
        using R = Row16<T>;
        constexpr int EPL = R::EPL;            // values per lane per row
        constexpr int LPR = DH / EPL;          // lanes per row
        constexpr int RPI = 64 / LPR;          // rows per wave instruction
        constexpr int STEP = kWaves * RPI;
        constexpr int UNR = 4;
        constexpr int BATCH = STEP * UNR;
        const int rg = lane / LPR;
        const int sub = lane - rg * LPR;
        const int first = wave * RPI + rg;
        const int g_v = h_q / h_v;
        const int i0 = kh * g;                 // first query head of the key head
        const int vlo = i0 / g_v;
        const int ng = (g_v + HP - 1) / HP;    // head groups per value head
        const int np = ((i0 + g - 1) / g_v - vlo + 1) * ng;
        const int nb = (n + BATCH - 1) / BATCH;
        const int nbt = np * nb;
        const T* vbase = v + ((int64_t)b * h_v * S_max + c0) * DH + sub * EPL;
        // rows of batch f (clamped: past the chunk, or past the last batch, the
        // loads re-read a live row and are never used)
        auto issue = [&](u32x4 (&dst)[UNR], int f) {
            f = f < nbt ? f : nbt - 1;
            const int vh = vlo + (f / nb) / ng;
            const int r0 = (f % nb) * BATCH;
            const T* vb = vbase + (int64_t)vh * S_max * DH;
    #pragma unroll
            for (int j = 0; j < UNR; ++j) {
                int r = r0 + first + j * STEP;
                r = r < n ? r : n - 1;
                dst[j] = load_stream(reinterpret_cast<const u32x4*>(vb + (int64_t)r * DH));
            }
        };
        u32x4 ra[UNR], rb[UNR];
        issue(ra, 0);

        // ---- 2. softmax statistics of the chunk, per query head
        const int64_t rec_stride = (int64_t)nchunk * (DH + 2);   // next head's record
        float* rec0 = part + ((int64_t)(b * h_q + kh * g) * nchunk + chunk) * (DH + 2);
        for (int u = wave; u < g; u += kWaves) {
            float* s = sc + u * SR;
            float mx = -__builtin_inff();
    #pragma unroll
            for (int j = 0; j < C / 64; ++j) mx = fmaxf(mx, s[lane + 64 * j]);
            mx = wave_fmax(mx);   // finite: row 0 of the chunk is live
            float l = 0.f;
    #pragma unroll
            for (int j = 0; j < C / 64; ++j) {
                const float p = __expf(s[lane + 64 * j] - mx);
                s[lane + 64 * j] = p;
                l += p;
            }
            l = wave_fsum(l);
            if (lane == 0) {
                rec0[u * rec_stride] = mx;
                rec0[u * rec_stride + 1] = l;
            }
        }
        __syncthreads();

        // ---- 3. weighted sums of the value rows
        float* red = reinterpret_cast<float*>(aux);   // [kWaves][HP][DH]
        float acc[HP][EPL];
    #pragma unroll
        for (int u = 0; u < HP; ++u)
    #pragma unroll
            for (int c = 0; c < EPL; ++c) acc[u][c] = 0.f;
        // batch f: accumulate its rows; after a pass's last batch, reduce over the
        // row groups and the waves and write the pass's partial sums
        auto use = [&](const u32x4 (&raw)[UNR], int f) {
            const int pi = f / nb;
            const int kb = f - pi * nb;
            const int vh = vlo + pi / ng;
            const int ulo = (vh * g_v > i0 ? vh * g_v : i0) - i0;
            const int uhi = ((vh + 1) * g_v < i0 + g ? (vh + 1) * g_v : i0 + g) - i0;
            const int u0 = ulo + (pi % ng) * HP;
            const int nh = uhi - u0 < HP ? uhi - u0 : HP;   // <= 0: an empty group
            const int r0 = kb * BATCH;
            // weights of the batch's rows (rows past n hold 0), all read before
            // any is used; heads past the pass's last read a valid row of the
            // logit array and accumulate sums that are never written
            float wv[UNR][HP];
    #pragma unroll
            for (int u = 0; u < HP; ++u) {
                const int hu = u0 + u < g - 1 ? u0 + u : g - 1;
                const float* pw = sc + hu * SR + r0 + first;
    #pragma unroll
                for (int j = 0; j < UNR; ++j) wv[j][u] = pw[j * STEP];
            }
    #pragma unroll
            for (int j = 0; j < UNR; ++j) {
                float fv[EPL];
                R::cvt(raw[j], fv);
    #pragma unroll
                for (int u = 0; u < HP; ++u)
    #pragma unroll
                    for (int c = 0; c < EPL; ++c) acc[u][c] += wv[j][u] * fv[c];
            }
            if (kb == nb - 1) {   // uniform: the pass is complete
    #pragma unroll
                for (int o = LPR; o < 64; o <<= 1)
    #pragma unroll
                    for (int u = 0; u < HP; ++u)
    #pragma unroll
                        for (int c = 0; c < EPL; ++c) acc[u][c] += __shfl_xor(acc[u][c], o, 64);
                if (rg == 0)
    #pragma unroll
                    for (int u = 0; u < HP; ++u)
    #pragma unroll
                        for (int c = 0; c < EPL; ++c)
                            red[(wave * HP + u) * DH + sub * EPL + c] = acc[u][c];
    #pragma unroll
                for (int u = 0; u < HP; ++u)
    #pragma unroll
                    for (int c = 0; c < EPL; ++c) acc[u][c] = 0.f;
                __syncthreads();
                for (int x = tid; x < nh * DH; x += kDenseThreads) {
                    const int u = x / DH;
                    const int c = x - u * DH;
                    float sum = 0.f;
    #pragma unroll
                    for (int w = 0; w < kWaves; ++w) sum += red[(w * HP + u) * DH + c];
                    rec0[(u0 + u) * rec_stride + 2 + c] = sum;
                }
                __syncthreads();   // red is rewritten by the next pass
            }
        };
    #pragma unroll 1
        for (int f = 0; f < nbt; f += 2) {
            issue(rb, f + 1);
            use(ra, f);
            issue(ra, f + 2);
            if (f + 1 < nbt) use(rb, f + 1);   // uniform
        }

    }
}

// out[row] = sum_s acc_s e^(m_s - M) / sum_s l_s e^(m_s - M) over the live
// chunks s of the row (every live chunk has l >= 1: its largest logit has
// weight 1); a row with no live chunk (L_b = 0) gets 0. One workgroup per
// row: kMergeGroups groups of DH threads (one per column) take every
// kMergeGroups-th chunk each, so a long row's partials are read with that
// many loads in flight per column; the groups' sums, each relative to the
// group's own largest m, are then combined in group order.
constexpr int kMergeGroups = 8;
template <int DH>
__global__ __launch_bounds__(DH * kMergeGroups) void dense_merge(
    const float* __restrict__ part, int nchunk, int C, const int32_t* __restrict__ lens,
    int64_t S_max, float* __restrict__ out, int h_q) {
    constexpr int G = kMergeGroups;
    __shared__ float s_m[G], s_den[G], s_num[G][DH];
    const int row = blockIdx.x;
    const int c = threadIdx.x % DH;
    const int grp = threadIdx.x / DH;
    const int64_t L = clamp_len(lens[row / h_q], S_max);
    const int64_t live = (L + C - 1) / C;
    const int ns = (int)(live < nchunk ? live : nchunk);
    const float* p = part + (int64_t)row * nchunk * (DH + 2);
    float m = -__builtin_inff();
#pragma unroll 4
    for (int s = grp; s < ns; s += G) m = fmaxf(m, p[s * (DH + 2)]);
    float num = 0.f, den = 0.f;
#pragma unroll 4
    for (int s = grp; s < ns; s += G) {
        const float* r = p + s * (DH + 2);
        const float f = __expf(r[0] - m);
        den += r[1] * f;
        num += r[2 + c] * f;
    }
    if (c == 0) {
        s_m[grp] = m;
        s_den[grp] = den;
    }
    s_num[grp][c] = num;
    __syncthreads();
    if (grp != 0) return;
    float M = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < G; ++j) M = fmaxf(M, s_m[j]);
    float n_ = 0.f, d_ = 0.f;
#pragma unroll
    for (int j = 0; j < G; ++j)
        if (s_m[j] > -__builtin_inff()) {   // a group with no chunk adds nothing
            const float f = __expf(s_m[j] - M);
            d_ += s_den[j] * f;
            n_ += s_num[j][c] * f;
        }
    out[(int64_t)row * DH + c] = d_ > 0.f ? n_ / d_ : 0.f;
}

template <typename T, int DH, int NHT, int C>
hipError_t go_dense(const void* q, const void* k, const void* v, const int32_t* lens, float* part,
                    int B, int h_q, int h_k, int h_v, int64_t S_max, hipStream_t st) {
    const int g = h_q / h_k;
    const int nchunk = (int)((S_max + C - 1) / C);
    const size_t lds = dense_logit_bytes(g, C) + dense_aux_bytes<T, DH>();
    static_assert(16 * NHT * C * sizeof(float) + dense_aux_bytes<T, DH>() <= 160 * 1024,
                  "logits of 16 NHT heads must fit the LDS");
    auto kern = &dense_attn<T, DH, NHT, C>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
    }
    const int64_t nwork = (int64_t)B * h_k * nchunk;
    const float scale = (float)(1.0 / __builtin_sqrt((double)DH));
    hipLaunchKernelGGL(kern, dim3((unsigned)nwork), dim3(kDenseThreads), lds, st, (const T*)q,
                       (const T*)k, (const T*)v, lens, part, h_q, h_k, h_v, S_max, nchunk, scale);
    return hipGetLastError();
}

template <typename T, int DH>
hipError_t go_dense_g(const void* q, const void* k, const void* v, const int32_t* lens,
                      float* part, int B, int h_q, int h_k, int h_v, int64_t S_max,
                      hipStream_t st) {
    const int g = h_q / h_k;
    if (g <= 16) {
        const int C = dense_chunk(B, h_k, S_max, g);
        if (C == 1024)
            return go_dense<T, DH, 1, 1024>(q, k, v, lens, part, B, h_q, h_k, h_v, S_max, st);
        if (C == 512)
            return go_dense<T, DH, 1, 512>(q, k, v, lens, part, B, h_q, h_k, h_v, S_max, st);
        return go_dense<T, DH, 1, 256>(q, k, v, lens, part, B, h_q, h_k, h_v, S_max, st);
    }
    if (g <= 32) return go_dense<T, DH, 2, 256>(q, k, v, lens, part, B, h_q, h_k, h_v, S_max, st);
    return go_dense<T, DH, 4, 256>(q, k, v, lens, part, B, h_q, h_k, h_v, S_max, st);
}

}  // namespace

int dense_chunk(int B, int h_k, int64_t S_max, int g) {
    if (g > 16) return 256;
    const int64_t rows = (int64_t)B * h_k;
    int shortest = 1024;   // when even 1024 leaves more partials than the cap
    for (int C = 1024; C >= 256; C /= 2) {
        const int64_t parts = (S_max + C - 1) / C;
        if (parts > kDenseMaxParts) break;
        if (rows * parts >= kDenseMinItems) return C;
        shortest = C;
    }
    return shortest;
}
int dense_nsplit(int B, int h_k, int64_t S_max, int g) {
    const int C = dense_chunk(B, h_k, S_max, g);
    return (int)((S_max + C - 1) / C);
}

hipError_t launch_dense_attn(const void* q, const void* k, const void* v, const int32_t* lens,
                             float* part, float* out, int B, int h_q, int h_k, int h_v, int d,
                             int64_t S_max, bool bf16, hipStream_t st) {
    hipError_t e;
    if (bf16)
        e = d == 64 ? go_dense_g<uint16_t, 64>(q, k, v, lens, part, B, h_q, h_k, h_v, S_max, st)
                    : go_dense_g<uint16_t, 128>(q, k, v, lens, part, B, h_q, h_k, h_v, S_max, st);
    else
        e = d == 64 ? go_dense_g<float, 64>(q, k, v, lens, part, B, h_q, h_k, h_v, S_max, st)
                    : go_dense_g<float, 128>(q, k, v, lens, part, B, h_q, h_k, h_v, S_max, st);
    if (e != hipSuccess) return e;
    const int g = h_q / h_k;
    const int nchunk = dense_nsplit(B, h_k, S_max, g);
    const int C = dense_chunk(B, h_k, S_max, g);
    if (d == 64)
        hipLaunchKernelGGL((dense_merge<64>), dim3((unsigned)(B * h_q)),
                           dim3(64 * kMergeGroups), 0, st, part,
                           nchunk, C, lens, S_max, out, h_q);
    else
        hipLaunchKernelGGL((dense_merge<128>), dim3((unsigned)(B * h_q)),
                           dim3(128 * kMergeGroups), 0, st, part,
                           nchunk, C, lens, S_max, out, h_q);
    return hipGetLastError();
}

}  // namespace saga
