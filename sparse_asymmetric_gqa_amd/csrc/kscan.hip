// K-scan: logits s[b, i, t] = <q[b, i], K[b, kh(i), t]> / sqrt(d) for t < L_b.
//
// Eq. 2 of "More Value per Key" (§2.1) for one decode query row (§2.2 Eq. 5);
// query head i uses key head i / (h_q / h_k) (App. B Eq. 29, §3.2).
//
// The g = h_q / h_k query heads that share a key head form the N side of a
// 16x16 matrix-core tile, the cached positions the M side, and the head
// dimension the K side, so every K row is read from HBM exactly once per call
// and reused for all g heads inside the MFMA. Loads: each lane fetches 16
// contiguous bytes of one K row per k-step, 16 rows per wave instruction,
// 64 contiguous bytes per row per instruction (full 64-byte segments).
#include "saga_internal.h"

namespace saga {
using namespace dev;

namespace {

constexpr int kWaves = 4;
constexpr int kTilesPerIter = 2;   // 16-row tiles a wave keeps in flight per iteration

// bf16: v_mfma_f32_16x16x32_bf16. Lane l supplies row (A) / column (B) l % 16
// and the 8 d-elements [32 s + 8 (l / 16), +8) of k-step s; A and B use the
// same lane -> d mapping, so the contraction covers every d exactly once.
template <int DH, int NHT, bool VST>
__global__ __launch_bounds__(256) void kscan_bf16(const uint16_t* __restrict__ q,
                                                  const uint16_t* __restrict__ k,
                                                  const int32_t* __restrict__ lens,
                                                  float* __restrict__ scores, int64_t s_stride,
                                                  int h_q, int h_k, int64_t S_max, float scale) {
    constexpr int KS = DH / 32;
    constexpr int U = kTilesPerIter;
    const int g = h_q / h_k;
    const int bkh = blockIdx.y;
    const int b = bkh / h_k;
    const int kh = bkh - b * h_k;
    const int64_t L = clamp_len(lens[b], S_max);
    const int64_t c0 = (int64_t)blockIdx.x * kScanChunk;
    if (c0 >= L) return;
    const int64_t c1 = c0 + kScanChunk < L ? c0 + kScanChunk : L;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15;
    const int grp = lane >> 4;

    bf16x8 bq[NHT][KS];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        const int n = ht * 16 + r16;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (n < g) {
                const uint16_t* src = q + ((int64_t)(b * h_q + kh * g + n) * DH + 32 * s + 8 * grp);
                bq[ht][s] = *reinterpret_cast<const bf16x8*>(src);
            } else {
                bq[ht][s] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
            }
        }
    }

    const uint16_t* kb = k + (int64_t)bkh * S_max * DH + 8 * grp;
    const int ntiles = (int)((c1 - c0 + 15) / 16);
    const int nit = (ntiles + kWaves * U - 1) / (kWaves * U);
    const int64_t last = L - 1;

    bf16x8 cur[U][KS], nxt[U][KS];
    auto load = [&](bf16x8 (&dst)[U][KS], int it) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t row = c0 + 16 * (int64_t)(wave + kWaves * (u + U * it)) + r16;
            row = row < last ? row : last;
            const uint16_t* src = kb + row * DH;
#pragma unroll
            for (int s = 0; s < KS; ++s)
                dst[u][s] = *reinterpret_cast<const bf16x8*>(src + 32 * s);
        }
    };

    load(cur, 0);
    for (int it = 0; it < nit; ++it) {
        if (it + 1 < nit) load(nxt, it + 1);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t p = c0 + 16 * (int64_t)(wave + kWaves * (u + U * it)) + 4 * grp;
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur[u][s], bq[ht][s], acc, 0, 0, 0);
                const int n = ht * 16 + r16;
                if (n < g && p < c1) {
                    float* dst = scores + (int64_t)(b * h_q + kh * g + n) * s_stride + p;
                    if (VST && p + 3 < c1) {
                        *reinterpret_cast<f32x4*>(dst) = acc * scale;
                    } else {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            if (p + v < c1) dst[v] = acc[v] * scale;
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int s = 0; s < KS; ++s) cur[u][s] = nxt[u][s];
    }
}

// fp32: v_mfma_f32_16x16x4_f32. Lane l loads float4 j4 of row l % 16 at
// d-elements [16 j4 + 4 (l / 16), +4); component c of it feeds k-step (j4, c)
// with k-index l / 16. The query operand uses the same mapping.
template <int DH, int NHT, bool VST>
__global__ __launch_bounds__(256) void kscan_f32(const float* __restrict__ q,
                                                 const float* __restrict__ k,
                                                 const int32_t* __restrict__ lens,
                                                 float* __restrict__ scores, int64_t s_stride,
                                                 int h_q, int h_k, int64_t S_max, float scale) {
    constexpr int K4 = DH / 16;
    constexpr int U = kTilesPerIter;
    const int g = h_q / h_k;
    const int bkh = blockIdx.y;
    const int b = bkh / h_k;
    const int kh = bkh - b * h_k;
    const int64_t L = clamp_len(lens[b], S_max);
    const int64_t c0 = (int64_t)blockIdx.x * kScanChunk;
    if (c0 >= L) return;
    const int64_t c1 = c0 + kScanChunk < L ? c0 + kScanChunk : L;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15;
    const int grp = lane >> 4;

    f32x4 bq[NHT][K4];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        const int n = ht * 16 + r16;
#pragma unroll
        for (int j4 = 0; j4 < K4; ++j4) {
            if (n < g)
                bq[ht][j4] = *reinterpret_cast<const f32x4*>(
                    q + (int64_t)(b * h_q + kh * g + n) * DH + 16 * j4 + 4 * grp);
            else
                bq[ht][j4] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    const float* kb = k + (int64_t)bkh * S_max * DH + 4 * grp;
    const int ntiles = (int)((c1 - c0 + 15) / 16);
    const int nit = (ntiles + kWaves * U - 1) / (kWaves * U);
    const int64_t last = L - 1;

    f32x4 cur[U][K4], nxt[U][K4];
    auto load = [&](f32x4 (&dst)[U][K4], int it) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t row = c0 + 16 * (int64_t)(wave + kWaves * (u + U * it)) + r16;
            row = row < last ? row : last;
            const float* src = kb + row * DH;
#pragma unroll
            for (int j4 = 0; j4 < K4; ++j4)
                dst[u][j4] = *reinterpret_cast<const f32x4*>(src + 16 * j4);
        }
    };

    load(cur, 0);
    for (int it = 0; it < nit; ++it) {
        if (it + 1 < nit) load(nxt, it + 1);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t p = c0 + 16 * (int64_t)(wave + kWaves * (u + U * it)) + 4 * grp;
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j4 = 0; j4 < K4; ++j4)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(cur[u][j4][c], bq[ht][j4][c],
                                                                   acc, 0, 0, 0);
                const int n = ht * 16 + r16;
                if (n < g && p < c1) {
                    float* dst = scores + (int64_t)(b * h_q + kh * g + n) * s_stride + p;
                    if (VST && p + 3 < c1) {
                        *reinterpret_cast<f32x4*>(dst) = acc * scale;
                    } else {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            if (p + v < c1) dst[v] = acc[v] * scale;
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j4 = 0; j4 < K4; ++j4) cur[u][j4] = nxt[u][j4];
    }
}

template <int DH, int NHT, bool VST>
hipError_t go(const void* q, const void* k, const int32_t* lens, float* scores,
              int64_t s_stride, int B, int h_q, int h_k, int64_t S_max, bool bf16,
              hipStream_t st) {
    dim3 grid((unsigned)((S_max + kScanChunk - 1) / kScanChunk), (unsigned)(B * h_k));
    const float scale = (float)(1.0 / __builtin_sqrt((double)DH));
    if (bf16)
        hipLaunchKernelGGL((kscan_bf16<DH, NHT, VST>), grid, dim3(256), 0, st,
                           (const uint16_t*)q, (const uint16_t*)k, lens, scores, s_stride, h_q,
                           h_k, S_max, scale);
    else
        hipLaunchKernelGGL((kscan_f32<DH, NHT, VST>), grid, dim3(256), 0, st,
                           (const float*)q, (const float*)k, lens, scores, s_stride, h_q, h_k,
                           S_max, scale);
    return hipGetLastError();
}

template <int DH, bool VST>
hipError_t by_nht(int nht, const void* q, const void* k, const int32_t* lens, float* scores,
                  int64_t s_stride, int B, int h_q, int h_k, int64_t S_max, bool bf16,
                  hipStream_t st) {
    switch (nht) {
        case 1: return go<DH, 1, VST>(q, k, lens, scores, s_stride, B, h_q, h_k, S_max, bf16, st);
        case 2: return go<DH, 2, VST>(q, k, lens, scores, s_stride, B, h_q, h_k, S_max, bf16, st);
        default: return go<DH, 4, VST>(q, k, lens, scores, s_stride, B, h_q, h_k, S_max, bf16, st);
    }
}

}  // namespace

hipError_t launch_kscan(const void* q, const void* k, const int32_t* lens, float* scores,
                        int64_t s_stride, int B, int h_q, int h_k, int d, int64_t S_max,
                        bool bf16, hipStream_t st) {
    const int g = h_q / h_k;
    const int nht = (g + 15) / 16;   // 1, 2 or 4 head tiles (g <= 64)
    const bool vst = (s_stride % 4 == 0) && ((reinterpret_cast<uintptr_t>(scores) & 15) == 0);
    const int nh = nht <= 1 ? 1 : (nht <= 2 ? 2 : 4);
    if (d == 64)
        return vst ? by_nht<64, true>(nh, q, k, lens, scores, s_stride, B, h_q, h_k, S_max, bf16, st)
                   : by_nht<64, false>(nh, q, k, lens, scores, s_stride, B, h_q, h_k, S_max, bf16, st);
    return vst ? by_nht<128, true>(nh, q, k, lens, scores, s_stride, B, h_q, h_k, S_max, bf16, st)
               : by_nht<128, false>(nh, q, k, lens, scores, s_stride, B, h_q, h_k, S_max, bf16, st);
}

}  // namespace saga
