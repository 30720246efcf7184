/*
 * Seeded synthetic inputs for single-token decode attention under SAGA.
 *
 * This file creates inputs only. It holds none of the attention arithmetic
 * (no dot products, no selection, no softmax), so the CPU oracle and the HIP
 * path can both consume what it writes without sharing any of the method.
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used counter-style: draw n
 * of stream (seed, s) is mix64(base(seed, s) + (n + 1) * GAMMA), so any
 * element can be produced independently of the others and the result does
 * not depend on the thread count.
 * Normals: Box-Muller (1958) on two uniforms in (0, 1], in fp64.
 * Storage: fp64 -> fp32 round-to-nearest-even (the C cast), then for bf16
 * fp32 -> bf16 round-to-nearest-even on the bit pattern.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint64_t stream) {
    return mix64(mix64(seed) ^ ((stream + 1) * GAMMA));
}

static inline uint64_t draw(uint64_t base, uint64_t n) {
    return mix64(base + (n + 1) * GAMMA);
}

/* uniform in (0, 1] with 53 random bits */
static inline double uniform01(uint64_t base, uint64_t n) {
    return ((double)(draw(base, n) >> 11) + 1.0) * (1.0 / 9007199254740992.0);
}

static inline double normal(uint64_t base, uint64_t n) {
    uint64_t p = n >> 1;
    double u1 = uniform01(base, 2 * p);
    double u2 = uniform01(base, 2 * p + 1);
    double r = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    return (n & 1) ? r * sin(th) : r * cos(th);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Raw 64-bit draws of stream (seed, stream) at counters [offset, offset+count). */
void synth_draws(uint64_t seed, uint64_t stream, uint64_t offset, int64_t count,
                 uint64_t* out) {
    uint64_t base = stream_base(seed, stream);
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < count; ++n) out[n] = draw(base, offset + (uint64_t)n);
}

/*
 * Fill a [rows][d] tensor with N(0,1) draws of stream (seed, stream): element
 * (r, c) is normal number r*d + c. If row_scale is not NULL, row r is
 * multiplied by row_scale[r] in fp64 before rounding. dtype 0 writes float32,
 * dtype 1 writes bf16 bit patterns (uint16).
 */
void synth_fill_normal(uint64_t seed, uint64_t stream, int64_t rows, int d,
                       const double* row_scale, int dtype, void* out) {
    uint64_t base = stream_base(seed, stream);
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double sc = row_scale ? row_scale[r] : 1.0;
        for (int c = 0; c < d; ++c) {
            uint64_t n = (uint64_t)r * (uint64_t)d + (uint64_t)c;
            float f = (float)(normal(base, n) * sc);
            if (dtype == 0)
                ((float*)out)[n] = f;
            else
                ((uint16_t*)out)[n] = f32_to_bf16_rne(f);
        }
    }
}

/*
 * Heavy-hitter rows: for every (b, kh) pick `count[b]` distinct positions
 * uniformly from [0, lens[b]) by a partial Fisher-Yates shuffle driven by
 * stream (seed, stream) at counters ((b*h + kh) << 32) + j, and set
 * row_scale[(b*h + kh)*S_max + t] = factor for them (row_scale must hold 1.0
 * elsewhere on entry).
 */
int synth_heavy_rows(uint64_t seed, uint64_t stream, int B, int h, int64_t S_max,
                     const int32_t* lens, const int32_t* count, double factor,
                     double* row_scale) {
    uint64_t base = stream_base(seed, stream);
    int bad = 0;
    #pragma omp parallel for schedule(static) collapse(2) reduction(|:bad)
    for (int b = 0; b < B; ++b) {
        for (int kh = 0; kh < h; ++kh) {
            int64_t L = lens[b];
            int64_t H = count[b];
            if (L < 0 || L > S_max || H < 0 || H > L) { bad = 1; continue; }
            int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)(L > 0 ? L : 1));
            if (!perm) { bad = 1; continue; }
            for (int64_t t = 0; t < L; ++t) perm[t] = (int32_t)t;
            uint64_t ctr = ((uint64_t)(b * h + kh)) << 32;
            for (int64_t j = 0; j < H; ++j) {
                uint64_t span = (uint64_t)(L - j);
                int64_t pick = j + (int64_t)(draw(base, ctr + (uint64_t)j) % span);
                int32_t tmp = perm[j]; perm[j] = perm[pick]; perm[pick] = tmp;
                row_scale[((int64_t)b * h + kh) * S_max + perm[j]] = factor;
            }
            free(perm);
        }
    }
    return bad ? -1 : 0;
}

/* Lengths uniform in [lo, hi] inclusive, one per batch row, from stream (seed, stream). */
void synth_lengths(uint64_t seed, uint64_t stream, int B, int32_t lo, int32_t hi,
                   int32_t* lens) {
    uint64_t base = stream_base(seed, stream);
    uint64_t span = (uint64_t)(hi - lo) + 1;
    for (int b = 0; b < B; ++b) lens[b] = lo + (int32_t)(draw(base, (uint64_t)b) % span);
}
