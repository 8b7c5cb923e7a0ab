/*
 * Seeded, counter-based input generator for the Q4_0 GEMV workloads.
 *
 * This module produces input BYTES only (packed Q4_0 weight rows and f16
 * activation vectors).  It holds none of the method's arithmetic: it never
 * decodes a block, never multiplies weights by activations.  Both the CPU
 * oracle (oracle/) and the GPU path read what this module writes; the two
 * sides share nothing else.
 *
 * Random numbers: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  The i-th output of a
 * stream with initial state s0 is mix(s0 + (i+1)*GAMMA), which makes every
 * element addressable by its index: any row of any tensor can be regenerated
 * without generating the rest.
 *
 * Tensor streams: s0 = mix(seed ^ mix((stream + 1) * GAMMA)).
 *
 * Q4_0 weights (the layout of the packed format: 32-element blocks, each an
 * f16 scale followed by 16 bytes of 4-bit codes, code j in the low nibble and
 * code j+16 in the high nibble of byte j):
 *   block g (g = row * K/32 + b) uses outputs 3g, 3g+1, 3g+2 of the stream:
 *     code bytes 0..7  = little-endian bytes of output 3g,
 *     code bytes 8..15 = little-endian bytes of output 3g+1
 *       (so every code is uniform on 0..15, independently),
 *     scale d = f16_rne(0.001 + 0.019 * u), u = (output(3g+2) >> 11) * 2^-53
 *       (so d is U[0.001, 0.02] rounded to the nearest f16),
 *     stored little-endian in bytes 0..1 of the block.
 *
 * Q8_0 weights (34-byte blocks: an f16 scale, then 32 signed code bytes):
 *   block g uses outputs 5g .. 5g+4 of the stream:
 *     code bytes 0..31 = little-endian bytes of outputs 5g .. 5g+3
 *       (every code uniform on -128..127, independently),
 *     scale d = f16_rne(0.0001 + 0.0019 * u), u = (output(5g+4) >> 11) * 2^-53
 *       (d uniform on [0.0001, 0.002], so code * d spans about +-0.25 like
 *       the Q4_0 weights), stored little-endian in bytes 0..1.
 *
 * f16 activations ~ N(0,1): element i uses the Box-Muller pair built from
 * outputs 2*(i/2) and 2*(i/2)+1:
 *     u1 = ((o0 >> 11) + 1) * 2^-53  in (0, 1]
 *     u2 =  (o1 >> 11)      * 2^-53  in [0, 1)
 *     r = sqrt(-2 ln u1), t = 2 pi u2
 *     even i -> r cos t, odd i -> r sin t, then f16_rne.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t stream_state(uint64_t seed, uint64_t stream) {
    return mix64(seed ^ mix64((stream + 1ull) * GAMMA));
}

static inline uint64_t stream_at(uint64_t s0, uint64_t i) {
    return mix64(s0 + (i + 1ull) * GAMMA);
}

/* Round a double to the nearest binary16 value, ties to even, and return its
 * bit pattern.  Written from the IEEE 754 binary16 format: 1 sign bit, 5
 * exponent bits (bias 15), 10 fraction bits; the quantum is 2^(e-10) in the
 * binade [2^e, 2^(e+1)) for e >= -14 and 2^-24 below 2^-14 (subnormals). */
uint16_t synth_f64_to_f16(double v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v)) return (uint16_t)(sign | 0x7E00u);
    if (isinf(v)) return (uint16_t)(sign | 0x7C00u);
    int e;
    (void)frexp(a, &e);              /* a = f * 2^e, f in [0.5, 1) */
    int ub = e - 1;                  /* a in [2^ub, 2^(ub+1)) */
    if (ub < -14) ub = -14;          /* subnormal range shares the 2^-24 quantum */
    double quantum = ldexp(1.0, ub - 10);
    double r = nearbyint(a / quantum) * quantum; /* exact scaling, RNE */
    if (r > 65504.0) return (uint16_t)(sign | 0x7C00u); /* 65520 and up round to inf */
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -14)) {
        return (uint16_t)(sign | (uint16_t)(r * ldexp(1.0, 24)));
    }
    (void)frexp(r, &e);
    int ex = e - 1;                  /* r in [2^ex, 2^(ex+1)) */
    uint16_t mant = (uint16_t)((r / ldexp(1.0, ex) - 1.0) * 1024.0);
    return (uint16_t)(sign | (uint16_t)((ex + 15) << 10) | mant);
}

void synth_f64_to_f16_array(const double* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = synth_f64_to_f16(v[i]);
}

uint64_t synth_u64(uint64_t seed, uint64_t stream, uint64_t index) {
    return stream_at(stream_state(seed, stream), index);
}

static void q4_0_block(uint64_t s0, uint64_t g, uint8_t* blk) {
    uint64_t c0 = stream_at(s0, 3ull * g);
    uint64_t c1 = stream_at(s0, 3ull * g + 1ull);
    uint64_t r = stream_at(s0, 3ull * g + 2ull);
    double u = (double)(r >> 11) * 0x1.0p-53;
    uint16_t d = synth_f64_to_f16(0.001 + 0.019 * u);
    blk[0] = (uint8_t)(d & 0xFFu);
    blk[1] = (uint8_t)(d >> 8);
    for (int i = 0; i < 8; ++i) {
        blk[2 + i] = (uint8_t)(c0 >> (8 * i));
        blk[10 + i] = (uint8_t)(c1 >> (8 * i));
    }
}

/* Rows [row_begin, row_begin + row_count) of a Q4_0 matrix with K columns
 * (K % 32 == 0), written densely into out (row_count * K/32 * 18 bytes). */
void synth_q4_0_rows(uint64_t seed, uint64_t stream, int64_t k,
                     int64_t row_begin, int64_t row_count, uint8_t* out) {
    const uint64_t s0 = stream_state(seed, stream);
    const int64_t bpr = k / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < row_count; ++r) {
        for (int64_t b = 0; b < bpr; ++b) {
            uint64_t g = (uint64_t)((row_begin + r) * bpr + b);
            q4_0_block(s0, g, out + (r * bpr + b) * 18);
        }
    }
}

static void q8_0_block(uint64_t s0, uint64_t g, uint8_t* blk) {
    for (int w = 0; w < 4; ++w) {
        const uint64_t o = stream_at(s0, 5 * g + (uint64_t)w);
        for (int i = 0; i < 8; ++i) blk[2 + 8 * w + i] = (uint8_t)(o >> (8 * i));
    }
    const double u = (double)(stream_at(s0, 5 * g + 4) >> 11) * 0x1.0p-53;
    const uint16_t d = synth_f64_to_f16(0.0001 + 0.0019 * u);
    blk[0] = (uint8_t)(d & 0xFF);
    blk[1] = (uint8_t)(d >> 8);
}

/* Rows [row_begin, row_begin + row_count) of a K-column Q8_0 matrix. */
void synth_q8_0_rows(uint64_t seed, uint64_t stream, int64_t k,
                     int64_t row_begin, int64_t row_count, uint8_t* out) {
    const uint64_t s0 = stream_state(seed, stream);
    const int64_t bpr = k / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < row_count; ++r) {
        for (int64_t b = 0; b < bpr; ++b) {
            uint64_t g = (uint64_t)((row_begin + r) * bpr + b);
            q8_0_block(s0, g, out + (r * bpr + b) * 34);
        }
    }
}

/* Any subset of rows: rows[i] of the matrix goes to out + i * K/32 * 18. */
void synth_q4_0_row_list(uint64_t seed, uint64_t stream, int64_t k,
                         const int64_t* rows, int64_t nrows, uint8_t* out) {
    const uint64_t s0 = stream_state(seed, stream);
    const int64_t bpr = k / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        for (int64_t b = 0; b < bpr; ++b) {
            uint64_t g = (uint64_t)(rows[i] * bpr + b);
            q4_0_block(s0, g, out + (i * bpr + b) * 18);
        }
    }
}

/* Elements [begin, begin + count) of an f16 N(0,1) stream. */
void synth_f16_normal(uint64_t seed, uint64_t stream, int64_t begin,
                      int64_t count, uint16_t* out) {
    const uint64_t s0 = stream_state(seed, stream);
    const double two_pi = 6.283185307179586476925286766559;
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        uint64_t i = (uint64_t)(begin + t);
        uint64_t p = i & ~1ull;
        uint64_t o0 = stream_at(s0, p);
        uint64_t o1 = stream_at(s0, p + 1ull);
        double u1 = (double)((o0 >> 11) + 1ull) * 0x1.0p-53;
        double u2 = (double)(o1 >> 11) * 0x1.0p-53;
        double r = sqrt(-2.0 * log(u1));
        double z = (i & 1ull) ? r * sin(two_pi * u2) : r * cos(two_pi * u2);
        out[t] = synth_f64_to_f16(z);
    }
}
