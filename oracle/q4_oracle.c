/*
 * CPU ORACLE for the Q4_0 dequantize-and-multiply hot path.
 * TEST INFRASTRUCTURE ONLY: called by the tests, by the package's smoke check
 * and by the benchmark's CPU-baseline leg, never by the product path.  It
 * shares no code, header, table or constant with the GPU library.
 *
 * What it computes follows the decode engine of "Every Device Brings a Slice:
 * How SwarmLLM Runs a 27B Model Across Browser Tabs" (originshq.com), section
 * "The Engine: ~50 WGSL Kernels Written From Scratch": the output activation is
 * the matrix-vector product of the Q4_0 weights with the input activation, the
 * 4-bit values being expanded to real weights before they are multiplied.
 * The pages name the weight format "GGUF Q4_0" (taozi.news, section
 * "支持模型与限制"; the originshq.com page, opening paragraph) but do not
 * define it.  The reading used here (listed with the other readings in the
 * design notes):
 *   - a row of K weights is K/32 blocks of 18 bytes, blocks contiguous along K;
 *   - bytes 0..1 of a block: the scale d, IEEE binary16, little-endian;
 *   - bytes 2..17: 16 code bytes; byte j holds code j in its low nibble and
 *     code j+16 in its high nibble (codes 0..15);
 *   - weight k of the block = (code_k - 8) * d.
 *
 * Definition computed (no blocking, no reassociation):
 *   y[m][n] = sum over k = 0..K-1, in increasing k, of w[n][k] * x[m][k]
 *   a[m][n] = sum over the same k of |w[n][k] * x[m][k]|
 * in IEEE binary64.  Every w[n][k] and every product is exact in binary64
 * (d has 11 significant bits, code-8 has 4, x has 11), so y differs from the
 * exact real sum only by the rounding of the additions.
 * The greedy token is the lowest index among the maxima of y.
 * Greedy verify of a speculative draft (the trunk checks the tokens a draft
 * proposed in one batched pass: aipolix.com SwarmLLM page, section
 * "Speculation is used to amortize network round trips"): the greedy token of
 * every row, and the number of leading rows whose greedy token equals the
 * draft's token for that row (the prefix ends at the first mismatch).
 * Parallelism: OpenMP over independent outputs only; each sum is sequential.
 */
#include <math.h>
#include <stdint.h>

/* IEEE 754 binary16 -> binary64, exact: sign, 5-bit exponent (bias 15),
 * 10-bit fraction; exponent 0 = subnormal (fraction * 2^-24), exponent 31 =
 * infinity (fraction 0) or NaN. */
double q4o_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return sign ? -v : v;
}

void q4o_f16_to_f64_array(const uint16_t* h, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = q4o_f16_to_f64(h[i]);
}

/* Weight k (0..31) of one 18-byte block. */
static double block_weight(const uint8_t* blk, int k) {
    uint16_t dbits = (uint16_t)(blk[0] | ((uint16_t)blk[1] << 8));
    double d = q4o_f16_to_f64(dbits);
    uint8_t byte = blk[2 + (k & 15)];
    int code = (k < 16) ? (byte & 0x0F) : (byte >> 4);
    return (double)(code - 8) * d;
}

/* The K weights of one packed row, as binary64. */
void q4o_dequant_row(const uint8_t* row, int64_t k, double* out) {
    for (int64_t i = 0; i < k; ++i) out[i] = block_weight(row + (i / 32) * 18, (int)(i % 32));
}

/*
 * y = X * W^T over the given packed rows.
 *   w_rows : nrows packed rows, each K/32*18 bytes, consecutive
 *   x      : M x K binary16 bit patterns, row-major
 *   y, a   : M x nrows binary64, row-major (a may be NULL)
 */
void q4o_gemm_rows(const uint8_t* w_rows, int64_t nrows, int64_t k,
                   const uint16_t* x, int64_t m, double* y, double* a) {
    const int64_t rb = (k / 32) * 18;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < nrows; ++n) {
        const uint8_t* row = w_rows + n * rb;
        for (int64_t mm = 0; mm < m; ++mm) {
            const uint16_t* xr = x + mm * k;
            double acc = 0.0, mag = 0.0;
            for (int64_t i = 0; i < k; ++i) {
                double p = block_weight(row + (i / 32) * 18, (int)(i % 32)) * q4o_f16_to_f64(xr[i]);
                acc += p;
                mag += fabs(p);
            }
            y[mm * nrows + n] = acc;
            if (a) a[mm * nrows + n] = mag;
        }
    }
}

/* Lowest index i with y[i] equal to the maximum of y (n >= 1, no NaN). */
int64_t q4o_argmax(const double* y, int64_t n) {
    int64_t best = 0;
    for (int64_t i = 1; i < n; ++i) {
        if (y[i] > y[best]) best = i;
    }
    return best;
}

/* Leading positions i = 0, 1, ... at which tokens[i] == draft[i]; stops at
 * the first mismatch (m >= 0). */
int64_t q4o_accepted_prefix(const int64_t* tokens, const int64_t* draft, int64_t m) {
    int64_t i = 0;
    while (i < m && tokens[i] == draft[i]) ++i;
    return i;
}
