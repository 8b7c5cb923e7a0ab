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
 * The final norm before the LM head (the host applies it to the hidden state
 * the last stage returns, then the LM head and sampling: originshq.com page,
 * section "The Architecture: Layers Distributed, Activations in Flight";
 * taozi.news, section "技术架构").  The pages name the step only; the reading
 * used here is RMS normalisation with a learned per-element gain g and a
 * small constant eps:
 *   r   = 1 / sqrt( (sum over i = 0..K-1, in increasing i, of h_i^2) / K + eps )
 *   v_i = h_i * g_i * r                       (binary64)
 *   x_i = v_i rounded to binary16, nearest, ties to even
 * and x is the activation the LM head multiplies.
 * The pages' other weight format, "GGUF Q8_0", used by the small dense Qwen3
 * models (taozi.news, section "支持模型与限制"), is named but not defined
 * either; the reading used here:
 *   - a row of K weights is K/32 blocks of 34 bytes, blocks contiguous along K;
 *   - bytes 0..1 of a block: the scale d, IEEE binary16, little-endian;
 *   - byte 2 + j (j = 0..31): code j, a two's-complement signed byte;
 *   - weight j of the block = code_j * d.
 * Its products are exact in binary64 as well (8-bit codes, 11-bit d and x).
 * The hand-off at the end of a stage's layer range (each device converts the
 * hidden state it produced to f16 and sends it to the next participant:
 * aipolix.com en-us page, section "A model can be larger than any one browser
 * can hold"; its pt-pt page, section "O modelo pode ser maior do que a
 * memória de cada dispositivo").  Read as the epilogue of the range's last
 * GEMV with the residual stream added first:
 *   h16[n] = binary16 rounding (nearest, ties to even) of r[n] + y[n]
 * with y[n] the binary64 sum above and r an optional binary32 residual.
 * Parallelism: OpenMP over independent outputs only; each sum is sequential.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>

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

/*
 * y = X * W^T over the given packed rows.
 *   w_rows : nrows packed rows, each K/32*18 bytes, consecutive
 *   x      : M x K binary16 bit patterns, row-major
 *   y, a   : M x nrows binary64, row-major (a may be NULL)
 * Each weight is decoded once and meets the M activations of its column; the
 * M sums of a row advance together, each still taken in increasing k.
 * Returns 0, or -1 when the scratch copy of x cannot be allocated.
 */
int q4o_gemm_rows(const uint8_t* w_rows, int64_t nrows, int64_t k,
                  const uint16_t* x, int64_t m, double* y, double* a) {
    const int64_t rb = (k / 32) * 18;
    /* x decoded once, column-major: xt[i * m + mm] = x[mm][i] */
    double* xt = (double*)malloc((size_t)(k * m) * sizeof(double));
    if (!xt) return -1;
    for (int64_t mm = 0; mm < m; ++mm) {
        const uint16_t* xr = x + mm * k;
        for (int64_t i = 0; i < k; ++i) xt[i * m + mm] = q4o_f16_to_f64(xr[i]);
    }
    int failed = 0;
    #pragma omp parallel
    {
        double* acc = (double*)malloc((size_t)(2 * m) * sizeof(double));
        double* mag = acc ? acc + m : NULL;
        if (!acc) {
            #pragma omp atomic write
            failed = 1;
        }
        #pragma omp for schedule(dynamic, 4)
        for (int64_t n = 0; n < nrows; ++n) {
            if (!acc) continue;
            const uint8_t* row = w_rows + n * rb;
            for (int64_t mm = 0; mm < m; ++mm) acc[mm] = mag[mm] = 0.0;
            for (int64_t i = 0; i < k; ++i) {
                const double wv = block_weight(row + (i / 32) * 18, (int)(i % 32));
                const double* xi = xt + i * m;
                for (int64_t mm = 0; mm < m; ++mm) {
                    const double p = wv * xi[mm];
                    acc[mm] += p;
                    mag[mm] += fabs(p);
                }
            }
            for (int64_t mm = 0; mm < m; ++mm) {
                y[mm * nrows + n] = acc[mm];
                if (a) a[mm * nrows + n] = mag[mm];
            }
        }
        free(acc);
    }
    free(xt);
    return failed ? -1 : 0;
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

/* binary64 -> binary16, round to nearest, ties to even (IEEE 754
 * roundTiesToEven).  The result's quantum is 2^(E-10) for |v| in the binade
 * [2^E, 2^(E+1)), E >= -14, and 2^-24 below 2^-14 (subnormals); |v| >= 65520
 * (the midpoint above the largest finite value 65504, whose last fraction bit
 * is odd) rounds to infinity; NaN gives the quiet NaN 0x7E00. */
uint16_t q4o_f64_to_f16(double v) {
    if (isnan(v)) return 0x7E00;
    const uint16_t sign = signbit(v) ? 0x8000 : 0;
    const double a = fabs(v);
    if (a >= 65520.0) return sign | 0x7C00;
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);           /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    if (E < -14) E = -14;    /* subnormals share the smallest binade's quantum */
    const double t = ldexp(a, 10 - E);  /* a in quanta: exact (power-of-two scaling) */
    double q = floor(t);
    const double rem = t - q;           /* exact */
    if (rem > 0.5 || (rem == 0.5 && fmod(q, 2.0) != 0.0)) q += 1.0;
    /* value = q * 2^(E-10), 0 <= q <= 2048 */
    if (q >= 2048.0) {  /* carried into the next binade */
        q = 1024.0;
        E += 1;
    }
    if (q < 1024.0) return sign | (uint16_t)q;  /* subnormal (only when E == -14) or zero */
    return sign | (uint16_t)(((E + 15) << 10) | ((int)q - 1024));
}

void q4o_f64_to_f16_array(const double* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = q4o_f64_to_f16(v[i]);
}

/* The final norm: h and g binary16 [K], eps >= 0; v (binary64 [K], may be
 * NULL) receives h_i g_i r, x (binary16 [K]) its rounding. */
void q4o_rms_norm(const uint16_t* h, const uint16_t* g, int64_t k, double eps, double* v, uint16_t* x) {
    double ss = 0.0;
    for (int64_t i = 0; i < k; ++i) {
        const double hi = q4o_f16_to_f64(h[i]);
        ss += hi * hi;
    }
    const double r = 1.0 / sqrt(ss / (double)k + eps);
    for (int64_t i = 0; i < k; ++i) {
        const double vi = q4o_f16_to_f64(h[i]) * q4o_f16_to_f64(g[i]) * r;
        if (v) v[i] = vi;
        x[i] = q4o_f64_to_f16(vi);
    }
}

/* The stage hand-off: out16[n] = binary16(r[n] + y[n]) for one activation x
 * (binary16 [K]) and rows w_rows [nrows]; r (binary32 [nrows]) may be NULL
 * (zero); y and a (binary64 [nrows], a may be NULL) as q4o_gemm_rows. */
int q4o_gemv_handoff(const uint8_t* w_rows, int64_t nrows, int64_t k, const uint16_t* x, const float* r,
                     uint16_t* out16, double* y, double* a) {
    if (q4o_gemm_rows(w_rows, nrows, k, x, 1, y, a)) return -1;
    for (int64_t n = 0; n < nrows; ++n) out16[n] = q4o_f64_to_f16((r ? (double)r[n] : 0.0) + y[n]);
    return 0;
}

/* Weight kk (0..31) of a Q8_0 block. */
static double q8_block_weight(const uint8_t* blk, int kk) {
    const double d = q4o_f16_to_f64((uint16_t)(blk[0] | ((uint16_t)blk[1] << 8)));
    const int code = (int)(int8_t)blk[2 + kk];
    return (double)code * d;
}

/* y[m][n] and a[m][n] as q4o_gemm_rows, for Q8_0 rows (34-byte blocks). */
void q4o_q8_gemm_rows(const uint8_t* w_rows, int64_t nrows, int64_t k,
                      const uint16_t* x, int64_t m, double* y, double* a) {
    const int64_t rb = (k / 32) * 34;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < nrows; ++n) {
        const uint8_t* row = w_rows + n * rb;
        for (int64_t mm = 0; mm < m; ++mm) {
            const uint16_t* xr = x + mm * k;
            double acc = 0.0, mag = 0.0;
            for (int64_t i = 0; i < k; ++i) {
                double p = q8_block_weight(row + (i / 32) * 34, (int)(i % 32)) * q4o_f16_to_f64(xr[i]);
                acc += p;
                mag += fabs(p);
            }
            y[mm * nrows + n] = acc;
            if (a) a[mm * nrows + n] = mag;
        }
    }
}

/* Team size of the parallel loops above (timing only; what is computed does
 * not depend on it): set, and read back. */
void q4o_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int q4o_threads(void) { return omp_get_max_threads(); }
