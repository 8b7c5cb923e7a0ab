// Small-M Q4_0 GEMM: Y[m][n] = sum_k w[n][k] X[m][k] for 2 <= M <= 16.
//
// The batched pass that verifies speculative drafts, and 16-token prefill
// chunks ("SwarmLLM v0.2.0 ..." on aipolix.com, section "Speculation is used to
// amortize network round trips"; taozi.news, section "技术架构").  Every weight
// is read from memory and expanded from its 4-bit code exactly once for all M
// activation rows.
//
// With up to 16 activation rows this is a dense contraction, so the products
// run on the matrix cores (v_mfma_f32_16x16x32_f16): the vector ALUs only
// expand the weights, at the same cost per weight as the M = 1 kernel,
// whatever M is.  (A vector-ALU version with one v_dot2 chain per activation
// row was measured at 1.8 TB/s for M = 2 down to 0.4 TB/s for M = 16 on the
// 64-layer sweep, bound by its LDS reads.)
//
// Work split: a workgroup owns 64 weight rows (16 per wave) and one K-range of
// at most kMaxChunks chunks of 1024 columns.  It stages the activations of
// that K-range for all 16 rows once into LDS (chunk order of q4_device.h,
// zero beyond M), then streams its weight rows.  When K is split over S
// ranges each range writes a partial product to the workspace and a second
// kernel adds the S partials in a fixed order, so results are deterministic.
// S is chosen from the shape alone so that the grid has enough workgroups.
//
// Lane (g, n) = (lane / 16, lane % 16) of a wave reads block pairs g, g+4,
// g+8, g+12 of each 16-pair chunk of weight row n (4 lanes cover 144
// contiguous bytes).  Each pair expands to 8 chunks of 8 halves ((code - 8) * d
// rounded once to f16: error <= 2^-11 of each weight, inside the 1e-3 bound);
// chunk c of lane (g, n) is the B operand for weight row n, and the A operand
// of lane (g, m) is chunk c of the same pair of activation row m.  The 32 k of
// one MFMA are 8 k from each of 4 pairs; both operands use the same
// assignment, so the sum is the full dot product.  Rows beyond N and pairs
// beyond K/64 read clamped in-range addresses and meet zero activations.
#include "q4_device.h"
#include "q4_launch.h"

#include <algorithm>

namespace q4 {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) float g_f32;

constexpr int kSmThreads = 256;        // 4 waves x 16 rows
constexpr int kSmRows = 64;
constexpr int kPC = 16;                // pairs per chunk (1024 columns)
constexpr int kPairsPerLane = 4;       // pairs g, g+4, g+8, g+12 of a chunk
constexpr int kChunkU4 = kPC * 8 * 16; // u4 entries of one chunk: [pair][chunk][m]
constexpr int kMaxChunks = 2;          // chunks per K-range (64 KiB of activations)

// Activation chunks of pairs [p0, p0 + npairs) of rows 0..15 into
// buf[(pl * 8 + c) * 16 + m]; rows >= m_real and pairs >= np are zero.
__device__ void stage_range(const uint16_t* __restrict__ x, int64_t k, int m_real, int np, int p0,
                            int npairs, u4* __restrict__ buf) {
    for (int it = threadIdx.x; it < 16 * 2 * npairs; it += kSmThreads) {
        const int mm = it & 15;
        const int b = it >> 4;  // block within the range
        const int p = p0 + (b >> 1);
        uint32_t v[16];
        if (mm < m_real && p < np) {
            const g_u4* src = (const g_u4*)(x + (int64_t)mm * k + 32 * (int64_t)(2 * p0 + b));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u4 t = src[i];
                v[4 * i + 0] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = 0u;
        }
        auto xe = [&](int j) -> uint32_t { return (v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu; };
        auto put = [&](int half) {
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                int pos[4];
                chunk_positions(4 * half + cc, pos);
                const int off = 32 * half;
                const int a = pos[0] - off, bb = pos[1] - off, c = pos[2] - off, e = pos[3] - off;
                u4 ent;
                ent.x = xe(a) | (xe(c) << 16);
                ent.y = xe(a + 16) | (xe(c + 16) << 16);
                ent.z = xe(bb) | (xe(e) << 16);
                ent.w = xe(bb + 16) | (xe(e + 16) << 16);
                buf[((b >> 1) * 8 + 4 * half + cc) * 16 + mm] = ent;
            }
        };
        if (b & 1) put(1); else put(0);
    }
}

struct SmArgs {
    const uint8_t* w;
    const uint16_t* x;
    float* out;   // y (splits == 1) or the partials [split][m][n]
    int64_t n;
    int k;
    int m;
    int splits;
    int cps;      // chunks per split
};

__global__ void __launch_bounds__(kSmThreads) k_smallm(SmArgs a) {
    extern __shared__ u4 xbuf[];
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int wave = threadIdx.x >> 6;
    const int np = a.k >> 6;
    const int64_t rb = (int64_t)np * kPairBytes;
    const int split = blockIdx.x % a.splits;
    const int64_t tile = blockIdx.x / a.splits;
    const int c0 = split * a.cps;
    const int nchunks = (np + kPC - 1) / kPC;
    const int c1 = min(c0 + a.cps, nchunks);

    const int64_t row = tile * kSmRows + 16 * wave + l16;  // weight row of this lane
    const uint8_t* wrow = a.w + min(row, a.n - 1) * rb;

    uint32_t A[kPairsPerLane][9], B[kPairsPerLane][9];
    auto load_chunk = [&](int ch, uint32_t (&D)[kPairsPerLane][9]) {
#pragma unroll
        for (int jj = 0; jj < kPairsPerLane; ++jj) {
            const int p = min(ch * kPC + g + 4 * jj, np - 1);
            load_pair(wrow + (int64_t)p * kPairBytes, D[jj]);
        }
    };
    f4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
    auto mma_chunk = [&](int ch, const uint32_t (&D)[kPairsPerLane][9]) {
        const u4* xc = xbuf + (ch - c0) * kChunkU4;
#pragma unroll
        for (int jj = 0; jj < kPairsPerLane; ++jj) {
            const int pl = g + 4 * jj;
            const _Float16 d0 = as_h2(D[jj][0]).x, d1 = as_h2(D[jj][4]).y;
            const h2 s0 = {d0, d0}, s1 = {d1, d1};
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t code = (c == 0) ? realign_block0(D[jj][0], D[jj][4]) : D[jj][c < 4 ? c : c + 1];
                const Codes4 q = expand(code);
                const h2 s = c < 4 ? s0 : s1;
                u4 bw;
                bw.x = as_u32(q.q0 * s);
                bw.y = as_u32(q.q1 * s);
                bw.z = as_u32(q.q2 * s);
                bw.w = as_u32(q.q3 * s);
                const u4 ax = xc[(pl * 8 + c) * 16 + l16];
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, ax),
                                                             __builtin_bit_cast(h8, bw), acc, 0, 0, 0);
            }
        }
    };

    load_chunk(c0, A);  // weight loads first: they do not depend on the staged activations
    stage_range(a.x, a.k, a.m, np, c0 * kPC, (c1 - c0) * kPC, xbuf);
    __syncthreads();
    for (int ch = c0; ch < c1; ch += 2) {
        if (ch + 1 < c1) load_chunk(ch + 1, B);
        mma_chunk(ch, A);
        if (ch + 1 >= c1) break;
        if (ch + 2 < c1) load_chunk(ch + 2, A);
        mma_chunk(ch + 1, B);
    }

    // D layout of the 16x16 product: lane (g, l16), element r -> activation row 4g + r, weight row l16
    if (row < a.n) {
        float* out = a.out + (int64_t)split * a.m * a.n;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int mm = 4 * g + r;
            if (mm < a.m) ((g_f32*)out)[(int64_t)mm * a.n + row] = acc[r];
        }
    }
}

// y[i] = sum over s of part[s][i], s in increasing order.
__global__ void __launch_bounds__(256) k_sum_splits(const float* __restrict__ part, float* __restrict__ y,
                                                    int64_t count, int splits) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
        float v = part[i];
        for (int s = 1; s < splits; ++s) v += part[(int64_t)s * count + i];
        y[i] = v;
    }
}

}  // namespace

// Split of K for a shape: enough workgroups to cover the device twice over,
// at most kMaxChunks chunks of activations per workgroup.  Depends on the
// shape only, so the workspace size is known before any launch.
void smallm_split(int64_t n, int64_t k, int* splits, int* cps) {
    const int64_t tiles = (n + kSmRows - 1) / kSmRows;
    const int nchunks = (int)(((k / 64) + kPC - 1) / kPC);
    int s = (int)std::min<int64_t>(nchunks, std::max<int64_t>(1, (512 + tiles - 1) / tiles));
    int c = (nchunks + s - 1) / s;
    if (c > kMaxChunks) {
        c = kMaxChunks;
        s = (nchunks + c - 1) / c;
    }
    s = (nchunks + c - 1) / c;
    *splits = s;
    *cps = c;
}

size_t smallm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    int s, c;
    smallm_split(n, k, &s, &c);
    return s > 1 ? (size_t)s * (size_t)m * (size_t)n * sizeof(float) : 0;
}

hipError_t launch_gemm_smallm(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                              int64_t k, float* workspace, hipStream_t s) {
    int splits, cps;
    smallm_split(n, k, &splits, &cps);
    SmArgs a;
    a.w = w;
    a.x = x;
    a.out = splits > 1 ? workspace : y;
    a.n = n;
    a.k = (int)k;
    a.m = (int)m;
    a.splits = splits;
    a.cps = cps;
    const int64_t tiles = (n + kSmRows - 1) / kSmRows;
    const size_t lds = (size_t)cps * kChunkU4 * sizeof(u4);
    hipLaunchKernelGGL(k_smallm, dim3((unsigned)(tiles * splits)), dim3(kSmThreads), lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const int64_t count = m * n;
    const int grid = (int)std::min<int64_t>((count + 255) / 256, (int64_t)device_cu_count() * 8);
    hipLaunchKernelGGL(k_sum_splits, dim3(grid), dim3(256), 0, s, workspace, y, count, splits);
    return hipGetLastError();
}

}  // namespace q4
