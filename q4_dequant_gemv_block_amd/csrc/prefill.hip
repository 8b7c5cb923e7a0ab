// Prefill Q4_0 GEMM on the matrix cores: Y[m][n] = sum_k w[n][k] X[m][k].
//
// Prompt processing multiplies every weight by many token rows at once; the
// pages call their prefill GEMM young and measure it far below decode
// (taozi.news, section "基准成绩"; originshq.com page, section "The Engine:
// ~50 WGSL Kernels Written From Scratch").  With M in the hundreds this is a
// real dense contraction, so the weights are expanded on chip and fed to the
// gfx950 matrix cores.
//
// Tiling: a workgroup of 4 waves owns a 128 (M) x 128 (N) output tile; wave
// (wm, wn) owns the 64 x 64 quarter at (64 wm, 64 wn) as 2 x 2 tiles of
// v_mfma_f32_32x32x16_f16 with f32 accumulators.  K advances 64 columns (one
// Q4_0 block pair per weight row) per step:
//   * threads 0..127 each expand one weight row's pair: exact (code - 8) f16
//     pairs (v_and_or_b32 + v_pk_add_f16), times the block scale d in f16
//     (one rounding: relative error <= 2^-11, inside the 1e-3 bound), written
//     to LDS as 8 chunks of 8 halves;
//   * threads 128..255 copy one activation row's 64 halves into the same chunk
//     order (q4_device.h), so chunk c of an activation row meets chunk c of a
//     weight row: the k order inside a pair is permuted identically on both
//     sides and each chunk is exactly one 8-half MFMA operand.
// Rows past M or N are zero in LDS and never stored.  Both tiles are double
// buffered: the next step's global loads are issued before the current
// step's matrix work.
// Grid order is XCD-aware: workgroup b runs on XCD b % 8, and all M-tiles of
// one N-tile are given to consecutive workgroups of the same XCD, so a weight
// tile is fetched from HBM once and served from that XCD's L2 to the others.
#include "q4_device.h"
#include "q4_launch.h"

#include <algorithm>

namespace q4 {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) float g_f32;

constexpr int kPfThreads = 256;
constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kRowBytes = 8 * 16 + 16;  // 8 chunks + 16 bytes of padding (bank stagger)
constexpr int kTileBytes = 128 * kRowBytes;
constexpr int kXcd = 8;

struct PfArgs {
    const uint8_t* w;
    const uint16_t* x;
    float* y;
    int64_t m, n;
    int k;
    int mt, nt;  // tiles along M and N
};

// One weight row's pair, expanded and scaled, as the 8 chunks of the pair.
__device__ __forceinline__ void expand_pair_scaled(const uint32_t (&D)[9], u4 (&out)[8]) {
    const _Float16 d0 = as_h2(D[0]).x;
    const _Float16 d1 = as_h2(D[4]).y;
    const h2 s0 = {d0, d0}, s1 = {d1, d1};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t code = (c == 0) ? realign_block0(D[0], D[4]) : D[c < 4 ? c : c + 1];
        const Codes4 q = expand(code);
        const h2 s = c < 4 ? s0 : s1;
        out[c].x = as_u32(q.q0 * s);
        out[c].y = as_u32(q.q1 * s);
        out[c].z = as_u32(q.q2 * s);
        out[c].w = as_u32(q.q3 * s);
    }
}

// One activation row's 64 halves (two blocks) in chunk order.
__device__ __forceinline__ void permute_x(const uint32_t (&v)[32], u4 (&out)[8]) {
    auto xe = [&](int j) -> uint32_t { return (v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu; };
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        int pos[4];
        chunk_positions(c, pos);
        const int a = pos[0], b = pos[1], cc = pos[2], e = pos[3];
        out[c].x = xe(a) | (xe(cc) << 16);
        out[c].y = xe(a + 16) | (xe(cc + 16) << 16);
        out[c].z = xe(b) | (xe(e) << 16);
        out[c].w = xe(b + 16) | (xe(e + 16) << 16);
    }
}

__global__ void __launch_bounds__(kPfThreads) k_prefill(PfArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kTileBytes];  // [buffer][X | W]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;

    // XCD-aware tile order
    const int b = blockIdx.x;
    const int xcd = b % kXcd;
    const int local = b / kXcd;
    const int m_tile = local % a.mt;
    const int n_tile = (local / a.mt) * kXcd + xcd;
    if (n_tile >= a.nt) return;  // whole workgroup leaves together (grid padded to a multiple of 8 N-tiles)
    const int64_t m0 = (int64_t)m_tile * kBM;
    const int64_t n0 = (int64_t)n_tile * kBN;

    const int np = a.k >> 6;
    const int64_t rb = (int64_t)np * kPairBytes;
    // loader role: weight row (tid < 128) or activation row (tid >= 128)
    const bool is_w = tid < 128;
    const int r = tid & 127;
    const int64_t wrow = min(n0 + r, a.n - 1);
    const bool x_ok = m0 + r < a.m;
    const uint16_t* xrow = a.x + min(m0 + r, a.m - 1) * (int64_t)a.k;
    const bool w_ok = n0 + r < a.n;

    uint32_t Dw[9];
    uint32_t Xv[32];
    auto load_step = [&](int s) {
        if (is_w) {
            load_pair(a.w + wrow * rb + (int64_t)s * kPairBytes, Dw);
        } else {
            const g_u4* src = (const g_u4*)(xrow + 64 * (int64_t)s);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u4 t = src[i];
                Xv[4 * i] = t.x; Xv[4 * i + 1] = t.y; Xv[4 * i + 2] = t.z; Xv[4 * i + 3] = t.w;
            }
        }
    };
    auto store_step = [&](int buf) {
        u4 ch[8];
        uint8_t* dst;
        if (is_w) {
            expand_pair_scaled(Dw, ch);
            if (!w_ok) {
#pragma unroll
                for (int c = 0; c < 8; ++c) ch[c] = u4{0, 0, 0, 0};
            }
            dst = &lds[buf][1][r * kRowBytes];
        } else {
            permute_x(Xv, ch);
            if (!x_ok) {
#pragma unroll
                for (int c = 0; c < 8; ++c) ch[c] = u4{0, 0, 0, 0};
            }
            dst = &lds[buf][0][r * kRowBytes];
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) *(u4*)(dst + 16 * c) = ch[c];
    };

    f16v acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    load_step(0);
    store_step(0);
    __syncthreads();
    for (int s = 0; s < np; ++s) {
        const int buf = s & 1;
        if (s + 1 < np) load_step(s + 1);
        // matrix work on buffer `buf`
        const uint8_t* xt = &lds[buf][0][0];
        const uint8_t* wt = &lds[buf][1][0];
        const int li = lane & 31, g = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int c = 2 * ks + g;
            h8 af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *(const h8*)(xt + (64 * wm + 32 * i + li) * kRowBytes + 16 * c);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bf[j] = *(const h8*)(wt + (64 * wn + 32 * j + li) * kRowBytes + 16 * c);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (s + 1 < np) store_step(buf ^ 1);
        __syncthreads();
    }

    // D layout of the 32x32 product: lane (li, g), element e -> row 8*(e/4) + 4*g + e%4, column li
    const int li = lane & 31, g = lane >> 5;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + 64 * wn + 32 * j + li;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                if (row < a.m && col < a.n) ((g_f32*)a.y)[row * a.n + col] = acc[i][j][e];
            }
        }
}

}  // namespace

hipError_t launch_gemm_prefill(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                               int64_t k, hipStream_t s) {
    PfArgs a;
    a.w = w;
    a.x = x;
    a.y = y;
    a.m = m;
    a.n = n;
    a.k = (int)k;
    a.mt = (int)((m + kBM - 1) / kBM);
    a.nt = (int)((n + kBN - 1) / kBN);
    const int64_t ngroups = (a.nt + kXcd - 1) / kXcd;
    const int64_t grid = ngroups * kXcd * a.mt;
    hipLaunchKernelGGL(k_prefill, dim3((unsigned)grid), dim3(kPfThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace q4
