// Prefill Q4_0 GEMM on the matrix cores: Y[m][n] = sum_k w[n][k] X[m][k].
//
// Prompt processing multiplies every weight by many token rows at once; the
// pages call their prefill GEMM young and measure it far below decode
// (taozi.news, section "基准成绩"; originshq.com page, section "The Engine:
// ~50 WGSL Kernels Written From Scratch").  With M in the hundreds this is a
// real dense contraction, so the weights are expanded on chip and fed to the
// gfx950 matrix cores (v_mfma_f32_32x32x16_f16, f32 accumulation).
//
// Tiling: a workgroup of NW waves owns BM = 32 IT activation rows x BN = 64 NW
// weight rows.  Wave w owns weight rows [64 w, 64 w + 64) of the tile as two
// 32-column MFMA tiles (j) and all IT 32-row tiles (i) of the activations.
// K advances 64 columns (one Q4_0 block pair per weight row) per step:
//  * the activation tile [BM][64] (f16, natural k order) moves from HBM into
//    LDS with global_load_lds_dwordx4, in a ring of three; the 16-byte chunk c of
//    row i is stored at slot 8 i + (c ^ swz(i)), chosen through each lane's
//    source address, so the MFMA operand reads of 32 rows spread over the
//    banks;
//  * the step's weight pairs (36 bytes per row) move into LDS the same way
//    (dword pieces, row-major); lane (n, g) = (lane % 32, lane / 32) reads the
//    pairs of its two weight rows and expands, for k-substep ks, the 8
//    weights k = 16 ks + 8 g .. + 7
//    of the pair in natural order (block ks / 2; low nibbles of code bytes
//    8g .. 8g+7 for even ks, high nibbles for odd ks) straight into its B
//    operand: (code - 8) exact in f16 (v_perm_b32 + v_and_or_b32 +
//    v_pk_add_f16), times d rounded once (v_pk_mul_f16);
//  * the A operand of lane (i, g) at substep ks is the chunk 2 ks + g of
//    activation row i, so both operands cover the same 8 k.
// One barrier per step: every wave waits for its own loads of the step, the
// barrier makes all of them visible and frees the buffer of the step after
// next, whose loads are then issued before this step's matrix work (three
// steps in flight: a step's matrix work is shorter than a load's latency).
// Rows past M or N read clamped in-range addresses and are never stored.
// Grid order is XCD-aware: workgroup b runs on XCD b % 8, and all M-tiles of
// one N-tile go to consecutive workgroups of the same XCD, so a weight tile is
// read from HBM once and served from that XCD's L2 to the others.
#include "q4_device.h"
#include "q4_launch.h"

#include <algorithm>

namespace q4 {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) float g_f32;
typedef __attribute__((address_space(1))) void g_void;
typedef __attribute__((address_space(3))) void l_void;

constexpr int kXcd = 8;
constexpr int kRing = 3;  // steps in flight: activation tiles in LDS, weight pairs in registers
constexpr int kStepBytes = 64 * 2;  // one activation row of one step (64 halves)

typedef PfDesc PfArgs;

__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The four f16 pairs of natural-order weights from 8 code bytes (two dwords,
// byte j = codes j (low nibble) and j + 16 (high nibble) of the block):
// HI selects the high nibbles.  Exact (code - 8), then times the scale.
template <bool HI>
__device__ __forceinline__ u4 expand8(const uint32_t (&P)[4], h2 s) {
    const uint32_t mask = HI ? 0x00F000F0u : 0x000F000Fu;
    const uint32_t bias = HI ? 0x54005400u : 0x64006400u;
    const h2 off = HI ? h2{(_Float16)72.0f, (_Float16)72.0f} : h2{(_Float16)1032.0f, (_Float16)1032.0f};
    u4 r;
    r.x = as_u32((as_h2(and_or(P[0], mask, bias)) - off) * s);
    r.y = as_u32((as_h2(and_or(P[1], mask, bias)) - off) * s);
    r.z = as_u32((as_h2(and_or(P[2], mask, bias)) - off) * s);
    r.w = as_u32((as_h2(and_or(P[3], mask, bias)) - off) * s);
    return r;
}

// Position of chunk c of activation row i within the row's 8 LDS slots is
// c ^ swz(i).  Rows are 128 bytes apart; swz gives 8 consecutive rows 8
// distinct slots (no conflict with 32 banks of 4 bytes) and 16 consecutive
// rows distinct (row parity, slot) pairs (no conflict with 64 banks).
__device__ __forceinline__ int swz(int i) { return (i & 7) ^ ((i >> 3) & 1); }

// Code bytes 8g .. 8g+7 of a block as four dwords [b, 0, b', 0] (consecutive
// byte pairs spread to the two halves), from the block's code dwords E0, E1.
__device__ __forceinline__ void spread(uint32_t e0, uint32_t e1, uint32_t (&P)[4]) {
    P[0] = __builtin_amdgcn_perm(e0, e0, 0x0C010C00u);
    P[1] = __builtin_amdgcn_perm(e0, e0, 0x0C030C02u);
    P[2] = __builtin_amdgcn_perm(e1, e1, 0x0C010C00u);
    P[3] = __builtin_amdgcn_perm(e1, e1, 0x0C030C02u);
}

template <int IT, int NW, bool BATCH>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
k_prefill(PfArgs one, const PfDesc* __restrict__ descs, int count, int64_t total) {
    constexpr int BM = 32 * IT;
    constexpr int kTile = BM * kStepBytes;           // bytes of one activation tile
    constexpr int kInstr = kTile / (64 * 16) / NW;   // DMA instructions per wave per tile
    constexpr int kWTile = 64 * NW * kPairBytes;     // bytes of one step's weight pairs
    static_assert(kInstr * NW * 64 * 16 == kTile, "tile split over the waves");
    constexpr int kWInstr = kWTile / 4 / 64 / NW;    // dword DMA instructions per wave per step (9)
    static_assert(kWInstr * NW * 64 * 4 == kWTile, "weight tile split over the waves");
    constexpr int kPerStep = kInstr + kWInstr;       // load instructions per wave per step
    static_assert(kPerStep < 32, "vmcnt encoding below");
    __shared__ __attribute__((aligned(16))) uint8_t xs[kRing][kTile];
    __shared__ __attribute__((aligned(16))) uint32_t wsh[kRing][kWTile / 4];

    const int lane = threadIdx.x & 63;
    const int li = lane & 31;
    const int g = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));

    // One output tile: activation rows [m0, m0 + BM) x weight rows [n0, n0 + 64 NW).
    auto tile = [&](const PfArgs& a, int64_t m0, int64_t n0) {
    const int64_t rb = (int64_t)a.np * kPairBytes;
    // Per-lane source offsets (bytes, 32-bit: a weight matrix or an
    // activation tile is far below 4 GiB from its base) fixed for the whole
    // K loop; the uniform bases advance by one pair / 64 halves per step.
    //  * weights: dword G of the step's tile (row G / 9, dword G % 9; rows past
    //    N read row N - 1) goes to LDS word G, a row-major tile with a 36-byte
    //    pitch; instruction t of this wave covers G = 64 (9 wave + t) + lane.
    //  * activations: slot S = 64 (kInstr wave + q) + lane holds chunk
    //    (S % 8) ^ (row % 8) of row S / 8 (rows past M read row M - 1).
    const uint8_t* wbase = a.w + n0 * rb;
    const uint8_t* xbase = (const uint8_t*)(a.x + m0 * (int64_t)a.k);
    const int64_t n_last = a.n - 1 - n0;  // last valid row of the tile
    const int64_t m_last = a.m - 1 - m0;
    uint32_t woff[kWInstr], xoff[kInstr];
#pragma unroll
    for (int t = 0; t < kWInstr; ++t) {
        const int G = 64 * (kWInstr * wave + t) + lane;
        const int64_t row = min((int64_t)(G / 9), n_last);
        woff[t] = (uint32_t)(row * rb + 4 * (G % 9));
    }
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
        const int slot = 64 * (wave * kInstr + q) + lane;
        const int i = slot >> 3;
        const int c = (slot & 7) ^ swz(i);
        const int64_t row = min((int64_t)i, m_last);
        xoff[q] = (uint32_t)((row * a.k + 8 * c) * 2);
    }
    auto issue = [&](int s, int buf) {
        const uint8_t* xb = xbase + (int64_t)s * kStepBytes;
        const uint8_t* wb = wbase + (int64_t)s * kPairBytes;
#pragma unroll
        for (int q = 0; q < kInstr; ++q)
            __builtin_amdgcn_global_load_lds((g_void*)(xb + xoff[q]),
                                             (l_void*)(&xs[buf][0] + 1024 * (wave * kInstr + q)), 16, 0, 0);
#pragma unroll
        for (int t = 0; t < kWInstr; ++t)
            __builtin_amdgcn_global_load_lds((g_void*)(wb + woff[t]),
                                             (l_void*)(&wsh[buf][0] + 64 * (kWInstr * wave + t)), 4, 0, 0);
    };

    // LDS read offsets: the A chunk c = 2 ks + g of row 32 i + li sits at slot
    // 256 i + 8 li + (c ^ swz(li)) (swz(32 i + li) = swz(li)); the weight pairs
    // of rows 64 wave + 32 j + li.
    uint32_t aoff[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) aoff[ks] = 16u * (uint32_t)(8 * li + ((2 * ks + g) ^ swz(li)));
    const uint32_t doff = 4u * (uint32_t)((64 * wave + li) * 9);

    f16v acc[IT][2];
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    auto compute = [&](int buf) {
        const uint8_t* xt = &xs[buf][0];
        const uint8_t* wt = (const uint8_t*)&wsh[buf][0] + doff;
        uint32_t D[2][9];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int c = 0; c < 9; ++c) D[j][c] = *(const uint32_t*)(wt + 32 * 36 * j + 4 * c);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            uint32_t P[2][4];
            h2 sc[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                uint32_t e0, e1;
                if (blk == 0) {
                    // block 0 codes start at byte 2 of the pair: bytes 8g .. 8g+7 of the codes
                    // are bytes 2 .. 9 of dwords D[2g] .. D[2g+2]
                    const uint32_t lo = g ? D[j][2] : D[j][0];
                    const uint32_t mid = g ? D[j][3] : D[j][1];
                    const uint32_t hi = g ? D[j][4] : D[j][2];
                    e0 = __builtin_amdgcn_perm(mid, lo, 0x05040302u);
                    e1 = __builtin_amdgcn_perm(hi, mid, 0x05040302u);
                    const _Float16 d = as_h2(D[j][0]).x;
                    sc[j] = h2{d, d};
                } else {
                    e0 = g ? D[j][7] : D[j][5];
                    e1 = g ? D[j][8] : D[j][6];
                    const _Float16 d = as_h2(D[j][4]).y;
                    sc[j] = h2{d, d};
                }
                spread(e0, e1, P[j]);
            }
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
                const int ks = 2 * blk + hi;
                u4 bw[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) bw[j] = hi ? expand8<true>(P[j], sc[j]) : expand8<false>(P[j], sc[j]);
#pragma unroll
                for (int i = 0; i < IT; ++i) {
                    const h8 av = *(const h8*)(xt + aoff[ks] + 4096 * i);
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, __builtin_bit_cast(h8, bw[j]),
                                                                           acc[i][j], 0, 0, 0);
                }
            }
        }
    };

    // Ring of three steps: step s uses buffers s % 3; the loads of step s + 2
    // are issued (after the barrier that frees their buffers) before step s is
    // computed.
    issue(0, 0);
    if (a.np > 1) issue(1, 1);
    int buf = 0;
    for (int s = 0; s < a.np; ++s) {
        // this wave's loads of step s have landed: at most the ones of step s + 1 are outstanding
        if (s + 1 < a.np)
            __builtin_amdgcn_s_waitcnt(kPerStep < 16 ? (0x0F70 | kPerStep) : (0x4F70 | (kPerStep - 16)));
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();  // everyone's loads of step s are visible; the buffers of step s + 2 are free
        const int fill = buf == 0 ? 2 : buf - 1;
        if (s + 2 < a.np) issue(s + 2, fill);
        compute(buf);
        buf = buf == kRing - 1 ? 0 : buf + 1;
    }

    // D layout of the 32x32 product: lane (li, g), element e -> row 8*(e/4) + 4*g + e%4, column li
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + 64 * wave + 32 * j + li;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                if (row < a.m && col < a.n) ((g_f32*)a.y)[row * a.n + col] = acc[i][j][e];
            }
        }
    };

    if (!BATCH) {
        // XCD-aware tile order
        const int b = blockIdx.x;
        const int xcd = b % kXcd;
        const int local = b / kXcd;
        const int m_tile = local % one.mt;
        const int n_tile = (local / one.mt) * kXcd + xcd;
        if (n_tile >= one.nt) return;  // whole workgroup leaves together (grid padded to a multiple of 8 N-tiles)
        tile(one, (int64_t)m_tile * BM, (int64_t)n_tile * (64 * NW));
        return;
    }
    // Batch: the tiles (GEMM, N-tile, M-tile; M-tile fastest, so consecutive
    // tiles reuse a weight tile from L2) whose start cost (steps) lies in this
    // workgroup's byte-balanced share [T g / G, T (g + 1) / G).
    const int64_t G = gridDim.x;
    const int64_t c_lo = uniform64((total / G) * blockIdx.x + ((total % G) * blockIdx.x) / G);
    const int64_t c_hi = uniform64((total / G) * (blockIdx.x + 1) + ((total % G) * ((int64_t)blockIdx.x + 1)) / G);
    if (c_lo >= c_hi) return;
    int lo = 0, hi = count - 1;  // last descriptor starting at or before c_lo
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (descs[mid].cost_begin <= c_lo) lo = mid; else hi = mid - 1;
    }
    int d = lo;
    PfDesc D = descs[d];
    int64_t t = uniform64((c_lo - D.cost_begin + D.np - 1) / D.np);
    for (;;) {
        if (t >= (int64_t)D.mt * D.nt) {
            if (++d >= count) break;
            D = descs[d];
            t = 0;
        }
        if (D.cost_begin + t * D.np >= c_hi) break;
        __syncthreads();  // the previous tile's buffers are no longer read
        tile(D, (t % D.mt) * BM, (t / D.mt) * (64 * NW));
        ++t;
    }
}

template <int IT, int NW>
hipError_t launch(PfArgs a, hipStream_t s) {
    a.mt = (int)((a.m + 32 * IT - 1) / (32 * IT));
    a.nt = (int)((a.n + 64 * NW - 1) / (64 * NW));
    a.cost_begin = 0;
    const int64_t ngroups = (a.nt + kXcd - 1) / kXcd;
    const int64_t grid = ngroups * kXcd * a.mt;
    hipLaunchKernelGGL((k_prefill<IT, NW, false>), dim3((unsigned)grid), dim3(NW * 64), 0, s, a, nullptr, 0,
                       (int64_t)0);
    return hipGetLastError();
}

template <int IT, int NW>
hipError_t launch_batch(const PfDesc* descs, int count, int64_t total, hipStream_t s) {
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(total, 2 * (int64_t)device_cu_count()));
    PfArgs none = {};
    hipLaunchKernelGGL((k_prefill<IT, NW, true>), dim3(grid), dim3(NW * 64), 0, s, none, descs, count, total);
    return hipGetLastError();
}

}  // namespace

// Tile shape by size: the largest tile (activation rows 32 IT x weight rows
// 64 NW) that still gives every CU a workgroup, else the smallest.  (128 x
// 128 is left out: it needs more than 256 registers, one wave per SIMD.)
hipError_t launch_gemm_prefill(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                               int64_t k, hipStream_t s) {
    PfArgs a;
    a.w = w;
    a.x = x;
    a.y = y;
    a.m = m;
    a.n = n;
    a.k = (int)k;
    a.np = (int)(k / 64);
    const int64_t cus = device_cu_count();
    auto tiles = [&](int it, int nw) { return ((m + 32 * it - 1) / (32 * it)) * ((n + 64 * nw - 1) / (64 * nw)); };
    if (m > 96 && tiles(4, 4) >= cus) return launch<4, 4>(a, s);
    if (tiles(2, 4) >= cus) return launch<2, 4>(a, s);
    return launch<2, 2>(a, s);
}

// Tile rows for a batch of M-row GEMMs: 128 unless 64-row tiles pad M by
// clearly less (M = 169: 192 rows against 256).
int prefill_batch_tile_m(int64_t m) {
    const int64_t p128 = (m + 127) / 128 * 128, p64 = (m + 63) / 64 * 64;
    return (double)p128 <= 1.15 * (double)p64 ? 128 : 64;
}

// Fills mt, nt, np and cost_begin for the batch tile shape; returns the cost.
int64_t prefill_fill(PfDesc* d, int tile_m, int64_t cost_begin) {
    d->np = d->k / 64;
    d->mt = (int)((d->m + tile_m - 1) / tile_m);
    d->nt = (int)((d->n + 255) / 256);
    d->cost_begin = cost_begin;
    return (int64_t)d->mt * d->nt * d->np;
}

hipError_t launch_gemm_prefill_batch(const PfDesc* descs, int count, int tile_m, int64_t total, hipStream_t s) {
    return tile_m == 128 ? launch_batch<4, 4>(descs, count, total, s) : launch_batch<2, 4>(descs, count, total, s);
}

}  // namespace q4
