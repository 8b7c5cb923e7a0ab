// Prefill Q4_0 GEMM on the matrix cores: Y[m][n] = sum_k w[n][k] X[m][k].
//
// Prompt processing multiplies every weight by many token rows at once; the
// pages call their prefill GEMM young and measure it far below decode
// (taozi.news, section "基准成绩"; originshq.com page, section "The Engine:
// ~50 WGSL Kernels Written From Scratch").  With M in the hundreds this is a
// real dense contraction, so the weights are expanded on chip and fed to the
// gfx950 matrix cores (v_mfma_f32_32x32x16_f16, f32 accumulation).
//
// Two kernels.  k_prefill_q (k % 256 == 0, every shape of the 27B sweep)
// moves a weight row's next four block pairs in one 144-byte chunk and splits
// each block pair between two waves; it is described above its definition.
// k_prefill (any k % 64 == 0) is the plain per-step form:
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
// next, whose loads are then issued before this step's matrix work.
// Rows past M or N read clamped in-range addresses and are never stored.
//
// Both kernels issue their direct-to-LDS loads through asm and wait for them
// with explicit vmcnt counts, and use a barrier without a release fence (see
// dma_x4 and step_barrier): the compiler's own waits would drain every
// outstanding load at each step.
//
// A single GEMM runs an XCD-aware grid: workgroup b runs on XCD b % 8, and
// all M-tiles of one N-tile go to consecutive workgroups of the same XCD, so
// a weight tile is read from HBM once and served from that XCD's L2 to the
// others.  A list of GEMMs (the batch entry point) numbers its tiles in list
// order (GEMM, N-tile, M-tile), cuts that order into one range per XCD and
// hands each range's tiles out one at a time to the workgroups of its XCD
// (run_batch), so the M-tiles of a weight tile meet in one L2 and an
// activation matrix is read by one XCD.
#include "q4_device.h"
#include "q4_launch.h"

#include <algorithm>
#include <cmath>
#include <type_traits>
#include <utility>

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

// The four f16 pairs of natural-order weights from 8 code bytes, given as
// four dwords [b, 0x64, b', 0x64] (spread below): as f16 halves they read
// 1024 + b and 1024 + b', b = low nibble + 16 * high nibble.  The low
// nibbles come first (HI = false): H = (P & 0x00F000F0) | 0x5408 5408 reads
// 64.5 + high nibble (0x5400 is 64.0 with spacing 1/16; bit 3 adds 0.5), and
// P - 16 H is exactly low nibble - 8 (one packed fma); H then replaces P.
// The high nibbles (HI = true) are H - 72.5 = high nibble - 8.  Every
// intermediate is exact in f16; the product with the scale rounds once.
template <bool HI>
__device__ __forceinline__ u4 expand8(uint32_t (&P)[4], h2 s) {
    uint32_t q[4];
    if (HI) {
        const h2 off = {(_Float16)72.5f, (_Float16)72.5f};
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = as_u32(as_h2(P[i]) - off);
    } else {
        const h2 m16 = {(_Float16)-16.0f, (_Float16)-16.0f};
        // in stages, so that no instruction reads the result of the one before it
        uint32_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = and_or(P[i], 0x00F000F0u, 0x54085408u);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = as_u32(__builtin_elementwise_fma(as_h2(h[i]), m16, as_h2(P[i])));
#pragma unroll
        for (int i = 0; i < 4; ++i) P[i] = h[i];
    }
    u4 r;
    r.x = as_u32(as_h2(q[0]) * s);
    r.y = as_u32(as_h2(q[1]) * s);
    r.z = as_u32(as_h2(q[2]) * s);
    r.w = as_u32(as_h2(q[3]) * s);
    return r;
}

// Position of chunk c of activation row i within the row's 8 LDS slots is
// c ^ swz(i).  Rows are 128 bytes apart; swz gives 8 consecutive rows 8
// distinct slots (no conflict with 32 banks of 4 bytes) and 16 consecutive
// rows distinct (row parity, slot) pairs (no conflict with 64 banks).
__device__ __forceinline__ int swz(int i) { return (i & 7) ^ ((i >> 3) & 1); }

// Code bytes 8g .. 8g+7 of a block as four dwords [b, 0x64, b', 0x64]
// (consecutive byte pairs spread to the two halves under the exponent byte of
// 1024.0), from the block's code dwords E0, E1.
__device__ __forceinline__ void spread(uint32_t e0, uint32_t e1, uint32_t (&P)[4]) {
    P[0] = __builtin_amdgcn_perm(0x64646464u, e0, 0x04010400u);
    P[1] = __builtin_amdgcn_perm(0x64646464u, e0, 0x04030402u);
    P[2] = __builtin_amdgcn_perm(0x64646464u, e1, 0x04010400u);
    P[3] = __builtin_amdgcn_perm(0x64646464u, e1, 0x04030402u);
}

// Direct-to-LDS loads (lane i's bytes land at M0 + size * i) issued through
// asm, so the compiler does not track them: it cannot tell the ring slot being
// filled from the one being read and would wait for every fill before the
// first LDS read.  The kernel waits for them itself (explicit vmcnt before
// each step's barrier).  They write no register.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void dma_x4(const void* src, uint32_t m0) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma_x1(const void* src, uint32_t m0) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

// Workgroup barrier without the release fence of __syncthreads: that fence
// would wait for every outstanding load of this wave, the ones of the next
// steps included.  The caller first waits (vmcnt) for its own loads of the
// step; the asm is a compiler memory barrier, so no LDS access moves across.
__device__ __forceinline__ void step_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Instruction order of one pipeline phase for the scheduler: each MFMA is
// followed by one LDS read (for the first NR MFMAs) and NV vector ALU ops,
// so the reads and the expansion for the next phase run under the MFMAs.
template <int M, int NR, int NV>
__device__ __forceinline__ void sched_one() {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if constexpr (M < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // VALU
}
template <int NR, int NV, int... M>
__device__ __forceinline__ void sched_phase(std::integer_sequence<int, M...>) {
    (sched_one<M, NR, NV>(), ...);
}

// The batch schedule of both kernels.  The plan cuts the list's tiles
// (numbered GEMM, N-tile, M-tile; M-tile fastest) into one contiguous range
// per XCD.  Workgroup b runs on XCD b % 8 (the dispatcher deals workgroups
// to the XCDs in turn) and takes that XCD's tiles one at a time, so the
// M-tiles of a weight tile run side by side on one XCD: the weight tile is
// fetched into that XCD's L2 once and read from there by the others, and an
// activation matrix is read by one XCD (two at a range's ends), not by all
// eight.  A workgroup whose range is used up helps the next XCD's range, and
// so on round the eight.  The next tile number is fetched while the current
// tile runs.  tile(D, t) computes tile t of descriptor D.
template <typename Tile>
__device__ __forceinline__ void run_batch(const PfDesc* __restrict__ descs, int count, PfHead* head, Tile&& tile) {
    __shared__ uint32_t ticket;
    const int home = (int)(blockIdx.x % kPfQueues);
    for (int v = 0; v < kPfQueues; ++v) {
        PfQueue* q = &head->q[(home + v) % kPfQueues];
        const int64_t begin = q->begin, end = q->end;
        if (begin >= end) continue;
        int d = q->d_first;
        if (threadIdx.x == 0) ticket = atomicAdd(&q->next, 1u);
        __syncthreads();
        uint32_t t = __builtin_amdgcn_readfirstlane(ticket);
        while (begin + (int64_t)t < end) {
            const int64_t gt = begin + (int64_t)t;
            while (d + 1 < count && descs[d + 1].tile_begin <= gt) ++d;
            const PfDesc D = descs[d];
            uint32_t following = 0;
            if (threadIdx.x == 0) following = atomicAdd(&q->next, 1u);
            tile(D, gt - D.tile_begin);
            __syncthreads();  // every wave is done with this tile's LDS and has read `ticket`
            if (threadIdx.x == 0) ticket = following;
            __syncthreads();
            t = __builtin_amdgcn_readfirstlane(ticket);
        }
        __syncthreads();  // every wave has read `ticket` before the next range's first number lands in it
    }
    if (threadIdx.x == 0) {
        __threadfence();  // this workgroup's counter updates come first
        if (atomicAdd(&head->done, 1u) == gridDim.x - 1) {  // last workgroup of the launch
            for (int i = 0; i < kPfQueues; ++i) atomicExch(&head->q[i].next, 0u);
            atomicExch(&head->done, 0u);
        }
    }
}

template <int IT, int NW, bool BATCH>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
k_prefill(PfArgs one, const PfDesc* __restrict__ descs, int count, PfHead* head) {
    constexpr int BM = 32 * IT;
    constexpr int kTile = BM * kStepBytes;           // bytes of one activation tile
    constexpr int kInstr = kTile / (64 * 16) / NW;   // DMA instructions per wave per tile
    constexpr int kWTile = 64 * NW * kPairBytes;     // bytes of one step's weight pairs
    static_assert(kInstr * NW * 64 * 16 == kTile, "tile split over the waves");
    constexpr int kWInstr = kWTile / 4 / 64 / NW;    // dword DMA instructions per wave per step (9)
    static_assert(kWInstr * NW * 64 * 4 == kWTile, "weight tile split over the waves");
    constexpr int kPerStep = kInstr + kWInstr;       // load instructions per wave per step
    static_assert(kPerStep < 32, "vmcnt encoding below");
    // One array per ring slot; the step loop below is unrolled by the ring, so
    // every slot address is a constant.
    __shared__ __attribute__((aligned(16))) uint8_t xs0[kTile], xs1[kTile], xs2[kTile];
    __shared__ __attribute__((aligned(16))) uint32_t ws0[kWTile / 4], ws1[kWTile / 4], ws2[kWTile / 4];
    static_assert(kRing == 3, "three named slots");

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
    auto issue = [&](int s, uint8_t* xdst, uint32_t* wdst) {
        const uint8_t* xb = xbase + (int64_t)s * kStepBytes;
        const uint8_t* wb = wbase + (int64_t)s * kPairBytes;
#pragma unroll
        for (int q = 0; q < kInstr; ++q) dma_x4(xb + xoff[q], lds_addr(xdst + 1024 * (wave * kInstr + q)));
#pragma unroll
        for (int t = 0; t < kWInstr; ++t) dma_x1(wb + woff[t], lds_addr(wdst + 64 * (kWInstr * wave + t)));
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

    auto compute = [&](const uint8_t* xt, const uint32_t* wsl) {
        const uint8_t* wt = (const uint8_t*)wsl + doff;
        uint32_t D[2][9];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int c = 0; c < 9; ++c) D[j][c] = *(const uint32_t*)(wt + 32 * 36 * j + 4 * c);
        h8 av[2][IT];
#pragma unroll
        for (int i = 0; i < IT; ++i) av[0][i] = *(const h8*)(xt + aoff[0] + 4096 * i);
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
                // A operands of the next substep are read before this substep's products
                if (ks + 1 < 4) {
#pragma unroll
                    for (int i = 0; i < IT; ++i) av[(ks + 1) & 1][i] = *(const h8*)(xt + aoff[ks + 1] + 4096 * i);
                }
                u4 bw[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) bw[j] = hi ? expand8<true>(P[j], sc[j]) : expand8<false>(P[j], sc[j]);
#pragma unroll
                for (int i = 0; i < IT; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[ks & 1][i], __builtin_bit_cast(h8, bw[j]),
                                                                           acc[i][j], 0, 0, 0);
            }
        }
    };

    // Ring of three steps: step s computes from slot s % 3; the loads of step
    // s + 2 go to slot (s + 2) % 3 (freed by the barrier of step s) before
    // step s is computed.  The loop is unrolled by the ring so every slot is
    // named statically.
    auto step = [&](int s, const uint8_t* xt, const uint32_t* wt, uint8_t* xf, uint32_t* wf) {
        // this wave's loads of step s have landed: at most the ones of step s + 1 are outstanding
        if (s + 1 < a.np)
            __builtin_amdgcn_s_waitcnt(kPerStep < 16 ? (0x0F70 | kPerStep) : (0x4F70 | (kPerStep - 16)));
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);
        step_barrier();  // everyone's loads of step s are visible; the slot of step s + 2 is free
        if (s + 2 < a.np) issue(s + 2, xf, wf);
        compute(xt, wt);
    };
    issue(0, xs0, ws0);
    if (a.np > 1) issue(1, xs1, ws1);
    for (int s = 0; s < a.np; s += 3) {
        step(s, xs0, ws0, xs2, ws2);
        if (s + 1 < a.np) step(s + 1, xs1, ws1, xs0, ws0);
        if (s + 2 < a.np) step(s + 2, xs2, ws2, xs1, ws1);
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
    run_batch(descs, count, head, [&](const PfDesc& D, int64_t local) {
        tile(D, (local % D.mt) * BM, (local / D.mt) * (64 * NW));
    });
}

// Prefill for k % 256 == 0: weights move in 144-byte row chunks.
//
// The other kernel brings each step's 36 bytes per weight row into LDS; a
// 128-byte line then serves three or four consecutive steps and is requested
// from the caches once for each, and those requests (not the bytes) bound it.
// Here a weight row's next four block pairs (144 bytes, nine 16-byte pieces,
// about two lines) move in one go, every four steps, into a ring of two
// slots, so each line is requested about once per tile.
//
// A workgroup of 2 NWN waves owns BM = 32 IT activation rows x BN = 64 NWN
// weight rows.  Waves (h, s) = (wave / NWN, wave % NWN): slice s owns weight
// rows [64 s, 64 s + 64) as two 32-column MFMA tiles and all IT 32-row
// activation tiles, and of each step's block pair, wave h takes block h
// (k 32 h .. 32 h + 31 of the step: two 16-wide k-substeps).  So the weights
// are expanded once and the two waves of a slice hold partial sums of the
// same outputs, which meet once per tile: in rounds of one activation tile,
// each wave hands the partner the tile the partner stores, through LDS, and
// adds what it receives (own + partner; the sum is the same either way).
//
// The K loop is software-pipelined.  A step's work for a wave is two phases
// (its two k-substeps), each 2 IT MFMAs from one set of A registers and two B
// operands.  While a phase's MFMAs run, the wave reads the next phase's A
// operands from LDS and expands the next B operands, so the matrix cores are
// not left waiting for LDS latency or the dequantization:
//   phase (s, 0): MFMAs of substep 0; read A(s, 1) and the raw weights of
//                 step s + 1; expand B(s, 1)
//   phase (s, 1): MFMAs of substep 1; read A(s + 1, 0); spread the weights of
//                 step s + 1 and expand B(s + 1, 0)
// Steps go in pairs between workgroup barriers, and the last phase of pair t
// already reads step 2t + 2, so the barrier of pair t guarantees steps up to
// 2t + 2: activations live in a ring of five step slots, and the loads
// issued after the barrier of pair t (steps 2t + 3, 2t + 4, and weight chunk
// t / 2 + 1 at even t) refill the slots of pair t - 1.  Every wave waits for
// all of its loads before each barrier.
template <int IT, int NWN, bool BATCH>
__global__ void __launch_bounds__(128 * NWN) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_prefill_q(PfArgs one, const PfDesc* __restrict__ descs, int count, PfHead* head) {
    constexpr int NW = 2 * NWN;
    constexpr int BM = 32 * IT;
    constexpr int BN = 64 * NWN;
    constexpr int kX = BM * kStepBytes;           // activation tile of one step
    constexpr int kXTot = kX / 1024;              // its dwordx4 DMA instructions
    constexpr int kXFull = kXTot / NW;            // ... of every wave
    constexpr int kXRem = kXTot % NW;             // waves below this one issue one more
    static_assert(kXFull >= 1 && kXTot * 1024 == kX, "activation tile split over the waves");
    constexpr int kChunk = 4 * kPairBytes;        // a weight row's bytes for four steps
    constexpr int kW = BN * kChunk;               // weight slot
    constexpr int kWPieces = kW / 16;             // 9 per row
    constexpr int kWFull = kWPieces / (NW * 64);  // weight DMA instructions of every wave (4)
    static_assert(kWPieces - kWFull * NW * 64 == NW * 32, "the rest is one instruction of half the waves");
    constexpr int kXS = 5;                        // activation step slots
    constexpr int kLds = kXS * kX + 2 * kW;       // activation ring, weight ring of two chunks
    constexpr int kLo = (IT + 1) / 2;             // wave h = 0 of a slice stores tiles [0, kLo), h = 1 the rest
    static_assert(NW * 64 * 32 * 4 <= kLds, "exchange rounds fit the ring space");
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];

    const int lane = threadIdx.x & 63;
    const int li = lane & 31;
    const int g = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wh = wave / NWN;  // block of each step's pair this wave takes
    const int wsl = wave % NWN; // weight slice
    const uint32_t lds0 = lds_addr(lds);

    // A-operand offsets: chunk 2 ks + g of activation row 32 i + li, ks = 2 wh + hk.
    uint32_t aoff[2];
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) aoff[hk] = 16u * (uint32_t)(8 * li + ((2 * (2 * wh + hk) + g) ^ swz(li)));
    // Weight dwords of rows 64 wsl + 32 j + li (144-byte pitch in a slot): block 0
    // codes 8g .. 8g+7 sit in dwords 2g .. 2g+2 and its scale in dword 0; block 1
    // codes in dwords 5+2g, 6+2g and its scale in the high half of dword 4.
    const uint32_t wrow = (uint32_t)((64 * wsl + li) * kChunk);
    const uint32_t wcode = wrow + 4u * (uint32_t)(wh ? 5 + 2 * g : 2 * g);
    const uint32_t wscale = wrow + 4u * (uint32_t)(wh ? 4 : 0);

    auto tile = [&](const PfArgs& a, int64_t m0, int64_t n0) {
    const int64_t rb = (int64_t)a.np * kPairBytes;
    const int nsup = a.np / 4;
    const uint8_t* wbase = a.w + n0 * rb;
    const uint8_t* xbase = (const uint8_t*)(a.x + m0 * (int64_t)a.k);
    const int64_t n_last = a.n - 1 - n0;
    const int64_t m_last = a.m - 1 - m0;
    // Source offsets, fixed for the K loop (rows past N or M read the last row):
    //  * weight piece P = 64 (NW q + wave) + lane of a slot is piece P % 9 of
    //    row P / 9 and lands at byte 16 P of the slot;
    //  * activation slot S = 64 (NW q + wave) + lane holds chunk (S % 8) ^ swz
    //    of row S / 8, as in the other kernel.
    uint32_t woff[kWFull + 1], xoff[kXFull + 1];
#pragma unroll
    for (int q = 0; q <= kWFull; ++q) {
        const int P = min(64 * (NW * q + wave) + lane, kWPieces - 1);
        const int64_t row = min((int64_t)(P / 9), n_last);
        woff[q] = (uint32_t)(row * rb + 16 * (P % 9));
    }
#pragma unroll
    for (int q = 0; q <= kXFull; ++q) {
        const int slot = min(64 * (NW * q + wave) + lane, 64 * kXTot - 1);
        const int i = slot >> 3;
        const int c = (slot & 7) ^ swz(i);
        const int64_t row = min((int64_t)i, m_last);
        xoff[q] = (uint32_t)((row * a.k + 8 * c) * 2);
    }
    auto issue_x = [&](int s) {
        const uint8_t* xb = xbase + (int64_t)s * kStepBytes;
        const uint32_t dst = lds0 + (uint32_t)((s % kXS) * kX) + 1024u * (uint32_t)wave;
#pragma unroll
        for (int q = 0; q < kXFull; ++q) dma_x4(xb + xoff[q], dst + 1024u * (uint32_t)(NW * q));
        if (kXRem > 0 && wave < kXRem) dma_x4(xb + xoff[kXFull], dst + 1024u * (uint32_t)(NW * kXFull));
    };
    auto issue_w = [&](int u) {
        const uint8_t* wb = wbase + (int64_t)u * kChunk;
        const uint32_t dst = lds0 + (uint32_t)(kXS * kX + (u & 1) * kW) + 1024u * (uint32_t)wave;
#pragma unroll
        for (int q = 0; q < kWFull; ++q) dma_x4(wb + woff[q], dst + 1024u * (uint32_t)(NW * q));
        if (wave < NW / 2) dma_x4(wb + woff[kWFull], dst + 1024u * (uint32_t)(NW * kWFull));
    };

    f16v acc[IT][2];
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // A operands of substep hk of step s: IT activation tiles.
    auto read_a = [&](int s, int hk, h8 (&A)[IT]) {
        const uint8_t* xt = lds + (s % kXS) * kX;
#pragma unroll
        for (int i = 0; i < IT; ++i) A[i] = *(const h8*)(xt + aoff[hk] + 4096 * i);
    };
    // Raw weight dwords of step s for rows j = 0, 1: block H of the step's pair
    // (H is this wave's block half, a template constant, so no per-lane select
    // between the two layouts): code dwords c[j][0..2] and the scale dword.
    auto read_w = [&](int s, auto Hc, uint32_t (&c)[2][3], uint32_t (&sd)[2]) {
        constexpr int H = decltype(Hc)::value;
        const uint8_t* wt = lds + kXS * kX + ((s >> 2) & 1) * kW + kPairBytes * (s & 3);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint8_t* r = wt + 32 * kChunk * j;
            c[j][0] = *(const uint32_t*)(r + wcode);
            c[j][1] = *(const uint32_t*)(r + wcode + 4);
            if constexpr (H == 0) c[j][2] = *(const uint32_t*)(r + wcode + 8);  // block 0 codes start at byte 2
            sd[j] = *(const uint32_t*)(r + wscale);
        }
    };
    // Code pairs P (spread) and scales of the raw dwords.
    auto spread_w = [&](auto Hc, const uint32_t (&c)[2][3], const uint32_t (&sd)[2], uint32_t (&P)[2][4],
                        h2 (&sc)[2]) {
        constexpr int H = decltype(Hc)::value;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            uint32_t e0, e1;
            _Float16 d;
            if constexpr (H == 0) {
                e0 = __builtin_amdgcn_perm(c[j][1], c[j][0], 0x05040302u);
                e1 = __builtin_amdgcn_perm(c[j][2], c[j][1], 0x05040302u);
                d = as_h2(sd[j]).x;
            } else {
                e0 = c[j][0];
                e1 = c[j][1];
                d = as_h2(sd[j]).y;
            }
            spread(e0, e1, P[j]);
            sc[j] = h2{d, d};
        }
    };
    auto expand = [&](auto HKc, uint32_t (&P)[2][4], const h2 (&sc)[2], u4 (&bw)[2]) {
#pragma unroll
        for (int j = 0; j < 2; ++j) bw[j] = decltype(HKc)::value ? expand8<true>(P[j], sc[j]) : expand8<false>(P[j], sc[j]);
    };
    auto mfma = [&](const h8 (&A)[IT], const u4 (&bw)[2]) {
#pragma unroll
        for (int i = 0; i < IT; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i], __builtin_bit_cast(h8, bw[j]), acc[i][j], 0, 0, 0);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // Pipeline registers: A0/bw0 feed substep 0, A1/bw1 substep 1; Pc/scc are
    // the spread weights of the current step, cn/sdn the raw ones of the next.
    h8 A0[IT], A1[IT];
    u4 bw0[2], bw1[2];
    uint32_t Pc[2][4], cn[2][3], sdn[2];
    h2 scc[2];

    // One step s (its two phases); sn is the step whose operands are read
    // ahead (s + 1, clamped to the last step: reads past the end are unused).
    auto step = [&](int s, int sn, auto Hc) {
        // phase (s, 0)
        mfma(A0, bw0);
        read_a(s, 1, A1);
        read_w(sn, Hc, cn, sdn);
        expand(I1{}, Pc, scc, bw1);
        sched_phase<IT + 4, 3>(std::make_integer_sequence<int, 2 * IT>{});
        __builtin_amdgcn_sched_barrier(0);
        // phase (s, 1)
        mfma(A1, bw1);
        read_a(sn, 0, A0);
        spread_w(Hc, cn, sdn, Pc, scc);
        expand(I0{}, Pc, scc, bw0);
        sched_phase<IT, 5>(std::make_integer_sequence<int, 2 * IT>{});
        __builtin_amdgcn_sched_barrier(0);
    };

    const int np = a.np;
    const int npairs = np >> 1;
    // Prologue: weight chunk 0 and steps 0 .. 2, then the barrier of pair 0
    // and the first step's operands.
    issue_w(0);
    issue_x(0);
    issue_x(1);
    issue_x(2);  // np >= 4
    auto kloop = [&](auto Hc) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        step_barrier();
        if (3 < np) issue_x(3);
        if (4 < np) issue_x(4);
        if (1 < nsup) issue_w(1);
        read_a(0, 0, A0);
        {
            uint32_t c[2][3], sd[2];
            read_w(0, Hc, c, sd);
            spread_w(Hc, c, sd, Pc, scc);
        }
        expand(I0{}, Pc, scc, bw0);
        for (int t = 0; t < npairs; ++t) {
            const int s0 = 2 * t;
            step(s0, s0 + 1, Hc);
            step(s0 + 1, min(s0 + 2, np - 1), Hc);
            if (t + 1 == npairs) break;
            // barrier of pair t + 1: steps up to 2t + 4 and their weight chunk are in LDS
            __builtin_amdgcn_s_waitcnt(0x0F70);
            step_barrier();
            if (s0 + 5 < np) issue_x(s0 + 5);
            if (s0 + 6 < np) issue_x(s0 + 6);
            if (!((t + 1) & 1) && ((t + 1) >> 1) + 1 < nsup) issue_w(((t + 1) >> 1) + 1);
        }
    };
    if (wh == 0)
        kloop(I0{});
    else
        kloop(I1{});

    // The slice's two partial sums meet: in round r, wave h = 0 hands over
    // tile kLo + r (when there is one) and receives tile r, wave h = 1 hands
    // over tile r and receives tile kLo + r.  Each lane's 32 floats go to
    // (slot e4, lane) of the wave's 8 KiB region.  The sum is partner's plus
    // own, the same value whichever wave stores it.
    auto put = [&](int i) {
        float4* mine = (float4*)(lds + 8192 * wave);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
                mine[(4 * j + e4) * 64 + lane] =
                    float4{acc[i][j][4 * e4], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2], acc[i][j][4 * e4 + 3]};
    };
    auto take = [&](int i) {
        const float4* theirs = (const float4*)(lds + 8192 * (wh ? wave - NWN : wave + NWN));
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const float4 v = theirs[(4 * j + e4) * 64 + lane];
                acc[i][j][4 * e4] += v.x;
                acc[i][j][4 * e4 + 1] += v.y;
                acc[i][j][4 * e4 + 2] += v.z;
                acc[i][j][4 * e4 + 3] += v.w;
            }
    };
#pragma unroll
    for (int r = 0; r < kLo; ++r) {
        __syncthreads();  // the last step's (or the previous round's) LDS reads are done
        if (wh == 0) {
            if (kLo + r < IT) put(kLo + r);
        } else {
            put(r);
        }
        __syncthreads();
        if (wh == 0)
            take(r);
        else if (kLo + r < IT)
            take(kLo + r);
    }

    // D layout of the 32x32 product: lane (li, g), element e -> row 8*(e/4) + 4*g + e%4, column li
    auto store = [&](int i, int j) {
        const int64_t col = n0 + 64 * wsl + 32 * j + li;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t row = m0 + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
            if (row < a.m && col < a.n) ((g_f32*)a.y)[row * a.n + col] = acc[i][j][e];
        }
    };
    if (wh == 0) {
#pragma unroll
        for (int i = 0; i < kLo; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) store(i, j);
    } else {
#pragma unroll
        for (int i = kLo; i < IT; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) store(i, j);
    }
    };

    if (!BATCH) {
        // XCD-aware tile order, as in the other kernel
        const int b = blockIdx.x;
        const int xcd = b % kXcd;
        const int local = b / kXcd;
        const int m_tile = local % one.mt;
        const int n_tile = (local / one.mt) * kXcd + xcd;
        if (n_tile >= one.nt) return;
        tile(one, (int64_t)m_tile * BM, (int64_t)n_tile * BN);
        return;
    }
    run_batch(descs, count, head, [&](const PfDesc& D, int64_t local) {
        tile(D, (local % D.mt) * BM, (local / D.mt) * BN);
    });
}

template <int IT, int NW>
hipError_t launch(PfArgs a, hipStream_t s) {
    a.mt = (int)((a.m + 32 * IT - 1) / (32 * IT));
    a.nt = (int)((a.n + 64 * NW - 1) / (64 * NW));
    a.tile_begin = 0;
    const int64_t ngroups = (a.nt + kXcd - 1) / kXcd;
    const int64_t grid = ngroups * kXcd * a.mt;
    hipLaunchKernelGGL((k_prefill<IT, NW, false>), dim3((unsigned)grid), dim3(NW * 64), 0, s, a, nullptr, 0,
                       nullptr);
    return hipGetLastError();
}

template <int IT, int NW>
hipError_t launch_batch(PfHead* head, const PfDesc* descs, int count, int64_t tiles, hipStream_t s) {
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(tiles, 2 * (int64_t)device_cu_count()));
    PfArgs none = {};
    hipLaunchKernelGGL((k_prefill<IT, NW, true>), dim3(grid), dim3(NW * 64), 0, s, none, descs, count, head);
    return hipGetLastError();
}

template <int IT, int NWN>
hipError_t launch_q(PfArgs a, hipStream_t s) {
    a.mt = (int)((a.m + 32 * IT - 1) / (32 * IT));
    a.nt = (int)((a.n + 64 * NWN - 1) / (64 * NWN));
    a.tile_begin = 0;
    const int64_t ngroups = (a.nt + kXcd - 1) / kXcd;
    const int64_t grid = ngroups * kXcd * a.mt;
    hipLaunchKernelGGL((k_prefill_q<IT, NWN, false>), dim3((unsigned)grid), dim3(NWN * 128), 0, s, a, nullptr, 0,
                       nullptr);
    return hipGetLastError();
}

template <int IT, int NWN>
hipError_t launch_batch_q(PfHead* head, const PfDesc* descs, int count, int64_t tiles, hipStream_t s) {
    // one workgroup of 2 NWN waves per CU (the LDS ring takes most of a CU's 160 KiB)
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(tiles, (int64_t)device_cu_count()));
    PfArgs none = {};
    hipLaunchKernelGGL((k_prefill_q<IT, NWN, true>), dim3(grid), dim3(NWN * 128), 0, s, none, descs, count, head);
    return hipGetLastError();
}

}  // namespace

// Tile shape by size: the batch rule's activation rows (128, 96 or 64 x 256
// weight rows) when that still gives every CU a workgroup, else 64 x 256,
// else 64 x 128.
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
    // the batch tile when it still gives every CU a workgroup, else the smallest
    const int tm = prefill_batch_tile_m(m);
    if (k % 256 == 0) {
        if (tm == 128 && tiles(4, 4) >= cus) return launch_q<4, 4>(a, s);
        if (tm == 96 && tiles(3, 4) >= cus) return launch_q<3, 4>(a, s);
        if (tiles(2, 4) >= cus) return launch_q<2, 4>(a, s);
        return launch_q<2, 2>(a, s);
    }
    if (tm == 128 && tiles(4, 4) >= cus) return launch<4, 4>(a, s);
    if (tm == 96 && tiles(3, 4) >= cus) return launch<3, 4>(a, s);
    if (tiles(2, 4) >= cus) return launch<2, 4>(a, s);
    return launch<2, 2>(a, s);
}

// Tile rows for a batch of M-row GEMMs: 128 unless 64-row tiles pad M by
// clearly less (M = 169: 192 rows against 256).
int prefill_batch_tile_m(int64_t m) {
    // the largest of 128, 96 and 64 rows whose padded M is within 15 % of the
    // least padded M (a larger tile re-reads weights and expands them less often)
    const int64_t p128 = (m + 127) / 128 * 128, p96 = (m + 95) / 96 * 96, p64 = (m + 63) / 64 * 64;
    const double least = (double)std::min(p128, std::min(p96, p64));
    if ((double)p128 <= 1.15 * least) return 128;
    if ((double)p96 <= 1.15 * least) return 96;
    return 64;
}

// The other kernel's batched form has no 96-row tile (it would spill
// registers); it runs 64-row tiles instead.
int prefill_other_tile_m(int tile_m) { return tile_m == 96 ? 64 : tile_m; }

// Fills mt, nt, np and tile_begin for the batch tile shape; returns the tiles.
int64_t prefill_fill(PfDesc* d, int tile_m, int64_t tile_begin) {
    d->np = d->k / 64;
    d->mt = (int)((d->m + tile_m - 1) / tile_m);
    d->nt = (int)((d->n + 255) / 256);
    d->tile_begin = tile_begin;
    return (int64_t)d->mt * d->nt;
}

void prefill_queues(const PfDesc* descs, int count, int64_t tiles, PfHead* head) {
    // Work of a tile ~ its K (block pairs); the cut points fall on N-tile
    // boundaries, at the first one where the work before reaches x/8 of all.
    double total = 0.0;
    for (int i = 0; i < count; ++i) total += (double)descs[i].mt * descs[i].nt * descs[i].np;
    int64_t cut[kPfQueues + 1];
    cut[0] = 0;
    cut[kPfQueues] = tiles;
    int d = 0;
    double before = 0.0;  // work of the descriptors before d
    for (int x = 1; x < kPfQueues; ++x) {
        const double target = total * x / kPfQueues;
        while (d < count && before + (double)descs[d].mt * descs[d].nt * descs[d].np < target) {
            before += (double)descs[d].mt * descs[d].nt * descs[d].np;
            ++d;
        }
        if (d == count) {
            cut[x] = tiles;
            continue;
        }
        const double group = (double)descs[d].mt * descs[d].np;  // one N-tile's M-tiles
        int64_t groups = (int64_t)std::ceil((target - before) / group);
        groups = std::min<int64_t>(std::max<int64_t>(groups, 0), descs[d].nt);
        cut[x] = std::max(cut[x - 1], descs[d].tile_begin + groups * descs[d].mt);
    }
    *head = PfHead{};
    int first = 0;
    for (int x = 0; x < kPfQueues; ++x) {
        while (first + 1 < count && descs[first + 1].tile_begin <= cut[x]) ++first;
        head->q[x].begin = cut[x];
        head->q[x].end = cut[x + 1];
        head->q[x].d_first = first;
    }
}

hipError_t launch_gemm_prefill_batch(void* plan, int n_chunked, int64_t tiles_chunked, int n_other,
                                     int64_t tiles_other, int tile_m, hipStream_t s) {
    PfHead* head = static_cast<PfHead*>(plan);
    const PfDesc* descs = reinterpret_cast<const PfDesc*>(head + 2);
    hipError_t e = hipSuccess;
    if (n_chunked > 0)
        e = tile_m == 128  ? launch_batch_q<4, 4>(head, descs, n_chunked, tiles_chunked, s)
            : tile_m == 96 ? launch_batch_q<3, 4>(head, descs, n_chunked, tiles_chunked, s)
                           : launch_batch_q<2, 4>(head, descs, n_chunked, tiles_chunked, s);
    if (e == hipSuccess && n_other > 0)
        e = prefill_other_tile_m(tile_m) == 128 ? launch_batch<4, 4>(head + 1, descs + n_chunked, n_other, tiles_other, s)
                                                : launch_batch<2, 4>(head + 1, descs + n_chunked, n_other, tiles_other, s);
    return e;
}

}  // namespace q4
