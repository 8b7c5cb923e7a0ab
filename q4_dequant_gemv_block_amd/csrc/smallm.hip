// Small-M Q4_0 GEMM: Y[m][n] = sum_k w[n][k] X[m][k] for 2 <= M <= 16, for
// one GEMM or a list of GEMMs in one launch.
//
// The batched pass that verifies speculative drafts, and 16-token prefill
// chunks ("SwarmLLM v0.2.0 ..." on aipolix.com, section "Speculation is used to
// amortize network round trips"; taozi.news, section "技术架构").  Every weight
// is read from memory and expanded from its 4-bit code exactly once for all M
// activation rows.
//
// With up to 16 activation rows this is a dense contraction, so the products
// run on the matrix cores (v_mfma_f32_16x16x32_f16): the vector ALUs only
// expand and scale the weights, at the same cost per weight as the M = 1
// kernel, whatever M is.  (A vector-ALU version with one v_dot2 chain per
// activation row was measured at 1.8 TB/s for M = 2 down to 0.4 TB/s for
// M = 16, bound by its LDS reads.)
//
// Work: a workgroup owns tiles of 16 weight rows per wave and one K-range of
// its GEMM; the K-range is the longest run of 16-pair spans whose activations
// for all M rows fit the LDS the weights leave free.  Items (GEMM, K-range,
// tile) are ordered GEMM, K-range, tile, and every workgroup takes a
// byte-balanced contiguous run of them, so the activations of a K-range are
// staged once and serve many tiles.  When a GEMM has several K-ranges each
// range writes its partial product to the workspace and a second kernel adds
// the partials in range order, so results are deterministic.
//
// Each pair expands to 8 chunks of 8 halves ((code - 8) * d rounded once to
// f16: error <= 2^-11 of each weight, inside the 1e-3 bound); chunk c of lane
// (g, n) = (lane / 16, lane % 16) is the B operand for weight row n, and the A
// operand of lane (g, m) is chunk c of the same pair of activation row m,
// read from LDS (rows m >= M read row M - 1; those products are never
// stored).  The 32 k of one MFMA are 8 k from each of 4 pairs; both operands
// use the same assignment, so the sum is the full dot product.  Pairs beyond
// K/64 meet zero activations.
//
// Two engines move the weights:
//  * LDS ring (k_smallm_lds, M <= 7).  Weights move from HBM straight into
//    LDS in whole lines, as in the M = 1 engine.  A workgroup of 8 waves owns
//    128-row tiles; a wave's unit is its 16 rows x one 8-pair segment (288
//    bytes per row), six buffer loads of 16 bytes per lane straight to LDS
//    into a ring of two unit slots per wave (86 KiB in all, the activations
//    get the other 76 KiB: K = 17,408 splits from M = 4 on), waited for
//    with explicit vmcnt counts; a unit is read into registers and its slot
//    refilled before it is computed.  The loads are cached: a segment shares
//    its end lines with the row's next segment, which the same wave loads
//    next (with the non-temporal hint those lines were fetched twice, 1.24x
//    the bytes).  In a slot, row n's segment is four 80-byte groups, one per
//    lane group g (bytes 72 g .. 72 g + 63 in four 16-byte pieces, then bytes
//    72 g + 56 .. 72 g + 71), so the pairs 2g, 2g+1 of lane (g, n) start on a
//    16-byte boundary; rows are 21 pieces apart (one pad piece), so the 16
//    rows of one ds_read_b128 fall on distinct banks; the lane reads its pairs
//    with five ds_read_b128.  Rows beyond N and bytes past the matrix end
//    load zeros (the buffer descriptor ends at the matrix end).
//  * Register loads (k_smallm_reg, M > 7), when the activations need the
//    whole LDS (M = 16: 5,120 columns in one K-range).  A workgroup of 16
//    waves owns 256-row tiles; lane (g, n) loads pairs g, g+4, g+8, g+12 of
//    its row's 16-pair segment (the four lanes of a row cover its 576
//    contiguous bytes) into registers, the next unit's loads issued before
//    the current one is computed.  These loads touch about 32 lines per
//    instruction and bind the L1's tag lookups; rows beyond N and pairs
//    beyond K/64 read clamped in-range addresses.
#include "q4_device.h"
#include "q4_launch.h"

#include <algorithm>
#include <type_traits>

namespace q4 {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) float g_f32;

// Two ways to move the weights (see above): ENG = 0 register loads, 1 LDS
// ring.  Waves per workgroup, rows per tile, pairs per unit and row, the LDS
// the weight rings take and the LDS left for the staged activations.
template <int ENG>
struct Geo;
template <>
struct Geo<0> {
    static constexpr int kWaves = 16, kTileRows = 256, kSegPairs = 16, kXBytes = 160 * 1024;
};
#ifndef Q4_SM_WAVES
#define Q4_SM_WAVES 8
#endif
#ifndef Q4_SM_NB
#define Q4_SM_NB 2
#endif
template <>
struct Geo<1> {
    static constexpr int kWaves = Q4_SM_WAVES, kTileRows = 16 * kWaves, kSegPairs = 8;
    static constexpr int kPieces = 21;               // 16-byte pieces per row in a slot: 4 lane groups x 5, one pad
    static constexpr int kPitch = 16 * kPieces;      // 336
    static constexpr int kSlot = 16 * kPitch;        // 5376 bytes: one unit of one wave
    static constexpr int kNB = Q4_SM_NB;             // unit slots per wave
    static constexpr int kRing = kWaves * kNB * kSlot;      // 86016 bytes at the start of LDS
    static constexpr int kLoads = (16 * kPieces + 63) / 64;  // 6 load instructions per unit
    static constexpr int kXBytes = 160 * 1024 - kRing;       // 77824
};
// M up to this uses the LDS ring; larger M the register loads, whose
// activations may take the whole LDS (measured on the 448-GEMM sweep: the
// ring is 5-7 % faster at M = 2..5, 2 % slower at M = 8).
constexpr int kLdsMaxM = 7;
__host__ __device__ constexpr int engine_of(int64_t m) { return m <= kLdsMaxM ? 1 : 0; }

__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Segments (SEG pairs) of K-range c of a descriptor.
template <int SEG>
__device__ __forceinline__ int segs_of(const SmDesc& D, int c) {
    return (min(D.P, D.np - c * D.P) + SEG - 1) / SEG;
}

// First unit (cost) of item (c, t): ranges before c are full.
template <int SEG>
__device__ __forceinline__ int64_t item_start(const SmDesc& D, int c, int t) {
    return D.cost_begin + (int64_t)c * D.tiles * (D.P / SEG) + (int64_t)t * segs_of<SEG>(D, c);
}

// Direct-to-LDS loads through asm (the compiler does not track them; the
// kernel waits with explicit vmcnt counts): 16 bytes per lane at byte offset
// voff of the buffer into LDS at M0 + 16 * lane.  They write no register; the
// s_nop covers the M0 write just before.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
struct Rsrc {
    u4 w;
};
// Raw buffer of `bytes` bytes at base (gfx9: stride 0, 32-bit data format);
// loads at or past `bytes` return zeros.  Every field is wave-uniform.
__device__ __forceinline__ Rsrc make_rsrc(const uint8_t* base, uint64_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    Rsrc r;
    r.w.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r.w.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
    r.w.z = __builtin_amdgcn_readfirstlane((uint32_t)min(bytes, (uint64_t)0xFFFFFFFFu));
    r.w.w = 0x00020000u;
    return r;
}
__device__ __forceinline__ void dma16(const Rsrc& r, uint32_t voff, uint32_t m0) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r.w), "{m0}"(m0) : "memory");
}
// s_waitcnt vmcnt(N) (a compiler barrier too: no LDS read of a slot moves above it).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Greedy-pick epilogue (keys != null): each lane keeps, for its four
// activation rows, the largest argmax key over the outputs it stored; at the
// end the workgroup reduces them and writes row mm's key to
// keys[mm * gridDim.x + blockIdx.x] (0 when it stored none of that row).
// `scratch` is LDS no wave still reads (2 KiB).
template <int WAVES>
__device__ __forceinline__ void write_keys(uint64_t (&best)[4], int m, uint64_t* __restrict__ keys, void* scratch) {
    const int lane = threadIdx.x & 63, g = lane >> 4, wave = threadIdx.x >> 6;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) {  // over the 16 lanes of the group
            const uint64_t v = __shfl_xor(best[e], o, 64);
            best[e] = v > best[e] ? v : best[e];
        }
    uint64_t* sh = static_cast<uint64_t*>(scratch);
    __syncthreads();  // every wave is done with the LDS
    if ((lane & 15) == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sh[wave * 16 + 4 * g + e] = best[e];
    }
    __syncthreads();
    if ((int)threadIdx.x < m) {
        uint64_t r = 0;
        for (int w = 0; w < WAVES; ++w) r = sh[w * 16 + threadIdx.x] > r ? sh[w * 16 + threadIdx.x] : r;
        keys[(int64_t)threadIdx.x * gridDim.x + blockIdx.x] = r;
    }
}

struct SmCursor {
    int d, c, t, jb;
};

// Staged activations, two layouts.  Padded (SWZ = false): row r holds its P
// pairs x 8 chunks (16 bytes each) from chunk r (8P + 1) on, chunk c of pair
// pl at 8 pl + c; the odd row stride puts the 16 rows a wave reads at once on
// different LDS banks.  Swizzled (SWZ = true, when the padding does not fit:
// M = 16 rows of 5120 columns take exactly 160 KiB): row stride 8P, chunk c of
// pair pl at 8 (pl ^ ((r >> 3) & 1)) + (c ^ (r & 7)), which spreads the 16
// rows over the banks without extra space (P is even, so pl ^ 1 stays in the
// range); it costs per-lane read offsets, so it is used only there.
template <bool SWZ>
__device__ __forceinline__ int x_stride(const SmDesc& D) { return SWZ ? 8 * D.P : 8 * D.P + 1; }
template <bool SWZ>
__device__ __forceinline__ int x_slot(int r, int pl, int c) {
    return SWZ ? 8 * (pl ^ ((r >> 3) & 1)) + (c ^ (r & 7)) : 8 * pl + c;
}

// Activations of pairs [c*P, c*P + SEG*segs) of all M rows into their slots
// (THREADS threads); pairs past K/64 are zero.
template <bool SWZ, int SEG, int THREADS>
__device__ void stage_range(const SmDesc& D, int c, int m, u4* __restrict__ xs) {
    const int p0 = c * D.P;
    const int npairs = SEG * segs_of<SEG>(D, c);
    for (int it = threadIdx.x; it < 2 * npairs * m; it += THREADS) {
        const int mm = it % m;
        const int b = it / m;  // block within the range
        const int p = p0 + (b >> 1);
        uint32_t v[16];
        if (p < D.np) {
            const g_u4* src = (const g_u4*)(D.x + (int64_t)mm * D.k + 32 * (int64_t)(2 * p0 + b));
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
        // The block half as a compile-time constant, so that every position
        // below is one too (with a run-time half each half-word extraction
        // was a select over the 16 registers: twice the kernel's code).
        auto put = [&](auto H) {
            constexpr int half = decltype(H)::value;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                int pos[4];
                chunk_positions(4 * half + cc, pos);
                const int off = 32 * half;
                const int a = pos[0] - off, bb = pos[1] - off, cq = pos[2] - off, e = pos[3] - off;
                u4 ent;
                ent.x = xe(a) | (xe(cq) << 16);
                ent.y = xe(a + 16) | (xe(cq + 16) << 16);
                ent.z = xe(bb) | (xe(e) << 16);
                ent.w = xe(bb + 16) | (xe(e + 16) << 16);
                xs[mm * x_stride<SWZ>(D) + x_slot<SWZ>(mm, b >> 1, 4 * half + cc)] = ent;
            }
        };
        if (b & 1)
            put(std::integral_constant<int, 1>{});
        else
            put(std::integral_constant<int, 0>{});
    }
    // Every staging load has been consumed, but on the path that skips both
    // halves the compiler would keep one pending into the GEMM loop and wait
    // there for every outstanding load, the ring's included, at each unit.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

// The LDS-ring engine (M <= kLdsMaxM).
template <bool SWZ>
__global__ void __launch_bounds__(Geo<1>::kWaves * 64) k_smallm_lds(const SmDesc* __restrict__ descs, int count,
                                                                     SmDesc one, int m, int64_t total,
                                                                     float* __restrict__ ws, uint64_t* __restrict__ keys) {
    using E = Geo<1>;
    constexpr int kSegPairs = E::kSegPairs, kTileRows = E::kTileRows, kPieces = E::kPieces, kPitch = E::kPitch;
    constexpr int kSlot = E::kSlot, kNB = E::kNB, kRing = E::kRing, kLoads = E::kLoads;
    extern __shared__ u4 lds_u4[];
    uint8_t* lds = reinterpret_cast<uint8_t*>(lds_u4);
    u4* xs = reinterpret_cast<u4*>(lds + kRing);  // staged activations after the weight rings
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int n_desc = descs ? count : 1;
    auto get = [&](int d) -> SmDesc { return descs ? descs[d] : one; };
    const uint32_t ring0 = lds_addr(lds) + (uint32_t)(wave * kNB * kSlot);

    const int64_t G = gridDim.x;
    const int64_t c_lo = uniform64((total / G) * blockIdx.x + ((total % G) * blockIdx.x) / G);
    const int64_t c_hi = uniform64((total / G) * (blockIdx.x + 1) + ((total % G) * ((int64_t)blockIdx.x + 1)) / G);
    if (c_lo >= c_hi) {  // whole workgroup leaves together
        if (keys && (int)threadIdx.x < m) keys[(int64_t)threadIdx.x * gridDim.x + blockIdx.x] = 0;
        return;
    }

    // First item starting at or after c_lo.
    int lo = 0, hi = n_desc - 1;  // last descriptor starting at or before c_lo
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (get(mid).cost_begin <= c_lo) lo = mid; else hi = mid - 1;
    }
    SmCursor cl;
    cl.d = lo;
    cl.jb = 0;
    SmDesc Dl = get(lo);
    {
        const int64_t full = (int64_t)Dl.tiles * (Dl.P / kSegPairs);  // units of a full K-range
        const int64_t o = c_lo - Dl.cost_begin;
        int c = (int)(o / full < Dl.nranges - 1 ? o / full : Dl.nranges - 1);
        const int64_t r = o - c * full;
        const int sg = segs_of<kSegPairs>(Dl, c);
        int64_t t = (r + sg - 1) / sg;
        if (t >= Dl.tiles) {
            t = 0;
            if (++c == Dl.nranges) {
                c = 0;
                if (++cl.d < n_desc) Dl = get(cl.d);
            }
        }
        cl.c = c;
        cl.t = (int)t;
    }
    bool have_l = cl.d < n_desc && item_start<kSegPairs>(Dl, cl.c, cl.t) < c_hi;
    if (!have_l) {
        if (keys && (int)threadIdx.x < m) keys[(int64_t)threadIdx.x * gridDim.x + blockIdx.x] = 0;
        return;
    }

    auto advance_l = [&]() {
        if (++cl.jb < segs_of<kSegPairs>(Dl, cl.c)) return;
        cl.jb = 0;
        if (++cl.t == Dl.tiles) {
            cl.t = 0;
            if (++cl.c == Dl.nranges) {
                cl.c = 0;
                if (++cl.d >= n_desc) {
                    have_l = false;
                    return;
                }
                Dl = get(cl.d);
            }
        }
        have_l = item_start<kSegPairs>(Dl, cl.c, cl.t) < c_hi;
    };

    // This lane's piece of load q of a unit: slot piece L = 64 q + lane is
    // piece L % 21 of row L / 21; piece 5 gg + i (gg < 4) holds bytes
    // 72 gg + 16 i of the row's segment for i < 4 and 72 gg + 56 for i = 4;
    // piece 20 is padding (loaded with a copy of piece 19).  Lanes past the
    // slot's 336 pieces do not load.
    int prow[kLoads], poff[kLoads];
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
        const int L = min(64 * q + lane, 16 * kPieces - 1);
        const int pc = min(L % kPieces, 4 * 5 - 1);
        const int gg = pc / 5, i = pc % 5;
        prow[q] = L / kPieces;
        poff[q] = 72 * gg + (i < 4 ? 16 * i : 56);
    }
    const bool last_live = 64 * (kLoads - 1) + lane < 16 * kPieces;

    // Loads of the unit at the cursor into slot `slot`: rows t*128 + 16*wave + n,
    // pairs c*P + 8*jb ..; the descriptor ends at the matrix end.
    auto issue = [&](int slot) {
        const int64_t rb = (int64_t)Dl.np * kPairBytes;
        const int64_t row0 = (int64_t)cl.t * kTileRows + 16 * wave;
        const int64_t off0 = row0 * rb + (int64_t)(cl.c * Dl.P + kSegPairs * cl.jb) * kPairBytes;
        const int64_t bytes = Dl.n * rb;
        const Rsrc rs = make_rsrc(Dl.w + min(off0, bytes), (uint64_t)max(bytes - off0, (int64_t)0));
        const uint32_t dst = ring0 + (uint32_t)(slot * kSlot);
#pragma unroll
        for (int q = 0; q < kLoads - 1; ++q) dma16(rs, (uint32_t)(prow[q] * rb + poff[q]), dst + 1024u * q);
        if (last_live)
            dma16(rs, (uint32_t)(prow[kLoads - 1] * rb + poff[kLoads - 1]), dst + 1024u * (kLoads - 1));
    };

    struct Rec {
        int d, c, t, jb;
    };
    f4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
    uint64_t best[4] = {0, 0, 0, 0};
    int dc = -1, staged_d = -1, staged_c = -1;
    SmDesc Dc;

    // Lane (g, n)'s pairs 2g, 2g+1 of the unit in `slot`, as 20 dwords (pair 0
    // is dwords 0..8, pair 1 dwords 9..15, 18, 19), once the unit's loads are
    // done (`after`: the units whose loads were issued behind it, at most
    // kNB - 1).  The reads have returned when this returns, so the slot may be
    // refilled.
    auto fetch = [&](int slot, uint32_t after, uint32_t (&D)[20]) {
        static_assert(kNB >= 2 && kNB <= 4, "ring depth");
        if (kNB > 3 && after >= 3u)
            wait_vmcnt<(kNB > 3 ? 3 * kLoads : 0)>();
        else if (kNB > 2 && after >= 2u)
            wait_vmcnt<(kNB > 2 ? 2 * kLoads : 0)>();
        else if (after >= 1u)
            wait_vmcnt<kLoads>();
        else
            wait_vmcnt<0>();
        const u4* src = reinterpret_cast<const u4*>(lds + wave * kNB * kSlot + slot * kSlot + l16 * kPitch + 80 * g);
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const u4 v = src[i];
            D[4 * i] = v.x; D[4 * i + 1] = v.y; D[4 * i + 2] = v.z; D[4 * i + 3] = v.w;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };

    auto process = [&](const Rec& r, const uint32_t (&D)[20]) {
        if (r.d != dc) {
            Dc = get(r.d);
            dc = r.d;
        }
        if (r.d != staged_d || r.c != staged_c) {
            __syncthreads();
            stage_range<SWZ, kSegPairs, E::kWaves * 64>(Dc, r.c, m, xs);
            __syncthreads();
            staged_d = r.d;
            staged_c = r.c;
        }
        // A operand rows m >= M only produce product rows that are never
        // stored, so those lanes read activation row M - 1 (an LDS broadcast).
        // Pair 8 jb + 2 g + pp: 8 jb + 2 g is even, so its slot is
        // 8 (8 jb + 2 g) + slot(row, pp, c) in both layouts.
        const int xr = min(l16, m - 1);
        const u4* xu = xs + xr * x_stride<SWZ>(Dc) + 64 * r.jb + 16 * g;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            uint32_t P[9];
#pragma unroll
            for (int i = 0; i < 9; ++i) P[i] = pp == 0 ? D[i] : D[i < 7 ? 9 + i : 11 + i];
            const _Float16 d0 = as_h2(P[0]).x, d1 = as_h2(P[4]).y;
            const h2 s0 = {d0, d0}, s1 = {d1, d1};
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t code = (c == 0) ? realign_block0(P[0], P[4]) : P[c < 4 ? c : c + 1];
                const Codes4 q = expand(code);
                const h2 sc = c < 4 ? s0 : s1;
                u4 bw;
                bw.x = as_u32(q.q0 * sc);
                bw.y = as_u32(q.q1 * sc);
                bw.z = as_u32(q.q2 * sc);
                bw.w = as_u32(q.q3 * sc);
                const u4 ax = xu[x_slot<SWZ>(xr, pp, c)];
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, ax), __builtin_bit_cast(h8, bw),
                                                             acc, 0, 0, 0);
            }
        }
        if (r.jb + 1 == segs_of<kSegPairs>(Dc, r.c)) {  // last segment of the item: store the tile
            // D layout of the 16x16 product: lane (g, l16), element e -> activation row 4g + e, weight row l16
            const int64_t row = (int64_t)r.t * kTileRows + 16 * wave + l16;
            if (row < Dc.n) {
                float* out = Dc.nranges > 1 ? ws + Dc.ws_off + (int64_t)r.c * m * Dc.n : Dc.y;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int mm = 4 * g + e;
                    if (mm < m) {
                        ((g_f32*)out)[(int64_t)mm * Dc.n + row] = acc[e];
                        if (keys) {
                            const uint64_t kk = argmax_key(acc[e], row);
                            best[e] = kk > best[e] ? kk : best[e];
                        }
                    }
                }
            }
            acc = f4v{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };

    // Ring of kNB slots, kNB units in flight while a unit is computed: a
    // unit's pairs are read into registers, its slot is refilled with the unit
    // kNB ahead, and then the unit is computed from the registers.
    Rec RR[kNB];
    bool live[kNB];
    uint32_t n_issued = 0, n_done = 0;
    // The first item's activations are staged before the ring's first loads:
    // staged behind them, their loads' wait would also wait for the units in
    // flight (measured 0.5 % faster on the vocabulary-sized verify GEMM).
    Dc = get(cl.d);
    dc = cl.d;
    stage_range<SWZ, kSegPairs, E::kWaves * 64>(Dc, cl.c, m, xs);
    __syncthreads();
    staged_d = cl.d;
    staged_c = cl.c;
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
        live[i] = have_l;
        if (have_l) {
            RR[i] = Rec{cl.d, cl.c, cl.t, cl.jb};
            issue(i);
            ++n_issued;
            advance_l();
        }
    }
    bool go = true;  // (the first unit always exists)
    while (go) {
#pragma unroll
        for (int i = 0; i < kNB; ++i) {
            if (go) {
                uint32_t D[20];
                fetch(i, n_issued - 1u - n_done, D);
                ++n_done;
                const Rec u = RR[i];
                if (have_l) {
                    RR[i] = Rec{cl.d, cl.c, cl.t, cl.jb};
                    issue(i);
                    ++n_issued;
                    advance_l();
                } else {
                    live[i] = false;
                }
                process(u, D);
                go = live[(i + 1) % kNB];
            }
        }
    }
    if (keys) write_keys<Geo<1>::kWaves>(best, m, keys, lds);
}

struct SmBuf {
    uint32_t d[4][9];  // pairs g, g+4, g+8, g+12 of a 16-pair segment
};

// The register-load engine (M > kLdsMaxM).
template <bool SWZ>
__global__ void __launch_bounds__(Geo<0>::kWaves * 64) k_smallm_reg(const SmDesc* __restrict__ descs, int count,
                                                                     SmDesc one, int m, int64_t total,
                                                                     float* __restrict__ ws, uint64_t* /*keys: M <= 7 only*/) {
    using E = Geo<0>;
    constexpr int kSegPairs = E::kSegPairs, kTileRows = E::kTileRows;
    extern __shared__ u4 xs[];
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int n_desc = descs ? count : 1;
    auto get = [&](int d) -> SmDesc { return descs ? descs[d] : one; };

    const int64_t G = gridDim.x;
    const int64_t c_lo = uniform64((total / G) * blockIdx.x + ((total % G) * blockIdx.x) / G);
    const int64_t c_hi = uniform64((total / G) * (blockIdx.x + 1) + ((total % G) * ((int64_t)blockIdx.x + 1)) / G);
    if (c_lo >= c_hi) return;  // whole workgroup leaves together

    // First item starting at or after c_lo.
    int lo = 0, hi = n_desc - 1;  // last descriptor starting at or before c_lo
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (get(mid).cost_begin <= c_lo) lo = mid; else hi = mid - 1;
    }
    SmCursor cl;
    cl.d = lo;
    cl.jb = 0;
    SmDesc Dl = get(lo);
    {
        const int64_t full = (int64_t)Dl.tiles * (Dl.P / kSegPairs);  // units of a full K-range
        const int64_t o = c_lo - Dl.cost_begin;
        int c = (int)(o / full < Dl.nranges - 1 ? o / full : Dl.nranges - 1);
        const int64_t r = o - c * full;
        const int sg = segs_of<kSegPairs>(Dl, c);
        int64_t t = (r + sg - 1) / sg;
        if (t >= Dl.tiles) {
            t = 0;
            if (++c == Dl.nranges) {
                c = 0;
                if (++cl.d < n_desc) Dl = get(cl.d);
            }
        }
        cl.c = c;
        cl.t = (int)t;
    }
    bool have_l = cl.d < n_desc && item_start<kSegPairs>(Dl, cl.c, cl.t) < c_hi;
    if (!have_l) return;

    auto advance_l = [&]() {
        if (++cl.jb < segs_of<kSegPairs>(Dl, cl.c)) return;
        cl.jb = 0;
        if (++cl.t == Dl.tiles) {
            cl.t = 0;
            if (++cl.c == Dl.nranges) {
                cl.c = 0;
                if (++cl.d >= n_desc) {
                    have_l = false;
                    return;
                }
                Dl = get(cl.d);
            }
        }
        have_l = item_start<kSegPairs>(Dl, cl.c, cl.t) < c_hi;
    };

    auto issue = [&](SmBuf& b) {
        const int64_t row = min((int64_t)cl.t * kTileRows + 16 * wave + l16, Dl.n - 1);
        const uint8_t* wrow = Dl.w + row * (int64_t)Dl.np * kPairBytes;
        const int p0 = cl.c * Dl.P + 16 * cl.jb + g;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int p = min(p0 + 4 * jj, Dl.np - 1);
            load_pair(wrow + (int64_t)p * kPairBytes, b.d[jj]);
        }
    };

    struct Rec {
        int d, c, t, jb;
    };
    f4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
    int dc = -1, staged_d = -1, staged_c = -1;
    SmDesc Dc;

    auto process = [&](const Rec& r, const SmBuf& b) {
        if (r.d != dc) {
            Dc = get(r.d);
            dc = r.d;
        }
        if (r.d != staged_d || r.c != staged_c) {
            __syncthreads();
            stage_range<SWZ, kSegPairs, E::kWaves * 64>(Dc, r.c, m, xs);
            __syncthreads();
            staged_d = r.d;
            staged_c = r.c;
        }
        // A operand rows m >= M only produce product rows that are never
        // stored, so those lanes read activation row M - 1 (an LDS broadcast).
        // Pair 16 jb + g + 4 jj: 16 jb + 4 jj is even, so its slot is
        // 8 (16 jb + 4 jj) + slot(row, g, c) in both layouts.
        const int xr = min(l16, m - 1);
        const u4* xu = xs + xr * x_stride<SWZ>(Dc) + 128 * r.jb;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const _Float16 d0 = as_h2(b.d[jj][0]).x, d1 = as_h2(b.d[jj][4]).y;
            const h2 s0 = {d0, d0}, s1 = {d1, d1};
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t code = (c == 0) ? realign_block0(b.d[jj][0], b.d[jj][4]) : b.d[jj][c < 4 ? c : c + 1];
                const Codes4 q = expand(code);
                const h2 s = c < 4 ? s0 : s1;
                u4 bw;
                bw.x = as_u32(q.q0 * s);
                bw.y = as_u32(q.q1 * s);
                bw.z = as_u32(q.q2 * s);
                bw.w = as_u32(q.q3 * s);
                const u4 ax = xu[32 * jj + x_slot<SWZ>(xr, g, c)];
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, ax), __builtin_bit_cast(h8, bw),
                                                             acc, 0, 0, 0);
            }
        }
        if (r.jb + 1 == segs_of<kSegPairs>(Dc, r.c)) {  // last segment of the item: store the tile
            // D layout of the 16x16 product: lane (g, l16), element e -> activation row 4g + e, weight row l16
            const int64_t row = (int64_t)r.t * kTileRows + 16 * wave + l16;
            if (row < Dc.n) {
                float* out = Dc.nranges > 1 ? ws + Dc.ws_off + (int64_t)r.c * m * Dc.n : Dc.y;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int mm = 4 * g + e;
                    if (mm < m) ((g_f32*)out)[(int64_t)mm * Dc.n + row] = acc[e];
                }
            }
            acc = f4v{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };

    // The other buffer's loads are issued before each unit is computed, also
    // when no unit is left (they then re-read clamped in-range addresses and
    // go unused): with a conditional issue the compiler's wait after the
    // join of the two paths covered the other buffer's loads as well, and a
    // wave then computed each unit with nothing in flight.
    SmBuf A, B;
    Rec ra, rb;
    ra = Rec{cl.d, cl.c, cl.t, cl.jb};
    issue(A);
    advance_l();
    for (;;) {
        bool more = have_l;
        rb = Rec{cl.d, cl.c, cl.t, cl.jb};
        issue(B);
        if (more) advance_l();
        process(ra, A);
        if (!more) break;
        more = have_l;
        ra = Rec{cl.d, cl.c, cl.t, cl.jb};
        issue(A);
        if (more) advance_l();
        process(rb, B);
        if (!more) break;
    }
}

// y[mm][n] = sum over ranges c (in order) of the partials, for every
// descriptor with more than one K-range (blockIdx.y).
__global__ void __launch_bounds__(256) k_sum_ranges(const SmDesc* __restrict__ descs, int count, SmDesc one,
                                                    int m, const float* __restrict__ ws) {
    for (int d = blockIdx.y; d < count; d += gridDim.y) {
        const SmDesc D = descs ? descs[d] : one;
        if (D.nranges < 2) continue;
        const int64_t n_out = (int64_t)m * D.n;
        const float* part = ws + D.ws_off;
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_out; i += (int64_t)gridDim.x * 256) {
            float v = part[i];
            for (int c = 1; c < D.nranges; ++c) v += part[(int64_t)c * n_out + i];
            ((g_f32*)D.y)[i] = v;
        }
    }
}

}  // namespace

// LDS left for the staged activations, rows per tile and pairs per unit of
// the engine that runs m activation rows.
static int sm_xbytes(int64_t m) { return engine_of(m) ? Geo<1>::kXBytes : Geo<0>::kXBytes; }
static int sm_tile_rows(int64_t m) { return engine_of(m) ? Geo<1>::kTileRows : Geo<0>::kTileRows; }
static int sm_seg(int64_t m) { return engine_of(m) ? Geo<1>::kSegPairs : Geo<0>::kSegPairs; }

// Pairs per K-range for m activation rows: the longest run of whole 16-pair
// spans whose activations fit the engine's LDS in the padded layout, or in
// the swizzled one (no padding, a little longer) when that takes fewer ranges.
static int smallm_range_pairs(int64_t k, int64_t m) {
    const int np = (int)(k / 64);
    const int np16 = (np + 15) / 16 * 16;
    const int row_chunks = (int)(sm_xbytes(m) / (16 * m));  // 16-byte chunks per activation row
    const int fit_pad = std::max(16, (row_chunks - 1) / kChunksPerPair / 16 * 16);
    const int fit_swz = std::max(16, row_chunks / kChunksPerPair / 16 * 16);
    if ((np + fit_swz - 1) / fit_swz < (np + fit_pad - 1) / fit_pad) return std::min(fit_swz, np16);
    return std::min(fit_pad, np16);
}

// Fills the derived fields of a descriptor; returns its workspace floats.
int64_t smallm_fill(SmDesc* d, int64_t m, int64_t ws_off, int64_t cost_begin) {
    d->np = (int32_t)(d->k / 64);
    d->P = smallm_range_pairs(d->k, m);
    d->nranges = (d->np + d->P - 1) / d->P;
    d->tiles = (int32_t)((d->n + sm_tile_rows(m) - 1) / sm_tile_rows(m));
    d->cost_begin = cost_begin;
    d->m = (int32_t)m;
    const int64_t floats = d->nranges > 1 ? (int64_t)d->nranges * m * d->n : 0;
    d->ws_off = floats ? ws_off : 0;
    return floats;
}

int64_t smallm_cost(const SmDesc& d) {
    const int seg = sm_seg(d.m);
    int64_t c = 0;
    for (int r = 0; r < d.nranges; ++r) c += (int64_t)d.tiles * ((std::min(d.P, d.np - r * d.P) + seg - 1) / seg);
    return c;
}

size_t smallm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    SmDesc d = {};
    d.n = n;
    d.k = (int32_t)k;
    return (size_t)smallm_fill(&d, m, 0, 0) * sizeof(float);
}

static int smallm_grid(int64_t total) {
    return (int)std::max<int64_t>(1, std::min<int64_t>(total, (int64_t)device_cu_count()));
}

// Staged activations: m rows of max_range_pairs * 8 chunks, plus one chunk of
// padding per row when that still fits the LDS (then the padded layout); the
// LDS-ring engine's rings come first.
static bool smallm_swizzle(int64_t max_range_pairs, int64_t m) {
    return (max_range_pairs * kChunksPerPair + 1) * m * (int64_t)sizeof(u4) > sm_xbytes(m);
}
static size_t smallm_lds(int64_t max_range_pairs, int64_t m) {
    return (size_t)(engine_of(m) ? Geo<1>::kRing : 0) +
           (size_t)(max_range_pairs * kChunksPerPair + (smallm_swizzle(max_range_pairs, m) ? 0 : 1)) * m * sizeof(u4);
}

template <class K>
static hipError_t launch_k(K kern, int threads, const SmDesc* descs, int count, const SmDesc& one, int64_t m,
                           int64_t total, size_t lds, float* ws, uint64_t* keys, hipStream_t s) {
    if (lds > 65536) {
        const hipError_t e = allow_dynamic_lds((const void*)kern, lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(smallm_grid(total)), dim3(threads), lds, s, descs, count, one, (int)m, total, ws,
                       keys);
    return hipGetLastError();
}

static hipError_t launch_sm(const SmDesc* descs, int count, const SmDesc& one, int64_t m, int64_t total,
                            int max_p, float* ws, uint64_t* keys, hipStream_t s) {
    const size_t lds = smallm_lds(max_p, m);
    const bool swz = smallm_swizzle(max_p, m);
    if (engine_of(m)) {
        constexpr int t = Geo<1>::kWaves * 64;
        return swz ? launch_k(k_smallm_lds<true>, t, descs, count, one, m, total, lds, ws, keys, s)
                   : launch_k(k_smallm_lds<false>, t, descs, count, one, m, total, lds, ws, keys, s);
    }
    constexpr int t = Geo<0>::kWaves * 64;
    return swz ? launch_k(k_smallm_reg<true>, t, descs, count, one, m, total, lds, ws, keys, s)
               : launch_k(k_smallm_reg<false>, t, descs, count, one, m, total, lds, ws, keys, s);
}

int smallm_key_slices(int64_t m, int64_t n, int64_t k) {
    SmDesc d = {};
    d.n = n;
    d.k = (int32_t)k;
    smallm_fill(&d, m, 0, 0);
    return d.nranges == 1 && engine_of(m) ? smallm_grid(smallm_cost(d)) : 0;  // the LDS-ring engine only
}

hipError_t launch_gemm_smallm_keys(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n, int64_t k,
                                   uint64_t* keys, hipStream_t s) {
    SmDesc d = {};
    d.w = w;
    d.x = x;
    d.y = y;
    d.n = n;
    d.k = (int32_t)k;
    smallm_fill(&d, m, 0, 0);
    if (d.nranges != 1 || !engine_of(m)) return hipErrorInvalidValue;
    return launch_sm(nullptr, 1, d, m, smallm_cost(d), d.P, nullptr, keys, s);
}

hipError_t launch_gemm_smallm(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n, int64_t k,
                              float* workspace, hipStream_t s) {
    SmDesc d = {};
    d.w = w;
    d.x = x;
    d.y = y;
    d.n = n;
    d.k = (int32_t)k;
    smallm_fill(&d, m, 0, 0);
    const int64_t total = smallm_cost(d);
    hipError_t e = launch_sm(nullptr, 1, d, m, total, d.P, workspace, nullptr, s);
    if (e != hipSuccess || d.nranges < 2) return e;
    const int grid = (int)std::min<int64_t>((m * n + 255) / 256, (int64_t)device_cu_count() * 4);
    hipLaunchKernelGGL(k_sum_ranges, dim3(grid, 1), dim3(256), 0, s, nullptr, 1, d, (int)m, workspace);
    return hipGetLastError();
}

hipError_t launch_gemm_smallm_batch(const SmDesc* descs, int count, int64_t m, int64_t total, int max_p,
                                    int64_t max_mn, bool any_split, float* workspace, hipStream_t s) {
    SmDesc none = {};
    hipError_t e = launch_sm(descs, count, none, m, total, max_p, workspace, nullptr, s);
    if (e != hipSuccess || !any_split) return e;
    const int gx = (int)std::max<int64_t>(1, std::min<int64_t>((max_mn + 255) / 256, 64));
    const int gy = std::min(count, 65535);
    hipLaunchKernelGGL(k_sum_ranges, dim3(gx, gy), dim3(256), 0, s, descs, count, none, (int)m, workspace);
    return hipGetLastError();
}

}  // namespace q4
