// Q4_0 matrix-vector kernels for gfx950: a single GEMV, a list of GEMVs in
// one launch (a whole decode weight sweep), the LM head with greedy argmax,
// and a generic kernel for shapes the fast path does not take.
//
// Decode reads every weight once per token and is bound by memory bandwidth
// ("Every Device Brings a Slice: How SwarmLLM Runs a 27B Model Across Browser
// Tabs", originshq.com, section "The Engine: ~50 WGSL Kernels Written From
// Scratch").  The kernels keep that structure, laid out for CDNA4:
//
//  * Weights move from HBM straight into LDS with the non-temporal hint, so
//    no registers hold loads in flight.  For K a multiple of 1024 (the quad
//    engine) four consecutive rows are a whole number of 2304-byte slabs, 18
//    aligned 128-byte lines each, and every line is requested once; other K
//    load 576-byte row segments (the segment engine).  Each wave keeps a ring
//    of units in its own LDS window and waits for a unit with an explicit
//    vmcnt before reading its pairs back.
//  * 4-bit codes become exact (code - 8) f16 pairs with one v_and_or_b32 and
//    one v_pk_add_f16 per pair and meet the activations in v_dot2_f32_f16; the
//    block scale is applied once per block in f32.
//  * The activation vector is staged once per workgroup and GEMV into LDS in
//    the chunk order of q4_device.h, at a fixed chunk stride so every LDS read
//    is one base register plus an immediate offset.
//  * Rows past N are never stored; their loads read zeros (quad engine) or
//    clamped rows (segment engine), and pairs past a row's end get zero scales.
//  * Every row is summed in one fixed association in both engines, so results
//    are deterministic and independent of where a row sits, which engine ran
//    it, or which workgroup computed it.
//
// Work split: a work item is a row step (96 rows in the wide shapes) of one
// GEMV; its cost is proportional to its bytes.  The single GEMV and the LM
// head split their steps statically into byte-balanced contiguous ranges; a
// batch follows the plan's schedule (a static first chunk per workgroup, then
// chunks taken from a shared counter), so workgroups that stream faster take
// more work.
#include "q4_device.h"
#include "q4_launch.h"

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>
#include <vector>

namespace q4 {

// Build-time shape of the engine (defaults measured best on MI355X).
#ifndef Q4_SWEEP_R
#define Q4_SWEEP_R 2
#endif
#ifndef Q4_SWEEP_WG_PER_CU
#define Q4_SWEEP_WG_PER_CU 1
#endif
#ifndef Q4_SWEEP_THREADS
#define Q4_SWEEP_THREADS 768
#endif
#ifndef Q4_SWEEP_WPE
#define Q4_SWEEP_WPE 4
#endif

constexpr int kWavesPerEu = Q4_SWEEP_WPE;   // register budget: waves per SIMD the sweep kernel must fit

// Workgroup shapes of the sweep kernel: waves per workgroup, rows per 16-lane
// group (segment engine), workgroups per CU, and the engine.  A batch and the
// large single GEMVs (LM head) use a wide shape; single GEMVs too small to
// give every CU two wide workgroups use a narrow one.  The quad engine takes
// every list whose k are multiples of 1024 from 4096 up, the segment engine
// the rest.
#ifndef Q4_QUAD_NB
#define Q4_QUAD_NB 2
#endif
constexpr int kQuadNB = Q4_QUAD_NB;  // units per wave in the quad engine's LDS ring
#ifndef Q4_QUAD_TAIL_X4
#define Q4_QUAD_TAIL_X4 0
#endif
#ifndef Q4_SWEEP_FAIR
#define Q4_SWEEP_FAIR 1
#endif
constexpr bool kFairPriority = Q4_SWEEP_FAIR != 0;  // waves behind the workgroup's leader get a higher priority
#ifndef Q4_FAIR_BEFORE_FETCH
#define Q4_FAIR_BEFORE_FETCH 1
#endif
#ifndef Q4_FAIR_EVERY
#define Q4_FAIR_EVERY 4  // units between priority updates (a power of two)
#endif
#ifndef Q4_FAIR_HIGH
#define Q4_FAIR_HIGH 4
#endif
#ifndef Q4_FAIR_MID
#define Q4_FAIR_MID 2
#endif
constexpr bool kFairBeforeFetch = Q4_FAIR_BEFORE_FETCH != 0;  // priority set before the wait for the unit
constexpr int kFairHigh = Q4_FAIR_HIGH, kFairMid = Q4_FAIR_MID;  // lag (units) for priority 3 and 2

struct Shape {
    int waves, r, wg_per_cu;
    bool quad;
    constexpr int rows_per_step() const { return waves * 4 * r; }
};
constexpr Shape kWide = {Q4_SWEEP_THREADS / 64, Q4_SWEEP_R, Q4_SWEEP_WG_PER_CU, false};
constexpr Shape kNarrow = {4, 1, 2, false};
#ifndef Q4_QUAD_R
#define Q4_QUAD_R 2
#endif
#ifndef Q4_QUAD_WAVES
#define Q4_QUAD_WAVES 12
#endif
constexpr Shape kQuadWide = {Q4_QUAD_WAVES, Q4_QUAD_R, 1, true};
constexpr Shape kQuadNarrow = {4, 1, 2, true};
// Wide shapes with 8 waves, for lists and GEMVs whose staged activations (k
// above 24,576) leave too little LDS for the rings of 12 waves.
constexpr Shape kWide8 = {8, Q4_SWEEP_R, 1, false};
constexpr Shape kQuadWide8 = {8, Q4_QUAD_R, 1, true};
// The quad engine with 11 waves, for single wide GEMVs whose 8-row groups
// spread more evenly over 11 waves per workgroup than over 12.
constexpr Shape kQuadWide11 = {11, Q4_QUAD_R, 1, true};
constexpr int kXStride = 288;  // activation chunk stride in pairs: k <= 18432 (36 KiB of LDS)


typedef __attribute__((address_space(1))) float g_f32;

// ---------------------------------------------------------------------------
// Activation staging: the 8 chunks of every block pair, chunk c of pair p at
// xs[c * stride + p]; pairs >= k/64 up to npl*16 are zero.
// ---------------------------------------------------------------------------
template <int HALF>
__device__ __forceinline__ void stage_block(const uint32_t (&v)[16], int p, int stride, u4* __restrict__ xs) {
    auto xe = [&](int j) -> uint32_t { return (v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu; };
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
        int pos[4];
        chunk_positions(4 * HALF + cc, pos);
        const int off = 32 * HALF;
        const int a = pos[0] - off, b = pos[1] - off, c = pos[2] - off, e = pos[3] - off;
        u4 ent;
        ent.x = xe(a) | (xe(c) << 16);
        ent.y = xe(a + 16) | (xe(c + 16) << 16);
        ent.z = xe(b) | (xe(e) << 16);
        ent.w = xe(b + 16) | (xe(e + 16) << 16);
        xs[(4 * HALF + cc) * stride + p] = ent;
    }
}

// Every load of the staging has returned when its loop ends (each value is
// consumed), but the compiler also considers the path on which both branches
// of the chunk layout are skipped and would keep those loads pending into the
// GEMV loop, where it then waited for every outstanding load (the ring's
// included) before each step's LDS reads.  An explicit vmcnt(0) here costs
// nothing and clears that.
__device__ __forceinline__ void staged_loads_done() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ void stage_x(const uint16_t* __restrict__ x, int nblocks, int npairs_pad, int stride,
                        u4* __restrict__ xs) {
    const int nb_pad = 2 * npairs_pad;
    for (int b = threadIdx.x; b < nb_pad; b += blockDim.x) {
        uint32_t v[16];  // the 32 f16 values of block b, two per dword
        if (b < nblocks) {
            g_u4* src = (g_u4*)(x + 32 * (int64_t)b);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u4 t = src[i];
                v[4 * i + 0] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = 0u;
        }
        if (b & 1)
            stage_block<1>(v, b >> 1, stride, xs);
        else
            stage_block<0>(v, b >> 1, stride, xs);
    }
    staged_loads_done();
}

// The final norm before the LM head, applied while the activations are staged
// (the host normalises the hidden state the last stage returns before the LM
// head: "Every Device Brings a Slice", originshq.com, section "The
// Architecture: Layers Distributed, Activations in Flight").  Read as RMS
// normalisation with a per-element gain g: r = 1/sqrt(mean(h^2) + eps),
// x_i = binary16(h_i r g_i), nearest-even.  Every workgroup reads the k values
// of h (L2-resident after the first) and reduces their squares in one fixed
// order (thread t takes blocks t, t + blockDim, ...; butterfly within the
// wave; the waves' partials summed in wave order), so all workgroups stage the
// same x; workgroup 0 also writes x to x_out when that is set.
// The same struct carries the stage hand-off's residual (the epilogue that
// writes binary16(residual + y) in place of y; see k_sweep).
struct NormArgs {
    const uint16_t* gamma;  // g [k], binary16; unused without the norm
    uint16_t* x_out;        // x [k], binary16, or null
    float eps;
    const float* residual;  // hand-off: r [n], binary32, or null (zero)
};

__device__ __forceinline__ float half_lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu)); }
__device__ __forceinline__ float half_hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }
__device__ __forceinline__ uint32_t half_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// Block threadIdx.x of h and of g, loaded once: the sum of squares and the
// scaling both read them from registers.
struct NormHeld {
    uint32_t h[16], g[16];
};

__device__ __forceinline__ void load_block16(const uint16_t* __restrict__ p, int64_t b, uint32_t (&v)[16]) {
    g_u4* src = (g_u4*)(p + 32 * b);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u4 t = src[i];
        v[4 * i + 0] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
}

__device__ __forceinline__ void norm_prefetch(const uint16_t* __restrict__ h, const NormArgs& nm, int k,
                                              NormHeld& held) {
    if ((int)threadIdx.x < (k >> 5)) {
        load_block16(h, threadIdx.x, held.h);
        load_block16(nm.gamma, threadIdx.x, held.g);
    }
}

__device__ __forceinline__ float sum_squares16(const uint32_t (&v)[16], float ss) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float lo = half_lo(v[j]), hi = half_hi(v[j]);
        ss = __builtin_fmaf(lo, lo, ss);
        ss = __builtin_fmaf(hi, hi, ss);
    }
    return ss;
}

// The caller has synchronised the workgroup: xs holds nothing still to be read.
template <int WAVES>
__device__ void stage_x_norm(const uint16_t* __restrict__ h, const NormArgs& nm, const NormHeld& held, int k,
                             int npairs_pad, int stride, u4* __restrict__ xs) {
    const int nblocks = k >> 5;
    float ss = 0.0f;
    if ((int)threadIdx.x < nblocks) ss = sum_squares16(held.h, ss);
    for (int b = threadIdx.x + blockDim.x; b < nblocks; b += blockDim.x) {  // k beyond 32 values per thread
        uint32_t v[16];
        load_block16(h, b, v);
        ss = sum_squares16(v, ss);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    float* part = reinterpret_cast<float*>(xs);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int wv = 0; wv < WAVES; ++wv) tot += part[wv];
    __syncthreads();  // every wave has its total before xs is overwritten
    const float r = 1.0f / __builtin_sqrtf(tot / (float)k + nm.eps);
    const bool write_out = nm.x_out != nullptr && blockIdx.x == 0;

    const int nb_pad = 2 * npairs_pad;
    for (int b = threadIdx.x; b < nb_pad; b += blockDim.x) {
        uint32_t v[16];  // the 32 binary16 values of x in block b, two per dword
        if (b < nblocks) {
            uint32_t hv[16], gv[16];
            if (b == (int)threadIdx.x) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    hv[j] = held.h[j];
                    gv[j] = held.g[j];
                }
            } else {
                load_block16(h, b, hv);
                load_block16(nm.gamma, b, gv);
            }
#pragma unroll
            for (int j = 0; j < 16; ++j)
                v[j] = half_bits(half_lo(hv[j]) * r * half_lo(gv[j])) |
                       (half_bits(half_hi(hv[j]) * r * half_hi(gv[j])) << 16);
            if (write_out) {
                u4* dst = reinterpret_cast<u4*>(nm.x_out + 32 * (int64_t)b);
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i] = u4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = 0u;
        }
        if (b & 1)
            stage_block<1>(v, b >> 1, stride, xs);
        else
            stage_block<0>(v, b >> 1, stride, xs);
    }
    staged_loads_done();
}

// ---------------------------------------------------------------------------
// GEMV engines.  Both keep one contract with the sweep kernel below: a row
// step of a GEMV gives every wave kRowsPerWave consecutive rows, which the
// wave works through in npl units (npl = k/1024 rounded up); `issue` starts
// the loads of a unit into a slot of the wave's LDS ring, `fetch` waits for a
// unit and moves this lane's part of it into registers, `math` accumulates it,
// and `finish` (after the rows' last unit) sums the rows and hands them out.
// ---------------------------------------------------------------------------
// A wave-uniform 64-bit value moved to scalar registers (64-bit divisions run
// on the vector unit, and a uniform value left in vector registers costs
// registers and, when spilled, a scratch reload that waits on every load).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// R rows' pairs (nine dwords each, D[i]) against the activation chunks at
// xb[c * stride]: the two block sums of each pair (s0[i], s1[i], unscaled),
// chunk-outer and row-inner, so one activation chunk is live at a time.
template <int R>
__device__ __forceinline__ void block_sums(const uint32_t (&D)[R][9], const u4* __restrict__ xb, int stride,
                                           float (&s0)[R], float (&s1)[R]) {
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
        const u4 X = xb[ch * stride];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const uint32_t code = ch == 0 ? realign_block0(D[i][0], D[i][4]) : D[i][ch < 4 ? ch : ch + 1];
            if (ch < 4)
                s0[i] = dot_chunk(expand(code), X, ch == 0 ? 0.0f : s0[i]);
            else
                s1[i] = dot_chunk(expand(code), X, ch == 4 ? 0.0f : s1[i]);
        }
    }
}

// One pair into a row accumulator: a = d1 * s1 + (d0 * s0 + a), two roundings,
// with d0 the f16 in the low half of w0 (the pair's first dword) and d1 the
// f16 in the high half of w4 (its fifth).
__device__ __forceinline__ float pair_acc(float a, uint32_t w0, float s0, uint32_t w4, float s1) {
    return fma_hi(w4, s1, fma_lo(w0, s0, a));
}

// Row sums in a fixed association that both engines share.  Pair p of a row
// belongs to class c = (p / 16) % 4 of lane slot p % 16; a class is summed in
// pair order by pair_acc, the four classes as (c0 + c2) + (c1 + c3), and the
// 16 lane slots by row16_sum.  Every row's result thus depends only on its
// own bytes and the activations, not on its position or on the engine.

// s_waitcnt vmcnt(n), the other counters left free.  As asm with a memory
// clobber it is also a compiler barrier: no LDS read of a ring slot moves
// above the wait for that slot's loads.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until this wave's LDS reads have returned (before a slot they read is refilled).
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier for LDS hand-overs only: this wave's LDS accesses are
// complete, then s_barrier.  __syncthreads' release fence would also wait for
// every outstanding load of the wave, the ring's included, and drain it.
__device__ __forceinline__ void lds_barrier() {
    wait_lgkm0();
    asm volatile("s_barrier" ::: "memory");
}

// Wait until a unit's loads are done, given the units issued after it (each
// of at least L load instructions) in a ring of NB slots: at most that many
// times L loads may still be outstanding.  Fewer is always safe.
template <int L, int NB>
__device__ __forceinline__ void wait_unit(uint32_t after) {
    static_assert(NB >= 2 && NB <= 4, "ring depth");
    if (NB > 3 && after >= 3u)
        wait_vmcnt<(NB > 3 ? 3 * L : 0)>();
    else if (NB > 2 && after >= 2u)
        wait_vmcnt<(NB > 2 ? 2 * L : 0)>();
    else if (after >= 1u)
        wait_vmcnt<L>();
    else
        wait_vmcnt<0>();
}

// Fourth dword of a raw buffer descriptor on gfx9 (32-bit data format, no
// swizzle); loads past the descriptor's size return zero.
constexpr int kBufferWord3 = 0x00020000;

// Loads from global memory straight into LDS, non-temporal: lane i's 16 (4)
// bytes land at M0 + 16 i (4 i), M0 being the wave-uniform LDS address of the
// destination.  They are issued through asm, so the compiler does not track
// them: it cannot tell the ring slot being refilled from the one being read,
// and for the builtins it waited for every outstanding load before each
// step's first LDS read, which left one unit per wave in flight instead of
// the ring's NB.  The engines wait for their own loads (explicit vmcnt before
// reading a slot, lgkmcnt(0) after reading it and before refilling it).  The
// loads write no register; the s_nop covers the M0 write just before.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void dma16(const uint8_t* src, uint8_t* dst) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "{m0}"(lds_addr(dst)) : "memory");
}
__device__ __forceinline__ void dma4(const uint8_t* src, uint8_t* dst) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off nt" ::"v"(src), "{m0}"(lds_addr(dst)) : "memory");
}

// Buffer resource of a raw byte buffer (gfx9: base, stride 0, size in bytes,
// 32-bit data format); loads at offsets at or past `bytes` return zeros.
// Every field is wave-uniform.
struct Rsrc {
    u4 w;
};
__device__ __forceinline__ Rsrc make_rsrc(const uint8_t* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    Rsrc r;
    r.w.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r.w.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
    r.w.z = __builtin_amdgcn_readfirstlane(bytes);
    r.w.w = (uint32_t)kBufferWord3;
    return r;
}
// The same buffer moved `step` bytes on (base + step, size - step, at least 0).
__device__ __forceinline__ Rsrc rsrc_advance(Rsrc r, uint32_t step) {
    const uint64_t a = (((uint64_t)(r.w.y & 0xFFFFu)) << 32 | r.w.x) + step;
    r.w.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r.w.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
    r.w.z = __builtin_amdgcn_readfirstlane(r.w.z > step ? r.w.z - step : 0u);
    return r;
}
// 16 (4) bytes per lane at byte offset voff of the buffer into LDS at M0 + 16 i (4 i).
__device__ __forceinline__ void dma16(const Rsrc& r, uint32_t voff, uint8_t* dst) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(r.w), "{m0}"(lds_addr(dst))
                 : "memory");
}
__device__ __forceinline__ void dma4(const Rsrc& r, uint32_t voff, uint8_t* dst) {
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen nt lds" ::"v"(voff), "s"(r.w), "{m0}"(lds_addr(dst))
                 : "memory");
}

// Segment engine, for any k % 64 == 0.  A wave's unit is 4R consecutive rows
// x one segment of 16 pairs (576 bytes) per row; lane group q = lane / 16
// owns rows q*R .. q*R+R-1, lane l = lane % 16 owns pair l of the segment.
// Each row's segment is fetched by one global_load_lds_dwordx4 (36 lanes x 16
// bytes, non-temporal) into the wave's window in LDS, and the lanes read
// their pair (nine dwords) back.  Segments that run past the row end
// (k % 1024 != 0) load only the row's bytes (whole 16-byte pieces, then
// dwords); pairs past the row end have their scales zeroed before use, and
// meet zero activations.  A 128-byte line that straddles two segments of a
// row is requested by both.
template <int WAVES, int R, int XS>
struct DmaEngine {
    static constexpr int kWaves = WAVES;
    static constexpr int kNB = 2;
    static constexpr int kRowsPerWave = 4 * R;
    static constexpr int kLoads = 4 * R;          // load instructions per unit, at least
    static constexpr int kSeg = 16 * kPairBytes;  // 576
    // Row pitch 576 bytes = 144 dwords: lane l of a 16-lane group reads dword 9l + c
    // of its row, and rows 144 dwords apart put the four groups of a wave on
    // disjoint banks (9 is invertible modulo 32 and 64).
    static constexpr int kPitch = kSeg;
    static constexpr int kSlot = 4 * R * kPitch;
    static constexpr int kWaveLds = kNB * kSlot;
    struct Regs {
        uint32_t d[R][9];
    };
    // Per row of the lane, one accumulator per pair class, as separate
    // variables (a run-time class index would move them to memory).
    struct Acc {
        float c0[R], c1[R], c2[R], c3[R];
    };
    int lane, l16;
    uint32_t rr0;    // row of this lane's first row within a step
    uint32_t wrow0;  // first row of this wave within a step
    int64_t rbase = 0;  // first row of row step 0 (a single GEMV's workgroup range)
    uint8_t* wl;     // this wave's window

    // Activations of GEMV D into xs (chunk order of q4_device.h).
    template <class L>
    __device__ static void stage(const L& D, u4* __restrict__ xs) {
        stage_x(D.x, D.k >> 5, D.npl * 16, XS > 0 ? XS : D.npl * 16, xs);
    }
    __device__ __forceinline__ void init(uint8_t* window) {
        lane = threadIdx.x & 63;
        l16 = lane & 15;
        const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
        wrow0 = (uint32_t)(wave * 4 * R);
        rr0 = wrow0 + (uint32_t)((lane >> 4) * R);
        wl = window;
    }
    __device__ __forceinline__ void init_acc(Acc& a) const {
#pragma unroll
        for (int i = 0; i < R; ++i) a.c0[i] = a.c1[i] = a.c2[i] = a.c3[i] = 0.0f;
    }

    // Whether the unit reads clamped rows or a short segment (uniform).
    template <class DS>
    __device__ __forceinline__ bool edge(const DS& D, int s) const {
        return !(rbase + (int64_t)s * (WAVES * 4 * R) + wrow0 + 4 * R <= D.n && ((D.k >> 6) & 15) == 0);
    }

    // Row step being loaded and its next segment.
    const uint8_t* cw;
    int64_t cn;
    int32_t ck, cs, cjb;
    template <class DS>
    __device__ __forceinline__ void begin(const DS& D, int s) {
        cw = D.w;
        cn = D.n;
        ck = D.k;
        cs = s;
        cjb = 0;
    }
    struct Cursor {
        const uint8_t* w;
        int64_t n;
        int32_t k;
    };
    __device__ __forceinline__ void issue(int slot) {
        issue_at(Cursor{cw, cn, ck}, cs, cjb, slot);
        ++cjb;
    }
    template <class DS>
    __device__ __forceinline__ void issue_at(const DS& D, int s, int jb, int slot) const {
        const int np = D.k >> 6;
        const uint32_t rb = (uint32_t)np * kPairBytes;
        const int64_t row0 = rbase + (int64_t)s * (WAVES * 4 * R) + wrow0;
        const uint32_t seg = (uint32_t)jb * kSeg;
        uint8_t* dst = wl + slot * kSlot;
        if (!edge(D, s)) {
            const uint8_t* src = D.w + row0 * rb + seg + 16 * lane;
#pragma unroll
            for (int r = 0; r < 4 * R; ++r)
                if (lane < kSeg / 16) dma16(src + (uint32_t)r * rb, dst + r * kPitch);
        } else {
            // rows past N read the last row (never stored)
            const uint32_t avail = min((uint32_t)kSeg, rb - seg);
            const uint32_t full = avail >> 4, rem = avail & 15;
            const int last_row = (int)(D.n - 1);
#pragma unroll
            for (int r = 0; r < 4 * R; ++r) {
                const uint32_t rr = (uint32_t)min((int)row0 + r, last_row);
                const uint8_t* row = D.w + (uint64_t)rr * rb + seg;
                if ((uint32_t)lane < full) dma16(row + 16 * lane, dst + r * kPitch);
                if ((uint32_t)lane < (rem >> 2)) dma4(row + 16 * full + 4 * lane, dst + r * kPitch + 16 * full);
            }
        }
    }

    // Wait for the unit in `slot` (`after` units were issued behind it), read
    // this lane's pairs from the window into registers, and wait for those
    // reads, so the slot may be refilled.
    template <class DS>
    __device__ __forceinline__ void fetch(const DS& Dp, int s, int jb, int slot, uint32_t after, Regs& W) const {
        wait_unit<kLoads, kNB>(after);
        const uint32_t* p = (const uint32_t*)(wl + slot * kSlot + (rr0 - wrow0) * kPitch + kPairBytes * l16);
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int c = 0; c < 9; ++c) W.d[i][c] = p[i * (kPitch / 4) + c];
        wait_lgkm0();  // the reads are done before the slot is reloaded
        if (edge(Dp, s) && 16 * jb + l16 >= (Dp.k >> 6)) {
#pragma unroll
            for (int i = 0; i < R; ++i) {
                W.d[i][0] &= 0xFFFF0000u;  // d of block 0
                W.d[i][4] &= 0x0000FFFFu;  // d of block 1
            }
        }
    }

    template <class DS>
    __device__ __forceinline__ void math(const DS& Dp, int jb, const u4* __restrict__ xs, const Regs& W,
                                         Acc& acc) const {
        const int stride = XS > 0 ? XS : Dp.npl * 16;
        float s0[R], s1[R];
        block_sums<R>(W.d, xs + (l16 + 16 * jb), stride, s0, s1);
        auto add = [&](float(&a)[R]) {
#pragma unroll
            for (int i = 0; i < R; ++i) a[i] = pair_acc(a[i], W.d[i][0], s0[i], W.d[i][4], s1[i]);
        };
        switch (jb & 3) {  // the pairs' class (uniform)
            case 0: add(acc.c0); break;
            case 1: add(acc.c1); break;
            case 2: add(acc.c2); break;
            default: add(acc.c3); break;
        }
    }

    // After the last unit of row step s: row sums, in a fixed order.
    template <class F>
    __device__ __forceinline__ void finish(int s, Acc& acc, F&& store) const {
        const int64_t r0 = rbase + (int64_t)s * (WAVES * 4 * R) + rr0;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const float v = row16_sum((acc.c0[i] + acc.c2[i]) + (acc.c1[i] + acc.c3[i]));
            acc.c0[i] = acc.c1[i] = acc.c2[i] = acc.c3[i] = 0.0f;
            if (l16 == 0) store(i, r0 + i, v);
        }
    }
};

// Quad engine, for k % 1024 == 0 and k >= 4096 (np = k/64 pairs per row, a
// multiple of 16 and at least 64).  Four consecutive rows are 4*np*36 bytes,
// exactly np/16 slabs of 64 pairs (2304 bytes, 18 lines of 128 bytes).  A
// wave's rows in a row step are R such quads (4R consecutive rows), taken
// slab by slab: a unit is slab t of each of the R quads, three buffer loads
// straight to LDS per slab (64 lanes x 16, 16 and 4 bytes, non-temporal).  Slabs start on 128-byte boundaries relative to the matrix
// start, so no line is requested twice.  Lane j computes pair j of each slab;
// slab t of every quad holds the same pairs of the same quad rows, so the R
// pairs of a lane meet the same activations.  A pair's row is the quad row
// that holds it (a slab meets at most two rows, as np >= 64), and the lane
// adds the pair into its accumulator for that row.  After the quads' last
// slab each quad's four accumulators are summed over the wave.
template <int WAVES, int R, int NB, int XS>
struct QuadEngine {
    static constexpr int kWaves = WAVES;
    static constexpr int kNB = NB;
    static constexpr int kRowsPerWave = 4 * R;
    static constexpr int kLoads = 3 * R;
    static constexpr int kSlab = 64 * kPairBytes;  // 2304
    static constexpr int kSlot = R * kSlab;
    static constexpr int kWaveLds = NB * kSlot;
    struct Regs {
        uint32_t d[R][9];
    };
    // Per quad, the partial sums of the quad's four rows, as separate
    // variables (every index a compile-time constant: a run-time row index
    // would move them to memory).  The slabs add into cur (the row rc) and,
    // in lanes past a row end, nxt (row rc + 1); when row rc is complete its
    // sum moves to its named slot, once per row rather than once per slab.
    struct Acc {
        float a0[R], a1[R], a2[R], a3[R];
        float cur[R], nxt[R];
        int rc;  // quad row of the slab's first pair (uniform)
        int nb;  // first pair of quad row rc + 1, from the quad start (uniform)
    };
    typedef const __attribute__((address_space(3))) uint32_t* lds_u32;
    int lane;
    uint32_t lane16;  // 16 * lane: this lane's byte offset in a chunk row of the activations
    uint32_t wrow0;   // first row of this wave within a step
    int64_t rbase = 0;  // first row of row step 0 (a single GEMV's workgroup range)
    uint8_t* wl;      // this wave's ring
    lds_u32 rd[NB][R];  // this lane's pair in each slot and quad

    // Activations of GEMV D into xs (chunk order of q4_device.h).
    template <class L>
    __device__ static void stage(const L& D, u4* __restrict__ xs) {
        stage_x(D.x, D.k >> 5, D.npl * 16, XS > 0 ? XS : D.npl * 16, xs);
    }
    __device__ __forceinline__ void init(uint8_t* window) {
        lane = threadIdx.x & 63;
        lane16 = (uint32_t)lane * 16u;
        const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
        wrow0 = (uint32_t)(wave * 4 * R);
        wl = window;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < R; ++i) {
                // held in a register of its own: recomputed from one base at
                // every read, the offsets past the paired reads' reach cost
                // vector adds on every unit
                uint32_t a = (uint32_t)(uintptr_t)(window + b * kSlot + i * kSlab + kPairBytes * lane);
                asm volatile("" : "+v"(a));
                rd[b][i] = (lds_u32)(uintptr_t)a;
            }
    }
    __device__ __forceinline__ void init_acc(Acc& a) const {
#pragma unroll
        for (int i = 0; i < R; ++i) a.a0[i] = a.a1[i] = a.a2[i] = a.a3[i] = a.cur[i] = a.nxt[i] = 0.0f;
        a.rc = 0;
        a.nb = 0;
    }

    // A slab is two full-wave loads of 16 bytes per lane and one of 4 bytes
    // per lane (1024 + 1024 + 256 bytes), buffer loads from a descriptor
    // whose base is the slab and whose size ends at the matrix end: the
    // hardware returns zeros past the end (rows past N, never stored), every
    // lane is active, and the per-lane offsets are fixed.
    // Descriptors of each quad's next slab.  A row step computes them once
    // (begin); each issued unit moves them one slab on, so a unit costs a few
    // scalar instructions.  (Scalar work between a unit's arrival and the
    // next loads delays them: 128 dependent scalar instructions per unit cost
    // 2 % of the read rate in a load-only probe of this access pattern.)
    Rsrc cur[R];
    template <class DS>
    __device__ __forceinline__ void begin(const DS& D, int s) {
        const uint64_t rb = (uint32_t)(D.k >> 6) * kPairBytes;
        const uint64_t row0 = (uint64_t)rbase + (uint64_t)s * (WAVES * 4 * R) + wrow0;
        const uint64_t end = (uint64_t)(uint32_t)D.n * rb;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const uint64_t off = (row0 + 4 * i) * rb;
            // bytes left after `off`, clamped to [0, 2^32 - 1] with 32-bit compares
            const int64_t left = (int64_t)(end - off);
            const int32_t hi = (int32_t)((uint64_t)left >> 32);
            const uint32_t nrec = hi < 0 ? 0u : (hi > 0 ? 0xFFFFFFFFu : (uint32_t)left);
            cur[i] = make_rsrc(D.w + off, nrec);
        }
    }
    __device__ __forceinline__ void issue(int slot) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            // The piece offsets ride in the per-lane offset: an instruction
            // offset would move the LDS destination as well.
            uint8_t* dst = wl + slot * kSlot + i * kSlab;
            dma16(cur[i], 16 * lane, dst);
            dma16(cur[i], 1024 + 16 * lane, dst + 1024);
            if (Q4_QUAD_TAIL_X4) {  // the last 256 bytes as 16 lanes x 16 bytes (same LDS layout)
                if (lane < 16) dma16(cur[i], 2048 + 16 * lane, dst + 2048);
            } else {
                dma4(cur[i], 2048 + 4 * lane, dst + 2048);
            }
            cur[i] = rsrc_advance(cur[i], kSlab);
        }
    }

    template <class DS>
    __device__ __forceinline__ void fetch(const DS& Dp, int s, int jb, int slot, uint32_t after, Regs& W) const {
        (void)Dp;
        (void)s;
        (void)jb;
        wait_unit<kLoads, kNB>(after);
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int c = 0; c < 9; ++c) W.d[i][c] = rd[slot][i][c];
        wait_lgkm0();  // the reads are done before the slot is reloaded
    }

    template <class DS>
    __device__ __forceinline__ void math(const DS& Dp, int jb, const u4* __restrict__ xs, const Regs& W,
                                         Acc& acc) const {
        const int np = Dp.k >> 6;
        const int o = 64 * jb;  // first pair of the slab within the quad
        if (jb == 0) {
            acc.rc = 0;
            acc.nb = np;
        }
        const int b = acc.nb - o;  // lanes >= b hold pairs of row rc + 1 (b >= 64: none)
        const bool next = lane >= b;
        // pair within its row, as a byte offset of its activation chunk row:
        // 16 * (o - (nb - np) + lane - (next ? np : 0))
        const uint32_t px = lane16 + (uint32_t)(16 * (o - acc.nb + np)) + (next ? (uint32_t)(-16 * np) : 0u);
        const int stride = XS > 0 ? XS : Dp.npl * 16;
        float s0[R], s1[R];
        block_sums<R>(W.d, (const u4*)((const uint8_t*)xs + px), stride, s0, s1);
        // each lane takes its row's sum, adds the pair and puts it back; one
        // form for slabs inside a row (no lane is past a row end) and slabs
        // across one: a branch between the two left the compiler copying the
        // sums between registers at the join, on every slab
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const float t = pair_acc(next ? acc.nxt[i] : acc.cur[i], W.d[i][0], s0[i], W.d[i][4], s1[i]);
            acc.cur[i] = next ? acc.cur[i] : t;
            acc.nxt[i] = next ? t : acc.nxt[i];
        }
        if (o + 64 >= acc.nb) {  // row rc is complete (a slab ends at most one row)
            auto put = [&](float(&A)[R]) {
#pragma unroll
                for (int i = 0; i < R; ++i) A[i] = acc.cur[i];
            };
            switch (acc.rc) {
                case 0: put(acc.a0); break;
                case 1: put(acc.a1); break;
                case 2: put(acc.a2); break;
                default: put(acc.a3); break;
            }
#pragma unroll
            for (int i = 0; i < R; ++i) {
                acc.cur[i] = acc.nxt[i];
                acc.nxt[i] = 0.0f;
            }
            ++acc.rc;
            acc.nb += np;
        }
    }

    // After the quads' last slab: each row's 64 lane partials summed in a
    // fixed order.  Rows 0|1 and 2|3 are paired across the wave halves, then
    // across 16-lane groups, then summed inside each group, so lane 0, 16, 32
    // and 48 end with rows 0, 2, 1 and 3 of the quad.
    template <class F>
    __device__ __forceinline__ void finish(int s, Acc& acc, F&& store) const {
        const bool h = (lane & 32) != 0;
        const bool g = (lane & 16) != 0;
        const int partner = (lane ^ 32) << 2;
        auto bperm = [&](float v) {
            return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(partner, __builtin_bit_cast(int, v)));
        };
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const float b01 = (h ? acc.a1[i] : acc.a0[i]) + bperm(h ? acc.a0[i] : acc.a1[i]);
            const float b23 = (h ? acc.a3[i] : acc.a2[i]) + bperm(h ? acc.a2[i] : acc.a3[i]);
            const float t = g ? b01 : b23;
            const float sw =
                __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, t), 0x401F));
            const float e = row16_sum((g ? b23 : b01) + sw);
            if ((lane & 15) == 0)
                store(i, rbase + (int64_t)s * (WAVES * 4 * R) + wrow0 + 4 * i + (g ? 2 : 0) + (h ? 1 : 0), e);
        }
    }
};


// Q8_0 slab engine.  A Q8_0 block is an f16 scale then 32 two's-complement
// code bytes (34 bytes; taozi.news, section "支持模型与限制", for the small
// dense models that carry this format); a pair of blocks is 68 bytes, 17
// dwords.  A wave's rows of a row step are 8 consecutive rows (an oct) whose
// 8 np pairs (np = k/64, a multiple of 8) are 8 np / 64 whole slabs of 64
// pairs (4,352 bytes: four 1 KiB loads and one of 16 lanes x 16 bytes; 64
// lanes x 4 bytes measured 0.5 % slower); lane l holds
// pair 64 jb + l of the oct in slab jb, which belongs to oct row
// (64 jb + l) / np.  With np >= 32 a slab holds pairs of at most three rows.
//  * Codes become exact f16 pairs: byte xor 0x80 is code + 128, placed under
//    the exponent byte 0x64 it reads 1024 + code + 128, and 1152 is taken off.
//    Block 0's codes start two bytes into the pair: its first and last two
//    codes share one dword (one v_perm), the others are read as they lie, so
//    no code dword is realigned; the activations are paired to match.
//  * Each lane accumulates its pairs of a row in pair order, block 0 then
//    block 1, each block's dot product chained from zero and scaled by one
//    FMA.  A row's pairs sit in lanes (r np + p) mod 64, a rotation of the
//    row's pair order by a multiple of 8 lanes; the row sum adds lanes l and
//    l + 32, then l and l + 16, then l and l + 8 (pairs of classes that a
//    rotation by 8 lanes maps onto each other), then the 8 lanes of a class
//    slot p % 8 in a fixed tree, so a row's result depends on its own bytes
//    only, wherever it sits.
//  * The activations are staged in natural order: chunk c (halves 8c..8c+7)
//    of pair p at xs[c * stride + p].
// Code dword u (four codes) against x dwords (xa: codes 0,1; xb: codes 2,3).
__device__ __forceinline__ float q8_dot4(uint32_t u, uint32_t xa, uint32_t xb, float s) {
    const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t v = u ^ 0x80808080u;
    const h2 lo = as_h2(__builtin_amdgcn_perm(0x64646464u, v, 0x04010400u)) - bias;
    const h2 hi = as_h2(__builtin_amdgcn_perm(0x64646464u, v, 0x04030402u)) - bias;
    s = __builtin_amdgcn_fdot2(lo, as_h2(xa), s, false);
    return __builtin_amdgcn_fdot2(hi, as_h2(xb), s, false);
}

// One Q8_0 pair (17 dwords D) against its 64 activations (X[c]: halves
// 8c..8c+7): the two blocks' dot products s0, s1, each chained from zero.
// Block 0's codes start two bytes into the pair: its last and first two
// codes share one dword (one v_perm), the others are taken as they lie
// (codes 4d-2 .. 4d+1 in dword d), and each code pair meets the activation
// dword of the same two columns.
__device__ __forceinline__ void q8_pair_sums(const uint32_t (&D)[17], const u4 (&X)[8], float& s0_out,
                                             float& s1_out) {
    float s0 = q8_dot4(__builtin_amdgcn_perm(D[0], D[8], 0x07060100u), X[3].w, X[0].x, 0.0f);
#pragma unroll
    for (int d = 1; d < 8; ++d) {  // x dwords 2d-1 and 2d (halves 4d-2 .. 4d+1)
        const int m0 = 2 * d - 1, m1 = 2 * d;
        s0 = q8_dot4(D[d], X[m0 >> 2][m0 & 3], X[m1 >> 2][m1 & 3], s0);
    }
    float s1 = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d)  // block 1: codes 4d .. 4d+3 in dword 9 + d
        s1 = q8_dot4(D[9 + d], X[4 + (d >> 1)][2 * (d & 1)], X[4 + (d >> 1)][2 * (d & 1) + 1], s1);
    s0_out = s0;
    s1_out = s1;
}
// The pair into a row accumulator: a = d1 s1 + (d0 s0 + a).
__device__ __forceinline__ float q8_pair_acc(const uint32_t (&D)[17], float s0, float s1, float a) {
    return fma_hi(D[8], s1, fma_lo(D[0], s0, a));
}

// The last steps of a Q8_0 row sum: w holds, in each lane l, the row's
// partial over lanes l, l^8, l^16, ... (classes), for class slot l % 8; the 8
// slots of each group of 8 lanes are summed in a fixed tree, the total landing
// in the group's first lane.
__device__ __forceinline__ float q8_slot_tree(float w) {
    float t = w + dpp_mov<0xB1>(w);  // quad_perm [1,0,3,2]
    t = t + dpp_mov<0x4E>(t);        // quad_perm [2,3,0,1]
    return t + dpp_mov<0x104>(t);    // row_shl:4
}

template <int WAVES, int NB, int XS>
struct Q8Engine {
    static constexpr int kWaves = WAVES;
    static constexpr int kNB = NB;
    static constexpr int kRowsPerWave = 8;
    static constexpr int kPair = 68;                 // two 34-byte blocks
    static constexpr int kSlab = 64 * kPair;        // 4352
    static constexpr int kLoads = 5;
    static constexpr int kWaveLds = NB * kSlab;
    struct Regs {
        uint32_t d[17];
    };
    // One accumulator per oct row, as separate variables (compile-time indices only).
    struct Acc {
        float a[8];
        int rc;  // oct row of the slab's first pair (uniform)
        int nb;  // first pair of oct row rc + 1, counted from the oct start (uniform)
    };
    int lane;
    uint32_t wrow0;     // first row of this wave within a step
    int64_t rbase = 0;  // first row of row step 0 (a single GEMV's workgroup range)
    uint8_t* wl;        // this wave's ring
    Rsrc cur;           // the oct's next slab

    __device__ __forceinline__ void init(uint8_t* window) {
        lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
        wrow0 = (uint32_t)(wave * 8);
        wl = window;
    }
    __device__ __forceinline__ void init_acc(Acc& a) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) a.a[i] = 0.0f;
        a.rc = 0;
        a.nb = 0;
    }
    template <class L>
    __device__ static void stage(const L& D, u4* __restrict__ xs) {
        const int stride = XS > 0 ? XS : D.npl * 8;
        const int n = D.k >> 3;  // chunks of 8 halves
        for (int i = threadIdx.x; i < n; i += WAVES * 64) xs[(i & 7) * stride + (i >> 3)] = ((g_u4*)D.x)[i];
        staged_loads_done();
    }
    template <class DS>
    __device__ __forceinline__ void begin(const DS& D, int s) {
        const uint64_t rb = (uint32_t)(D.k >> 6) * (uint64_t)kPair;
        const uint64_t row0 = (uint64_t)rbase + (uint64_t)s * (WAVES * 8) + wrow0;
        const uint64_t end = (uint64_t)(uint32_t)D.n * rb;
        const uint64_t off = row0 * rb;
        const int64_t left = (int64_t)(end - off);
        const int32_t hi = (int32_t)((uint64_t)left >> 32);
        const uint32_t nrec = hi < 0 ? 0u : (hi > 0 ? 0xFFFFFFFFu : (uint32_t)left);
        cur = make_rsrc(D.w + off, nrec);
    }
    __device__ __forceinline__ void issue(int slot) {
        uint8_t* dst = wl + slot * kSlab;
#pragma unroll
        for (int q = 0; q < 4; ++q) dma16(cur, 1024 * q + 16 * lane, dst + 1024 * q);
        if (lane < 16) dma16(cur, 4096 + 16 * lane, dst + 4096);  // the last 256 bytes
        cur = rsrc_advance(cur, kSlab);
    }
    template <class DS>
    __device__ __forceinline__ void fetch(const DS& Dp, int s, int jb, int slot, uint32_t after, Regs& W) const {
        (void)Dp;
        (void)s;
        (void)jb;
        wait_unit<kLoads, kNB>(after);
        typedef const __attribute__((address_space(3))) uint32_t* lds_u32;
        const lds_u32 src = (lds_u32)(wl + slot * kSlab + kPair * lane);
#pragma unroll
        for (int c = 0; c < 17; ++c) W.d[c] = src[c];
        wait_lgkm0();  // the reads are done before the slot is reloaded
    }

    template <class DS>
    __device__ __forceinline__ void math(const DS& Dp, int jb, const u4* __restrict__ xs, const Regs& W,
                                         Acc& acc) const {
        const int np = Dp.k >> 6;
        const int o = 64 * jb;  // first pair of the slab within the oct
        if (jb == 0) {
            acc.rc = 0;
            acc.nb = np;
        }
        const int b1 = acc.nb - o;  // lanes >= b1 hold pairs of row rc + 1 (b1 >= 64: none)
        const int b2 = b1 + np;     // lanes >= b2 hold pairs of row rc + 2
        const int j = (lane >= b1 ? 1 : 0) + (lane >= b2 ? 1 : 0);
        const int p = o + lane - (acc.nb - np) - j * np;  // pair within its row
        const int stride = XS > 0 ? XS : Dp.npl * 8;
        const u4* xb = xs + p;
        u4 X[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) X[c] = xb[c * stride];
        float s0, s1;
        q8_pair_sums(W.d, X, s0, s1);
        auto upd = [&](auto R) {
            constexpr int r = decltype(R)::value;
            if (b1 >= 64) {
                acc.a[r] = q8_pair_acc(W.d, s0, s1, acc.a[r]);
                return;
            }
            float t = acc.a[r];
            if constexpr (r + 1 < 8) t = j == 1 ? acc.a[r + 1] : t;
            if constexpr (r + 2 < 8) t = j == 2 ? acc.a[r + 2] : t;
            t = q8_pair_acc(W.d, s0, s1, t);
            acc.a[r] = j == 0 ? t : acc.a[r];
            if constexpr (r + 1 < 8) acc.a[r + 1] = j == 1 ? t : acc.a[r + 1];
            if constexpr (r + 2 < 8) acc.a[r + 2] = j == 2 ? t : acc.a[r + 2];
        };
        switch (acc.rc) {
            case 0: upd(std::integral_constant<int, 0>{}); break;
            case 1: upd(std::integral_constant<int, 1>{}); break;
            case 2: upd(std::integral_constant<int, 2>{}); break;
            case 3: upd(std::integral_constant<int, 3>{}); break;
            case 4: upd(std::integral_constant<int, 4>{}); break;
            case 5: upd(std::integral_constant<int, 5>{}); break;
            case 6: upd(std::integral_constant<int, 6>{}); break;
            default: upd(std::integral_constant<int, 7>{}); break;
        }
        while (acc.nb <= o + 64) {  // the next slab's first row
            ++acc.rc;
            acc.nb += np;
        }
    }

    // After the oct's last slab: row r of the oct ends in lane 8r.
    template <class F>
    __device__ __forceinline__ void finish(int s, Acc& acc, F&& store) const {
        // Each level keeps half of the rows a lane holds and adds the partner's
        // value of them: lanes 0..31 keep rows 0..3, lanes 32..63 rows 4..7;
        // then, within each half, lanes with bit 4 clear keep the half's rows
        // 0, 1, the others 2, 3.
        const bool b5 = (lane & 32) != 0, b4 = (lane & 16) != 0;
        float u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = (b5 ? acc.a[i + 4] : acc.a[i]) + __shfl_xor(b5 ? acc.a[i] : acc.a[i + 4], 32, 64);
        float v[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) v[i] = (b4 ? u[i + 2] : u[i]) + __shfl_xor(b4 ? u[i] : u[i + 2], 16, 64);
        // bit 3 picks one of the two; the partner is 8 lanes away
        const bool b3 = (lane & 8) != 0;
        const float w = (b3 ? v[1] : v[0]) + dpp_mov<0x128>(b3 ? v[0] : v[1]);  // row_ror:8
        const float t = q8_slot_tree(w);  // lane 8r: the total of row r
#pragma unroll
        for (int i = 0; i < 8; ++i) acc.a[i] = 0.0f;
        if ((lane & 7) == 0) store(0, rbase + (int64_t)s * (WAVES * 8) + wrow0 + (lane >> 3), t);
    }
};

// Rows kernel for single GEMVs too small to fill the engines (whose unit of
// parallelism is a wave's 4R rows of a row step): one wave per row at a time,
// lane l takes pairs l, l + 64, ... of the row (cached 36-byte loads, two
// pairs in flight), the activations staged in LDS as the engines stage them.
// A row gets the engines' association exactly: lane l holds lane slot l % 16
// of class l / 16 (the engines' lanes differ by a rotation of whole 16-lane
// classes, or keep the classes in separate accumulators), its pairs in pair
// order through pair_acc; then lanes l and l + 32 (classes c and c + 2), l and
// l + 16, and the 16 slots by row16_sum.  So a row has the same bits on
// either path, and a single call equals a list's.  With H16 the row is
// written as binary16(residual + y) (the stage hand-off) in place of y.
constexpr int kRowWaves = 8;

template <int XS, bool H16>
__global__ void __launch_bounds__(kRowWaves * 64) k_gemv_rows(const uint8_t* __restrict__ w,
                                                            const uint16_t* __restrict__ x, float* __restrict__ y,
                                                            const float* __restrict__ residual, int64_t n, int k) {
    extern __shared__ u4 xs[];
    const int np = k >> 6;
    const int npl16 = (np + 15) / 16 * 16;
    const int stride = XS > 0 ? XS : npl16;
    stage_x(x, k >> 5, npl16, stride, xs);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int64_t rb = (int64_t)np * kPairBytes;
    const int64_t nwaves = (int64_t)gridDim.x * kRowWaves;
    for (int64_t row = (int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6); row < n; row += nwaves) {
        const uint8_t* wr = w + row * rb;
        float a = 0.0f;
        for (int p0 = lane; p0 < np; p0 += 128) {
            uint32_t D[2][1][9];
#pragma unroll
            for (int u = 0; u < 2; ++u)
                if (p0 + 64 * u < np) load_pair(wr + (int64_t)(p0 + 64 * u) * kPairBytes, D[u][0]);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int p = p0 + 64 * u;
                if (p < np) {
                    float s0[1], s1[1];
                    block_sums<1>(D[u], xs + p, stride, s0, s1);
                    a = pair_acc(a, D[u][0][0], s0[0], D[u][0][4], s1[0]);
                }
            }
        }
        const float b = a + __shfl_xor(a, 32, 64);
        const float e = row16_sum(b + __shfl_xor(b, 16, 64));
        if (lane == 0) {
            if (H16)
                reinterpret_cast<uint16_t*>(y)[row] = (uint16_t)half_bits(residual ? e + residual[row] : e);
            else
                y[row] = e;
        }
    }
}

// The fields of a GEMV the sweep kernel keeps in scalar registers.
struct Live {
    const uint8_t* w;
    const uint16_t* x;
    float* y;
    const float* residual;
    int32_t n, k, npl, steps;
    int64_t cost_begin;
    bool h16;
};

__device__ __forceinline__ Live live_of(const PlanDesc& p) {
    Live l;
    l.w = p.w;
    l.x = p.x;
    l.y = p.y;
    l.n = (int32_t)p.n;
    l.k = p.k;
    l.npl = p.npl;
    l.steps = (int32_t)p.steps;
    l.cost_begin = p.cost_begin;
    l.residual = p.residual;
    l.h16 = p.h16 != 0;
    return l;
}

// The sweep kernel.  A workgroup works through chunks; a chunk is the row
// steps from (d0, s0) on, in list order, that start before cost c_end.
//  * Single GEMV / LM head (BATCH false): one chunk per workgroup, its
//    byte-balanced share [T*g/G, T*(g+1)/G) of the one descriptor `one`.
//  * Batch: chunk g of the plan's schedule first, then further chunks taken
//    from the shared counter head->next as the workgroup runs out of work, so
//    workgroups that stream faster take more.  Chunk ids travel through two
//    LDS slots: at its t-th chunk change the workgroup reads the id of chunk
//    t+1 from q_next[(t+1)&1] and fetches that chunk's entry; in the
//    following step lane 0 takes the id of chunk t+2 from the counter before
//    that step's loads and stores it to q_next[t&1] after its compute, when
//    the atomic has long returned.  The schedule gives every chunk but the
//    list's last at least two units, so chunk changes are at least one step
//    apart.  The last workgroup to finish resets the counters for the next
//    launch.
// Every wave walks the same unit sequence (its own rows of each row step), so
// the barriers of chunk changes and activation staging are reached by all.
// The NB-slot ring of each wave: the slot of the unit being computed is
// refilled once its pairs are read, so NB units are in flight during the math.
template <class E, int XS, bool BATCH, bool ARGMAX, bool NORM, bool H16>
__global__ void __launch_bounds__(E::kWaves * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerEu)))
k_sweep(const PlanDesc* __restrict__ descs, int count, SchedHead* head, const SchedChunk* __restrict__ chunks,
        PlanDesc one, int xs_bytes, uint64_t* __restrict__ keys, NormArgs nrm) {
    constexpr int NB = E::kNB;
    extern __shared__ u4 xs[];
    __shared__ int q_next[2];  // ids of this workgroup's coming chunks (batch schedule)
    __shared__ uint32_t lead;  // most units any wave of the workgroup has started (wave priority)
    if (threadIdx.x == 0) lead = 0;  // (a barrier follows before the first use: chunk setup or staging)
    E eng;
    eng.init(reinterpret_cast<uint8_t*>(xs) + xs_bytes +
             __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) * E::kWaveLds);
    const int n_desc = BATCH ? count : 1;
    PlanDesc one_wg = one;  // a single GEMV: this workgroup's rows (below)
    auto get = [&](int d) -> Live { return live_of(BATCH ? descs[d] : one_wg); };

    // The workgroup's first chunk.
    int cl_d, cl_s, cl_jb;  // next unit to load: descriptor, row step, unit within the step
    int64_t hl;             // end (cost) of the chunk being loaded
    bool have_l;
    Live Dl;
    if (BATCH) {
        const SchedChunk ch = chunks[blockIdx.x];
        cl_d = ch.d0;
        cl_s = ch.s0;
        hl = ch.c_end;
        have_l = true;
    } else {
        // A single GEMV: workgroup g takes the rows of wave-row groups
        // [groups * g / G, groups * (g + 1) / G) (groups of one wave's rows
        // per step), its row steps counted from its first row; rows past its
        // range are neither loaded nor stored.  Whole row steps per
        // workgroup would leave some with one step more than others.
        constexpr int64_t kGroup = E::kRowsPerWave;
        constexpr int64_t kStep = (int64_t)E::kWaves * E::kRowsPerWave;
        const int64_t groups = (one.n + kGroup - 1) / kGroup;
        const int64_t G = gridDim.x;
        const int64_t r0 = uniform64(groups * blockIdx.x / G * kGroup);
        const int64_t r1 = uniform64(min(one.n, groups * ((int64_t)blockIdx.x + 1) / G * kGroup));
        eng.rbase = r0;
        one_wg.n = r1;
        one_wg.steps = (r1 - r0 + kStep - 1) / kStep;
        hl = one_wg.steps * one.npl;
        cl_d = 0;
        cl_s = 0;
        have_l = r1 > r0;
    }
    cl_jb = 0;
    if (have_l) Dl = get(cl_d);

    const int n_static = gridDim.x;
    const int n_chunks = BATCH ? head->nchunks : 0;
    SchedChunk nx;         // entry of the chunk after the one being loaded
    bool nx_ok = false;
    int trans = 0;         // chunk changes so far
    bool grab = false;     // this step takes a chunk id from the counter
    uint32_t pending = 0;  // lane 0: the id taken
    if (BATCH) {
        if (threadIdx.x == 0) {
            q_next[1] = n_static + (int)atomicAdd(&head->next, 1u);
            q_next[0] = n_static + (int)atomicAdd(&head->next, 1u);
        }
        __syncthreads();
        const int id = __builtin_amdgcn_readfirstlane(q_next[1]);
        nx_ok = id < n_chunks;
        if (nx_ok) nx = chunks[id];
    }

    // Move the load cursor one unit on; at the end of a chunk go to the next
    // one (batch) or stop.
    auto advance_l = [&]() {
        if (cl_jb + 1 < Dl.npl) {  // the next unit of the same row step
            ++cl_jb;
            return;
        }
        int d2 = cl_d, s2 = cl_s, jb2 = cl_jb + 1;
        if (jb2 >= Dl.npl) {
            jb2 = 0;
            if (++s2 == Dl.steps) {
                ++d2;
                s2 = 0;
            }
        }
        if (d2 < n_desc) {
            if (d2 != cl_d) Dl = get(d2);
            if (Dl.cost_begin + (int64_t)s2 * Dl.npl < hl) {
                cl_d = d2;
                cl_s = s2;
                cl_jb = jb2;
                return;
            }
        }
        if (!nx_ok) {
            have_l = false;
            return;
        }
        cl_d = nx.d0;
        cl_s = nx.s0;
        cl_jb = 0;
        hl = nx.c_end;
        Dl = get(cl_d);
        ++trans;
        lds_barrier();  // q_next[(trans+1)&1] is written and q_next[trans&1] read by every wave
        const int id = __builtin_amdgcn_readfirstlane(q_next[(trans + 1) & 1]);
        nx_ok = id < n_chunks;
        if (nx_ok) nx = chunks[id];
        grab = true;
    };

    uint64_t best = 0;
    if (have_l) {
        struct Rec {  // a unit in a slot: descriptor (-1: none), row step, unit within the step
            int32_t d, s, jb;
        };
        Rec RR[NB];
        typename E::Acc acc;
        eng.init_acc(acc);
        uint32_t n_issued = 0, n_done = 0;  // units issued, units computed
        int dc = -1;      // descriptor held in Dc (compute side)
        int staged = -1;  // descriptor whose activations are in LDS
        Live Dc;

        auto issue_next = [&](Rec& r, int slot) {
            r.d = cl_d;
            r.s = cl_s;
            r.jb = cl_jb;
            if (cl_jb == 0) eng.begin(Dl, cl_s);  // (every row step starts at unit 0)
            eng.issue(slot);
            ++n_issued;
            advance_l();
        };
        // Among waves of equal priority a SIMD issues the oldest first, so the
        // youngest wave of each SIMD falls behind, and the workgroup's barriers
        // (chunk changes, activation staging) then hold the others, whose rings
        // drain meanwhile.  A wave behind the leader raises its priority by how
        // far it lags.
        auto update_priority = [&]() {
            if (!kFairPriority) return;
            if ((n_done & (Q4_FAIR_EVERY - 1)) != 0) return;
            if ((threadIdx.x & 63) == 0) atomicMax(&lead, n_done);
            const int32_t behind = __builtin_amdgcn_readfirstlane(
                (int)(__hip_atomic_load(&lead, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) - n_done));
            if (behind >= kFairHigh)
                __builtin_amdgcn_s_setprio(3);
            else if (behind >= kFairMid)
                __builtin_amdgcn_s_setprio(2);
            else if (behind >= 1)
                __builtin_amdgcn_s_setprio(1);
            else
                __builtin_amdgcn_s_setprio(0);
        };
        // One step on the unit in (r, slot): take a chunk id if one is owed,
        // stage the activations if the GEMV changed, read the unit's pairs,
        // refill its slot with the next unit to load, compute, store the
        // taken id.  Returns whether the unit after this one (r_next) is loaded.
        auto step = [&](Rec& r, int slot, const Rec& r_next) -> bool {
            const bool took = grab;
            grab = false;
            if (took && threadIdx.x == 0) pending = atomicAdd(&head->next, 1u);
            const Rec u = r;
            if (u.d != dc) {
                Dc = get(u.d);
                dc = u.d;
            }
            if (!NORM && u.d != staged) {  // (with the norm, staged before the first step)
                lds_barrier();  // every wave is done with the previous activations
                E::stage(Dc, xs);
                lds_barrier();
                staged = u.d;
            }
            typename E::Regs W;
            if (kFairBeforeFetch) update_priority();
            eng.fetch(Dc, u.s, u.jb, slot, n_issued - 1u - n_done, W);
            ++n_done;
            if (have_l)
                issue_next(r, slot);
            else
                r.d = -1;
            if (!kFairBeforeFetch) update_priority();
            eng.math(Dc, u.jb, xs, W, acc);
            if (u.jb + 1 >= Dc.npl) {  // last unit of the wave's rows in this step
                eng.finish(u.s, acc, [&](int, int64_t row, float v) {
                    if (row < Dc.n) {
                        if (H16 || (BATCH && Dc.h16)) {
                            // stage hand-off: binary16 (nearest-even) of residual + y, into y's place
                            const float* res = H16 ? nrm.residual : Dc.residual;
                            const float t = res ? v + res[row] : v;
                            reinterpret_cast<uint16_t*>(Dc.y)[row] = (uint16_t)half_bits(t);
                            return;
                        }
                        ((g_f32*)Dc.y)[row] = v;
                        if (ARGMAX) {
                            const uint64_t kk = argmax_key(v, row);
                            best = kk > best ? kk : best;
                        }
                    }
                });
            }
            if (took && threadIdx.x == 0) q_next[trans & 1] = n_static + (int)pending;
            return r_next.d >= 0;
        };
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (have_l)
                issue_next(RR[i], i);
            else
                RR[i].d = -1;
        }
        if constexpr (NORM) {
            // h and g are loaded behind the first weight units, so their wait
            // overlaps the one the first step makes anyway; then the norm is
            // staged once for the whole launch.
            NormHeld held;
            norm_prefetch(one.x, nrm, one.k, held);
            stage_x_norm<E::kWaves>(one.x, nrm, held, one.k, one.npl * 16, XS > 0 ? XS : one.npl * 16, xs);
            __syncthreads();
        }
        bool go = true;
        while (go) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
                if (go) go = step(RR[i], i, RR[(i + 1) % NB]);
        }
    }
    if (BATCH && threadIdx.x == 0) {
        __threadfence();  // this workgroup's grabs are complete
        if (atomicAdd(&head->done, 1u) == gridDim.x - 1) {
            atomicExch(&head->next, 0u);
            atomicExch(&head->done, 0u);
        }
    }
    if (ARGMAX) {
        __shared__ uint64_t sh[E::kWaves];
        const uint64_t b = block_max_u64(best, sh);
        if (threadIdx.x == 0) keys[blockIdx.x] = b;
    }
}

constexpr int kFinalThreads = 256;

__global__ void __launch_bounds__(kFinalThreads) k_argmax_final(const uint64_t* __restrict__ keys,
                                                           int count, int32_t* __restrict__ token) {
    __shared__ uint64_t sh[kFinalThreads / 64];
    uint64_t best = 0;
    for (int i = threadIdx.x; i < count; i += kFinalThreads) best = keys[i] > best ? keys[i] : best;
    const uint64_t b = block_max_u64(best, sh);
    if (threadIdx.x == 0) token[0] = (int32_t)(0xFFFFFFFFu - (uint32_t)(b & 0xFFFFFFFFu));
}

// ---------------------------------------------------------------------------
// Generic path: any k % 32 == 0, rows at 2-byte alignment, 1 <= m <= 16.
// One wave per weight row, lanes stride over blocks, activations from global
// memory; used for shapes the fast kernels do not take.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

constexpr int kGenThreads = 256;  // generic kernel: 4 waves, one row each

__global__ void __launch_bounds__(kGenThreads) k_gemm_generic(const uint8_t* __restrict__ w,
                                                           const uint16_t* __restrict__ x,
                                                           float* __restrict__ y, int m, int64_t n,
                                                           int64_t k) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n) return;  // no barriers in this kernel
    const int64_t nb = k / 32;
    const uint8_t* wr = w + row * nb * kBlockBytes;
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    for (int64_t b = lane; b < nb; b += 64) {
        const uint8_t* blk = wr + b * kBlockBytes;
        const float d = h2f((uint16_t)(blk[0] | (blk[1] << 8)));
        uint8_t codes[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) codes[j] = blk[2 + j];
#pragma unroll
        for (int mm = 0; mm < 16; ++mm) {
            if (mm < m) {
                const uint16_t* xr = x + mm * k + b * 32;
                float s = 0.0f;
#pragma unroll
                for (int j = 0; j < 16; ++j) s = __builtin_fmaf((float)((int)(codes[j] & 15) - 8), h2f(xr[j]), s);
#pragma unroll
                for (int j = 0; j < 16; ++j) s = __builtin_fmaf((float)((int)(codes[j] >> 4) - 8), h2f(xr[16 + j]), s);
                acc[mm] = __builtin_fmaf(d, s, acc[mm]);
            }
        }
    }
#pragma unroll
    for (int mm = 0; mm < 16; ++mm) {
        if (mm < m) {
            float v = acc[mm];
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
            if (lane == 0) y[(int64_t)mm * n + row] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

hipError_t allow_dynamic_lds(const void* kern, size_t bytes) {
    struct Entry {
        const void* kern;
        int dev;
        size_t bytes;
    };
    static std::mutex mu;
    static std::vector<Entry> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry& x : done)
        if (x.kern == kern && x.dev == dev && x.bytes >= bytes) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) done.push_back(Entry{kern, dev, bytes});
    return e;
}

static int npl_of(int64_t k) { return (int)(((k / 64) + 15) / 16); }

// LDS of the staged activations: the fixed stride when k fits it, else k's own padding.
static bool fixed_stride(int64_t max_k) { return npl_of(max_k) * 16 <= kXStride; }
static size_t x_lds_bytes(int64_t max_k) {
    const int pairs = fixed_stride(max_k) ? kXStride : npl_of(max_k) * 16;
    return (size_t)pairs * kChunksPerPair * sizeof(u4);
}

// The wide shape for activations of up to max_k columns: 12 waves when their
// rings fit beside the staged activations in LDS, else 8.
static const Shape& wide_shape(bool quad, int64_t max_k) {
    const size_t ring = quad ? (size_t)QuadEngine<kQuadWide.waves, kQuadWide.r, kQuadNB, 0>::kWaveLds
                             : (size_t)DmaEngine<kWide.waves, kWide.r, 0>::kWaveLds;
    const Shape& w = quad ? kQuadWide : kWide;
    if (x_lds_bytes(max_k) + (size_t)w.waves * ring + 1024 <= 160 * 1024) return w;
    return quad ? kQuadWide8 : kWide8;
}

static PlanDesc single_desc(const uint8_t* w, const uint16_t* x, float* y, int64_t n, int64_t k, const Shape& sh) {
    PlanDesc d;
    d.w = w;
    d.x = x;
    d.y = y;
    d.n = n;
    d.k = (int32_t)k;
    d.npl = npl_of(k);
    d.steps = (n + sh.rows_per_step() - 1) / sh.rows_per_step();
    d.cost_begin = 0;
    d.residual = nullptr;
    d.h16 = 0;
    d.reserved = 0;
    return d;
}

static bool quad_ok(int64_t k) { return k % 1024 == 0 && k >= 4096; }

template <class E, int XS, bool BATCH, bool AM, bool NORM, bool H16>
static hipError_t launch_sweep(const PlanDesc* descs, int count, SchedHead* head, const SchedChunk* chunks,
                               const PlanDesc& one, int64_t max_k, int grid, uint64_t* keys, const NormArgs& nrm,
                               hipStream_t s) {
    const size_t xsb = x_lds_bytes(max_k);
    const size_t lds = xsb + (size_t)E::kWaves * E::kWaveLds;
    auto kern = k_sweep<E, XS, BATCH, AM, NORM, H16>;
    if (lds > 65536) {
        const hipError_t e = allow_dynamic_lds((const void*)kern, lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(E::kWaves * 64), lds, s, descs, count, head, chunks, one, (int)xsb,
                       keys, nrm);
    return hipGetLastError();
}

// The kernel of a shape, for the activation stride max_k needs.
template <class E, class EV, bool BATCH, bool AM, bool NORM, bool H16>
static hipError_t launch_stride(const PlanDesc* descs, int count, SchedHead* head, const SchedChunk* chunks,
                                const PlanDesc& one, int64_t max_k, int grid, uint64_t* keys, const NormArgs& nrm,
                                hipStream_t s) {
    return fixed_stride(max_k)
               ? launch_sweep<E, kXStride, BATCH, AM, NORM, H16>(descs, count, head, chunks, one, max_k, grid, keys,
                                                                  nrm, s)
               : launch_sweep<EV, 0, BATCH, AM, NORM, H16>(descs, count, head, chunks, one, max_k, grid, keys, nrm, s);
}

// A batch (descs, head, chunks) runs on a wide shape; a single GEMV passes
// its descriptor in `one`.
template <bool BATCH, bool AM, bool NORM = false, bool H16 = false>
static hipError_t launch_any(const Shape& sh, const PlanDesc* descs, int count, SchedHead* head,
                             const SchedChunk* chunks, const PlanDesc& one, int64_t max_k, int grid, uint64_t* keys,
                             hipStream_t s, const NormArgs& nrm = NormArgs{nullptr, nullptr, 0.0f, nullptr}) {
    constexpr int W = kWide.waves, WN = kNarrow.waves, R = kWide.r;
    static_assert(!(BATCH && NORM), "the norm prologue belongs to a single LM head");
    static_assert(!(H16 && (BATCH || AM || NORM)), "the hand-off epilogue belongs to a single GEMV");
    if constexpr (!BATCH) {
        if (sh.waves == WN && sh.quad)
            return launch_stride<QuadEngine<WN, 1, 4, kXStride>, QuadEngine<WN, 1, 4, 0>, BATCH, AM, NORM, H16>(
                descs, count, head, chunks, one, max_k, grid, keys, nrm, s);
        if (sh.waves == WN)
            return launch_stride<DmaEngine<WN, kNarrow.r, kXStride>, DmaEngine<WN, kNarrow.r, 0>, BATCH, AM, NORM, H16>(
                descs, count, head, chunks, one, max_k, grid, keys, nrm, s);
    }
    if constexpr (!BATCH) {
        if (sh.waves == kQuadWide11.waves && sh.quad)
            return launch_stride<QuadEngine<kQuadWide11.waves, kQuadWide11.r, kQuadNB, kXStride>,
                                 QuadEngine<kQuadWide11.waves, kQuadWide11.r, kQuadNB, 0>, BATCH, AM, NORM, H16>(
                descs, count, head, chunks, one, max_k, grid, keys, nrm, s);
    }
    if (sh.waves == kQuadWide8.waves && sh.quad)  // k above 24,576: the unfixed stride only
        return launch_sweep<QuadEngine<kQuadWide8.waves, kQuadWide8.r, kQuadNB, 0>, 0, BATCH, AM, NORM, H16>(
            descs, count, head, chunks, one, max_k, grid, keys, nrm, s);
    if (sh.waves == kWide8.waves)
        return launch_sweep<DmaEngine<kWide8.waves, kWide8.r, 0>, 0, BATCH, AM, NORM, H16>(
            descs, count, head, chunks, one, max_k, grid, keys, nrm, s);
    if (sh.quad)
        return launch_stride<QuadEngine<kQuadWide.waves, kQuadWide.r, kQuadNB, kXStride>,
                             QuadEngine<kQuadWide.waves, kQuadWide.r, kQuadNB, 0>,
                             BATCH, AM, NORM, H16>(
            descs, count, head, chunks, one, max_k, grid, keys, nrm, s);
    return launch_stride<DmaEngine<W, R, kXStride>, DmaEngine<W, R, 0>, BATCH, AM, NORM, H16>(
        descs, count, head, chunks, one, max_k, grid, keys, nrm, s);
}

// Workgroups for a static split of `steps` row steps.
static int static_grid(int64_t steps, const Shape& sh, int cap) {
    return (int)std::max<int64_t>(
        1, std::min<int64_t>({steps, (int64_t)device_cu_count() * sh.wg_per_cu, (int64_t)cap}));
}

// Shape for a single GEMV of n rows: the wide one when it gives every CU a
// row step (measured per call, cold weights: 24,576 x 5,120 18.0 us wide
// against 20.3 on the rows kernel, 45,000 x 5,120 28.1 against 31.9; at half
// that, 12,288 rows, 13.7 against 11.6), else the narrow one (which single
// calls replace by the rows kernel).
// The longest wave's share of a single wide GEMV's 8-row groups over the
// average: workgroup g of G takes groups [groups g / G, groups (g + 1) / G)
// and its waves the groups of each row step in turn, so the launch lasts as
// long as the waves with the most groups.
static double wave_imbalance(int64_t n, const Shape& sh) {
    const int64_t steps = (n + sh.rows_per_step() - 1) / sh.rows_per_step();
    const int64_t G = std::max<int64_t>(1, std::min<int64_t>(steps, device_cu_count()));
    const int64_t groups = (n + 4 * sh.r - 1) / (4 * sh.r);
    const int64_t most = ((groups + G - 1) / G + sh.waves - 1) / sh.waves;
    return (double)most * (double)(G * sh.waves) / (double)groups;
}

static const Shape& single_shape(int64_t n, int64_t k) {
    const bool quad = quad_ok(k);
    const Shape& wide = wide_shape(quad, k);
    const int64_t wide_steps = (n + wide.rows_per_step() - 1) / wide.rows_per_step();
    if (wide_steps < (int64_t)device_cu_count()) return quad ? kQuadNarrow : kNarrow;
    // 11 waves when that spreads the groups clearly more evenly (the LM head,
    // 151,936 rows: the busiest wave 1.13 x the average with 12 waves, 1.04
    // with 11; measured 78.6-79.2 against 75.3-75.6 us per call)
    if (&wide == &kQuadWide && wave_imbalance(n, kQuadWide11) < wave_imbalance(n, kQuadWide) - 0.03)
        return kQuadWide11;
    return wide;
}

// Single GEMVs the narrow engine shape would take run on the rows kernel
// (measured per call, cold weights: 17408 x 5120 15.5 against 20.2 us,
// 5120 x 17408 16.7 against 21.3, 5120 x 5120 8.6-9.5 against 9.6).
static bool rows_single(int64_t n, int64_t k) { return &single_shape(n, k) == &kQuadNarrow || &single_shape(n, k) == &kNarrow; }

template <bool H16>
static hipError_t launch_rows(const uint8_t* w, const uint16_t* x, float* y, const float* residual, int64_t n,
                              int64_t k, hipStream_t s) {
    const int64_t wgs = (n + kRowWaves - 1) / kRowWaves;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(wgs, 4 * (int64_t)device_cu_count()));
    const size_t xsb = x_lds_bytes(k);
    if (fixed_stride(k))
        hipLaunchKernelGGL((k_gemv_rows<kXStride, H16>), dim3(grid), dim3(kRowWaves * 64), xsb, s, w, x, y, residual,
                           n, (int)k);
    else
        hipLaunchKernelGGL((k_gemv_rows<0, H16>), dim3(grid), dim3(kRowWaves * 64), xsb, s, w, x, y, residual, n,
                           (int)k);
    return hipGetLastError();
}

hipError_t launch_gemv(const uint8_t* w, const uint16_t* x, float* y, int64_t n, int64_t k,
                       hipStream_t s) {
    if (rows_single(n, k)) return launch_rows<false>(w, x, y, nullptr, n, k, s);
    const Shape& sh = single_shape(n, k);
    const PlanDesc d = single_desc(w, x, y, n, k, sh);
    return launch_any<false, false>(sh, nullptr, 1, nullptr, nullptr, d, k, static_grid(d.steps, sh, INT32_MAX),
                                    nullptr, s);
}

int argmax_blocks(int64_t n, int64_t k) {
    const Shape& sh = single_shape(n, k);
    return static_grid((n + sh.rows_per_step() - 1) / sh.rows_per_step(), sh, kArgmaxMaxBlocks);
}

hipError_t launch_lm_head(const uint8_t* w, const uint16_t* h, float* logits, int32_t* token,
                          int64_t n, int64_t k, uint64_t* keys, hipStream_t s) {
    const Shape& sh = single_shape(n, k);
    const PlanDesc d = single_desc(w, h, logits, n, k, sh);
    const int grid = argmax_blocks(n, k);
    hipError_t e = launch_any<false, true>(sh, nullptr, 1, nullptr, nullptr, d, k, grid, keys, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_argmax_final, dim3(1), dim3(kFinalThreads), 0, s, keys, grid, token);
    return hipGetLastError();
}

// The LM head's per-workgroup keys for callers that cannot allocate device
// memory: one fixed array per device, held until the process ends and shared
// by every such call on that device.  Host code never passes the array's name
// to a kernel (on the host it is a stand-in, not a device address); it uses
// the device address looked up once per device below.
static __device__ __align__(256) uint64_t scratch[kLmHeadScratchKeys];

hipError_t lm_head_scratch(uint64_t** keys) {
    static std::atomic<uint64_t*> addr[64];
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    uint64_t* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(mu);
        p = addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            void* sym = nullptr;
            e = hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch));  // with `dev` current
            if (e != hipSuccess) return e;
            if (!sym) return hipErrorInvalidSymbol;
            p = static_cast<uint64_t*>(sym);
            addr[dev].store(p, std::memory_order_release);
        }
    }
    *keys = p;
    return hipSuccess;
}

hipError_t launch_lm_head_norm(const uint8_t* w, const uint16_t* h, const uint16_t* gamma, float eps,
                               uint16_t* x_out, float* logits, int32_t* token, int64_t n, int64_t k, uint64_t* keys,
                               hipStream_t s) {
    const Shape& sh = single_shape(n, k);
    const PlanDesc d = single_desc(w, h, logits, n, k, sh);
    const int grid = argmax_blocks(n, k);
    hipError_t e = launch_any<false, true, true>(sh, nullptr, 1, nullptr, nullptr, d, k, grid, keys, s,
                                                 NormArgs{gamma, x_out, eps, nullptr});
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_argmax_final, dim3(1), dim3(kFinalThreads), 0, s, keys, grid, token);
    return hipGetLastError();
}

hipError_t launch_gemv_handoff(const uint8_t* w, const uint16_t* x, const float* residual, uint16_t* h16,
                               int64_t n, int64_t k, hipStream_t s) {
    if (rows_single(n, k)) return launch_rows<true>(w, x, reinterpret_cast<float*>(h16), residual, n, k, s);
    const Shape& sh = single_shape(n, k);
    const PlanDesc d = single_desc(w, x, reinterpret_cast<float*>(h16), n, k, sh);
    return launch_any<false, false, false, true>(sh, nullptr, 1, nullptr, nullptr, d, k,
                                                 static_grid(d.steps, sh, INT32_MAX), nullptr, s,
                                                 NormArgs{nullptr, nullptr, 0.0f, residual});
}

hipError_t launch_gemm_generic(const uint8_t* w, const uint16_t* x, float* y, int64_t m,
                               int64_t n, int64_t k, hipStream_t s) {
    const int64_t grid = (n + 3) / 4;
    hipLaunchKernelGGL(k_gemm_generic, dim3((unsigned)grid), dim3(kGenThreads), 0, s, w, x, y, (int)m,
                       n, k);
    return hipGetLastError();
}

// Schedule of a batch.  The list is reordered (larger row steps first, list
// order kept otherwise); row steps are then taken in that order and grouped into
// atoms of at least two units (a step of one unit, k <= 1024, is paired with
// the next), so a chunk made of whole atoms has at least two units, as the
// kernel's chunk-id hand-over requires.  The first `grid` chunks (one per
// workgroup, assigned statically) cover about kStaticShare of the work in
// equal parts; the rest is cut into chunks of about remaining / (3 * grid)
// (guided self-scheduling), at least one atom each, which workgroups take
// from the shared counter as they run out of work.  Depends only on the
// shapes and the device's CU count.
#ifndef Q4_SCHED_STATIC
#define Q4_SCHED_STATIC 0.6
#endif
#ifndef Q4_SCHED_DIV
#define Q4_SCHED_DIV 3
#endif
static constexpr double kStaticShare = Q4_SCHED_STATIC;
static constexpr int kGuidedDiv = Q4_SCHED_DIV;  // dynamic chunks: remaining / (kGuidedDiv * grid)

// The schedule of a list whose row steps have `rows_per_step` rows and whose
// GEMV of width k takes npl(k) units per wave and row step; returns the grid.
static int schedule_list(PlanDesc* descs, int count, int rows_per_step, int wg_per_cu, int (*npl)(int64_t),
                         std::vector<SchedChunk>* out) {
    // GEMVs with more units per row step first: the chunks handed out last
    // are then the shortest, and so is the wait for the last workgroup.
    std::stable_sort(descs, descs + count,
                     [npl](const PlanDesc& a, const PlanDesc& b) { return npl(a.k) > npl(b.k); });
    struct Atom {
        int32_t d, s;
        int64_t cost;  // start cost of its first step
    };
    std::vector<Atom> atoms;
    int64_t total = 0;
    int open_units = 2;  // units of the last atom
    for (int i = 0; i < count; ++i) {
        PlanDesc& p = descs[i];
        p.npl = npl(p.k);
        p.steps = (p.n + rows_per_step - 1) / rows_per_step;
        p.cost_begin = total;
        const int units = p.npl;  // one unit per 16 pairs of a row
        for (int64_t st = 0; st < p.steps; ++st) {
            if (open_units >= 2) {
                atoms.push_back(Atom{i, (int32_t)st, total + st * p.npl});
                open_units = 0;
            }
            open_units += units;
        }
        total += p.steps * p.npl;
    }
    if (open_units < 2 && atoms.size() > 1) atoms.pop_back();  // a lone one-unit step joins the atom before it
    const int64_t n_atoms = (int64_t)atoms.size();
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(n_atoms, (int64_t)device_cu_count() * wg_per_cu));
    out->clear();
    int64_t a = 0;
    auto cost_at = [&](int64_t i) { return i < n_atoms ? atoms[i].cost : total; };
    for (int g = 0; g < grid; ++g) {
        out->push_back(SchedChunk{atoms[a].d, atoms[a].s, 0});
        const int64_t end = (int64_t)(kStaticShare * (double)total * (g + 1) / grid);
        ++a;
        while (n_atoms - a > grid - 1 - g && cost_at(a) < end) ++a;
    }
    while (a < n_atoms) {
        out->push_back(SchedChunk{atoms[a].d, atoms[a].s, 0});
        const int64_t size =
            std::max<int64_t>(1, (total - cost_at(a) + kGuidedDiv * grid - 1) / (kGuidedDiv * (int64_t)grid));
        const int64_t end = cost_at(a) + size;
        ++a;
        while (a < n_atoms && cost_at(a) < end) ++a;
    }
    for (size_t i = 0; i + 1 < out->size(); ++i) {
        const SchedChunk& nx = (*out)[i + 1];
        (*out)[i].c_end = descs[nx.d0].cost_begin + (int64_t)nx.s0 * descs[nx.d0].npl;
    }
    out->back().c_end = total;
    return grid;
}

void build_schedule(PlanDesc* descs, int count, std::vector<SchedChunk>* out, int* grid_out, int* flags_out) {
    bool quad = true;
    int64_t max_k = 0;
    for (int i = 0; i < count; ++i) {
        quad = quad && quad_ok(descs[i].k);
        max_k = std::max<int64_t>(max_k, descs[i].k);
    }
    const Shape& sh = wide_shape(quad, max_k);
    *grid_out = schedule_list(descs, count, sh.rows_per_step(), sh.wg_per_cu, npl_of, out);
    *flags_out = (quad ? kPlanQuad : 0) | (sh.waves == kWide8.waves ? kPlanWide8 : 0);
}

hipError_t launch_gemv_batch(const void* plan, int count, int nchunks, int grid, int max_k, int flags,
                             hipStream_t s) {
    (void)nchunks;
    const uint8_t* base = static_cast<const uint8_t*>(plan);
    SchedHead* head = (SchedHead*)base;
    const PlanDesc* descs = (const PlanDesc*)(base + sizeof(SchedHead));
    const SchedChunk* chunks = (const SchedChunk*)(base + sizeof(SchedHead) + (size_t)count * sizeof(PlanDesc));
    PlanDesc none = {};
    const Shape& sh = (flags & kPlanWide8) ? ((flags & kPlanQuad) ? kQuadWide8 : kWide8)
                                           : ((flags & kPlanQuad) ? kQuadWide : kWide);
    return launch_any<true, false>(sh, descs, count, head, chunks, none, max_k,
                                   grid, nullptr, s);
}

// Q8_0 rows kernel, for single GEMVs too small to fill the slab engine
// (whose parallelism is one 8-row group per wave): one wave per row at a
// time, lane l takes pairs l, l + 64, ... of the row, two pairs' loads in
// flight, the activations staged in LDS as the slab engine stages them.  A
// row gets the slab engine's association exactly: lane p mod 64 holds pair p
// (the engine's lanes are the same up to a rotation by a multiple of 8, which
// the tree below does not see), the same per-pair arithmetic in pair order,
// the same lane tree.  Either kernel gives a row the same bits.
constexpr int kQ8RowWaves = 8;

__device__ __forceinline__ void load_q8_pair(const uint8_t* p, uint32_t (&D)[17]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u4a4 v = *(g_u4a4*)(p + 16 * i);
        D[4 * i] = v.x; D[4 * i + 1] = v.y; D[4 * i + 2] = v.z; D[4 * i + 3] = v.w;
    }
    D[16] = *(g_u32*)(p + 64);
}

__global__ void __launch_bounds__(kQ8RowWaves * 64) k_q8_rows(const uint8_t* __restrict__ w,
                                                            const uint16_t* __restrict__ x, float* __restrict__ y,
                                                            int64_t n, int k) {
    extern __shared__ u4 xs[];  // chunk c of pair p at xs[c * np + p]
    const int np = k >> 6;
    for (int i = threadIdx.x; i < (k >> 3); i += blockDim.x) xs[(i & 7) * np + (i >> 3)] = ((g_u4*)x)[i];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int64_t rb = (int64_t)np * 68;
    const int64_t nwaves = (int64_t)gridDim.x * kQ8RowWaves;
    for (int64_t row = (int64_t)blockIdx.x * kQ8RowWaves + (threadIdx.x >> 6); row < n; row += nwaves) {
        const uint8_t* wr = w + row * rb;
        float a = 0.0f;
        for (int p0 = lane; p0 < np; p0 += 128) {
            uint32_t D[2][17];
#pragma unroll
            for (int u = 0; u < 2; ++u)
                if (p0 + 64 * u < np) load_q8_pair(wr + 68 * (int64_t)(p0 + 64 * u), D[u]);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int p = p0 + 64 * u;
                if (p < np) {
                    u4 X[8];
#pragma unroll
                    for (int c = 0; c < 8; ++c) X[c] = xs[c * np + p];
                    float s0, s1;
                    q8_pair_sums(D[u], X, s0, s1);
                    a = q8_pair_acc(D[u], s0, s1, a);
                }
            }
        }
        a = a + __shfl_xor(a, 32, 64);
        a = a + __shfl_xor(a, 16, 64);
        a = a + __shfl_xor(a, 8, 64);
        const float t = q8_slot_tree(a);
        if (lane == 0) y[row] = t;
    }
}

// ---------------------------------------------------------------------------
// Q8_0 on the sweep kernel (Q8Engine): a single GEMV and a list.
// ---------------------------------------------------------------------------
#ifndef Q4_Q8_XS
#define Q4_Q8_XS 448
#endif
constexpr int kQ8XStride = Q4_Q8_XS;  // activation chunk stride in pairs: k <= 64 * stride
// 8 waves with three slabs in flight each (measured over the Qwen3-4B-shaped
// list: 12 x 2 slots 0.78, 8 x 3 0.82-0.83, 9 x 3 and 10 x 3 with a smaller
// activation stride 0.78, 6 x 4 0.74 of 8 TB/s).
#ifndef Q4_Q8_WAVES
#define Q4_Q8_WAVES 8
#endif
#ifndef Q4_Q8_NB
#define Q4_Q8_NB 3
#endif
using Q8Wide = Q8Engine<Q4_Q8_WAVES, Q4_Q8_NB, kQ8XStride>;
constexpr int kQ8WideRows = Q8Wide::kWaves * 8;  // rows per row step

bool q8_slab_ok(int64_t k) { return k % 512 == 0 && k >= 2048 && k <= 64 * (int64_t)kQ8XStride; }
static int q8_npl(int64_t k) { return (int)(k / 512); }  // slabs of a wave's 8 rows

template <class E, int XS, bool BATCH>
static hipError_t launch_q8_sweep(const PlanDesc* descs, int count, SchedHead* head, const SchedChunk* chunks,
                                  const PlanDesc& one, int64_t max_k, int grid, hipStream_t s) {
    const size_t xsb = (size_t)(XS > 0 ? XS : max_k / 64) * kChunksPerPair * sizeof(u4);
    const size_t lds = xsb + (size_t)E::kWaves * E::kWaveLds;
    auto kern = k_sweep<E, XS, BATCH, false, false, false>;
    if (lds > 65536) {
        const hipError_t e = allow_dynamic_lds((const void*)kern, lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(E::kWaves * 64), lds, s, descs, count, head, chunks, one, (int)xsb,
                       nullptr, NormArgs{nullptr, nullptr, 0.0f, nullptr});
    return hipGetLastError();
}

// A single GEMV: the slab engine when it gives every CU two workgroups' row
// steps, else the rows kernel (the same bits either way).
hipError_t launch_q8_slab_gemv(const uint8_t* w, const uint16_t* x, float* y, int64_t n, int64_t k, hipStream_t s) {
    const int cus = device_cu_count();
    if ((n + kQ8WideRows - 1) / kQ8WideRows >= 2 * (int64_t)cus) {
        PlanDesc d = {};
        d.w = w;
        d.x = x;
        d.y = y;
        d.n = n;
        d.k = (int32_t)k;
        d.npl = q8_npl(k);
        d.steps = (n + kQ8WideRows - 1) / kQ8WideRows;
        const int grid = (int)std::min<int64_t>(d.steps, cus);
        return launch_q8_sweep<Q8Wide, kQ8XStride, false>(nullptr, 1, nullptr, nullptr, d, k, grid, s);
    }
    const int64_t wgs = (n + kQ8RowWaves - 1) / kQ8RowWaves;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(wgs, 2 * (int64_t)cus));
    hipLaunchKernelGGL(k_q8_rows, dim3(grid), dim3(kQ8RowWaves * 64), (size_t)k * 2, s, w, x, y, n, (int)k);
    return hipGetLastError();
}

int build_schedule_q8(PlanDesc* descs, int count, std::vector<SchedChunk>* out) {
    return schedule_list(descs, count, kQ8WideRows, 1, q8_npl, out);
}

hipError_t launch_q8_slab_batch(const void* plan, int count, int grid, hipStream_t s) {
    const uint8_t* base = static_cast<const uint8_t*>(plan);
    SchedHead* head = (SchedHead*)base;
    const PlanDesc* descs = (const PlanDesc*)(base + sizeof(SchedHead));
    const SchedChunk* chunks = (const SchedChunk*)(base + sizeof(SchedHead) + (size_t)count * sizeof(PlanDesc));
    PlanDesc none = {};
    return launch_q8_sweep<Q8Wide, kQ8XStride, true>(descs, count, head, chunks, none, 64 * kQ8XStride, grid, s);
}

}  // namespace q4
