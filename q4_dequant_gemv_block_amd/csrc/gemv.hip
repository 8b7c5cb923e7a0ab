// Q4_0 matrix-vector kernels for gfx950: a single GEMV, a list of GEMVs in
// one launch (a whole decode weight sweep), the LM head with greedy argmax,
// and a generic kernel for shapes the fast path does not take.
//
// Decode reads every weight once per token and is bound by memory bandwidth
// ("Every Device Brings a Slice: How SwarmLLM Runs a 27B Model Across Browser
// Tabs", originshq.com, section "The Engine: ~50 WGSL Kernels Written From
// Scratch").  The kernels keep that structure, laid out for CDNA4:
//
//  * 16 lanes (one DPP row) own one weight row; lane l takes block pairs
//    l, l+16, l+32, ... so the 16 lanes of a row read 576 contiguous bytes per
//    step.  Each lane group carries R consecutive rows at the same pair
//    positions, so one read of the activation chunks from LDS serves R rows.
//  * Weights are read with cached global dwordx4/dword loads (36-byte pairs
//    at 4-byte alignment).  The unit's base address is uniform (scalar
//    registers) and every lane adds a fixed 32-bit offset, so issuing loads
//    costs one multiply-add per row and no 64-bit vector arithmetic.
//  * 4-bit codes become exact (code - 8) f16 pairs with one v_and_or_b32 and
//    one v_pk_add_f16 per pair and meet the activations in v_dot2_f32_f16; the
//    block scale is applied once per block in f32 (v_fma_mix).
//  * The activation vector is staged once per workgroup and GEMV into LDS in
//    the chunk order of q4_device.h, at a fixed chunk stride so every LDS read
//    is one base register plus an immediate offset.
//  * Every wave walks a sequence of units (4R rows x JB pairs per lane) and
//    issues the loads of the next unit before computing the current one, also
//    across row groups and GEMV boundaries.
//  * Units at the end of a matrix (rows past N, or K not a multiple of 1024)
//    load from clamped in-range addresses instead of branching per lane:
//    padding pairs meet zero activation chunks and add exactly 0, padding
//    rows are never stored.
//  * The row sum is a fixed-order DPP tree inside the 16-lane row, so results
//    are deterministic and independent of where a row sits.
//
// Work split: a work item is (GEMV d, row step s); it starts at cost
// cost_begin[d] + s * npl[d], npl (pairs per lane) being proportional to its
// bytes.  Workgroup g takes every item starting in [T*g/G, T*(g+1)/G):
// contiguous, byte-balanced ranges, so a workgroup stages few activation
// vectors.  The single-GEMV and LM-head entry points run the same kernel on a
// one-descriptor list passed by value.
#include "q4_device.h"
#include "q4_launch.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace q4 {

// Build-time shape of the engine (defaults measured best on MI355X).
#ifndef Q4_SWEEP_R
#define Q4_SWEEP_R 2
#endif
#ifndef Q4_SWEEP_JB
#define Q4_SWEEP_JB 1
#endif
#ifndef Q4_SWEEP_WG_PER_CU
#define Q4_SWEEP_WG_PER_CU 2
#endif
#ifndef Q4_SWEEP_THREADS
#define Q4_SWEEP_THREADS 512
#endif
#ifndef Q4_SWEEP_WPE
#define Q4_SWEEP_WPE 4
#endif
#ifndef Q4_SWEEP_NB
#define Q4_SWEEP_NB 2
#endif

constexpr int kThreads = Q4_SWEEP_THREADS;  // the waves of a workgroup share one staged activation vector
constexpr int kWaves = kThreads / 64;
constexpr int kWavesPerEu = Q4_SWEEP_WPE;   // register budget: waves per SIMD the sweep kernel must fit
constexpr int kR = Q4_SWEEP_R;              // rows per 16-lane group
constexpr int kJB = Q4_SWEEP_JB;            // pairs per lane per unit
constexpr int kNB = Q4_SWEEP_NB;            // unit buffers in the prefetch ring (2 or 3)
constexpr int kWgPerCu = Q4_SWEEP_WG_PER_CU;
constexpr int kRowsPerStep = kWaves * 4 * kR;
constexpr int kXStride = 288;               // activation chunk stride in pairs: k <= 18432 (36 KiB of LDS)

int batch_rows_per_step() { return kRowsPerStep; }

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
}

// Order-preserving key: larger logit first, then lower index; -0 counts as +0.
__device__ __forceinline__ uint64_t argmax_key(float v, int64_t idx) {
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    if ((u << 1) == 0u) u = 0u;  // -0 -> +0
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}

__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* sh) {
    sh[threadIdx.x] = v;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) {
            const uint64_t o = sh[threadIdx.x + s];
            if (o > sh[threadIdx.x]) sh[threadIdx.x] = o;
        }
        __syncthreads();
    }
    return sh[0];
}

// ---------------------------------------------------------------------------
// The GEMV engine.  A wave's unit is 4R consecutive rows x JB pairs per lane
// (pairs [16*jb, 16*(jb+JB)) of each row); lane group q = lane / 16 owns rows
// q*R .. q*R+R-1 of the unit, lane l = lane % 16 owns pairs l + 16*(jb+t).
// ---------------------------------------------------------------------------
// A wave-uniform 64-bit value moved to scalar registers (64-bit divisions run
// on the vector unit, and a uniform value left in vector registers costs
// registers and, when spilled, a scratch reload that waits on every load).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

struct Cursor {
    int d;       // descriptor
    int64_t s;   // row step within the descriptor
    int jb;      // first pair-per-lane index of the unit
};

template <int R, int JB, int XS>
struct Engine {
    static constexpr int kR = R;
    static constexpr int kJB = JB;
    static constexpr int kWaveLds = 0;
    struct Buf {
        uint32_t d[JB][R][9];
    };
    int lane, l16;
    uint32_t rr0;  // row of this lane's first row within a step (its R rows are rr0 .. rr0+R-1)
    uint32_t l36;  // this lane's byte offset within a 16-pair segment

    __device__ __forceinline__ void init(uint8_t* wl) {
        (void)wl;
        lane = threadIdx.x & 63;
        l16 = lane & 15;
        const int wave = threadIdx.x >> 6;
        rr0 = (uint32_t)(wave * 4 * R + (lane >> 4) * R);
        l36 = (uint32_t)(l16 * kPairBytes);
    }

    __device__ __forceinline__ void issue(const PlanDesc& D, const Cursor& c, Buf& b) const {
        const int np = D.k >> 6;
        const uint32_t rb = (uint32_t)np * kPairBytes;
        const int64_t row0 = c.s * (int64_t)(kWaves * 4 * R);
        const bool interior = row0 + kWaves * 4 * R <= D.n && (np & 15) == 0;  // uniform
        if (interior) {
            const uint8_t* base = D.w + row0 * rb + (int64_t)c.jb * (16 * kPairBytes);
#pragma unroll
            for (int t = 0; t < JB; ++t) {
                if (c.jb + t < D.npl) {  // uniform
#pragma unroll
                    for (int i = 0; i < R; ++i)
                        load_pair(base + ((rr0 + i) * rb + l36 + (uint32_t)t * (16 * kPairBytes)), b.d[t][i]);
                }
            }
        } else {
            // rows and pairs fit 31 bits (the boundary checks n and k)
            const int last_row = (int)(D.n - 1);
            const int r0 = (int)row0 + (int)rr0;
#pragma unroll
            for (int t = 0; t < JB; ++t) {
                const int j = c.jb + t;
                if (j < D.npl) {
                    const uint32_t p = (uint32_t)min(l16 + 16 * j, np - 1);
#pragma unroll
                    for (int i = 0; i < R; ++i) {
                        const uint32_t r = (uint32_t)min(r0 + i, last_row);
                        load_pair(D.w + (uint64_t)r * rb + p * kPairBytes, b.d[t][i]);
                    }
                }
            }
        }
    }

    __device__ __forceinline__ void compute(const PlanDesc& D, const Cursor& c, const u4* __restrict__ xs,
                                            const Buf& b, float (&acc)[R]) const {
        const int stride = XS > 0 ? XS : D.npl * 16;
        const u4* xb = xs + (l16 + 16 * c.jb);
#pragma unroll
        for (int t = 0; t < JB; ++t) {
            if (c.jb + t < D.npl) {
                // chunk-outer, row-inner: one activation chunk is live at a time
                float s0[R], s1[R];
#pragma unroll
                for (int i = 0; i < R; ++i) s0[i] = s1[i] = 0.0f;
#pragma unroll
                for (int ch = 0; ch < 8; ++ch) {
                    const u4 X = xb[ch * stride + 16 * t];
#pragma unroll
                    for (int i = 0; i < R; ++i) {
                        const uint32_t* Dw = b.d[t][i];
                        const uint32_t code = ch == 0 ? realign_block0(Dw[0], Dw[4]) : Dw[ch < 4 ? ch : ch + 1];
                        if (ch < 4)
                            s0[i] = dot_chunk(expand(code), X, s0[i]);
                        else
                            s1[i] = dot_chunk(expand(code), X, s1[i]);
                    }
                }
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    acc[i] = __builtin_fmaf(f16_lo(b.d[t][i][0]), s0[i], acc[i]);
                    acc[i] = __builtin_fmaf(f16_hi(b.d[t][i][4]), s1[i], acc[i]);
                }
            }
        }
    }
};

// The same units loaded as fully coalesced 16-byte pieces with the
// non-temporal hint (each 128-byte line is requested once), parked in a
// wave-private LDS window and read back as 36-byte pairs.  On a load-only
// copy this access pattern streams at 6.6-6.8 TB/s against about 6.15 TB/s
// for per-lane pair loads (which cannot take the non-temporal hint: their
// lines are touched by three instructions and would be refetched).
template <int R, int JB, int XS>
struct CoalEngine {
    static constexpr int kR = R;
    static constexpr int kJB = JB;
    static constexpr int kSegBytes = 16 * kPairBytes * JB;  // one row's part of a unit
    static constexpr int kSegStride = kSegBytes + 32;        // padding staggers LDS banks between rows
    static constexpr int kPieces = kSegBytes / 16 * 4 * R;   // 16-byte pieces per wave unit
    static_assert(kPieces % 32 == 0, "R * JB must be even");
    static constexpr int kPerLane = (kPieces + 63) / 64;     // the last slot may cover half the lanes
    static constexpr int kWaveLds = 4 * R * kSegStride;
    struct Buf {
        u4 v[kPerLane];
    };
    int lane, l16;
    uint32_t rr0;           // row of this lane's first row within a step
    uint32_t wrow0;         // first row of this wave within a step (wave-uniform)
    uint8_t* wl;            // this wave's LDS window
    uint32_t pg[kPerLane];  // row (0 .. 4R-1) of each of this lane's pieces
    uint32_t po[kPerLane];  // byte offset of each piece within its row's segment

    __device__ __forceinline__ void init(uint8_t* window) {
        lane = threadIdx.x & 63;
        l16 = lane & 15;
        const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
        wrow0 = (uint32_t)(wave * 4 * R);
        rr0 = wrow0 + (uint32_t)((lane >> 4) * R);
        wl = window;
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            const int P = 64 * k + lane;
            const int g = P / (kSegBytes / 16);
            pg[k] = (uint32_t)g;
            po[k] = (uint32_t)(16 * (P - g * (kSegBytes / 16)));
        }
    }

    __device__ __forceinline__ bool valid_piece(int k) const { return 64 * k + lane < kPieces; }

    __device__ __forceinline__ void issue(const PlanDesc& D, const Cursor& c, Buf& b) const {
        const int np = D.k >> 6;
        const uint32_t rb = (uint32_t)np * kPairBytes;
        const int64_t row0 = c.s * (int64_t)(kWaves * 4 * R);
        const bool interior = row0 + kWaves * 4 * R <= D.n && (np & 15) == 0;  // uniform
        const int64_t seg0 = (int64_t)c.jb * (16 * kPairBytes);
        if (interior) {
            const uint8_t* base = D.w + (row0 + wrow0) * rb + seg0;
#pragma unroll
            for (int k = 0; k < kPerLane; ++k) {
                const int t = (int)(po[k] / (16 * kPairBytes));
                if (valid_piece(k) && c.jb + t < D.npl)
                    b.v[k] = __builtin_nontemporal_load((g_u4*)(base + (pg[k] * rb + po[k])));
            }
        } else {
            // Rows past N read the last row (never stored).  With k % 1024 != 0 a
            // segment runs past the row end: load dword by dword (a row is a
            // multiple of 4 bytes, so no dword straddles its end) and leave the
            // dwords past it zero; their pairs get zero scales in compute().
            const int last_row = (int)(D.n - 1);
#pragma unroll
            for (int k = 0; k < kPerLane; ++k) {
                const int t = (int)(po[k] / (16 * kPairBytes));
                if (valid_piece(k) && c.jb + t < D.npl) {
                    const uint32_t r = (uint32_t)min((int)(row0 + wrow0 + pg[k]), last_row);
                    const uint32_t off = (uint32_t)seg0 + po[k];
                    const uint8_t* row = D.w + (uint64_t)r * rb;
                    uint32_t dw[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        dw[e] = off + 4u * e < rb ? *(g_u32*)(row + off + 4u * e) : 0u;
                    b.v[k] = u4{dw[0], dw[1], dw[2], dw[3]};
                }
            }
        }
    }

    __device__ __forceinline__ void compute(const PlanDesc& D, const Cursor& c, const u4* __restrict__ xs,
                                            const Buf& b, float (&acc)[R]) const {
#pragma unroll
        for (int k = 0; k < kPerLane; ++k)
            if (valid_piece(k)) *(u4*)(wl + pg[k] * kSegStride + po[k]) = b.v[k];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int stride = XS > 0 ? XS : D.npl * 16;
        const u4* xb = xs + (l16 + 16 * c.jb);
        const uint8_t* mine = wl + (lane >> 4) * R * kSegStride + l16 * kPairBytes;
        const int np = D.k >> 6;
#pragma unroll
        for (int t = 0; t < JB; ++t) {
            if (c.jb + t < D.npl) {
                uint32_t Dw[R][9];
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const uint32_t* src = (const uint32_t*)(mine + i * kSegStride + t * 16 * kPairBytes);
#pragma unroll
                    for (int e = 0; e < 9; ++e) Dw[i][e] = src[e];
                    // a pair past the row end (k % 1024 != 0) holds other bytes: zero its scales
                    if (l16 + 16 * (c.jb + t) >= np) {
                        Dw[i][0] &= 0xFFFF0000u;
                        Dw[i][4] &= 0x0000FFFFu;
                    }
                }
                float s0[R], s1[R];
#pragma unroll
                for (int i = 0; i < R; ++i) s0[i] = s1[i] = 0.0f;
#pragma unroll
                for (int ch = 0; ch < 8; ++ch) {
                    const u4 X = xb[ch * stride + 16 * t];
#pragma unroll
                    for (int i = 0; i < R; ++i) {
                        const uint32_t code = ch == 0 ? realign_block0(Dw[i][0], Dw[i][4]) : Dw[i][ch < 4 ? ch : ch + 1];
                        if (ch < 4)
                            s0[i] = dot_chunk(expand(code), X, s0[i]);
                        else
                            s1[i] = dot_chunk(expand(code), X, s1[i]);
                    }
                }
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    acc[i] = __builtin_fmaf(f16_lo(Dw[i][0]), s0[i], acc[i]);
                    acc[i] = __builtin_fmaf(f16_hi(Dw[i][4]), s1[i], acc[i]);
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
};

__device__ __forceinline__ Cursor next_unit(const PlanDesc& D, Cursor c, int JB) {
    c.jb += JB;
    if (c.jb >= D.npl) {
        c.jb = 0;
        if (++c.s == D.steps) {
            ++c.d;
            c.s = 0;
        }
    }
    return c;
}

template <class E, int NB, int XS, bool ARGMAX>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEu)))
k_sweep(const PlanDesc* __restrict__ descs, int count, PlanDesc one, int64_t total, int xs_bytes,
        uint64_t* __restrict__ keys) {
    extern __shared__ u4 xs[];
    constexpr int R = E::kR;
    constexpr int JB = E::kJB;
    E eng;
    eng.init(reinterpret_cast<uint8_t*>(xs) + xs_bytes + (threadIdx.x >> 6) * E::kWaveLds);
    const int n_desc = descs ? count : 1;
    auto get = [&](int d) -> PlanDesc { return descs ? descs[d] : one; };
    const int64_t G = gridDim.x;
    const int64_t c_lo = uniform64((total / G) * blockIdx.x + ((total % G) * blockIdx.x) / G);
    const int64_t c_hi = uniform64((total / G) * (blockIdx.x + 1) + ((total % G) * ((int64_t)blockIdx.x + 1)) / G);
    auto owned = [&](const PlanDesc& D, const Cursor& c) { return D.cost_begin + c.s * D.npl < c_hi; };

    uint64_t best = 0;
    Cursor cur;
    bool have = c_lo < c_hi;
    PlanDesc D;
    if (have) {
        int lo = 0, hi = n_desc - 1;  // last descriptor starting at or before c_lo
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (get(mid).cost_begin <= c_lo) lo = mid; else hi = mid - 1;
        }
        cur.d = lo;
        D = get(lo);
        cur.s = uniform64((c_lo - D.cost_begin + D.npl - 1) / D.npl);
        cur.jb = 0;
        if (cur.s >= D.steps) {
            cur.d++;
            cur.s = 0;
            have = cur.d < n_desc;
            if (have) D = get(cur.d);
        }
        have = have && owned(D, cur);
    }

    if (have) {
        // A ring of NB unit buffers: unit u is loaded NB-1 steps before it is
        // computed, so every wave keeps NB-1 units of loads in flight.
        typename E::Buf A, B, C;
        float acc[R];
#pragma unroll
        for (int i = 0; i < R; ++i) acc[i] = 0.0f;
        int staged = -1;
        Cursor cl = cur;  // next unit to load
        PlanDesc Dl = D;
        bool have_l = true;
        auto advance_l = [&]() {
            Cursor c2 = next_unit(Dl, cl, JB);
            if (c2.d != cl.d && c2.d < n_desc) Dl = get(c2.d);
            have_l = c2.d < n_desc && owned(Dl, c2);
            cl = c2;
        };
        eng.issue(Dl, cl, A);
        advance_l();
        if (NB == 3 && have_l) {
            eng.issue(Dl, cl, B);
            advance_l();
        }

        // One step: load the next unit into `into` (the buffer computed in the
        // previous step), compute the unit in `now`, finish the row group when
        // its last unit is done.  Returns false after the last unit.
        auto step = [&](typename E::Buf& now, typename E::Buf& into) -> bool {
            if (have_l) {
                eng.issue(Dl, cl, into);
                advance_l();
            }
            if (staged != cur.d) {
                __syncthreads();
                stage_x(D.x, D.k >> 5, D.npl * 16, XS > 0 ? XS : D.npl * 16, xs);
                __syncthreads();
                staged = cur.d;
            }
            eng.compute(D, cur, xs, now, acc);
            if (cur.jb + JB >= D.npl) {  // last unit of this row group
                const int64_t r0 = cur.s * (int64_t)(kWaves * 4 * R) + eng.rr0;
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const float v = row16_sum(acc[i]);
                    acc[i] = 0.0f;
                    if (eng.l16 == 0 && r0 + i < D.n) {
                        ((g_f32*)D.y)[r0 + i] = v;
                        if (ARGMAX) {
                            const uint64_t kk = argmax_key(v, r0 + i);
                            best = kk > best ? kk : best;
                        }
                    }
                }
            }
            Cursor c2 = next_unit(D, cur, JB);
            if (c2.d != cur.d && c2.d < n_desc) D = get(c2.d);
            const bool more = c2.d < n_desc && owned(D, c2);
            cur = c2;
            return more;
        };
        if (NB == 3) {
            for (;;) {
                if (!step(A, C)) break;
                if (!step(B, A)) break;
                if (!step(C, B)) break;
            }
        } else {
            for (;;) {
                if (!step(A, B)) break;
                if (!step(B, A)) break;
            }
        }
    }
    if (ARGMAX) {
        __shared__ uint64_t sh[kThreads];
        const uint64_t b = block_max_u64(best, sh);
        if (threadIdx.x == 0) keys[blockIdx.x] = b;
    }
}

__global__ void __launch_bounds__(kThreads) k_argmax_final(const uint64_t* __restrict__ keys,
                                                           int count, int32_t* __restrict__ token) {
    __shared__ uint64_t sh[kThreads];
    uint64_t best = 0;
    for (int i = threadIdx.x; i < count; i += kThreads) best = keys[i] > best ? keys[i] : best;
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

static int npl_of(int64_t k) { return (int)(((k / 64) + 15) / 16); }

// LDS of the staged activations: the fixed stride when k fits it, else k's own padding.
static bool fixed_stride(int64_t max_k) { return npl_of(max_k) * 16 <= kXStride; }
static size_t x_lds_bytes(int64_t max_k) {
    const int pairs = fixed_stride(max_k) ? kXStride : npl_of(max_k) * 16;
    return (size_t)pairs * kChunksPerPair * sizeof(u4);
}

static PlanDesc single_desc(const uint8_t* w, const uint16_t* x, float* y, int64_t n, int64_t k) {
    PlanDesc d;
    d.w = w;
    d.x = x;
    d.y = y;
    d.n = n;
    d.k = (int32_t)k;
    d.npl = npl_of(k);
    d.steps = (n + kRowsPerStep - 1) / kRowsPerStep;
    d.cost_begin = 0;
    return d;
}

#ifndef Q4_SWEEP_COAL
#define Q4_SWEEP_COAL 0
#endif
template <int XS>
using SweepEngine = typename std::conditional<Q4_SWEEP_COAL != 0, CoalEngine<kR, kJB, XS>, Engine<kR, kJB, XS>>::type;

template <int XS, bool AM>
static hipError_t launch_sweep(const PlanDesc* descs, int count, const PlanDesc& one, int64_t total,
                               int64_t max_k, int64_t max_steps, uint64_t* keys, int grid_cap,
                               int* grid_out, hipStream_t s) {
    using E = SweepEngine<XS>;
    const size_t xsb = x_lds_bytes(max_k);
    const size_t lds = xsb + kWaves * (size_t)E::kWaveLds;
    auto kern = k_sweep<E, kNB, XS, AM>;
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    int grid = (int)std::max<int64_t>(1, std::min<int64_t>(max_steps, (int64_t)device_cu_count() * kWgPerCu));
    grid = std::min(grid, grid_cap);
    if (grid_out) *grid_out = grid;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, s, descs, count, one, total, (int)xsb, keys);
    return hipGetLastError();
}

template <bool AM>
static hipError_t launch_any(const PlanDesc* descs, int count, const PlanDesc& one, int64_t total,
                             int64_t max_k, int64_t max_steps, uint64_t* keys, int grid_cap, int* grid_out,
                             hipStream_t s) {
    if (fixed_stride(max_k))
        return launch_sweep<kXStride, AM>(descs, count, one, total, max_k, max_steps, keys, grid_cap, grid_out, s);
    return launch_sweep<0, AM>(descs, count, one, total, max_k, max_steps, keys, grid_cap, grid_out, s);
}

hipError_t launch_gemv(const uint8_t* w, const uint16_t* x, float* y, int64_t n, int64_t k,
                       hipStream_t s) {
    const PlanDesc d = single_desc(w, x, y, n, k);
    return launch_any<false>(nullptr, 1, d, d.steps * d.npl, k, d.steps, nullptr, INT32_MAX, nullptr, s);
}

int argmax_blocks(int64_t n, int64_t k) {
    (void)k;
    const int64_t steps = (n + kRowsPerStep - 1) / kRowsPerStep;
    return (int)std::min<int64_t>(steps, kArgmaxMaxBlocks);
}

hipError_t launch_lm_head(const uint8_t* w, const uint16_t* h, float* logits, int32_t* token,
                          int64_t n, int64_t k, uint64_t* keys, hipStream_t s) {
    const PlanDesc d = single_desc(w, h, logits, n, k);
    int grid = 0;
    hipError_t e = launch_any<true>(nullptr, 1, d, d.steps * d.npl, k, d.steps, keys, argmax_blocks(n, k), &grid, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_argmax_final, dim3(1), dim3(kThreads), 0, s, keys, grid, token);
    return hipGetLastError();
}

hipError_t launch_gemm_generic(const uint8_t* w, const uint16_t* x, float* y, int64_t m,
                               int64_t n, int64_t k, hipStream_t s) {
    const int64_t grid = (n + 3) / 4;
    hipLaunchKernelGGL(k_gemm_generic, dim3((unsigned)grid), dim3(kGenThreads), 0, s, w, x, y, (int)m,
                       n, k);
    return hipGetLastError();
}

hipError_t launch_gemv_batch(const PlanDesc* descs, int count, int64_t total_cost, int max_k,
                             bool all_k1024, hipStream_t s) {
    (void)all_k1024;
    PlanDesc none = {};
    return launch_any<false>(descs, count, none, total_cost, max_k, INT64_MAX, nullptr, INT32_MAX, nullptr, s);
}

}  // namespace q4
