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
//    l, l+16, l+32, ...; a wave's unit is 4 rows x one 576-byte segment
//    (16 pairs) per row.
//  * Weights move from HBM straight into LDS: one global_load_lds_dwordx4 per
//    row segment, 36 lanes x 16 contiguous bytes with the non-temporal hint,
//    so every 128-byte line is requested once and no registers hold loads in
//    flight.  Each wave keeps a ring of units in its own LDS window and waits
//    for a unit with an explicit vmcnt before reading its pairs back.
//  * 4-bit codes become exact (code - 8) f16 pairs with one v_and_or_b32 and
//    one v_pk_add_f16 per pair and meet the activations in v_dot2_f32_f16; the
//    block scale is applied once per block in f32 (v_fma_mix).
//  * The activation vector is staged once per workgroup and GEMV into LDS in
//    the chunk order of q4_device.h, at a fixed chunk stride so every LDS read
//    is one base register plus an immediate offset.
//  * Units at the end of a matrix (rows past N, or K not a multiple of 1024)
//    read clamped rows and only the bytes of the row; pairs past the row end
//    get zero scales and meet zero activations, padding rows are never stored.
//  * The row sum is a fixed-order DPP tree inside the 16-lane row, so results
//    are deterministic and independent of where a row sits or which
//    workgroup computed it.
//
// Work split: a work item is a row step (64 rows) of one GEMV; its cost is
// proportional to its bytes.  The single GEMV and the LM head split their
// steps statically into byte-balanced contiguous ranges; a batch follows the
// plan's schedule (a static first chunk per workgroup, then chunks taken from
// a shared counter), so workgroups that stream faster take more work.
#include "q4_device.h"
#include "q4_launch.h"

#include <algorithm>
#include <atomic>
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
#ifndef Q4_SWEEP_NB
#define Q4_SWEEP_NB 2
#endif

constexpr int kWavesPerEu = Q4_SWEEP_WPE;   // register budget: waves per SIMD the sweep kernel must fit
constexpr int kNB = Q4_SWEEP_NB;            // units per wave in the LDS ring (2)

// Workgroup shapes of the sweep kernel: waves per workgroup, rows per 16-lane
// group, workgroups per CU.  The batch and the large single GEMVs (LM head)
// use the wide shape; single GEMVs too small to give every CU two wide
// workgroups use the narrow one (16 rows per step instead of 96).
struct Shape {
    int waves, r, wg_per_cu;
    constexpr int rows_per_step() const { return waves * 4 * r; }
};
constexpr Shape kWide = {Q4_SWEEP_THREADS / 64, Q4_SWEEP_R, Q4_SWEEP_WG_PER_CU};
constexpr Shape kNarrow = {4, 1, 2};
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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o);
        const uint64_t t = ((uint64_t)hi << 32) | lo;
        v = t > v ? t : v;
    }
    return v;
}

// Maximum over the workgroup; sh holds one entry per wave.
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* sh) {
    v = wave_max_u64(v);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    uint64_t r = 0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r = sh[i] > r ? sh[i] : r;
    return r;
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

// R rows' pairs (nine dwords each, D[i]) against the activation chunks at
// xb[c * stride], accumulated into acc[i]: chunk-outer, row-inner, so one
// activation chunk is live at a time; the block sums are scaled once each.
template <int R>
__device__ __forceinline__ void rows_dot(const uint32_t (&D)[R][9], const u4* __restrict__ xb, int stride,
                                         float (&acc)[R]) {
    float s0[R], s1[R];
#pragma unroll
    for (int i = 0; i < R; ++i) s0[i] = s1[i] = 0.0f;
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
        const u4 X = xb[ch * stride];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const uint32_t code = ch == 0 ? realign_block0(D[i][0], D[i][4]) : D[i][ch < 4 ? ch : ch + 1];
            if (ch < 4)
                s0[i] = dot_chunk(expand(code), X, s0[i]);
            else
                s1[i] = dot_chunk(expand(code), X, s1[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        acc[i] = __builtin_fmaf(f16_lo(D[i][0]), s0[i], acc[i]);
        acc[i] = __builtin_fmaf(f16_hi(D[i][4]), s1[i], acc[i]);
    }
}

// s_waitcnt vmcnt(n) with the other counters left free (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

typedef __attribute__((address_space(1))) void g_void;
typedef __attribute__((address_space(3))) void l_void;

// Direct-to-LDS engine.  A wave's unit is 4R consecutive rows x one segment
// of 16 pairs (576 bytes) per row.  Each row's segment is fetched by one
// global_load_lds_dwordx4 (36 lanes x 16 bytes, non-temporal) into the
// wave's window in LDS: every 128-byte line is requested by one instruction
// and no registers hold loads in flight.  The lanes then read their pair
// (nine dwords) back from the window.  The wait before a unit is computed is
// an explicit vmcnt: every unit issues at least 4R load instructions, so
// "4R times the units issued since" bounds what may still be outstanding.
// Segments that run past the row end (k % 1024 != 0) load only the row's
// bytes (whole 16-byte pieces, then dwords); pairs past the row end have
// their scales zeroed before use, and meet zero activations.
template <int WAVES, int R, int NB, int XS>
struct DmaEngine {
    static constexpr int kWaves = WAVES;
    static constexpr int kR = R;
    static constexpr int kJB = 1;
    static constexpr int kSeg = 16 * kPairBytes;  // 576
    // Row pitch 576 bytes = 144 dwords: lane l of a 16-lane group reads dword 9l + c
    // of its row, and rows 144 dwords apart put the four groups of a wave on
    // disjoint banks (9 is invertible modulo 32 and 64).
    static constexpr int kPitch = kSeg;
    static constexpr int kSlot = 4 * R * kPitch;
    static constexpr int kWaveLds = NB * kSlot;
    struct Buf {
        int slot;
        uint32_t seq;  // issue order of the unit in the slot
        bool edge;
    };
    int lane, l16;
    uint32_t rr0;    // row of this lane's first row within a step
    uint32_t wrow0;  // first row of this wave within a step
    uint32_t seq;    // units issued so far
    uint8_t* wl;     // this wave's window

    __device__ __forceinline__ void init(uint8_t* window) {
        lane = threadIdx.x & 63;
        l16 = lane & 15;
        const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
        wrow0 = (uint32_t)(wave * 4 * R);
        rr0 = wrow0 + (uint32_t)((lane >> 4) * R);
        seq = 0;
        wl = window;
    }
    __device__ __forceinline__ void init_buf(Buf& b, int slot) const {
        b.slot = slot;
        b.seq = 0;
        b.edge = false;
    }

    __device__ __forceinline__ void issue(const PlanDesc& D, const Cursor& c, Buf& b) {
        const int np = D.k >> 6;
        const uint32_t rb = (uint32_t)np * kPairBytes;
        const int64_t row0 = c.s * (int64_t)(WAVES * 4 * R) + wrow0;
        const uint32_t seg = (uint32_t)c.jb * kSeg;
        uint8_t* dst = wl + b.slot * kSlot;
        b.seq = seq++;
        b.edge = !(row0 + 4 * R <= D.n && (np & 15) == 0);  // uniform
        if (!b.edge) {
            const uint8_t* src = D.w + row0 * rb + seg + 16 * lane;
#pragma unroll
            for (int r = 0; r < 4 * R; ++r)
                if (lane < kSeg / 16)
                    __builtin_amdgcn_global_load_lds((g_void*)(src + (uint32_t)r * rb), (l_void*)(dst + r * kPitch),
                                                     16, 0, 2);
        } else {
            // rows past N read the last row (never stored)
            const uint32_t avail = min((uint32_t)kSeg, rb - seg);
            const uint32_t full = avail >> 4, rem = avail & 15;
            const int last_row = (int)(D.n - 1);
#pragma unroll
            for (int r = 0; r < 4 * R; ++r) {
                const uint32_t rr = (uint32_t)min((int)row0 + r, last_row);
                const uint8_t* row = D.w + (uint64_t)rr * rb + seg;
                if ((uint32_t)lane < full)
                    __builtin_amdgcn_global_load_lds((g_void*)(row + 16 * lane), (l_void*)(dst + r * kPitch), 16, 0,
                                                     2);
                if ((uint32_t)lane < (rem >> 2))
                    __builtin_amdgcn_global_load_lds((g_void*)(row + 16 * full + 4 * lane),
                                                     (l_void*)(dst + r * kPitch + 16 * full), 4, 0, 2);
            }
        }
    }

    // Wait for the unit in `b`, read this lane's pairs from the window into
    // registers, and wait for those reads, so the slot may be refilled.
    __device__ __forceinline__ void fetch(int k, int jb, const Buf& b, uint32_t (&D)[R][9]) const {
        const uint32_t after = seq - 1u - b.seq;  // units issued after this one (uniform)
        if (after >= 2u)
            wait_vmcnt<8 * R>();
        else if (after == 1u)
            wait_vmcnt<4 * R>();
        else
            wait_vmcnt<0>();
        const uint32_t* p = (const uint32_t*)(wl + b.slot * kSlot + (rr0 - wrow0) * kPitch + kPairBytes * l16);
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int c = 0; c < 9; ++c) D[i][c] = p[i * (kPitch / 4) + c];
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the reads are done before the slot is reloaded
        if (b.edge && 16 * jb + l16 >= (k >> 6)) {
#pragma unroll
            for (int i = 0; i < R; ++i) {
                D[i][0] &= 0xFFFF0000u;  // d of block 0
                D[i][4] &= 0x0000FFFFu;  // d of block 1
            }
        }
    }

    __device__ __forceinline__ void math(int npl, int jb, const u4* __restrict__ xs, const uint32_t (&D)[R][9],
                                         float (&acc)[R]) const {
        const int stride = XS > 0 ? XS : npl * 16;
        rows_dot<R>(D, xs + (l16 + 16 * jb), stride, acc);
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

// The sweep kernel.  A workgroup works through chunks; a chunk is the row
// steps from (d0, s0) on, in list order, that start before cost c_end.
//  * Single GEMV / LM head (head == nullptr): one chunk per workgroup, its
//    byte-balanced share [T*g/G, T*(g+1)/G) of the one descriptor `one`.
//  * Batch (head != nullptr): chunk g of the plan's schedule first, then
//    further chunks taken from the shared counter head->next as the workgroup
//    runs out of work, so workgroups that stream faster take more.  Chunk ids
//    travel through two LDS slots: at its t-th chunk change the workgroup
//    reads the id of chunk t+1 from q_next[(t+1)&1] and fetches that chunk's
//    entry; in the following half-step lane 0 takes the id of chunk t+2 from
//    the counter before that half-step's loads and stores it to q_next[t&1]
//    after its compute, when the atomic has long returned.  The schedule
//    gives every chunk but the list's last at least two units, so chunk
//    changes are at least one half-step apart.  The last workgroup to finish
//    resets the counters for the next launch.
// Every wave walks the same unit sequence (its own rows of each step), so the
// barriers of chunk changes and activation staging are reached by all.
template <class E, int NB, int XS, bool ARGMAX>
__global__ void __launch_bounds__(E::kWaves * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerEu)))
k_sweep(const PlanDesc* __restrict__ descs, int count, SchedHead* head, const SchedChunk* __restrict__ chunks,
        PlanDesc one, int64_t total, int xs_bytes, uint64_t* __restrict__ keys) {
    static_assert(NB == 2, "two slots per wave: the slot of the unit being computed is refilled once its pairs are read");
    extern __shared__ u4 xs[];
    __shared__ int q_next[2];  // ids of this workgroup's coming chunks (batch schedule)
    constexpr int R = E::kR;
    constexpr int JB = E::kJB;
    E eng;
    eng.init(reinterpret_cast<uint8_t*>(xs) + xs_bytes +
             __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) * E::kWaveLds);
    const bool dyn = head != nullptr;  // uniform
    const int n_desc = descs ? count : 1;
    auto get = [&](int d) -> PlanDesc { return descs ? descs[d] : one; };

    // The workgroup's first chunk.
    Cursor cl;       // next unit to load
    int64_t hl;      // end (cost) of the chunk being loaded
    bool have_l;
    PlanDesc Dl;
    if (dyn) {
        const SchedChunk ch = chunks[blockIdx.x];
        cl.d = ch.d0;
        cl.s = ch.s0;
        hl = ch.c_end;
        have_l = true;
    } else {
        const int64_t G = gridDim.x;
        const int64_t c_lo = uniform64((total / G) * blockIdx.x + ((total % G) * blockIdx.x) / G);
        hl = uniform64((total / G) * (blockIdx.x + 1) + ((total % G) * ((int64_t)blockIdx.x + 1)) / G);
        cl.d = 0;
        cl.s = uniform64((c_lo + one.npl - 1) / one.npl);
        have_l = cl.s < one.steps && cl.s * one.npl < hl;
    }
    cl.jb = 0;
    if (have_l) Dl = get(cl.d);

    const int n_static = gridDim.x;
    const int n_chunks = dyn ? head->nchunks : 0;
    SchedChunk nx;         // entry of the chunk after the one being loaded
    bool nx_ok = false;
    int trans = 0;         // chunk changes so far
    bool grab = false;     // this half-step takes a chunk id from the counter
    uint32_t pending = 0;  // lane 0: the id taken
    if (dyn) {
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
        Cursor c2 = next_unit(Dl, cl, JB);
        if (c2.d < n_desc) {
            if (c2.d != cl.d) Dl = get(c2.d);
            if (Dl.cost_begin + c2.s * Dl.npl < hl) {
                cl = c2;
                return;
            }
        }
        if (!nx_ok) {
            have_l = false;
            return;
        }
        cl.d = nx.d0;
        cl.s = nx.s0;
        cl.jb = 0;
        hl = nx.c_end;
        Dl = get(cl.d);
        ++trans;
        __syncthreads();  // q_next[(trans+1)&1] is written and q_next[trans&1] read by every wave
        const int id = __builtin_amdgcn_readfirstlane(q_next[(trans + 1) & 1]);
        nx_ok = id < n_chunks;
        if (nx_ok) nx = chunks[id];
        grab = true;
    };

    uint64_t best = 0;
    if (have_l) {
        // Unit ring: the next unit's loads are issued before the current one
        // is computed, across row groups, GEMVs and chunks.
        struct Rec {  // a loaded unit: descriptor, row step, pair-per-lane index
            int32_t d;
            int32_t jb;
            int64_t s;
            bool valid;
        };
        auto record = [&](Rec& r) {
            r.d = cl.d;
            r.jb = cl.jb;
            r.s = cl.s;
        };
        typename E::Buf B0, B1;
        eng.init_buf(B0, 0);
        eng.init_buf(B1, 1);
        Rec R0, R1;
        float acc[R];
#pragma unroll
        for (int i = 0; i < R; ++i) acc[i] = 0.0f;
        int dc = -1;      // descriptor held in Dc (compute side)
        int staged = -1;  // descriptor whose activations are in LDS
        PlanDesc Dc;

        // One half-step on the unit in (r, b): take a chunk id if one is
        // owed, stage the activations if the GEMV changed, read the unit's
        // pairs, refill its slot with the next unit to load (so two units
        // are in flight during the math), compute, store the taken id.
        // Returns whether the unit after this one (r_next) is loaded.
        auto half_step = [&](Rec& r, typename E::Buf& b, const Rec& r_next) -> bool {
            const bool took = grab;
            grab = false;
            if (took && threadIdx.x == 0) pending = atomicAdd(&head->next, 1u);
            const Rec u = r;
            if (u.d != dc) {
                Dc = get(u.d);
                dc = u.d;
            }
            if (u.d != staged) {
                __syncthreads();
                stage_x(Dc.x, Dc.k >> 5, Dc.npl * 16, XS > 0 ? XS : Dc.npl * 16, xs);
                __syncthreads();
                staged = u.d;
            }
            uint32_t W[R][9];
            eng.fetch(Dc.k, u.jb, b, W);
            r.valid = have_l;
            if (have_l) {
                record(r);
                eng.issue(Dl, cl, b);
                advance_l();
            }
            eng.math(Dc.npl, u.jb, xs, W, acc);
            if (u.jb + JB >= Dc.npl) {  // last unit of this row group
                const int64_t r0 = u.s * (int64_t)(E::kWaves * 4 * R) + eng.rr0;
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const float v = row16_sum(acc[i]);
                    acc[i] = 0.0f;
                    if (eng.l16 == 0 && r0 + i < Dc.n) {
                        ((g_f32*)Dc.y)[r0 + i] = v;
                        if (ARGMAX) {
                            const uint64_t kk = argmax_key(v, r0 + i);
                            best = kk > best ? kk : best;
                        }
                    }
                }
            }
            if (took && threadIdx.x == 0) q_next[trans & 1] = n_static + (int)pending;
            return r_next.valid;
        };
        R0.valid = true;
        record(R0);
        eng.issue(Dl, cl, B0);
        advance_l();
        R1.valid = have_l;
        if (have_l) {
            record(R1);
            eng.issue(Dl, cl, B1);
            advance_l();
        }
        for (;;) {
            if (!half_step(R0, B0, R1)) break;
            if (!half_step(R1, B1, R0)) break;
        }
    }
    if (dyn && threadIdx.x == 0) {
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

static int npl_of(int64_t k) { return (int)(((k / 64) + 15) / 16); }

// LDS of the staged activations: the fixed stride when k fits it, else k's own padding.
static bool fixed_stride(int64_t max_k) { return npl_of(max_k) * 16 <= kXStride; }
static size_t x_lds_bytes(int64_t max_k) {
    const int pairs = fixed_stride(max_k) ? kXStride : npl_of(max_k) * 16;
    return (size_t)pairs * kChunksPerPair * sizeof(u4);
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
    return d;
}

// The sweep engine for a workgroup shape and an activation stride.
template <int WAVES, int R, int XS>
using SweepEngine = DmaEngine<WAVES, R, kNB, XS>;

template <int WAVES, int R, int XS, bool AM>
static hipError_t launch_sweep(const PlanDesc* descs, int count, SchedHead* head, const SchedChunk* chunks,
                               const PlanDesc& one, int64_t total, int64_t max_k, int grid, uint64_t* keys,
                               hipStream_t s) {
    using E = SweepEngine<WAVES, R, XS>;
    const size_t xsb = x_lds_bytes(max_k);
    const size_t lds = xsb + (size_t)WAVES * E::kWaveLds;
    auto kern = k_sweep<E, kNB, XS, AM>;
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(WAVES * 64), lds, s, descs, count, head, chunks, one, total, (int)xsb,
                       keys);
    return hipGetLastError();
}

template <bool AM>
static hipError_t launch_any(const Shape& sh, const PlanDesc* descs, int count, SchedHead* head,
                             const SchedChunk* chunks, const PlanDesc& one, int64_t total, int64_t max_k, int grid,
                             uint64_t* keys, hipStream_t s) {
    const bool fixed = fixed_stride(max_k);
    if (sh.waves == kNarrow.waves && sh.r == kNarrow.r)
        return fixed ? launch_sweep<kNarrow.waves, kNarrow.r, kXStride, AM>(descs, count, head, chunks, one, total,
                                                                            max_k, grid, keys, s)
                     : launch_sweep<kNarrow.waves, kNarrow.r, 0, AM>(descs, count, head, chunks, one, total, max_k,
                                                                      grid, keys, s);
    return fixed ? launch_sweep<kWide.waves, kWide.r, kXStride, AM>(descs, count, head, chunks, one, total, max_k,
                                                                    grid, keys, s)
                 : launch_sweep<kWide.waves, kWide.r, 0, AM>(descs, count, head, chunks, one, total, max_k, grid,
                                                              keys, s);
}

// Workgroups for a static split of `steps` row steps.
static int static_grid(int64_t steps, const Shape& sh, int cap) {
    return (int)std::max<int64_t>(
        1, std::min<int64_t>({steps, (int64_t)device_cu_count() * sh.wg_per_cu, (int64_t)cap}));
}

// Shape for a single GEMV of n rows: the wide one when it gives every CU two
// workgroups of work, else the narrow one.
static const Shape& single_shape(int64_t n) {
    const int64_t wide_steps = (n + kWide.rows_per_step() - 1) / kWide.rows_per_step();
    return wide_steps >= 2 * (int64_t)device_cu_count() ? kWide : kNarrow;
}

hipError_t launch_gemv(const uint8_t* w, const uint16_t* x, float* y, int64_t n, int64_t k,
                       hipStream_t s) {
    const Shape& sh = single_shape(n);
    const PlanDesc d = single_desc(w, x, y, n, k, sh);
    return launch_any<false>(sh, nullptr, 1, nullptr, nullptr, d, d.steps * d.npl, k,
                             static_grid(d.steps, sh, INT32_MAX), nullptr, s);
}

int argmax_blocks(int64_t n, int64_t k) {
    (void)k;
    const Shape& sh = single_shape(n);
    return static_grid((n + sh.rows_per_step() - 1) / sh.rows_per_step(), sh, kArgmaxMaxBlocks);
}

hipError_t launch_lm_head(const uint8_t* w, const uint16_t* h, float* logits, int32_t* token,
                          int64_t n, int64_t k, uint64_t* keys, hipStream_t s) {
    const Shape& sh = single_shape(n);
    const PlanDesc d = single_desc(w, h, logits, n, k, sh);
    const int grid = argmax_blocks(n, k);
    hipError_t e = launch_any<true>(sh, nullptr, 1, nullptr, nullptr, d, d.steps * d.npl, k, grid, keys, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_argmax_final, dim3(1), dim3(kFinalThreads), 0, s, keys, grid, token);
    return hipGetLastError();
}

hipError_t launch_gemm_generic(const uint8_t* w, const uint16_t* x, float* y, int64_t m,
                               int64_t n, int64_t k, hipStream_t s) {
    const int64_t grid = (n + 3) / 4;
    hipLaunchKernelGGL(k_gemm_generic, dim3((unsigned)grid), dim3(kGenThreads), 0, s, w, x, y, (int)m,
                       n, k);
    return hipGetLastError();
}

// Schedule of a batch.  Row steps are taken in list order and grouped into
// atoms of at least two units (a step of one unit, k <= 1024, is paired with
// the next), so a chunk made of whole atoms has at least two units, as the
// kernel's chunk-id hand-over requires.  The first `grid` chunks (one per
// workgroup, assigned statically) cover about kStaticShare of the work in
// equal parts; the rest is cut into chunks of about remaining / (3 * grid)
// (guided self-scheduling), at least one atom each, which workgroups take
// from the shared counter as they run out of work.  Depends only on the
// shapes and the device's CU count.
static constexpr double kStaticShare = 0.6;

void build_schedule(PlanDesc* descs, int count, std::vector<SchedChunk>* out, int* grid_out) {
    struct Atom {
        int32_t d, s;
        int64_t cost;  // start cost of its first step
    };
    std::vector<Atom> atoms;
    int64_t total = 0;
    int open_units = 2;  // units of the last atom
    for (int i = 0; i < count; ++i) {
        PlanDesc& p = descs[i];
        p.npl = npl_of(p.k);
        p.steps = (p.n + kWide.rows_per_step() - 1) / kWide.rows_per_step();
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
    const int grid = static_grid(n_atoms, kWide, INT32_MAX);
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
        const int64_t size = std::max<int64_t>(1, (total - cost_at(a) + 3 * grid - 1) / (3 * grid));
        const int64_t end = cost_at(a) + size;
        ++a;
        while (a < n_atoms && cost_at(a) < end) ++a;
    }
    for (size_t i = 0; i + 1 < out->size(); ++i) {
        const SchedChunk& nx = (*out)[i + 1];
        (*out)[i].c_end = descs[nx.d0].cost_begin + (int64_t)nx.s0 * descs[nx.d0].npl;
    }
    out->back().c_end = total;
    *grid_out = grid;
}

hipError_t launch_gemv_batch(const void* plan, int count, int nchunks, int grid, int max_k, hipStream_t s) {
    (void)nchunks;
    const uint8_t* base = static_cast<const uint8_t*>(plan);
    SchedHead* head = (SchedHead*)base;
    const PlanDesc* descs = (const PlanDesc*)(base + sizeof(SchedHead));
    const SchedChunk* chunks = (const SchedChunk*)(base + sizeof(SchedHead) + (size_t)count * sizeof(PlanDesc));
    PlanDesc none = {};
    return launch_any<false>(kWide, descs, count, head, chunks, none, 0, max_k, grid, nullptr, s);
}

}  // namespace q4
