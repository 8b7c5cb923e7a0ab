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
// Work: a workgroup of 16 waves owns a tile of 256 weight rows (16 per wave)
// and one K-range of its GEMM; the K-range is the longest run of 16-pair
// segments whose activations for all M rows fit kXBytes of LDS, so K is split
// only for large M and K (M = 16: 5120 columns).  Items (GEMM, K-range, tile)
// are ordered GEMM, K-range, tile, and every workgroup takes a byte-balanced
// contiguous run of them, so the activations of a K-range are staged once and
// serve many tiles.  When a GEMM has several K-ranges each range writes its
// partial product to the workspace and a second kernel adds the partials in
// range order, so results are deterministic.
//
// A wave's unit is its 16 rows x one 16-pair segment.  Lane (g, n) = (lane /
// 16, lane % 16) loads pairs g, g+4, g+8, g+12 of the segment of weight row n
// (the four lanes of a row cover its 576 contiguous bytes) into registers; the
// loads of the next unit are issued before the current one is computed, also
// across tiles, K-ranges and GEMMs.  Each pair expands to 8 chunks of 8 halves
// ((code - 8) * d rounded once to f16: error <= 2^-11 of each weight, inside
// the 1e-3 bound); chunk c of lane (g, n) is the B operand for weight row n,
// and the A operand of lane (g, m) is chunk c of the same pair of activation
// row m, read from LDS (rows m >= M are zero).  The 32 k of one MFMA are 8 k
// from each of 4 pairs; both operands use the same assignment, so the sum is
// the full dot product.  Rows beyond N and pairs beyond K/64 read clamped
// in-range addresses and meet zero activations.
#include "q4_device.h"
#include "q4_launch.h"

#include <algorithm>

namespace q4 {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) float g_f32;

constexpr int kSmWaves = 16;
constexpr int kSmThreads = kSmWaves * 64;
constexpr int kTileRows = 16 * kSmWaves;  // 256
constexpr int kPairsPerLane = 4;          // pairs g, g+4, g+8, g+12 of a segment
constexpr int kXBytes = 160 * 1024;       // activations of one K-range, all M rows (the whole LDS)

__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Segments (16 pairs) of K-range c of a descriptor.
__device__ __forceinline__ int segs_of(const SmDesc& D, int c) {
    return (min(D.P, D.np - c * D.P) + 15) >> 4;
}

// First unit (cost) of item (c, t): ranges before c are full.
__device__ __forceinline__ int64_t item_start(const SmDesc& D, int c, int t) {
    return D.cost_begin + (int64_t)c * D.tiles * (D.P >> 4) + (int64_t)t * segs_of(D, c);
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

// Activations of pairs [c*P, c*P + 16*segs) of all M rows into their slots;
// pairs past K/64 are zero.
template <bool SWZ>
__device__ void stage_range(const SmDesc& D, int c, int m, u4* __restrict__ xs) {
    const int p0 = c * D.P;
    const int npairs = 16 * segs_of(D, c);
    for (int it = threadIdx.x; it < 2 * npairs * m; it += kSmThreads) {
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
        const int half = b & 1;
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
    }
}

struct SmBuf {
    uint32_t d[kPairsPerLane][9];
};

template <bool SWZ>
__global__ void __launch_bounds__(kSmThreads) k_smallm(const SmDesc* __restrict__ descs, int count, SmDesc one,
                                                       int m, int64_t total, float* __restrict__ ws) {
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
        const int64_t full = (int64_t)Dl.tiles * (Dl.P >> 4);  // units of a full K-range
        const int64_t o = c_lo - Dl.cost_begin;
        int c = (int)(o / full < Dl.nranges - 1 ? o / full : Dl.nranges - 1);
        const int64_t r = o - c * full;
        const int sg = segs_of(Dl, c);
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
    bool have_l = cl.d < n_desc && item_start(Dl, cl.c, cl.t) < c_hi;
    if (!have_l) return;

    auto advance_l = [&]() {
        if (++cl.jb < segs_of(Dl, cl.c)) return;
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
        have_l = item_start(Dl, cl.c, cl.t) < c_hi;
    };

    auto issue = [&](SmBuf& b) {
        const int64_t row = min((int64_t)cl.t * kTileRows + 16 * wave + l16, Dl.n - 1);
        const uint8_t* wrow = Dl.w + row * (int64_t)Dl.np * kPairBytes;
        const int p0 = cl.c * Dl.P + 16 * cl.jb + g;
#pragma unroll
        for (int jj = 0; jj < kPairsPerLane; ++jj) {
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
            stage_range<SWZ>(Dc, r.c, m, xs);
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
        for (int jj = 0; jj < kPairsPerLane; ++jj) {
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
        if (r.jb + 1 == segs_of(Dc, r.c)) {  // last segment of the item: store the tile
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

    SmBuf A, B;
    Rec ra, rb;
    ra = Rec{cl.d, cl.c, cl.t, cl.jb};
    issue(A);
    advance_l();
    for (;;) {
        bool more = have_l;
        if (more) {
            rb = Rec{cl.d, cl.c, cl.t, cl.jb};
            issue(B);
            advance_l();
        }
        process(ra, A);
        if (!more) break;
        more = have_l;
        if (more) {
            ra = Rec{cl.d, cl.c, cl.t, cl.jb};
            issue(A);
            advance_l();
        }
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

// Pairs per K-range for m activation rows: the longest run of whole 16-pair
// segments whose activations fit kXBytes in the padded layout, or in the
// swizzled one (no padding, a little longer) when that takes fewer ranges.
static int smallm_range_pairs(int64_t k, int64_t m) {
    const int np = (int)(k / 64);
    const int np16 = (np + 15) / 16 * 16;
    const int row_chunks = (int)(kXBytes / (16 * m));  // 16-byte chunks per activation row
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
    d->tiles = (int32_t)((d->n + kTileRows - 1) / kTileRows);
    d->cost_begin = cost_begin;
    const int64_t floats = d->nranges > 1 ? (int64_t)d->nranges * m * d->n : 0;
    d->ws_off = floats ? ws_off : 0;
    return floats;
}

int64_t smallm_cost(const SmDesc& d) {
    int64_t c = 0;
    for (int r = 0; r < d.nranges; ++r) c += (int64_t)d.tiles * ((std::min(d.P, d.np - r * d.P) + 15) / 16);
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
// padding per row when that still fits the LDS (then the padded layout).
static bool smallm_swizzle(int64_t max_range_pairs, int64_t m) {
    return (max_range_pairs * kChunksPerPair + 1) * m * (int64_t)sizeof(u4) > kXBytes;
}
static size_t smallm_lds(int64_t max_range_pairs, int64_t m) {
    return (size_t)(max_range_pairs * kChunksPerPair + (smallm_swizzle(max_range_pairs, m) ? 0 : 1)) * m * sizeof(u4);
}

static hipError_t launch_sm(const SmDesc* descs, int count, const SmDesc& one, int64_t m, int64_t total,
                            int max_p, float* ws, hipStream_t s) {
    const size_t lds = smallm_lds(max_p, m);
    const void* kern = smallm_swizzle(max_p, m) ? (const void*)k_smallm<true> : (const void*)k_smallm<false>;
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (smallm_swizzle(max_p, m))
        hipLaunchKernelGGL(k_smallm<true>, dim3(smallm_grid(total)), dim3(kSmThreads), lds, s, descs, count, one,
                           (int)m, total, ws);
    else
        hipLaunchKernelGGL(k_smallm<false>, dim3(smallm_grid(total)), dim3(kSmThreads), lds, s, descs, count, one,
                           (int)m, total, ws);
    return hipGetLastError();
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
    hipError_t e = launch_sm(nullptr, 1, d, m, total, d.P, workspace, s);
    if (e != hipSuccess || d.nranges < 2) return e;
    const int grid = (int)std::min<int64_t>((m * n + 255) / 256, (int64_t)device_cu_count() * 4);
    hipLaunchKernelGGL(k_sum_ranges, dim3(grid, 1), dim3(256), 0, s, nullptr, 1, d, (int)m, workspace);
    return hipGetLastError();
}

hipError_t launch_gemm_smallm_batch(const SmDesc* descs, int count, int64_t m, int64_t total, int max_p,
                                    int64_t max_mn, bool any_split, float* workspace, hipStream_t s) {
    SmDesc none = {};
    hipError_t e = launch_sm(descs, count, none, m, total, max_p, workspace, s);
    if (e != hipSuccess || !any_split) return e;
    const int gx = (int)std::max<int64_t>(1, std::min<int64_t>((max_mn + 255) / 256, 64));
    const int gy = std::min(count, 65535);
    hipLaunchKernelGGL(k_sum_ranges, dim3(gx, gy), dim3(256), 0, s, descs, count, none, (int)m, workspace);
    return hipGetLastError();
}

}  // namespace q4
