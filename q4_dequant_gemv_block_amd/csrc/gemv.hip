// Q4_0 matrix-vector kernels for gfx950: single GEMV, the one-launch batch of
// GEMVs (a whole decode weight sweep), the LM head with greedy argmax, and a
// generic kernel for shapes the fast path does not take.
//
// Decode reads every weight once per token and is bound by memory bandwidth
// ("Every Device Brings a Slice: How SwarmLLM Runs a 27B Model Across Browser
// Tabs", originshq.com, section "The Engine: ~50 WGSL Kernels Written From
// Scratch").  The kernels here keep that structure but are laid out for CDNA4:
//
//  * 16 lanes (one DPP row) own one weight row; lane l takes block pairs
//    l, l+16, l+32, ... so the 16 lanes of a row read 576 contiguous bytes per
//    step, and the 4 rows of a wave are R rows apart.  Each lane keeps R rows
//    in flight at the same pair positions, so one read of the activation
//    chunks from LDS serves R rows.
//  * Weights are read with non-temporal dwordx4/dword loads (36-byte pairs at
//    4-byte alignment); the 4-bit codes become exact (code - 8) f16 pairs with
//    one v_and_or_b32 and one v_pk_add_f16 per pair and meet the activations
//    in v_dot2_f32_f16; the block scale is applied once per block in f32.
//  * The activation vector is staged once per workgroup into LDS in the
//    chunk order of q4_device.h, conflict-free for the 16-lane row reads.
//  * The row sum is a fixed-order DPP tree inside the 16-lane row, so results
//    are deterministic and independent of where a row sits.
#include "q4_device.h"
#include "q4_launch.h"

#include <algorithm>
#include <atomic>

namespace q4 {

constexpr int kThreads = 256;  // 4 waves
constexpr int kBatchR = 2;     // rows per lane group in the batch kernel
constexpr int kBatchJB = 4;    // pairs per lane loaded before compute

int batch_rows_per_step() { return 16 * kBatchR; }

// ---------------------------------------------------------------------------
// Activation staging: the 8 chunks of every block pair, chunk c of pair p at
// xs[c * npp + p]; pairs >= k/64 (padding up to npp) are zero.
// ---------------------------------------------------------------------------
__device__ void stage_x(const uint16_t* __restrict__ x, int nblocks, int npp, u4* __restrict__ xs) {
    const int nb_pad = 2 * npp;
    for (int b = threadIdx.x; b < nb_pad; b += blockDim.x) {
        uint32_t v[16];  // 32 f16 values of block b, two per dword
        if (b < nblocks) {
            const u4* src = reinterpret_cast<const u4*>(x + 32 * (int64_t)b);
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
        const int p = b >> 1;
        const int base = (b & 1) ? 4 : 0;
        const int off = (b & 1) ? 32 : 0;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            int pos[4];
            chunk_positions(base + cc, pos);
            const int a = pos[0] - off, bb = pos[1] - off, c = pos[2] - off, e = pos[3] - off;
            u4 ent;
            ent.x = xe(a) | (xe(c) << 16);
            ent.y = xe(a + 16) | (xe(c + 16) << 16);
            ent.z = xe(bb) | (xe(e) << 16);
            ent.w = xe(bb + 16) | (xe(e + 16) << 16);
            xs[(base + cc) * npp + p] = ent;
        }
    }
}

// ---------------------------------------------------------------------------
// One wave, 4*R rows: rows row0 + 4*i + q (q = lane / 16) for i < R... laid out
// as lane group q taking rows row0 + q*R + i.  Returns the 16-lane sums.
// ---------------------------------------------------------------------------
template <int R, int JB>
__device__ __forceinline__ void rows_dot(const uint8_t* __restrict__ w, int64_t rb, int64_t n,
                                         int np, int npl, const u4* __restrict__ xs, int npp,
                                         int64_t row0, float (&out)[R]) {
    const int lane = threadIdx.x & 63;
    const int l = lane & 15;
    const int64_t rbase = row0 + (lane >> 4) * R;
    float acc[R];
#pragma unroll
    for (int i = 0; i < R; ++i) acc[i] = 0.0f;

    for (int jb = 0; jb < npl; jb += JB) {
        uint32_t D[JB][R][9];
#pragma unroll
        for (int t = 0; t < JB; ++t) {
            const int j = jb + t;
            if (j < npl) {
                const int p = l + 16 * j;
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const int64_t r = rbase + i;
                    if (r < n && p < np)
                        load_pair(w + r * rb + (int64_t)p * kPairBytes, D[t][i]);
                    else
                        zero_pair(D[t][i]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < JB; ++t) {
            const int j = jb + t;
            if (j < npl) {
                const int p = l + 16 * j;
                u4 X[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) X[c] = xs[c * npp + p];
#pragma unroll
                for (int i = 0; i < R; ++i) acc[i] = pair_dot(D[t][i], X, acc[i]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) out[i] = row16_sum(acc[i]);
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
        if ((int)threadIdx.x < s) sh[threadIdx.x] = sh[threadIdx.x] > sh[threadIdx.x + s] ? sh[threadIdx.x] : sh[threadIdx.x + s];
        __syncthreads();
    }
    return sh[0];
}

// ---------------------------------------------------------------------------
// Single GEMV (optionally with per-workgroup argmax keys).
// ---------------------------------------------------------------------------
template <int R, int JB, bool ARGMAX>
__global__ void __launch_bounds__(kThreads) k_gemv(const uint8_t* __restrict__ w,
                                                   const uint16_t* __restrict__ x,
                                                   float* __restrict__ y, int64_t n, int k,
                                                   uint64_t* __restrict__ keys) {
    extern __shared__ u4 xs[];
    const int np = k / 64;
    const int npp = (np + 15) & ~15;
    const int npl = npp / 16;
    const int64_t rb = (int64_t)np * kPairBytes;
    stage_x(x, k / 32, npp, xs);
    __syncthreads();

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t rows_per_step = 16 * R;
    uint64_t best = 0;
    for (int64_t step = blockIdx.x; step * rows_per_step < n; step += gridDim.x) {
        const int64_t row0 = step * rows_per_step + (int64_t)wave * 4 * R;
        float out[R];
        rows_dot<R, JB>(w, rb, n, np, npl, xs, npp, row0, out);
        if ((lane & 15) == 0) {
            const int64_t rbase = row0 + (lane >> 4) * R;
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const int64_t r = rbase + i;
                if (r < n) {
                    y[r] = out[i];
                    if (ARGMAX) {
                        const uint64_t kk = argmax_key(out[i], r);
                        best = kk > best ? kk : best;
                    }
                }
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
// Batch of independent GEMVs in one persistent launch.  Work item = (desc,
// row step of 16*R rows); item (d, s) "starts" at cost cost_begin[d] + s*npl[d]
// (npl is proportional to the bytes of one step).  Workgroup g takes every item
// that starts in [total*g/G, total*(g+1)/G): contiguous, byte-balanced ranges,
// so consecutive items of one workgroup share the staged activations.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t split_point(int64_t total, int64_t g, int64_t G) {
    return (total / G) * g + ((total % G) * g) / G;
}

template <int R, int JB>
__global__ void __launch_bounds__(kThreads) k_gemv_batch(const PlanDesc* __restrict__ descs,
                                                         int count, int64_t total) {
    extern __shared__ u4 xs[];
    const int64_t G = gridDim.x;
    const int64_t c_lo = split_point(total, blockIdx.x, G);
    const int64_t c_hi = split_point(total, (int64_t)blockIdx.x + 1, G);
    if (c_lo >= c_hi) return;  // whole workgroup leaves together

    int lo = 0, hi = count - 1;  // last descriptor whose range starts at or before c_lo
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (descs[mid].cost_begin <= c_lo) lo = mid; else hi = mid - 1;
    }
    int d = lo;
    int64_t s = (c_lo - descs[d].cost_begin + descs[d].npl - 1) / descs[d].npl;
    if (s >= descs[d].steps) { ++d; s = 0; }

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    int staged = -1;
    while (d < count) {
        const PlanDesc D = descs[d];
        if (D.cost_begin + s * D.npl >= c_hi) break;
        const int np = D.k / 64;
        const int npp = D.npl * 16;
        if (staged != d) {
            __syncthreads();
            stage_x(D.x, D.k / 32, npp, xs);
            __syncthreads();
            staged = d;
        }
        const int64_t row0 = s * (16 * R) + (int64_t)wave * 4 * R;
        float out[R];
        rows_dot<R, JB>(D.w, (int64_t)np * kPairBytes, D.n, np, D.npl, xs, npp, row0, out);
        if ((lane & 15) == 0) {
            const int64_t rbase = row0 + (lane >> 4) * R;
#pragma unroll
            for (int i = 0; i < R; ++i)
                if (rbase + i < D.n) D.y[rbase + i] = out[i];
        }
        if (++s == D.steps) { ++d; s = 0; }
    }
}

// ---------------------------------------------------------------------------
// Generic path: any k % 32 == 0, rows at 2-byte alignment, 1 <= m <= 16.
// One wave per weight row, lanes stride over blocks, activations from global
// memory; used for shapes the fast kernels do not take.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__global__ void __launch_bounds__(kThreads) k_gemm_generic(const uint8_t* __restrict__ w,
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

static size_t x_lds_bytes(int64_t k) {
    const int64_t np = k / 64;
    const int64_t npp = (np + 15) & ~int64_t(15);
    return (size_t)npp * kChunksPerPair * sizeof(u4);
}

hipError_t launch_gemv(const uint8_t* w, const uint16_t* x, float* y, int64_t n, int64_t k,
                       hipStream_t s) {
    const size_t lds = x_lds_bytes(k);
    const int cus = device_cu_count();
    // Small matrices: one row per lane group so more workgroups share the rows.
    if (n <= (int64_t)cus * 64) {
        const int64_t steps = (n + 15) / 16;
        const int grid = (int)std::min<int64_t>(steps, (int64_t)cus * 8);
        hipLaunchKernelGGL((k_gemv<1, 4, false>), dim3(grid), dim3(kThreads), lds, s, w, x, y, n,
                           (int)k, nullptr);
    } else {
        const int64_t steps = (n + 31) / 32;
        const int grid = (int)std::min<int64_t>(steps, (int64_t)cus * 4);
        hipLaunchKernelGGL((k_gemv<2, 4, false>), dim3(grid), dim3(kThreads), lds, s, w, x, y, n,
                           (int)k, nullptr);
    }
    return hipGetLastError();
}

int argmax_blocks(int64_t n, int64_t k) {
    (void)k;
    const int64_t steps = (n + 31) / 32;
    return (int)std::min<int64_t>(steps, kArgmaxMaxBlocks);
}

hipError_t launch_lm_head(const uint8_t* w, const uint16_t* h, float* logits, int32_t* token,
                          int64_t n, int64_t k, uint64_t* keys, hipStream_t s) {
    const size_t lds = x_lds_bytes(k);
    const int grid = std::min(argmax_blocks(n, k), device_cu_count() * 4);
    hipLaunchKernelGGL((k_gemv<2, 4, true>), dim3(grid), dim3(kThreads), lds, s, w, h, logits, n,
                       (int)k, keys);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_argmax_final, dim3(1), dim3(kThreads), 0, s, keys, grid, token);
    return hipGetLastError();
}

hipError_t launch_gemm_generic(const uint8_t* w, const uint16_t* x, float* y, int64_t m,
                               int64_t n, int64_t k, hipStream_t s) {
    const int64_t grid = (n + 3) / 4;
    hipLaunchKernelGGL(k_gemm_generic, dim3((unsigned)grid), dim3(kThreads), 0, s, w, x, y, (int)m,
                       n, k);
    return hipGetLastError();
}

hipError_t launch_gemv_batch(const PlanDesc* descs, int count, int64_t total_cost, int max_k,
                             hipStream_t s) {
    const size_t lds = x_lds_bytes(max_k);
    const int grid = device_cu_count() * 4;
    hipLaunchKernelGGL((k_gemv_batch<kBatchR, kBatchJB>), dim3(grid), dim3(kThreads), lds, s,
                       descs, count, total_cost);
    return hipGetLastError();
}

}  // namespace q4
