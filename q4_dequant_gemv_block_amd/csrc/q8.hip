// Q8_0 matrix-vector product: y[n] = sum_k w[n][k] x[k], w in Q8_0 blocks.
//
// The pages' other weight format, used by the small dense Qwen3 models
// (taozi.news, section "支持模型与限制"), read as: 34-byte blocks of 32
// weights, an f16 scale d (little-endian) then 32 two's-complement code bytes,
// weight j = code_j * d; a row of K weights is K/32 consecutive blocks.
//
// The kernel streams rows from HBM: one wave per row at a time, lane l takes
// blocks l, l + 64, ... of the row, so the 64 lanes of one load instruction
// cover 64 consecutive blocks (2,176 contiguous bytes).  A block sits at an
// even byte offset; a lane reads the 36-byte dword-aligned window around it
// (two dwordx4 and one dword) and realigns the codes with v_alignbyte when the
// block starts 2 bytes into a dword.  Codes become f16 exactly (byte xor 0x80
// under the exponent of 1024 via v_perm, minus 1152), products and sums go
// through v_dot2_f32_f16 against x staged once per workgroup in LDS, and the
// block's sum is scaled by d with one FMA.  The row's lanes are summed by a
// fixed butterfly, so every row has one association wherever it runs.
#include "q4_device.h"
#include "q4_launch.h"

#include <algorithm>
#include <climits>
#include <vector>

namespace q4 {

namespace {

constexpr int kQ8BlockBytes = 34;
constexpr int kQ8Waves = 8;   // waves per workgroup
constexpr int kQ8Unroll = 2;  // blocks per lane loaded before their math
constexpr double kQ8StaticShare = 0.85;  // of a list's bytes, split statically before the chunks

typedef __attribute__((address_space(1))) const uint16_t g_u16;

// One block in registers: its 32 codes (code 4j + i in byte i of c[j]) and d.
struct Q8Block {
    uint32_t c[8];
    float d;
};

// `end`: one past the matrix's last byte.  Only the matrix's last block can
// have a window that reaches past it (when that block starts on a dword).
__device__ __forceinline__ void load_q8(const uint8_t* blk, const uint8_t* end, Q8Block& B) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(blk);
    const bool odd = (a & 2u) != 0;  // the block starts 2 bytes into a dword
    const uint8_t* al = reinterpret_cast<const uint8_t*>(a & ~(uintptr_t)3);
    const u4a4 p = *(g_u4a4*)al;
    const u4a4 q = *(g_u4a4*)(al + 16);
    uint32_t t;
    if (odd || al + 36 <= end)
        t = *(g_u32*)(al + 32);
    else
        t = (uint32_t)*(g_u16*)(al + 32);
    const uint32_t D[9] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w, t};
    B.d = odd ? f16_hi(D[0]) : f16_lo(D[0]);
#pragma unroll
    for (int j = 0; j < 8; ++j) B.c[j] = odd ? D[j + 1] : __builtin_amdgcn_alignbyte(D[j + 1], D[j], 2);
}

// sum_j code_j x_j over one block (binary32 through v_dot2_f32_f16), codes
// exact in f16: byte ^ 0x80 = code + 128, placed under 0x64 it reads as
// 1024 + code + 128, and subtracting 1152 leaves the code.
__device__ __forceinline__ float q8_dot(const Q8Block& B, const u4 (&xv)[4]) {
    const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t u = B.c[j] ^ 0x80808080u;
        const h2 lo = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - bias;  // codes 4j, 4j+1
        const h2 hi = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - bias;  // codes 4j+2, 4j+3
        const u4 xc = xv[j >> 1];
        const uint32_t x0 = (j & 1) ? xc.z : xc.x;
        const uint32_t x1 = (j & 1) ? xc.w : xc.y;
        s = __builtin_amdgcn_fdot2(lo, as_h2(x0), s, false);
        s = __builtin_amdgcn_fdot2(hi, as_h2(x1), s, false);
    }
    return s;
}

__global__ void __launch_bounds__(kQ8Waves * 64) k_q8_gemv(const uint8_t* __restrict__ w,
                                                          const uint16_t* __restrict__ x, float* __restrict__ y,
                                                          int64_t n, int k) {
    extern __shared__ u4 xs[];  // x, k binary16
    for (int i = threadIdx.x; i < (k >> 3); i += blockDim.x) xs[i] = ((g_u4*)x)[i];
    __syncthreads();
    const int nb = k >> 5;
    const int lane = threadIdx.x & 63;
    const int64_t rb = (int64_t)nb * kQ8BlockBytes;
    const uint8_t* end = w + n * rb;
    const int64_t nwaves = (int64_t)gridDim.x * kQ8Waves;
    for (int64_t row = (int64_t)blockIdx.x * kQ8Waves + (threadIdx.x >> 6); row < n; row += nwaves) {
        const uint8_t* wr = w + row * rb;
        float acc = 0.0f;
        for (int b0 = lane; b0 < nb; b0 += 64 * kQ8Unroll) {
            Q8Block B[kQ8Unroll];
#pragma unroll
            for (int u = 0; u < kQ8Unroll; ++u)
                if (b0 + 64 * u < nb) load_q8(wr + (int64_t)(b0 + 64 * u) * kQ8BlockBytes, end, B[u]);
#pragma unroll
            for (int u = 0; u < kQ8Unroll; ++u) {
                const int b = b0 + 64 * u;
                if (b < nb) {
                    const u4 xv[4] = {xs[4 * b], xs[4 * b + 1], xs[4 * b + 2], xs[4 * b + 3]};
                    acc = __builtin_fmaf(B[u].d, q8_dot(B[u], xv), acc);
                }
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
        if (lane == 0) y[row] = acc;
    }
}

// Rows r0 and r0 + 1 (when has1) of one GEMV by one wave: the loads of both
// rows' blocks go out before their math, so each lane has up to four blocks
// in flight.  Each row keeps the association of k_q8_gemv (blocks in lane
// order, the same butterfly), so its bits equal the single call's.
__device__ __forceinline__ void q8_two_rows(const Q8Desc& D, int64_t r0, bool has1, const u4* __restrict__ xs,
                                            int lane) {
    const int nb = D.k >> 5;
    const int64_t rb = (int64_t)nb * kQ8BlockBytes;
    const uint8_t* end = D.w + D.n * rb;
    const uint8_t* w0 = D.w + r0 * rb;
    const uint8_t* w1 = w0 + rb;
    float a0 = 0.0f, a1 = 0.0f;
    for (int b0 = lane; b0 < nb; b0 += 64 * kQ8Unroll) {
        Q8Block B0[kQ8Unroll], B1[kQ8Unroll];
#pragma unroll
        for (int u = 0; u < kQ8Unroll; ++u) {
            const int b = b0 + 64 * u;
            if (b < nb) {
                load_q8(w0 + (int64_t)b * kQ8BlockBytes, end, B0[u]);
                if (has1) load_q8(w1 + (int64_t)b * kQ8BlockBytes, end, B1[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < kQ8Unroll; ++u) {
            const int b = b0 + 64 * u;
            if (b < nb) {
                const u4 xv[4] = {xs[4 * b], xs[4 * b + 1], xs[4 * b + 2], xs[4 * b + 3]};
                a0 = __builtin_fmaf(B0[u].d, q8_dot(B0[u], xv), a0);
                if (has1) a1 = __builtin_fmaf(B1[u].d, q8_dot(B1[u], xv), a1);
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        a0 += __shfl_xor(a0, o, 64);
        a1 += __shfl_xor(a1, o, 64);
    }
    if (lane == 0) {
        D.y[r0] = a0;
        if (has1) D.y[r0 + 1] = a1;
    }
}

// A GEMV list: workgroup g first takes units [wg_begin[g], wg_begin[g+1]) in
// list order (a unit: kQ8UnitRows rows of one GEMV, two per wave), then
// chunks of the remaining units from the counter as it runs out of work, so
// that workgroups that stream faster take more.  A GEMV's x is staged into
// LDS when a unit of it comes up after a unit of another GEMV.
__global__ void __launch_bounds__(kQ8Waves * 64) k_q8_batch(Q8Head* head, const Q8Desc* __restrict__ descs,
                                                           int count, const int64_t* __restrict__ wg_begin) {
    static_assert(kQ8UnitRows == 2 * kQ8Waves, "two rows per wave per unit");
    extern __shared__ u4 xs[];
    __shared__ uint32_t ticket;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int d = -1;  // the GEMV whose x is in LDS
    Q8Desc D;
    int64_t d_end = 0;  // one past its last unit
    auto run = [&](int64_t u_lo, int64_t u_hi) {
        for (int64_t u = u_lo; u < u_hi; ++u) {
            if (d < 0 || u < D.unit_begin || u >= d_end) {
                int lo = 0, hi = count - 1;  // last GEMV with unit_begin <= u
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (descs[mid].unit_begin <= u)
                        lo = mid;
                    else
                        hi = mid - 1;
                }
                d = lo;
                D = descs[d];
                d_end = d + 1 < count ? descs[d + 1].unit_begin : INT64_MAX;
                __syncthreads();  // every wave is done with the previous x
                for (int i = threadIdx.x; i < (D.k >> 3); i += blockDim.x) xs[i] = ((g_u4*)D.x)[i];
                __syncthreads();
            }
            const int64_t r0 = (u - D.unit_begin) * kQ8UnitRows + 2 * wave;
            if (r0 < D.n) q8_two_rows(D, r0, r0 + 1 < D.n, xs, lane);
        }
    };
    run(wg_begin[blockIdx.x], wg_begin[blockIdx.x + 1]);
    const int64_t dyn_begin = head->dyn_begin, dyn_end = head->dyn_end;
    const int chunk = head->chunk;
    for (;;) {  // ends when the counter passes the last chunk: every workgroup gets there
        if (threadIdx.x == 0) ticket = atomicAdd(&head->next, 1u);
        __syncthreads();
        const int64_t u0 = dyn_begin + (int64_t)__builtin_amdgcn_readfirstlane(ticket) * chunk;
        __syncthreads();  // every wave has read the ticket before the next one is taken
        if (u0 >= dyn_end) break;
        run(u0, std::min<int64_t>(u0 + chunk, dyn_end));
    }
    if (threadIdx.x == 0) {
        __threadfence();  // this workgroup's tickets come first
        if (atomicAdd(&head->done, 1u) == gridDim.x - 1) {
            atomicExch(&head->next, 0u);
            atomicExch(&head->done, 0u);
        }
    }
}

}  // namespace

int q8_batch_layout(Q8Desc* descs, int count, std::vector<int64_t>* wg_begin, Q8Head* head) {
    int64_t units = 0;
    double total = 0.0;
    for (int i = 0; i < count; ++i) {
        descs[i].unit_begin = units;
        units += (descs[i].n + kQ8UnitRows - 1) / kQ8UnitRows;
        total += (double)descs[i].n * (descs[i].k / 32) * kQ8BlockBytes;
    }
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(units, kQ8WgPerCu * (int64_t)device_cu_count()));
    // the first kQ8StaticShare of the bytes go out as one contiguous range per
    // workgroup (workgroup g from the first unit whose bytes-before reach
    // static * g / grid); the units after them go out in chunks
    const double share = total * kQ8StaticShare;
    int64_t dyn_begin = units;
    double static_bytes = total;
    {
        double before = 0.0;
        for (int i = 0; i < count && dyn_begin == units; ++i) {
            const double row = (double)(descs[i].k / 32) * kQ8BlockBytes;
            const int64_t nu = (descs[i].n + kQ8UnitRows - 1) / kQ8UnitRows;
            for (int64_t j = 0; j < nu; ++j) {
                if (before >= share) {
                    dyn_begin = descs[i].unit_begin + j;
                    static_bytes = before;
                    break;
                }
                before += row * (double)std::min<int64_t>(kQ8UnitRows, descs[i].n - j * kQ8UnitRows);
            }
        }
    }
    wg_begin->assign(grid + 1, dyn_begin);
    (*wg_begin)[0] = 0;
    int g = 1;
    double before = 0.0;
    for (int i = 0; i < count && g < grid; ++i) {
        const double row = (double)(descs[i].k / 32) * kQ8BlockBytes;
        const int64_t nu = (descs[i].n + kQ8UnitRows - 1) / kQ8UnitRows;
        for (int64_t j = 0; j < nu && g < grid && descs[i].unit_begin + j < dyn_begin; ++j) {
            while (g < grid && before >= static_bytes * g / grid) (*wg_begin)[g++] = descs[i].unit_begin + j;
            before += row * (double)std::min<int64_t>(kQ8UnitRows, descs[i].n - j * kQ8UnitRows);
        }
    }
    head->next = 0;
    head->done = 0;
    head->chunk = (int32_t)std::max<int64_t>(1, (units - dyn_begin) / (4 * (int64_t)grid));
    head->reserved = 0;
    head->dyn_begin = dyn_begin;
    head->dyn_end = units;
    return grid;
}

hipError_t launch_q8_batch(void* plan, int count, int grid, int max_k, hipStream_t s) {
    Q8Head* head = static_cast<Q8Head*>(plan);
    const Q8Desc* descs = reinterpret_cast<const Q8Desc*>(head + 1);
    const int64_t* wg_begin = reinterpret_cast<const int64_t*>(descs + count);
    hipLaunchKernelGGL(k_q8_batch, dim3(grid), dim3(kQ8Waves * 64), (size_t)max_k * 2, s, head, descs, count,
                       wg_begin);
    return hipGetLastError();
}

hipError_t launch_q8_gemv(const uint8_t* w, const uint16_t* x, float* y, int64_t n, int64_t k, hipStream_t s) {
    const int64_t wgs = (n + kQ8Waves - 1) / kQ8Waves;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(wgs, 2 * (int64_t)device_cu_count()));
    hipLaunchKernelGGL(k_q8_gemv, dim3(grid), dim3(kQ8Waves * 64), (size_t)k * 2, s, w, x, y, n, (int)k);
    return hipGetLastError();
}

}  // namespace q4
