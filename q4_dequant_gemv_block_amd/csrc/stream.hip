// Read-bandwidth ceiling of the device: every byte of a buffer read once and
// folded into one word, with the access patterns the Q4_0 GEMV kernels use.
//
// The pages judge their decode engine against the read bandwidth the machine
// delivers to a plain buffer read ("Every Device Brings a Slice: How SwarmLLM
// Runs a 27B Model Across Browser Tabs", originshq.com, section "The Engine:
// ~50 WGSL Kernels Written From Scratch"; taozi.news, section "基准成绩").
// This library measures that ceiling on the GPU so the GEMV's rate can be
// quoted against it as well as against the nominal HBM peak.  It is a
// measurement tool, not part of the GEMV library, and is loaded only by the
// benchmark.
//
// Patterns (all 16-byte loads, 64 lanes x 16 bytes = 1 KiB per wave load):
//   0  grid-stride, cached loads: the whole grid sweeps the buffer as one front
//   1  grid-stride, non-temporal loads
//   2  one contiguous range per workgroup, cached loads (the sweep kernel's
//      layout of work: every workgroup streams its own region)
//   3  one contiguous range per workgroup, non-temporal loads
//   4  one contiguous range per workgroup, non-temporal buffer loads straight
//      into a per-wave LDS ring, waited for with vmcnt and read back (the
//      GEMV engine's way of moving weights; 48 KiB of LDS per workgroup)
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define Q4S_API extern "C" __attribute__((visibility("default")))

namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) void g_void;
typedef __attribute__((address_space(3))) void l_void;

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // loads in flight per lane (register patterns)

__device__ __forceinline__ uint32_t fold(u4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

template <bool NT>
__device__ __forceinline__ u4 load16(const u4* p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

__device__ __forceinline__ void finish(uint32_t acc, uint32_t* out) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    __shared__ uint32_t part[kThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int i = 0; i < kThreads / 64; ++i) t ^= part[i];
        atomicXor(out, t);
    }
}

// Patterns 0/1: word i of the buffer (16 bytes) for i = tid, tid + T, ...
template <bool NT>
__global__ void __launch_bounds__(kThreads) k_stride(const u4* __restrict__ p, int64_t n16, uint32_t* out) {
    const int64_t T = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kUnroll - 1) * T < n16; i += kUnroll * T) {
        u4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = load16<NT>(p + i + u * T);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
    }
    for (; i < n16; i += T) acc ^= fold(load16<NT>(p + i));
    finish(acc, out);
}

// Workgroup g's words [g * n16 / G, (g + 1) * n16 / G).
__device__ __forceinline__ void wg_range(int64_t n16, int64_t& lo, int64_t& hi) {
    const int64_t G = gridDim.x, g = blockIdx.x;
    lo = n16 / G * g + (n16 % G) * g / G;
    hi = n16 / G * (g + 1) + (n16 % G) * (g + 1) / G;
}

// Patterns 2/3: each wave reads 1 KiB pieces of the workgroup's range, the
// workgroup's four waves side by side, kUnroll pieces per wave in flight.
template <bool NT>
__global__ void __launch_bounds__(kThreads) k_range(const u4* __restrict__ p, int64_t n16, uint32_t* out) {
    int64_t lo, hi;
    wg_range(n16, lo, hi);
    uint32_t acc = 0;
    int64_t i = lo + threadIdx.x;
    for (; i + (kUnroll - 1) * kThreads < hi; i += kUnroll * kThreads) {
        u4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = load16<NT>(p + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
    }
    for (; i < hi; i += kThreads) acc ^= fold(load16<NT>(p + i));
    finish(acc, out);
}

// Pattern 4: a wave's unit is 4 KiB (four 1 KiB buffer loads into LDS); the
// wave keeps kRing units in flight in its own LDS window.  The buffer
// descriptor ends at the workgroup range's end, so loads past it return zeros.
constexpr int kRing = 3;
constexpr int kUnitBytes = 4096;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__global__ void __launch_bounds__(kThreads) k_lds(const uint8_t* __restrict__ p, int64_t n16, uint32_t* out) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[kThreads / 64][kRing][kUnitBytes];
    int64_t lo, hi;
    wg_range(n16, lo, hi);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int64_t bytes = (hi - lo) * 16;
    const int64_t units = (bytes + kUnitBytes - 1) / kUnitBytes;
    const uint8_t* base = p + lo * 16;
    auto issue = [&](int64_t u, int slot) {
        const int64_t off = u * kUnitBytes;
        const int64_t left = bytes - off;
        const uint32_t nrec = left <= 0 ? 0u : (left >= 0x7FFFFFFF ? 0x7FFFFFFFu : (uint32_t)left);
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(base + off), (short)0, (int)nrec, 0x00020000);
        uint8_t* dst = ring[wave][slot];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (l_void*)(dst + 1024 * c), 16, 1024 * c + 16 * lane, 0, 0, 2);
    };
    uint32_t acc = 0;
    // units wave, wave + 4, wave + 8, ... of the workgroup's range
    int64_t next = wave;
#pragma unroll
    for (int s = 0; s < kRing; ++s) {
        issue(next, s);  // units past the range load zeros (size 0)
        next += kThreads / 64;
    }
    for (int64_t u = wave; u < units; u += kThreads / 64) {
        const int slot = (int)((u / (kThreads / 64)) % kRing);
        wait_vmcnt<4 * (kRing - 1)>();
        const u4* src = reinterpret_cast<const u4*>(ring[wave][slot]);
        u4 v0 = src[lane], v1 = src[64 + lane], v2 = src[128 + lane], v3 = src[192 + lane];
        __builtin_amdgcn_s_waitcnt(0xC07F);  // the slot's reads are done before it is refilled
        issue(next, slot);
        next += kThreads / 64;
        acc ^= fold(v0) ^ fold(v1) ^ fold(v2) ^ fold(v3);
    }
    wait_vmcnt<0>();
    finish(acc, out);
}

}  // namespace

// Fold every 16-byte word of buf (bytes, a multiple of 16; buf 16-byte
// aligned) into *out (XOR of the words, XOR-ed into *out) with access pattern
// `pattern` (0..4 above) and `wg_per_cu` workgroups of 256 threads per compute
// unit.  Returns 0, or -1 on a bad argument, or the HIP error of the launch.
Q4S_API int q4_stream_read(const void* buf, size_t bytes, uint32_t* out, int pattern, int wg_per_cu, void* stream) {
    if (!buf || !out || bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0) return -1;
    if (pattern < 0 || pattern > 4 || wg_per_cu < 1 || wg_per_cu > 8) return -1;
    if (pattern == 4 && wg_per_cu > 3) return -1;  // 48 KiB of LDS per workgroup
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return -1;
    const int64_t n16 = (int64_t)(bytes / 16);
    const int grid = cus * wg_per_cu;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const u4* p = static_cast<const u4*>(buf);
    switch (pattern) {
        case 0: hipLaunchKernelGGL(k_stride<false>, dim3(grid), dim3(kThreads), 0, s, p, n16, out); break;
        case 1: hipLaunchKernelGGL(k_stride<true>, dim3(grid), dim3(kThreads), 0, s, p, n16, out); break;
        case 2: hipLaunchKernelGGL(k_range<false>, dim3(grid), dim3(kThreads), 0, s, p, n16, out); break;
        case 3: hipLaunchKernelGGL(k_range<true>, dim3(grid), dim3(kThreads), 0, s, p, n16, out); break;
        default:
            hipLaunchKernelGGL(k_lds, dim3(grid), dim3(kThreads), 0, s, static_cast<const uint8_t*>(buf), n16, out);
            break;
    }
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : (int)e;
}
