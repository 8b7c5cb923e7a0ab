// Device-side building blocks for the Q4_0 kernels (gfx950, wave64).
//
// Q4_0 block (the format the pages call "GGUF Q4_0"; taozi.news, section
// "支持模型与限制"): 18 bytes = f16 scale d, then 16 code bytes, byte j holding
// code j (low nibble) and code j+16 (high nibble); weight = (code - 8) * d.
//
// Two consecutive blocks ("a pair", 36 bytes) start on a 4-byte boundary
// whenever the row stride is a multiple of 4 (K % 64 == 0), so a lane reads a
// pair as nine dwords D0..D8:
//   D0 = [d0 lo, d0 hi, c0, c1]      block 0 scale and code bytes 0-1
//   D1..D3 = block 0 code bytes 2..13
//   D4 = [c14, c15, d1 lo, d1 hi]    block 0 code bytes 14-15, block 1 scale
//   D5..D8 = block 1 code bytes 0..15
// Block 0's code bytes are re-aligned with one byte permute:
//   E0 = [c14, c15, c0, c1] = perm(D0, D4), E1..E3 = D1..D3.
//
// A code dword V with bytes (codes a, b, c, e in the low nibbles and a+16,
// b+16, c+16, e+16 in the high nibbles) expands to four f16 pairs with exact
// values code - 8, in eight operations and no shift:
//   L02 = (V & 0x00FF00FF) | 0x6400 6400       -> 1024 + byte, bytes 0 and 2
//   L13 = byte permute [V.1, 0x64, V.3, 0x64]  -> 1024 + byte, bytes 1 and 3
//   H   = (L & 0x00F000F0) | 0x5408 5408       -> 64.5 + high nibble
//   low  - 8 = L - 16 H   (one packed f16 fma)
//   high - 8 = H - 72.5   (one packed f16 add)
// (0x6400 is 1024.0 with unit spacing, so a byte under it adds exactly its
// value; 0x5400 is 64.0 with spacing 1/16, so a nibble in bits 4-7 adds
// exactly its value and bit 3 adds 0.5.  Every intermediate is a multiple of
// 1/2 below 2048 in magnitude and every result an integer in [-8, 7], all
// exact in f16.)  The pairs come out as
//   (a, c), (a+16, c+16), (b, e), (b+16, e+16).
// Each pair then meets the matching pair of activations in one v_dot2 (f16 x
// f16 products are exact in f32; sums round in f32), and the block sum is
// scaled once by d.
//
// The activations are therefore stored, per code dword, as the four f16
// pairs (x_a, x_c), (x_a+16, x_c+16), (x_b, x_e), (x_b+16, x_e+16): one 16-byte
// "chunk".  A pair of blocks has 8 chunks; in LDS chunk c of pair p lives at
// index c * npp + p (npp = pairs rounded up to a multiple of 16), so the 16
// lanes that share a row read 16 consecutive chunks (no bank conflicts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u2a4 __attribute__((ext_vector_type(2), aligned(4)));

constexpr int kWave = 64;
constexpr int kLanesPerRow = 16;   // one DPP row of lanes shares a weight row
constexpr int kPairBytes = 36;
constexpr int kBlockBytes = 18;
constexpr int kChunksPerPair = 8;

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// (v & mask) | bias as one v_and_or_b32; gfx9 VOP3 takes no literal, so the
// mask rides in an SGPR and the bias in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask, uint32_t bias) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(mask), "v"(bias));
    return r;
}

// Block 0 of a pair: code bytes 14,15 (low half of D4) then 0,1 (high half of D0).
__device__ __forceinline__ uint32_t realign_block0(uint32_t d0, uint32_t d4) {
    return __builtin_amdgcn_perm(d0, d4, 0x07060100u);
}

// Four exact (code - 8) f16 pairs of one code dword, in chunk order.
struct Codes4 {
    h2 q0, q1, q2, q3;
};

__device__ __forceinline__ Codes4 expand(uint32_t v) {
    const h2 m16 = {(_Float16)-16.0f, (_Float16)-16.0f};
    const h2 c72h = {(_Float16)72.5f, (_Float16)72.5f};
    // the four bit-level steps first, then the four packed f16 steps: a packed
    // read right after the VALU write of its operand costs a wait state
    const uint32_t l02 = and_or(v, 0x00FF00FFu, 0x64006400u);
    const uint32_t l13 = __builtin_amdgcn_perm(0x64646464u, v, 0x04030401u);
    const uint32_t h02 = and_or(v, 0x00F000F0u, 0x54085408u);
    const uint32_t h13 = and_or(l13, 0x00F000F0u, 0x54085408u);
    Codes4 r;
    r.q0 = __builtin_elementwise_fma(as_h2(h02), m16, as_h2(l02));
    r.q2 = __builtin_elementwise_fma(as_h2(h13), m16, as_h2(l13));
    r.q1 = as_h2(h02) - c72h;
    r.q3 = as_h2(h13) - c72h;
    return r;
}

__device__ __forceinline__ float dot_chunk(const Codes4& q, u4 x, float s) {
    s = __builtin_amdgcn_fdot2(q.q0, as_h2(x.x), s, false);
    s = __builtin_amdgcn_fdot2(q.q1, as_h2(x.y), s, false);
    s = __builtin_amdgcn_fdot2(q.q2, as_h2(x.z), s, false);
    s = __builtin_amdgcn_fdot2(q.q3, as_h2(x.w), s, false);
    return s;
}

// a + d * s with d the f16 in the low (fma_lo) or high (fma_hi) half of w, one
// rounding (the f16 widens exactly).
__device__ __forceinline__ float fma_lo(uint32_t w, float s, float a) {
    return __builtin_fmaf((float)as_h2(w).x, s, a);
}
__device__ __forceinline__ float fma_hi(uint32_t w, float s, float a) {
    return __builtin_fmaf((float)as_h2(w).y, s, a);
}

__device__ __forceinline__ float f16_lo(uint32_t v) { return (float)as_h2(v).x; }
__device__ __forceinline__ float f16_hi(uint32_t v) { return (float)as_h2(v).y; }

typedef __attribute__((address_space(1))) const u4a4 g_u4a4;
typedef __attribute__((address_space(1))) const uint32_t g_u32;
typedef __attribute__((address_space(1))) const u4 g_u4;

// One pair of blocks at a 4-byte aligned global address, as two dwordx4 and
// one dword load.  Ordinary (cached) loads on purpose: the 16 lanes of a row
// read pairs at a 36-byte stride, so every 128-byte line is touched by more
// than one of the three instructions, and with the non-temporal hint each
// touch refetches the line (measured 3.9 TB/s with the hint, 6.2 without, on
// a load-only copy of this pattern).
__device__ __forceinline__ void load_pair(const uint8_t* p, uint32_t (&D)[9]) {
    const u4a4 a = *(g_u4a4*)p;
    const u4a4 b = *(g_u4a4*)(p + 16);
    const uint32_t c = *(g_u32*)(p + 32);
    D[0] = a.x; D[1] = a.y; D[2] = a.z; D[3] = a.w;
    D[4] = b.x; D[5] = b.y; D[6] = b.z; D[7] = b.w;
    D[8] = c;
}

// Sum over the 16 lanes of a DPP row, in a fixed order; every lane gets a
// value, lane 0 of the row holds ((v0+v1)+(v2+v3)) + ... in the same order for
// every row, so equal rows give equal sums wherever they sit.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_mov<0x124>(v);  // row_ror:4
    v += dpp_mov<0x128>(v);  // row_ror:8
    return v;
}

// Activation chunk c (0..7) of pair p from 64 f16 values x[0..63] of that pair.
// Code-dword byte positions (low-nibble codes a, b, c, e):
//   chunk 0: 14, 15, 0, 1 (re-aligned block 0); chunks 1..3: 4c-2 .. 4c+1;
//   chunks 4..7: block 1, positions 4(c-4) .. 4(c-4)+3, offset 32.
__host__ __device__ inline void chunk_positions(int c, int (&pos)[4]) {
    if (c == 0) {
        pos[0] = 14; pos[1] = 15; pos[2] = 0; pos[3] = 1;
    } else if (c < 4) {
        pos[0] = 4 * c - 2; pos[1] = 4 * c - 1; pos[2] = 4 * c; pos[3] = 4 * c + 1;
    } else {
        const int b = 32 + 4 * (c - 4);
        pos[0] = b; pos[1] = b + 1; pos[2] = b + 2; pos[3] = b + 3;
    }
}

// Greedy pick: the maximum of these keys over a set of (logit, index) is the
// lowest index among the largest logits.
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

}  // namespace q4
