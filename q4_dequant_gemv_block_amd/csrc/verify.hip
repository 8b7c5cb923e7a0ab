// Greedy verify of a speculative draft: logits[i][n] = sum_k w[n][k] h[i][k]
// for the m <= 16 rows of h (the trunk's hidden states at the draft's
// positions), tokens[i] = lowest n among the largest logits[i][n], and
// accepted = the number of leading rows i with tokens[i] == draft[i].
//
// The trunk checks all the tokens a draft proposed in one batched pass
// (aipolix.com SwarmLLM page, section "Speculation is used to amortize network
// round trips"); decoding is greedy (taozi.news, section "基准成绩").  The
// logits come from the small-M GEMM (one pass over the vocabulary's weights
// for all m rows; the GEMV for m = 1); each row's logits are reduced to
// 64-bit keys (argmax_key: larger logit first, then lower index), by the
// small-M kernel itself as it stores them (one key per workgroup and row)
// when K fits one K-range, else by a pass over row slices; then one
// workgroup picks each row's token and counts the accepted prefix.
#include "q4_device.h"
#include "q4_launch.h"

#include <algorithm>

namespace q4 {

namespace {

constexpr int kRowThreads = 256;

// keys[i * B + b] = max key over slice b of row i (blockIdx.x = b, blockIdx.y = i).
__global__ void __launch_bounds__(kRowThreads) k_argmax_rows(const float* __restrict__ logits, int64_t n,
                                                            uint64_t* __restrict__ keys) {
    __shared__ uint64_t sh[kRowThreads / 64];
    const int64_t B = gridDim.x;
    const int64_t lo = n * blockIdx.x / B, hi = n * (blockIdx.x + 1) / B;
    const float* row = logits + (int64_t)blockIdx.y * n;
    uint64_t best = 0;
    for (int64_t j = lo + threadIdx.x; j < hi; j += kRowThreads) {
        const uint64_t kk = argmax_key(row[j], j);
        best = kk > best ? kk : best;
    }
    const uint64_t b = block_max_u64(best, sh);
    if (threadIdx.x == 0) keys[(int64_t)blockIdx.y * B + blockIdx.x] = b;
}

// One workgroup of 16 waves: wave i reduces row i's B keys to tokens[i]
// (rows run side by side), then one thread counts the accepted prefix.
constexpr int kFinalWaves = 16;
__global__ void __launch_bounds__(kFinalWaves * 64) k_verify_final(const uint64_t* __restrict__ keys, int B, int m,
                                                                  const int32_t* __restrict__ draft,
                                                                  int32_t* __restrict__ tokens,
                                                                  int32_t* __restrict__ accepted) {
    __shared__ int32_t tok[kFinalWaves];
    const int i = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (i < m) {
        uint64_t best = 0;
        for (int b = lane; b < B; b += 64) {
            const uint64_t v = keys[(int64_t)i * B + b];
            best = v > best ? v : best;
        }
        best = wave_max_u64(best);
        if (lane == 0) {
            tok[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
            tokens[i] = tok[i];
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int a = 0;
        while (a < m && tok[a] == draft[a]) ++a;
        accepted[0] = a;
    }
}

// Slices per row: about 2,048 logits each, at most 256.
int verify_slices(int64_t n) { return (int)std::max<int64_t>(1, std::min<int64_t>(256, (n + 2047) / 2048)); }

}  // namespace

// Keys per row: the separate pass's slices, or the small-M kernel's
// workgroups when it writes them itself (at most kArgmaxMaxBlocks).
static int key_slots(int64_t n) { return std::max(verify_slices(n), kArgmaxMaxBlocks); }

size_t verify_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    const size_t gemm = m >= 2 ? (smallm_workspace_bytes(m, n, k) + 255) / 256 * 256 : 0;
    return gemm + (size_t)m * key_slots(n) * sizeof(uint64_t);
}

hipError_t launch_lm_head_verify(const uint8_t* w, const uint16_t* h, float* logits, int32_t* tokens,
                                 const int32_t* draft, int32_t* accepted, int64_t m, int64_t n, int64_t k,
                                 void* workspace, hipStream_t s) {
    const size_t gemm = m >= 2 ? (smallm_workspace_bytes(m, n, k) + 255) / 256 * 256 : 0;
    uint64_t* keys = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(workspace) + gemm);
    // m >= 2 with K in one range (the LM head's): the small-M kernel writes the
    // keys of the logits it stores, one per workgroup and row.
    const int fused = m >= 2 ? smallm_key_slices(m, n, k) : 0;
    int B;
    hipError_t e;
    if (fused > 0 && fused <= key_slots(n)) {
        e = launch_gemm_smallm_keys(w, h, logits, m, n, k, keys, s);
        B = fused;
    } else {
        e = m >= 2 ? launch_gemm_smallm(w, h, logits, m, n, k, static_cast<float*>(workspace), s)
                   : launch_gemv(w, h, logits, n, k, s);
        if (e != hipSuccess) return e;
        B = verify_slices(n);
        hipLaunchKernelGGL(k_argmax_rows, dim3(B, (unsigned)m), dim3(kRowThreads), 0, s, logits, n, keys);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_verify_final, dim3(1), dim3(kFinalWaves * 64), 0, s, keys, B, (int)m, draft, tokens, accepted);
    return hipGetLastError();
}

}  // namespace q4
