// Host-side launchers of the Q4_0 kernels (internal to the library).
// Arguments reaching these functions have been validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q4 {

// Device-resident descriptor of one GEMV inside a batch plan.
struct PlanDesc {
    const uint8_t* w;
    const uint16_t* x;
    float* y;
    int64_t n;
    int32_t k;
    int32_t npl;         // pairs per lane: ceil(k/64 / 16)
    int64_t steps;       // row steps of kBatchRows rows
    int64_t cost_begin;  // sum of steps*npl over the earlier descriptors
};

// Rows one workgroup step covers in the batch kernel (4 waves x 4 rows x R).
int batch_rows_per_step();

// Largest k the LDS-staged fast path takes (activation chunks fit in 64 KiB).
constexpr int64_t kFastMaxK = 32768;

// Largest grid (and partial-key count) of the LM-head kernel.
constexpr int kArgmaxMaxBlocks = 2048;

int device_cu_count();

hipError_t launch_gemv(const uint8_t* w, const uint16_t* x, float* y, int64_t n, int64_t k,
                       hipStream_t s);
hipError_t launch_gemm_generic(const uint8_t* w, const uint16_t* x, float* y, int64_t m,
                               int64_t n, int64_t k, hipStream_t s);
void smallm_split(int64_t n, int64_t k, int* splits, int* cps);
size_t smallm_workspace_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_smallm(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                              int64_t k, float* workspace, hipStream_t s);
hipError_t launch_gemm_prefill(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                               int64_t k, hipStream_t s);
int argmax_blocks(int64_t n, int64_t k);
hipError_t launch_lm_head(const uint8_t* w, const uint16_t* h, float* logits, int32_t* token,
                          int64_t n, int64_t k, uint64_t* keys, hipStream_t s);
hipError_t launch_gemv_batch(const PlanDesc* descs, int count, int64_t total_cost, int max_k,
                             bool all_k1024, hipStream_t s);

}  // namespace q4
