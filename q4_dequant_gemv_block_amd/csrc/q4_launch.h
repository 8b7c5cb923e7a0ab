// Host-side launchers of the Q4_0 kernels (internal to the library).
// Arguments reaching these functions have been validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

namespace q4 {

// Device-resident descriptor of one GEMV inside a batch plan.
struct PlanDesc {
    const uint8_t* w;
    const uint16_t* x;
    float* y;
    int64_t n;
    int32_t k;
    int32_t npl;         // pairs per lane: ceil(k/64 / 16)
    int64_t steps;       // row steps of the engine's rows per step
    int64_t cost_begin;  // sum of steps*npl over the earlier descriptors
    const float* residual;  // stage hand-off (batch): r [n] or null
    int32_t h16;            // 1: this GEMV is the stage hand-off, y holds binary16(r + y) [n]
    int32_t reserved;
};

// Head of a batch plan's schedule (device memory, first bytes of the plan).
// `next` and `done` are zero between launches: a launch hands out chunks
// grid, grid+1, ... through `next`, counts finished workgroups in `done`, and
// its last workgroup sets both back to zero.
struct SchedHead {
    uint32_t next;
    uint32_t done;
    int32_t nchunks;
    int32_t grid;
};

// One chunk of a batch schedule: the row steps from step s0 of descriptor d0
// on, in list order, that start before cost c_end.
struct SchedChunk {
    int32_t d0;
    int32_t s0;
    int64_t c_end;
};

// Plan flags: the list runs on the quad engine (every k a multiple of 1024, at
// least 4096); the list runs with 8-wave workgroups (its largest k leaves too
// little LDS for 12 waves' rings).
constexpr int kPlanQuad = 1;
constexpr int kPlanWide8 = 2;

// Orders descs[0..count) by row-step size (largest first, stable), fills
// npl, steps and cost_begin and cuts the list into
// chunks for the current device; *grid is the launch's workgroup count (the
// number of chunks assigned statically), *flags the plan flags.
void build_schedule(PlanDesc* descs, int count, std::vector<SchedChunk>* out, int* grid, int* flags);

// Largest k the LDS-staged fast path takes (activation chunks fit in 64 KiB).
constexpr int64_t kFastMaxK = 32768;

// Largest grid (and partial-key count) of the LM-head kernel.
constexpr int kArgmaxMaxBlocks = 2048;

// Keys held in the library's own per-device array for the LM head entry
// point that allocates nothing; *keys receives its device address on the
// current device (looked up on the first call per device).
constexpr int kLmHeadScratchKeys = kArgmaxMaxBlocks;
hipError_t lm_head_scratch(uint64_t** keys);

int device_cu_count();

// Lets `kern` take `bytes` of dynamic LDS on the current device.  The runtime
// call is made once per kernel, device and larger size, not per launch.
hipError_t allow_dynamic_lds(const void* kern, size_t bytes);

hipError_t launch_gemv(const uint8_t* w, const uint16_t* x, float* y, int64_t n, int64_t k,
                       hipStream_t s);
hipError_t launch_gemm_generic(const uint8_t* w, const uint16_t* x, float* y, int64_t m,
                               int64_t n, int64_t k, hipStream_t s);
// One GEMM of a small-M list (device memory, or by value for a single GEMM).
// The fields after k are derived by smallm_fill.
struct SmDesc {
    const uint8_t* w;
    const uint16_t* x;   // m x k
    float* y;            // m x n
    int64_t n;
    int32_t k;
    int32_t np;          // pairs per row (k / 64)
    int32_t P;           // pairs per K-range (a multiple of 16)
    int32_t nranges;     // K-ranges
    int32_t tiles;       // row tiles (256 rows when m > 7, 128 when m <= 7)
    int32_t m;           // activation rows (the engine and its unit size depend on it)
    int64_t ws_off;      // first partial-sum float in the workspace (nranges > 1)
    int64_t cost_begin;  // units of the earlier descriptors
};

// Fills np, P, nranges, tiles, ws_off and cost_begin; returns the workspace
// floats the descriptor's partial sums take (0 with a single K-range).
int64_t smallm_fill(SmDesc* d, int64_t m, int64_t ws_off, int64_t cost_begin);
int64_t smallm_cost(const SmDesc& d);
size_t smallm_workspace_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_smallm(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                              int64_t k, float* workspace, hipStream_t s);
// A single small-M GEMM (m <= 7) whose K fits one K-range, which also writes row mm's
// greedy-pick key of each workgroup b to keys[mm * G + b] (argmax_key: larger
// logit, then lower index; 0 when the workgroup stored none of that row), G =
// smallm_key_slices(m, n, k); that is 0 when m > 7 or K does not fit one range.
int smallm_key_slices(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_smallm_keys(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n, int64_t k,
                                   uint64_t* keys, hipStream_t s);
// descs: `count` filled descriptors in device memory; total: sum of their costs.
hipError_t launch_gemm_smallm_batch(const SmDesc* descs, int count, int64_t m, int64_t total, int max_p,
                                    int64_t max_mn, bool any_split, float* workspace, hipStream_t s);
hipError_t launch_gemm_prefill(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                               int64_t k, hipStream_t s);
// One GEMM of a prefill list (device memory); m, n, k, w, x, y set by the
// caller, the rest by prefill_fill.
struct PfDesc {
    const uint8_t* w;
    const uint16_t* x;  // m x k
    float* y;           // m x n
    int64_t m, n;
    int k;
    int np;             // pairs per weight row (k / 64)
    int mt, nt;         // tiles along M and N
    int64_t tile_begin; // tiles of the earlier descriptors of the list
};
// One XCD's share of a prefill batch: tiles [begin, end) of the list's
// numbering, handed out one at a time through `next`; d_first is the
// descriptor that holds tile `begin`.
struct PfQueue {
    uint32_t next;
    int32_t d_first;
    int64_t begin, end;
    int64_t reserved;
};
constexpr int kPfQueues = 8;  // one per XCD
// Work counters of one kernel's part of a prefill batch plan.  Workgroups on
// XCD x take tiles from q[x] and, once it is empty, from the others in turn;
// `done` counts finished workgroups, and the last one of a launch sets every
// `next` and `done` back to zero, so the plan is ready for the next launch.
struct PfHead {
    uint32_t done;
    uint32_t reserved[7];
    PfQueue q[kPfQueues];
};
int prefill_batch_tile_m(int64_t m);
// Tile rows of the k % 256 != 0 part of a batch whose k % 256 == 0 part uses tile_m.
int prefill_other_tile_m(int tile_m);
int64_t prefill_fill(PfDesc* d, int tile_m, int64_t tile_begin);
// Cuts tiles [0, tiles) of `count` filled descriptors into the kPfQueues
// queues of *head: contiguous ranges of about equal work (tiles weighted by
// k), each starting at an N-tile, so every M-tile of a weight tile is run on
// one XCD.  `next` and `done` are left zero.
void prefill_queues(const PfDesc* descs, int count, int64_t tiles, PfHead* head);
// `plan`: two PfHead, then the `n_chunked` descriptors with k % 256 == 0
// (the kernel that moves weights in 144-byte chunks; tile numbers from 0),
// then the `n_other` others (tile numbers from 0).
hipError_t launch_gemm_prefill_batch(void* plan, int n_chunked, int64_t tiles_chunked, int n_other,
                                     int64_t tiles_other, int tile_m, hipStream_t s);
int argmax_blocks(int64_t n, int64_t k);
// Greedy verify of a draft (verify.hip): small-M logits (the GEMV for m = 1),
// row argmax keys, tokens and the accepted prefix; workspace as below.
size_t verify_workspace_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_lm_head_verify(const uint8_t* w, const uint16_t* h, float* logits, int32_t* tokens,
                                 const int32_t* draft, int32_t* accepted, int64_t m, int64_t n, int64_t k,
                                 void* workspace, hipStream_t s);
hipError_t launch_lm_head(const uint8_t* w, const uint16_t* h, float* logits, int32_t* token,
                          int64_t n, int64_t k, uint64_t* keys, hipStream_t s);
// Q8_0 GEMV (q8.hip): any k % 32 == 0 up to kFastMaxK, w 4-byte aligned, x 16-byte aligned.
hipError_t launch_q8_gemv(const uint8_t* w, const uint16_t* x, float* y, int64_t n, int64_t k, hipStream_t s);
// Q8_0 on the sweep kernel's slab engine (gemv.hip): k % 512 == 0, 2048 <= k <= 28672,
// w 16-byte aligned, x 16-byte aligned.  The library routes a GEMV there exactly
// when q8_slab_ok(k) holds and w is 16-byte aligned, single calls and lists alike.
bool q8_slab_ok(int64_t k);
hipError_t launch_q8_slab_gemv(const uint8_t* w, const uint16_t* x, float* y, int64_t n, int64_t k, hipStream_t s);
// A list on the slab engine: orders descs[0..count) (npl, steps and cost_begin
// filled as for the Q4_0 list, in units of 64-pair slabs) and cuts the
// schedule; returns the grid.  The plan in device memory: SchedHead, the
// `count` PlanDesc, the chunks.
int build_schedule_q8(PlanDesc* descs, int count, std::vector<SchedChunk>* out);
hipError_t launch_q8_slab_batch(const void* plan, int count, int grid, hipStream_t s);
// A Q8_0 GEMV list in one launch.  The plan in device memory: a Q8Head, then
// `count` Q8Desc, then grid + 1 int64 unit indices (workgroup g first takes
// units [b[g], b[g+1])); a unit is kQ8UnitRows consecutive rows of one GEMV.
// Units from dyn_begin on are handed out `chunk` at a time through `next`;
// `done` counts finished workgroups, the last one sets both back to zero.
struct Q8Head {
    uint32_t next, done;
    int32_t chunk, reserved;
    int64_t dyn_begin, dyn_end;
};
struct Q8Desc {
    const uint8_t* w;
    const uint16_t* x;
    float* y;
    int64_t n;
    int32_t k;
    int32_t reserved;
    int64_t unit_begin;  // index of this GEMV's first unit in the list
};
constexpr int kQ8UnitRows = 16;
constexpr int kQ8WgPerCu = 2;  // the launch grid is at most this many workgroups per compute unit
// Fills unit_begin, the head's dynamic part and the workgroups' first unit
// ranges (contiguous, byte-balanced); returns the grid.
int q8_batch_layout(Q8Desc* descs, int count, std::vector<int64_t>* wg_begin, Q8Head* head);
hipError_t launch_q8_batch(void* plan, int count, int grid, int max_k, hipStream_t s);
// A GEMV whose epilogue writes binary16(residual + y) (residual may be null).
hipError_t launch_gemv_handoff(const uint8_t* w, const uint16_t* x, const float* residual, uint16_t* h16,
                               int64_t n, int64_t k, hipStream_t s);
// The LM head with the final norm applied while h is staged (x_out may be null).
hipError_t launch_lm_head_norm(const uint8_t* w, const uint16_t* h, const uint16_t* gamma, float eps,
                               uint16_t* x_out, float* logits, int32_t* token, int64_t n, int64_t k, uint64_t* keys,
                               hipStream_t s);
// `plan`: SchedHead, then `count` PlanDesc, then `nchunks` SchedChunk.
hipError_t launch_gemv_batch(const void* plan, int count, int nchunks, int grid, int max_k, int flags,
                             hipStream_t s);

}  // namespace q4
