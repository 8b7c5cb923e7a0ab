/*
 * q4gemv.h - C ABI of the Q4_0 dequantize-and-multiply library for MI355X (gfx950).
 *
 * The operation: the decode engine's matrix-vector product over 4-bit block
 * quantized weights, where decode streams every layer's weights once per
 * token, expands the 4-bit values in registers and reduces the row products
 * on chip ("Every Device Brings a Slice: How SwarmLLM Runs a 27B Model Across
 * Browser Tabs", originshq.com, section "The Engine: ~50 WGSL Kernels Written
 * From Scratch").  The weight format is the one the pages call "GGUF Q4_0"
 * (taozi.news, section "支持模型与限制"):
 *
 *   - a weight row of K columns (K % 32 == 0) is K/32 blocks of 18 bytes,
 *     blocks consecutive along K, rows consecutive (row stride K/32*18 bytes);
 *   - block bytes 0..1: scale d, IEEE binary16, little-endian;
 *   - block bytes 2..17: byte j holds code j in its low nibble and code j+16
 *     in its high nibble;
 *   - weight = (code - 8) * d.
 *
 * Activations are IEEE binary16, outputs IEEE binary32.  For every output the
 * result lies within 1e-3 * sum_k |w_k x_k| of the exact sum.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or keeps them; nothing is retained after
 *     the call returns.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL means the null stream).  No call synchronizes the host,
 *     except the four ..._batch_plan calls and q4_0_gemv_batch_handoff (see
 *     there).
 *   - Outputs are overwritten.  Outputs must not overlap any input.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing has been launched and the output is untouched.
 *   - Thread safety: calls may come from several host threads.  The only
 *     library state is the per-thread text returned by q4_last_error().
 *   - Alignment: w and x (h) must be 16-byte aligned, outputs 4-byte aligned
 *     (fresh torch / hipMalloc allocations are 256-byte aligned).
 */
#ifndef Q4GEMV_H
#define Q4GEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define Q4_API __attribute__((visibility("default")))
#else
#define Q4_API
#endif

#define Q4_ABI_VERSION 1

typedef int q4_status;
#define Q4_OK 0
#define Q4_ERR_INVALID_ARG -1 /* null pointer, size <= 0, K % 32 != 0, M outside the entry point's range */
#define Q4_ERR_MISALIGNED -2  /* w or x not 16-byte aligned, or an output not 4-byte aligned */
#define Q4_ERR_WORKSPACE -3   /* workspace missing or smaller than q4_workspace_bytes() */
#define Q4_ERR_HIP -4         /* the HIP runtime refused a launch or copy; text in q4_last_error() */

/* Operation ids for q4_workspace_bytes(). */
#define Q4_OP_GEMV 0
#define Q4_OP_GEMM_SMALLM 1
#define Q4_OP_GEMM_PREFILL 2
#define Q4_OP_LM_HEAD_ARGMAX 3
#define Q4_OP_LM_HEAD_VERIFY 4
#define Q4_OP_LM_HEAD_NORM_ARGMAX 5

/* Version of this interface (Q4_ABI_VERSION of the library that was built). */
Q4_API int q4_abi_version(void);

/* Text of the last error on the calling thread ("" if none); valid until the
 * next call into the library on the same thread. */
Q4_API const char* q4_last_error(void);

/* Bytes of device workspace an entry point needs for the given shape (0 when
 * it needs none).  Returns 0 for an unknown op. */
Q4_API size_t q4_workspace_bytes(int op, int64_t m, int64_t n, int64_t k);

/*
 * y[n] = sum_k w[n][k] * x[k]                         (one Q4_0 GEMV, M = 1)
 *
 * The per-token product of the decode engine (originshq.com page, section
 * "The Engine: ~50 WGSL Kernels Written From Scratch").
 *   w : n rows of k/32 Q4_0 blocks (n * k/32 * 18 bytes)
 *   x : k binary16 values
 *   y : n binary32 values (written)
 *   n >= 1, k >= 32, k % 32 == 0.  k % 64 == 0 takes the fast path; other
 *   multiples of 32 take a slower path with the same results bound.
 * Deterministic: identical inputs give bit-identical outputs, and two rows
 * with identical bytes give bit-identical outputs wherever they sit.
 */
Q4_API q4_status q4_0_gemv(const void* w, const void* x, float* y, int64_t n, int64_t k, void* stream);

/*
 * Y[m][n] = sum_k w[n][k] * X[m][k]                   (small-M batched GEMM)
 *
 * The batched pass that verifies speculative drafts and carries 16-token
 * prefill chunks (aipolix.com en-us page, section "Speculation is used to
 * amortize network round trips"; taozi.news, section "技术架构").  Each
 * weight is read from memory and expanded once for all M rows.  For m >= 2
 * the products run on the matrix cores with (code - 8) * d rounded once to
 * binary16 (relative error <= 2^-11 per weight); m == 1 is q4_0_gemv.
 *   w : n rows of k/32 Q4_0 blocks
 *   x : m x k binary16, row-major
 *   y : m x n binary32, row-major (written)
 *   1 <= m <= 16, n >= 1, k >= 32, k % 32 == 0.  |d| <= 8188 (so that
 *   (code - 8) * d is finite in binary16).
 *   workspace : q4_workspace_bytes(Q4_OP_GEMM_SMALLM, m, n, k) bytes of
 *               device memory (may be NULL when that is 0); contents on entry
 *               do not matter.
 * Row m of the result satisfies the same bound as q4_0_gemv on X[m].
 * Deterministic for a given shape.
 */
Q4_API q4_status q4_0_gemm_smallm(const void* w, const void* x, float* y,
                                  int64_t m, int64_t n, int64_t k,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Y[m][n] = sum_k w[n][k] * X[m][k]                   (prefill GEMM, matrix cores)
 *
 * The prompt-processing matrix product (taozi.news, section "基准成绩";
 * originshq.com page, section "The Engine ...").  Weight tiles are expanded
 * to binary16 ((code - 8) * d rounded to nearest) on chip and multiplied on
 * the matrix cores with binary32 accumulation.
 *   w : n rows of k/32 Q4_0 blocks
 *   x : m x k binary16, row-major
 *   y : m x n binary32, row-major (written)
 *   m >= 1, n >= 1, k >= 32, k % 32 == 0.  |d| <= 8188.
 *   workspace : q4_workspace_bytes(Q4_OP_GEMM_PREFILL, m, n, k) bytes of
 *               device memory (may be NULL when that is 0).
 */
Q4_API q4_status q4_0_gemm_prefill(const void* w, const void* x, float* y,
                            int64_t m, int64_t n, int64_t k,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * logits[n] = sum_k w[n][k] * h[k];  token = lowest n with the largest logit
 *
 * The host's LM-head projection followed by the greedy pick (originshq.com
 * page, section "The Architecture: Layers Distributed, Activations in
 * Flight"; greedy decoding: taozi.news, section "基准成绩").  -0 and +0
 * compare equal.
 *   w      : n_vocab rows of k/32 Q4_0 blocks
 *   h      : k binary16 values
 *   logits : n_vocab binary32 values (written)
 *   token  : one int32 in device memory (written)
 *   workspace : q4_workspace_bytes(Q4_OP_LM_HEAD_ARGMAX, 1, n_vocab, k) bytes
 *               of device memory, 8-byte aligned; its contents on entry do not
 *               matter.
 *   n_vocab >= 1, k % 64 == 0, 64 <= k <= 32768, w 16-byte aligned (other k:
 *   Q4_ERR_INVALID_ARG).  Inputs must be finite.
 */
Q4_API q4_status lm_head_argmax(const void* w, const void* h, float* logits, int32_t* token,
                         int64_t n_vocab, int64_t k,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * lm_head_argmax without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same operation, kernels and results as lm_head_argmax
 * (logits and token bit-identical); w, h, logits, token, n_vocab and k as
 * there.  The per-workgroup keys live in an array the library holds on each
 * device until the process ends (2048 keys, 16 KiB per device); every grid
 * this call launches fits it, so no size is refused for it.  The call
 * allocates nothing: no hipMalloc, no hipFree, no library routine that
 * allocates.  Its first call on a device looks the array's address up there
 * (Q4_ERR_HIP if that fails).  All calls on one device share that array, so
 * calls that overlap in time on one device (on different streams, or from
 * different host threads without ordering) race and may return a wrong
 * token; calls ordered on one stream do not.  Nothing in the array needs
 * clearing: each call writes the keys it reads.
 */
Q4_API q4_status lm_head_argmax_noalloc(const void* w, const void* h, float* logits, int32_t* token,
                                        int64_t n_vocab, int64_t k, void* stream);

/*
 * y[n] = sum_k w[n][k] * x[k]  with w in Q8_0 blocks
 *
 * The pages' other weight format, "GGUF Q8_0", used by the small dense Qwen3
 * models (taozi.news, section "支持模型与限制"); the pages name it only.
 * Read as: a row of k weights is k/32 blocks of 34 bytes; bytes 0..1 of a
 * block are the scale d (binary16, little-endian), bytes 2..33 the 32 codes
 * as two's-complement signed bytes; weight j = code_j * d.  Same boundary
 * and bound as q4_0_gemv: |y - y_exact| <= 1e-3 * sum_k |w x| per row
 * (binary32 sums, one fixed association per row).
 *   w : n rows of k/32 Q8_0 blocks, 4-byte aligned (rows follow each other;
 *       a row starts 2 bytes into a dword when k/32 is odd)
 *   x : k binary16 values, 16-byte aligned;  y : n binary32 (written)
 *   n >= 1, k % 32 == 0, 32 <= k <= 32768.  Inputs finite.  y must not
 *   overlap w or x.
 * Two kernels, chosen by shape alone: k % 512 == 0 with 2048 <= k <= 28672
 * and w 16-byte aligned streams whole 64-pair slabs of 8-row groups through
 * LDS; any other shape reads each block through its own lane.  The two sum
 * a row in different orders (both within the bound); a row's result depends
 * only on its bytes, x and which kernel its shape selects.
 */
Q4_API q4_status q8_0_gemv(const void* w, const void* x, float* y, int64_t n, int64_t k, void* stream);

/*
 * h16[n] = binary16(residual[n] + sum_k w[n][k] * x[k]), rounded to nearest,
 * ties to even
 *
 * The hand-off at the end of a stage's layer range: the device converts the
 * hidden state it produced to f16 and sends it to the next participant
 * (aipolix.com en-us page, section "A model can be larger than any one
 * browser can hold"; 5,120 values, about 10 KB per hop).  Read as the
 * epilogue of the range's last GEMV (the down projection) with the residual
 * stream added first: the binary32 sum of q4_0_gemv (same kernel, same
 * association, so h16 equals the rounding of q4_0_gemv's y plus the residual
 * bit for bit) plus residual[n] in binary32, then one rounding to binary16.
 *   w        : n rows of k/32 Q4_0 blocks, 16-byte aligned
 *   x        : k binary16 values, 16-byte aligned
 *   residual : NULL (zero) or n binary32 values, 4-byte aligned
 *   h16      : n binary16 values (written), 2-byte aligned
 *   n >= 1, k % 64 == 0, 64 <= k <= 32768 (other k: Q4_ERR_INVALID_ARG).
 *   Inputs finite; |residual + y| >= 65520 gives an infinite h16.  h16 must
 *   not overlap an input.
 */
Q4_API q4_status q4_0_gemv_handoff(const void* w, const void* x, const float* residual, void* h16, int64_t n,
                                   int64_t k, void* stream);

/*
 * x = final_norm(h);  logits[n] = sum_k w[n][k] * x[k];  token = lowest n
 * with the largest logit
 *
 * The host normalises the hidden state the last stage returns, then applies
 * the LM head and the greedy pick (originshq.com page, section "The
 * Architecture: Layers Distributed, Activations in Flight"; taozi.news,
 * section "技术架构").  The norm is read as RMS normalisation with a gain:
 *   r = 1 / sqrt(mean over k of h[k]^2 + eps),  x[k] = binary16(h[k] r gamma[k])
 * rounded to nearest, ties to even; the statistics are taken in binary32.  It
 * runs inside the LM head's kernel (each workgroup normalises the 10 KB
 * hidden state while staging it; there is no separate pass).  Each x[k] is
 * the binary16 nearest to the binary64 value or, when that value lies within
 * about 2^-20 of a rounding midpoint, its other neighbour; the logits then
 * satisfy the bound of q4_0_gemv with x as the activation.
 *   w      : n_vocab rows of k/32 Q4_0 blocks
 *   h      : k binary16 values (the hidden state)
 *   gamma  : k binary16 values (the norm's gain), 16-byte aligned
 *   eps    : finite, > 0
 *   logits : n_vocab binary32 values (written)
 *   token  : one int32 in device memory (written)
 *   x_out  : NULL, or k binary16 in device memory, 16-byte aligned, that
 *            receive x (written)
 *   workspace : q4_workspace_bytes(Q4_OP_LM_HEAD_NORM_ARGMAX, 1, n_vocab, k)
 *               bytes of device memory, 8-byte aligned; contents on entry do
 *               not matter.
 *   n_vocab >= 1, k % 64 == 0, 64 <= k <= 32768, w 16-byte aligned.  Inputs
 *   finite, and |h[k] r gamma[k]| below 65520 (else x[k] is infinite).  No
 *   output may overlap another output or an input.
 */
Q4_API q4_status lm_head_norm_argmax(const void* w, const void* h, const void* gamma, float eps, float* logits,
                                     int32_t* token, void* x_out, int64_t n_vocab, int64_t k,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * logits[i][n] = sum_k w[n][k] * h[i][k];  tokens[i] = lowest n with the
 * largest logits[i][n];  *accepted = the number of leading i (from 0) with
 * tokens[i] == draft[i]
 *
 * Greedy verify of a speculative draft: the trunk checks every token a draft
 * proposed in one batched pass over the LM head's weights (aipolix.com
 * SwarmLLM page, section "Speculation is used to amortize network round
 * trips"; greedy decoding: taozi.news, section "基准成绩").  Row i of h is the
 * trunk's hidden state at the position the draft filled with draft[i]; the
 * caller keeps draft[0 .. accepted) and, when accepted < m, takes
 * tokens[accepted] in place of the rejected one.  The logits of row i satisfy
 * the bound of q4_0_gemm_smallm (q4_0_gemv for m == 1); tokens[i] is the
 * lowest index among the maxima of the returned logits[i] (-0 and +0 equal).
 *   w        : n_vocab rows of k/32 Q4_0 blocks
 *   h        : m x k binary16, row-major
 *   logits   : m x n_vocab binary32 (written)
 *   tokens   : m int32 (written);  draft : m int32 (read);  accepted : 1 int32
 *              (written); all in device memory, 4-byte aligned
 *   workspace : q4_workspace_bytes(Q4_OP_LM_HEAD_VERIFY, m, n_vocab, k) bytes
 *               of device memory, 16-byte aligned; contents on entry do not
 *               matter.
 *   1 <= m <= 16, n_vocab >= 1, k % 64 == 0, w and h 16-byte aligned.  Inputs
 *   finite.  No output may overlap another output or an input.
 */
Q4_API q4_status lm_head_verify(const void* w, const void* h, float* logits, int32_t* tokens,
                                const int32_t* draft, int32_t* accepted, int64_t m, int64_t n_vocab, int64_t k,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * A list of independent GEMVs run as ONE launch ("one command submit per
 * token": originshq.com page, section "The Engine ...").  A whole decode
 * weight sweep (every layer's projections) streams through a single
 * persistent kernel instead of hundreds of launches.
 *
 * Each descriptor is one y = W x as in q4_0_gemv (k % 64 == 0 here).  The
 * GEMVs must be independent: no y may overlap any w, x or other y of the
 * list.
 */
typedef struct q4_gemv_desc {
    const void* w;  /* n rows of k/32 Q4_0 blocks, 16-byte aligned */
    const void* x;  /* k binary16, 16-byte aligned */
    float* y;       /* n binary32, written */
    int64_t n;
    int64_t k;
} q4_gemv_desc;

/* Host-side handle of a batch plan.  Filled by q4_0_gemv_batch_plan; plain
 * data, may be copied. */
typedef struct q4_gemv_plan {
    void* device;  /* the caller's device buffer holding the plan */
    int count;     /* number of GEMVs */
    int max_k;     /* largest k in the list */
    int grid;      /* workgroups of one launch */
    int nchunks;   /* pieces of work in the plan's schedule */
    int flags;     /* internal: the kernel layout the schedule was made for */
} q4_gemv_plan;

/* Device bytes q4_0_gemv_batch_plan needs for this descriptor list (the size
 * depends on the shapes and on the current device's compute-unit count).
 * Returns 0, with q4_last_error() set, if the list is not valid. */
Q4_API size_t q4_0_gemv_batch_plan_bytes(const q4_gemv_desc* descs, int count);

/*
 * Validate `count` host-side descriptors and write the plan into the caller's
 * device buffer `plan_buf` (at least q4_0_gemv_batch_plan_bytes(descs, count)
 * bytes, 16-byte aligned), then fill `*plan`.  The plan holds the
 * descriptors, a schedule that cuts the list's row steps into chunks (one per
 * workgroup first, then smaller ones that workgroups take as they finish), and
 * two counters the launch uses to hand the chunks out; the counters are zero
 * between launches.  The copy is enqueued on `stream` and has completed when
 * this call returns (it synchronizes `stream`), so `descs` may be freed
 * afterwards.  The plan stays valid as long as `plan_buf` and the tensors it
 * names do, on the device that was current when it was made.  1 <= count <=
 * 1<<20; every k % 64 == 0 and k <= 32768; no output may overlap another
 * output, an input or the plan.
 */
Q4_API q4_status q4_0_gemv_batch_plan(const q4_gemv_desc* descs, int count, void* plan_buf,
                               size_t plan_bytes, q4_gemv_plan* plan, void* stream);

/* Run every GEMV of a plan in one launch on `stream`.  Launches of the same
 * plan must not overlap in time (they share its counters and outputs); the
 * results do not depend on how the chunks were handed out. */
Q4_API q4_status q4_0_gemv_batch(const q4_gemv_plan* plan, void* stream);

/*
 * Make the GEMV of a planned list whose descriptor named the output `y` the
 * stage hand-off (the end of a
 * device's layer range, whose hidden state goes to the next participant as
 * f16: aipolix.com en-us page, section "A model can be larger than any one
 * browser can hold"): from the next q4_0_gemv_batch launch on, that GEMV
 * writes h16[n] = binary16(residual[n] + y[n]) (nearest-even; the binary32 y
 * of the same kernel and association, residual added in binary32) instead of
 * its binary32 y, which is no longer written.  So a stage's whole layer range,
 * ending in the hand-off, is one launch.
 *   residual : NULL (zero) or n binary32, 4-byte aligned
 *   h16      : n binary16, 2-byte aligned; must not overlap any tensor of the
 *              list (other than that GEMV's own former y), the residual or the
 *              plan
 * (The plan keeps its own order of the list, so the GEMV is named by its
 * output.)  Reads the plan's descriptors back, checks, and writes the changed
 * one; the copies are enqueued on `stream` and complete before the call
 * returns.  No GEMV with output y in the plan: Q4_ERR_INVALID_ARG.
 * Launches of the plan must not be running meanwhile.
 */
Q4_API q4_status q4_0_gemv_batch_handoff(const q4_gemv_plan* plan, const float* y, const float* residual,
                                         void* h16, void* stream);

/* Host-side handle of a Q8_0 GEMV list plan.  Filled by q8_0_gemv_batch_plan;
 * plain data, may be copied. */
typedef struct q8_gemv_plan {
    void* device;        /* the caller's device buffer holding the plan */
    int count;           /* number of GEMVs */
    int n_slab;          /* internal: GEMVs on the slab kernel (the plan's first part) */
    int grid_slab;       /* internal: workgroups of their launch */
    int nchunks_slab;    /* internal: chunks of their schedule */
    int max_k;           /* internal: largest k of the other GEMVs */
    int grid;            /* internal: workgroups of the other GEMVs' launch */
    size_t offset_other; /* internal: byte offset of the other GEMVs' part in the plan */
} q8_gemv_plan;

/* Device bytes q8_0_gemv_batch_plan needs for this list on the current device
 * (0, with the error text set, when the list is invalid). */
Q4_API size_t q8_0_gemv_batch_plan_bytes(const q4_gemv_desc* descs, int count);

/*
 * A list of Q8_0 GEMVs (descriptors as q4_gemv_desc, with w holding n rows of
 * k/32 Q8_0 blocks) run as one launch per kernel (at most two), for the
 * layers of a small dense model in one submission.  Validate `count`
 * host-side descriptors (each as q8_0_gemv requires; no output may overlap
 * another output, an input or the plan) and split them by the kernel
 * q8_0_gemv would choose.  The slab kernel's GEMVs get the schedule of
 * q4_0_gemv_batch_plan (row steps of 64 rows, a static first chunk per
 * workgroup, then chunks from a counter); the others are laid out in units of
 * 16 rows of one GEMV, every workgroup taking one contiguous byte-balanced
 * range of the first 85 % of the bytes and then units in chunks from a
 * counter.  Copy the counters (zero), descriptors, chunks and ranges into the
 * caller's device buffer `plan_buf` (16-byte aligned, at least
 * q8_0_gemv_batch_plan_bytes bytes).  The copy is enqueued on `stream` and has completed when this call
 * returns.  Launches of one plan must not overlap in time (they share its
 * counters; the last workgroup of a launch sets them back to zero, which also
 * makes the launch safe to capture in a HIP graph).  Every row's result
 * equals q8_0_gemv's bit for bit.
 */
Q4_API q4_status q8_0_gemv_batch_plan(const q4_gemv_desc* descs, int count, void* plan_buf, size_t plan_bytes,
                                      q8_gemv_plan* plan, void* stream);

/* Run every GEMV of a Q8_0 plan on `stream` (one launch per kernel the list uses). */
Q4_API q4_status q8_0_gemv_batch(const q8_gemv_plan* plan, void* stream);

/* Host-side handle of a small-M batch plan.  Filled by
 * q4_0_gemm_smallm_batch_plan; plain data, may be copied. */
typedef struct q4_gemm_plan {
    void* device;            /* the caller's device buffer holding the descriptors */
    int count;               /* number of GEMMs */
    int m;                   /* activation rows of every GEMM */
    int max_p;               /* internal: longest K-range in block pairs */
    int flags;               /* internal: bit 0 = some GEMM splits K */
    int64_t total_cost;      /* internal: work units of the list */
    int64_t max_mn;          /* internal: largest m * n */
    size_t workspace_bytes;  /* device workspace q4_0_gemm_smallm_batch needs (may be 0) */
} q4_gemm_plan;

/* Device bytes q4_0_gemm_smallm_batch_plan needs for `count` descriptors. */
Q4_API size_t q4_0_gemm_smallm_batch_plan_bytes(int count);

/*
 * A list of small-M GEMMs with the same m, run as one launch: the verify pass
 * of a speculative draft over a whole layer stack (aipolix.com en-us page,
 * section "Speculation is used to amortize network round trips"), issued as
 * one submission per token as the decode engine does ("Every Device Brings a
 * Slice: How SwarmLLM Runs a 27B Model Across Browser Tabs", originshq.com,
 * section "The Engine: ~50 WGSL Kernels Written From Scratch").  Descriptor i names w (n rows of
 * k/32 Q4_0 blocks, 4-byte aligned), x (m x k binary16, 16-byte aligned) and
 * y (m x n binary32, written); every k % 64 == 0, 2 <= m <= 16, |d| <= 8188.
 * Each GEMM's result is bit-identical to q4_0_gemm_smallm on the same
 * operands.  Validates the list, writes its device form into `plan_buf`
 * (q4_0_gemm_smallm_batch_plan_bytes(count) bytes, 16-byte aligned) and
 * fills `*plan`; the copy has completed when this returns (it synchronizes
 * `stream`).  No output may overlap another output, an input or the plan.
 */
Q4_API q4_status q4_0_gemm_smallm_batch_plan(const q4_gemv_desc* descs, int count, int64_t m, void* plan_buf,
                                             size_t plan_bytes, q4_gemm_plan* plan, void* stream);

/* Run every GEMM of a small-M plan on `stream`: one launch, plus one that
 * adds K-range partial sums when plan->flags says some GEMM splits K.
 * `workspace`: plan->workspace_bytes of device memory, 16-byte aligned, not
 * overlapping the plan's tensors (NULL when that is 0). */
Q4_API q4_status q4_0_gemm_smallm_batch(const q4_gemm_plan* plan, void* workspace, size_t workspace_bytes,
                                        void* stream);

/* Host-side handle of a prefill batch plan.  Filled by
 * q4_0_gemm_prefill_batch_plan; plain data, may be copied. */
typedef struct q4_prefill_plan {
    void* device;          /* the caller's device buffer holding the descriptors */
    int count;             /* number of GEMMs */
    int m;                 /* token rows of every GEMM */
    int tile_m;            /* internal: activation rows per tile (64, 96 or 128) */
    int count_chunked;     /* internal: GEMMs with k % 256 == 0 (first in the device list) */
    int64_t tiles_chunked; /* internal: their tiles */
    int64_t tiles_other;   /* internal: tiles of the other GEMMs */
} q4_prefill_plan;

/* Device bytes q4_0_gemm_prefill_batch_plan needs for `count` descriptors. */
Q4_API size_t q4_0_gemm_prefill_batch_plan_bytes(int count);

/*
 * A list of prefill GEMMs with the same m, run as one launch: the prompt
 * matrices of independent projections (taozi.news, section "基准成绩";
 * originshq.com page, section "The Engine ...") share the machine instead of
 * each filling only part of it.  Descriptor i names w (n rows of k/32 Q4_0
 * blocks, 16-byte aligned), x (m x k binary16, 16-byte aligned) and y (m x n
 * binary32, written); every k % 64 == 0, m*n <= 2^40, |d| <= 8188.  Each
 * result equals that of q4_0_gemm_prefill on the same operands bit for bit
 * (each GEMM runs in the same kernel with the same f32 summation order; the
 * tile shape may differ, which does not change that order).
 * Validates the list, writes its device form into `plan_buf`
 * (q4_0_gemm_prefill_batch_plan_bytes(count) bytes, 16-byte aligned) and
 * fills `*plan`; the copy has completed when this returns.  No output may
 * overlap another output, an input or the plan.  The plan buffer also holds
 * the work counters of its launches, which every launch returns to their
 * initial state when it completes: run one call of a plan at a time (calls on
 * one stream are fine; the same plan on two streams at once is not).
 */
Q4_API q4_status q4_0_gemm_prefill_batch_plan(const q4_gemv_desc* descs, int count, int64_t m, void* plan_buf,
                                              size_t plan_bytes, q4_prefill_plan* plan, void* stream);

/* Run every GEMM of a prefill plan on `stream`: one launch, or two when the
 * list mixes k % 256 == 0 with other k (each GEMM runs in the kernel its own
 * q4_0_gemm_prefill call uses, so the results are the same bit for bit). */
Q4_API q4_status q4_0_gemm_prefill_batch(const q4_prefill_plan* plan, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4GEMV_H */
