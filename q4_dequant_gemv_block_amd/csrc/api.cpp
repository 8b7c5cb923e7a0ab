// C ABI of the Q4_0 library: argument validation, error text, dispatch to the
// kernel launchers.  Every check runs on the host before anything is enqueued.
#include "q4gemv.h"
#include "q4_launch.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

namespace {

thread_local char g_err[512];

q4_status fail(q4_status code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

q4_status ok() {
    g_err[0] = '\0';
    return Q4_OK;
}

q4_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(Q4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
// The Q8_0 GEMVs that run on the slab engine (single calls and lists alike).
bool q8_on_slabs(const void* w, int64_t k) { return q4::q8_slab_ok(k) && aligned(w, 16); }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range(const void* p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int64_t row_bytes(int64_t k) { return k / 32 * 18; }

// Largest sizes accepted anywhere: keeps every byte offset far inside int64
// and every row index inside the 32-bit fields the kernels use for it.
constexpr int64_t kMaxN = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxK = int64_t(1) << 24;

q4_status check_shape(const char* fn, int64_t m, int64_t m_max, int64_t n, int64_t k) {
    if (m < 1 || m > m_max) return fail(Q4_ERR_INVALID_ARG, "%s: m = %lld outside [1, %lld]", fn, (long long)m, (long long)m_max);
    if (n < 1 || n > kMaxN) return fail(Q4_ERR_INVALID_ARG, "%s: n = %lld outside [1, %lld]", fn, (long long)n, (long long)kMaxN);
    if (k < 32 || k > kMaxK || k % 32 != 0)
        return fail(Q4_ERR_INVALID_ARG, "%s: k = %lld must be a multiple of 32 in [32, %lld]", fn, (long long)k, (long long)kMaxK);
    return Q4_OK;
}

q4_status check_tensors(const char* fn, const void* w, const void* x, const void* y, int64_t m,
                        int64_t n, int64_t k, size_t y_bytes) {
    if (!w || !x || !y) return fail(Q4_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
    if (!aligned(w, 16) || !aligned(x, 16)) return fail(Q4_ERR_MISALIGNED, "%s: w and x must be 16-byte aligned", fn);
    if (!aligned(y, 4)) return fail(Q4_ERR_MISALIGNED, "%s: output must be 4-byte aligned", fn);
    const Range rw = range(w, (size_t)(n * row_bytes(k)));
    const Range rx = range(x, (size_t)(m * k * 2));
    const Range ry = range(y, y_bytes);
    if (overlap(ry, rw) || overlap(ry, rx)) return fail(Q4_ERR_INVALID_ARG, "%s: output overlaps an input", fn);
    return Q4_OK;
}

bool fast_path(const void* w, int64_t k) { return k % 64 == 0 && k <= q4::kFastMaxK && aligned(w, 4); }

}  // namespace

extern "C" {

int q4_abi_version(void) { return Q4_ABI_VERSION; }

const char* q4_last_error(void) { return g_err; }

size_t q4_workspace_bytes(int op, int64_t m, int64_t n, int64_t k) {
    switch (op) {
        case Q4_OP_GEMV:
        case Q4_OP_GEMM_PREFILL:
            return 0;
        case Q4_OP_GEMM_SMALLM:
            // only the matrix-core path (2 <= m <= 16, k % 64 == 0) splits K
            if (m < 2 || m > 16 || n < 1 || k < 64 || k % 64 != 0 || k > kMaxK || n > kMaxN) return 0;
            // (with w not 4-byte aligned the call takes the generic kernel and ignores the workspace)
            return q4::smallm_workspace_bytes(m, n, k);
        case Q4_OP_LM_HEAD_ARGMAX:
        case Q4_OP_LM_HEAD_NORM_ARGMAX:
            if (n < 1 || k < 32) return 0;
            return (size_t)q4::argmax_blocks(n, k) * sizeof(uint64_t);
        case Q4_OP_LM_HEAD_VERIFY:
            if (m < 1 || m > 16 || n < 1 || n > kMaxN || k < 64 || k % 64 != 0 || k > kMaxK) return 0;
            return q4::verify_workspace_bytes(m, n, k);
        default:
            return 0;
    }
}

q4_status q4_0_gemv(const void* w, const void* x, float* y, int64_t n, int64_t k, void* stream) {
    q4_status st = check_shape("q4_0_gemv", 1, 1, n, k);
    if (st) return st;
    st = check_tensors("q4_0_gemv", w, x, y, 1, n, k, (size_t)n * 4);
    if (st) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (fast_path(w, k))
        e = q4::launch_gemv(static_cast<const uint8_t*>(w), static_cast<const uint16_t*>(x), y, n, k, s);
    else
        e = q4::launch_gemm_generic(static_cast<const uint8_t*>(w), static_cast<const uint16_t*>(x), y, 1, n, k, s);
    return hip_status(e, "q4_0_gemv launch");
}

q4_status q4_0_gemm_smallm(const void* w, const void* x, float* y, int64_t m, int64_t n, int64_t k,
                           void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "q4_0_gemm_smallm";
    q4_status st = check_shape(fn, m, 16, n, k);
    if (st) return st;
    st = check_tensors(fn, w, x, y, m, n, k, (size_t)(m * n) * 4);
    if (st) return st;
    const size_t need = q4_workspace_bytes(Q4_OP_GEMM_SMALLM, m, n, k);
    if (need) {
        if (!workspace || workspace_bytes < need) return fail(Q4_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
        if (!aligned(workspace, 16)) return fail(Q4_ERR_MISALIGNED, "%s: workspace must be 16-byte aligned", fn);
        const Range rws = range(workspace, need);
        if (overlap(rws, range(w, (size_t)(n * row_bytes(k)))) || overlap(rws, range(x, (size_t)(m * k * 2))) ||
            overlap(rws, range(y, (size_t)(m * n) * 4)))
            return fail(Q4_ERR_INVALID_ARG, "%s: workspace overlaps a tensor", fn);
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    hipError_t e;
    if (m == 1 && fast_path(w, k))
        e = q4::launch_gemv(wb, xb, y, n, k, s);
    else if (m >= 2 && k % 64 == 0 && aligned(w, 4))
        e = q4::launch_gemm_smallm(wb, xb, y, m, n, k, static_cast<float*>(workspace), s);
    else
        e = q4::launch_gemm_generic(wb, xb, y, m, n, k, s);
    return hip_status(e, "q4_0_gemm_smallm launch");
}

q4_status q4_0_gemm_prefill(const void* w, const void* x, float* y, int64_t m, int64_t n, int64_t k,
                            void* workspace, size_t workspace_bytes, void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    q4_status st = check_shape("q4_0_gemm_prefill", m, kMaxN, n, k);
    if (st) return st;
    if (m * n > (int64_t(1) << 40)) return fail(Q4_ERR_INVALID_ARG, "q4_0_gemm_prefill: m*n too large");
    st = check_tensors("q4_0_gemm_prefill", w, x, y, m, n, k, (size_t)(m * n) * 4);
    if (st) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    if (k % 64 == 0 && aligned(w, 4) && m <= (int64_t(1) << 30) && n <= (int64_t(1) << 30))
        return hip_status(q4::launch_gemm_prefill(wb, xb, y, m, n, k, s), "q4_0_gemm_prefill launch");
    for (int64_t m0 = 0; m0 < m; m0 += 16) {
        const int64_t mm = std::min<int64_t>(16, m - m0);
        const hipError_t e = q4::launch_gemm_generic(wb, xb + m0 * k, y + m0 * n, mm, n, k, s);
        if (e != hipSuccess) return hip_status(e, "q4_0_gemm_prefill launch");
    }
    return ok();
}

q4_status lm_head_argmax(const void* w, const void* h, float* logits, int32_t* token, int64_t n_vocab,
                         int64_t k, void* workspace, size_t workspace_bytes, void* stream) {
    q4_status st = check_shape("lm_head_argmax", 1, 1, n_vocab, k);
    if (st) return st;
    st = check_tensors("lm_head_argmax", w, h, logits, 1, n_vocab, k, (size_t)n_vocab * 4);
    if (st) return st;
    if (!token) return fail(Q4_ERR_INVALID_ARG, "lm_head_argmax: null token pointer");
    if (!aligned(token, 4)) return fail(Q4_ERR_MISALIGNED, "lm_head_argmax: token must be 4-byte aligned");
    if (!fast_path(w, k))
        return fail(Q4_ERR_INVALID_ARG, "lm_head_argmax: needs k %% 64 == 0 and k <= %lld", (long long)q4::kFastMaxK);
    const size_t need = q4_workspace_bytes(Q4_OP_LM_HEAD_ARGMAX, 1, n_vocab, k);
    if (!workspace || workspace_bytes < need)
        return fail(Q4_ERR_WORKSPACE, "lm_head_argmax: workspace of %zu bytes needed", need);
    if (!aligned(workspace, 8)) return fail(Q4_ERR_MISALIGNED, "lm_head_argmax: workspace must be 8-byte aligned");
    const Range rws = range(workspace, need), rt = range(token, 4), rl = range(logits, (size_t)n_vocab * 4);
    if (overlap(rws, range(w, (size_t)(n_vocab * row_bytes(k)))) || overlap(rws, range(h, (size_t)k * 2)) ||
        overlap(rws, rl) || overlap(rws, rt) || overlap(rt, rl) ||
        overlap(rt, range(w, (size_t)(n_vocab * row_bytes(k)))) || overlap(rt, range(h, (size_t)k * 2)))
        return fail(Q4_ERR_INVALID_ARG, "lm_head_argmax: token, workspace and tensors must not overlap");
    const hipError_t e = q4::launch_lm_head(static_cast<const uint8_t*>(w), static_cast<const uint16_t*>(h), logits,
                                            token, n_vocab, k, static_cast<uint64_t*>(workspace),
                                            static_cast<hipStream_t>(stream));
    return hip_status(e, "lm_head_argmax launch");
}

q4_status lm_head_argmax_noalloc(const void* w, const void* h, float* logits, int32_t* token, int64_t n_vocab,
                                 int64_t k, void* stream) {
    const char* fn = "lm_head_argmax_noalloc";
    q4_status st = check_shape(fn, 1, 1, n_vocab, k);
    if (st) return st;
    st = check_tensors(fn, w, h, logits, 1, n_vocab, k, (size_t)n_vocab * 4);
    if (st) return st;
    if (!token) return fail(Q4_ERR_INVALID_ARG, "%s: null token pointer", fn);
    if (!aligned(token, 4)) return fail(Q4_ERR_MISALIGNED, "%s: token must be 4-byte aligned", fn);
    if (!fast_path(w, k))
        return fail(Q4_ERR_INVALID_ARG, "%s: needs k %% 64 == 0 and k <= %lld", fn, (long long)q4::kFastMaxK);
    const Range rt = range(token, 4), rl = range(logits, (size_t)n_vocab * 4);
    if (overlap(rt, rl) || overlap(rt, range(w, (size_t)(n_vocab * row_bytes(k)))) || overlap(rt, range(h, (size_t)k * 2)))
        return fail(Q4_ERR_INVALID_ARG, "%s: token must not overlap the tensors", fn);
    const int keys = q4::argmax_blocks(n_vocab, k);
    if (keys > q4::kLmHeadScratchKeys)
        return fail(Q4_ERR_INVALID_ARG, "%s: %d workgroup keys exceed the library's array of %d", fn, keys,
                    q4::kLmHeadScratchKeys);
    uint64_t* scratch = nullptr;
    hipError_t e = q4::lm_head_scratch(&scratch);
    if (e != hipSuccess) return hip_status(e, "lm_head_argmax_noalloc: scratch address");
    e = q4::launch_lm_head(static_cast<const uint8_t*>(w), static_cast<const uint16_t*>(h), logits, token, n_vocab, k,
                           scratch, static_cast<hipStream_t>(stream));
    return hip_status(e, "lm_head_argmax_noalloc launch");
}

q4_status q8_0_gemv(const void* w, const void* x, float* y, int64_t n, int64_t k, void* stream) {
    const char* fn = "q8_0_gemv";
    q4_status st = check_shape(fn, 1, 1, n, k);
    if (st) return st;
    if (!w || !x || !y) return fail(Q4_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
    if (!aligned(w, 4)) return fail(Q4_ERR_MISALIGNED, "%s: w must be 4-byte aligned", fn);
    if (!aligned(x, 16)) return fail(Q4_ERR_MISALIGNED, "%s: x must be 16-byte aligned", fn);
    if (!aligned(y, 4)) return fail(Q4_ERR_MISALIGNED, "%s: y must be 4-byte aligned", fn);
    if (k > q4::kFastMaxK) return fail(Q4_ERR_INVALID_ARG, "%s: k = %lld above %lld", fn, (long long)k, (long long)q4::kFastMaxK);
    const Range ry = range(y, (size_t)n * 4);
    if (overlap(ry, range(w, (size_t)(n * (k / 32) * 34))) || overlap(ry, range(x, (size_t)k * 2)))
        return fail(Q4_ERR_INVALID_ARG, "%s: output overlaps an input", fn);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = q8_on_slabs(w, k)
                             ? q4::launch_q8_slab_gemv(static_cast<const uint8_t*>(w), static_cast<const uint16_t*>(x), y, n, k, s)
                             : q4::launch_q8_gemv(static_cast<const uint8_t*>(w), static_cast<const uint16_t*>(x), y, n, k, s);
    return hip_status(e, "q8_0_gemv launch");
}

q4_status q4_0_gemv_handoff(const void* w, const void* x, const float* residual, void* h16, int64_t n, int64_t k,
                            void* stream) {
    const char* fn = "q4_0_gemv_handoff";
    q4_status st = check_shape(fn, 1, 1, n, k);
    if (st) return st;
    if (!w || !x || !h16) return fail(Q4_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
    if (!aligned(w, 16) || !aligned(x, 16)) return fail(Q4_ERR_MISALIGNED, "%s: w and x must be 16-byte aligned", fn);
    if (!aligned(h16, 2)) return fail(Q4_ERR_MISALIGNED, "%s: h16 must be 2-byte aligned", fn);
    if (residual && !aligned(residual, 4)) return fail(Q4_ERR_MISALIGNED, "%s: residual must be 4-byte aligned", fn);
    if (!fast_path(w, k))
        return fail(Q4_ERR_INVALID_ARG, "%s: needs k %% 64 == 0 and k <= %lld", fn, (long long)q4::kFastMaxK);
    const Range rh = range(h16, (size_t)n * 2);
    if (overlap(rh, range(w, (size_t)(n * row_bytes(k)))) || overlap(rh, range(x, (size_t)k * 2)) ||
        (residual && overlap(rh, range(residual, (size_t)n * 4))))
        return fail(Q4_ERR_INVALID_ARG, "%s: h16 overlaps an input", fn);
    const hipError_t e = q4::launch_gemv_handoff(static_cast<const uint8_t*>(w), static_cast<const uint16_t*>(x),
                                                 residual, static_cast<uint16_t*>(h16), n, k,
                                                 static_cast<hipStream_t>(stream));
    return hip_status(e, "q4_0_gemv_handoff launch");
}

q4_status lm_head_norm_argmax(const void* w, const void* h, const void* gamma, float eps, float* logits,
                              int32_t* token, void* x_out, int64_t n_vocab, int64_t k, void* workspace,
                              size_t workspace_bytes, void* stream) {
    const char* fn = "lm_head_norm_argmax";
    q4_status st = check_shape(fn, 1, 1, n_vocab, k);
    if (st) return st;
    st = check_tensors(fn, w, h, logits, 1, n_vocab, k, (size_t)n_vocab * 4);
    if (st) return st;
    if (!token || !gamma) return fail(Q4_ERR_INVALID_ARG, "%s: null token or gamma pointer", fn);
    if (!aligned(token, 4)) return fail(Q4_ERR_MISALIGNED, "%s: token must be 4-byte aligned", fn);
    if (!aligned(gamma, 16)) return fail(Q4_ERR_MISALIGNED, "%s: gamma must be 16-byte aligned", fn);
    if (x_out && !aligned(x_out, 16)) return fail(Q4_ERR_MISALIGNED, "%s: x_out must be 16-byte aligned", fn);
    if (!(eps > 0.0f) || !(eps <= 3.4e38f)) return fail(Q4_ERR_INVALID_ARG, "%s: eps must be finite and > 0", fn);
    if (!fast_path(w, k))
        return fail(Q4_ERR_INVALID_ARG, "%s: needs k %% 64 == 0 and k <= %lld", fn, (long long)q4::kFastMaxK);
    const size_t need = q4_workspace_bytes(Q4_OP_LM_HEAD_NORM_ARGMAX, 1, n_vocab, k);
    if (!workspace || workspace_bytes < need) return fail(Q4_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
    if (!aligned(workspace, 8)) return fail(Q4_ERR_MISALIGNED, "%s: workspace must be 8-byte aligned", fn);
    const Range rw = range(w, (size_t)(n_vocab * row_bytes(k))), rh = range(h, (size_t)k * 2),
                rg = range(gamma, (size_t)k * 2);
    const Range outs[4] = {range(logits, (size_t)n_vocab * 4), range(token, 4), range(workspace, need),
                           x_out ? range(x_out, (size_t)k * 2) : Range{0, 0}};
    for (int i = 0; i < 4; ++i) {
        if (outs[i].lo == outs[i].hi) continue;
        if (overlap(outs[i], rw) || overlap(outs[i], rh) || overlap(outs[i], rg))
            return fail(Q4_ERR_INVALID_ARG, "%s: an output or the workspace overlaps an input", fn);
        for (int j = i + 1; j < 4; ++j)
            if (outs[j].lo != outs[j].hi && overlap(outs[i], outs[j]))
                return fail(Q4_ERR_INVALID_ARG, "%s: outputs and workspace must not overlap", fn);
    }
    const hipError_t e = q4::launch_lm_head_norm(
        static_cast<const uint8_t*>(w), static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(gamma), eps,
        static_cast<uint16_t*>(x_out), logits, token, n_vocab, k, static_cast<uint64_t*>(workspace),
        static_cast<hipStream_t>(stream));
    return hip_status(e, "lm_head_norm_argmax launch");
}

q4_status lm_head_verify(const void* w, const void* h, float* logits, int32_t* tokens, const int32_t* draft,
                         int32_t* accepted, int64_t m, int64_t n_vocab, int64_t k, void* workspace,
                         size_t workspace_bytes, void* stream) {
    const char* fn = "lm_head_verify";
    q4_status st = check_shape(fn, m, 16, n_vocab, k);
    if (st) return st;
    st = check_tensors(fn, w, h, logits, m, n_vocab, k, (size_t)(m * n_vocab) * 4);
    if (st) return st;
    if (!tokens || !draft || !accepted) return fail(Q4_ERR_INVALID_ARG, "%s: null tokens, draft or accepted", fn);
    if (!aligned(tokens, 4) || !aligned(draft, 4) || !aligned(accepted, 4))
        return fail(Q4_ERR_MISALIGNED, "%s: tokens, draft and accepted must be 4-byte aligned", fn);
    if (!fast_path(w, k))
        return fail(Q4_ERR_INVALID_ARG, "%s: needs k %% 64 == 0 and k <= %lld", fn, (long long)q4::kFastMaxK);
    const size_t need = q4_workspace_bytes(Q4_OP_LM_HEAD_VERIFY, m, n_vocab, k);
    if (!workspace || workspace_bytes < need)
        return fail(Q4_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
    if (!aligned(workspace, 16)) return fail(Q4_ERR_MISALIGNED, "%s: workspace must be 16-byte aligned", fn);
    const Range rw = range(w, (size_t)(n_vocab * row_bytes(k))), rh = range(h, (size_t)(m * k) * 2),
                rl = range(logits, (size_t)(m * n_vocab) * 4), rt = range(tokens, (size_t)m * 4),
                rd = range(draft, (size_t)m * 4), ra = range(accepted, 4), rws = range(workspace, need);
    const Range outs[4] = {rl, rt, ra, rws}, ins[3] = {rw, rh, rd};
    for (int i = 0; i < 4; ++i) {
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return fail(Q4_ERR_INVALID_ARG, "%s: outputs must not overlap", fn);
        for (int j = 0; j < 3; ++j)
            if (overlap(outs[i], ins[j])) return fail(Q4_ERR_INVALID_ARG, "%s: an output overlaps an input", fn);
    }
    const hipError_t e = q4::launch_lm_head_verify(static_cast<const uint8_t*>(w), static_cast<const uint16_t*>(h),
                                                   logits, tokens, draft, accepted, m, n_vocab, k, workspace,
                                                   static_cast<hipStream_t>(stream));
    return hip_status(e, "lm_head_verify launch");
}

}  // extern "C"

namespace {

// Validates a descriptor list whose x are m x k and y m x n: shapes,
// alignment, k % 64 == 0 (and k <= k_max), no output overlapping another
// output or any input.  *max_k_out: the largest k.
q4_status check_list(const char* fn, const q4_gemv_desc* descs, int count, int64_t m, int64_t m_max, int64_t k_max,
                     int* max_k_out) {
    if (!descs) return fail(Q4_ERR_INVALID_ARG, "%s: null descriptor list", fn);
    if (count < 1 || count > (1 << 20)) return fail(Q4_ERR_INVALID_ARG, "%s: count = %d outside [1, 1<<20]", fn, count);
    std::vector<Range> outs, ins;
    outs.reserve(count);
    ins.reserve(2 * (size_t)count);
    int max_k = 0;
    for (int i = 0; i < count; ++i) {
        const q4_gemv_desc& d = descs[i];
        q4_status st = check_shape(fn, m, m_max, d.n, d.k);
        if (st) return fail(st, "%s: descriptor %d: %s", fn, i, std::string(g_err).c_str());
        if (d.k % 64 != 0 || d.k > k_max)
            return fail(Q4_ERR_INVALID_ARG, "%s: descriptor %d: k must be a multiple of 64 up to %lld", fn, i, (long long)k_max);
        st = check_tensors(fn, d.w, d.x, d.y, m, d.n, d.k, (size_t)(m * d.n) * 4);
        if (st) return fail(st, "%s: descriptor %d: %s", fn, i, std::string(g_err).c_str());
        max_k = std::max<int>(max_k, (int)d.k);
        outs.push_back(range(d.y, (size_t)(m * d.n) * 4));
        ins.push_back(range(d.w, (size_t)(d.n * row_bytes(d.k))));
        ins.push_back(range(d.x, (size_t)(m * d.k) * 2));
    }
    std::sort(outs.begin(), outs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
    for (size_t i = 1; i < outs.size(); ++i)
        if (outs[i].lo < outs[i - 1].hi) return fail(Q4_ERR_INVALID_ARG, "%s: two outputs overlap", fn);
    for (const Range& r : ins) {
        auto it = std::upper_bound(outs.begin(), outs.end(), r.lo, [](uintptr_t v, const Range& o) { return v < o.lo; });
        if (it != outs.end() && overlap(*it, r)) return fail(Q4_ERR_INVALID_ARG, "%s: an output overlaps an input", fn);
        if (it != outs.begin() && overlap(*(it - 1), r)) return fail(Q4_ERR_INVALID_ARG, "%s: an output overlaps an input", fn);
    }
    *max_k_out = max_k;
    return ok();
}

// A device buffer that must not overlap any tensor of the list.
q4_status check_buffer(const char* fn, const char* what, const void* buf, size_t bytes, const q4_gemv_desc* descs,
                       int count, int64_t m) {
    const Range rb = range(buf, bytes);
    for (int i = 0; i < count; ++i) {
        const q4_gemv_desc& d = descs[i];
        if (overlap(rb, range(d.y, (size_t)(m * d.n) * 4)) || overlap(rb, range(d.w, (size_t)(d.n * row_bytes(d.k)))) ||
            overlap(rb, range(d.x, (size_t)(m * d.k) * 2)))
            return fail(Q4_ERR_INVALID_ARG, "%s: %s overlaps a tensor of descriptor %d", fn, what, i);
    }
    return Q4_OK;
}

// Validates a GEMV list and lays out its plan: device descriptors, chunk
// schedule and launch grid.
q4_status plan_layout(const char* fn, const q4_gemv_desc* descs, int count, std::vector<q4::PlanDesc>* dev,
                      std::vector<q4::SchedChunk>* chunks, int* grid, int* flags, int* max_k_out) {
    const q4_status st = check_list(fn, descs, count, 1, 1, q4::kFastMaxK, max_k_out);
    if (st) return st;
    dev->assign(count, q4::PlanDesc{});
    for (int i = 0; i < count; ++i) {
        q4::PlanDesc& p = (*dev)[i];
        p.w = static_cast<const uint8_t*>(descs[i].w);
        p.x = static_cast<const uint16_t*>(descs[i].x);
        p.y = descs[i].y;
        p.n = descs[i].n;
        p.k = (int32_t)descs[i].k;
    }
    q4::build_schedule(dev->data(), count, chunks, grid, flags);
    return ok();
}

size_t plan_size(int count, size_t nchunks) {
    return sizeof(q4::SchedHead) + (size_t)count * sizeof(q4::PlanDesc) + nchunks * sizeof(q4::SchedChunk);
}

// A Q8_0 list: the GEMVs the slab engine takes (the same rule as a single
// call, so a GEMV gives the same bits either way) form the plan's first part
// (SchedHead, descriptors, chunks), the others its second part (Q8Head,
// descriptors, workgroup ranges), each run by its own launch.
struct Q8Layout {
    std::vector<q4::PlanDesc> slab;
    std::vector<q4::SchedChunk> chunks;
    int grid_slab = 0;
    std::vector<q4::Q8Desc> other;
    std::vector<int64_t> wg_begin;
    q4::Q8Head head{};
    int grid_other = 0, max_k_other = 0;
    size_t off_other = 0, bytes = 0;
    std::vector<Range> outs, ins;
};

q4_status q8_layout(const char* fn, const q4_gemv_desc* descs, int count, Q8Layout* L) {
    if (!descs) return fail(Q4_ERR_INVALID_ARG, "%s: null descriptor list", fn);
    if (count < 1 || count > (1 << 20)) return fail(Q4_ERR_INVALID_ARG, "%s: count = %d outside [1, 1<<20]", fn, count);
    for (int i = 0; i < count; ++i) {
        const q4_gemv_desc& d = descs[i];
        q4_status st = check_shape(fn, 1, 1, d.n, d.k);
        if (st) return fail(st, "%s: descriptor %d: %s", fn, i, std::string(g_err).c_str());
        if (d.k > q4::kFastMaxK) return fail(Q4_ERR_INVALID_ARG, "%s: descriptor %d: k above %lld", fn, i, (long long)q4::kFastMaxK);
        if (!d.w || !d.x || !d.y) return fail(Q4_ERR_INVALID_ARG, "%s: descriptor %d: null tensor pointer", fn, i);
        if (!aligned(d.w, 4) || !aligned(d.x, 16) || !aligned(d.y, 4))
            return fail(Q4_ERR_MISALIGNED, "%s: descriptor %d: w must be 4-, x 16-, y 4-byte aligned", fn, i);
        L->outs.push_back(range(d.y, (size_t)d.n * 4));
        L->ins.push_back(range(d.w, (size_t)(d.n * (d.k / 32) * 34)));
        L->ins.push_back(range(d.x, (size_t)d.k * 2));
        if (q8_on_slabs(d.w, d.k)) {
            q4::PlanDesc p = {};
            p.w = static_cast<const uint8_t*>(d.w);
            p.x = static_cast<const uint16_t*>(d.x);
            p.y = d.y;
            p.n = d.n;
            p.k = (int32_t)d.k;
            L->slab.push_back(p);
        } else {
            L->other.push_back(q4::Q8Desc{static_cast<const uint8_t*>(d.w), static_cast<const uint16_t*>(d.x), d.y, d.n,
                                          (int32_t)d.k, 0, 0});
            L->max_k_other = std::max<int>(L->max_k_other, (int)d.k);
        }
    }
    std::sort(L->outs.begin(), L->outs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
    for (size_t i = 1; i < L->outs.size(); ++i)
        if (L->outs[i].lo < L->outs[i - 1].hi) return fail(Q4_ERR_INVALID_ARG, "%s: two outputs overlap", fn);
    for (const Range& r : L->ins) {  // outputs are sorted and disjoint: only the neighbours of r.lo can overlap r
        auto it = std::upper_bound(L->outs.begin(), L->outs.end(), r.lo, [](uintptr_t v, const Range& o) { return v < o.lo; });
        if ((it != L->outs.end() && overlap(*it, r)) || (it != L->outs.begin() && overlap(*(it - 1), r)))
            return fail(Q4_ERR_INVALID_ARG, "%s: an output overlaps an input", fn);
    }
    if (!L->slab.empty()) L->grid_slab = q4::build_schedule_q8(L->slab.data(), (int)L->slab.size(), &L->chunks);
    if (!L->other.empty())
        L->grid_other = q4::q8_batch_layout(L->other.data(), (int)L->other.size(), &L->wg_begin, &L->head);
    const size_t first = L->slab.empty() ? 0 : plan_size((int)L->slab.size(), L->chunks.size());
    L->off_other = (first + 15) / 16 * 16;
    L->bytes = L->off_other + (L->other.empty() ? 0
                                                : sizeof(q4::Q8Head) + L->other.size() * sizeof(q4::Q8Desc) +
                                                      L->wg_begin.size() * sizeof(int64_t));
    return ok();
}

}  // namespace

extern "C" {

size_t q4_0_gemv_batch_plan_bytes(const q4_gemv_desc* descs, int count) {
    std::vector<q4::PlanDesc> dev;
    std::vector<q4::SchedChunk> chunks;
    int grid = 0, flags = 0, max_k = 0;
    if (plan_layout("q4_0_gemv_batch_plan_bytes", descs, count, &dev, &chunks, &grid, &flags, &max_k)) return 0;
    ok();
    return plan_size(count, chunks.size());
}

q4_status q4_0_gemv_batch_plan(const q4_gemv_desc* descs, int count, void* plan_buf, size_t plan_bytes,
                               q4_gemv_plan* plan, void* stream) {
    const char* fn = "q4_0_gemv_batch_plan";
    if (!plan || !plan_buf) return fail(Q4_ERR_INVALID_ARG, "%s: null pointer", fn);
    std::vector<q4::PlanDesc> dev;
    std::vector<q4::SchedChunk> chunks;
    int grid = 0, flags = 0, max_k = 0;
    const q4_status st = plan_layout(fn, descs, count, &dev, &chunks, &grid, &flags, &max_k);
    if (st) return st;
    const size_t need = plan_size(count, chunks.size());
    if (plan_bytes < need) return fail(Q4_ERR_WORKSPACE, "%s: plan buffer of %zu bytes needed", fn, need);
    if (!aligned(plan_buf, 16)) return fail(Q4_ERR_MISALIGNED, "%s: plan buffer must be 16-byte aligned", fn);
    if (check_buffer(fn, "plan buffer", plan_buf, need, descs, count, 1)) return Q4_ERR_INVALID_ARG;
    std::vector<uint8_t> host(need);
    q4::SchedHead head = {0u, 0u, (int32_t)chunks.size(), (int32_t)grid};
    std::memcpy(host.data(), &head, sizeof(head));
    std::memcpy(host.data() + sizeof(head), dev.data(), dev.size() * sizeof(q4::PlanDesc));
    std::memcpy(host.data() + sizeof(head) + dev.size() * sizeof(q4::PlanDesc), chunks.data(),
                chunks.size() * sizeof(q4::SchedChunk));
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(plan_buf, host.data(), need, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e, "q4_0_gemv_batch_plan copy");
    plan->device = plan_buf;
    plan->count = count;
    plan->max_k = max_k;
    plan->grid = grid;
    plan->nchunks = (int)chunks.size();
    plan->flags = flags;
    return ok();
}

q4_status q4_0_gemv_batch(const q4_gemv_plan* plan, void* stream) {
    if (!plan || !plan->device) return fail(Q4_ERR_INVALID_ARG, "q4_0_gemv_batch: null plan");
    if (plan->count < 1 || plan->max_k < 64 || plan->max_k > q4::kFastMaxK || plan->grid < 1 ||
        plan->nchunks < plan->grid || (plan->flags & ~(q4::kPlanQuad | q4::kPlanWide8)) != 0)
        return fail(Q4_ERR_INVALID_ARG, "q4_0_gemv_batch: plan was not filled by q4_0_gemv_batch_plan");
    const hipError_t e = q4::launch_gemv_batch(plan->device, plan->count, plan->nchunks, plan->grid, plan->max_k,
                                               plan->flags, static_cast<hipStream_t>(stream));
    return hip_status(e, "q4_0_gemv_batch launch");
}

q4_status q4_0_gemv_batch_handoff(const q4_gemv_plan* plan, const float* y, const float* residual, void* h16,
                                  void* stream) {
    const char* fn = "q4_0_gemv_batch_handoff";
    if (!plan || !plan->device) return fail(Q4_ERR_INVALID_ARG, "%s: null plan", fn);
    if (plan->count < 1 || plan->max_k < 64 || plan->max_k > q4::kFastMaxK || plan->grid < 1 ||
        plan->nchunks < plan->grid || (plan->flags & ~(q4::kPlanQuad | q4::kPlanWide8)) != 0)
        return fail(Q4_ERR_INVALID_ARG, "%s: plan was not filled by q4_0_gemv_batch_plan", fn);
    if (!y || !h16) return fail(Q4_ERR_INVALID_ARG, "%s: null y or h16", fn);
    if (!aligned(h16, 2)) return fail(Q4_ERR_MISALIGNED, "%s: h16 must be 2-byte aligned", fn);
    if (residual && !aligned(residual, 4)) return fail(Q4_ERR_MISALIGNED, "%s: residual must be 4-byte aligned", fn);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    std::vector<q4::PlanDesc> dev(plan->count);
    uint8_t* table = static_cast<uint8_t*>(plan->device) + sizeof(q4::SchedHead);
    hipError_t e = hipMemcpyAsync(dev.data(), table, dev.size() * sizeof(q4::PlanDesc), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e, "q4_0_gemv_batch_handoff read-back");
    int index = -1;
    for (int i = 0; i < plan->count; ++i)
        if (dev[i].y == y) index = i;
    if (index < 0) return fail(Q4_ERR_INVALID_ARG, "%s: no GEMV of the plan writes that y", fn);
    q4::PlanDesc& d = dev[index];
    const Range rh = range(h16, (size_t)d.n * 2);
    const Range rr = residual ? range(residual, (size_t)d.n * 4) : Range{0, 0};
    // the whole plan: head, descriptors and the chunk table the kernel reads during a launch
    const Range rp = range(plan->device, plan_size(plan->count, (size_t)plan->nchunks));
    if (overlap(rh, rp) || (residual && (overlap(rh, rr) || overlap(rr, rp))))
        return fail(Q4_ERR_INVALID_ARG, "%s: h16, the residual and the plan must not overlap", fn);
    for (int i = 0; i < plan->count; ++i) {
        const q4::PlanDesc& o = dev[i];
        const Range rw = range(o.w, (size_t)(o.n * row_bytes(o.k))), rx = range(o.x, (size_t)o.k * 2);
        if (overlap(rh, rw) || overlap(rh, rx))
            return fail(Q4_ERR_INVALID_ARG, "%s: h16 overlaps an input of descriptor %d", fn, i);
        if (i != index) {
            const Range ry = o.h16 ? range(o.y, (size_t)o.n * 2) : range(o.y, (size_t)o.n * 4);
            if (overlap(rh, ry) || (residual && overlap(rr, ry)))
                return fail(Q4_ERR_INVALID_ARG, "%s: h16 or the residual overlaps the output of descriptor %d", fn, i);
        }
    }
    d.y = static_cast<float*>(h16);
    d.residual = residual;
    d.h16 = 1;
    e = hipMemcpyAsync(table + (size_t)index * sizeof(q4::PlanDesc), &d, sizeof(d), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return hip_status(e, "q4_0_gemv_batch_handoff copy");
}

size_t q8_0_gemv_batch_plan_bytes(const q4_gemv_desc* descs, int count) {
    Q8Layout L;
    if (q8_layout("q8_0_gemv_batch_plan_bytes", descs, count, &L)) return 0;
    ok();
    return L.bytes;
}

q4_status q8_0_gemv_batch_plan(const q4_gemv_desc* descs, int count, void* plan_buf, size_t plan_bytes,
                               q8_gemv_plan* plan, void* stream) {
    const char* fn = "q8_0_gemv_batch_plan";
    if (!plan || !plan_buf) return fail(Q4_ERR_INVALID_ARG, "%s: null pointer", fn);
    Q8Layout L;
    const q4_status st = q8_layout(fn, descs, count, &L);
    if (st) return st;
    if (plan_bytes < L.bytes) return fail(Q4_ERR_WORKSPACE, "%s: plan buffer of %zu bytes needed", fn, L.bytes);
    if (!aligned(plan_buf, 16)) return fail(Q4_ERR_MISALIGNED, "%s: plan buffer must be 16-byte aligned", fn);
    const Range rp = range(plan_buf, L.bytes);
    for (const Range& r : L.outs)
        if (overlap(rp, r)) return fail(Q4_ERR_INVALID_ARG, "%s: the plan buffer overlaps a tensor", fn);
    for (const Range& r : L.ins)
        if (overlap(rp, r)) return fail(Q4_ERR_INVALID_ARG, "%s: the plan buffer overlaps a tensor", fn);
    std::vector<uint8_t> host(L.bytes, 0);
    if (!L.slab.empty()) {
        const q4::SchedHead sh = {0u, 0u, (int32_t)L.chunks.size(), (int32_t)L.grid_slab};
        std::memcpy(host.data(), &sh, sizeof(sh));
        std::memcpy(host.data() + sizeof(sh), L.slab.data(), L.slab.size() * sizeof(q4::PlanDesc));
        std::memcpy(host.data() + sizeof(sh) + L.slab.size() * sizeof(q4::PlanDesc), L.chunks.data(),
                    L.chunks.size() * sizeof(q4::SchedChunk));
    }
    if (!L.other.empty()) {
        uint8_t* o = host.data() + L.off_other;
        std::memcpy(o, &L.head, sizeof(L.head));
        std::memcpy(o + sizeof(L.head), L.other.data(), L.other.size() * sizeof(q4::Q8Desc));
        std::memcpy(o + sizeof(L.head) + L.other.size() * sizeof(q4::Q8Desc), L.wg_begin.data(),
                    L.wg_begin.size() * sizeof(int64_t));
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(plan_buf, host.data(), L.bytes, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e, "q8_0_gemv_batch_plan copy");
    plan->device = plan_buf;
    plan->count = count;
    plan->n_slab = (int)L.slab.size();
    plan->grid_slab = L.grid_slab;
    plan->nchunks_slab = (int)L.chunks.size();
    plan->max_k = L.max_k_other;
    plan->grid = L.grid_other;
    plan->offset_other = L.off_other;
    return ok();
}

q4_status q8_0_gemv_batch(const q8_gemv_plan* plan, void* stream) {
    const char* fn = "q8_0_gemv_batch";
    if (!plan || !plan->device) return fail(Q4_ERR_INVALID_ARG, "%s: null plan", fn);
    const int n_other = plan->count - plan->n_slab;
    const bool slab_ok = plan->n_slab == 0 ? plan->grid_slab == 0
                                           : plan->grid_slab >= 1 && plan->nchunks_slab >= plan->grid_slab;
    const bool other_ok = n_other == 0 ? plan->grid == 0
                                       : plan->grid >= 1 && plan->max_k >= 32 && plan->max_k <= q4::kFastMaxK &&
                                             plan->max_k % 32 == 0 && plan->offset_other % 16 == 0;
    if (plan->count < 1 || plan->n_slab < 0 || n_other < 0 || !slab_ok || !other_ok)
        return fail(Q4_ERR_INVALID_ARG, "%s: plan was not filled by q8_0_gemv_batch_plan", fn);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (plan->n_slab > 0) e = q4::launch_q8_slab_batch(plan->device, plan->n_slab, plan->grid_slab, s);
    if (e == hipSuccess && n_other > 0)
        e = q4::launch_q8_batch(static_cast<uint8_t*>(plan->device) + plan->offset_other, n_other, plan->grid,
                                plan->max_k, s);
    return hip_status(e, "q8_0_gemv_batch launch");
}

size_t q4_0_gemm_smallm_batch_plan_bytes(int count) {
    if (count < 1 || count > (1 << 20)) return 0;
    return (size_t)count * sizeof(q4::SmDesc);
}

q4_status q4_0_gemm_smallm_batch_plan(const q4_gemv_desc* descs, int count, int64_t m, void* plan_buf,
                                      size_t plan_bytes, q4_gemm_plan* plan, void* stream) {
    const char* fn = "q4_0_gemm_smallm_batch_plan";
    if (!plan || !plan_buf) return fail(Q4_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (m < 2 || m > 16) return fail(Q4_ERR_INVALID_ARG, "%s: m = %lld outside [2, 16]", fn, (long long)m);
    int max_k = 0;
    q4_status st = check_list(fn, descs, count, m, 16, kMaxK, &max_k);
    if (st) return st;
    const size_t need = q4_0_gemm_smallm_batch_plan_bytes(count);
    if (plan_bytes < need) return fail(Q4_ERR_WORKSPACE, "%s: plan buffer of %zu bytes needed", fn, need);
    if (!aligned(plan_buf, 16)) return fail(Q4_ERR_MISALIGNED, "%s: plan buffer must be 16-byte aligned", fn);
    if (check_buffer(fn, "plan buffer", plan_buf, need, descs, count, m)) return Q4_ERR_INVALID_ARG;
    for (int i = 0; i < count; ++i)
        if (!aligned(descs[i].w, 4)) return fail(Q4_ERR_MISALIGNED, "%s: descriptor %d: w must be 4-byte aligned", fn, i);
    std::vector<q4::SmDesc> dev(count);
    int64_t ws = 0, cost = 0, max_mn = 0;
    int max_p = 0;
    bool split = false;
    for (int i = 0; i < count; ++i) {
        q4::SmDesc& d = dev[i];
        d.w = static_cast<const uint8_t*>(descs[i].w);
        d.x = static_cast<const uint16_t*>(descs[i].x);
        d.y = descs[i].y;
        d.n = descs[i].n;
        d.k = (int32_t)descs[i].k;
        ws += q4::smallm_fill(&d, m, ws, cost);
        cost += q4::smallm_cost(d);
        max_p = std::max(max_p, (int)d.P);
        max_mn = std::max(max_mn, m * d.n);
        split = split || d.nranges > 1;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(plan_buf, dev.data(), need, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e, "q4_0_gemm_smallm_batch_plan copy");
    plan->device = plan_buf;
    plan->count = count;
    plan->m = (int)m;
    plan->max_p = max_p;
    plan->flags = split ? 1 : 0;
    plan->total_cost = cost;
    plan->max_mn = max_mn;
    plan->workspace_bytes = (size_t)ws * sizeof(float);
    return ok();
}

q4_status q4_0_gemm_smallm_batch(const q4_gemm_plan* plan, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "q4_0_gemm_smallm_batch";
    if (!plan || !plan->device) return fail(Q4_ERR_INVALID_ARG, "%s: null plan", fn);
    if (plan->count < 1 || plan->m < 2 || plan->m > 16 || plan->total_cost < 1 || plan->max_p < 16)
        return fail(Q4_ERR_INVALID_ARG, "%s: plan was not filled by q4_0_gemm_smallm_batch_plan", fn);
    if (plan->workspace_bytes) {
        if (!workspace || workspace_bytes < plan->workspace_bytes)
            return fail(Q4_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, plan->workspace_bytes);
        if (!aligned(workspace, 16)) return fail(Q4_ERR_MISALIGNED, "%s: workspace must be 16-byte aligned", fn);
    }
    const hipError_t e = q4::launch_gemm_smallm_batch(
        static_cast<const q4::SmDesc*>(plan->device), plan->count, plan->m, plan->total_cost, plan->max_p,
        plan->max_mn, (plan->flags & 1) != 0, static_cast<float*>(workspace), static_cast<hipStream_t>(stream));
    return hip_status(e, "q4_0_gemm_smallm_batch launch");
}

size_t q4_0_gemm_prefill_batch_plan_bytes(int count) {
    if (count < 1 || count > (1 << 20)) return 0;
    return 2 * sizeof(q4::PfHead) + (size_t)count * sizeof(q4::PfDesc);
}

q4_status q4_0_gemm_prefill_batch_plan(const q4_gemv_desc* descs, int count, int64_t m, void* plan_buf,
                                       size_t plan_bytes, q4_prefill_plan* plan, void* stream) {
    const char* fn = "q4_0_gemm_prefill_batch_plan";
    if (!plan || !plan_buf) return fail(Q4_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (m < 1 || m > (int64_t(1) << 30)) return fail(Q4_ERR_INVALID_ARG, "%s: m = %lld outside [1, 2^30]", fn, (long long)m);
    int max_k = 0;
    q4_status st = check_list(fn, descs, count, m, int64_t(1) << 30, kMaxK, &max_k);
    if (st) return st;
    for (int i = 0; i < count; ++i)
        if (m * descs[i].n > (int64_t(1) << 40) || descs[i].n > (int64_t(1) << 30))
            return fail(Q4_ERR_INVALID_ARG, "%s: descriptor %d: m*n too large", fn, i);
    const size_t need = q4_0_gemm_prefill_batch_plan_bytes(count);
    if (plan_bytes < need) return fail(Q4_ERR_WORKSPACE, "%s: plan buffer of %zu bytes needed", fn, need);
    if (!aligned(plan_buf, 16)) return fail(Q4_ERR_MISALIGNED, "%s: plan buffer must be 16-byte aligned", fn);
    if (check_buffer(fn, "plan buffer", plan_buf, need, descs, count, m)) return Q4_ERR_INVALID_ARG;
    const int tile_m = q4::prefill_batch_tile_m(m);
    // Two work heads (per-XCD tile ranges, counters zero), then the
    // descriptors with k % 256 == 0 (run by the kernel that moves weights in
    // 144-byte chunks), then the others, each part in list order and numbering
    // its tiles from 0.
    std::vector<uint8_t> host(need, 0);
    q4::PfDesc* dev = reinterpret_cast<q4::PfDesc*>(host.data() + 2 * sizeof(q4::PfHead));
    int64_t tiles[2] = {0, 0};
    int placed = 0;
    for (int part = 0; part < 2; ++part) {
        const int part_first = placed;
        for (int i = 0; i < count; ++i) {
            if ((descs[i].k % 256 == 0) != (part == 0)) continue;
            q4::PfDesc d = {};
            d.w = static_cast<const uint8_t*>(descs[i].w);
            d.x = static_cast<const uint16_t*>(descs[i].x);
            d.y = descs[i].y;
            d.m = m;
            d.n = descs[i].n;
            d.k = (int)descs[i].k;
            tiles[part] += q4::prefill_fill(&d, part == 0 ? tile_m : q4::prefill_other_tile_m(tile_m), tiles[part]);
            if (tiles[part] >= (int64_t(1) << 31)) return fail(Q4_ERR_INVALID_ARG, "%s: more than 2^31 tiles", fn);
            std::memcpy(&dev[placed++], &d, sizeof(d));
        }
        // the part's tile ranges per XCD (descriptor indices relative to the part)
        q4::PfHead head;
        if (placed > part_first) q4::prefill_queues(dev + part_first, placed - part_first, tiles[part], &head);
        else head = q4::PfHead{};
        std::memcpy(host.data() + part * sizeof(q4::PfHead), &head, sizeof(head));
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(plan_buf, host.data(), need, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e, "q4_0_gemm_prefill_batch_plan copy");
    int n_chunked = 0;
    for (int i = 0; i < count; ++i) n_chunked += descs[i].k % 256 == 0;
    plan->device = plan_buf;
    plan->count = count;
    plan->m = (int)m;
    plan->tile_m = tile_m;
    plan->count_chunked = n_chunked;
    plan->tiles_chunked = tiles[0];
    plan->tiles_other = tiles[1];
    return ok();
}

q4_status q4_0_gemm_prefill_batch(const q4_prefill_plan* plan, void* stream) {
    const char* fn = "q4_0_gemm_prefill_batch";
    if (!plan || !plan->device) return fail(Q4_ERR_INVALID_ARG, "%s: null plan", fn);
    const int n_other = plan->count - plan->count_chunked;
    if (plan->count < 1 || plan->m < 1 || (plan->tile_m != 64 && plan->tile_m != 96 && plan->tile_m != 128) || plan->count_chunked < 0 ||
        n_other < 0 || (plan->count_chunked > 0) != (plan->tiles_chunked > 0) || (n_other > 0) != (plan->tiles_other > 0))
        return fail(Q4_ERR_INVALID_ARG, "%s: plan was not filled by q4_0_gemm_prefill_batch_plan", fn);
    const hipError_t e =
        q4::launch_gemm_prefill_batch(plan->device, plan->count_chunked, plan->tiles_chunked, n_other,
                                      plan->tiles_other, plan->tile_m, static_cast<hipStream_t>(stream));
    return hip_status(e, "q4_0_gemm_prefill_batch launch");
}

}  // extern "C"
