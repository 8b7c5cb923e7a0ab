"""Q4_0 dequantize-and-multiply on MI355X (gfx950): Python binding of libq4gemv.so.

Argument marshalling only.  Every function checks dtypes, shapes, devices and
contiguity of torch tensors, then calls the C ABI declared in
``include/q4gemv.h`` with raw device pointers and torch's current HIP stream.
All arithmetic happens in the HIP kernels; there is no CPU fallback, and the
import fails loudly when the library has not been built
(``python -m q4_dequant_gemv_block_amd.build``).

Weight tensors are uint8 of shape [N, K/32*18] (packed Q4_0 rows, the block
format the pages call "GGUF Q4_0": f16 scale then 16 bytes of nibble codes,
weight = (code - 8) * scale); activations are float16; outputs float32.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4gemv.so")

Q4_OK = 0
Q4_ERR_INVALID_ARG = -1
Q4_ERR_MISALIGNED = -2
Q4_ERR_WORKSPACE = -3
Q4_ERR_HIP = -4

Q4_OP_GEMV = 0
Q4_OP_GEMM_SMALLM = 1
Q4_OP_GEMM_PREFILL = 2
Q4_OP_LM_HEAD_ARGMAX = 3
Q4_OP_LM_HEAD_VERIFY = 4
Q4_OP_LM_HEAD_NORM_ARGMAX = 5

# Every symbol include/q4gemv.h declares.
EXPORTS = (
    "q4_abi_version", "q4_last_error", "q4_workspace_bytes", "q4_0_gemv", "q4_0_gemm_smallm",
    "q4_0_gemm_prefill", "lm_head_argmax", "lm_head_argmax_noalloc", "lm_head_norm_argmax", "lm_head_verify",
    "q4_0_gemv_handoff", "q8_0_gemv", "q8_0_gemv_batch_plan_bytes",
    "q8_0_gemv_batch_plan", "q8_0_gemv_batch",
    "q4_0_gemv_batch_plan_bytes", "q4_0_gemv_batch_plan",
    "q4_0_gemm_smallm_batch_plan_bytes", "q4_0_gemm_smallm_batch_plan", "q4_0_gemm_smallm_batch",
    "q4_0_gemm_prefill_batch_plan_bytes", "q4_0_gemm_prefill_batch_plan", "q4_0_gemm_prefill_batch",
    "q4_0_gemv_batch", "q4_0_gemv_batch_handoff",
)


class Q4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("q4 status %d: %s" % (status, message))
        self.status = status


class GemvDesc(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64)]


class GemvPlan(ctypes.Structure):
    _fields_ = [("device", ctypes.c_void_p), ("count", ctypes.c_int), ("max_k", ctypes.c_int),
                ("grid", ctypes.c_int), ("nchunks", ctypes.c_int), ("flags", ctypes.c_int)]


class Q8Plan(ctypes.Structure):
    _fields_ = [("device", ctypes.c_void_p), ("count", ctypes.c_int), ("n_slab", ctypes.c_int),
                ("grid_slab", ctypes.c_int), ("nchunks_slab", ctypes.c_int), ("max_k", ctypes.c_int),
                ("grid", ctypes.c_int), ("offset_other", ctypes.c_size_t)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libq4gemv.so and declare its signatures (raises if it is not built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libq4gemv.so is not built (%s); run python -m q4_dequant_gemv_block_amd.build" % path)
    lib = ctypes.CDLL(path)
    vp, i64, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.q4_abi_version.restype = ctypes.c_int
    lib.q4_abi_version.argtypes = []
    lib.q4_last_error.restype = ctypes.c_char_p
    lib.q4_last_error.argtypes = []
    lib.q4_workspace_bytes.restype = ctypes.c_size_t
    lib.q4_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i64]
    lib.q4_0_gemv.restype = st
    lib.q4_0_gemv.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.q4_0_gemm_smallm.restype = st
    lib.q4_0_gemm_smallm.argtypes = [vp, vp, vp, i64, i64, i64, vp, ctypes.c_size_t, vp]
    lib.q4_0_gemm_prefill.restype = st
    lib.q4_0_gemm_prefill.argtypes = [vp, vp, vp, i64, i64, i64, vp, ctypes.c_size_t, vp]
    lib.lm_head_argmax.restype = st
    lib.lm_head_argmax.argtypes = [vp, vp, vp, vp, i64, i64, vp, ctypes.c_size_t, vp]
    lib.lm_head_argmax_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, vp]
    lib.lm_head_argmax_noalloc.restype = st
    lib.lm_head_verify.restype = st
    lib.q8_0_gemv.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.q8_0_gemv.restype = ctypes.c_int
    lib.q4_0_gemv_batch_handoff.argtypes = [ctypes.POINTER(GemvPlan), vp, vp, vp, vp]
    lib.q4_0_gemv_batch_handoff.restype = ctypes.c_int
    lib.q8_0_gemv_batch_plan_bytes.argtypes = [ctypes.POINTER(GemvDesc), ctypes.c_int]
    lib.q8_0_gemv_batch_plan_bytes.restype = ctypes.c_size_t
    lib.q8_0_gemv_batch_plan.argtypes = [ctypes.POINTER(GemvDesc), ctypes.c_int, vp, ctypes.c_size_t,
                                         ctypes.POINTER(Q8Plan), vp]
    lib.q8_0_gemv_batch_plan.restype = ctypes.c_int
    lib.q8_0_gemv_batch.argtypes = [ctypes.POINTER(Q8Plan), vp]
    lib.q8_0_gemv_batch.restype = ctypes.c_int
    lib.q4_0_gemv_handoff.argtypes = [vp, vp, vp, vp, i64, i64, vp]
    lib.q4_0_gemv_handoff.restype = ctypes.c_int
    lib.lm_head_norm_argmax.argtypes = [vp, vp, vp, ctypes.c_float, vp, vp, vp, i64, i64, vp, ctypes.c_size_t, vp]
    lib.lm_head_norm_argmax.restype = ctypes.c_int
    lib.lm_head_verify.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp, ctypes.c_size_t, vp]
    lib.q4_0_gemv_batch_plan_bytes.restype = ctypes.c_size_t
    lib.q4_0_gemv_batch_plan_bytes.argtypes = [ctypes.POINTER(GemvDesc), ctypes.c_int]
    lib.q4_0_gemv_batch_plan.restype = st
    lib.q4_0_gemv_batch_plan.argtypes = [ctypes.POINTER(GemvDesc), ctypes.c_int, vp, ctypes.c_size_t,
                                         ctypes.POINTER(GemvPlan), vp]
    lib.q4_0_gemv_batch.restype = st
    lib.q4_0_gemv_batch.argtypes = [ctypes.POINTER(GemvPlan), vp]
    lib.q4_0_gemm_smallm_batch_plan_bytes.restype = ctypes.c_size_t
    lib.q4_0_gemm_smallm_batch_plan_bytes.argtypes = [ctypes.c_int]
    lib.q4_0_gemm_smallm_batch_plan.restype = st
    lib.q4_0_gemm_smallm_batch_plan.argtypes = [ctypes.POINTER(GemvDesc), ctypes.c_int, i64, vp, ctypes.c_size_t,
                                                ctypes.POINTER(GemmPlan), vp]
    lib.q4_0_gemm_smallm_batch.restype = st
    lib.q4_0_gemm_smallm_batch.argtypes = [ctypes.POINTER(GemmPlan), vp, ctypes.c_size_t, vp]
    lib.q4_0_gemm_prefill_batch_plan_bytes.restype = ctypes.c_size_t
    lib.q4_0_gemm_prefill_batch_plan_bytes.argtypes = [ctypes.c_int]
    lib.q4_0_gemm_prefill_batch_plan.restype = st
    lib.q4_0_gemm_prefill_batch_plan.argtypes = [ctypes.POINTER(GemvDesc), ctypes.c_int, i64, vp, ctypes.c_size_t,
                                                 ctypes.POINTER(PrefillPlan), vp]
    lib.q4_0_gemm_prefill_batch.restype = st
    lib.q4_0_gemm_prefill_batch.argtypes = [ctypes.POINTER(PrefillPlan), vp]
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(status: int):
    if status != Q4_OK:
        raise Q4Error(status, load_library().q4_last_error().decode())


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t: torch.Tensor, dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def row_bytes(k: int) -> int:
    return k // 32 * 18


def _weights(w: torch.Tensor, k: int) -> int:
    if w.dim() == 2:
        if w.shape[1] != row_bytes(k):
            raise ValueError("w has %d bytes per row, k=%d needs %d" % (w.shape[1], k, row_bytes(k)))
        return w.shape[0]
    if w.dim() == 1 and w.numel() % row_bytes(k) == 0:
        return w.numel() // row_bytes(k)
    raise ValueError("w must be uint8 [N, K/32*18]")


def abi_version() -> int:
    return load_library().q4_abi_version()


def last_error() -> str:
    return load_library().q4_last_error().decode()


def workspace_bytes(op: int, m: int, n: int, k: int) -> int:
    return int(load_library().q4_workspace_bytes(op, m, n, k))


def q4_0_gemv(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = W x for packed Q4_0 rows W (uint8 [N, K/32*18]) and x (float16 [K]); y float32 [N]."""
    if x.dim() != 1:
        raise ValueError("x must be float16 [K]")
    k = x.shape[0]
    n = _weights(w, k)
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=x.device)
    elif out.numel() != n:
        raise ValueError("out must hold N=%d floats" % n)
    _check(load_library().q4_0_gemv(_ptr(w, torch.uint8, "w"), _ptr(x, torch.float16, "x"),
                                    _ptr(out, torch.float32, "out"), n, k, _stream(stream)))
    return out


def q4_0_gemm_smallm(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = X W^T for X float16 [M, K] with 1 <= M <= 16; Y float32 [M, N]."""
    if x.dim() != 2:
        raise ValueError("x must be float16 [M, K]")
    m, k = x.shape
    n = _weights(w, k)
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    elif out.numel() != m * n:
        raise ValueError("out must hold M*N floats")
    need = workspace_bytes(Q4_OP_GEMM_SMALLM, m, n, k)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wp = _ptr(workspace, torch.uint8, "workspace") if workspace is not None else None
    wb = workspace.numel() if workspace is not None else 0
    _check(load_library().q4_0_gemm_smallm(_ptr(w, torch.uint8, "w"), _ptr(x, torch.float16, "x"),
                                           _ptr(out, torch.float32, "out"), m, n, k, wp, wb, _stream(stream)))
    return out


def q4_0_gemm_prefill(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = X W^T for X float16 [M, K] (any M >= 1) on the matrix cores; Y float32 [M, N]."""
    if x.dim() != 2:
        raise ValueError("x must be float16 [M, K]")
    m, k = x.shape
    n = _weights(w, k)
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    elif out.numel() != m * n:
        raise ValueError("out must hold M*N floats")
    need = workspace_bytes(Q4_OP_GEMM_PREFILL, m, n, k)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wp = _ptr(workspace, torch.uint8, "workspace") if workspace is not None else None
    wb = workspace.numel() if workspace is not None else 0
    _check(load_library().q4_0_gemm_prefill(_ptr(w, torch.uint8, "w"), _ptr(x, torch.float16, "x"),
                                            _ptr(out, torch.float32, "out"), m, n, k, wp, wb, _stream(stream)))
    return out


def lm_head_argmax(w: torch.Tensor, h: torch.Tensor, logits: torch.Tensor | None = None,
                   token: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                   stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """(logits float32 [V], token int32 [1]) for the LM head W (uint8 [V, K/32*18]) and h (float16 [K])."""
    if h.dim() != 1:
        raise ValueError("h must be float16 [K]")
    k = h.shape[0]
    n = _weights(w, k)
    if logits is None:
        logits = torch.empty(n, dtype=torch.float32, device=h.device)
    if token is None:
        token = torch.empty(1, dtype=torch.int32, device=h.device)
    need = workspace_bytes(Q4_OP_LM_HEAD_ARGMAX, 1, n, k)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=h.device)
    _check(load_library().lm_head_argmax(_ptr(w, torch.uint8, "w"), _ptr(h, torch.float16, "h"),
                                         _ptr(logits, torch.float32, "logits"), _ptr(token, torch.int32, "token"),
                                         n, k, _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                         _stream(stream)))
    return logits, token


def lm_head_argmax_noalloc(w: torch.Tensor, h: torch.Tensor, logits: torch.Tensor | None = None,
                           token: torch.Tensor | None = None, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """lm_head_argmax with the per-workgroup keys in the library's own per-device
    array: the C call allocates nothing (pass logits and token to allocate nothing here either)."""
    if h.dim() != 1:
        raise ValueError("h must be float16 [K]")
    k = h.shape[0]
    n = _weights(w, k)
    if logits is None:
        logits = torch.empty(n, dtype=torch.float32, device=h.device)
    if token is None:
        token = torch.empty(1, dtype=torch.int32, device=h.device)
    _check(load_library().lm_head_argmax_noalloc(_ptr(w, torch.uint8, "w"), _ptr(h, torch.float16, "h"),
                                                 _ptr(logits, torch.float32, "logits"),
                                                 _ptr(token, torch.int32, "token"), n, k, _stream(stream)))
    return logits, token


def q8_row_bytes(k: int) -> int:
    """Bytes of one Q8_0 row of K weights (K/32 blocks of 34 bytes)."""
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    return k // 32 * 34


def q8_0_gemv(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y float32 [N] = W x for Q8_0 weights W (uint8 [N, K/32*34]) and x (float16 [K])."""
    if x.dim() != 1:
        raise ValueError("x must be float16 [K]")
    k = x.shape[0]
    if w.dim() != 2 or w.shape[1] != q8_row_bytes(k):
        raise ValueError("w must be uint8 [N, K/32*34]")
    n = w.shape[0]
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=x.device)
    _check(load_library().q8_0_gemv(_ptr(w, torch.uint8, "w"), _ptr(x, torch.float16, "x"),
                                    _ptr(out, torch.float32, "out"), n, k, _stream(stream)))
    return out


def q4_0_gemv_handoff(w: torch.Tensor, x: torch.Tensor, residual: torch.Tensor | None = None,
                      out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The stage hand-off: float16 [N] = binary16(residual + W x) for W (uint8 [N, K/32*18]),
    x (float16 [K]) and an optional float32 residual [N]."""
    if x.dim() != 1:
        raise ValueError("x must be float16 [K]")
    k = x.shape[0]
    n = _weights(w, k)
    if out is None:
        out = torch.empty(n, dtype=torch.float16, device=x.device)
    rp = 0
    if residual is not None:
        if residual.dim() != 1 or residual.shape[0] != n:
            raise ValueError("residual must be float32 [N]")
        rp = _ptr(residual, torch.float32, "residual")
    _check(load_library().q4_0_gemv_handoff(_ptr(w, torch.uint8, "w"), _ptr(x, torch.float16, "x"), rp,
                                            _ptr(out, torch.float16, "out"), n, k, _stream(stream)))
    return out


def lm_head_norm_argmax(w: torch.Tensor, h: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6,
                        logits: torch.Tensor | None = None, token: torch.Tensor | None = None,
                        x_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                        stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """Final norm of h, then the LM head: (logits float32 [V], token int32 [1]) for W
    (uint8 [V, K/32*18]), the hidden state h and the norm's gain gamma (float16 [K]).
    x_out (float16 [K], optional) receives the normed activation."""
    if h.dim() != 1 or gamma.dim() != 1 or gamma.shape[0] != h.shape[0]:
        raise ValueError("h and gamma must be float16 [K]")
    k = h.shape[0]
    n = _weights(w, k)
    if logits is None:
        logits = torch.empty(n, dtype=torch.float32, device=h.device)
    if token is None:
        token = torch.empty(1, dtype=torch.int32, device=h.device)
    need = workspace_bytes(Q4_OP_LM_HEAD_NORM_ARGMAX, 1, n, k)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=h.device)
    xo = 0
    if x_out is not None:
        if x_out.dim() != 1 or x_out.shape[0] != k:
            raise ValueError("x_out must be float16 [K]")
        xo = _ptr(x_out, torch.float16, "x_out")
    _check(load_library().lm_head_norm_argmax(_ptr(w, torch.uint8, "w"), _ptr(h, torch.float16, "h"),
                                              _ptr(gamma, torch.float16, "gamma"), float(eps),
                                              _ptr(logits, torch.float32, "logits"),
                                              _ptr(token, torch.int32, "token"), xo, n, k,
                                              _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                              _stream(stream)))
    return logits, token


def lm_head_verify(w: torch.Tensor, h: torch.Tensor, draft: torch.Tensor, logits: torch.Tensor | None = None,
                   tokens: torch.Tensor | None = None, accepted: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None, stream=None):
    """(logits float32 [M, V], tokens int32 [M], accepted int32 [1]) for the LM head W
    (uint8 [V, K/32*18]), the trunk's hidden states h (float16 [M, K], M <= 16) and the
    draft's tokens for the same positions (int32 [M])."""
    if h.dim() != 2:
        raise ValueError("h must be float16 [M, K]")
    m, k = h.shape
    n = _weights(w, k)
    if draft.dim() != 1 or draft.shape[0] != m:
        raise ValueError("draft must be int32 [M]")
    if logits is None:
        logits = torch.empty((m, n), dtype=torch.float32, device=h.device)
    if tokens is None:
        tokens = torch.empty(m, dtype=torch.int32, device=h.device)
    if accepted is None:
        accepted = torch.empty(1, dtype=torch.int32, device=h.device)
    need = workspace_bytes(Q4_OP_LM_HEAD_VERIFY, m, n, k)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=h.device)
    _check(load_library().lm_head_verify(_ptr(w, torch.uint8, "w"), _ptr(h, torch.float16, "h"),
                                         _ptr(logits, torch.float32, "logits"), _ptr(tokens, torch.int32, "tokens"),
                                         _ptr(draft, torch.int32, "draft"), _ptr(accepted, torch.int32, "accepted"),
                                         m, n, k, _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                         _stream(stream)))
    return logits, tokens, accepted


class GemmPlan(ctypes.Structure):
    _fields_ = [("device", ctypes.c_void_p), ("count", ctypes.c_int), ("m", ctypes.c_int),
                ("max_p", ctypes.c_int), ("flags", ctypes.c_int), ("total_cost", ctypes.c_int64),
                ("max_mn", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t)]


class PrefillPlan(ctypes.Structure):
    _fields_ = [("device", ctypes.c_void_p), ("count", ctypes.c_int), ("m", ctypes.c_int),
                ("tile_m", ctypes.c_int), ("count_chunked", ctypes.c_int), ("tiles_chunked", ctypes.c_int64),
                ("tiles_other", ctypes.c_int64)]


class GemvBatch:
    """A list of independent GEMVs (w, x, y) planned once and run as one launch per call."""

    def __init__(self, items, stream=None):
        items = list(items)
        descs = (GemvDesc * len(items))()
        self._keep = []
        for i, (w, x, y) in enumerate(items):
            k = x.shape[-1]
            n = _weights(w, k)
            if y.numel() != n:
                raise ValueError("descriptor %d: y must hold N=%d floats" % (i, n))
            descs[i] = GemvDesc(_ptr(w, torch.uint8, "w"), _ptr(x, torch.float16, "x"),
                                _ptr(y, torch.float32, "y"), n, k)
            self._keep.append((w, x, y))
        lib = load_library()
        dev = items[0][0].device if items else torch.device("cuda")
        self.plan = GemvPlan()
        with torch.cuda.device(dev):  # the schedule is cut for this device
            nbytes = int(lib.q4_0_gemv_batch_plan_bytes(descs, len(items)))
            if nbytes == 0:
                _check(Q4_ERR_INVALID_ARG)
            self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            _check(lib.q4_0_gemv_batch_plan(descs, len(items), self.buffer.data_ptr(), self.buffer.numel(),
                                            ctypes.byref(self.plan), _stream(stream)))

    def set_handoff(self, index: int, h16: torch.Tensor, residual: torch.Tensor | None = None, stream=None):
        """Make item `index` of the list the stage hand-off: it writes float16 h16 [N] =
        residual + W x (rounded once) instead of its float32 y."""
        n = self._keep[index][2].numel()
        if h16.numel() != n:
            raise ValueError("h16 must hold N=%d float16 values" % n)
        rp = 0
        if residual is not None:
            if residual.numel() != n:
                raise ValueError("residual must hold N=%d float32 values" % n)
            rp = _ptr(residual, torch.float32, "residual")
        y = self._keep[index][2]
        _check(load_library().q4_0_gemv_batch_handoff(ctypes.byref(self.plan), _ptr(y, torch.float32, "y"), rp,
                                                      _ptr(h16, torch.float16, "h16"), _stream(stream)))
        self._keep.append((h16, residual))

    def __call__(self, stream=None):
        _check(load_library().q4_0_gemv_batch(ctypes.byref(self.plan), _stream(stream)))


class Q8Batch:
    """A list of Q8_0 GEMVs (w, x, y), w uint8 [N, K/32*34], planned once and run as
    one launch per call."""

    def __init__(self, items, stream=None):
        items = list(items)
        descs = (GemvDesc * len(items))()
        self._keep = []
        for i, (w, x, y) in enumerate(items):
            k = x.shape[-1]
            if w.dim() != 2 or w.shape[1] != q8_row_bytes(k):
                raise ValueError("descriptor %d: w must be uint8 [N, K/32*34]" % i)
            n = w.shape[0]
            if y.numel() != n:
                raise ValueError("descriptor %d: y must hold N=%d floats" % (i, n))
            descs[i] = GemvDesc(_ptr(w, torch.uint8, "w"), _ptr(x, torch.float16, "x"),
                                _ptr(y, torch.float32, "y"), n, k)
            self._keep.append((w, x, y))
        lib = load_library()
        dev = items[0][0].device if items else torch.device("cuda")
        self.plan = Q8Plan()
        with torch.cuda.device(dev):  # the ranges are cut for this device's compute units
            nbytes = int(lib.q8_0_gemv_batch_plan_bytes(descs, len(items)))
            if nbytes == 0:
                _check(Q4_ERR_INVALID_ARG)
            self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            _check(lib.q8_0_gemv_batch_plan(descs, len(items), self.buffer.data_ptr(), self.buffer.numel(),
                                            ctypes.byref(self.plan), _stream(stream)))

    def __call__(self, stream=None):
        _check(load_library().q8_0_gemv_batch(ctypes.byref(self.plan), _stream(stream)))


class SmallMBatch:
    """A list of small-M GEMMs (w, x, y) with x of shape (m, k) and y (m, n), the
    same m for all, planned once and run as one launch (plus one reduction of
    K-range partials when some GEMM splits K) per call."""

    def __init__(self, items, stream=None):
        items = list(items)
        if not items:
            raise ValueError("empty list")
        m = items[0][1].shape[0] if items[0][1].dim() == 2 else 1
        descs = (GemvDesc * len(items))()
        self._keep = []
        for i, (w, x, y) in enumerate(items):
            if x.dim() != 2 or x.shape[0] != m:
                raise ValueError("descriptor %d: x must be (m, k) with m = %d" % (i, m))
            k = x.shape[1]
            n = _weights(w, k)
            if y.numel() != m * n:
                raise ValueError("descriptor %d: y must hold m*N=%d floats" % (i, m * n))
            descs[i] = GemvDesc(_ptr(w, torch.uint8, "w"), _ptr(x, torch.float16, "x"),
                                _ptr(y, torch.float32, "y"), n, k)
            self._keep.append((w, x, y))
        lib = load_library()
        dev = items[0][0].device
        self.m = m
        self.plan = GemmPlan()
        with torch.cuda.device(dev):
            nbytes = int(lib.q4_0_gemm_smallm_batch_plan_bytes(len(items)))
            self.buffer = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
            _check(lib.q4_0_gemm_smallm_batch_plan(descs, len(items), m, self.buffer.data_ptr(),
                                                   self.buffer.numel(), ctypes.byref(self.plan),
                                                   _stream(stream)))
            self.workspace = torch.empty(max(int(self.plan.workspace_bytes), 16), dtype=torch.uint8, device=dev)

    def __call__(self, stream=None):
        _check(load_library().q4_0_gemm_smallm_batch(ctypes.byref(self.plan), self.workspace.data_ptr(),
                                                     self.workspace.numel(), _stream(stream)))


class PrefillBatch:
    """A list of prefill GEMMs (w, x, y) with x of shape (m, k) and y (m, n), the
    same m for all, planned once and run as one launch per call."""

    def __init__(self, items, stream=None):
        items = list(items)
        if not items:
            raise ValueError("empty list")
        m = items[0][1].shape[0]
        descs = (GemvDesc * len(items))()
        self._keep = []
        for i, (w, x, y) in enumerate(items):
            if x.dim() != 2 or x.shape[0] != m:
                raise ValueError("descriptor %d: x must be (m, k) with m = %d" % (i, m))
            k = x.shape[1]
            n = _weights(w, k)
            if y.numel() != m * n:
                raise ValueError("descriptor %d: y must hold m*N=%d floats" % (i, m * n))
            descs[i] = GemvDesc(_ptr(w, torch.uint8, "w"), _ptr(x, torch.float16, "x"),
                                _ptr(y, torch.float32, "y"), n, k)
            self._keep.append((w, x, y))
        lib = load_library()
        dev = items[0][0].device
        self.m = m
        self.plan = PrefillPlan()
        with torch.cuda.device(dev):
            nbytes = int(lib.q4_0_gemm_prefill_batch_plan_bytes(len(items)))
            self.buffer = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
            _check(lib.q4_0_gemm_prefill_batch_plan(descs, len(items), m, self.buffer.data_ptr(),
                                                    self.buffer.numel(), ctypes.byref(self.plan),
                                                    _stream(stream)))

    def __call__(self, stream=None):
        _check(load_library().q4_0_gemm_prefill_batch(ctypes.byref(self.plan), _stream(stream)))


# Short names.
gemv = q4_0_gemv
gemm_smallm = q4_0_gemm_smallm
gemm_prefill = q4_0_gemm_prefill
