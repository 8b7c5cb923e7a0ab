"""Helpers of the GPU tests: device tensors from numpy, the parity bar, library loading."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle

TOL = oracle.TOL  # |y_gpu - y_ref| <= TOL * sum_k |w_k x_k| per output


def lib():
    import q4_dequant_gemv_block_amd as q4
    if not os.path.exists(q4.LIB_PATH):
        from q4_dequant_gemv_block_amd import build
        build.build()
    q4.load_library()
    return q4


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def dev_f16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).astype(np.float16, copy=False)).to(device())


def assert_parity(y_gpu, y_ref, a_ref, what=""):
    """Every output within TOL * a of the oracle; outputs with a == 0 exactly zero."""
    y = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y - y_ref)
    bound = TOL * a_ref
    bad = err > bound
    assert not bad.any(), "%s: %d outputs out of bound, worst err/a = %g at %s" % (
        what, int(bad.sum()), float(np.max(err / np.maximum(a_ref, 1e-300))), np.argwhere(bad)[:5].tolist())
    zero = a_ref == 0
    assert np.all(y[zero] == 0), what
    ratio = float(np.max(err / np.where(a_ref > 0, a_ref, 1.0))) if y.size else 0.0
    return ratio
