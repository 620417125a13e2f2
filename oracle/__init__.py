"""CPU oracle for the TP1 decode projection y[B,N] = x[B,K] . W^T.

TEST INFRASTRUCTURE ONLY: the product library never imports, links or calls
anything here; only tests/, the smoke check and the benchmark's CPU-baseline
leg do.  The oracle shares no code with the GPU path.

It follows the vLLM API page "vllm.models.kimi_k3.nvidia.specialized_decode.
runtime.dep": section "DepProjection" defines the result as the stock
linear's GEMM of x with the weight's transpose (weight in nn.Linear N x K
layout), and the page's opening text fixes the precision (BF16 in, FP32
accumulation, BF16 out, split-K order free).  The C code (oracle.c) sums in
double in ascending k and rounds once to BF16, ties to even.

`exact.py` holds a second, independent brute force over exact rationals for
tiny shapes; it is one of the pins, not a replacement.

Every function here is pinned (see tests/test_oracle.py); none is "parity
unpinned".
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIBS: dict = {}


def _lib(mutant: int = 0):
    lib = _LIBS.get(mutant)
    if lib is not None:
        return lib
    path = _build.lib_path(mutant)
    if not os.path.exists(path) or (
            os.path.getmtime(path) < os.path.getmtime(_build.SRC)):
        _build.build(mutant)
    lib = ctypes.CDLL(path)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    lib.oracle_proj.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                u16p, ctypes.c_long, u16p, ctypes.c_long,
                                u16p, ctypes.c_long, f64p, ctypes.c_long,
                                ctypes.c_int]
    lib.oracle_proj.restype = ctypes.c_int
    lib.oracle_round_bf16.argtypes = [f64p, u16p, ctypes.c_long]
    lib.oracle_round_bf16.restype = None
    lib.oracle_mutant.restype = ctypes.c_int
    _LIBS[mutant] = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _u16(a):
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError("BF16 operands are passed as uint16 bit patterns")
    return a


def proj(x_bits, w_bits, *, threads: int | None = None, want_sum: bool = False,
         mutant: int = 0):
    """y_bits[B,N] (uint16 BF16 patterns) = RNE_bf16(sum_k x[b,k] W[n,k]).

    x_bits: uint16 [B, K] (any row stride, unit column stride)
    w_bits: uint16 [N, K] (any row stride, unit column stride)
    want_sum: also return the unrounded double sums S[B, N].
    """
    x = _u16(x_bits)
    w = _u16(w_bits)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"shape mismatch: x{tuple(x.shape)} W{tuple(w.shape)}")
    if x.strides[1] != 2:
        x = np.ascontiguousarray(x)
    if w.strides[1] != 2:
        w = np.ascontiguousarray(w)
    B, K = x.shape
    N = w.shape[0]
    y = np.zeros((B, N), dtype=np.uint16)
    S = np.zeros((B, N), dtype=np.float64) if want_sum else None
    lib = _lib(mutant)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    ldx = x.strides[0] // 2 if B > 1 else K
    ldw = w.strides[0] // 2 if N > 1 else K
    rc = lib.oracle_proj(
        B, N, K,
        x.ctypes.data_as(u16p), ldx,
        w.ctypes.data_as(u16p), ldw,
        y.ctypes.data_as(u16p), N,
        S.ctypes.data_as(f64p) if S is not None else None, N,
        threads if threads is not None else default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_proj failed ({rc})")
    return (y, S) if want_sum else y


def round_bf16(values, *, mutant: int = 0):
    """uint16 BF16 patterns of float64 `values`, rounded once, ties to even."""
    s = np.ascontiguousarray(np.asarray(values, dtype=np.float64))
    out = np.zeros(s.shape, dtype=np.uint16)
    _lib(mutant).oracle_round_bf16(
        s.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), s.size)
    return out


def bf16_bits_to_f64(bits):
    """Exact decode of BF16 bit patterns to float64 (widen to binary32)."""
    b = _u16(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)
