"""CPU oracle for the block-scaled small-M GEMV (ctypes front end of qgemv_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only users. The product path never imports
this package, and this package imports nothing from the product.

The C file computes Y = A . dequant(W)^T (+ an optional per-column bias) and
S = sum |a*w| in float64 with plain loops; see its header for the pages it follows. This module only marshals
numpy arrays into it, builds it with gcc when the shared object is missing, and
states the acceptance bound the GPU results are held to.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qgemv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

FORMAT_CODES = {"u4": 1, "u8": 2, "fp8": 3, "nvfp4": 4}
ACT_CODES = {"f16": 1, "bf16": 2}

# Acceptance bound per output: |y - y_ref| <= REL * S + ABS with S = sum_k |a*w|.
TOL_REL = 1e-3
TOL_ABS = 1e-3


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fused multiply-add contraction, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [
        ("format", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("pad_", ctypes.c_int32),
        ("N", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("W", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("zp", ctypes.c_void_p),
        ("tensor_scale", ctypes.c_double),
        ("bias", ctypes.c_void_p),
    ]


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            P = ctypes.POINTER(_Problem)
            dp = ctypes.POINTER(ctypes.c_double)
            lib.oracle_tables.argtypes = [dp, dp]
            lib.oracle_decode_f16.argtypes = [ctypes.c_void_p, ctypes.c_int64, dp]
            lib.oracle_decode_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, dp]
            lib.oracle_dequant.argtypes = [P, ctypes.c_int64, ctypes.c_int64]
            lib.oracle_dequant.restype = ctypes.c_double
            lib.oracle_dequant_columns.argtypes = [P, ctypes.c_int64, ctypes.c_int64, dp]
            lib.oracle_gemv.argtypes = [P, ctypes.c_void_p, ctypes.c_int, dp, dp, ctypes.c_int]
            lib.oracle_gemv_points.argtypes = [P, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                               ctypes.c_void_p, ctypes.c_void_p, dp, dp]
            lib.oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _dp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


class _Bound:
    """Keeps the numpy buffers alive while the C structure points at them."""

    def __init__(self, prob):
        self.W = np.ascontiguousarray(prob.W)
        self.scales = np.ascontiguousarray(prob.scales)
        self.zp = None if prob.zp is None else np.ascontiguousarray(prob.zp)
        bias = getattr(prob, "bias", None)
        self.bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
        self.s = _Problem(
            FORMAT_CODES[prob.fmt], ACT_CODES[prob.act], int(prob.bs), 0, int(prob.N), int(prob.K),
            self.W.ctypes.data, self.scales.ctypes.data,
            None if self.zp is None else self.zp.ctypes.data, float(prob.tensor_scale),
            None if self.bias is None else self.bias.ctypes.data,
        )


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected the problem (code {rc})")


# ---------------------------------------------------------------------------------
# public API


def tables() -> Tuple[np.ndarray, np.ndarray]:
    """(E2M1 table [16], E4M3 table [256]) in float64, built from closed forms."""
    lib = _load()
    e2 = np.zeros(16, dtype=np.float64)
    e4 = np.zeros(256, dtype=np.float64)
    lib.oracle_tables(_dp(e2), _dp(e4))
    return e2, e4


def decode_activation_bits(bits: np.ndarray, act: str) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.zeros(bits.shape, dtype=np.float64)
    fn = _load().oracle_decode_f16 if act == "f16" else _load().oracle_decode_bf16
    fn(bits.ctypes.data, bits.size, _dp(out))
    return out


def dequant_columns(prob, n0: int = 0, count: Optional[int] = None) -> np.ndarray:
    """dequant(W)[n0:n0+count, :] in float64."""
    count = prob.N - n0 if count is None else count
    b = _Bound(prob)
    out = np.zeros((count, prob.K), dtype=np.float64)
    _check(_load().oracle_dequant_columns(ctypes.byref(b.s), n0, count, _dp(out)), "dequant")
    return out


def gemv(prob, A: Optional[np.ndarray] = None, M: Optional[int] = None,
         nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Full product: returns (Y [M, N], S [M, N]) in float64."""
    A = prob.A if A is None else A
    M = A.shape[0] if M is None else M
    A = np.ascontiguousarray(A[:M], dtype=np.uint16)
    b = _Bound(prob)
    Y = np.zeros((M, prob.N), dtype=np.float64)
    S = np.zeros((M, prob.N), dtype=np.float64)
    _check(_load().oracle_gemv(ctypes.byref(b.s), A.ctypes.data, M, _dp(Y), _dp(S), nthreads), "gemv")
    return Y, S


def gemv_points(prob, ms: Sequence[int], ns: Sequence[int], A: Optional[np.ndarray] = None,
                M: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Selected outputs (ms[i], ns[i]) only: returns (y [P], S [P]) in float64."""
    A = prob.A if A is None else A
    M = A.shape[0] if M is None else M
    A = np.ascontiguousarray(A[:M], dtype=np.uint16)
    ms = np.ascontiguousarray(ms, dtype=np.int32)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    y = np.zeros(ms.size, dtype=np.float64)
    s = np.zeros(ms.size, dtype=np.float64)
    b = _Bound(prob)
    _check(_load().oracle_gemv_points(ctypes.byref(b.s), A.ctypes.data, M, ms.size, ms.ctypes.data,
                                      ns.ctypes.data, _dp(y), _dp(s)), "gemv_points")
    return y, s


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def tolerance(S: np.ndarray) -> np.ndarray:
    """Per-output acceptance bound for a result accumulated in fp32."""
    return TOL_REL * np.asarray(S, dtype=np.float64) + TOL_ABS


# The output type's unit roundoff, relative, allowed on top of the bound for synthetic
# edge cases whose |y| approaches S. Only bf16 needs it: rounding an fp32 result to
# bf16 (8 significant bits) moves it by up to 2^-8 |y|, more than the 1e-3 * S term
# when |y| is close to S. Rounding to fp16 (11 significant bits) moves it by at most
# 2^-11 |y| <= 2^-11 S, about half of 1e-3 * S, so fp16 outputs are held to the bound
# as it stands.
OUTPUT_HALF_ULP = {"f16": 0.0, "bf16": 2.0 ** -8}


def within_tolerance(y: np.ndarray, y_ref: np.ndarray, S: np.ndarray,
                     out_dtype: Optional[str] = None) -> Tuple[bool, float]:
    """(all outputs inside the bound, max(err / bound)).

    The bound is REL * S + ABS. With ``out_dtype`` "bf16", the output type's final
    rounding (2^-8 of |y_ref|) is allowed on top; fp16 outputs and calls
    without ``out_dtype`` (the named workloads) are held to the bound as it stands."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    bound = tolerance(S)
    if out_dtype is not None:
        bound = bound + OUTPUT_HALF_ULP[out_dtype] * np.abs(y_ref)
    ratio = err / bound
    ok = bool(np.all(np.isfinite(y)) and np.all(ratio <= 1.0))
    return ok, float(np.max(ratio)) if ratio.size else 0.0
