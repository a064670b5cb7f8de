"""CPU oracle for the small-T groupwise-int projection.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's
CPU-baseline leg are the only code that may import this package.  The product
path (the HIP library and its Python binding) never loads it.

The arithmetic lives in ``ngq_oracle.c`` (plain C, fp64, one scalar loop per
output); this module only loads the shared object and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ngq_oracle.c")
_LIB = os.path.join(_HERE, "libngq_oracle.so")

GROUP = 64
# offset-binary bias of each code width: u = c + BIAS[bits]
_BITS = (4, 5, 8)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE arithmetic: no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        i8p = ctypes.POINTER(ctypes.c_int8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        i32p = ctypes.POINTER(ctypes.c_int32)
        dp = ctypes.POINTER(ctypes.c_double)
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_round_bf16.argtypes = [ctypes.c_double]
        L.oracle_round_bf16.restype = ctypes.c_uint16
        L.oracle_packed_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.oracle_packed_bytes.restype = ctypes.c_size_t
        L.oracle_code_at.argtypes = [u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.oracle_code_at.restype = ctypes.c_int
        L.oracle_pack.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i8p, u8p]
        L.oracle_pack.restype = ctypes.c_int
        L.oracle_unpack.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, u8p, i8p]
        L.oracle_unpack.restype = ctypes.c_int
        L.oracle_dequant_f64.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, u8p, u16p, ctypes.c_int, dp]
        L.oracle_dequant_f64.restype = ctypes.c_int
        L.oracle_gemm_f64.argtypes = [ctypes.c_int] * 5 + [u16p, u8p, u16p, i32p, ctypes.c_int,
                                                           dp, dp, dp, ctypes.c_int]
        L.oracle_gemm_f64.restype = ctypes.c_int
        L.oracle_swiglu_f64.argtypes = [ctypes.c_int, dp, dp, dp]
        L.oracle_swiglu_f64.restype = ctypes.c_int
        L.oracle_round_bf16_array.argtypes = [ctypes.c_int, dp, u16p]
        L.oracle_round_bf16_array.restype = ctypes.c_int
        L.oracle_rms_rescale.argtypes = [ctypes.c_int, ctypes.c_int, u16p, u16p]
        L.oracle_rms_rescale.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class OracleError(ValueError):
    pass


def f16_to_f64(h: int) -> float:
    return lib().oracle_f16_to_f64(int(h) & 0xFFFF)


def bf16_to_f64(b: int) -> float:
    return lib().oracle_bf16_to_f64(int(b) & 0xFFFF)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Vectorised exact decode of bf16 bit patterns (uint16) to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(v: float) -> int:
    return int(lib().oracle_round_bf16(float(v)))


def round_bf16_array(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_round_bf16_array(v.size, _ptr(v, ctypes.c_double), _ptr(out, ctypes.c_uint16))
    return out


def packed_bytes(K: int, N: int, bits: int) -> int:
    return int(lib().oracle_packed_bytes(K, N, bits))


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    K, N = codes.shape
    out = np.zeros(max(packed_bytes(K, N, bits), 1), dtype=np.uint8)
    rc = lib().oracle_pack(K, N, bits, _ptr(codes, ctypes.c_int8), _ptr(out, ctypes.c_uint8))
    if rc != 0:
        raise OracleError(f"oracle_pack rejected K={K} N={N} bits={bits}")
    return out[: packed_bytes(K, N, bits)]


def unpack(packed: np.ndarray, K: int, N: int, bits: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    if packed.size < packed_bytes(K, N, bits):
        raise OracleError("packed buffer too small")
    out = np.zeros((K, N), dtype=np.int8)
    rc = lib().oracle_unpack(K, N, bits, _ptr(packed, ctypes.c_uint8), _ptr(out, ctypes.c_int8))
    if rc != 0:
        raise OracleError("oracle_unpack rejected arguments")
    return out


def code_at(packed: np.ndarray, K: int, N: int, bits: int, k: int, n: int) -> int:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    return int(lib().oracle_code_at(_ptr(packed, ctypes.c_uint8), K, N, bits, k, n))


def dequant(packed: np.ndarray, scales: np.ndarray, K: int, N: int, bits: int, scale_bf16: bool) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    w = np.zeros((K, N), dtype=np.float64)
    rc = lib().oracle_dequant_f64(K, N, bits, _ptr(packed, ctypes.c_uint8), _ptr(scales, ctypes.c_uint16),
                                  int(bool(scale_bf16)), _ptr(w, ctypes.c_double))
    if rc != 0:
        raise OracleError("oracle_dequant_f64 rejected arguments")
    return w


def gemm(x_bits: np.ndarray, packed: np.ndarray, scales: np.ndarray, K: int, N: int, bits: int,
         scale_bf16: bool, cols=None, nthreads: int = 1, with_bounds: bool = False):
    """Exact projection in fp64.  Returns y64 [T][len(cols)] (and, with
    ``with_bounds``, the magnitudes sum|x w| and sum|x| s of each output)."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T = x_bits.shape[0] if x_bits.ndim == 2 else 0
    if x_bits.ndim == 2 and x_bits.shape[1] != K:
        raise OracleError("x must be [T][K]")
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    if cols is None:
        cols_arr = None
        ncols = N
    else:
        cols_arr = np.ascontiguousarray(cols, dtype=np.int32)
        ncols = cols_arr.size
    y = np.zeros((T, ncols), dtype=np.float64)
    axw = np.zeros((T, ncols), dtype=np.float64)
    axs = np.zeros((T, ncols), dtype=np.float64)
    rc = lib().oracle_gemm_f64(
        T, K, N, bits, int(bool(scale_bf16)),
        _ptr(x_bits, ctypes.c_uint16) if x_bits.size else None,
        _ptr(packed, ctypes.c_uint8) if packed.size else None,
        _ptr(scales, ctypes.c_uint16) if scales.size else None,
        _ptr(cols_arr, ctypes.c_int32) if cols_arr is not None else None, ncols,
        _ptr(y, ctypes.c_double), _ptr(axw, ctypes.c_double), _ptr(axs, ctypes.c_double), int(nthreads))
    if rc != 0:
        raise OracleError("oracle_gemm_f64 rejected arguments")
    if with_bounds:
        return y, axw, axs
    return y


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    if g.shape != u.shape:
        raise OracleError("gate and up shapes differ")
    h = np.zeros(g.shape, dtype=np.float64)
    lib().oracle_swiglu_f64(g.size, _ptr(g, ctypes.c_double), _ptr(u, ctypes.c_double), _ptr(h, ctypes.c_double))
    return h


def add_residual(y64: np.ndarray, r_bits: np.ndarray, axw: np.ndarray | None = None):
    """The residual connection closing a stacked layer (harness, not a step the
    pages describe): y + r in fp64, with r given as bf16 bit patterns and
    decoded exactly, so the sum is the exact value the closing epilogue rounds
    once.  With ``axw`` (the projection's sum |x w|) also returns the
    magnitude |x w| summed with |r|, which bounds the rounding error of an
    fp32 evaluation of the same sum."""
    y64 = np.asarray(y64, dtype=np.float64)
    r = bf16_bits_to_f64(r_bits)
    if r.shape != y64.shape:
        raise OracleError("the residual must have the projection's shape")
    if axw is None:
        return y64 + r
    return y64 + r, np.asarray(axw, dtype=np.float64) + np.abs(r)


def rms_rescale(z_bits: np.ndarray) -> np.ndarray:
    z = np.ascontiguousarray(z_bits, dtype=np.uint16)
    T, N = z.shape
    out = np.zeros_like(z)
    lib().oracle_rms_rescale(T, N, _ptr(z, ctypes.c_uint16), _ptr(out, ctypes.c_uint16))
    return out
