"""CPU oracle for the weight-only-quantized decode GEMV (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it and
has no fallback to it.  The arithmetic lives in ``oracle.c`` (plain C, built
with gcc ``-O2 -ffp-contract=off``); this module only builds it and marshals
numpy arrays through ctypes.

Pages followed (cited by title and section):
  * "gemv_q2_vec.rs", module doc and ``mod tests`` helper ``gemv_row``:
    the Q2_0 per-row reference (fp32, ascending k, BF16 store).
  * "w8a16_gemm_m16.rs", module doc: FP8 E4M3 weights with FP32 128x128 block
    scales; each 128-K block's fp32 sum is scaled once and added to an fp32
    total per output.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (host only)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-pthread", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    f32p = ctypes.POINTER(ctypes.c_float)
    u32 = ctypes.c_uint32
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32.restype = ctypes.c_float
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_e4m3fn_to_f32.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3fn_to_f32.restype = ctypes.c_float
    lib.oracle_q2_0_unpack.argtypes = [u8p, u32, u32, u8p, u16p]
    lib.oracle_q2_0_unpack.restype = ctypes.c_int
    lib.oracle_q2_0_gemv.argtypes = [u16p, u8p, u16p, u16p, u32, u32, u32, ctypes.c_int]
    lib.oracle_q2_0_gemv.restype = ctypes.c_int
    lib.oracle_w8a16_gemm.argtypes = [u16p, u8p, f32p, u16p, u32, u32, u32, ctypes.c_int]
    lib.oracle_w8a16_gemm.restype = ctypes.c_int
    lib.oracle_default_threads.argtypes = []
    lib.oracle_default_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def default_threads() -> int:
    return int(_load().oracle_default_threads())


# ------------------------------------------------------------------ codecs
def f16_to_f32(bits: int) -> float:
    return float(_load().oracle_f16_to_f32(int(bits)))


def bf16_to_f32(bits: int) -> float:
    return float(_load().oracle_bf16_to_f32(int(bits)))


def f32_to_bf16(x: float) -> int:
    return int(_load().oracle_f32_to_bf16(float(x)))


def e4m3fn_to_f32(code: int) -> float:
    return float(_load().oracle_e4m3fn_to_f32(int(code)))


# ----------------------------------------------------------- Q2_0 unpacker
def q2_0_unpack(packed: np.ndarray, N: int, K: int):
    """Byte-wise unpack of ``[N][K/128]`` 34-byte blocks -> (codes u8 [N,K], d fp16 bits [N,K/128])."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    assert packed.size == N * (K // 128) * 34
    codes = np.empty((N, K), np.uint8)
    d = np.empty((N, K // 128), np.uint16)
    rc = _load().oracle_q2_0_unpack(_ptr(packed, ctypes.c_uint8), N, K,
                                    _ptr(codes, ctypes.c_uint8), _ptr(d, ctypes.c_uint16))
    if rc != 0:
        raise ValueError(f"oracle_q2_0_unpack: K={K} not a multiple of 128")
    return codes, d


# ------------------------------------------------------------ the GEMVs
def q2_0_gemv(A_bf16: np.ndarray, codes: np.ndarray, d_f16: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """Oracle Q2_0: A bf16 bits [M,K], codes u8 [N,K], d fp16 bits [N,K/128] -> C bf16 bits [M,N]."""
    A = np.ascontiguousarray(A_bf16, dtype=np.uint16)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    d = np.ascontiguousarray(d_f16, dtype=np.uint16)
    if A.ndim == 1:
        A = A[None, :]
    M, K = A.shape
    N = codes.shape[0]
    assert codes.shape == (N, K) and d.shape == (N, K // 128)
    C = np.zeros((M, N), np.uint16)
    rc = _load().oracle_q2_0_gemv(_ptr(A, ctypes.c_uint16), _ptr(codes, ctypes.c_uint8),
                                  _ptr(d, ctypes.c_uint16), _ptr(C, ctypes.c_uint16),
                                  M, N, K, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_q2_0_gemv failed rc={rc} (K={K})")
    return C


def w8a16_gemm(A_bf16: np.ndarray, W_e4m3: np.ndarray, S: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """Oracle W8A16: A bf16 bits [M,K], W E4M3FN bytes [N,K], S fp32 [ceil(N/128),K/128] -> C bf16 bits [M,N]."""
    A = np.ascontiguousarray(A_bf16, dtype=np.uint16)
    W = np.ascontiguousarray(W_e4m3, dtype=np.uint8)
    S = np.ascontiguousarray(S, dtype=np.float32)
    if A.ndim == 1:
        A = A[None, :]
    M, K = A.shape
    N = W.shape[0]
    assert W.shape == (N, K) and S.shape == ((N + 127) // 128, K // 128)
    C = np.zeros((M, N), np.uint16)
    rc = _load().oracle_w8a16_gemm(_ptr(A, ctypes.c_uint16), _ptr(W, ctypes.c_uint8),
                                   _ptr(S, ctypes.c_float), _ptr(C, ctypes.c_uint16),
                                   M, N, K, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_w8a16_gemm failed rc={rc} (K={K})")
    return C
