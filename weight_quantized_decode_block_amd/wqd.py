"""Python binding of libwqd.so: argument marshalling only.

Every function here forwards to the C ABI declared in ``include/wqd.h`` with
the same name.  Device arguments may be torch tensors (their ``data_ptr()`` is
passed) or raw integer device addresses; ``stream`` defaults to torch's current
stream on the current device.  A non-zero status raises :class:`WqdError` with
the library's message.  The library must be built first
(``python -m weight_quantized_decode_block_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwqd.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "wqd.h")

WQD_OK, WQD_EINVAL, WQD_ENULL, WQD_EALIGN, WQD_EUNSUPPORTED, WQD_ENODEV, WQD_EHIP = range(7)
Q2_0_GROUP = 128
Q2_0_BLOCK_BYTES = 34
Q2_0_BATCHM_MAX_M = 8
W8A16_MAX_M = 16
Q2_0_TIER_WIDTHS = (1, 2, 4, 6, 8)  # WQD_Q2_0_TIER_WIDTHS, narrowest first

_lib = None


class WqdError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libwqd.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m weight_quantized_decode_block_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, u32, sz = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_size_t
    L.q2_0_gemv.argtypes = [vp, vp, vp, u32, u32, u32, vp]
    L.q2_0_gemv_batchm.argtypes = [vp, vp, vp, u32, u32, u32, u32, vp]
    L.w8a16_gemm_m16.argtypes = [vp, vp, vp, vp, u32, u32, u32, vp]
    L.w8a16_gemm_m16_n64.argtypes = [vp, vp, vp, vp, u32, u32, u32, vp]
    L.w8a16_gemm_m16_strided.argtypes = [vp, vp, vp, vp, u32, u32, u32, u32, u32, vp]
    L.w8a16_gemv_batch16.argtypes = [vp, vp, vp, vp, u32, u32, u32, vp]
    L.w8a16_gemv_batch16_strided.argtypes = [vp, vp, vp, vp, u32, u32, u32, u32, u32, vp]
    for f in (L.q2_0_gemv, L.q2_0_gemv_batchm, L.w8a16_gemm_m16, L.w8a16_gemm_m16_n64,
              L.w8a16_gemm_m16_strided, L.w8a16_gemv_batch16, L.w8a16_gemv_batch16_strided):
        f.restype = ctypes.c_int
    L.q2_0_packed_bytes.argtypes = [u32, u32]
    L.q2_0_packed_bytes.restype = sz
    L.q2_0_pack.argtypes = [vp, vp, u32, u32, vp]
    L.q2_0_pack.restype = ctypes.c_int
    L.q2_0_batchm_chunks.argtypes = [u32, u32, u32, ctypes.POINTER(ctypes.c_uint64), u32]
    L.q2_0_batchm_chunks.restype = u32
    L.q2_0_select_tier.argtypes = [u32, u32, ctypes.c_int]
    L.q2_0_select_tier.restype = ctypes.c_int
    L.q2_0_tier_width.argtypes = [u32]
    L.q2_0_tier_width.restype = u32
    L.q2_0_exact_m_tiers_enabled.argtypes = []
    L.q2_0_exact_m_tiers_enabled.restype = ctypes.c_int
    L.wqd_last_error.argtypes = []
    L.wqd_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions include/wqd.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z][a-z0-9_]*)\s*\(", text, flags=re.M)


def last_error() -> str:
    return lib().wqd_last_error().decode()


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


_current_raw_stream = None


def _stream(stream) -> int | None:
    global _current_raw_stream
    if stream is None:
        if _current_raw_stream is None:
            import torch
            raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
            if raw is not None:
                _current_raw_stream = lambda: raw(torch.cuda.current_device())
            else:
                _current_raw_stream = lambda: int(torch.cuda.current_stream().cuda_stream)
        return _current_raw_stream()
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check(fn: str, rc: int) -> None:
    if rc != WQD_OK:
        raise WqdError(fn, rc, last_error())


# -------------------------------------------------------------- GPU calls
def q2_0_gemv(A, B, C, N: int, K: int, group: int = Q2_0_GROUP, stream=None) -> None:
    _check("q2_0_gemv", lib().q2_0_gemv(_ptr(A), _ptr(B), _ptr(C), N, K, group, _stream(stream)))


def q2_0_gemv_batchm(A, B, C, N: int, K: int, group: int = Q2_0_GROUP, M: int = 1, stream=None) -> None:
    _check("q2_0_gemv_batchm",
           lib().q2_0_gemv_batchm(_ptr(A), _ptr(B), _ptr(C), N, K, group, M, _stream(stream)))


def w8a16_gemm_m16(A, W, S, C, M: int, N: int, K: int, stream=None) -> None:
    _check("w8a16_gemm_m16",
           lib().w8a16_gemm_m16(_ptr(A), _ptr(W), _ptr(S), _ptr(C), M, N, K, _stream(stream)))


def w8a16_gemm_m16_n64(A, W, S, C, M: int, N: int, K: int, stream=None) -> None:
    _check("w8a16_gemm_m16_n64",
           lib().w8a16_gemm_m16_n64(_ptr(A), _ptr(W), _ptr(S), _ptr(C), M, N, K, _stream(stream)))


def w8a16_gemm_m16_strided(A, W, S, C, M: int, N: int, K: int, a_row_stride: int, c_row_stride: int,
                           stream=None) -> None:
    _check("w8a16_gemm_m16_strided",
           lib().w8a16_gemm_m16_strided(_ptr(A), _ptr(W), _ptr(S), _ptr(C), M, N, K, a_row_stride,
                                        c_row_stride, _stream(stream)))


def w8a16_gemv_batch16(A, W, S, C, M: int, N: int, K: int, stream=None) -> None:
    _check("w8a16_gemv_batch16",
           lib().w8a16_gemv_batch16(_ptr(A), _ptr(W), _ptr(S), _ptr(C), M, N, K, _stream(stream)))


def w8a16_gemv_batch16_strided(A, W, S, C, M: int, N: int, K: int, a_row_stride: int, c_row_stride: int,
                               stream=None) -> None:
    _check("w8a16_gemv_batch16_strided",
           lib().w8a16_gemv_batch16_strided(_ptr(A), _ptr(W), _ptr(S), _ptr(C), M, N, K, a_row_stride,
                                            c_row_stride, _stream(stream)))


# ------------------------------------------------------------ host helpers
def q2_0_packed_bytes(N: int, K: int) -> int:
    return int(lib().q2_0_packed_bytes(N, K))


def q2_0_pack(codes: np.ndarray, d_f16: np.ndarray) -> np.ndarray:
    """Pack codes u8 [N,K] and fp16 scale bits [N,K/128] into block_q2_0 bytes."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    d = np.ascontiguousarray(d_f16, dtype=np.uint16)
    N, K = codes.shape
    if d.shape != (N, K // 128):
        raise ValueError(f"d_f16 shape {d.shape} != {(N, K // 128)}")
    out = np.empty(max(q2_0_packed_bytes(N, K), 1), np.uint8)
    rc = lib().q2_0_pack(codes.ctypes.data, d.ctypes.data, N, K, out.ctypes.data)
    if rc != WQD_OK:
        raise WqdError("q2_0_pack", rc, "codes must be 0..2 and K a positive multiple of 128")
    return out[:q2_0_packed_bytes(N, K)]


def q2_0_batchm_chunks(M: int, K: int, N: int) -> list[tuple[int, int, int]]:
    L = lib()
    count = int(L.q2_0_batchm_chunks(M, K, N, None, 0))
    buf = (ctypes.c_uint64 * max(3 * count, 1))()
    L.q2_0_batchm_chunks(M, K, N, buf, count)
    return [(int(buf[3 * i]), int(buf[3 * i + 1]), int(buf[3 * i + 2])) for i in range(count)]


def q2_0_select_tier(m: int, present_mask: int, exact_m: bool) -> int | None:
    """Index into Q2_0_TIER_WIDTHS of the tier that serves m rows, or None."""
    i = int(lib().q2_0_select_tier(m, present_mask, 1 if exact_m else 0))
    return None if i < 0 else i


def q2_0_tier_width(m: int) -> int:
    """Row width the Q2_0 matrix-core kernel runs m rows on in this process (0: none)."""
    return int(lib().q2_0_tier_width(m))


def q2_0_exact_m_tiers_enabled() -> bool:
    return bool(lib().q2_0_exact_m_tiers_enabled())
