"""Shared helpers for the GPU parity tests: device marshalling through the C
ABI and the acceptance rule.

Acceptance (the tolerance the design fixes for both formats, since the pages
name their constants without printing them): an output passes if its BF16
value is within 2 ulp of the oracle's (ulp distance on the ordered bf16
integers, -0 == +0) OR within 1e-2 x the RMS of the oracle's output row.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from weight_quantized_decode_block_amd import inputs as gen
from weight_quantized_decode_block_amd import wqd

CANARY = 0x7FBF  # a NaN pattern no kernel writes

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def ordered(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_parity(gpu: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    gpu = np.asarray(gpu, np.uint16)
    ref = np.asarray(ref, np.uint16)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    dist = np.abs(ordered(gpu) - ordered(ref))
    g = gen.bf16_values(gpu).astype(np.float64)
    r = gen.bf16_values(ref).astype(np.float64)
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    ok = (dist <= 2) | (np.abs(g - r) <= 1e-2 * rms)
    if not ok.all():
        idx = np.argwhere(~ok)
        m, n = idx[0] if idx.shape[1] == 2 else (0, idx[0][0])
        raise AssertionError(f"{what}: {len(idx)} of {ok.size} outputs outside tolerance; first at {tuple(idx[0])}: "
                             f"gpu={g[tuple(idx[0])]!r} oracle={r[tuple(idx[0])]!r} max ulp={dist.max()}")


def ulp_histogram(gpu: np.ndarray, ref: np.ndarray) -> dict:
    dist = np.abs(ordered(gpu) - ordered(ref))
    return {int(k): int(v) for k, v in zip(*np.unique(np.minimum(dist, 9), return_counts=True))}


# ---------------------------------------------------------- device helpers
def dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to("cuda")


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to("cuda")


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda")


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def q2_0_gpu(A_bits: np.ndarray, packed, N: int, K: int, extra_rows: int = 0, single: bool = False) -> np.ndarray:
    """Run q2_0_gemv_batchm (or q2_0_gemv when single) and return C bits.
    `packed` may be a numpy array or a device tensor; C gets `extra_rows`
    canary rows after the M computed ones (returned too)."""
    A_bits = np.atleast_2d(A_bits)
    M = A_bits.shape[0]
    A = dev_u16(A_bits)
    B = packed if isinstance(packed, torch.Tensor) else dev_u8(packed)
    C = torch.full((M + extra_rows, N), CANARY, dtype=torch.int16, device="cuda")
    if single:
        assert M == 1
        wqd.q2_0_gemv(A, B, C, N, K)
    else:
        wqd.q2_0_gemv_batchm(A, B, C, N, K, 128, M)
    torch.cuda.synchronize()
    return host_u16(C)


def w8a16_gpu(A_bits: np.ndarray, W, S, N: int, K: int, c_rows: int | None = None) -> np.ndarray:
    A_bits = np.atleast_2d(A_bits)
    M = A_bits.shape[0]
    A = dev_u16(A_bits)
    Wd = W if isinstance(W, torch.Tensor) else dev_u8(W)
    Sd = S if isinstance(S, torch.Tensor) else dev_f32(S)
    C = torch.full((c_rows or M, N), CANARY, dtype=torch.int16, device="cuda")
    wqd.w8a16_gemm_m16(A, Wd, Sd, C, M, N, K)
    torch.cuda.synchronize()
    return host_u16(C)
