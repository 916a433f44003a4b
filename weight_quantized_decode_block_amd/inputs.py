"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method itself: it only draws random
numbers and rounds them to the storage formats the operations take (BF16
activations, fp16 Q2_0 scales, FP8 E4M3FN weights, fp32 block scales), using
numpy's and torch's own conversions.  Packing into ``block_q2_0`` is not done
here; that is the product's host packer.

Every generator is a numpy ``Generator(PCG64([workload_id, tensor_id]))`` so
that a (workload, tensor) pair always yields the same bytes on any machine.

Workload ids (the five synthetic workloads the design notes list):
  1  Q2_0 GEMV M=1, N=256, K=1024
  2  Q2_0 GEMV M=1, N=K=5120
  3  Q2_0 batched GEMV M in {2,4,5,8,16}, N=K=5120
  4  W8A16 M in {1,8,16}, N=K=5120
  5  FFN sweep (N=17408,K=5120 and N=5120,K=17408), both formats
"""
from __future__ import annotations

import numpy as np
import torch

T_A, T_CODES, T_D, T_W, T_S = 1, 2, 3, 4, 5
A_ROWS = 32  # activations are drawn as [32, K]; a call with M rows uses the first M


def rng(workload_id: int, tensor_id: int, salt: int = 0) -> np.random.Generator:
    key = [int(workload_id), int(tensor_id)] + ([int(salt)] if salt else [])
    return np.random.Generator(np.random.PCG64(key))


# ------------------------------------------------------------- conversions
def bf16_bits(x) -> np.ndarray:
    """float -> bfloat16 bit patterns (round to nearest even, torch's cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f16_bits(x) -> np.ndarray:
    """float -> IEEE binary16 bit patterns (numpy's round to nearest even)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16).copy()


def e4m3fn_bits(x) -> np.ndarray:
    """float (already within +-448) -> OCP E4M3FN bytes (torch's cast, RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


# ------------------------------------------------------------- Q2_0 inputs
def activations(workload_id: int, K: int, M: int, salt: int = 0) -> np.ndarray:
    """BF16 bits [M, K] drawn from N(0,1); the first M of (at least) 32 rows."""
    rows = max(A_ROWS, M)
    a = rng(workload_id, T_A, salt).standard_normal((rows, K), dtype=np.float32)
    return bf16_bits(a[:M])


def q2_0_weights(workload_id: int, N: int, K: int, salt: int = 0):
    """Ternary codes u8 [N, K] iid uniform on {0,1,2} and fp16 scale bits
    [N, K/128] with d = |N(0, 0.02)| + 1e-3."""
    codes = rng(workload_id, T_CODES, salt).integers(0, 3, size=(N, K), dtype=np.uint8)
    d = np.abs(rng(workload_id, T_D, salt).normal(0.0, 0.02, size=(N, K // 128))) + 1e-3
    return codes, f16_bits(d)


def w8a16_weights(workload_id: int, N: int, K: int, salt: int = 0):
    """E4M3FN bytes [N, K] from N(0,1) clipped to +-448, and fp32 block scales
    [ceil(N/128), K/128] drawn from U(0.001, 0.01)."""
    w = np.clip(rng(workload_id, T_W, salt).standard_normal((N, K), dtype=np.float32), -448.0, 448.0)
    s = rng(workload_id, T_S, salt).uniform(0.001, 0.01, size=((N + 127) // 128, K // 128))
    return e4m3fn_bits(w), s.astype(np.float32)


# ----------------------------------------------- exact-integer regime inputs
def exact_activations(seed: int, M: int, K: int) -> np.ndarray:
    """Integers in [-8, 8] as BF16 bits."""
    a = rng(900, T_A, seed).integers(-8, 9, size=(M, K)).astype(np.float32)
    return bf16_bits(a)


def exact_q2_0_scales(seed: int, N: int, K: int) -> np.ndarray:
    """Scales 2^-j, j in 0..6, as fp16 bits [N, K/128]."""
    j = rng(900, T_D, seed).integers(0, 7, size=(N, K // 128))
    return f16_bits(np.ldexp(1.0, -j))


def exact_w8a16_weights(seed: int, N: int, K: int):
    """FP8 integers in [-16, 16] (all exact in E4M3FN) and scales 2^-j."""
    q = rng(900, T_W, seed).integers(-16, 17, size=(N, K)).astype(np.float32)
    j = rng(900, T_S, seed).integers(0, 7, size=((N + 127) // 128, K // 128))
    return e4m3fn_bits(q), np.ldexp(1.0, -j).astype(np.float32)


# ------------------------------------- the pages' deterministic test vectors
def pages_test_vectors(m: int, n: int, k: int):
    """The deterministic vectors of the Q2_0 page's unit tests (``gen_inputs``):
    activations sin(0.09131 i) * 1.3, codes ((i * 2654435761) >> 6) % 3 and
    scales 0.015 + 0.01 (i % 5).  The activations are rounded to BF16 and the
    scales to fp16, the storage formats the operation takes."""
    i = np.arange(m * k, dtype=np.float32)
    act = (np.sin(i * np.float32(0.09131)) * np.float32(1.3)).astype(np.float32)
    ic = np.arange(n * k, dtype=np.uint64)
    codes = (((ic * np.uint64(2654435761)) >> np.uint64(6)) % np.uint64(3)).astype(np.uint8)
    isc = np.arange(n * (k // 128))
    scales = (0.015 + 0.01 * (isc % 5)).astype(np.float32)
    return (bf16_bits(act.reshape(m, k)), codes.reshape(n, k),
            f16_bits(scales.reshape(n, k // 128)))
