"""Pins for the rounding order of the two oracle definitions.

The other oracle pins (exact-integer regime, float64 error bound, closed
forms) pass under any summation order.  These examples do not: each is built
so that the sequence of binary32 roundings the pages define gives one BF16
value and every plausible other order or fold gives another.

Q2_0: page "gemv_q2_vec.rs", ``mod tests`` helper ``gemv_row`` (one fp32
accumulator, ascending k, a rounding per add).  W8A16: page
"w8a16_gemm_m16.rs", module doc (fp32 sum inside each 128-K block, the block
scale applied to that sum once, multiply then add).

Expected bits come from the hand derivations in ``golden/rounding_order.json``;
the checks here re-derive their arithmetic facts with exact rationals.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from weight_quantized_decode_block_amd import inputs as gen

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rounding_order.json")))
S_003 = float(np.float32(0.003))  # binary32 nearest to 0.003 (numpy's own rounding)


def _bf16_rne(x: float) -> int:
    """BF16 bits of a value exactly representable in binary32, through torch's RNE cast."""
    assert float(np.float32(x)) == x
    return int(torch.tensor([x], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF


def _e4m3(values) -> np.ndarray:
    return gen.e4m3fn_bits(np.asarray(values, dtype=np.float32))


def _ex(name):
    for group in ("q2_0", "w8a16"):
        for e in GOLDEN[group]:
            if e["name"] == name:
                return e
    raise KeyError(name)


# ------------------------------------------------------------------ Q2_0
def test_q2_0_ascending_k_absorbs_unit_terms(oracle_mod):
    ex = _ex("q2_ascending_k_absorbs_unit_terms")
    K = ex["K"]
    a = np.ones(K, np.float32)
    a[0] = a[K - 1] = 2.0 ** 24
    codes = np.full(K, 2, np.uint8)
    codes[K - 1] = 0
    A = gen.bf16_bits(a)[None, :]
    assert int(A[0, 0]) == 0x4B80 and int(A[0, 1]) == 0x3F80
    d = np.array([[int(x, 16) for x in ex["d_f16"]]], np.uint16)
    assert d.view(np.float16)[0].tolist() == [1.0, 1.0]

    # the example's arithmetic facts, with exact rationals
    w = [(int(c) - 1) for c in codes]
    exact = sum(Fraction(float(x)) * wk for x, wk in zip(a, w))
    assert exact == ex["exact_value"] == 254
    # 2^24 + 1 lies halfway between the two binary32 neighbours 2^24 and 2^24 + 2
    assert float(np.float32(2.0 ** 24 + 1)) == 2.0 ** 24
    for alt in ex["alternatives"].values():
        assert _bf16_rne(float(alt["value"])) == int(alt["bf16"], 16)
        assert int(alt["bf16"], 16) != int(ex["expected_bf16"], 16)

    out = oracle_mod.q2_0_gemv(A, codes[None, :], d)
    assert int(out[0, 0]) == int(ex["expected_bf16"], 16) == 0x0000


# ----------------------------------------------------------------- W8A16
def test_w8a16_inner_ascending_k_absorbs_unit_terms(oracle_mod):
    ex = _ex("w8_inner_ascending_k_absorbs_unit_terms")
    K = ex["K"]
    a = np.ones(K, np.float32)
    a[0], a[K - 1] = 2.0 ** 16, -(2.0 ** 16)
    wv = np.ones(K, np.float32)
    wv[0] = wv[K - 1] = 256.0
    A = gen.bf16_bits(a)[None, :]
    W = _e4m3(wv)[None, :]
    assert int(W[0, 0]) == 0x78 and int(W[0, 1]) == 0x38
    S = np.array([[1.0]], np.float32)
    exact = sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a, wv))
    assert exact == ex["exact_value"] == 126
    for alt in ex["alternatives"].values():
        assert _bf16_rne(float(alt["value"])) == int(alt["bf16"], 16)
        assert int(alt["bf16"], 16) != int(ex["expected_bf16"], 16)
    out = oracle_mod.w8a16_gemm(A, W, S)
    assert int(out[0, 0]) == int(ex["expected_bf16"], 16) == 0x0000


def test_w8a16_scale_once_per_block_not_per_element(oracle_mod):
    ex = _ex("w8_scale_once_per_block_not_per_element")
    K = ex["K"]
    a = np.zeros(K, np.float32)
    a[0], a[1], a[2] = 4096.0, 1.0, -4096.0
    wv = np.zeros(K, np.float32)
    wv[0], wv[1], wv[2] = 256.0, 1.0, 256.0
    A, W = gen.bf16_bits(a)[None, :], _e4m3(wv)[None, :]
    S = np.array([[S_003]], np.float32)
    s = Fraction(S_003)
    assert s == Fraction(12884902, 2 ** 32)
    assert int(np.array([S_003], np.float32).view(np.uint32)[0]) == 0x3B449BA6
    # expected: the block sum is exactly 1, so the output is bf16(s)
    assert _bf16_rne(S_003) == int(ex["expected_bf16"], 16) == 0x3B45
    # per element: s * 2^20 is a multiple of 2^-12; adding s (12.29 units of
    # 2^-12) rounds to 12 units; removing s * 2^20 leaves 12 * 2^-12
    big = s * 2 ** 20
    assert (big / Fraction(1, 2 ** 12)).denominator == 1 and 2048 <= big < 4096
    assert s / Fraction(1, 2 ** 12) > 12 and s / Fraction(1, 2 ** 12) < Fraction(25, 2)
    per_elem = Fraction(12, 2 ** 12)
    alt = ex["alternatives"]["scale_per_element"]
    assert _bf16_rne(float(per_elem)) == int(alt["bf16"], 16) != int(ex["expected_bf16"], 16)
    out = oracle_mod.w8a16_gemm(A, W, S)
    assert int(out[0, 0]) == 0x3B45


def test_w8a16_fold_multiply_then_add_unfused(oracle_mod):
    ex = _ex("w8_fold_multiply_then_add_unfused")
    K = ex["K"]
    a = np.zeros(K, np.float32)
    a[0], a[128] = -1.0, 1.0
    wv = np.zeros(K, np.float32)
    wv[0] = wv[128] = 1.125
    A, W = gen.bf16_bits(a)[None, :], _e4m3(wv)[None, :]
    assert int(W[0, 0]) == 0x39
    S = np.array([[S_003, S_003]], np.float32)
    prod = Fraction(S_003) * Fraction(9, 8)
    assert prod == Fraction(1449551475, 100) * Fraction(1, 2 ** 32)  # 14495514.75 * 2^-32
    q = Fraction(float(np.float32(float(prod))))  # binary32 rounding of the product
    assert q == Fraction(14495515, 2 ** 32)
    residual = prod - q  # what a fused multiply-add fold would leave
    assert residual == -Fraction(1, 2 ** 34)
    alt = ex["alternatives"]["fused_multiply_add_fold"]
    assert _bf16_rne(float(residual)) == int(alt["bf16"], 16) == 0xAE80
    out = oracle_mod.w8a16_gemm(A, W, S)
    assert int(out[0, 0]) == int(ex["expected_bf16"], 16) == 0x0000
