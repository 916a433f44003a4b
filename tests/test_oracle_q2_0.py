"""Pins for the Q2_0 oracle against things other than itself.

Definition followed: page "gemv_q2_vec.rs", module doc (w = (code-1)*d, inline
fp16 d per 128-code block) and ``mod tests`` helper ``gemv_row`` (fp32 sum in
ascending k, BF16 store, round to nearest even).

Pins: closed forms and worked examples re-derived with exact rationals, the
exact-integer regime against an exact float64 matmul, an error bound against
float64 on random data, the byte-wise unpacker against the golden block, and
invariants (rows independent, thread count irrelevant).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from weight_quantized_decode_block_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q2_0_closed_forms.json")


def _bf16_of_exact(x: np.ndarray) -> np.ndarray:
    """Round float64 values that are exactly representable in float32 to bf16 (torch RNE)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64))
    return gen.bf16_bits(x32)


def _dequant_f64(codes, d_bits):
    d = d_bits.view(np.float16).astype(np.float64)
    N, K = codes.shape
    return (codes.astype(np.float64) - 1.0) * np.repeat(d, 128, axis=1).reshape(N, K)


def _frac_of_bf16(bits):
    return Fraction(float(gen.bf16_values(np.array([bits], np.uint16))[0]))


def _rne_bf16_of_fraction(x: Fraction) -> int:
    f = float(x)  # examples are chosen so that this conversion is exact
    assert Fraction(f) == x
    return int(_bf16_of_exact(np.array([f]))[0])


# --------------------------------------------------------------- golden
def _example_inputs(name):
    K = 128
    if name == "ex1_codes_mod3_unit_a":
        a = np.ones(K, np.float32)
        c = (np.arange(K) % 3).astype(np.uint8)
        d = [2.0 ** -6]
    elif name == "ex2_exact_regime":
        K = 256
        a = ((np.arange(K) % 7) - 3).astype(np.float32)
        c = (np.arange(K) % 3).astype(np.uint8)
        d = [0.5, 0.25]
    elif name == "ex3_rne_tie_at_store":
        a = np.zeros(K, np.float32)
        a[0], a[1] = 256.0, 3.0
        c = np.ones(K, np.uint8)
        c[0] = c[1] = 2
        d = [2.0 ** -8]
    elif name == "ex4_single_nonzero_code":
        a = np.full(K, -1.7, np.float32)
        c = np.ones(K, np.uint8)
        c[77] = 0
        d = [0.0137]
    elif name == "ex5_all_codes_one":
        a = np.random.Generator(np.random.PCG64(5)).standard_normal(K).astype(np.float32)
        c = np.ones(K, np.uint8)
        d = [0.02]
    else:
        raise KeyError(name)
    return K, gen.bf16_bits(a)[None, :], c[None, :], gen.f16_bits(np.array(d))[None, :]


@pytest.mark.parametrize("ex", json.load(open(GOLDEN))["examples"], ids=lambda e: e["name"])
def test_worked_examples(oracle_mod, ex):
    K, A, codes, d = _example_inputs(ex["name"])
    # exact rational value of the definition, then RNE to bf16
    exact = Fraction(0)
    for k in range(K):
        dv = Fraction(float(d.view(np.float16)[0, k // 128]))
        exact += _frac_of_bf16(A[0, k]) * (int(codes[0, k]) - 1) * dv
    expected = int(ex["expected_bf16"], 16)
    if ex["name"] != "ex3_rne_tie_at_store":  # ex3's exact value is the tie itself
        assert _rne_bf16_of_fraction(exact) == expected
    else:
        assert exact == Fraction(1) + Fraction(3, 256)
        assert expected == 0x3F82  # ties to even; truncation would give 0x3F81
    out = oracle_mod.q2_0_gemv(A, codes, d)
    assert int(out[0, 0]) == expected


def test_unpacker_reads_golden_block(oracle_mod):
    g = json.load(open(GOLDEN))["pack_golden"]
    packed = np.frombuffer(bytes.fromhex(g["bytes_hex"]), dtype=np.uint8)
    codes, d = oracle_mod.q2_0_unpack(packed, 1, 128)
    assert int(d[0, 0]) == int(g["d_f16"], 16)
    assert np.array_equal(codes[0], (np.arange(128) % 3).astype(np.uint8))


# ----------------------------------------------------------- closed forms
@pytest.mark.parametrize("code", [0, 2, 3])
def test_single_nonzero_code_closed_form(oracle_mod, code):
    """One code != 1 at position k: out = bf16(a_k * (code-1) * d) exactly
    (code 3 decodes to +2d, per (code & 3) - 1)."""
    r = np.random.Generator(np.random.PCG64(100 + code))
    K, N = 512, 6
    A = gen.bf16_bits(r.standard_normal((2, K)).astype(np.float32))
    codes = np.ones((N, K), np.uint8)
    d = gen.f16_bits(np.abs(r.normal(0, 0.02, (N, K // 128))) + 1e-3)
    ks = r.integers(0, K, N)
    for n in range(N):
        codes[n, ks[n]] = code
    out = oracle_mod.q2_0_gemv(A, codes, d)
    av = gen.bf16_values(A).astype(np.float64)
    dv = d.view(np.float16).astype(np.float64)
    for m in range(2):
        for n in range(N):
            k = ks[n]
            exp = av[m, k] * (code - 1) * dv[n, k // 128]  # exact in float64 and float32
            assert int(out[m, n]) == int(_bf16_of_exact(np.array([exp]))[0])


def test_all_codes_one_gives_positive_zero(oracle_mod):
    r = np.random.Generator(np.random.PCG64(11))
    A = gen.bf16_bits(r.standard_normal((3, 256)).astype(np.float32))
    codes = np.ones((9, 256), np.uint8)
    d = gen.f16_bits(np.full((9, 2), 0.02))
    out = oracle_mod.q2_0_gemv(A, codes, d)
    assert np.all(out == 0)


# ------------------------------------------------------ exact-integer regime
@pytest.mark.parametrize("M,N,K", [(1, 7, 128), (3, 37, 640), (5, 16, 1024)])
def test_exact_integer_regime_equals_exact_matmul(oracle_mod, M, N, K):
    """a in [-8, 8], d = 2^-j: every product and partial sum is exact in fp32,
    so the oracle must equal the exact float64 matmul rounded once to bf16."""
    A = gen.exact_activations(M * 1000 + N, M, K)
    codes = gen.rng(901, 2, N).integers(0, 4, size=(N, K), dtype=np.uint8)  # includes code 3
    d = gen.exact_q2_0_scales(N + K, N, K)
    exact = gen.bf16_values(A).astype(np.float64) @ _dequant_f64(codes, d).T
    assert np.all(np.abs(exact) < 2 ** 24)
    out = oracle_mod.q2_0_gemv(A, codes, d)
    assert np.array_equal(out, _bf16_of_exact(exact))


# ------------------------------------------------------------ error bound
@pytest.mark.parametrize("M,N,K", [(2, 64, 1024), (1, 33, 5120)])
def test_within_fp32_sequential_bound_of_f64(oracle_mod, M, N, K):
    """|oracle - exact| <= gamma_K * sum|a w| + half a bf16 ulp, and the oracle
    equals bf16(exact) for all but a handful of rounding-boundary cases."""
    A = gen.activations(1, K, M)
    codes, d = gen.q2_0_weights(1, N, K)
    av = gen.bf16_values(A).astype(np.float64)
    W = _dequant_f64(codes, d)
    exact = av @ W.T
    absum = np.abs(av) @ np.abs(W).T
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    out = oracle_mod.q2_0_gemv(A, codes, d)
    o = gen.bf16_values(out).astype(np.float64)
    half_ulp = np.abs(o) * 2.0 ** -8 + 2.0 ** -133
    assert np.all(np.abs(o - exact) <= gamma * absum + half_ulp)
    rounded = gen.bf16_values(gen.bf16_bits(exact.astype(np.float32))).astype(np.float64)
    assert np.mean(o == rounded) >= 0.98


def test_pages_test_vectors_within_bound(oracle_mod):
    """The deterministic vectors of the page's unit tests (n=5, k=256)."""
    A, codes, d = gen.pages_test_vectors(16, 5, 256)
    out = oracle_mod.q2_0_gemv(A, codes, d)
    exact = gen.bf16_values(A).astype(np.float64) @ _dequant_f64(codes, d).T
    o = gen.bf16_values(out).astype(np.float64)
    assert np.all(np.abs(o - exact) <= 256 * 2.0 ** -24 * 50 + np.abs(exact) * 2.0 ** -8)


# --------------------------------------------------------------- brute force
def _emulate_row(a_bits, codes_row, d_row):
    """Step-by-step float32 emulation of one output (tiny inputs only).

    This restates the oracle's own loop in numpy, so it checks the C side's
    plumbing (codecs, indexing, block of each k) on random inputs, not the
    summation order; the order is pinned by the hand-derived examples in
    test_oracle_order.py."""
    acc = np.float32(0.0)
    a = gen.bf16_values(a_bits)
    dv = d_row.view(np.float16).astype(np.float32)
    for k in range(a.size):
        w = np.float32(int(codes_row[k] & 3) - 1) * dv[k // 128]
        acc = np.float32(acc + np.float32(a[k] * w))
    return int(gen.bf16_bits(np.array([acc], np.float32))[0])


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (3, 4, 256), (2, 3, 128)])
def test_brute_force_float32_emulation(oracle_mod, M, N, K):
    r = np.random.Generator(np.random.PCG64(M * 100 + N * 10 + K))
    A = gen.bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    codes = r.integers(0, 3, (N, K), dtype=np.uint8)
    d = gen.f16_bits(np.abs(r.normal(0, 0.02, (N, K // 128))) + 1e-3)
    out = oracle_mod.q2_0_gemv(A, codes, d)
    for m in range(M):
        for n in range(N):
            assert int(out[m, n]) == _emulate_row(A[m], codes[n], d[n])


# --------------------------------------------------------------- invariants
def test_rows_independent_and_thread_count_invariant(oracle_mod):
    M, N, K = 9, 70, 1024
    A = gen.activations(3, K, M)
    codes, d = gen.q2_0_weights(3, N, K)
    ref = oracle_mod.q2_0_gemv(A, codes, d, nthreads=1)
    for t in (2, 3, 8, 0):
        assert np.array_equal(oracle_mod.q2_0_gemv(A, codes, d, nthreads=t), ref)
    for m in range(M):
        assert np.array_equal(oracle_mod.q2_0_gemv(A[m:m + 1], codes, d), ref[m:m + 1])


def test_rejects_k_not_multiple_of_128(oracle_mod):
    with pytest.raises(Exception):
        oracle_mod.q2_0_gemv(np.zeros((1, 100), np.uint16), np.zeros((2, 100), np.uint8),
                             np.zeros((2, 0), np.uint16))
