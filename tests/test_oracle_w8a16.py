"""Pins for the W8A16 oracle against things other than itself.

Definition followed: page "w8a16_gemm_m16.rs", module doc (FP8 E4M3 weights
[N,K], FP32 block scales [N/128, K/128] folded once per 128-K block onto an
fp32 outer accumulator, BF16 in and out).

Pins: the exact-integer regime against an exact float64 matmul of the
per-element-scaled weights (equal to the block fold in exact arithmetic), a
two-level summation error bound on random data, closed forms (single nonzero
weight, scale indexing with distinct powers of two), and invariants.
"""
import numpy as np
import pytest
import torch

from weight_quantized_decode_block_amd import inputs as gen


def _bf16_of_exact(x):
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64))
    return gen.bf16_bits(x32)


def _w_f64(W_bits):
    return torch.from_numpy(W_bits).view(torch.float8_e4m3fn).double().numpy()


def _scaled_weights_f64(W_bits, S):
    """W[n,k] * S[n//128, k//128] in float64 (an element-wise expansion of the
    block scales; equal to folding them per block in exact arithmetic)."""
    N, K = W_bits.shape
    s_full = np.repeat(np.repeat(S.astype(np.float64), 128, axis=0)[:N], 128, axis=1)
    return _w_f64(W_bits) * s_full


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (4, 200, 384), (16, 130, 1024)])
def test_exact_integer_regime(oracle_mod, M, N, K):
    A = gen.exact_activations(M + N, M, K)
    W, S = gen.exact_w8a16_weights(K + N, N, K)
    exact = gen.bf16_values(A).astype(np.float64) @ _scaled_weights_f64(W, S).T
    assert np.all(np.abs(exact) < 2 ** 24)
    out = oracle_mod.w8a16_gemm(A, W, S)
    assert np.array_equal(out, _bf16_of_exact(exact))


@pytest.mark.parametrize("M,N,K", [(3, 256, 1024), (1, 64, 5120)])
def test_within_two_level_sum_bound(oracle_mod, M, N, K):
    A = gen.activations(4, K, M)
    W, S = gen.w8a16_weights(4, N, K)
    av = gen.bf16_values(A).astype(np.float64)
    Ws = _scaled_weights_f64(W, S)
    exact = av @ Ws.T
    absum = np.abs(av) @ np.abs(Ws).T
    u = 2.0 ** -24
    nb = K // 128
    g = lambda n: n * u / (1 - n * u)
    bound = (g(128) + g(nb) + 2 * u) * 1.01 * absum
    out = oracle_mod.w8a16_gemm(A, W, S)
    o = gen.bf16_values(out).astype(np.float64)
    assert np.all(np.abs(o - exact) <= bound + np.abs(o) * 2.0 ** -8 + 2.0 ** -133)
    rounded = gen.bf16_values(gen.bf16_bits(exact.astype(np.float32))).astype(np.float64)
    assert np.mean(o == rounded) >= 0.98


def test_single_nonzero_weight(oracle_mod):
    r = np.random.Generator(np.random.PCG64(21))
    M, N, K = 2, 140, 512
    A = gen.bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    W = np.zeros((N, K), np.uint8)
    ks = r.integers(0, K, N)
    codes = r.integers(1, 0x7F, N).astype(np.uint8)  # finite nonzero positive codes
    W[np.arange(N), ks] = codes
    S = r.uniform(0.001, 0.01, ((N + 127) // 128, K // 128)).astype(np.float32)
    out = oracle_mod.w8a16_gemm(A, W, S)
    av = gen.bf16_values(A)
    wv = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    for m in range(M):
        for n in range(N):
            k = ks[n]
            inner = np.float32(av[m, k] * wv[n])          # exact product
            exp = np.float32(S[n // 128, k // 128] * inner)  # one rounding, then + 0
            assert int(out[m, n]) == int(gen.bf16_bits(np.array([exp]))[0])


def test_scale_indexing_distinct_powers_of_two(oracle_mod):
    """W = 1, a = 1, S[r][b] = 2^-(3r+b): out[n] = 128 * sum_b S[n//128][b].
    A transposed or mis-indexed scale tensor changes the value."""
    M, N, K = 1, 256, 384
    A = gen.bf16_bits(np.ones((M, K), np.float32))
    W = np.full((N, K), 0x38, np.uint8)  # 1.0
    S = np.array([[2.0 ** -(3 * r + b) for b in range(3)] for r in range(2)], np.float32)
    out = oracle_mod.w8a16_gemm(A, W, S)
    expected = np.array([128 * S[n // 128].astype(np.float64).sum() for n in range(N)])
    assert np.array_equal(out[0], _bf16_of_exact(expected))


def test_zero_weights_give_positive_zero(oracle_mod):
    A = gen.activations(4, 256, 3)
    out = oracle_mod.w8a16_gemm(A, np.zeros((10, 256), np.uint8), np.full((1, 2), 0.005, np.float32))
    assert np.all(out == 0)


def test_rows_independent_and_thread_count_invariant(oracle_mod):
    M, N, K = 16, 130, 640
    A = gen.activations(4, K, M)
    W, S = gen.w8a16_weights(4, N, K)
    ref = oracle_mod.w8a16_gemm(A, W, S, nthreads=1)
    for t in (2, 5, 0):
        assert np.array_equal(oracle_mod.w8a16_gemm(A, W, S, nthreads=t), ref)
    for m in (0, 7, 15):
        assert np.array_equal(oracle_mod.w8a16_gemm(A[m:m + 1], W, S), ref[m:m + 1])
