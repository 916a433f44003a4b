"""GPU parity of the W8A16 M16 GEMM against the CPU oracle, through the C ABI.

Bar: every output within 2 BF16 ulp or 1e-2 x row RMS of the oracle; each
output row bit-identical whatever M is; the exact-integer regime bit-identical
to the oracle; rows >= M never written (page "w8a16_gemm_m16.rs", doc of
w8a16_gemm_m16).
"""
import numpy as np
import pytest
import torch

from parity import CANARY, check_parity, dev_f32, dev_u8, dev_u16, host_u16, requires_gpu, ulp_histogram, w8a16_gpu
from weight_quantized_decode_block_amd import inputs as gen

pytestmark = [pytest.mark.gpu, requires_gpu]


def _case(wid, N, K, M, salt=0):
    A = gen.activations(wid, K, M, salt)
    W, S = gen.w8a16_weights(wid, N, K, salt)
    return A, W, S


def test_all_256_e4m3fn_codes_decode_on_device(oracle_mod):
    """W[n,0] = code n, A = e_0, S = 1: C[0,n] is the device's decode of code n."""
    N, K = 256, 128
    W = np.zeros((N, K), np.uint8)
    W[:, 0] = np.arange(256, dtype=np.uint8)
    A = np.zeros((1, K), np.float32)
    A[0, 0] = 1.0
    got = w8a16_gpu(gen.bf16_bits(A), W, np.ones((2, 1), np.float32), N, K)[0]
    ref = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()
    gv = gen.bf16_values(got)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(gv), nan)
    assert np.array_equal(gv[~nan], ref[~nan])
    assert np.array_equal(got[~nan], oracle_mod.w8a16_gemm(gen.bf16_bits(A), W, np.ones((2, 1), np.float32))[0][~nan])


@pytest.mark.parametrize("M", [1, 8, 16])
def test_qkv_parity(oracle_mod, M):
    """N=K=5120, M in {1, 8, 16}."""
    A, W, S = _case(4, 5120, 5120, M)
    got = w8a16_gpu(A, W, S, 5120, 5120)
    ref = oracle_mod.w8a16_gemm(A, W, S)
    check_parity(got, ref, f"w8a16 5120^2 M={M}")
    print("ulp histogram", ulp_histogram(got, ref))


def test_rows_bit_identical_across_m(oracle_mod):
    N, K = 5120, 5120
    A, W, S = _case(4, N, K, 16)
    Wd, Sd = dev_u8(W), dev_f32(S)
    full = w8a16_gpu(A, Wd, Sd, N, K)
    assert np.array_equal(w8a16_gpu(A[:8], Wd, Sd, N, K), full[:8])
    for m in (0, 5, 15):
        assert np.array_equal(w8a16_gpu(A[m:m + 1], Wd, Sd, N, K), full[m:m + 1])


@pytest.mark.parametrize("N,K,M", [(5120, 5120, 2), (5120, 5120, 3), (5120, 5120, 4), (5120, 17408, 1),
                                   (1000, 17408, 3), (1000, 5120, 4), (520, 4096, 1), (264, 4096, 3),
                                   (136, 4096, 5), (136, 4096, 6), (72, 4096, 7), (72, 4096, 8), (1040, 12288, 3),
                                   (200, 8192, 5), (264, 6144, 8)])
def test_every_staging_tier_rows_bit_identical(oracle_mod, N, K, M):
    """The resident-activation kernel copies A with exactly the 16-byte chunks
    per thread that cover it in one round, M * K / 4096 of them: 1 to 10 here
    (K = 4096 at M = 1..8, K = 12288 at M = 3, K = 8192 at M = 5; M = 2, 3, 4
    at K = 5120 take 3, 4, 5 with idle slots; M = 1 at K = 17408 takes 5), and
    two rounds at K = 6144, M = 8 and K = 17408, M = 3 (one 16-row tile per
    workgroup, where these activations stay with this kernel): every row
    bit-identical to its own M=1
    call, a canary row past M untouched, a column sample within tolerance of
    the oracle."""
    A, W, S = _case(43, N, K, M, salt=N + K + M)
    Wd, Sd = dev_u8(W), dev_f32(S)
    got = w8a16_gpu(A, Wd, Sd, N, K, c_rows=M + 1)
    assert np.all(got[M] == CANARY)
    got = got[:M]
    for m in range(M):
        assert np.array_equal(w8a16_gpu(A[m:m + 1], Wd, Sd, N, K), got[m:m + 1]), m
    cols = np.arange(N) if N <= 256 else np.sort(gen.rng(943, N, K).choice(N, 256, replace=False))
    ref = np.concatenate([oracle_mod.w8a16_gemm(A, W[c:c + 1], S[c // 128:c // 128 + 1]) for c in cols], axis=1)
    check_parity(got[:, cols], ref, f"w8a16 {N}x{K} M={M}")


@pytest.mark.parametrize("N,K,M", [(300, 640, 13), (4100, 5120, 16), (20480, 2048, 9), (20736, 1024, 12),
                                   (20744, 5120, 16), (12000, 5120, 16), (10240, 17408, 12), (16400, 6144, 11)])
def test_nine_to_sixteen_rows_kernels(oracle_mod, N, K, M):
    """Nine to sixteen rows: the segmented kernel over one, two and five
    16-row tiles per workgroup (on 256 CUs: N = 300, 4100, 20480), its
    two-group form from three tiles on (N = 12000 and 10240: three, 47 and 40
    rows; N = 16400: five, the last one ragged), and the
    registers kernel where a workgroup's rows need more than five tiles
    (N = 20736, K = 1024: 81 rows, six tiles; N = 20744, K = 5120: five
    blocks per wave).  Every row bit-identical to its own M=1 call (the units
    kernel), rows past M untouched, a column sample (holding the last one)
    within tolerance of the oracle."""
    A, W, S = _case(27, N, K, M, salt=N + 7 * K)
    Wd, Sd = dev_u8(W), dev_f32(S)
    got = w8a16_gpu(A, Wd, Sd, N, K, c_rows=16)
    assert np.all(got[M:] == CANARY)
    got = got[:M]
    for m in range(M):
        assert np.array_equal(w8a16_gpu(A[m:m + 1], Wd, Sd, N, K), got[m:m + 1]), f"row {m}"
    cols = np.arange(N) if N <= 400 else np.union1d(gen.rng(911, N, K).choice(N, 256, replace=False), [N - 1])
    ref = np.concatenate([oracle_mod.w8a16_gemm(A, W[c:c + 1], S[c // 128:c // 128 + 1]) for c in cols], axis=1)
    check_parity(got[:, cols], ref, f"w8a16 {N}x{K} M={M}")


@pytest.mark.parametrize("N,K,M", [(130, 1024, 16), (16, 128, 1), (300, 640, 7)])
def test_exact_integer_regime_bit_identical(oracle_mod, N, K, M):
    A = gen.exact_activations(N + M + 1, M, K)
    W, S = gen.exact_w8a16_weights(N * 3 + K, N, K)
    got = w8a16_gpu(A, W, S, N, K)
    assert np.array_equal(got, oracle_mod.w8a16_gemm(A, W, S))


@pytest.mark.parametrize("N,K,M", [(17, 384, 3), (130, 1152, 16), (1, 128, 1), (200, 256, 9), (4095, 640, 2)])
def test_ragged_shapes_and_canary_rows(oracle_mod, N, K, M):
    A, W, S = _case(14, N, K, M, salt=N + K)
    got = w8a16_gpu(A, W, S, N, K, c_rows=16)
    assert np.all(got[M:] == CANARY)
    check_parity(got[:M], oracle_mod.w8a16_gemm(A, W, S), f"w8a16 N={N} K={K} M={M}")


@pytest.mark.parametrize("N,K", [(17408, 5120), (5120, 17408)])
def test_ffn_shapes(oracle_mod, N, K):
    """FFN up/down shapes: M=16 in full, M=1 bit-identical to row 0, and M=32
    as two calls on contiguous 16-row halves (the page's row-halves rule)."""
    A, W, S = _case(5, N, K, 32)
    Wd, Sd = dev_u8(W), dev_f32(S)
    got16 = w8a16_gpu(A[:16], Wd, Sd, N, K)
    check_parity(got16, oracle_mod.w8a16_gemm(A[:16], W, S), f"w8a16 {N}x{K} M=16")
    assert np.array_equal(w8a16_gpu(A[:1], Wd, Sd, N, K), got16[:1])
    Ad = torch.from_numpy(A.view(np.int16)).to("cuda")
    C = torch.full((32, N), CANARY, dtype=torch.int16, device="cuda")
    from weight_quantized_decode_block_amd import wqd
    wqd.w8a16_gemm_m16(Ad[:16], Wd, Sd, C[:16], 16, N, K)
    wqd.w8a16_gemm_m16(Ad[16:], Wd, Sd, C[16:], 16, N, K)
    torch.cuda.synchronize()
    got32 = C.cpu().numpy().view(np.uint16)
    assert np.array_equal(got32[:16], got16)
    cols = np.sort(gen.rng(906, N, K).choice(N, 384, replace=False))
    ref = np.concatenate([oracle_mod.w8a16_gemm(A[16:], W[c:c + 1], S[c // 128:c // 128 + 1]) for c in cols], axis=1)
    check_parity(got32[16:, cols], ref, f"w8a16 {N}x{K} rows 16..31 sampled")


@pytest.mark.parametrize("N,K,M", [(5120, 17408, 5), (5120, 17408, 8), (5120, 17408, 12), (1000, 16512, 9),
                                   (17408, 9216, 10), (300, 17408, 7), (5120, 17408, 3), (8192, 8192, 8),
                                   (5120, 6144, 8), (20736, 10240, 8), (20744, 6144, 12), (5120, 7168, 6),
                                   (5120, 6144, 7)])
def test_activations_larger_than_lds(oracle_mod, N, K, M):
    """Large activations are staged in segments of K: those larger than LDS
    (M x K x 2 bytes over 160 KB), and resident ones of 96 KB or more (84 KB
    at six to eight rows, more than 100 KB below five rows) over two or three
    16-row tiles per workgroup (N = 5120 K = 17408 M = 3, N = K = 8192 M = 8,
    N = 5120 K = 6144 M = 8 and 7, N = 5120 K = 7168 M = 6).
    Every row equals its own M=1 call (which keeps all of A in LDS) bit for
    bit, the 64-row-band call gives the same bits, and sampled columns are
    within the parity bar.  Covers K not a multiple of 1024 (16512), a
    workgroup with five 16-row tiles (N = 17408) and one tile (N = 300), and
    more than five tiles per workgroup, served as launches over ranges of
    whole 128-row scale groups (N = 20736 and 20744: six tiles, two ranges,
    the second of 20744 ending mid-group)."""
    from weight_quantized_decode_block_amd import wqd
    A, W, S = _case(31, N, K, M, salt=N + K)
    Wd, Sd = dev_u8(W), dev_f32(S)
    got = w8a16_gpu(A, Wd, Sd, N, K)
    for m in range(M):
        assert np.array_equal(w8a16_gpu(A[m:m + 1], Wd, Sd, N, K), got[m:m + 1]), f"row {m}"
    C = torch.full((16, N), CANARY, dtype=torch.int16, device="cuda")
    wqd.w8a16_gemm_m16_n64(dev_u16(A), Wd, Sd, C, M, N, K)
    torch.cuda.synchronize()
    band = host_u16(C)
    assert np.array_equal(band[:M], got)
    assert np.all(band[M:] == CANARY)
    cols = np.sort(gen.rng(907, N, K).choice(N, min(N, 256), replace=False))
    ref = np.concatenate([oracle_mod.w8a16_gemm(A, W[c:c + 1], S[c // 128:c // 128 + 1]) for c in cols], axis=1)
    check_parity(got[:, cols], ref, f"w8a16 {N}x{K} M={M} sampled")


# --------------------------------------------- _n64 and _strided variants
def _contiguous(A, Wd, Sd, N, K):
    return w8a16_gpu(A, Wd, Sd, N, K)


@pytest.mark.parametrize("N,K,M", [(5120, 5120, 1), (5120, 5120, 8), (5120, 5120, 16), (17, 384, 3),
                                   (130, 1152, 12), (200, 256, 9), (4095, 640, 2), (1, 128, 1), (80, 1024, 5)])
def test_n64_bit_identical_to_contiguous(oracle_mod, N, K, M):
    """64-row bands per workgroup (page "w8a16_gemm_m16.rs", w8a16_gemm_m16_n64):
    same sums in the same order, so every output equals w8a16_gemm_m16's; rows
    >= M stay untouched."""
    from weight_quantized_decode_block_amd import wqd
    A, W, S = _case(21, N, K, M, salt=N + 3 * K)
    Wd, Sd = dev_u8(W), dev_f32(S)
    ref = _contiguous(A, Wd, Sd, N, K)
    C = torch.full((16, N), CANARY, dtype=torch.int16, device="cuda")
    wqd.w8a16_gemm_m16_n64(dev_u16(A), Wd, Sd, C, M, N, K)
    torch.cuda.synchronize()
    got = host_u16(C)
    assert np.array_equal(got[:M], ref)
    assert np.all(got[M:] == CANARY)
    if N * K <= 1 << 20:
        check_parity(got[:M], oracle_mod.w8a16_gemm(A, W, S), f"w8a16 n64 N={N} K={K} M={M}")


@pytest.mark.parametrize("N,K,M,pa,pc", [
    (5120, 5120, 1, 0, 0), (5120, 5120, 8, 8, 1), (5120, 5120, 16, 136, 37),
    (130, 1024, 16, 8, 3), (17, 384, 3, 64, 0), (300, 640, 7, 0, 300), (33, 128, 9, 1024, 5),
    (300, 17408, 7, 72, 5), (2000, 16512, 12, 8, 0),
])
def test_strided_rows_equal_contiguous_and_padding_untouched(oracle_mod, N, K, M, pa, pc):
    """A and C as row slices of wider buffers (page "w8a16_gemm_m16.rs",
    w8a16_gemm_m16_strided): each output row equals the contiguous call's, the
    activation padding (filled with NaN bit patterns) is never read into a
    sum, and C's padding columns and rows >= M keep their canary.  The last
    two shapes run the segmented kernel, whose last K-segment copies part of
    each row's padding into LDS (K = 16512 ends in a partial segment)."""
    from weight_quantized_decode_block_amd import wqd
    A, W, S = _case(22, N, K, M, salt=N + 5 * K)
    Wd, Sd = dev_u8(W), dev_f32(S)
    ref = _contiguous(A, Wd, Sd, N, K)
    lda, ldc = K + pa, N + pc
    Ab = np.full((M, lda), 0x7FC1, np.uint16)  # NaN padding: a stray read would show in C
    Ab[:, :K] = A
    C = torch.full((M + 1, ldc), CANARY, dtype=torch.int16, device="cuda")
    wqd.w8a16_gemm_m16_strided(dev_u16(Ab), Wd, Sd, C, M, N, K, lda, ldc)
    torch.cuda.synchronize()
    got = host_u16(C)
    assert np.array_equal(got[:M, :N], ref)
    assert np.all(got[:M, N:] == CANARY)
    assert np.all(got[M:] == CANARY)
    if N * K <= 1 << 20:
        check_parity(got[:M, :N], oracle_mod.w8a16_gemm(A, W, S), f"w8a16 strided N={N} K={K} M={M}")


def test_strided_slices_of_a_shared_buffer(oracle_mod):
    """Two calls write column slices of one output buffer and read column
    slices of one activation buffer (a multi-sequence buffer with Q, K and V
    side by side): each slice equals its own contiguous call."""
    from weight_quantized_decode_block_amd import wqd
    M, K, N0, N1 = 6, 1024, 640, 384
    A2 = gen.activations(23, 2 * K, M, 0)  # [M, 2K]: two activation sets side by side
    W0, S0 = gen.w8a16_weights(24, N0, K, 0)
    W1, S1 = gen.w8a16_weights(25, N1, K, 0)
    Ad = dev_u16(A2)
    C = torch.full((M, N0 + N1 + 8), CANARY, dtype=torch.int16, device="cuda")
    wqd.w8a16_gemm_m16_strided(Ad, dev_u8(W0), dev_f32(S0), C, M, N0, K, 2 * K, N0 + N1 + 8)
    wqd.w8a16_gemm_m16_strided(Ad[:, K:], dev_u8(W1), dev_f32(S1), C[:, N0:], M, N1, K, 2 * K, N0 + N1 + 8)
    torch.cuda.synchronize()
    got = host_u16(C)
    assert np.array_equal(got[:, :N0], _contiguous(np.ascontiguousarray(A2[:, :K]), dev_u8(W0), dev_f32(S0), N0, K))
    assert np.array_equal(got[:, N0:N0 + N1],
                          _contiguous(np.ascontiguousarray(A2[:, K:]), dev_u8(W1), dev_f32(S1), N1, K))
    assert np.all(got[:, N0 + N1:] == CANARY)
    check_parity(got[:, :N0], oracle_mod.w8a16_gemm(np.ascontiguousarray(A2[:, :K]), W0, S0), "slice 0")
