"""GPU parity of the Q2_0 GEMV / batched GEMV against the CPU oracle, through
the C ABI.

Bar: every output within 2 BF16 ulp or 1e-2 x row RMS of the oracle; batched
rows bit-identical to the M=1 launch (page "gemv_q2_vec.rs", doc of
q2_0_gemv_vec_batchm); the exact-integer regime bit-identical to the oracle;
rows past M and columns past N never written.
"""
import json
import os

import numpy as np
import pytest
import torch

from parity import (CANARY, check_parity, dev_u8, q2_0_gpu, requires_gpu, ulp_histogram)
from weight_quantized_decode_block_amd import inputs as gen
from weight_quantized_decode_block_amd import wqd

pytestmark = [pytest.mark.gpu, requires_gpu]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q2_0_closed_forms.json")


def _case(wid, N, K, M, salt=0):
    A = gen.activations(wid, K, M, salt)
    codes, d = gen.q2_0_weights(wid, N, K, salt)
    return A, codes, d, wqd.q2_0_pack(codes, d)


def _m1_rows(A, packed_dev, N, K):
    return np.concatenate([q2_0_gpu(A[m:m + 1], packed_dev, N, K, single=True) for m in range(A.shape[0])])


def test_small_gemv_parity(oracle_mod):
    """N=256, K=1024, M=1 (the small Q2_0 workload)."""
    A, codes, d, packed = _case(1, 256, 1024, 1)
    got = q2_0_gpu(A, packed, 256, 1024, single=True)
    ref = oracle_mod.q2_0_gemv(A, codes, d)
    check_parity(got, ref, "q2_0 256x1024")
    print("ulp histogram", ulp_histogram(got, ref))


def test_qkv_gemv_parity(oracle_mod):
    """N=K=5120, M=1."""
    A, codes, d, packed = _case(2, 5120, 5120, 1)
    got = q2_0_gpu(A, packed, 5120, 5120, single=True)
    ref = oracle_mod.q2_0_gemv(A, codes, d)
    check_parity(got, ref, "q2_0 5120^2 M=1")
    print("ulp histogram", ulp_histogram(got, ref))


@pytest.mark.parametrize("M", [2, 4, 5, 8, 16])
def test_batched_rows_bit_identical_and_parity(oracle_mod, M):
    """N=K=5120, M in {2,4,5,8,16}; M=16 runs as two 8-row launches."""
    A, codes, d, packed = _case(3, 5120, 5120, M)
    Bd = dev_u8(packed)
    got = q2_0_gpu(A, Bd, 5120, 5120, extra_rows=1)
    assert np.all(got[M] == CANARY)
    got = got[:M]
    assert np.array_equal(got, _m1_rows(A, Bd, 5120, 5120))
    check_parity(got, oracle_mod.q2_0_gemv(A, codes, d), f"q2_0 5120^2 M={M}")


@pytest.mark.parametrize("N,K", [(1, 128), (37, 384), (100, 1152), (16, 256), (33, 640), (129, 2048), (8, 128)])
@pytest.mark.parametrize("M", [1, 3, 8, 9])
def test_ragged_shapes(oracle_mod, N, K, M):
    """Row tails (N % 16 != 0), odd block counts (K/128 odd, blocks at 2 mod 4
    offsets, the last block ending mid-dword) and chunk boundaries."""
    A, codes, d, packed = _case(11, N, K, M, salt=N * 7 + K)
    Bd = dev_u8(packed)
    got = q2_0_gpu(A, Bd, N, K, extra_rows=2)
    assert np.all(got[M:] == CANARY)
    got = got[:M]
    check_parity(got, oracle_mod.q2_0_gemv(A, codes, d), f"q2_0 N={N} K={K} M={M}")
    assert np.array_equal(got, _m1_rows(A, Bd, N, K))


@pytest.mark.parametrize("N,K,M", [(64, 1024, 1), (37, 640, 8), (300, 5120, 16)])
def test_exact_integer_regime_bit_identical(oracle_mod, N, K, M):
    """a in [-8,8] integers, d = 2^-j: exact in fp32 in any order, so the GPU
    must equal the oracle bit for bit."""
    A = gen.exact_activations(N + M, M, K)
    codes = gen.rng(902, 2, N).integers(0, 3, size=(N, K), dtype=np.uint8)
    d = gen.exact_q2_0_scales(N * K, N, K)
    got = q2_0_gpu(A, wqd.q2_0_pack(codes, d), N, K)
    assert np.array_equal(got, oracle_mod.q2_0_gemv(A, codes, d))


def test_code_3_decodes_to_plus_2d(oracle_mod):
    """The layout admits code 3 (the packer rejects it); (code & 3) - 1 makes it +2d."""
    N, K, M = 24, 512, 2
    A = gen.activations(12, K, M)
    codes = gen.rng(903, 2).integers(0, 3, size=(N, K), dtype=np.uint8)
    d = gen.f16_bits(np.full((N, K // 128), 0.03))
    packed = wqd.q2_0_pack(codes, d).copy()
    r = gen.rng(903, 9)
    for n in range(N):
        for k in r.choice(K, 9, replace=False):
            codes[n, k] = 3
            blk = (n * (K // 128) + k // 128) * 34
            packed[blk + 2 + (k % 128) // 4] |= np.uint8(3 << (2 * (k % 4)))
    c2, _ = oracle_mod.q2_0_unpack(packed, N, K)
    assert np.array_equal(c2, codes)
    check_parity(q2_0_gpu(A, packed, N, K), oracle_mod.q2_0_gemv(A, codes, d), "code 3")


def test_closed_forms_on_gpu(oracle_mod):
    """All codes 1 gives +0; one nonzero code gives bf16(a_k * (c-1) * d)."""
    N, K = 20, 1024
    A = gen.activations(13, K, 3)
    d = gen.f16_bits(np.abs(gen.rng(904, 3).normal(0, 0.02, (N, K // 128))) + 1e-3)
    ones = np.ones((N, K), np.uint8)
    got = q2_0_gpu(A, wqd.q2_0_pack(ones, d), N, K)
    assert np.all(got == 0)
    single = ones.copy()
    ks = gen.rng(904, 4).integers(0, K, N)
    single[np.arange(N), ks] = np.where(np.arange(N) % 2 == 0, 0, 2)
    got = q2_0_gpu(A, wqd.q2_0_pack(single, d), N, K)
    assert np.array_equal(got, oracle_mod.q2_0_gemv(A, single, d))


def test_worked_examples_on_gpu():
    """The closed-form examples of the golden file, bit for bit."""
    exs = {e["name"]: int(e["expected_bf16"], 16) for e in json.load(open(GOLDEN))["examples"]}
    from test_oracle_q2_0 import _example_inputs
    for name, expected in exs.items():
        K, A, codes, d = _example_inputs(name)
        got = q2_0_gpu(A, wqd.q2_0_pack(codes, d), 1, K, single=True)
        assert int(got[0, 0]) == expected, name


@pytest.mark.parametrize("N,K", [(17408, 5120), (5120, 17408)])
def test_ffn_shapes(oracle_mod, N, K):
    """FFN up/down shapes: M=1 in full; M=8 and M=32 (four 8-row launches)
    bit-identical to M=1 per row and within tolerance on a row sample."""
    A, codes, d, packed = _case(5, N, K, 32)
    Bd = dev_u8(packed)
    got1 = q2_0_gpu(A[:1], Bd, N, K, single=True)
    check_parity(got1, oracle_mod.q2_0_gemv(A[:1], codes, d), f"q2_0 {N}x{K} M=1")
    got32 = q2_0_gpu(A, Bd, N, K)
    got8 = q2_0_gpu(A[:8], Bd, N, K)
    assert np.array_equal(got8, got32[:8])
    for m in (0, 7, 8, 21, 31):
        assert np.array_equal(got32[m:m + 1], q2_0_gpu(A[m:m + 1], Bd, N, K, single=True))
    cols = np.sort(gen.rng(905, N, K).choice(N, 512, replace=False))
    ref = oracle_mod.q2_0_gemv(A, codes[cols], d[cols])
    check_parity(got32[:, cols], ref, f"q2_0 {N}x{K} M=32 sampled")


@pytest.mark.parametrize("N,K,M", [(37, 12288, 8), (200, 12288, 7), (1, 12288, 8), (333, 17408, 6), (2049, 10240, 8),
                                   (9216, 17408, 8), (10496, 17408, 5), (12304, 12288, 8), (18440, 10240, 8),
                                   (8200, 20480, 4)])
def test_large_k_batched_rows(oracle_mod, N, K, M):
    """Activations too large for LDS: the segmented kernel, over up to nine
    8-row tiles per workgroup (N = 9216, 10496 and 12304 on 256 CUs give 36,
    41 and 49 rows per workgroup: five, six and seven tiles, the last with
    one unit in flight), and as launches over row ranges beyond that
    (N = 18440: 73 rows, ten tiles, two ranges; N = 8200 M = 4: 33 rows, five
    tiles, two ranges for the 4-row instance's limit of four): ragged N,
    every row bit-identical to its own M=1 launch (the resident-activation
    kernel) and within tolerance of the oracle on a column sample."""
    A, codes, d, packed = _case(31, N, K, M, salt=N + K)
    Bd = dev_u8(packed)
    got = q2_0_gpu(A, Bd, N, K)
    for m in range(M):
        assert np.array_equal(got[m:m + 1], q2_0_gpu(A[m:m + 1], Bd, N, K, single=True)), m
    cols = np.arange(N) if N <= 400 else np.sort(gen.rng(931, N, K).choice(N, 256, replace=False))
    check_parity(got[:, cols], oracle_mod.q2_0_gemv(A, codes[cols], d[cols]), f"q2_0 {N}x{K} M={M}")


@pytest.mark.parametrize("N,K,M", [(5120, 5120, 3), (17408, 5120, 3), (17408, 5120, 4), (5120, 17408, 2),
                                   (5120, 17408, 3), (5120, 17408, 4), (4100, 5120, 3), (2052, 17408, 2)])
def test_two_to_four_rows_every_staging_tier(oracle_mod, N, K, M):
    """Two to four rows run at two workgroups per compute unit with a two-deep
    ring below 16 MB of weights, and at one with a three-deep ring whose third
    request follows the staging barrier above (and at K = 17408, N = 2052,
    where two copies of the activations do not fit in LDS), with the staging
    chunks per thread that cover A (M = 3 at K = 5120 takes 4, M = 4 takes 5,
    M = 2 at K = 17408 takes 9); M = 3 and 4 at N = 5120, K = 17408 (104 and
    139 KB of activations over three tiles per workgroup) run the segmented
    kernel; ragged N (4100 and 2052 end in a partial tile).  Every row bit-identical to its own
    M=1 launch, a canary row past M untouched, a column sample within
    tolerance of the oracle."""
    A, codes, d, packed = _case(41, N, K, M, salt=N * 7 + K + M)
    Bd = dev_u8(packed)
    got = q2_0_gpu(A, Bd, N, K, extra_rows=1)
    assert np.all(got[M] == CANARY)
    got = got[:M]
    for m in range(M):
        assert np.array_equal(got[m:m + 1], q2_0_gpu(A[m:m + 1], Bd, N, K, single=True)), m
    cols = np.sort(gen.rng(941, N, K).choice(N, 256, replace=False))
    cols = np.union1d(cols, [N - 1])
    check_parity(got[:, cols], oracle_mod.q2_0_gemv(A, codes[cols], d[cols]), f"q2_0 {N}x{K} M={M}")


@pytest.mark.parametrize("N,K,M", [(8, 5120, 8), (20, 1024, 5), (4104, 5120, 7), (17408, 5120, 6), (1032, 2048, 8),
                                   (3, 5120, 6), (16392, 5120, 8), (17400, 5120, 5), (15416, 4096, 8),
                                   (15424, 4096, 8)])
def test_five_to_eight_rows_tile_counts(oracle_mod, N, K, M):
    """Five to eight resident activation rows over tile counts 1, 3 (odd), 513,
    129 and N below one tile (one group of 8 waves per workgroup), and over
    2176, 2049 and 2175 tiles of matrices of 16 MB or more (two subgroups per
    workgroup, where the second walks padding tiles when it owns fewer), and
    both sides of that 16 MB switch at eight tiles per workgroup (K = 4096,
    N = 15416 just under, 15424 just over):
    every row bit-identical to its own M=1 launch, a canary row past M
    untouched, all columns (or a sample holding the last one) within
    tolerance of the oracle."""
    A, codes, d, packed = _case(47, N, K, M, salt=N * 3 + K + M)
    Bd = dev_u8(packed)
    got = q2_0_gpu(A, Bd, N, K, extra_rows=1)
    assert np.all(got[M] == CANARY)
    got = got[:M]
    for m in range(M):
        assert np.array_equal(got[m:m + 1], q2_0_gpu(A[m:m + 1], Bd, N, K, single=True)), m
    cols = np.arange(N) if N <= 400 else np.union1d(gen.rng(947, N, K).choice(N, 256, replace=False), [N - 1])
    check_parity(got[:, cols], oracle_mod.q2_0_gemv(A, codes[cols], d[cols]), f"q2_0 {N}x{K} M={M}")


@pytest.mark.parametrize("N,K,M", [(3, 20480, 8), (17, 17408, 8), (2049, 10240, 8), (4100, 17408, 5),
                                   (5120, 17408, 3), (4096, 12288, 4), (5120, 6144, 8), (5120, 8192, 6),
                                   (8192, 20480, 7), (17408, 10240, 8)])
def test_segmented_kernel_tiles_and_segments(oracle_mod, N, K, M):
    """The segmented kernel over every tile count per workgroup (on 256 CUs:
    N = 3 and 17, one tile holding 3 and 6 rows; 2049, two; 4100, three or
    two in one launch; 8192, four; 17408, nine, whose 576 outputs per
    workgroup outnumber its threads), full and partial last segments (K = 17408:
    four segments of 16 pairs and one of 4; 10240 and 6144: two and one, or
    one and one, of 8; 20480 and 8192: full ones only; 32-pair segments for up
    to four rows, K = 17408 M = 3: two and one of 4, K = 12288 M = 4: one and
    one of 16), the 4-, 6- and 8-row instances, and both ways in:
    activations too large for LDS, and resident ones of 96 KB or more over two
    or three tiles (4096 x 12288 M = 4, 5120 x 6144 M = 8, 5120 x 8192 M = 6).
    Every row bit-identical to its own M=1 launch (the resident-activation
    kernel), a canary row past M untouched, all columns (or a sample holding
    the last one) within tolerance of the oracle."""
    A, codes, d, packed = _case(59, N, K, M, salt=N * 5 + K + M)
    Bd = dev_u8(packed)
    got = q2_0_gpu(A, Bd, N, K, extra_rows=1)
    assert np.all(got[M] == CANARY)
    got = got[:M]
    for m in range(M):
        assert np.array_equal(got[m:m + 1], q2_0_gpu(A[m:m + 1], Bd, N, K, single=True)), m
    cols = np.arange(N) if N <= 400 else np.union1d(gen.rng(953, N, K).choice(N, 256, replace=False), [N - 1])
    check_parity(got[:, cols], oracle_mod.q2_0_gemv(A, codes[cols], d[cols]), f"q2_0 {N}x{K} M={M}")


@pytest.mark.parametrize("N,K,M", [(5120, 17408, 2), (4100, 16384, 2), (12288, 20480, 2), (20480, 16384, 2),
                                   (8192, 17408, 4), (8192, 17408, 3), (5120, 7168, 6), (4096, 7168, 5),
                                   (5120, 6144, 7), (5120, 11264, 4), (5120, 14336, 3), (7168, 6144, 7)])
def test_segmented_kernel_extra_routes(oracle_mod, N, K, M):
    """Two rows whose activations are 64 KB or more (K >= 16384) run the
    segmented kernel's 2-row instance over two to nine tiles per workgroup
    (on 256 CUs: N = 5120 and 4100, three, 20 and 17 rows; N = 12288, six),
    but not over ten (N = 20480 stays with the resident-activation kernel);
    three or four rows of 96 KB or more over four tiles run its 4-row
    instance (N = 8192, K = 17408); five to seven rows of 60 KB or more from
    K = 6144 on run its 6- and 8-row instances over two to four tiles
    (N = 5120 and 4096, K = 7168 and 6144; N = 7168, four tiles); three or four rows of 84 KB or
    more over three tiles run its 4-row instance (K = 11264 and 14336).
    Every
    row bit-identical to its own M=1 launch (the resident-activation kernel),
    a canary row past M untouched, a sample of columns holding the last one
    within tolerance of the oracle."""
    A, codes, d, packed = _case(71, N, K, M, salt=N * 17 + K + M)
    Bd = dev_u8(packed)
    got = q2_0_gpu(A, Bd, N, K, extra_rows=1)
    assert np.all(got[M] == CANARY)
    got = got[:M]
    for m in range(M):
        assert np.array_equal(got[m:m + 1], q2_0_gpu(A[m:m + 1], Bd, N, K, single=True)), m
    cols = np.union1d(gen.rng(977, N, K).choice(N, 256, replace=False), [N - 1])
    check_parity(got[:, cols], oracle_mod.q2_0_gemv(A, codes[cols], d[cols]), f"q2_0 {N}x{K} M={M}")


@pytest.mark.parametrize("N,K,M", [(9219, 17408, 8), (9000, 20480, 8), (12288, 17408, 7), (10496, 17408, 5),
                                   (12304, 17408, 6), (12304, 17408, 8), (8200, 17408, 8), (12288, 5120, 8),
                                   (9216, 5120, 8), (12288, 4096, 5), (14336, 5120, 6)])
def test_segmented_two_group_form(oracle_mod, N, K, M):
    """Five to seven tiles per workgroup at six or eight activation rows run the
    segmented kernel's two-group form (16 waves, the tiles split between two
    groups of 8 that own the same pairs): five tiles (N = 9219, a ragged last
    tile; N = 9000 with K = 20480, full segments only; N = 8200, 33 rows on
    some workgroups and 32 on others, so that group 0's third tile is real on
    some and empty on others), six (N = 12288, the 8-row instance at M = 7;
    N = 10496, the 6-row instance at M = 5) and seven (N = 12304, both
    instances); also with resident activations (K = 4096 and 5120, N = 9216
    to 14336, where it runs ahead of both forms of the resident-activation
    kernel).  Every row bit-identical to its own M=1 launch
    (the resident-activation kernel, 8 waves), a canary row past M untouched,
    a sample of columns holding the last one within tolerance of the oracle."""
    A, codes, d, packed = _case(67, N, K, M, salt=N * 13 + K + M)
    Bd = dev_u8(packed)
    got = q2_0_gpu(A, Bd, N, K, extra_rows=1)
    assert np.all(got[M] == CANARY)
    got = got[:M]
    for m in range(M):
        assert np.array_equal(got[m:m + 1], q2_0_gpu(A[m:m + 1], Bd, N, K, single=True)), m
    cols = np.union1d(gen.rng(971, N, K).choice(N, 256, replace=False), [N - 1])
    check_parity(got[:, cols], oracle_mod.q2_0_gemv(A, codes[cols], d[cols]), f"q2_0 {N}x{K} M={M}")


@pytest.mark.parametrize("N,K,M", [(37, 1280, 1), (37, 1280, 3), (300, 3328, 8), (1029, 3328, 5), (5120, 11008, 1),
                                   (5120, 11008, 4), (5120, 11008, 8), (600, 13824, 2), (300, 81920, 1),
                                   (200, 40960, 2)])
def test_even_block_counts_and_one_or_two_large_rows(oracle_mod, N, K, M):
    """K a multiple of 256 but not of 1024 (K / 128 = 10, 26, 86 and 108: odd
    pair counts and waves owning different numbers of pairs) runs the
    matrix-core kernels: the pairs kernel, and the segmented kernel where the
    activations are large (K = 11008: 86 KB at M = 4, 176 KB at M = 8).  One
    and two rows whose activations do not fit in LDS (K = 81920 and 40960:
    160 KB) run the segmented kernel's 1- and 2-row instances.  Every row
    bit-identical to its own M=1 launch, a canary row past M untouched, all
    columns (or a sample holding the last one) within tolerance of the
    oracle."""
    A, codes, d, packed = _case(61, N, K, M, salt=N * 11 + K + M)
    Bd = dev_u8(packed)
    got = q2_0_gpu(A, Bd, N, K, extra_rows=1)
    assert np.all(got[M] == CANARY)
    got = got[:M]
    for m in range(M):
        assert np.array_equal(got[m:m + 1], q2_0_gpu(A[m:m + 1], Bd, N, K, single=True)), m
    cols = np.arange(N) if N <= 400 else np.union1d(gen.rng(961, N, K).choice(N, 256, replace=False), [N - 1])
    check_parity(got[:, cols], oracle_mod.q2_0_gemv(A, codes[cols], d[cols]), f"q2_0 {N}x{K} M={M}")


_TIER_CHILD = r"""
import sys
import numpy as np
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + "/tests")
from parity import q2_0_gpu
from weight_quantized_decode_block_amd import inputs as gen, wqd
assert not wqd.q2_0_exact_m_tiers_enabled()
outs = {}
for N, K, M in [(5120, 5120, 3), (5120, 5120, 5), (5120, 5120, 6), (333, 17408, 6), (17400, 5120, 5)]:
    A = gen.activations(53, K, M, N + M)
    codes, d = gen.q2_0_weights(53, N, K, N + M)
    assert wqd.q2_0_tier_width(M) == 8
    outs[f"{N}_{K}_{M}"] = q2_0_gpu(A, wqd.q2_0_pack(codes, d), N, K)
np.savez(sys.argv[2], **outs)
"""


def test_exact_row_tiers_equal_base_tier_bits(tmp_path):
    """The kill switch moves 3, 5 and 6 rows from the exact 4- and 6-row tiers
    onto the 8-row tier (page "w4a16_gemv_tiers.rs", "Kill switch"); run in a
    child process with the switch set, every output is bit-identical to this
    process's exact-tier launch, over the resident-activation kernel, the
    segmented kernel (K = 17408) and the two-subgroup path (N = 17400)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, WQD_NO_EXACT_M_TIERS="1")
    out = tmp_path / "tiers.npz"
    print("child: kill switch set, shapes 5120^2 M=3,5,6; 333x17408 M=6; 17400x5120 M=5", flush=True)
    subprocess.run([sys.executable, "-c", _TIER_CHILD, root, str(out)], env=env, check=True, timeout=300)
    base = np.load(out)
    assert wqd.q2_0_exact_m_tiers_enabled()
    for key in base.files:
        N, K, M = map(int, key.split("_"))
        assert wqd.q2_0_tier_width(M) in (4, 6)
        A = gen.activations(53, K, M, N + M)
        codes, d = gen.q2_0_weights(53, N, K, N + M)
        got = q2_0_gpu(A, wqd.q2_0_pack(codes, d), N, K)
        assert np.array_equal(got, base[key]), key


@pytest.mark.parametrize("N,K,M", [(8, 1024, 2), (24, 1024, 3), (40, 2048, 4), (5000, 3072, 2), (300, 4096, 6),
                                   (1000, 5120, 3), (4104, 6144, 5)])
def test_two_deep_ring_drain_unit_counts(oracle_mod, N, K, M):
    """Batched rows on a two-deep ring finish with straight-line code sized to
    the units left: fewer units per wave than the ring (K = 1024: four pairs
    for eight waves, so each wave has one unit per tile or an empty one), two
    or three left after the loop (K = 2048 .. 6144 give 1 to 3 pairs per wave
    and tile, over one to several tiles per workgroup).  Every row equals its
    own M=1 launch, a canary row past M stays untouched and the outputs (or a
    column sample holding the last one) are within tolerance of the oracle."""
    print(f"drain N={N} K={K} M={M}", flush=True)
    A, codes, d, packed = _case(59, N, K, M, salt=N * 5 + K + M)
    Bd = dev_u8(packed)
    got = q2_0_gpu(A, Bd, N, K, extra_rows=1)
    assert np.all(got[M] == CANARY)
    got = got[:M]
    for m in range(M):
        assert np.array_equal(got[m:m + 1], q2_0_gpu(A[m:m + 1], Bd, N, K, single=True)), m
    cols = np.arange(N) if N <= 400 else np.union1d(gen.rng(959, N, K).choice(N, 256, replace=False), [N - 1])
    check_parity(got[:, cols], oracle_mod.q2_0_gemv(A, codes[cols], d[cols]), f"q2_0 {N}x{K} M={M}")


@pytest.mark.parametrize("N,K,M", [(520, 4096, 1), (520, 4096, 2), (264, 4096, 3), (264, 4096, 4), (136, 4096, 5),
                                   (136, 4096, 6), (72, 4096, 7), (72, 4096, 8), (1040, 12288, 3), (200, 8192, 5),
                                   (264, 6144, 8), (130, 2048, 1)])
def test_every_staging_width(oracle_mod, N, K, M):
    """The activation copy gives each thread exactly the 16-byte chunks that
    cover A in one round: M * K / 4096 of them here, every width from 1 to 10
    (K = 4096 at M = 1..8, K = 12288 at M = 3, K = 8192 at M = 5), more than
    one round (K = 6144 at M = 8: 12 chunks, two rounds of 10) and a round
    with idle slots (K = 2048 at M = 1).  Every row equals its own M=1 launch,
    a canary row past M stays untouched and the outputs are within tolerance
    of the oracle."""
    print(f"staging N={N} K={K} M={M}", flush=True)
    A, codes, d, packed = _case(61, N, K, M, salt=N * 7 + K + M)
    Bd = dev_u8(packed)
    got = q2_0_gpu(A, Bd, N, K, extra_rows=1)
    assert np.all(got[M] == CANARY)
    got = got[:M]
    for m in range(M):
        assert np.array_equal(got[m:m + 1], q2_0_gpu(A[m:m + 1], Bd, N, K, single=True)), m
    check_parity(got, oracle_mod.q2_0_gemv(A, codes, d), f"q2_0 {N}x{K} M={M}")
