"""Host-side tests of the C ABI (no GPU needed, nothing is launched).

Covers: the library loads and exports every function include/wqd.h declares;
argument validation happens before any HIP call (each error path returns its
status and message); the packer's layout (golden block, round trip through the
oracle's independent byte-wise unpacker); and the batched launch plan against
the worked example and coverage set printed on page "gemv_q2_vec.rs"
(``mod tests``).
"""
import ctypes
import json
import os

import numpy as np
import pytest

from weight_quantized_decode_block_amd import inputs as gen
from weight_quantized_decode_block_amd import wqd

GOLD = os.path.join(os.path.dirname(__file__), "golden")
FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced (validation fails first)


@pytest.fixture(scope="module")
def L():
    return wqd.lib()


def test_exports_every_declared_symbol(L):
    names = wqd.header_functions()
    assert set(names) >= {"q2_0_gemv", "q2_0_gemv_batchm", "w8a16_gemm_m16", "w8a16_gemm_m16_n64",
                          "w8a16_gemm_m16_strided", "w8a16_gemv_batch16", "w8a16_gemv_batch16_strided",
                          "q2_0_packed_bytes", "q2_0_pack",
                          "q2_0_batchm_chunks", "wqd_last_error"}
    for n in names:
        assert hasattr(L, n), n


def test_product_library_does_not_link_the_oracle():
    blob = open(wqd.LIB_PATH, "rb").read()
    assert b"oracle_" not in blob and b"liboracle" not in blob


def test_bench_read_helper_is_outside_the_product_library():
    """The plain-read kernel bench.py reports as the read ceiling lives in its
    own library; the product C ABI neither exports nor contains it."""
    import ctypes
    from weight_quantized_decode_block_amd import build as hip_build
    assert b"wqd_bench_read" not in open(wqd.LIB_PATH, "rb").read()
    helper = ctypes.CDLL(hip_build.BENCH_LIB)
    assert hasattr(helper, "wqd_bench_read")
    helper.wqd_bench_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    helper.wqd_bench_read.restype = ctypes.c_int
    # argument checks come before any HIP call: null pointer, size not a multiple of 16
    assert helper.wqd_bench_read(None, 16, 256, None) != 0
    assert helper.wqd_bench_read(256, 17, 256, None) != 0


# ------------------------------------------------------------- validation
@pytest.mark.parametrize("args,code,frag", [
    ((None, FAKE, FAKE, 16, 1024, 128), wqd.WQD_ENULL, "non-NULL"),
    ((FAKE, FAKE, FAKE, 16, 1024, 64), wqd.WQD_EINVAL, "group"),
    ((FAKE, FAKE, FAKE, 0, 1024, 128), wqd.WQD_EINVAL, "N must"),
    ((FAKE, FAKE, FAKE, 16, 1000, 128), wqd.WQD_EINVAL, "multiple of 128"),
    ((FAKE, FAKE, FAKE, 16, 0, 128), wqd.WQD_EINVAL, "multiple of 128"),
    ((FAKE + 8, FAKE, FAKE, 16, 1024, 128), wqd.WQD_EALIGN, "A must"),
    ((FAKE, FAKE + 2, FAKE, 16, 1024, 128), wqd.WQD_EALIGN, "B must"),
    ((FAKE, FAKE, FAKE + 1, 16, 1024, 128), wqd.WQD_EALIGN, "C must"),
])
def test_q2_0_gemv_validation(L, args, code, frag):
    rc = L.q2_0_gemv(*args, None)
    assert rc == code
    assert frag in wqd.last_error()


def test_q2_0_batchm_m0_is_noop(L):
    assert L.q2_0_gemv_batchm(FAKE, FAKE, FAKE, 16, 1024, 128, 0, None) == wqd.WQD_OK


def test_q2_0_batchm_validation(L):
    assert L.q2_0_gemv_batchm(FAKE, FAKE, FAKE, 16, 100, 128, 3, None) == wqd.WQD_EINVAL
    assert L.q2_0_gemv_batchm(FAKE, None, FAKE, 16, 1024, 128, 3, None) == wqd.WQD_ENULL


@pytest.mark.parametrize("args,code,frag", [
    ((FAKE, FAKE, FAKE, FAKE, 0, 64, 1024), wqd.WQD_EINVAL, "outside 1..16"),
    ((FAKE, FAKE, FAKE, FAKE, 17, 64, 1024), wqd.WQD_EINVAL, "outside 1..16"),
    ((FAKE, FAKE, FAKE, FAKE, 16, 64, 1000), wqd.WQD_EINVAL, "multiple of 128"),
    ((FAKE, FAKE, FAKE, FAKE, 16, 0, 1024), wqd.WQD_EINVAL, "N must"),
    ((FAKE, FAKE, None, FAKE, 16, 64, 1024), wqd.WQD_ENULL, "non-NULL"),
    ((FAKE, FAKE + 4, FAKE, FAKE, 16, 64, 1024), wqd.WQD_EALIGN, "W must"),
    ((FAKE, FAKE, FAKE + 2, FAKE, 16, 64, 1024), wqd.WQD_EALIGN, "S must"),
])
@pytest.mark.parametrize("fn", ["w8a16_gemm_m16", "w8a16_gemm_m16_n64", "w8a16_gemm_m16_strided",
                                "w8a16_gemv_batch16", "w8a16_gemv_batch16_strided"])
def test_w8a16_validation(L, fn, args, code, frag):
    """The three W8A16 entry points share the guards of page "w8a16_gemm_m16.rs"."""
    extra = (args[6], args[5]) if fn.endswith("_strided") else ()  # pitches = K, N
    rc = getattr(L, fn)(*args, *extra, None)
    assert rc == code
    assert frag in wqd.last_error()
    assert fn in wqd.last_error()


@pytest.mark.parametrize("M,N,K,lda,ldc,frag", [
    (4, 64, 1024, 1016, 64, "cover"),      # a_row_stride < K
    (4, 64, 1024, 1024, 63, "cover"),      # c_row_stride < N
    (4, 64, 1024, 1028, 64, "multiple of 8"),
    (4, 64, 1024, 1030, 70, "multiple of 8"),
    (16, 64, 1024, 0x12000000, 64, "too large"),   # 15 * pitch + K >= 2^32
    (16, 64, 1024, 1024, 0x12000000, "too large"),
])
@pytest.mark.parametrize("fn", ["w8a16_gemm_m16_strided", "w8a16_gemv_batch16_strided"])
def test_w8a16_strided_validation(L, fn, M, N, K, lda, ldc, frag):
    """Pitch rules of page "w8a16_gemm_m16.rs" (doc of w8a16_gemm_m16_strided)."""
    rc = getattr(L, fn)(FAKE, FAKE, FAKE, FAKE, M, N, K, lda, ldc, None)
    assert rc == wqd.WQD_EINVAL
    assert frag in wqd.last_error()


@pytest.mark.parametrize("K,code", [(81920, None), (82048, wqd.WQD_EUNSUPPORTED), (1 << 20, wqd.WQD_EUNSUPPORTED)])
def test_w8a16_gemv_k_limit(L, K, code):
    """The vector-ALU GEMV stages one activation row on chip: K <= 81920."""
    if code is None:  # a valid call: only checked where no GPU could run it on the fake pointers
        try:
            import torch
            if torch.cuda.is_available():
                pytest.skip("a GPU is present")
        except ImportError:
            pass
    rc = L.w8a16_gemv_batch16(FAKE, FAKE, FAKE, FAKE, 1, 64, K, None)
    if code is None:
        assert rc in (wqd.WQD_ENODEV, wqd.WQD_EHIP)
    else:
        assert rc == code and "81920" in wqd.last_error()


@pytest.mark.parametrize("lda,ldc", [(1024, 64), (1032, 65), (4096, 1000)])
def test_w8a16_strided_valid_pitches_reach_the_device_check(L, lda, ldc):
    """Pitches that meet the rules pass validation (no GPU here, so the call
    stops at the device check)."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    rc = L.w8a16_gemm_m16_strided(FAKE, FAKE, FAKE, FAKE, 4, 64, 1024, lda, ldc, None)
    assert rc in (wqd.WQD_ENODEV, wqd.WQD_EHIP)


def test_valid_call_without_gpu_reports_no_device(L):
    """On a host without a GPU a fully valid call must fail cleanly, not crash."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    rc = L.q2_0_gemv(FAKE, FAKE, FAKE, 16, 1024, 128, None)
    assert rc in (wqd.WQD_ENODEV, wqd.WQD_EHIP)
    assert wqd.last_error()


# ----------------------------------------------------------------- packer
def test_packed_bytes():
    assert wqd.q2_0_packed_bytes(5120, 5120) == 6_963_200
    assert wqd.q2_0_packed_bytes(256, 1024) == 69_632
    assert wqd.q2_0_packed_bytes(17408, 5120) == 23_674_880
    assert wqd.q2_0_packed_bytes(4, 100) == 0


def test_pack_golden_block():
    g = json.load(open(os.path.join(GOLD, "q2_0_closed_forms.json")))["pack_golden"]
    codes = (np.arange(128) % 3).astype(np.uint8)[None, :]
    d = np.array([[int(g["d_f16"], 16)]], np.uint16)
    assert wqd.q2_0_pack(codes, d).tobytes().hex() == g["bytes_hex"]


@pytest.mark.parametrize("N,K", [(1, 128), (3, 384), (17, 1024)])
def test_pack_roundtrip_through_oracle_unpacker(oracle_mod, N, K):
    codes, d = gen.q2_0_weights(77, N, K)
    packed = wqd.q2_0_pack(codes, d)
    c2, d2 = oracle_mod.q2_0_unpack(packed, N, K)
    assert np.array_equal(c2, codes) and np.array_equal(d2, d)


def test_pack_rejects_code_3():
    codes = np.ones((1, 128), np.uint8)
    codes[0, 5] = 3
    with pytest.raises(wqd.WqdError):
        wqd.q2_0_pack(codes, np.zeros((1, 1), np.uint16))


# ------------------------------------------------------------ launch plan
def test_launch_plan_worked_example_from_pages():
    g = json.load(open(os.path.join(GOLD, "batchm_launch_chunks.json")))
    ex = g["worked_example"]
    assert wqd.q2_0_batchm_chunks(ex["m"], ex["k"], ex["n"]) == [tuple(c) for c in ex["chunks"]]


def test_launch_plan_covers_rows_exactly():
    g = json.load(open(os.path.join(GOLD, "batchm_launch_chunks.json")))
    for m in g["coverage_m"]:
        plan = wqd.q2_0_batchm_chunks(m, 256, 5)
        r_next = 0
        for a_off, c_off, rows in plan:
            assert a_off == r_next * 256 * 2 and c_off == r_next * 5 * 2
            assert 1 <= rows <= g["max_rows_per_launch"]
            r_next += rows
        assert r_next == m
        assert (len(plan) == 0) == (m == 0)


def test_chunked_plan_with_oracle_as_kernel_equals_per_row(oracle_mod):
    """The page's model of the launch loop: each chunk (driven by the product's
    plan) is computed by the oracle standing in for the kernel, and must equal
    the per-row M=1 results bit for bit, across the 8-row boundaries."""
    n, k = 5, 256
    for m in (1, 2, 3, 8, 9, 16):
        A, codes, d = gen.pages_test_vectors(m, n, k)
        ref = np.concatenate([oracle_mod.q2_0_gemv(A[r:r + 1], codes, d) for r in range(m)])
        got = np.full((m, n), 0xFFFF, np.uint16)
        for a_off, c_off, rows in wqd.q2_0_batchm_chunks(m, k, n):
            r0 = a_off // (k * 2)
            assert c_off == r0 * n * 2
            got[r0:r0 + rows] = oracle_mod.q2_0_gemv(A[r0:r0 + rows], codes, d)
        assert np.array_equal(got, ref)
