"""Pins for the oracle's number codecs against library routines.

Each codec is written in the oracle from its format definition; here it is
checked against an independent implementation (numpy's float16, torch's
bfloat16 and float8_e4m3fn casts), exhaustively where the format is small.
"""
import math

import numpy as np
import pytest
import torch


def test_f16_to_f32_exhaustive(oracle_mod):
    """All 65,536 binary16 patterns decode exactly as numpy's float16 does."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle_mod.f16_to_f32(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_to_f32_matches_torch(oracle_mod):
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = np.array([oracle_mod.bf16_to_f32(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _crafted_f32():
    vals = []
    # exact ties at the bf16 boundary, odd and even upper halves, both signs
    for upper in (0x3F80, 0x3F81, 0x3F82, 0x0001, 0x0080, 0x7F7F, 0x7F7E, 0x4049):
        for lower in (0x7FFF, 0x8000, 0x8001, 0x0000, 0xFFFF):
            for s in (0, 0x8000):
                vals.append(((upper | s) << 16) | lower)
    vals += [0x7F800000, 0xFF800000, 0x00000000, 0x80000000, 0x00000001, 0x807FFFFF]
    return np.array(vals, dtype=np.uint32).view(np.float32)


def test_f32_to_bf16_rne_matches_torch(oracle_mod):
    """Round to nearest even, including ties, subnormals, overflow and signed
    zero, agrees bit for bit with torch's float -> bfloat16 cast."""
    rnd = np.random.Generator(np.random.PCG64(7)).standard_normal(20000).astype(np.float32)
    wide = (np.random.Generator(np.random.PCG64(8)).integers(0, 2**32, 20000, dtype=np.uint64)
            .astype(np.uint32).view(np.float32))
    x = np.concatenate([rnd, rnd * 1e-30, rnd * 1e30, wide, _crafted_f32()])
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle_mod.f32_to_bf16(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_f32_to_bf16_nan_stays_nan(oracle_mod):
    out = oracle_mod.f32_to_bf16(float("nan"))
    assert (out & 0x7F80) == 0x7F80 and (out & 0x007F) != 0


def test_e4m3fn_all_codes_match_torch(oracle_mod):
    """All 256 E4M3FN codes decode as torch.float8_e4m3fn does."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([oracle_mod.e4m3fn_to_f32(int(c)) for c in codes], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


@pytest.mark.parametrize("code,value", [
    (0x7E, 448.0), (0xFE, -448.0), (0x01, 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0xB8, -1.0), (0x40, 2.0), (0x00, 0.0), (0x07, 7 * 2.0 ** -9),
])
def test_e4m3fn_format_definition_values(oracle_mod, code, value):
    """Values fixed by the OCP E4M3FN definition: max 448, min subnormal 2^-9."""
    assert oracle_mod.e4m3fn_to_f32(code) == value


def test_e4m3fn_nan_codes(oracle_mod):
    assert math.isnan(oracle_mod.e4m3fn_to_f32(0x7F))
    assert math.isnan(oracle_mod.e4m3fn_to_f32(0xFF))
