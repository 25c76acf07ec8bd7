"""Pins for the oracle's storage-format code (oracle/formats.py).

The codec is pinned against (a) hand-derived values of the OCP E4M3 format in
tests/golden, (b) torch's independent float8_e4m3fn conversion over every
fp16 and every bf16 bit pattern, and (c) the round trip over all codes."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split()[:2])
    return rows


def test_e4m3_decode_golden():
    for code_s, val_s in _read_table("e4m3_codes.txt"):
        code = int(code_s, 16)
        got = F.e4m3_to_f64(np.array([code], np.uint8))[0]
        want = float(val_s)
        if math.isnan(want):
            assert math.isnan(got), code_s
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code_s


def test_e4m3_decode_all_codes_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_to_f64(codes.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.sum(nan) == 2                       # 0x7F and 0xFF only
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_e4m3_encode_golden():
    for x_s, code_s in _read_table("e4m3_encode_cases.txt"):
        x = np.float32(float(x_s))
        got = int(F.e4m3_encode_f32(np.array([x], np.float32))[0])
        assert got == int(code_s, 16), (x_s, hex(got), code_s)


def _torch_encode(x32: torch.Tensor) -> np.ndarray:
    """Independent reference: torch's fp32 -> float8_e4m3fn (round to nearest
    even) after saturation to +-448; NaN inputs are excluded by callers."""
    y = torch.clamp(x32, -448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 0.05, 3.0])
def test_e4m3_encode_every_16bit_input(fmt, scale):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = F.e4m3_quantize_bits(bits, fmt, scale)
    x32 = torch.from_numpy(F.bits16_to_f32(bits, fmt).copy())
    y32 = x32 / torch.tensor(scale, dtype=torch.float32)   # IEEE fp32 division
    nan = torch.isnan(y32).numpy()
    ref = _torch_encode(torch.where(torch.isnan(y32), torch.zeros_like(y32), y32))
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN keeps its sign with the all-ones pattern.
    sign = np.signbit(y32.numpy()[nan])
    assert np.array_equal(got[nan], np.where(sign, 0xFF, 0x7F).astype(np.uint8))


def test_e4m3_round_trip_all_codes():
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    vals = F.e4m3_to_f64(codes)
    keep = ~np.isnan(vals)
    back = F.e4m3_encode_f32(vals[keep].astype(np.float32))
    assert np.array_equal(back, codes[keep])


def test_16bit_decode_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy())
    for fmt, dt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        ref = t.view(dt).to(torch.float64).numpy()
        got = F.kv_bits_to_f64(bits, fmt)
        nan = np.isnan(ref)
        assert np.array_equal(nan, np.isnan(got))
        assert np.array_equal(ref[~nan], got[~nan])


def test_fp8_scale_applied_in_dequant():
    codes = np.array([0x38, 0xB8, 0x7E], np.uint8)
    assert np.array_equal(F.kv_bits_to_f64(codes, "e4m3", 0.05), np.array([0.05, -0.05, 448 * 0.05]))


# ---- E5M2 ----------------------------------------------------------------

def test_e5m2_decode_golden():
    for code_s, val_s in _read_table("e5m2_codes.txt"):
        code = int(code_s, 16)
        got = F.e5m2_to_f64(np.array([code], np.uint8))[0]
        want = float(val_s)
        if math.isnan(want):
            assert math.isnan(got), code_s
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code_s


def test_e5m2_decode_all_codes_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e5m2).to(torch.float64).numpy()
    got = F.e5m2_to_f64(codes.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.sum(nan) == 6                       # S.11111.{01,10,11}
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_e5m2_encode_golden():
    for x_s, code_s in _read_table("e5m2_encode_cases.txt"):
        x = np.float32(float(x_s))
        got = int(F.e5m2_encode_f32(np.array([x], np.float32))[0])
        assert got == int(code_s, 16), (x_s, hex(got), code_s)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 0.05, 3.0])
def test_e5m2_encode_every_16bit_input(fmt, scale):
    """Against torch's float8_e5m2 conversion (nearest even) of the same fp32
    quotient, clamped first to +-57344 (torch itself overflows to infinity)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = F.fp8_quantize_bits(bits, fmt, "e5m2", scale)
    x32 = torch.from_numpy(F.bits16_to_f32(bits, fmt).copy())
    y32 = x32 / torch.tensor(scale, dtype=torch.float32)
    nan = torch.isnan(y32).numpy()
    y = torch.clamp(torch.where(torch.isnan(y32), torch.zeros_like(y32), y32), -57344.0, 57344.0)
    ref = y.to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(got[~nan], ref[~nan])
    sign = np.signbit(y32.numpy()[nan])
    assert np.array_equal(got[nan], np.where(sign, 0xFF, 0x7F).astype(np.uint8))


def test_e5m2_round_trip_all_finite_codes():
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    vals = F.e5m2_to_f64(codes)
    keep = np.isfinite(vals)
    back = F.e5m2_encode_f32(vals[keep].astype(np.float32))
    assert np.array_equal(back, codes[keep])


def test_per_head_scales_in_dequant():
    """[T, Hkv, D] codes with one scale per kv-head (axis 1)."""
    codes = np.full((2, 3, 4), 0x3C, np.uint8)           # E5M2 1.0 everywhere
    got = F.kv_bits_to_f64(codes, "e5m2", np.array([0.5, 2.0, 0.25]))
    assert np.array_equal(got[:, 0], np.full((2, 4), 0.5))
    assert np.array_equal(got[:, 1], np.full((2, 4), 2.0))
    assert np.array_equal(got[:, 2], np.full((2, 4), 0.25))
