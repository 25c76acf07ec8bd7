"""Exact decoding of the KV / activation storage formats (oracle side).

* fp16: IEEE binary16; bf16: the upper 16 bits of an IEEE binary32.
* E4M3: the OCP 8-bit floating point format "E4M3" (OCP OFP8 specification,
  rev. 1.0): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
  infinities, a single NaN mantissa pattern S.1111.111, largest finite
  magnitude S.1111.110 = 448, subnormals 2^-6 * m/8.  The pages name FP8
  E4M3/E5M2 block-paged KV allocation ("Building and Deploying vllm.cpp",
  Step 6: Status of TurboQuant Support, native KV precision column) and
  state that fp8 pages hold one byte per element (Step 3, CLI configuration
  table, ``--kv-cache-dtype``).

* E5M2: the OCP format "E5M2" of the same specification: 1 sign bit, 5
  exponent bits with bias 15, 2 mantissa bits, IEEE-style infinities
  (S.11111.00) and NaNs (S.11111.xx, xx != 0), largest finite magnitude
  S.11110.11 = 57344, subnormals 2^-14 * m/4.

Encoding rule (the plainest reading; the pages do not fix rounding): the
16-bit input is converted exactly to fp32, divided by the fp32 scale with one
correctly-rounded IEEE division, saturated to the largest finite magnitude
(448 for E4M3, 57344 for E5M2; infinities included, so a cache never turns a
finite input into an infinity), then rounded to the nearest representable
value with ties going to the even code; NaN becomes 0x7F with the input's
sign (a NaN code in both formats); a zero result keeps the input's sign.

Scales: one fp32 scale per tensor, or one per kv-head (an array of Hkv
values applied along the head axis of [.., Hkv, .., D] arrays).

This file is test infrastructure (see the package docstring).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E5M2_MAX = 57344.0
FP8_FORMATS = ("e4m3", "e5m2")


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact): bf16 is the top half of fp32."""
    wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(all="ignore"):
        return wide.view(np.float32).astype(np.float64)


def bits16_to_f32(bits: np.ndarray, fmt: str) -> np.ndarray:
    """16-bit storage bits -> float32, exactly (both formats embed in fp32)."""
    if fmt == "f16":
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)
    if fmt == "bf16":
        wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32)
    raise ValueError(fmt)


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code, straight from the format definition."""
    s = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (2.0 ** -6) * (m / 8.0)
    return s * (2.0 ** (e - 7)) * (1.0 + m / 8.0)


# All 256 code values, built one by one from the definition above.
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes -> float64 (exact)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


# Non-negative finite magnitudes, ascending: codes 0x00 .. 0x7E.
_POS_VALUES = E4M3_TABLE[:0x7F]


def e4m3_encode_f32(y: np.ndarray) -> np.ndarray:
    """float32 values -> E4M3 codes: saturate to +-448, nearest, ties-to-even.

    Nearest is decided against the exact midpoint of the two neighbouring
    representable magnitudes (midpoints of E4M3 values are exact in fp64)."""
    y = np.asarray(y, dtype=np.float32)
    sign = np.signbit(y).astype(np.uint8) << np.uint8(7)
    a = np.abs(y.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))      # inf -> 448
    hi_idx = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi_idx = np.minimum(hi_idx, 0x7E)
    lo_idx = np.maximum(hi_idx - 1, 0)
    lo_v, hi_v = _POS_VALUES[lo_idx], _POS_VALUES[hi_idx]
    mid = (lo_v + hi_v) / 2.0
    exact = hi_v == a
    pick_hi = np.where(a > mid, True, np.where(a < mid, False, (hi_idx % 2) == 0))
    code = np.where(exact | pick_hi, hi_idx, lo_idx).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    return (code | sign).astype(np.uint8)


def e4m3_quantize_bits(bits: np.ndarray, fmt: str, scale: float) -> np.ndarray:
    """16-bit input bits -> E4M3 codes of (x / scale), with the rule above."""
    x = bits16_to_f32(bits, fmt)
    with np.errstate(all="ignore"):
        y = x / np.float32(scale)        # one IEEE fp32 division
    return e4m3_encode_f32(y)


def e5m2_value(code: int) -> float:
    """Value of one E5M2 code, straight from the format definition."""
    s = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 2) & 0x1F
    m = code & 0x3
    if e == 0x1F:
        return s * float("inf") if m == 0 else float("nan")
    if e == 0:
        return s * (2.0 ** -14) * (m / 4.0)
    return s * (2.0 ** (e - 15)) * (1.0 + m / 4.0)


E5M2_TABLE = np.array([e5m2_value(c) for c in range(256)], dtype=np.float64)
_POS_VALUES_E5M2 = E5M2_TABLE[:0x7C]        # finite non-negative magnitudes 0x00 .. 0x7B


def e5m2_to_f64(codes: np.ndarray) -> np.ndarray:
    """E5M2 codes -> float64 (exact)."""
    return E5M2_TABLE[np.asarray(codes, dtype=np.uint8)]


def _encode_sat_rne(y: np.ndarray, pos_values: np.ndarray, vmax: float) -> np.ndarray:
    """float32 values -> codes of a sign-magnitude 8-bit format whose finite
    non-negative magnitudes are ``pos_values`` (ascending, code = index):
    saturate to +-vmax, nearest, ties to the even code, NaN -> 0x7F."""
    y = np.asarray(y, dtype=np.float32)
    sign = np.signbit(y).astype(np.uint8) << np.uint8(7)
    a = np.abs(y.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, vmax))
    top = len(pos_values) - 1
    hi_idx = np.minimum(np.searchsorted(pos_values, a, side="left"), top)
    lo_idx = np.maximum(hi_idx - 1, 0)
    lo_v, hi_v = pos_values[lo_idx], pos_values[hi_idx]
    mid = (lo_v + hi_v) / 2.0
    exact = hi_v == a
    pick_hi = np.where(a > mid, True, np.where(a < mid, False, (hi_idx % 2) == 0))
    code = np.where(exact | pick_hi, hi_idx, lo_idx).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    return (code | sign).astype(np.uint8)


def e5m2_encode_f32(y: np.ndarray) -> np.ndarray:
    """float32 values -> E5M2 codes: saturate to +-57344, nearest, ties-to-even."""
    return _encode_sat_rne(y, _POS_VALUES_E5M2, E5M2_MAX)


def fp8_quantize_bits(bits: np.ndarray, src_fmt: str, fp8_fmt: str, scale: float) -> np.ndarray:
    """16-bit input bits -> FP8 codes of (x / scale), with the rule above."""
    x = bits16_to_f32(bits, src_fmt)
    with np.errstate(all="ignore"):
        y = x / np.float32(scale)        # one IEEE fp32 division
    if fp8_fmt == "e4m3":
        return e4m3_encode_f32(y)
    if fp8_fmt == "e5m2":
        return e5m2_encode_f32(y)
    raise ValueError(fp8_fmt)


def scale_along_heads(scale, ndim: int, head_axis: int) -> np.ndarray:
    """A per-tensor scale (number) or per-kv-head scales ([Hkv]) shaped to
    broadcast against an array of ``ndim`` dims whose heads lie on
    ``head_axis``."""
    sc = np.asarray(scale, dtype=np.float64)
    if sc.ndim == 0:
        return sc
    shape = [1] * ndim
    shape[head_axis] = sc.size
    return sc.reshape(shape)


def kv_bits_to_f64(bits: np.ndarray, fmt: str, scale=1.0, head_axis: int = 1) -> np.ndarray:
    """Pool bits -> float64 values.  fp8 pools are dequantized as
    value(code) * scale in fp64 (scale: a number, or [Hkv] along
    ``head_axis``); 16-bit pools ignore the scale."""
    if fmt == "f16":
        return f16_bits_to_f64(bits)
    if fmt == "bf16":
        return bf16_bits_to_f64(bits)
    if fmt in FP8_FORMATS:
        vals = e4m3_to_f64(bits) if fmt == "e4m3" else e5m2_to_f64(bits)
        return vals * scale_along_heads(scale, np.ndim(bits), head_axis)
    raise ValueError(fmt)


def q_bits_to_f64(bits: np.ndarray, fmt: str) -> np.ndarray:
    return kv_bits_to_f64(bits, fmt)
