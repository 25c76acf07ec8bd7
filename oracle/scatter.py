"""Oracle for the cache write that fills the block-paged KV pool.

For every token i whose slot s = slot_mapping[i] is non-negative, the K (and
V) vector of every kv-head is written to physical page s // 16, row s % 16 of
the pool laid out [num_blocks, Hkv, 16, D].  Negative slots mark padding
tokens and are skipped.  The pages describe KV stored in fixed 16-token
physical pages and per-sequence block tables that point at them ("Building
and Deploying vllm.cpp", Step 3: technical mechanics of the radix cache and
the ``--block-size 16`` launch flags); the slot convention is the plainest
encoding of (page, row) for such a pool.

16-bit pools receive the input bits unchanged; FP8 pools (E4M3 or E5M2)
receive the code of (x / scale) by the rule in ``oracle.formats``, with one
scale per tensor or one per kv-head.

This file is test infrastructure (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .formats import FP8_FORMATS, fp8_quantize_bits

BLOCK = 16

_CODE_TABLES = {}


def fp8_code_table(src_fmt: str, fp8_fmt: str, scale: float) -> np.ndarray:
    """The FP8 code of every one of the 65,536 16-bit inputs, each computed by
    ``formats.fp8_quantize_bits``.  The input domain is finite, so encoding
    by lookup in this table is the same function, only memoized."""
    key = (src_fmt, fp8_fmt, float(np.float32(scale)))
    if key not in _CODE_TABLES:
        every = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        _CODE_TABLES[key] = fp8_quantize_bits(every, src_fmt, fp8_fmt, scale)
    return _CODE_TABLES[key]


def e4m3_code_table(src_fmt: str, scale: float) -> np.ndarray:
    return fp8_code_table(src_fmt, "e4m3", scale)


def encode_rows(bits: np.ndarray, src_fmt: str, cache_fmt: str, scale=1.0) -> np.ndarray:
    """What the pool stores for input rows ``bits`` (raw 16-bit patterns,
    [T, Hkv, D]); ``scale`` is a number or [Hkv] per-head scales."""
    if cache_fmt == src_fmt:
        return np.asarray(bits, dtype=np.uint16).copy()
    if cache_fmt in FP8_FORMATS:
        b = np.asarray(bits, dtype=np.uint16)
        sc = np.asarray(scale, dtype=np.float64)
        if sc.ndim == 0:
            return fp8_code_table(src_fmt, cache_fmt, float(sc))[b]
        out = np.empty(b.shape, dtype=np.uint8)
        for h in range(b.shape[1]):
            out[:, h] = fp8_code_table(src_fmt, cache_fmt, float(sc[h]))[b[:, h]]
        return out
    raise ValueError(f"unsupported {src_fmt} -> {cache_fmt}")


def cache_write(pool: np.ndarray, bits: np.ndarray, slots: np.ndarray,
                src_fmt: str, cache_fmt: str, scale: float = 1.0) -> np.ndarray:
    """Return a copy of ``pool`` [num_blocks, Hkv, 16, D] with token rows
    ``bits`` [T, Hkv, D] written at ``slots`` [T] (negative = skip).

    Written one token at a time, in order, exactly as the definition reads."""
    out = np.array(pool, copy=True)
    enc = encode_rows(bits, src_fmt, cache_fmt, scale)
    for i, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        out[s // BLOCK, :, s % BLOCK, :] = enc[i]
    return out


def cache_write_fast(pool: np.ndarray, bits: np.ndarray, slots: np.ndarray,
                     src_fmt: str, cache_fmt: str, scale: float = 1.0) -> np.ndarray:
    """Same result as ``cache_write`` for slot lists without duplicates, with
    one vectorised numpy assignment (used for large pools)."""
    out = np.array(pool, copy=True)
    enc = encode_rows(bits, src_fmt, cache_fmt, scale)
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    s = slots[keep]
    out[s // BLOCK, :, s % BLOCK, :] = enc[keep]
    return out
