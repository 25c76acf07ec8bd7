"""Shared test helpers: turn a workloads.Case into the oracle's inputs."""
import numpy as np

from oracle import scatter
from oracle.formats import kv_bits_to_f64
from workloads import raw_bits


def oracle_pools(case):
    """Pools (raw bits) after the oracle's cache write of the whole fill."""
    pool0 = raw_bits(case.sentinel_pool())
    slots = case.fill_slots.numpy()
    kp = scatter.cache_write_fast(pool0, raw_bits(case.fill_k), slots,
                                  case.kv_src_dtype, case.kv_dtype, case.k_scale)
    vp = scatter.cache_write_fast(pool0, raw_bits(case.fill_v), slots,
                                  case.kv_src_dtype, case.kv_dtype, case.v_scale)
    return kp, vp


def contiguous_kv(case, s, kp=None, vp=None):
    """K/V of sequence s [n, Hkv, D] in float64 straight from the fill rows
    (never through the block tables).  For fp8 pools the fill rows are
    quantized by the oracle's codec first."""
    rows = case.seq_rows[s].numpy()
    kb, vb = raw_bits(case.fill_k)[rows], raw_bits(case.fill_v)[rows]
    if case.kv_dtype in ("e4m3", "e5m2"):
        kq = scatter.encode_rows(kb, case.kv_src_dtype, case.kv_dtype, case.k_scale)
        vq = scatter.encode_rows(vb, case.kv_src_dtype, case.kv_dtype, case.v_scale)
        return (kv_bits_to_f64(kq, case.kv_dtype, case.k_scale),
                kv_bits_to_f64(vq, case.kv_dtype, case.v_scale))
    return kv_bits_to_f64(kb, case.kv_dtype), kv_bits_to_f64(vb, case.kv_dtype)


def np_bits(t):
    return raw_bits(t)


def max_abs(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))
