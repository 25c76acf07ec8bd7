"""Run the HIP path (through the C ABI binding) on a workloads.Case."""
import numpy as np
import torch

import paged_kv_cache_183_amd as P
from workloads import STORAGE_TORCH

DEV = "cuda"


def pool_view(pool_bits: torch.Tensor, kv_dtype: str) -> torch.Tensor:
    """Typed view of a raw-bits pool (int16 -> f16/bf16; uint8 stays E4M3
    codes; E5M2 codes are viewed as torch.float8_e5m2)."""
    if kv_dtype == "e4m3":
        return pool_bits
    if kv_dtype == "e5m2":
        return pool_bits.view(torch.float8_e5m2)
    return pool_bits.view(STORAGE_TORCH[kv_dtype])


def dev_scale(x, dev=DEV):
    """A per-tensor scale stays a number; per-head scales become a float32
    device tensor."""
    if isinstance(x, (tuple, list)):
        return torch.tensor(x, dtype=torch.float32, device=dev)
    return x


def gpu_fill(case, dev=DEV):
    """Sentinel pools on the device, filled by the library's cache write."""
    kc = case.sentinel_pool().to(dev)
    vc = case.sentinel_pool().to(dev)
    P.vllm_paged_cache_write(case.fill_k.to(dev), case.fill_v.to(dev), case.fill_slots.to(dev),
                             pool_view(kc, case.kv_dtype), pool_view(vc, case.kv_dtype),
                             k_scale=dev_scale(case.k_scale), v_scale=dev_scale(case.v_scale))
    return kc, vc


def gpu_decode(case, kc, vc, partition=0, workspace=None, q=None, bt=None, ctx=None,
               window=None, dev=DEV):
    q = (case.q if q is None else q).to(dev)
    out = torch.empty_like(q)
    bt = (case.block_tables if bt is None else bt).to(dev)
    ctx = (case.context_lens if ctx is None else ctx).to(dev)
    P.vllm_paged_attn_decode(out, q, pool_view(kc, case.kv_dtype), pool_view(vc, case.kv_dtype),
                             bt, ctx, case.scale, case.window if window is None else window,
                             k_scale=dev_scale(case.k_scale), v_scale=dev_scale(case.v_scale),
                             partition_size=partition, workspace=workspace)
    return out


def gpu_prefill(case, kc, vc, dev=DEV):
    q = case.q.to(dev)
    out = torch.empty_like(q)
    P.vllm_paged_attn_prefill(out, q, pool_view(kc, case.kv_dtype), pool_view(vc, case.kv_dtype),
                              case.block_tables.to(dev), case.query_start_loc.to(dev),
                              case.context_lens.to(dev), case.max_query_len, case.scale,
                              case.window)
    return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.cpu().contiguous()
    if t.dtype in (torch.float16, torch.bfloat16, torch.int16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.uint8).numpy()


TOL = {"f16": 2e-3, "bf16": 8e-3, "e4m3": 3e-2, "e5m2": 3e-2}


def tol_for(case) -> float:
    return TOL[case.kv_dtype] if case.kv_dtype in ("e4m3", "e5m2") else TOL[case.q_dtype]


# Explicit mantissa bits of the 16-bit output formats.
_MANT = {"f16": 10, "bf16": 7}


def out_ulp(ref: np.ndarray, q_dtype: str) -> np.ndarray:
    """One unit in the last place of q's 16-bit format at |ref| (normal range)."""
    a = np.maximum(np.abs(ref), 2.0 ** -14)
    return np.exp2(np.floor(np.log2(a)) - _MANT[q_dtype])


def elem_bound(case, ref: np.ndarray) -> np.ndarray:
    """Per-element bar: the stated max-abs tolerance for the arithmetic plus
    half an ulp of the output format.  The kernel's fp32 result x lies within
    tol of the exact value, and the output is x rounded to nearest even in
    q's 16-bit format, which moves it by at most half an ulp at |x| <=
    |ref| + tol: rounding that no implementation of the stated output format
    can avoid."""
    tol = tol_for(case)
    return tol + 0.5 * out_ulp(np.abs(ref) + tol, case.q_dtype)


def assert_close(case, got: np.ndarray, ref: np.ndarray, what: str = "") -> float:
    """Element-by-element check against the oracle; returns the max abs error."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if not ref.size:
        return 0.0
    assert np.all(np.isfinite(got)), f"{case.name}{what}: non-finite output"
    e = np.abs(got - ref)
    bad = e > elem_bound(case, ref)
    if np.any(bad):
        i = np.unravel_index(np.argmax(np.where(bad, e, -1.0)), e.shape)
        raise AssertionError(f"{case.name}{what}: {int(bad.sum())} elements beyond the bar; "
                             f"at {tuple(int(x) for x in i)} ref {ref[i]:.6f} got {got[i]:.6f} "
                             f"(err {e[i]:.3e}, tol {tol_for(case)})")
    return float(e.max())
