"""GPU: the fused newest-token cache write + decode against the two separate
calls.  Both paths compute the same thing in the same arithmetic, so the
outputs and the pools after the call are compared bit for bit; one case is
also checked against the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from workloads import make_case, raw_bits

from _gpu import gpu_fill, to_f64, pool_view, assert_close, dev_scale, bits, DEV

pytestmark = pytest.mark.gpu

import paged_kv_cache_183_amd as P  # noqa: E402


def newest(case, seed):
    """Fresh K/V rows for every sequence's last token, and their slots."""
    g = torch.Generator().manual_seed(seed)
    B, Hkv, D = case.num_seqs, case.num_kv_heads, case.head_dim
    dt = torch.float16 if case.q_dtype == "f16" else torch.bfloat16
    k = torch.randn(B, Hkv, D, generator=g).to(dt)
    v = torch.randn(B, Hkv, D, generator=g).to(dt)
    n = case.context_lens.numpy().astype(np.int64)
    bt = case.block_tables.numpy().astype(np.int64)
    slots = np.array([bt[s, (n[s] - 1) // 16] * 16 + (n[s] - 1) % 16 for s in range(B)], np.int64)
    return k, v, torch.from_numpy(slots)


def both_paths(case, window=0, partition=0, drop=()):
    k, v, slots = newest(case, 1234)
    for s in drop:
        slots[s] = -1                           # no write for this sequence
    ks, vs = dev_scale(case.k_scale), dev_scale(case.v_scale)
    q = case.q.to(DEV)
    kc1, vc1 = gpu_fill(case)
    kc2, vc2 = kc1.clone(), vc1.clone()
    bt, ctx = case.block_tables.to(DEV), case.context_lens.to(DEV)
    # separate: cache write, then decode
    P.vllm_paged_cache_write(k.to(DEV), v.to(DEV), slots.to(DEV), pool_view(kc1, case.kv_dtype),
                             pool_view(vc1, case.kv_dtype), k_scale=ks, v_scale=vs)
    out1 = torch.empty_like(q)
    P.vllm_paged_attn_decode(out1, q, pool_view(kc1, case.kv_dtype), pool_view(vc1, case.kv_dtype),
                             bt, ctx, case.scale, window, k_scale=ks, v_scale=vs,
                             partition_size=partition)
    # fused
    out2 = torch.empty_like(q)
    P.vllm_paged_attn_decode_append(out2, q, k.to(DEV), v.to(DEV), slots.to(DEV),
                                    pool_view(kc2, case.kv_dtype), pool_view(vc2, case.kv_dtype),
                                    bt, ctx, case.scale, window, k_scale=ks, v_scale=vs,
                                    partition_size=partition)
    return out1, out2, (kc1, vc1), (kc2, vc2)


CASES = {
    "bf16": dict(idx=1, B=12, ctx_range=(1, 1500)),
    "f16_d64": dict(idx=0),
    "g10": dict(idx=1, B=6, ctx_range=(1, 900), Hq=40, Hkv=4),
    "e4m3": dict(idx=3, B=8, shared_tokens=64, suffix_range=(1, 500)),
    "e5m2_heads": dict(idx=1, B=6, ctx_range=(1, 700), kv="e5m2", q="f16", kv_src="f16",
                       k_scale=(0.05, 0.3, 0.02, 0.5, 0.1, 0.07, 0.2, 0.04),
                       v_scale=(0.5, 0.05, 0.09, 0.02, 0.3, 0.07, 0.2, 0.04)),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("partition", [0, 32])
def test_fused_equals_separate(name, partition):
    kw = dict(CASES[name])
    case = make_case(kw.pop("idx"), seed=77, **kw)
    out1, out2, (k1, v1), (k2, v2) = both_paths(case, partition=partition)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert np.array_equal(bits(k1), bits(k2)) and np.array_equal(bits(v1), bits(v2))


@pytest.mark.parametrize("window", [1, 17, 300])
def test_fused_with_window_and_padding(window):
    case = make_case(1, seed=78, B=10, ctx_range=(1, 1200))
    out1, out2, (k1, v1), (k2, v2) = both_paths(case, window=window, drop=(2, 7))
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert np.array_equal(bits(k1), bits(k2)) and np.array_equal(bits(v1), bits(v2))


def test_fused_against_oracle():
    case = make_case(1, seed=79, B=8, ctx_range=(1, 1000))
    _, out2, _, (k2, v2) = both_paths(case)
    ref = A.decode(raw_bits(case.q), case.q_dtype, bits(k2), bits(v2), case.kv_dtype,
                   case.block_tables.numpy(), case.context_lens.numpy(), case.scale)
    assert_close(case, to_f64(out2), ref)


def test_fused_full_size():
    """The 8B-class batch at its full size, in the benchmark's launch."""
    case = make_case(1)
    out1, out2, (k1, v1), (k2, v2) = both_paths(case)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert np.array_equal(bits(k1), bits(k2))
