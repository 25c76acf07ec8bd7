"""The allocation-free decode (vllm_paged_attn_decode_noalloc) against the
decode with a workspace (vllm_paged_attn_decode), through the C ABI.

Both run the same kernels with the same split, so the outputs must agree bit
for bit; each is also checked against the fp64 oracle within the stated
tolerance plus half an output ulp.  Two calls in a row on the library's one
scratch array, the second with a smaller batch, show that the array needs no
clearing between calls."""
import pytest
import torch

from oracle import attention as A
from workloads import make_case, raw_bits

from _util import oracle_pools
from _gpu import gpu_fill, gpu_decode, to_f64, pool_view, assert_close, dev_scale, DEV

pytestmark = pytest.mark.gpu

import paged_kv_cache_183_amd as P  # noqa: E402


def noalloc_decode(case, kc, vc, partition=0):
    q = case.q.to(DEV)
    out = torch.full_like(q, float("nan"))
    P.vllm_paged_attn_decode_noalloc(out, q, pool_view(kc, case.kv_dtype),
                                     pool_view(vc, case.kv_dtype), case.block_tables.to(DEV),
                                     case.context_lens.to(DEV), case.scale, case.window,
                                     k_scale=dev_scale(case.k_scale),
                                     v_scale=dev_scale(case.v_scale), partition_size=partition)
    return out


def oracle(case, kp, vp):
    return A.decode(raw_bits(case.q), case.q_dtype, kp, vp, case.kv_dtype,
                    case.block_tables.numpy(), case.context_lens.numpy(), case.scale,
                    case.window, case.k_scale, case.v_scale)


def test_noalloc_matches_decode_on_two_calls():
    # first call: the full 8B-class batch (about 16 MiB of scratch)
    big = make_case(1)
    # second call: a smaller batch of another shape and dtype, with a window
    small = make_case(1, seed=77, B=3, ctx_range=(1, 700), Hq=8, Hkv=2, D=64, kv="f16", q="f16",
                      window=300)
    for case, part in ((big, 0), (small, 0), (small, 64)):
        n = P.vllm_paged_attn_workspace_size(case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                             case.head_dim, case.block_tables.shape[1], part)
        assert 0 < n <= P.binding.NOALLOC_SCRATCH_BYTES
        kc, vc = gpu_fill(case)
        got = noalloc_decode(case, kc, vc, part)
        want = gpu_decode(case, kc, vc, partition=part)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{case.name}: noalloc differs from decode"
        kp, vp = oracle_pools(case)
        assert_close(case, to_f64(got), oracle(case, kp, vp), f" noalloc partition {part}")


def test_noalloc_fp8_and_repeat():
    """FP8 pools with per-head scales; repeated calls agree bit for bit."""
    case = make_case(3, seed=78, B=5, shared_tokens=0, ctx_range=(1, 900), kv="e4m3", q="f16",
                     kv_src="f16", k_scale=(0.05, 0.04, 0.06, 0.05, 0.03, 0.05, 0.07, 0.05),
                     v_scale=0.05)
    kc, vc = gpu_fill(case)
    first = noalloc_decode(case, kc, vc)
    assert torch.equal(first, gpu_decode(case, kc, vc))
    for _ in range(3):
        assert torch.equal(noalloc_decode(case, kc, vc), first)
    kp, vp = oracle_pools(case)
    assert_close(case, to_f64(first), oracle(case, kp, vp))


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """A split that needs more than the scratch array is refused on the host
    (nothing is launched; the output keeps its contents)."""
    case = make_case(2, B=2, ctx_range=(16384, 16384))
    need = P.vllm_paged_attn_workspace_size(case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                            case.head_dim, case.block_tables.shape[1], 16)
    assert need > P.binding.NOALLOC_SCRATCH_BYTES
    q = case.q.to(DEV)
    out = torch.zeros_like(q)
    pool = torch.zeros(case.num_blocks, case.num_kv_heads, 16, case.head_dim,
                       dtype=torch.float16, device=DEV)
    with pytest.raises(P.VllmError) as ei:
        P.vllm_paged_attn_decode_noalloc(out, q, pool, pool, case.block_tables.to(DEV),
                                         case.context_lens.to(DEV), case.scale,
                                         partition_size=16)
    assert ei.value.status == P.binding.VLLM_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(out == 0))
