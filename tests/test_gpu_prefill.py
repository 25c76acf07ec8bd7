"""GPU parity of the MFMA chunked-prefill attention against the fp64 oracle.

Everything goes through the C ABI (the ctypes binding).  Outputs are compared
element by element with the oracle (max-abs 2e-3 fp16, 8e-3 bf16, plus half
an ulp of the output format); the
properties that the kernel's arithmetic order makes exact (page permutation,
table padding, causality) are checked bit for bit."""
import pytest
import torch

from oracle import attention as A
from workloads import make_case, raw_bits

from _util import oracle_pools
from _gpu import gpu_fill, gpu_decode, to_f64, pool_view, assert_close, DEV

pytestmark = pytest.mark.gpu

import paged_kv_cache_183_amd as P  # noqa: E402


def oracle_prefill(case, kp, vp, rows=None, window=None):
    return A.prefill(raw_bits(case.q), case.q_dtype, kp, vp, case.kv_dtype,
                     case.block_tables.numpy(), case.query_start_loc.numpy(),
                     case.context_lens.numpy(), case.scale,
                     case.window if window is None else window, rows=rows)


def run_prefill(case, kc, vc, bt=None, window=None, max_query_len=None, q=None):
    q = (case.q if q is None else q).to(DEV)
    out = torch.full_like(q, float("nan"))
    P.vllm_paged_attn_prefill(out, q, pool_view(kc, case.kv_dtype), pool_view(vc, case.kv_dtype),
                              (case.block_tables if bt is None else bt).to(DEV),
                              case.query_start_loc.to(DEV), case.context_lens.to(DEV),
                              case.max_query_len if max_query_len is None else max_query_len,
                              case.scale, case.window if window is None else window)
    return out


def check_all_rows(case, out, kp, vp, window=None):
    return assert_close(case, to_f64(out), oracle_prefill(case, kp, vp, window=window))


@pytest.mark.parametrize("window", [0, 1, 16, 33, 100, 4096])
def test_prefill_reduced(window):
    """Config 4's structure at small sizes: ragged chunks over ragged caches."""
    case = make_case(4, B=5, qlen_range=(1, 300), cached_range=(1, 600))
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    check_all_rows(case, run_prefill(case, kc, vc, window=window), kp, vp, window=window)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (4, 1), (10, 2), (64, 8), (12, 1), (3, 3)])
@pytest.mark.parametrize("qd", ["bf16", "f16"])
def test_prefill_heads_dtypes(hq, hkv, qd):
    case = make_case(4, seed=300 + hq, B=3, qlen_range=(1, 150), cached_range=(0, 300),
                     Hq=hq, Hkv=hkv, kv=qd, q=qd, window=64 if hq % 2 else 0)
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    check_all_rows(case, run_prefill(case, kc, vc), kp, vp)


@pytest.mark.parametrize("hq,hkv", [(3, 1), (14, 2), (32, 1), (128, 1), (256, 2)])
@pytest.mark.parametrize("d", [128, 64])
def test_prefill_extreme_groups(hq, hkv, d):
    """Head groups whose rows do not fill a tile by whole tokens (g = 3 and
    7: 42 and 18 tokens, 126 rows each) and large groups up to the largest
    supported, g = 128 (one token per tile); windows on half of them."""
    qd = "bf16" if d == 128 else "f16"
    case = make_case(4, seed=450 + hq + d, B=4, qlen_range=(1, 70), cached_range=(0, 250),
                     Hq=hq, Hkv=hkv, D=d, kv=qd, q=qd, window=40 if hq % 3 == 2 else 0)
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    check_all_rows(case, run_prefill(case, kc, vc), kp, vp)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (4, 1), (10, 2), (64, 8), (32, 8)])
@pytest.mark.parametrize("qd", ["bf16", "f16"])
def test_prefill_head_dim_64(hq, hkv, qd):
    """head_dim 64: ragged chunks over ragged caches, windows on odd groups."""
    case = make_case(4, seed=400 + hq, B=4, qlen_range=(1, 200), cached_range=(0, 400),
                     Hq=hq, Hkv=hkv, D=64, kv=qd, q=qd, window=100 if hq % 2 else 0,
                     scale=0.125)
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    check_all_rows(case, run_prefill(case, kc, vc), kp, vp)


def test_prefill_head_dim_64_single_token_chunks_match_decode():
    """Q = 1 at head_dim 64: prefill and decode agree with the oracle."""
    case = make_case(4, B=6, qlen_range=(1, 1), cached_range=(0, 700), window=0, D=64,
                     scale=0.125)
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    ref = A.decode(raw_bits(case.q), case.q_dtype, kp, vp, case.kv_dtype,
                   case.block_tables.numpy(), case.context_lens.numpy(), case.scale, 0)
    assert_close(case, to_f64(run_prefill(case, kc, vc)), ref, " prefill")
    assert_close(case, to_f64(gpu_decode(case, kc, vc)), ref, " decode")


@pytest.mark.fullsize("prefill4")
def test_prefill_full_size_every_row():
    """The full chunked-prefill workload (64 sequences, 16,411 query rows,
    window 4096) in the launch configuration of the benchmark: every output
    element against the oracle's reference (computed by the background oracle
    process from the same seeded inputs)."""
    import _fullsize
    case = make_case(4)
    kc, vc = gpu_fill(case)
    out = to_f64(run_prefill(case, kc, vc))
    ref = _fullsize.result("prefill4")
    assert ref.shape == out.shape
    assert_close(case, out, ref)


def test_prefill_single_token_chunks_match_oracle_decode():
    """Q = 1 everywhere: each row is a decode query; both kernels agree with
    the oracle's decode of the same sequences."""
    case = make_case(4, B=6, qlen_range=(1, 1), cached_range=(0, 700), window=0)
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    ref = A.decode(raw_bits(case.q), case.q_dtype, kp, vp, case.kv_dtype,
                   case.block_tables.numpy(), case.context_lens.numpy(), case.scale, 0)
    assert_close(case, to_f64(run_prefill(case, kc, vc)), ref, " prefill")
    assert_close(case, to_f64(gpu_decode(case, kc, vc)), ref, " decode")


def test_prefill_page_permutation_bit_identical():
    case = make_case(4, B=4, qlen_range=(20, 200), cached_range=(50, 500))
    kc, vc = gpu_fill(case)
    out = run_prefill(case, kc, vc)
    perm = torch.randperm(case.num_blocks, generator=torch.Generator().manual_seed(11))
    kc2, vc2 = torch.empty_like(kc), torch.empty_like(vc)
    kc2[perm.to(DEV)] = kc
    vc2[perm.to(DEV)] = vc
    bt = case.block_tables
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0).long()].int(), bt)
    assert torch.equal(out, run_prefill(case, kc2, vc2, bt=bt2))


def test_prefill_table_padding_never_read():
    case = make_case(4, B=4, qlen_range=(1, 100), cached_range=(1, 300), max_blocks=60)
    kc, vc = gpu_fill(case)
    out = run_prefill(case, kc, vc)
    bt = case.block_tables.clone()
    junk = torch.randint(0, case.num_blocks, bt.shape, generator=torch.Generator().manual_seed(3)).int()
    bt = torch.where(bt < 0, junk, bt)
    assert torch.equal(out, run_prefill(case, kc, vc, bt=bt))


def test_prefill_causal_perturbation():
    """Changing the K/V of position p + 1 leaves every row at position <= p
    bit-identical and changes the row at p + 1."""
    case = make_case(4, B=1, qlen_list=[90], cached_list=[150], window=0)
    kc, vc = gpu_fill(case)
    out = run_prefill(case, kc, vc)
    n = int(case.context_lens[0])
    Q = 90
    p = n - Q + 40                                   # a query position inside the chunk
    t = p + 1
    blk = int(case.block_tables[0, t // 16])
    kc2, vc2 = kc.clone(), vc.clone()
    kc2[blk, :, t % 16, :] = torch.randn(kc.shape[1], kc.shape[3]).to(torch.bfloat16).view(torch.int16).to(DEV)
    vc2[blk, :, t % 16, :] = torch.randn(vc.shape[1], vc.shape[3]).to(torch.bfloat16).view(torch.int16).to(DEV)
    out2 = run_prefill(case, kc2, vc2)
    i = p - (n - Q)                                   # chunk row of position p
    assert torch.equal(out[:i + 1], out2[:i + 1])
    assert not torch.equal(out[i + 1], out2[i + 1])


def test_prefill_empty_chunks_and_upper_bound():
    """Sequences with Q = 0, a generous max_query_len, and an empty batch."""
    case = make_case(4, B=4, qlen_list=[0, 37, 0, 130], cached_list=[100, 0, 50, 260], window=0)
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    out = run_prefill(case, kc, vc)
    check_all_rows(case, out, kp, vp)
    assert torch.equal(out, run_prefill(case, kc, vc, max_query_len=4 * case.max_query_len))
    empty = case.q[:0].to(DEV)
    P.vllm_paged_attn_prefill(torch.empty_like(empty), empty, pool_view(kc, case.kv_dtype),
                              pool_view(vc, case.kv_dtype), case.block_tables.to(DEV),
                              torch.zeros(5, dtype=torch.int32, device=DEV),
                              case.context_lens.to(DEV), 0, case.scale, 0)
    torch.cuda.synchronize()
