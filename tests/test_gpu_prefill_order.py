"""GPU checks of the chunked prefill's tile order: the order kernel builds a
per-XCD list of tiles (sequences sorted by their longest tile, every pair's
tiles together, no empty tiles), and the tile kernel runs whatever the list
holds.  A tile missing from the list would leave its rows of ``out`` at the
NaN they start with; a list that were wrong in any other way would move rows
to the wrong query.  Every case is compared with the fp64 oracle, on batches
that take the order kernel's several code paths: more pairs than one pass of
its workgroup (1,024), sort sizes above one key per thread, kv-head counts
that do not divide by 8 (the lists of the XCDs then differ), chunks of length
0 between the others, and a batch above the 4,096 sequences the order is built
for (it runs in launch order, without a workspace)."""
import pytest
import torch

from workloads import make_case

from _util import oracle_pools
from _gpu import gpu_fill, to_f64, pool_view, assert_close, DEV
from test_gpu_prefill import oracle_prefill, run_prefill

pytestmark = pytest.mark.gpu

import paged_kv_cache_183_amd as P  # noqa: E402


def call(case, kc, vc, out, workspace=None, max_query_len=None):
    P.vllm_paged_attn_prefill(out, case.q.to(DEV), pool_view(kc, case.kv_dtype),
                              pool_view(vc, case.kv_dtype), case.block_tables.to(DEV),
                              case.query_start_loc.to(DEV), case.context_lens.to(DEV),
                              max_query_len or case.max_query_len, case.scale, case.window,
                              workspace=workspace)


def test_prefill_order_caller_workspace_matches_own():
    """A caller's workspace of exactly the reported size gives the same bits
    as the library's own; one byte less is refused before any launch.  The
    generous max_query_len (an upper bound) makes a grid of 2,256 workgroups,
    most of them empty tiles, which the order leaves out."""
    case = make_case(4, seed=51, B=9, qlen_range=(0, 200), cached_range=(0, 300), Hq=8, Hkv=2)
    mq = 3000
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    own = run_prefill(case, kc, vc, max_query_len=mq)
    assert_close(case, to_f64(own), oracle_prefill(case, kp, vp))
    assert torch.equal(own, run_prefill(case, kc, vc))      # the small grid: launch order
    n = P.vllm_paged_attn_prefill_workspace_size(case.num_seqs, case.num_q_heads,
                                                 case.num_kv_heads, mq)
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    out = torch.full_like(own, float("nan"))
    call(case, kc, vc, out, workspace=ws, max_query_len=mq)
    assert torch.equal(out, own)
    # a second call reuses the workspace as it was left
    out2 = torch.full_like(own, float("nan"))
    call(case, kc, vc, out2, workspace=ws, max_query_len=mq)
    assert torch.equal(out2, own)
    small = torch.empty(n - 1, dtype=torch.uint8, device=DEV)
    with pytest.raises(P.VllmError) as err:
        call(case, kc, vc, torch.empty_like(own), workspace=small, max_query_len=mq)
    assert err.value.status == 4


@pytest.mark.parametrize("hkv,g", [(1, 4), (3, 2), (8, 2)])
def test_prefill_order_many_sequences(hkv, g):
    """1,500 sequences, a fifth of them with no query rows: 1,500 Hkv pairs
    (beyond one pass of the order kernel for Hkv = 3 and 8) and a sort of
    2,048 keys."""
    case = make_case(4, seed=60 + hkv, B=1500, qlen_range=(0, 40), cached_range=(0, 100),
                     Hq=g * hkv, Hkv=hkv, D=64, window=0 if hkv == 3 else 50)
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    assert P.vllm_paged_attn_prefill_workspace_size(case.num_seqs, case.num_q_heads,
                                                    case.num_kv_heads, case.max_query_len) > 0
    assert_close(case, to_f64(run_prefill(case, kc, vc)), oracle_prefill(case, kp, vp))


def test_prefill_beyond_order_limit():
    """4,100 sequences: no tile order (workspace size 0), launch order."""
    case = make_case(4, seed=70, B=4100, qlen_range=(0, 3), cached_range=(0, 30), Hq=2, Hkv=1,
                     D=64, window=0)
    assert P.vllm_paged_attn_prefill_workspace_size(case.num_seqs, case.num_q_heads,
                                                    case.num_kv_heads, case.max_query_len) == 0
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    assert_close(case, to_f64(run_prefill(case, kc, vc)), oracle_prefill(case, kp, vp))


@pytest.mark.parametrize("B", [256, 257, 4096])
def test_prefill_order_sort_forms(B):
    """256 sequences are ranked in one pass, 257 and 4,096 (the most the
    order takes) sorted bitonically (512 and 4,096 keys): every order gives
    every row its query.  Many sequences share a cost (ties broken by index);
    max_query_len = 320 (an upper bound) makes a grid of 2,560 or more
    workgroups, most tiles empty."""
    case = make_case(4, seed=80 + B, B=B, qlen_range=(0, 40), cached_range=(0, 60), Hq=4, Hkv=1,
                     D=64, window=0)
    mq = 320
    assert P.vllm_paged_attn_prefill_workspace_size(case.num_seqs, case.num_q_heads,
                                                    case.num_kv_heads, mq) > 0
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    assert_close(case, to_f64(run_prefill(case, kc, vc, max_query_len=mq)),
                 oracle_prefill(case, kp, vp))


@pytest.mark.parametrize("qd", ["bf16", "f16"])
def test_prefill_order_direct_loads(qd):
    """D = 128 with 16-bit pools (K/V loaded straight into LDS) under the tile
    order: 3 kv-heads (the XCD lists differ), a window of 50, chunks of 0 to
    100 tokens over caches of up to 300; max_query_len = 1,600 makes a grid of
    7,600 workgroups."""
    case = make_case(4, seed=90, B=100, qlen_range=(0, 100), cached_range=(0, 300), Hq=6, Hkv=3,
                     kv=qd, q=qd, window=50)
    mq = 1600
    assert P.vllm_paged_attn_prefill_workspace_size(case.num_seqs, case.num_q_heads,
                                                    case.num_kv_heads, mq) > 0
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    out = run_prefill(case, kc, vc, max_query_len=mq)
    assert_close(case, to_f64(out), oracle_prefill(case, kp, vp))
    assert torch.equal(out, run_prefill(case, kc, vc))      # the launch order, same bits


SWEEP_HEADS = [(8, 8), (16, 8), (4, 1), (12, 3), (16, 4), (6, 2), (5, 5), (16, 2)]


@pytest.mark.parametrize("seed", range(8))
def test_prefill_random_shapes(seed):
    """Seeded random metadata through whichever path and order a call takes:
    1 to 120 sequences, head groupings of 1 to 8, D = 64 or 128, bf16 or f16,
    windows of 0 to 1,000, chunks of 0 to 150 tokens over caches of 0 to 300,
    max_query_len tight or 8 or 64 times generous."""
    import numpy as np
    r = np.random.RandomState(1000 + seed)
    hq, hkv = SWEEP_HEADS[r.randint(len(SWEEP_HEADS))]
    qd = ["bf16", "f16"][r.randint(2)]
    case = make_case(4, seed=2000 + seed, B=int(r.randint(1, 121)),
                     qlen_range=(0, int(r.randint(1, 151))), cached_range=(0, int(r.randint(0, 301))),
                     Hq=hq, Hkv=hkv, D=[64, 128][r.randint(2)], kv=qd, q=qd,
                     window=[0, 16, 100, 1000][r.randint(4)])
    mq = max(case.max_query_len, 1) * [1, 8, 64][r.randint(3)]
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    assert_close(case, to_f64(run_prefill(case, kc, vc, max_query_len=mq)),
                 oracle_prefill(case, kp, vp))


@pytest.mark.parametrize("seed", range(4))
def test_prefill_random_shapes_fp8(seed):
    """The same sweep over E4M3 and E5M2 pools (register staging, codes
    converted exactly to q's format, the K scale folded into the score scale
    and the V scale into the output), with per-tensor scales."""
    import numpy as np
    from oracle import attention as A
    from workloads import raw_bits
    from _gpu import dev_scale
    r = np.random.RandomState(1100 + seed)
    hq, hkv = SWEEP_HEADS[r.randint(len(SWEEP_HEADS))]
    qd = ["bf16", "f16"][r.randint(2)]
    kv = ["e4m3", "e5m2"][r.randint(2)]
    case = make_case(4, seed=2100 + seed, B=int(r.randint(1, 121)),
                     qlen_range=(0, int(r.randint(1, 151))), cached_range=(0, int(r.randint(0, 301))),
                     Hq=hq, Hkv=hkv, D=[64, 128][r.randint(2)], kv=kv, q=qd, kv_src=qd,
                     window=[0, 16, 100, 1000][r.randint(4)])
    ks, vs = 0.05, 0.07
    mq = max(case.max_query_len, 1) * [1, 8, 64][r.randint(3)]
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    q = case.q.to(DEV)
    out = torch.full_like(q, float("nan"))
    P.vllm_paged_attn_prefill(out, q, pool_view(kc, kv), pool_view(vc, kv),
                              case.block_tables.to(DEV), case.query_start_loc.to(DEV),
                              case.context_lens.to(DEV), mq, case.scale, case.window,
                              k_scale=dev_scale(ks), v_scale=dev_scale(vs))
    ref = A.prefill(raw_bits(case.q), qd, kp, vp, kv, case.block_tables.numpy(),
                    case.query_start_loc.numpy(), case.context_lens.numpy(), case.scale,
                    case.window, np.array(ks), np.array(vs))
    assert_close(case, to_f64(out), ref)
