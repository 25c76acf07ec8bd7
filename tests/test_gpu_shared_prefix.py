"""GPU parity of decode with a batch-wide shared prefix read once against the
fp64 oracle's decode (the same definition: the shared pages are part of every
sequence's context through its block table).

Bars: element by element within the stated tolerances plus half an ulp of
the output format; properties the arithmetic order makes exact are
checked bit for bit."""
import pytest
import torch

from oracle import attention as A
from workloads import make_case, raw_bits

from _util import oracle_pools
from _gpu import gpu_fill, gpu_decode, to_f64, pool_view, assert_close, dev_scale, DEV

pytestmark = pytest.mark.gpu

import paged_kv_cache_183_amd as P  # noqa: E402


def shared_decode(case, kc, vc, shared_pages, bt=None, ctx=None, window=None, partition=0,
                  workspace=None):
    q = case.q.to(DEV)
    out = torch.full_like(q, float("nan"))
    P.vllm_paged_attn_decode_shared_prefix(
        out, q, pool_view(kc, case.kv_dtype), pool_view(vc, case.kv_dtype),
        (case.block_tables if bt is None else bt).to(DEV),
        (case.context_lens if ctx is None else ctx).to(DEV), shared_pages, case.scale,
        case.window if window is None else window, k_scale=dev_scale(case.k_scale),
        v_scale=dev_scale(case.v_scale),
        partition_size=partition, workspace=workspace)
    return out


def oracle(case, kp, vp, ctx=None, window=None, seqs=None):
    return A.decode(raw_bits(case.q), case.q_dtype, kp, vp, case.kv_dtype,
                    case.block_tables.numpy(),
                    (case.context_lens if ctx is None else ctx).numpy(), case.scale,
                    case.window if window is None else window, case.k_scale, case.v_scale,
                    seqs=seqs)


def shared_case(seed, **over):
    cfg = dict(B=6, shared_tokens=256, suffix_range=(1, 700))
    cfg.update(over)
    return make_case(3, seed=seed, **cfg)


@pytest.mark.parametrize("partition", [0, 32])
def test_shared_prefix_batch_beyond_lds_prefix(partition):
    """More sequences (2,100) than the decode keeps its page prefix for in LDS
    (2,048): in the one-grid launch the page prefix then comes from its own
    kernel first, and the prefix tiles cover 4,200 rows per kv-head."""
    case = shared_case(46, B=2100, shared_tokens=32, suffix_range=(1, 40), Hq=4, Hkv=2)
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    out = shared_decode(case, kc, vc, 2, partition=partition)
    assert_close(case, to_f64(out), oracle(case, kp, vp))


@pytest.mark.parametrize("kvq", [("e4m3", "f16"), ("e4m3", "bf16"), ("f16", "f16"), ("bf16", "bf16")])
def test_shared_prefix_dtypes(kvq):
    kv, qd = kvq
    over = dict(kv=kv, q=qd, kv_src=qd if kv == "e4m3" else kv)
    if kv != "e4m3":
        over.update(k_scale=1.0, v_scale=1.0)
    case = shared_case(40, **over)
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    assert_close(case, to_f64(shared_decode(case, kc, vc, 16)), oracle(case, kp, vp))


@pytest.mark.parametrize("shared_pages", [1, 5, 33, 63, 64, 65, 127, 130])
def test_shared_prefix_lengths(shared_pages):
    """Splits of 64 pages: fewer, exactly one, one page past it, a ragged
    last split, three splits (the prefix is the first shared_pages of 130
    pages every sequence maps alike)."""
    case = shared_case(41, B=5, shared_tokens=16 * 130, suffix_range=(0, 300))
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    assert_close(case, to_f64(shared_decode(case, kc, vc, shared_pages)), oracle(case, kp, vp))


@pytest.mark.parametrize("window", [1, 7, 100, 300, 5000])
def test_shared_prefix_windows(window):
    case = shared_case(42, B=5, shared_tokens=320, suffix_range=(0, 400))
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    out = shared_decode(case, kc, vc, 20, window=window)
    assert_close(case, to_f64(out), oracle(case, kp, vp, window=window))


def test_sequences_shorter_than_the_prefix():
    """A sequence with n below the shared length keeps only its first n keys;
    n <= 0 gives a zero row."""
    case = shared_case(43, B=6, shared_tokens=512, suffix_range=(1, 200))
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    ctx = case.context_lens.clone()
    ctx[1] = 100                 # inside the first split
    ctx[2] = 300                 # inside the second split
    ctx[3] = 1
    ctx[4] = 0
    out = shared_decode(case, kc, vc, 32, ctx=ctx)
    assert torch.all(out[4] == 0)
    keep = [0, 1, 2, 3, 5]
    assert_close(case, to_f64(out)[keep], oracle(case, kp, vp, ctx=ctx, seqs=keep))


@pytest.mark.parametrize("hq,hkv", [(4, 1), (10, 2), (32, 8), (16, 16), (64, 8)])
def test_shared_prefix_head_groups(hq, hkv):
    case = shared_case(44 + hq, B=4, Hq=hq, Hkv=hkv, shared_tokens=256, suffix_range=(0, 300))
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    assert_close(case, to_f64(shared_decode(case, kc, vc, 16, partition=64)), oracle(case, kp, vp))


@pytest.mark.parametrize("kvq", [("e4m3", "f16"), ("bf16", "bf16"), ("f16", "f16")])
@pytest.mark.parametrize("hq,hkv", [(4, 1), (8, 2), (32, 8)])
def test_shared_prefix_head_dim_64(kvq, hq, hkv):
    kv, qd = kvq
    over = dict(kv=kv, q=qd, kv_src=qd if kv == "e4m3" else kv, D=64, Hq=hq, Hkv=hkv, scale=0.125)
    if kv != "e4m3":
        over.update(k_scale=1.0, v_scale=1.0)
    case = shared_case(60 + hq, B=5, shared_tokens=16 * 20, suffix_range=(0, 400), **over)
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    for sp, part in ((20, 0), (7, 64), (1, 0)):
        assert_close(case, to_f64(shared_decode(case, kc, vc, sp, partition=part)),
                     oracle(case, kp, vp), f" shared pages {sp}")


def test_zero_shared_pages_is_plain_decode():
    case = shared_case(45)
    kc, vc = gpu_fill(case)
    assert torch.equal(shared_decode(case, kc, vc, 0), gpu_decode(case, kc, vc))


def test_other_sequences_prefix_entries_not_read():
    """Only sequence 0's table is read for the shared pages: junk in the
    others' first entries changes nothing, bit for bit."""
    case = shared_case(46, shared_tokens=256)
    kc, vc = gpu_fill(case)
    out = shared_decode(case, kc, vc, 16)
    bt = case.block_tables.clone()
    bt[1:, :16] = -7
    assert torch.equal(out, shared_decode(case, kc, vc, 16, bt=bt))


def test_workspace_caller_and_internal_identical():
    case = shared_case(47)
    kc, vc = gpu_fill(case)
    n = P.vllm_paged_attn_shared_prefix_workspace_size(case.num_seqs, case.num_q_heads,
                                                       case.num_kv_heads, case.head_dim,
                                                       case.block_tables.shape[1], 16, 0)
    assert n > 0
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=DEV)    # garbage: no init needed
    a = shared_decode(case, kc, vc, 16, workspace=ws)
    b = shared_decode(case, kc, vc, 16)
    assert torch.equal(a, b)


@pytest.mark.fullsize("decode3")
def test_full_size_prefix_shared_fp8():
    """The full prefix-shared workload (128 sequences, 256 shared pages, FP8)
    in the launch configuration of the benchmark: every output element
    against the oracle's decode reference (computed by the background oracle
    process from the same seeded inputs)."""
    import _fullsize
    case = make_case(3)
    kc, vc = gpu_fill(case)
    out = to_f64(shared_decode(case, kc, vc, 256))
    ref = _fullsize.result("decode3")
    assert ref.shape == out.shape
    assert_close(case, out, ref)


def test_many_whole_units_in_one_chunk():
    """Short private suffixes and long chunks: several units end inside one
    chunk, each needing its own partial next to the shared-prefix ones."""
    case = shared_case(48, B=8, shared_tokens=256, suffix_range=(1, 40))
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    for part in (1024, 256, 16):
        assert_close(case, to_f64(shared_decode(case, kc, vc, 16, partition=part)),
                     oracle(case, kp, vp), f" partition {part}")


SP_HEADS = [(4, 1), (8, 2), (32, 8), (10, 2), (16, 16), (40, 8), (24, 3)]


@pytest.mark.parametrize("seed", range(8))
def test_shared_prefix_random_shapes(seed):
    """Seeded random shared-prefix batches: 1 to 60 sequences, prefixes of 1
    to 130 pages with the shared part passed as a random count of them,
    suffixes of 0 to 500 tokens, head groups of 1 to 8, D = 64 or 128, all
    four pool formats, windows of 0 to 3,000, automatic or fixed splits."""
    import numpy as np
    r = np.random.RandomState(5000 + seed)
    hq, hkv = SP_HEADS[r.randint(len(SP_HEADS))]
    kv = ["f16", "bf16", "e4m3", "e5m2"][r.randint(4)]
    qd = kv if kv in ("f16", "bf16") else ["f16", "bf16"][r.randint(2)]
    pages = int(r.randint(1, 131))
    over = dict(B=int(r.randint(1, 61)), shared_tokens=16 * pages,
                suffix_range=(0, int(r.randint(1, 501))), Hq=hq, Hkv=hkv,
                D=[64, 128][r.randint(2)], kv=kv, q=qd,
                kv_src=qd if kv in ("e4m3", "e5m2") else kv,
                window=[0, 0, 50, 700, 3000][r.randint(5)])
    if kv in ("f16", "bf16"):
        over.update(k_scale=1.0, v_scale=1.0)
    case = shared_case(6000 + seed, **over)
    shared = int(r.randint(1, pages + 1))
    part = [0, 0, 32, 512][r.randint(4)]
    kc, vc = gpu_fill(case)
    kp, vp = oracle_pools(case)
    assert_close(case, to_f64(shared_decode(case, kc, vc, shared, partition=part)),
                 oracle(case, kp, vp))
