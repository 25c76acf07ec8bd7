"""Pins for the oracle's attention (oracle/attention.py).

* brute force: pure-Python math.exp loops over the *contiguous fill rows*
  (never the pool or block tables), agreeing to 1e-12;
* library special case: torch's scaled_dot_product_attention in float64 on
  CPU with K/V repeated per query group (identity tables, no window);
* invariants: softmax rows sum to 1; physical page permutation and shared vs
  private prefix pages give bit-identical outputs; keys outside the kept range
  (NaN sentinels, tail garbage, window) never matter; W >= n equals W = 0;
* closed forms: one key -> its value; equal keys or q = 0 -> mean of V;
  kv-head j holding v = j pins the GQA mapping;
* split-K: the log-sum-exp combine of partition triples equals the single pass;
* prefill: a one-token chunk equals decode; a causal perturbation of token
  p + 1 changes no row <= p;
* results do not depend on the worker count.
"""
import math
import os
import json

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle.formats import q_bits_to_f64
from workloads import make_case, raw_bits

from _util import oracle_pools, contiguous_kv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_decode_seq(q, K, V, scale, window):
    """Pure-Python reference for one sequence: q [Hq][D], K/V [n][Hkv][D]."""
    Hq, D = len(q), len(q[0])
    n, Hkv = len(K), len(K[0])
    g = Hq // Hkv
    lo = max(0, n - window) if window > 0 else 0
    out = []
    for h in range(Hq):
        kv = h // g
        z = []
        for t in range(lo, n):
            acc = 0.0
            for d in range(D):
                acc += q[h][d] * K[t][kv][d]
            z.append(scale * acc)
        m = max(z)
        e = [math.exp(v - m) for v in z]
        s = sum(e)
        row = [0.0] * D
        for i, t in enumerate(range(lo, n)):
            w = e[i] / s
            for d in range(D):
                row[d] += w * V[t][kv][d]
        out.append(row)
    return out


def oracle_decode(case, kp=None, vp=None, **kw):
    if kp is None:
        kp, vp = oracle_pools(case)
    args = dict(scale=case.scale, window=case.window, k_scale=case.k_scale, v_scale=case.v_scale)
    args.update(kw)
    return A.decode(raw_bits(case.q), case.q_dtype, kp, vp, case.kv_dtype,
                    case.block_tables.numpy(), case.context_lens.numpy(), **args)


SMALL = [
    (0, {}),
    (0, dict(window=5)),
    (1, dict(B=3, ctx_range=(1, 40), Hq=4, Hkv=1, D=64)),             # MQA
    (1, dict(B=2, ctx_range=(17, 48), Hq=2, Hkv=2, D=64, window=20)),   # MHA + window
    (2, dict(B=2, ctx_range=(20, 50), Hq=10, Hkv=2, D=64)),             # g = 5
    (3, dict(B=3, shared_tokens=16, suffix_range=(1, 20), Hq=4, Hkv=2, D=64)),
]


@pytest.mark.parametrize("idx,over", SMALL)
def test_decode_vs_brute_force(idx, over):
    case = make_case(idx, **over)
    out = oracle_decode(case)
    qf = q_bits_to_f64(raw_bits(case.q), case.q_dtype)
    for s in range(case.num_seqs):
        K, V = contiguous_kv(case, s)
        ref = brute_decode_seq(qf[s].tolist(), K.tolist(), V.tolist(), case.scale, case.window)
        assert np.max(np.abs(out[s] - np.array(ref))) < 1e-12


def test_decode_vs_torch_sdpa():
    """Identity tables, no window, equal lengths: torch SDPA in fp64 on CPU."""
    B, Hq, Hkv, D, n = 3, 8, 2, 64, 48
    case = make_case(1, B=B, ctx_range=(n, n), Hq=Hq, Hkv=Hkv, D=D)
    # rebuild with identity tables: pages of seq s are 3s .. 3s+2
    kp, vp = oracle_pools(case)
    bt = case.block_tables.numpy()
    ident = np.arange(B * 3, dtype=np.int32).reshape(B, 3)
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[ident.reshape(-1)] = kp[bt.reshape(-1)]
    vp2[ident.reshape(-1)] = vp[bt.reshape(-1)]
    out = A.decode(raw_bits(case.q), case.q_dtype, kp2, vp2, case.kv_dtype, ident,
                   case.context_lens.numpy(), case.scale)
    qf = torch.from_numpy(q_bits_to_f64(raw_bits(case.q), case.q_dtype))      # [B, Hq, D]
    K = torch.stack([torch.from_numpy(contiguous_kv(case, s)[0]) for s in range(B)])  # [B,n,Hkv,D]
    V = torch.stack([torch.from_numpy(contiguous_kv(case, s)[1]) for s in range(B)])
    g = Hq // Hkv
    Kr = K.permute(0, 2, 1, 3).repeat_interleave(g, dim=1).contiguous()   # [B, Hq, n, D]
    Vr = V.permute(0, 2, 1, 3).repeat_interleave(g, dim=1).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(
        qf[:, :, None, :], Kr, Vr, scale=case.scale)[:, :, 0, :]
    assert np.max(np.abs(out - ref.numpy())) < 1e-12


def test_softmax_rows_sum_to_one():
    case = make_case(1, B=4, ctx_range=(1, 300), Hq=8, Hkv=2, D=64, window=100)
    _, weights = oracle_decode(case, return_weights=True)
    for per_seq in weights:
        for p in per_seq:
            assert np.all(np.abs(p.sum(axis=1) - 1.0) < 1e-12)
            assert np.all(p >= 0)


def test_physical_page_permutation_invariance():
    case = make_case(1, B=4, ctx_range=(1, 100), Hq=8, Hkv=2, D=64)
    kp, vp = oracle_pools(case)
    out = oracle_decode(case, kp, vp)
    perm = np.random.default_rng(1).permutation(kp.shape[0])   # new id of page i
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    bt = case.block_tables.numpy()
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    out2 = A.decode(raw_bits(case.q), case.q_dtype, kp2, vp2, case.kv_dtype, bt2,
                    case.context_lens.numpy(), case.scale)
    assert np.array_equal(out, out2)


def test_shared_prefix_equals_private_copies():
    case = make_case(3, B=3, shared_tokens=32, suffix_range=(1, 30), Hq=4, Hkv=2, D=64)
    kp, vp = oracle_pools(case)
    out = oracle_decode(case, kp, vp)
    bt = case.block_tables.numpy().copy()
    shared_ids = bt[0, :2].copy()
    extra = []
    nb = kp.shape[0]
    for s in range(1, case.num_seqs):          # give every later seq private copies
        for j in range(2):
            extra.append(shared_ids[j])
            bt[s, j] = nb + len(extra) - 1
    kp2 = np.concatenate([kp, kp[np.array(extra)]])
    vp2 = np.concatenate([vp, vp[np.array(extra)]])
    out2 = A.decode(raw_bits(case.q), case.q_dtype, kp2, vp2, case.kv_dtype, bt,
                    case.context_lens.numpy(), case.scale, k_scale=case.k_scale,
                    v_scale=case.v_scale)
    assert np.array_equal(out, out2)


def test_outside_range_never_matters():
    case = make_case(1, B=3, ctx_range=(20, 60), Hq=4, Hkv=2, D=64, window=12)
    kp, vp = oracle_pools(case)
    out = oracle_decode(case, kp, vp)
    rng = np.random.default_rng(3)
    kp2, vp2 = kp.copy(), vp.copy()
    bt = case.block_tables.numpy()
    for s in range(case.num_seqs):
        n = int(case.context_lens[s])
        for t in list(range(0, n - 12)) + list(range(n, ((n + 15) // 16) * 16)):
            b, r = bt[s, t // 16], t % 16
            kp2[b, :, r, :] = rng.integers(0, 65535, size=kp2[b, :, r, :].shape)
            vp2[b, :, r, :] = 0x7E00
    bt2 = bt.copy()
    bt2[bt2 < 0] = 0                            # padding entries are never read
    out2 = A.decode(raw_bits(case.q), case.q_dtype, kp2, vp2, case.kv_dtype, bt2,
                    case.context_lens.numpy(), case.scale, window=12)
    assert np.array_equal(out, out2)
    assert np.array_equal(oracle_decode(case, kp, vp, window=0),
                          oracle_decode(case, kp, vp, window=10 ** 6))


def test_closed_forms():
    case = make_case(0)
    kp, vp = oracle_pools(case)
    out = oracle_decode(case, kp, vp)
    # ctx = 1 -> output is v_0 exactly (seq 0 of the tiny config)
    _, V0 = contiguous_kv(case, 0)
    g = case.num_q_heads // case.num_kv_heads
    for h in range(case.num_q_heads):
        assert np.array_equal(out[0, h], V0[0, h // g])
    # q = 0 -> uniform weights -> mean of V over the kept range
    q0 = np.zeros_like(raw_bits(case.q))
    out0 = A.decode(q0, case.q_dtype, kp, vp, case.kv_dtype, case.block_tables.numpy(),
                    case.context_lens.numpy(), case.scale, window=5)
    for s in range(case.num_seqs):
        _, V = contiguous_kv(case, s)
        n = V.shape[0]
        lo = max(0, n - 5)
        for h in range(case.num_q_heads):
            assert np.max(np.abs(out0[s, h] - V[lo:n, h // g].mean(axis=0))) < 1e-12
    # kv-head j holds v = j (as fp16 bits of small integers) -> head h gives h // g
    vp_j = vp.copy()
    for j in range(case.num_kv_heads):
        vp_j[:, j] = np.float16(j).view(np.uint16)
    outj = A.decode(raw_bits(case.q), case.q_dtype, kp, vp_j, case.kv_dtype,
                    case.block_tables.numpy(), case.context_lens.numpy(), case.scale)
    for h in range(case.num_q_heads):
        assert np.max(np.abs(outj[:, h] - h // g)) < 1e-12


def test_golden_closed_form_fixture():
    with open(os.path.join(GOLDEN, "decode_closed_form.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], np.float16).view(np.uint16)[None]          # [1, Hq, D]
        K = np.array(c["k"], np.float16)                                # [n, Hkv, D]
        V = np.array(c["v"], np.float16)
        n, Hkv, D = K.shape
        pool_k = np.full((1, Hkv, 16, D), 0x7E00, np.uint16)
        pool_v = pool_k.copy()
        pool_k[0, :, :n, :] = K.view(np.uint16).transpose(1, 0, 2)
        pool_v[0, :, :n, :] = V.view(np.uint16).transpose(1, 0, 2)
        out = A.decode(q, "f16", pool_k, pool_v, "f16", np.array([[0]], np.int32),
                       np.array([n]), c["scale"], window=c.get("window", 0))
        assert np.max(np.abs(out[0] - np.array(c["out"]))) < 1e-12, c["name"]


@pytest.mark.parametrize("part", [16, 32, 48, 512])
def test_splitk_lse_combine_equals_single_pass(part):
    case = make_case(2, B=3, ctx_range=(1, 200), Hq=10, Hkv=2, D=64, window=70)
    kp, vp = oracle_pools(case)
    out = oracle_decode(case, kp, vp)
    m, l, o = A.decode_partials(raw_bits(case.q), case.q_dtype, kp, vp, case.kv_dtype,
                                case.block_tables.numpy(), case.context_lens.numpy(),
                                case.scale, case.window, part)
    assert np.max(np.abs(A.lse_combine(m, l, o) - out)) < 1e-12


def test_worker_count_invariance():
    case = make_case(1, B=6, ctx_range=(1, 300), Hq=8, Hkv=2, D=64)
    kp, vp = oracle_pools(case)
    a = oracle_decode(case, kp, vp, workers=1)
    b = oracle_decode(case, kp, vp, workers=3)
    assert np.array_equal(a, b)


def brute_prefill_seq(q, K, V, scale, window):
    """Pure-Python chunked prefill for one sequence: q [Q][Hq][D]."""
    Q, n = len(q), len(K)
    out = []
    for i in range(Q):
        p = n - Q + i
        lo = max(0, p - window + 1) if window > 0 else 0
        out.append(brute_decode_seq(q[i], K[:p + 1], V[:p + 1], scale,
                                    (p + 1 - lo) if window > 0 else 0))
    return out


def oracle_prefill(case, kp=None, vp=None, **kw):
    if kp is None:
        kp, vp = oracle_pools(case)
    args = dict(scale=case.scale, window=case.window)
    args.update(kw)
    return A.prefill(raw_bits(case.q), case.q_dtype, kp, vp, case.kv_dtype,
                     case.block_tables.numpy(), case.query_start_loc.numpy(),
                     case.context_lens.numpy(), **args)


@pytest.mark.parametrize("over", [
    dict(B=3, qlen_range=(1, 6), cached_range=(3, 30), Hq=4, Hkv=2, D=64, window=0),
    dict(B=3, qlen_range=(1, 9), cached_range=(5, 40), Hq=4, Hkv=1, D=64, window=7),
])
def test_prefill_vs_brute_force(over):
    case = make_case(4, **over)
    out = oracle_prefill(case)
    qsl = case.query_start_loc.numpy()
    qf = q_bits_to_f64(raw_bits(case.q), case.q_dtype)
    for s in range(case.num_seqs):
        K, V = contiguous_kv(case, s)
        ref = brute_prefill_seq(qf[qsl[s]:qsl[s + 1]].tolist(), K.tolist(), V.tolist(),
                                case.scale, case.window)
        assert np.max(np.abs(out[qsl[s]:qsl[s + 1]] - np.array(ref))) < 1e-12


def test_prefill_worker_count_invariance():
    """Forked workers (longest sequences first) give the single process's
    result bit for bit, for all rows and for a row selection."""
    case = make_case(4, B=5, qlen_range=(1, 140), cached_range=(0, 300), Hq=8, Hkv=2, D=64,
                     window=50)
    kp, vp = oracle_pools(case)
    assert np.array_equal(oracle_prefill(case, kp, vp, workers=1),
                          oracle_prefill(case, kp, vp, workers=3))
    qsl = case.query_start_loc.numpy()
    rows = {s: [0, int(qsl[s + 1] - qsl[s]) - 1] for s in (0, 2, 4) if qsl[s + 1] > qsl[s]}
    a = oracle_prefill(case, kp, vp, rows=rows, workers=1)
    b = oracle_prefill(case, kp, vp, rows=rows, workers=2)
    assert a.keys() == b.keys() and all(np.array_equal(a[s], b[s]) for s in a)


def test_prefill_single_token_equals_decode():
    case = make_case(4, B=4, qlen_range=(1, 1), cached_range=(5, 70), Hq=8, Hkv=2, D=64, window=20)
    kp, vp = oracle_pools(case)
    pre = oracle_prefill(case, kp, vp)
    dec = A.decode(raw_bits(case.q), case.q_dtype, kp, vp, case.kv_dtype,
                   case.block_tables.numpy(), case.context_lens.numpy(), case.scale,
                   window=case.window)
    assert np.max(np.abs(pre - dec)) < 1e-12


def test_prefill_causal_perturbation():
    case = make_case(4, B=1, qlen_list=[12], cached_list=[20], Hq=4, Hkv=2, D=64, window=0)
    kp, vp = oracle_pools(case)
    base = oracle_prefill(case, kp, vp)
    n, Q = 32, 12
    bt = case.block_tables.numpy()
    for p in range(n - Q, n - 1):            # edit key/value p + 1
        t = p + 1
        kp2, vp2 = kp.copy(), vp.copy()
        kp2[bt[0, t // 16], :, t % 16, :] ^= 0x1234
        vp2[bt[0, t // 16], :, t % 16, :] ^= 0x0ABC
        out = oracle_prefill(case, kp2, vp2)
        i = p - (n - Q)
        assert np.array_equal(out[:i + 1], base[:i + 1])
        assert not np.array_equal(out[i + 1:], base[i + 1:])


def test_per_head_scales_map_to_kv_heads():
    """Decode with per-kv-head FP8 scales: the query heads of kv-head h equal
    a per-tensor decode with scale[h] (pins the head axis of the scales)."""
    import numpy as np
    from workloads import make_case, raw_bits
    from oracle import attention as A
    from oracle import scatter as S
    case = make_case(1, B=3, ctx_range=(5, 60), Hq=6, Hkv=3, kv="e5m2", q="f16", kv_src="f16")
    pool0 = raw_bits(case.sentinel_pool())
    slots = case.fill_slots.numpy()
    kp = S.cache_write_fast(pool0, raw_bits(case.fill_k), slots, "f16", "e5m2", 0.1)
    vp = S.cache_write_fast(pool0, raw_bits(case.fill_v), slots, "f16", "e5m2", 0.1)
    ks, vs = np.array([0.5, 0.1, 2.0]), np.array([0.2, 1.5, 0.05])
    args = (raw_bits(case.q), "f16", kp, vp, "e5m2", case.block_tables.numpy(),
            case.context_lens.numpy(), case.scale, 0)
    got = A.decode(*args, ks, vs)
    for h in range(3):
        ref = A.decode(*args, float(ks[h]), float(vs[h]))
        assert np.array_equal(got[:, 2 * h:2 * h + 2], ref[:, 2 * h:2 * h + 2]), h


# ---- chunked-local attention ------------------------------------------------

def brute_chunked_local_seq(q, K, V, scale, L):
    """Pure-Python chunked-local attention for one sequence: query i at
    position p = n - Q + i sees keys floor(p / L) * L .. p."""
    Q, n = len(q), len(K)
    out = []
    for i in range(Q):
        p = n - Q + i
        lo = (p // L) * L
        out.append(brute_decode_seq(q[i], K[lo:p + 1], V[lo:p + 1], scale, 0))
    return out


def oracle_chunked_local(case, L, kp=None, vp=None):
    if kp is None:
        kp, vp = oracle_pools(case)
    return A.prefill_chunked_local(raw_bits(case.q), case.q_dtype, kp, vp, case.kv_dtype,
                                   case.block_tables.numpy(), case.query_start_loc.numpy(),
                                   case.context_lens.numpy(), case.scale, L)


@pytest.mark.parametrize("L", [16, 32])
def test_chunked_local_vs_brute_force(L):
    case = make_case(4, B=3, qlen_range=(1, 40), cached_range=(1, 50), Hq=4, Hkv=2, D=64)
    out = oracle_chunked_local(case, L)
    qsl = case.query_start_loc.numpy()
    qf = q_bits_to_f64(raw_bits(case.q), case.q_dtype)
    for s in range(case.num_seqs):
        K, V = contiguous_kv(case, s)
        ref = brute_chunked_local_seq(qf[qsl[s]:qsl[s + 1]].tolist(), K.tolist(), V.tolist(),
                                      case.scale, L)
        assert np.max(np.abs(out[qsl[s]:qsl[s + 1]] - np.array(ref))) < 1e-12


def test_chunked_local_with_a_chunk_beyond_every_context_is_causal_prefill():
    case = make_case(4, B=3, qlen_range=(1, 30), cached_range=(1, 60), Hq=4, Hkv=2, D=64, window=0)
    kp, vp = oracle_pools(case)
    a = oracle_chunked_local(case, 1024, kp, vp)
    b = oracle_prefill(case, kp, vp)
    assert np.max(np.abs(a - b)) < 1e-12


def test_chunked_local_virtual_batch_is_the_same_attention():
    """Ordinary causal prefill over the plan's virtual batch (chunk-start
    contexts, gathered table slices, q rows in place) equals chunked-local
    attention computed directly from its mask."""
    for L in (16, 48):
        case = make_case(4, seed=9, B=4, qlen_range=(1, 100), cached_range=(0, 120), Hq=4, Hkv=2,
                         D=64, window=0)
        kp, vp = oracle_pools(case)
        V = case.query_start_loc[-1].item() // L + 2 * case.num_seqs
        vq, vctx, vbt = A.chunked_local_plan(case.query_start_loc.numpy(), case.context_lens.numpy(),
                                             case.block_tables.numpy(), L, V)
        got = A.prefill(raw_bits(case.q), case.q_dtype, kp, vp, case.kv_dtype, vbt, vq, vctx,
                        case.scale, 0)
        ref = oracle_chunked_local(case, L, kp, vp)
        assert np.max(np.abs(got - ref)) < 1e-12, L


def test_chunked_local_plan_small_example():
    """By hand: one sequence, 40 cached + 30 new tokens (positions 40..69),
    chunks of 32: chunk 1 holds positions 40..63 (24 rows, context 32), chunk
    2 holds 64..69 (6 rows, context 6)."""
    bt = np.array([[7, 3, 9, 5, 1, -1]], np.int32)
    vq, vctx, vbt = A.chunked_local_plan(np.array([0, 30]), np.array([70]), bt, 32, 4)
    assert vq.tolist() == [0, 24, 30, 30, 30]
    assert vctx.tolist() == [32, 6, 0, 0]
    assert vbt.tolist() == [[9, 5], [1, -1], [-1, -1], [-1, -1]]


def test_dead_pages():
    # by hand: n = 100, window 40 -> keys <= 60 dead (61 tokens) -> 3 full pages;
    # chunk 32 -> chunk start 96 -> 6 pages; both -> 6
    assert A.dead_pages([100], 40, 0).tolist() == [3]
    assert A.dead_pages([100], 0, 32).tolist() == [6]
    assert A.dead_pages([100], 40, 32).tolist() == [6]
    assert A.dead_pages([10, 0], 40, 0).tolist() == [0, 0]
    # property: no key a future query keeps lies in a dead page
    for n in range(0, 200, 7):
        for W, L in ((40, 0), (0, 32), (17, 48)):
            d = int(A.dead_pages([n], W, L)[0]) * 16
            for p in range(n, n + 100):
                lo = 0
                if W:
                    lo = max(lo, p - W + 1)
                if L:
                    lo = max(lo, (p // L) * L)
                assert lo >= d, (n, W, L, p)
