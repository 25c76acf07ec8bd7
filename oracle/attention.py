"""fp64 oracle for attention over a block-paged KV cache.

What it computes (paged attention as in the PagedAttention paper the pages
cite, Kwon et al. 2023, and the "paged attention (block-paged KV cache)" of
the model forward in the vllm.cpp repository listing, "What's implemented"):

1. Reassemble.  Sequence s with n = context_lens[s] tokens owns logical pages
   0 .. ceil(n/16)-1; logical page j lives in physical page
   block_tables[s, j] (tables may point several sequences at the same
   physical pages -- a prefix hit binds a new sequence's block table to
   existing pages, "Building and Deploying vllm.cpp", Step 3).  Token t is
   row t % 16 of page block_tables[s, t // 16].  Table entries past
   ceil(n/16) are never read.
2. Heads.  Query head h reads kv-head h // g with g = Hq / Hkv (grouped-query
   attention, consecutive grouping).
3. Mask.  Decode: the query is the sequence's last token, position n - 1; it
   keeps keys t in [max(0, n - W), n) when the window W > 0, all n keys when
   W = 0.  Prefill: query row i of a Q-token chunk sits at position
   p = n - Q + i and keeps keys t <= p with t > p - W (W > 0).  The sliding
   window comes from the listing's local-attention section ("What's
   implemented": SlidingWindowSpec and the sliding-window operator); W keys
   including the query's own position is the plainest reading.
4. Score z_t = scale * <q, k_t>; softmax p_t = exp(z_t - max z) / sum;
   output sum_t p_t v_t.  All in float64.

Split-K: partition P covers logical tokens [P*part, P*part + P) intersected
with the kept range; it yields m_P = max z, l_P = sum exp(z - m_P) and
o_P = sum exp(z - m_P) v / l_P (empty partition: l_P = 0).  The log-sum-exp
combine M = max m_P, w_P = l_P exp(m_P - M), out = sum w_P o_P / sum w_P
reproduces the single pass exactly in real arithmetic.

This file is test infrastructure (see the package docstring).
"""
from __future__ import annotations

import multiprocessing
from concurrent.futures import ProcessPoolExecutor
from typing import Optional

import numpy as np

from .formats import kv_bits_to_f64, q_bits_to_f64

BLOCK = 16


def reassemble(pool: np.ndarray, fmt: str, scale: float, bt_row: np.ndarray, n: int) -> np.ndarray:
    """K or V of one sequence, contiguous: [n, Hkv, D] float64."""
    if n <= 0:
        return np.zeros((0,) + pool.shape[1:2] + pool.shape[3:], dtype=np.float64)
    npages = (n + BLOCK - 1) // BLOCK
    phys = np.asarray(bt_row[:npages], dtype=np.int64)
    pages = kv_bits_to_f64(pool[phys], fmt, scale)          # [npages, Hkv, 16, D]
    rows = pages.transpose(0, 2, 1, 3).reshape(npages * BLOCK, pool.shape[1], pool.shape[3])
    return rows[:n]


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """Row softmax in float64; rows that are entirely -inf give all zeros."""
    m = np.max(z, axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(z - m)
    s = np.sum(e, axis=-1, keepdims=True)
    return np.divide(e, s, out=np.zeros_like(e), where=s > 0)


def decode_window(n: int, window: int) -> tuple[int, int]:
    """Kept key range [lo, hi) of a decode query at position n - 1."""
    lo = max(0, n - window) if window > 0 else 0
    return lo, n


def _decode_one(args):
    """One sequence: q [Hq, D] f64, K/V [n, Hkv, D] f64 -> out [Hq, D]."""
    q, K, V, scale, window, want_w = args
    Hq, D = q.shape
    n, Hkv = K.shape[0], K.shape[1]
    g = Hq // Hkv
    out = np.zeros((Hq, D), dtype=np.float64)
    weights = []
    lo, hi = decode_window(n, window)
    for kv in range(Hkv):
        qg = q[kv * g:(kv + 1) * g]                       # [g, D]
        if hi <= lo:
            weights.append(np.zeros((g, 0)))
            continue
        z = scale * (qg @ K[lo:hi, kv, :].T)              # [g, n_kept]
        p = softmax_rows(z)
        out[kv * g:(kv + 1) * g] = p @ V[lo:hi, kv, :]
        weights.append(p)
    return (out, weights) if want_w else out


def _seq_args(s, q, k_pool, v_pool, kv_fmt, block_tables, context_lens, scale,
              window, k_scale, v_scale, q_fmt, want_w):
    n = int(context_lens[s])
    K = reassemble(k_pool, kv_fmt, k_scale, block_tables[s], n)
    V = reassemble(v_pool, kv_fmt, v_scale, block_tables[s], n)
    return (q_bits_to_f64(q[s], q_fmt), K, V, float(scale), int(window), want_w)


# Inputs of the current multi-process decode, inherited by forked workers.
_FORK_ARGS = None


def _decode_seq_job(s):
    return _decode_one(_seq_args(s, *_FORK_ARGS))


def decode(q: np.ndarray, q_fmt: str, k_pool: np.ndarray, v_pool: np.ndarray,
           kv_fmt: str, block_tables: np.ndarray, context_lens: np.ndarray,
           scale: float, window: int = 0, k_scale=1.0,
           v_scale=1.0, seqs: Optional[list] = None, workers: int = 1,
           return_weights: bool = False):
    """Paged decode attention.  q: raw bits [B, Hq, D]; pools: raw bits
    [num_blocks, Hkv, 16, D].  Returns float64 [len(seqs), Hq, D] (all
    sequences by default) and, if asked, the per-kv-head softmax weights.

    ``workers`` > 1 splits whole sequences over forked processes (which read
    the inputs they inherit); each sequence is computed identically, so the
    result does not depend on the worker count.
    """
    global _FORK_ARGS
    B = q.shape[0]
    seqs = list(range(B)) if seqs is None else list(seqs)
    args = (q, k_pool, v_pool, kv_fmt, block_tables, context_lens, scale, window,
            k_scale, v_scale, q_fmt, return_weights)
    if workers > 1 and len(seqs) > 1:
        _FORK_ARGS = args
        try:
            ctx = multiprocessing.get_context("fork")
            with ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
                res = list(ex.map(_decode_seq_job, seqs))
        finally:
            _FORK_ARGS = None
    else:
        res = [_decode_one(_seq_args(s, *args)) for s in seqs]
    if return_weights:
        return np.stack([r[0] for r in res]), [r[1] for r in res]
    return np.stack(res) if res else np.zeros((0,) + q.shape[1:], np.float64)


def decode_partials(q: np.ndarray, q_fmt: str, k_pool: np.ndarray, v_pool: np.ndarray,
                    kv_fmt: str, block_tables: np.ndarray, context_lens: np.ndarray,
                    scale: float, window: int, partition: int,
                    k_scale=1.0, v_scale=1.0):
    """Per-partition (m, l, o) of a decode: shapes [B, Hq, P], [B, Hq, P],
    [B, Hq, P, D] with P = ceil(max context / partition)."""
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    g = Hq // Hkv
    P = max(1, max((int(n) + partition - 1) // partition for n in context_lens))
    m = np.full((B, Hq, P), -np.inf)
    l = np.zeros((B, Hq, P))
    o = np.zeros((B, Hq, P, D))
    for s in range(B):
        n = int(context_lens[s])
        K = reassemble(k_pool, kv_fmt, k_scale, block_tables[s], n)
        V = reassemble(v_pool, kv_fmt, v_scale, block_tables[s], n)
        qs = q_bits_to_f64(q[s], q_fmt)
        lo, hi = decode_window(n, window)
        for part in range(P):
            a, b = max(lo, part * partition), min(hi, (part + 1) * partition)
            if b <= a:
                continue
            for kv in range(Hkv):
                z = scale * (qs[kv * g:(kv + 1) * g] @ K[a:b, kv, :].T)   # [g, b-a]
                mp = z.max(axis=1)
                e = np.exp(z - mp[:, None])
                lp = e.sum(axis=1)
                m[s, kv * g:(kv + 1) * g, part] = mp
                l[s, kv * g:(kv + 1) * g, part] = lp
                o[s, kv * g:(kv + 1) * g, part] = (e @ V[a:b, kv, :]) / lp[:, None]
    return m, l, o


def lse_combine(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Combine partition triples over the last partition axis."""
    M = np.max(m, axis=-1, keepdims=True)
    M = np.where(np.isfinite(M), M, 0.0)
    w = np.where(l > 0, l * np.exp(np.where(l > 0, m, 0.0) - M), 0.0)   # [..., P]
    den = w.sum(axis=-1)
    num = np.einsum("...p,...pd->...d", w, o)
    return np.divide(num, den[..., None], out=np.zeros_like(num), where=den[..., None] > 0)


def prefill_mask(n: int, Q: int, window: int) -> np.ndarray:
    """Boolean [Q, n]: query row i (position n - Q + i) keeps key t."""
    p = (n - Q + np.arange(Q))[:, None]
    t = np.arange(n)[None, :]
    keep = t <= p
    if window > 0:
        keep &= t > p - window
    return keep


def _prefill_one(args):
    qs, K, V, scale, window, rows = args          # qs [Q, Hq, D] f64
    Q, Hq, D = qs.shape
    n, Hkv = K.shape[0], K.shape[1]
    g = Hq // Hkv
    mask = prefill_mask(n, Q, window)
    rows = range(Q) if rows is None else rows
    rows = np.asarray(list(rows), dtype=np.int64)
    out = np.zeros((rows.size, Hq, D))
    for c0 in range(0, rows.size, 128):
        r = rows[c0:c0 + 128]
        for kv in range(Hkv):
            # the (row, head) pairs of this kv-head as the rows of one product
            qg = qs[r, kv * g:(kv + 1) * g, :].reshape(r.size * g, D)
            z = scale * (qg @ K[:, kv, :].T)                      # [r * g, n]
            z = np.where(np.repeat(mask[r], g, axis=0), z, -np.inf)
            p = softmax_rows(z)
            out[c0:c0 + r.size, kv * g:(kv + 1) * g] = (p @ V[:, kv, :]).reshape(r.size, g, D)
    return out


def _prefill_job_args(s, q, q_fmt, k_pool, v_pool, kv_fmt, block_tables, query_start_loc,
                      context_lens, scale, window, k_scale, v_scale, rows):
    a, b = int(query_start_loc[s]), int(query_start_loc[s + 1])
    n = int(context_lens[s])
    K = reassemble(k_pool, kv_fmt, k_scale, block_tables[s], n)
    V = reassemble(v_pool, kv_fmt, v_scale, block_tables[s], n)
    return (q_bits_to_f64(q[a:b], q_fmt), K, V, float(scale), int(window),
            None if rows is None else rows[s])


# Inputs of the current multi-process prefill, inherited by forked workers.
_FORK_PREFILL = None


def _prefill_seq_job(s):
    return _prefill_one(_prefill_job_args(s, *_FORK_PREFILL))


def prefill(q: np.ndarray, q_fmt: str, k_pool: np.ndarray, v_pool: np.ndarray,
            kv_fmt: str, block_tables: np.ndarray, query_start_loc: np.ndarray,
            context_lens: np.ndarray, scale: float, window: int = 0,
            k_scale=1.0, v_scale=1.0,
            rows: Optional[dict] = None, workers: int = 1) -> np.ndarray:
    """Chunked-prefill attention.  q: raw bits [sumQ, Hq, D].  Returns float64
    [sumQ, Hq, D]; with ``rows`` = {seq: [row indices within the chunk]} only
    those rows are computed and returned in a dict {seq: [len, Hq, D]}.

    ``workers`` > 1 splits whole sequences over forked processes (which read
    the inputs they inherit); each sequence is computed identically, so the
    result does not depend on the worker count."""
    global _FORK_PREFILL
    B = len(context_lens)
    seqs = list(range(B)) if rows is None else sorted(rows)
    args = (q, q_fmt, k_pool, v_pool, kv_fmt, block_tables, query_start_loc, context_lens,
            scale, window, k_scale, v_scale, rows)
    if workers > 1 and len(seqs) > 1:
        _FORK_PREFILL = args
        try:
            ctx = multiprocessing.get_context("fork")
            with ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
                # longest sequences first: the pool's last jobs are short ones
                order = sorted(seqs, key=lambda j: -int(query_start_loc[j + 1] - query_start_loc[j])
                               * int(context_lens[j]))
                done = dict(zip(order, ex.map(_prefill_seq_job, order)))
            res = [done[j] for j in seqs]
        finally:
            _FORK_PREFILL = None
    else:
        res = [_prefill_one(_prefill_job_args(j, *args)) for j in seqs]
    if rows is not None:
        return dict(zip(seqs, res))
    return np.concatenate(res, axis=0) if res else np.zeros(q.shape, np.float64)


# ---- chunked-local attention -------------------------------------------------
#
# Local attention in fixed chunks of L tokens (the local-attention section of
# the vllm.cpp repository listing, "What's implemented": a chunked-local
# attention spec, exact virtual Q/K batches and a reusable block-table
# gather/update plan): the query at position p attends to keys t <= p with
# floor(t / L) == floor(p / L), i.e. t in [floor(p / L) * L, p].


def chunked_local_mask(n: int, Q: int, L: int) -> np.ndarray:
    """Boolean [Q, n]: query row i (position n - Q + i) keeps key t."""
    p = (n - Q + np.arange(Q))[:, None]
    t = np.arange(n)[None, :]
    return (t <= p) & (t >= (p // L) * L)


def prefill_chunked_local(q: np.ndarray, q_fmt: str, k_pool: np.ndarray, v_pool: np.ndarray,
                          kv_fmt: str, block_tables: np.ndarray, query_start_loc: np.ndarray,
                          context_lens: np.ndarray, scale: float, chunk: int,
                          k_scale=1.0, v_scale=1.0) -> np.ndarray:
    """Chunked-local attention of every query row (float64 [sumQ, Hq, D])."""
    B = len(context_lens)
    out = np.zeros(q.shape, np.float64)
    for s in range(B):
        a, b = int(query_start_loc[s]), int(query_start_loc[s + 1])
        if b <= a:
            continue
        n = int(context_lens[s])
        K = reassemble(k_pool, kv_fmt, k_scale, block_tables[s], n)
        V = reassemble(v_pool, kv_fmt, v_scale, block_tables[s], n)
        qs = q_bits_to_f64(q[a:b], q_fmt)
        Q, Hq, D = qs.shape
        Hkv = K.shape[1]
        g = Hq // Hkv
        mask = chunked_local_mask(n, Q, chunk)
        for kv in range(Hkv):
            qg = qs[:, kv * g:(kv + 1) * g, :].reshape(Q * g, D)
            z = scale * (qg @ K[:, kv, :].T)                      # [Q * g, n]
            z = np.where(np.repeat(mask, g, axis=0), z, -np.inf)
            out[a:b, kv * g:(kv + 1) * g] = (softmax_rows(z) @ V[:, kv, :]).reshape(Q, g, D)
    return out


def chunked_local_plan(query_start_loc, context_lens, block_tables, chunk: int, num_virtual: int):
    """The virtual batch of chunked-local attention: every (sequence, chunk)
    that holds query tokens becomes one ordinary causal sequence, in
    (sequence, chunk) order.  Its query rows are the chunk's rows of q (in
    place), its context runs from the chunk start to its last query token,
    and its block table is the slice of pages from the chunk start (padded
    with -1 to chunk / 16 entries).  Unused entries up to ``num_virtual``
    have no query rows (start = end = sumQ), context 0 and -1 tables.

    Returns (v_query_start_loc [V + 1], v_context_lens [V], v_block_tables
    [V, chunk / 16]) as int32."""
    qsl = np.asarray(query_start_loc, np.int64)
    ctx = np.asarray(context_lens, np.int64)
    bt = np.asarray(block_tables, np.int64)
    P = chunk // 16
    sumq = int(qsl[-1])
    vq = [0]
    vctx, vbt = [], []
    for s in range(len(ctx)):
        a, b = int(qsl[s]), int(qsl[s + 1])
        n = int(ctx[s])
        if b <= a:
            continue
        first = n - (b - a)                       # position of the first query token
        for c in range(first // chunk, (n - 1) // chunk + 1):
            lo, hi = max(first, c * chunk), min(n - 1, c * chunk + chunk - 1)
            rows = hi - lo + 1
            vq.append(vq[-1] + rows)
            vlen = hi + 1 - c * chunk
            vctx.append(vlen)
            row = np.full(P, -1, np.int64)
            npg = (vlen + 15) // 16
            row[:npg] = bt[s, c * P:c * P + npg]
            vbt.append(row)
    assert len(vctx) <= num_virtual
    while len(vctx) < num_virtual:
        vq.append(sumq)
        vctx.append(0)
        vbt.append(np.full(P, -1, np.int64))
    return (np.asarray(vq, np.int32), np.asarray(vctx, np.int32),
            np.asarray(vbt, np.int32).reshape(num_virtual, P))


def dead_pages(context_lens, window: int, chunk: int) -> np.ndarray:
    """Leading logical pages of each sequence that no query at position >= n
    (n = context_lens[s], the next token's position) can attend to: with a
    sliding window W, keys t <= n - W; with chunked-local attention of L,
    keys below floor(n / L) * L; the larger of the two (0 = off)."""
    out = []
    for n in np.asarray(context_lens, np.int64):
        dead = 0
        if window > 0:
            dead = max(dead, int(n) + 1 - window)
        if chunk > 0:
            dead = max(dead, (int(n) // chunk) * chunk)
        out.append(max(0, dead) // 16)
    return np.asarray(out, np.int32)


__all__ = ["reassemble", "decode", "decode_partials", "lse_combine", "prefill",
           "prefill_mask", "softmax_rows", "decode_window", "chunked_local_mask",
           "prefill_chunked_local", "chunked_local_plan", "dead_pages"]
