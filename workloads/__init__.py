"""Seeded synthetic inputs for the paged KV-cache hot path.

This module only *draws* inputs: context lengths, physical page permutations,
block tables, slot mappings and N(0, 1) activations.  It performs none of the
attention or cache arithmetic, so both the fp64 oracle and the HIP path can
consume what it produces without sharing any of the method's code.

Workload shapes follow the block-paged FP16/FP8 KV cache with 16-token pages
and per-sequence block tables described in "Building and Deploying vllm.cpp"
(sigmablogger walkthrough, Step 3: RadixTree Prefix Caching, CLI configuration
table: ``--kv-cache-dtype`` and the block size used in the launch commands).

Conventions
-----------
* All draws happen on the CPU with ``torch.Generator`` seeded by the config
  index (or an explicit seed).  Integer "uniform in [a, b]" is inclusive.
* q, k, v are drawn N(0, 1) in fp32 and rounded to nearest-even into the
  storage dtype (fp16 or bf16).  fp8 pools are produced by the cache-write
  step from the 16-bit k/v drawn here (in fp16).
* Every page of the pool starts as a NaN sentinel so that any read of an
  unwritten slot poisons the result.
* The "fill" lists every (token, slot) pair that populates the pool: slot =
  physical_block * 16 + offset.  Shared-prefix pages are filled once.
* ``block_tables`` rows are padded with -1 past ceil(context_len / 16).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

BLOCK_SIZE = 16

# Raw NaN bit patterns used to poison unwritten pool slots.
SENTINEL_BITS = {"f16": 0x7E00, "bf16": 0x7FC0, "e4m3": 0x7F, "e5m2": 0x7F}
STORAGE_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}
ELEM_BYTES = {"f16": 2, "bf16": 2, "e4m3": 1, "e5m2": 1}
FP8 = ("e4m3", "e5m2")

# The five synthetic workloads.  Decode configs draw one query token per
# sequence; the prefill config draws query chunks over cached contexts.
CONFIGS = {
    0: dict(name="tiny_decode", kind="decode", B=4, ctx_list=[1, 7, 16, 33],
            Hq=4, Hkv=2, D=64, kv="f16", q="f16", num_blocks=64,
            scale=1.0 / 8.0, window=0),
    1: dict(name="decode_8b_bf16", kind="decode", B=32, ctx_range=(512, 4096),
            Hq=32, Hkv=8, D=128, kv="bf16", q="bf16",
            scale=1.0 / math.sqrt(128.0), window=0),
    2: dict(name="decode_long_splitk_f16", kind="decode", B=16,
            ctx_range=(16384, 32768), Hq=40, Hkv=8, D=128, kv="f16", q="f16",
            scale=1.0 / math.sqrt(128.0), window=0, partition=512),
    3: dict(name="decode_prefix_shared_fp8", kind="decode", B=128,
            shared_tokens=4096, suffix_range=(256, 4096), Hq=32, Hkv=8, D=128,
            kv="e4m3", q="f16", kv_src="f16", k_scale=0.05, v_scale=0.05,
            scale=1.0 / math.sqrt(128.0), window=0),
    4: dict(name="chunked_prefill_bf16", kind="prefill", B=64,
            qlen_range=(1, 512), cached_range=(1024, 8192), Hq=32, Hkv=8, D=128,
            kv="bf16", q="bf16", scale=1.0 / math.sqrt(128.0), window=4096),
}


@dataclasses.dataclass
class Case:
    """One synthetic batch.  Tensors are CPU torch tensors."""
    name: str
    kind: str                      # "decode" or "prefill"
    q: torch.Tensor                # decode [B, Hq, D]; prefill [sumQ, Hq, D]
    q_dtype: str                   # "f16" | "bf16"
    kv_dtype: str                  # "f16" | "bf16" | "e4m3" | "e5m2"
    kv_src_dtype: str              # dtype of fill_k / fill_v ("f16" | "bf16")
    num_blocks: int
    num_kv_heads: int
    head_dim: int
    fill_k: torch.Tensor           # [T, Hkv, D] 16-bit
    fill_v: torch.Tensor
    fill_slots: torch.Tensor       # [T] int64
    block_tables: torch.Tensor     # [B, max_blocks] int32, -1 padded
    context_lens: torch.Tensor     # [B] int32 (includes the query tokens)
    scale: float
    window: int
    k_scale: object = 1.0          # FP8: a number, or a tuple of Hkv per-head scales
    v_scale: object = 1.0
    query_start_loc: Optional[torch.Tensor] = None   # prefill [B+1] int32
    max_query_len: int = 1
    partition: int = 0
    # The per-step new token of each decode sequence (its last position):
    # rows of fill_k / fill_v re-written by a decode step.
    step_rows: Optional[torch.Tensor] = None          # [B] int64 rows of fill
    # For each sequence, the rows of fill_k / fill_v holding its positions
    # 0 .. n-1 in order (lets a checker rebuild K/V without the tables).
    seq_rows: Optional[list] = None

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.numel())

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[1])

    def sentinel_pool(self) -> torch.Tensor:
        """A fresh pool [num_blocks, Hkv, 16, D] of raw sentinel bits
        (int16 for 16-bit formats, uint8 for fp8)."""
        shape = (self.num_blocks, self.num_kv_heads, BLOCK_SIZE, self.head_dim)
        bits = SENTINEL_BITS[self.kv_dtype]
        if self.kv_dtype in FP8:
            return torch.full(shape, bits, dtype=torch.uint8)
        return torch.full(shape, bits, dtype=torch.int16)


def _scale(x):
    """A per-tensor FP8 scale (number) or per-kv-head scales (a sequence)."""
    if isinstance(x, (list, tuple)):
        return tuple(float(v) for v in x)
    return float(x)


def _uniform_int(gen: torch.Generator, lo: int, hi: int, n: int) -> torch.Tensor:
    return torch.randint(lo, hi + 1, (n,), generator=gen, dtype=torch.int64)


def _normal(gen: torch.Generator, shape, dtype: str) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    return x.to(STORAGE_TORCH[dtype])


def _tables_from_pages(pages_per_seq, perm, max_blocks):
    """Consecutive slices of one permutation become each sequence's table."""
    B = len(pages_per_seq)
    bt = torch.full((B, max_blocks), -1, dtype=torch.int32)
    cursor = 0
    for s, npg in enumerate(pages_per_seq):
        bt[s, :npg] = perm[cursor:cursor + npg].to(torch.int32)
        cursor += npg
    return bt, cursor


def _slots_for(bt_row: torch.Tensor, positions: torch.Tensor) -> torch.Tensor:
    blk = bt_row.to(torch.int64)[positions // BLOCK_SIZE]
    return blk * BLOCK_SIZE + positions % BLOCK_SIZE


def make_case(idx: int, seed: Optional[int] = None, **over) -> Case:
    """Draw config ``idx`` (0..4).  Keyword overrides shrink or reshape it
    (e.g. ``B=4, ctx_range=(100, 300)``) for tests that must finish fast."""
    cfg = dict(CONFIGS[idx])
    cfg.update(over)
    gen = torch.Generator().manual_seed(idx if seed is None else seed)
    if cfg["kind"] == "decode":
        if "shared_tokens" in cfg and cfg.get("shared_tokens"):
            return _make_shared(cfg, gen)
        return _make_decode(cfg, gen)
    return _make_prefill(cfg, gen)


def _draw_ctx(cfg, gen):
    if "ctx_list" in cfg:
        return torch.tensor(cfg["ctx_list"], dtype=torch.int64)
    lo, hi = cfg["ctx_range"]
    return _uniform_int(gen, lo, hi, cfg["B"])


def _make_decode(cfg, gen) -> Case:
    B, Hq, Hkv, D = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    ctx = _draw_ctx(cfg, gen)
    pages = [(int(n) + BLOCK_SIZE - 1) // BLOCK_SIZE for n in ctx]
    total_pages = sum(pages)
    num_blocks = max(cfg.get("num_blocks", total_pages), total_pages)
    perm = torch.randperm(num_blocks, generator=gen)
    max_blocks = cfg.get("max_blocks", max(pages))
    bt, _ = _tables_from_pages(pages, perm, max_blocks)
    src = cfg.get("kv_src", cfg["kv"])
    q = _normal(gen, (B, Hq, D), cfg["q"])
    T = int(ctx.sum())
    fill_k = _normal(gen, (T, Hkv, D), src)
    fill_v = _normal(gen, (T, Hkv, D), src)
    slots, step_rows, seq_rows, cur = [], [], [], 0
    for s in range(B):
        n = int(ctx[s])
        slots.append(_slots_for(bt[s], torch.arange(n)))
        step_rows.append(cur + n - 1)
        seq_rows.append(torch.arange(cur, cur + n))
        cur += n
    return Case(name=cfg["name"], kind="decode", q=q, q_dtype=cfg["q"],
                kv_dtype=cfg["kv"], kv_src_dtype=src, num_blocks=num_blocks,
                num_kv_heads=Hkv, head_dim=D, fill_k=fill_k, fill_v=fill_v,
                fill_slots=torch.cat(slots), block_tables=bt,
                context_lens=ctx.to(torch.int32), scale=float(cfg["scale"]),
                window=int(cfg.get("window", 0)),
                k_scale=_scale(cfg.get("k_scale", 1.0)),
                v_scale=_scale(cfg.get("v_scale", 1.0)),
                partition=int(cfg.get("partition", 0)),
                step_rows=torch.tensor(step_rows, dtype=torch.int64),
                seq_rows=seq_rows)


def _make_shared(cfg, gen) -> Case:
    """Every table starts with the same shared physical pages (a prefix hit
    bound to existing pages), followed by private suffix pages."""
    B, Hq, Hkv, D = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    shared = int(cfg["shared_tokens"])
    assert shared % BLOCK_SIZE == 0
    shared_pages = shared // BLOCK_SIZE
    lo, hi = cfg["suffix_range"]
    suffix = _uniform_int(gen, lo, hi, B)
    ctx = suffix + shared
    suf_pages = [(int(x) + BLOCK_SIZE - 1) // BLOCK_SIZE for x in suffix]
    num_blocks = shared_pages + sum(suf_pages)
    perm = torch.randperm(num_blocks, generator=gen)
    shared_ids = perm[:shared_pages].to(torch.int32)
    max_blocks = cfg.get("max_blocks", shared_pages + max(suf_pages))
    bt = torch.full((B, max_blocks), -1, dtype=torch.int32)
    cursor = shared_pages
    for s in range(B):
        bt[s, :shared_pages] = shared_ids
        bt[s, shared_pages:shared_pages + suf_pages[s]] = \
            perm[cursor:cursor + suf_pages[s]].to(torch.int32)
        cursor += suf_pages[s]
    src = cfg.get("kv_src", cfg["kv"])
    q = _normal(gen, (B, Hq, D), cfg["q"])
    T = shared + int(suffix.sum())
    fill_k = _normal(gen, (T, Hkv, D), src)
    fill_v = _normal(gen, (T, Hkv, D), src)
    slots = [_slots_for(bt[0], torch.arange(shared))]
    step_rows, seq_rows, cur = [], [], shared
    for s in range(B):
        pos = torch.arange(shared, int(ctx[s]))
        slots.append(_slots_for(bt[s], pos))
        seq_rows.append(torch.cat([torch.arange(shared), torch.arange(cur, cur + pos.numel())]))
        cur += pos.numel()
        step_rows.append(cur - 1)
    return Case(name=cfg["name"], kind="decode", q=q, q_dtype=cfg["q"],
                kv_dtype=cfg["kv"], kv_src_dtype=src, num_blocks=num_blocks,
                num_kv_heads=Hkv, head_dim=D, fill_k=fill_k, fill_v=fill_v,
                fill_slots=torch.cat(slots), block_tables=bt,
                context_lens=ctx.to(torch.int32), scale=float(cfg["scale"]),
                window=int(cfg.get("window", 0)),
                k_scale=_scale(cfg.get("k_scale", 1.0)),
                v_scale=_scale(cfg.get("v_scale", 1.0)),
                partition=int(cfg.get("partition", 0)),
                step_rows=torch.tensor(step_rows, dtype=torch.int64),
                seq_rows=seq_rows)


def _make_prefill(cfg, gen) -> Case:
    """Query chunks of length Q over C cached tokens: context_len = C + Q and
    the Q new tokens' K/V are already in the pool when attention runs."""
    B, Hq, Hkv, D = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    if "qlen_list" in cfg:
        qlen = torch.tensor(cfg["qlen_list"], dtype=torch.int64)
        cached = torch.tensor(cfg["cached_list"], dtype=torch.int64)
    else:
        qlen = _uniform_int(gen, *cfg["qlen_range"], B)
        cached = _uniform_int(gen, *cfg["cached_range"], B)
    ctx = qlen + cached
    pages = [(int(n) + BLOCK_SIZE - 1) // BLOCK_SIZE for n in ctx]
    num_blocks = sum(pages)
    perm = torch.randperm(num_blocks, generator=gen)
    bt, _ = _tables_from_pages(pages, perm, cfg.get("max_blocks", max(pages)))
    src = cfg.get("kv_src", cfg["kv"])
    sumq = int(qlen.sum())
    q = _normal(gen, (sumq, Hq, D), cfg["q"])
    T = int(ctx.sum())
    fill_k = _normal(gen, (T, Hkv, D), src)
    fill_v = _normal(gen, (T, Hkv, D), src)
    slots = [_slots_for(bt[s], torch.arange(int(ctx[s]))) for s in range(B)]
    starts = torch.cumsum(ctx, 0) - ctx
    seq_rows = [torch.arange(int(starts[s]), int(starts[s]) + int(ctx[s])) for s in range(B)]
    qsl = torch.zeros(B + 1, dtype=torch.int32)
    qsl[1:] = torch.cumsum(qlen, 0).to(torch.int32)
    return Case(name=cfg["name"], kind="prefill", q=q, q_dtype=cfg["q"],
                kv_dtype=cfg["kv"], kv_src_dtype=src, num_blocks=num_blocks,
                num_kv_heads=Hkv, head_dim=D, fill_k=fill_k, fill_v=fill_v,
                fill_slots=torch.cat(slots), block_tables=bt,
                context_lens=ctx.to(torch.int32), scale=float(cfg["scale"]),
                window=int(cfg.get("window", 0)), query_start_loc=qsl,
                max_query_len=int(qlen.max()), seq_rows=seq_rows)


def raw_bits(t: torch.Tensor):
    """Raw storage bits of a CPU tensor as a numpy array (uint16 for 16-bit
    floats, uint8 for bytes, unchanged for integers)."""
    import numpy as np
    if t.dtype in (torch.float16, torch.bfloat16, torch.int16):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.contiguous().numpy()
    return t.contiguous().numpy()
