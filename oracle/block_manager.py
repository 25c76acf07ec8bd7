"""Prefix-caching KV block manager (oracle side): the step before the paged
attention path, which builds each sequence's block table and the cache
write's slot mapping.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix ("Building and Deploying vllm.cpp", Step 3, "Technical
Mechanics of the Radix Cache"; the vllm.cpp repository listing, "What's
implemented", hash-based prefix-caching KV cache manager):

* a prompt is looked up in a radix trie whose nodes stand for runs of
  physical token blocks; the longest matching prefix is reused;
* a hit binds the new sequence's block table directly to the existing
  physical pages (no copy, no prefill for that part);
* when memory runs out, leaf nodes with the oldest access timestamps are
  dropped and their blocks go back to the global page pool.

Readings taken where the pages leave a step open (the plainest ones):

* Granularity: one trie node per full 16-token block.  A node is keyed by
  (parent node, its 16 token ids); the root is "no parent" (-1).  Only full
  blocks whose tokens are known are cached.
* The index behind the trie is a hash map keyed by the chain hash of the
  block's whole token prefix (Karp and Rabin's polynomial hash, modulo 2^64,
  base R, token t entering as the digit t + 1, seeded with 1).  A match is
  exact: the found block must hold the same 16 tokens and hang under the
  block matched one level up.  Cached blocks have distinct chain hashes: a
  block whose hash is already taken stays uncached.
* A new request (no tokens in the cache yet) reuses at most
  floor((len - 1) / 16) blocks, so that at least one token is computed.
* One call admits or extends a batch in request order.  Lookups see the
  index as it stood at the start of the call; insertions go in request
  order, then block order, and an insertion that finds its hash taken stops
  that request's insertions (its later blocks would hang under an uncached
  block).
* Timestamps are a caller-supplied step counter ``now``.  A block is touched
  when it is hit, allocated or released.  Eviction takes unreferenced cached
  blocks in increasing (timestamp, -depth, block id) order: a node is never
  older than its children (every touch covers a root path) and ties go to
  the deeper node, so only leaves are ever dropped.
* Free blocks sit on a stack.  Initially it holds N-1 .. 0, so the first
  allocations take 0, 1, 2, ...  Evicted blocks are pushed in increasing id
  order, then allocations pop (request order, block order).  A release
  pushes the uncached blocks of each row (request order, block order);
  cached blocks stay in the index, unreferenced and evictable.
* A call that cannot be served (more blocks needed than free plus
  evictable) changes nothing and reports status 1; metadata that do not fit
  (rows too short, token counts that disagree) report status 2.
"""
from __future__ import annotations

import numpy as np

BLOCK = 16
ROOT = -1
MASK64 = (1 << 64) - 1
HASH_BASE = 0x9E3779B97F4A7C15     # odd: 2^64 / golden ratio
HASH_SEED = 1

OK, OUT_OF_BLOCKS, BAD_METADATA = 0, 1, 2


def chain_hash(parent_hash: int, block_tokens) -> int:
    """Chain hash one block further: h * R^16 + sum (t_k + 1) R^(15 - k), mod 2^64
    (Horner's rule over the block's 16 digits)."""
    h = parent_hash
    for t in block_tokens:
        h = (h * HASH_BASE + (int(t) & 0xFFFFFFFF) + 1) & MASK64
    return h


def prefix_hashes(tokens, n_blocks: int) -> list:
    """Chain hashes of the first n_blocks full blocks of ``tokens``."""
    out, h = [], HASH_SEED
    for j in range(n_blocks):
        h = chain_hash(h, tokens[BLOCK * j:BLOCK * (j + 1)])
        out.append(h)
    return out


def ceil_blocks(n: int) -> int:
    return (n + BLOCK - 1) // BLOCK


def max_hit_blocks(new_len: int) -> int:
    """Blocks a new request of new_len tokens may reuse: one token is left
    to compute."""
    return (new_len - 1) // BLOCK


class BlockManager:
    """State of a pool of ``num_blocks`` physical blocks."""

    def __init__(self, num_blocks: int):
        N = int(num_blocks)
        self.N = N
        self.free = list(range(N - 1, -1, -1))          # stack, top = end
        self.ref = np.zeros(N, np.int64)
        self.ts = np.zeros(N, np.int64)
        self.depth = np.zeros(N, np.int64)
        self.parent = np.full(N, ROOT, np.int64)
        self.cached = np.zeros(N, bool)
        self.tokens = np.zeros((N, BLOCK), np.int64)
        self.chash = np.zeros(N, np.uint64)
        self.index: dict = {}                            # chain hash -> block

    # ---- schedule ---------------------------------------------------------
    def schedule(self, token_ids, token_start, num_computed, query_start_loc, block_tables, now):
        """Admit (num_computed[r] = 0) or extend the requests of a batch.

        Request r holds old = num_computed[r] tokens in the cache and adds
        q = query_start_loc[r+1] - query_start_loc[r]; its token ids (all
        old + q of them) are token_ids[token_start[r] : token_start[r+1]].
        Returns (status, block_tables, slot_mapping [sum q] int64,
        num_cached_tokens [B]); block_tables is a copy with entries
        ceil(old/16) .. ceil((old+q)/16) - 1 filled in."""
        tok = np.asarray(token_ids, np.int64)
        ts_ = np.asarray(token_start, np.int64)
        old = np.asarray(num_computed, np.int64)
        qsl = np.asarray(query_start_loc, np.int64)
        bt = np.array(block_tables, np.int64, copy=True)
        B = len(old)
        mb = bt.shape[1]
        sumq = int(qsl[-1]) if B else 0
        slots = np.full(sumq, -1, np.int64)
        ncached = np.zeros(B, np.int64)
        # ---- validation: nothing changes on failure
        for r in range(B):
            q = int(qsl[r + 1] - qsl[r])
            new = int(old[r]) + q
            nb_in = ceil_blocks(int(old[r]))
            if (old[r] < 0 or q < 0 or int(ts_[r + 1] - ts_[r]) != new or ceil_blocks(new) > mb
                    or any(not (0 <= bt[r, j] < self.N) for j in range(nb_in))):
                return BAD_METADATA, np.array(block_tables, np.int64), slots, ncached
        # ---- lookups against the index as it stands
        hits = []
        for r in range(B):
            seq = tok[ts_[r]:ts_[r + 1]]
            new = len(seq)
            h = 0
            if old[r] == 0 and new > 0:
                hs = prefix_hashes(seq, max_hit_blocks(new))
                prev = ROOT
                for j, c in enumerate(hs):
                    b = self.index.get(c)
                    if (b is None or self.parent[b] != prev
                            or not np.array_equal(self.tokens[b], seq[BLOCK * j:BLOCK * (j + 1)])):
                        break
                    prev = b
                    h += 1
            hits.append(h)
        hit_blocks = set()
        for r in range(B):
            if hits[r]:
                hit_blocks |= set(self._walk(tok[ts_[r]:ts_[r + 1]], hits[r]))
        need = []
        for r in range(B):
            new = int(ts_[r + 1] - ts_[r])
            need.append(ceil_blocks(new) - ceil_blocks(int(old[r])) - hits[r])
        total = sum(need)
        evictable = [b for b in range(self.N)
                     if self.cached[b] and self.ref[b] == 0 and b not in hit_blocks]
        if total > len(self.free) + len(evictable):
            return OUT_OF_BLOCKS, np.array(block_tables, np.int64), slots, ncached
        # ---- LRU eviction of unreferenced cached leaves
        E = total - len(self.free)
        if E > 0:
            order = sorted(evictable, key=self.eviction_key)
            for v in sorted(order[:E]):
                del self.index[int(self.chash[v])]
                self.cached[v] = False
                self.free.append(v)
        # ---- bind hits, allocate the rest
        for r in range(B):
            seq = tok[ts_[r]:ts_[r + 1]]
            for j, b in enumerate(self._walk(seq, hits[r])):
                bt[r, j] = b
                self.ref[b] += 1
                self.ts[b] = now
        for r in range(B):
            new = int(ts_[r + 1] - ts_[r])
            for j in range(ceil_blocks(int(old[r])) + hits[r], ceil_blocks(new)):
                b = self.free.pop()
                bt[r, j] = b
                self.ref[b] = 1
                self.ts[b] = now
                self.depth[b] = j
                self.parent[b] = bt[r, j - 1] if j > 0 else ROOT
        # ---- cache the blocks that became full, request by request
        for r in range(B):
            seq = tok[ts_[r]:ts_[r + 1]]
            new = len(seq)
            first = hits[r] if old[r] == 0 else int(old[r]) // BLOCK
            last = new // BLOCK
            if first >= last:
                continue
            if first > 0 and not self.cached[bt[r, first - 1]]:
                continue
            hs = prefix_hashes(seq, last)
            for j in range(first, last):
                c = hs[j]
                if c in self.index:
                    break
                b = int(bt[r, j])
                self.index[c] = b
                self.cached[b] = True
                self.chash[b] = np.uint64(c)
                self.tokens[b] = seq[BLOCK * j:BLOCK * (j + 1)]
                self.parent[b] = bt[r, j - 1] if j > 0 else ROOT
                self.depth[b] = j
        # ---- slot mapping of the computed tokens
        for r in range(B):
            o = int(old[r])
            start = max(o, BLOCK * hits[r])
            ncached[r] = start
            for t in range(o, o + int(qsl[r + 1] - qsl[r])):
                if t >= start:
                    slots[qsl[r] + t - o] = int(bt[r, t // BLOCK]) * BLOCK + t % BLOCK
        return OK, bt, slots, ncached

    def eviction_key(self, b):
        """Oldest first; among equal timestamps the deeper block (a leaf)
        first; then the lower id."""
        return (int(self.ts[b]), -int(self.depth[b]), b)

    def _walk(self, seq, n_blocks):
        """Blocks of the cached chain that ``seq`` matches, n_blocks deep."""
        out, prev = [], ROOT
        for c in prefix_hashes(seq, n_blocks):
            b = self.index[c]
            assert self.parent[b] == prev
            out.append(b)
            prev = b
        return out

    # ---- release ----------------------------------------------------------
    def release(self, block_tables, num_tokens, now):
        """Sequences end: each of their blocks loses one reference and is
        touched at ``now``; uncached ones go back to the free stack."""
        bt = np.asarray(block_tables, np.int64)
        for r, n in enumerate(np.asarray(num_tokens, np.int64)):
            for j in range(ceil_blocks(int(n))):
                b = int(bt[r, j])
                if not (0 <= b < self.N):
                    continue
                self.ref[b] = max(0, self.ref[b] - 1)
                self.ts[b] = now
                if not self.cached[b]:
                    self.free.append(b)

    # ---- views for comparisons ----------------------------------------------
    def snapshot(self) -> dict:
        return dict(free=list(self.free), ref=self.ref.copy(), ts=self.ts.copy(),
                    cached=self.cached.copy(), parent=self.parent.copy(), depth=self.depth.copy(),
                    tokens=self.tokens.copy(), chash=self.chash.copy(), index=dict(self.index))


__all__ = ["BlockManager", "chain_hash", "prefix_hashes", "BLOCK", "ROOT", "OK", "OUT_OF_BLOCKS",
           "BAD_METADATA", "HASH_BASE", "HASH_SEED"]
