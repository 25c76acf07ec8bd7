"""Pins of the oracle's prefix-caching block manager.

* A hand-derived worked example (tests/golden/block_manager_walkthrough.json).
* Brute force: the hit length of every admitted prompt is the longest cached
  token prefix, found by rebuilding every cached block's whole token prefix
  from its parent links (no hashing involved), capped so one token is left.
* Soundness: a hit block's whole prefix equals the prompt's.
* Conservation: every block is exactly one of free, referenced, or cached and
  unreferenced; reference counts equal the number of live rows holding each
  block.
* LRU: no unreferenced cached block that survives a call is older, in
  (timestamp, -depth, id) order, than one the call evicted; the cache stays
  closed under parents (only leaves are dropped).
* The chain hash equals the polynomial evaluated over the whole prefix at
  once.
* A call that cannot be served changes nothing."""
import copy
import json
import os

import numpy as np
import pytest

from oracle import block_manager as M
from workloads.requests import RequestStream

from _bm import Driver

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_manager_walkthrough.json")


def run_walkthrough(mgr, check):
    doc = json.load(open(GOLDEN))
    mb = doc["max_blocks"]
    for st in doc["steps"]:
        if st["op"] == "schedule":
            reqs = st["requests"]
            toks = np.array(sum((r["tokens"] for r in reqs), []), np.int32)
            tstart = np.cumsum([0] + [len(r["tokens"]) for r in reqs]).astype(np.int32)
            old = np.array([r["old"] for r in reqs], np.int32)
            qsl = np.cumsum([0] + [len(r["tokens"]) - r["old"] for r in reqs]).astype(np.int32)
            rows = np.full((len(reqs), mb), -1, np.int32)
            if "rows" in st:        # running requests carry their rows in
                for i, r in enumerate(reqs):
                    nb = (r["old"] + 15) // 16
                    rows[i, :nb] = st["rows"][i][:nb]
            status, bt, slots, ncached = mgr.schedule(toks, tstart, old, qsl, rows, st["now"])
            assert status == st["status"], st["why"]
            if status == 0:
                for i, row in enumerate(st["rows"]):
                    assert list(bt[i, :len(row)]) == row, st["why"]
                    assert all(x == -1 for x in bt[i, len(row):])
                assert list(slots) == st["slots"], st["why"]
                assert list(ncached) == st["num_cached"], st["why"]
        else:
            rows = np.full((len(st["rows"]), mb), -1, np.int32)
            for i, row in enumerate(st["rows"]):
                rows[i, :len(row)] = row
            mgr.release(rows, np.array(st["num_tokens"], np.int32), st["now"])
        check(mgr, st)


def test_walkthrough():
    def check(mgr, st):
        assert mgr.free == st["free_after"], st["why"]
        assert sorted(np.nonzero(mgr.cached)[0].tolist()) == st["cached_after"], st["why"]
        if "ref_after" in st:
            assert mgr.ref.tolist() == st["ref_after"], st["why"]
    run_walkthrough(M.BlockManager(6), check)


def test_chain_hash_is_the_prefix_polynomial():
    g = np.random.default_rng(0)
    for n_blocks in (1, 2, 7):
        toks = g.integers(0, 2 ** 31, 16 * n_blocks).tolist()
        hs = M.prefix_hashes(toks, n_blocks)
        for j in range(n_blocks):
            n = 16 * (j + 1)
            # seed * R^n + sum_i (t_i + 1) R^(n - 1 - i), as one big integer
            want = M.HASH_SEED * M.HASH_BASE ** n
            want += sum((t + 1) * M.HASH_BASE ** (n - 1 - i) for i, t in enumerate(toks[:n]))
            assert hs[j] == want % 2 ** 64
    # zero tokens still give distinct hashes per length
    z = M.prefix_hashes([0] * 64, 4)
    assert len(set(z)) == 4


def cached_prefixes(mgr):
    """Whole token prefix of every cached block, rebuilt from parent links."""
    out = {}
    for b in np.nonzero(mgr.cached)[0]:
        chain, x = [], int(b)
        while x != M.ROOT:
            assert mgr.cached[x], "cached block under an uncached parent"
            chain.append(x)
            x = int(mgr.parent[x])
        chain.reverse()
        assert int(mgr.depth[b]) == len(chain) - 1
        out[int(b)] = tuple(int(t) for c in chain for t in mgr.tokens[c])
    return out


def key(mgr, b):
    return (int(mgr.ts[b]), -int(mgr.depth[b]), int(b))


class Checked:
    """Wraps the oracle and checks the pins around every call."""

    def __init__(self, N, driver_ref):
        self.m = M.BlockManager(N)
        self.N = N
        self.driver = driver_ref
        self.evictions = 0
        self.hits = 0

    def release(self, rows, ntok, now):
        self.m.release(rows, ntok, now)

    def schedule(self, toks, tstart, old, qsl, rows, now):
        m = self.m
        before = copy.deepcopy(m.snapshot())
        prefixes = cached_prefixes(m)
        by_prefix = {p: b for b, p in prefixes.items()}
        res = m.schedule(toks, tstart, old, qsl, rows, now)
        status, bt, slots, ncached = res
        if status != 0:
            after = m.snapshot()
            for k in ("ref", "ts", "cached", "parent", "depth", "tokens", "chash"):
                assert np.array_equal(before[k], after[k]), k
            assert before["free"] == after["free"] and before["index"] == after["index"]
            return res
        B = len(old)
        hit_blocks = set()
        for r in range(B):
            seq = toks[tstart[r]:tstart[r + 1]].tolist()
            if old[r] == 0:
                # brute force: longest cached whole prefix, at most (len-1)//16 blocks
                best = 0
                for j in range(1, (len(seq) - 1) // 16 + 1):
                    if tuple(seq[:16 * j]) in by_prefix:
                        best = j
                    else:
                        break
                assert ncached[r] == 16 * best
                self.hits += best
                for j in range(best):
                    b = int(bt[r, j])
                    assert prefixes[b] == tuple(seq[:16 * (j + 1)])      # sound reuse
                    hit_blocks.add(b)
            else:
                assert ncached[r] == old[r]
        # slots: unique, inside the row's blocks, -1 exactly for hit tokens
        live = slots[slots >= 0]
        assert len(np.unique(live)) == len(live)
        for r in range(B):
            for t in range(int(old[r]), int(tstart[r + 1] - tstart[r])):
                s = slots[qsl[r] + t - old[r]]
                if t < ncached[r]:
                    assert s == -1
                else:
                    assert s // 16 == bt[r, t // 16] and s % 16 == t % 16
        # LRU and closure
        # (an evicted block may be allocated again and cached under a new
        # prefix in the same call: decide by the entry it had before)
        survived = lambda b: m.index.get(int(before["chash"][b])) == b  # noqa: E731
        dropped = [b for b in range(self.N) if before["cached"][b] and not survived(b)]
        if dropped:
            self.evictions += len(dropped)
            kept = [b for b in range(self.N) if before["cached"][b] and survived(b)
                    and before["ref"][b] == 0 and b not in hit_blocks]
            kb = lambda b: (int(before["ts"][b]), -int(before["depth"][b]), b)  # noqa: E731
            assert not kept or max(kb(b) for b in dropped) < min(kb(b) for b in kept)
            assert all(before["ref"][b] == 0 and b not in hit_blocks for b in dropped)
        cached_prefixes(m)                                   # asserts closure
        return res


def conservation(mgr, driver, N):
    free = mgr.free
    assert len(set(free)) == len(free)
    ref = driver.live_refs(N)
    assert np.array_equal(mgr.ref, ref)
    for b in range(N):
        states = (b in free) + (ref[b] > 0) + (bool(mgr.cached[b]) and ref[b] == 0)
        assert states == 1, b


@pytest.mark.parametrize("seed,N,mb", [(1, 64, 16), (2, 40, 12), (3, 400, 24), (4, 24, 8)])
def test_random_streams_hold_the_pins(seed, N, mb):
    stream = RequestStream(seed, vocab=50 if seed % 2 else 1000)
    chk = Checked(N, None)
    d = Driver(chk, stream, mb)
    chk.driver = d
    for _ in range(60):
        d.step()
        conservation(chk.m, d, N)
    assert chk.hits > 0
    if N <= 64:
        assert chk.evictions > 0


def test_out_of_blocks_changes_nothing():
    m = M.BlockManager(4)
    toks = np.arange(100, dtype=np.int32)
    st, bt, _, _ = m.schedule(toks[:70], [0, 70], [0], [0, 70], np.full((1, 8), -1, np.int32), 1)
    assert st == M.OUT_OF_BLOCKS and (bt == -1).all() and m.free == [3, 2, 1, 0]
    st, _, _, _ = m.schedule(toks[:64], [0, 64], [0], [0, 64], np.full((1, 8), -1, np.int32), 2)
    assert st == M.OK and m.free == []


def test_bad_metadata():
    m = M.BlockManager(8)
    rows = np.full((1, 2), -1, np.int32)
    toks = np.arange(40, dtype=np.int32)
    assert m.schedule(toks, [0, 40], [0], [0, 40], rows, 1)[0] == M.BAD_METADATA      # 3 blocks > 2
    assert m.schedule(toks, [0, 39], [0], [0, 40], np.full((1, 4), -1, np.int32), 1)[0] == M.BAD_METADATA
    assert m.schedule(toks[:20], [0, 20], [4], [0, 16], np.full((1, 4), -1, np.int32), 1)[0] == M.BAD_METADATA
    assert m.free == list(range(7, -1, -1))


def test_identical_prompts_in_one_batch_cache_once():
    m = M.BlockManager(16)
    p = np.arange(40, dtype=np.int32)
    toks = np.concatenate([p, p])
    st, bt, slots, nc = m.schedule(toks, [0, 40, 80], [0, 0], [0, 40, 80],
                                   np.full((2, 4), -1, np.int32), 1)
    assert st == 0 and list(nc) == [0, 0]          # lookups see the index of the call's start
    assert list(bt[0, :3]) == [0, 1, 2] and list(bt[1, :3]) == [3, 4, 5]
    assert sorted(np.nonzero(m.cached)[0].tolist()) == [0, 1]   # the first request's blocks
    st, bt, slots, nc = m.schedule(p, [0, 40], [0], [0, 40], np.full((1, 4), -1, np.int32), 2)
    assert list(nc) == [32] and list(bt[0, :2]) == [0, 1]


def test_a_fully_cached_prompt_still_computes_its_last_token():
    m = M.BlockManager(8)
    p = np.arange(32, dtype=np.int32)
    rows = np.full((1, 4), -1, np.int32)
    m.schedule(p, [0, 32], [0], [0, 32], rows, 1)
    m.release(np.array([[0, 1, -1, -1]], np.int32), np.array([32], np.int32), 2)
    st, bt, slots, nc = m.schedule(p, [0, 32], [0], [0, 32], rows, 3)
    # both blocks are cached, but the second is taken fresh so that token 31 is computed
    assert st == 0 and list(nc) == [16] and list(bt[0, :2]) == [0, 2]
    assert list(slots[:16]) == [-1] * 16 and list(slots[16:]) == list(range(32, 48))
