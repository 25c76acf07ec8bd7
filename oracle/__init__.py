"""Plain, slow, obviously-correct CPU oracle for the paged KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only the test-suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It
shares no code with the HIP library (no kernels, headers, helpers, tables or
pre/post-processing); the only common dependency is the seeded input
generator in ``workloads``, which holds none of the method's arithmetic.

Everything is computed in float64 with numpy from the raw storage bits of the
inputs.  Modules:

* ``formats``   -- exact decode of fp16 / bf16 bits and the OCP FP8 E4M3
                   codec (decode of all 256 codes, nearest-even encode).
* ``scatter``   -- the cache write: token i goes to page slot_mapping[i]//16,
                   row slot_mapping[i] % 16, every kv-head; negative slots are
                   skipped.
* ``attention`` -- paged decode and chunked-prefill attention over K/V
                   reassembled contiguously from the block tables, plus the
                   per-partition (max, sum, output) triples and their
                   log-sum-exp combination; chunked-local attention, its
                   virtual-batch plan and the dead pages of local attention.
* ``block_manager`` -- the prefix-caching block manager that builds block
                   tables and slot mappings: exact block-level trie behind
                   a chain-hash index, reference counts, LRU leaf eviction.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
brute force, library special cases, closed forms and invariants; none is left
"parity unpinned".
"""
from . import formats, scatter, attention, block_manager  # noqa: F401
