"""Seeded synthetic request streams for the prefix-caching block manager.

Only draws inputs: which prompts arrive, their token ids, how many tokens each
running sequence adds per step, and which sequences finish.  Prompts come
from a few families that share long prefixes (a system prompt, a few-shot
template), so that later prompts hit blocks cached by earlier ones, as in
the repeated-template case of "Building and Deploying vllm.cpp" (Step 3,
RadixTree prefix caching).  No block-manager arithmetic lives here.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass
class StepPlan:
    admit: list          # token lists of new requests (their whole prompts)
    extend: dict         # sequence id -> new token ids (decode: one token; prefill chunk: more)
    finish: list         # sequence ids that end before this step


class RequestStream:
    """Running sequences are named by increasing ids; the caller admits the
    planned prompts under ids next_id, next_id + 1, ... in order."""

    def __init__(self, seed: int, families: int = 4, family_len=(8, 90), suffix_len=(0, 60),
                 vocab: int = 1000, max_admit: int = 4, max_running: int = 12,
                 finish_p: float = 0.15, chunk_p: float = 0.2, chunk_len=(2, 40)):
        self.g = np.random.default_rng(seed)
        self.vocab = vocab
        lo, hi = family_len
        self.families = [self.g.integers(0, vocab, self.g.integers(lo, hi + 1)).tolist()
                         for _ in range(families)]
        self.suffix_len = suffix_len
        self.max_admit = max_admit
        self.max_running = max_running
        self.finish_p = finish_p
        self.chunk_p = chunk_p
        self.chunk_len = chunk_len
        self.running: list = []
        self.next_id = 0

    def prompt(self) -> list:
        g = self.g
        fam = self.families[g.integers(0, len(self.families))]
        keep = fam if g.random() < 0.7 else fam[:g.integers(0, len(fam) + 1)]
        suffix = g.integers(0, self.vocab, g.integers(self.suffix_len[0], self.suffix_len[1] + 1))
        p = list(keep) + suffix.tolist()
        return p if p else [int(g.integers(0, self.vocab))]

    def step(self) -> StepPlan:
        g = self.g
        finish = [s for s in self.running if g.random() < self.finish_p]
        self.running = [s for s in self.running if s not in finish]
        extend = {}
        for s in self.running:
            n = int(g.integers(*self.chunk_len)) if g.random() < self.chunk_p else 1
            extend[s] = g.integers(0, self.vocab, n).tolist()
        room = max(0, self.max_running - len(self.running))
        k = int(g.integers(0, min(self.max_admit, room) + 1))
        admit = [self.prompt() for _ in range(k)]
        ids = list(range(self.next_id, self.next_id + k))
        self.next_id += k
        self.running += ids
        return StepPlan(admit=admit, extend=extend, finish=finish)
