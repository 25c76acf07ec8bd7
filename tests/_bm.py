"""Drive a block manager (the oracle's, or the library's through a wrapper with
the same two methods) with a seeded request stream, the way an engine's
scheduler would: finished sequences are released, running ones extended,
new prompts admitted; every call's inputs and outputs are recorded."""
from __future__ import annotations

import numpy as np

from workloads.requests import RequestStream

BLOCK = 16


class Driver:
    def __init__(self, mgr, stream: RequestStream, max_blocks: int):
        self.mgr = mgr
        self.stream = stream
        self.mb = max_blocks
        self.seqs: dict = {}          # id -> dict(tokens, computed, row)
        self.now = 0
        self.log: list = []

    def batch_inputs(self, ids, new_tokens):
        """CSR token ids, computed counts, query offsets and table rows of
        the requests ``ids`` (in that order), ``new_tokens[id]`` added."""
        toks, tstart, old, qsl, rows = [], [0], [], [0], []
        for s in ids:
            rec = self.seqs[s]
            t = rec["tokens"] + new_tokens[s]
            toks += t
            tstart.append(len(toks))
            old.append(rec["computed"])
            qsl.append(qsl[-1] + len(new_tokens[s]))
            rows.append(rec["row"])
        rows = np.array(rows, np.int32).reshape(len(ids), self.mb)
        return (np.array(toks, np.int32), np.array(tstart, np.int32), np.array(old, np.int32),
                np.array(qsl, np.int32), rows)

    def release(self, ids):
        if not ids:
            return
        self.now += 1
        rows = np.array([self.seqs[s]["row"] for s in ids], np.int32).reshape(len(ids), self.mb)
        ntok = np.array([self.seqs[s]["computed"] for s in ids], np.int32)
        self.mgr.release(rows, ntok, self.now)
        self.log.append(("release", ids, rows, ntok, self.now))
        for s in ids:
            del self.seqs[s]

    def schedule(self, ids, new_tokens):
        self.now += 1
        inp = self.batch_inputs(ids, new_tokens)
        status, bt, slots, ncached = self.mgr.schedule(*inp, self.now)
        self.log.append(("schedule", ids, inp, (status, bt, slots, ncached), self.now))
        if status == 0:
            for i, s in enumerate(ids):
                rec = self.seqs[s]
                rec["tokens"] = rec["tokens"] + new_tokens[s]
                rec["computed"] = len(rec["tokens"])
                rec["row"] = np.asarray(bt[i], np.int32).copy()
        return status, inp, (bt, slots, ncached)

    def step(self):
        """One engine step; returns the list of schedule results."""
        plan = self.stream.step()
        self.release([s for s in plan.finish if s in self.seqs])
        first = self.stream.next_id - len(plan.admit)
        for k, p in enumerate(plan.admit):
            self.seqs[first + k] = dict(tokens=[], computed=0, row=np.full(self.mb, -1, np.int32))
        new_tokens = {s: t for s, t in plan.extend.items() if s in self.seqs}
        for k, p in enumerate(plan.admit):
            new_tokens[first + k] = list(p)
        # requests whose sequences would outgrow their rows end first
        too_long = [s for s in list(new_tokens)
                    if (len(self.seqs[s]["tokens"]) + len(new_tokens[s]) + BLOCK - 1) // BLOCK > self.mb]
        for s in too_long:
            del new_tokens[s]
        self.release([s for s in too_long if self.seqs[s]["computed"] > 0])
        for s in too_long:
            self.seqs.pop(s, None)
            if s in self.stream.running:
                self.stream.running.remove(s)
        ids = sorted(new_tokens)
        out = []
        if not ids:
            return out
        status, inp, res = self.schedule(ids, new_tokens)
        out.append((status, inp, res))
        if status == 1:
            # out of blocks: admit nothing new this step, and if even the
            # running sequences do not fit, finish the oldest ones
            fresh = [s for s in ids if self.seqs[s]["computed"] == 0]
            for s in fresh:
                del self.seqs[s]
                self.stream.running.remove(s)
            run = [s for s in ids if s in self.seqs]
            while run:
                status, inp, res = self.schedule(run, {s: new_tokens[s] for s in run})
                out.append((status, inp, res))
                if status != 1:
                    break
                victim = run.pop(0)
                self.release([victim])
                self.stream.running.remove(victim)
        return out

    def live_refs(self, N):
        """Reference counts implied by the live rows."""
        ref = np.zeros(N, np.int64)
        for rec in self.seqs.values():
            nb = (rec["computed"] + BLOCK - 1) // BLOCK
            for b in rec["row"][:nb]:
                ref[b] += 1
        return ref
