"""Oracle references of the full-size workloads, computed in a child process.

The full-size parity tests compare every output element of the benchmark's
workloads with the fp64 oracle.  The oracle needs tens of seconds of CPU for
some of them, so one child process (a fresh interpreter that never touches
the GPU) computes them with forked workers while the other GPU tests run; the
tests then wait for the results.  The child reads only the seeded generators
and ``oracle/``; nothing it computes comes from the HIP path.

    python tests/_fullsize.py OUTDIR JOB [JOB ...]     # the child

writes OUTDIR/JOB.npy (float64) for each job in order, each one atomically
(a temporary name, then a rename), and OUTDIR/JOB.err on failure.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# job name -> (workload index, what is computed)
JOBS = {
    "decode2": (2, "decode"),        # long-context split-K, fp16: all 16 sequences
    "decode3": (3, "decode"),        # prefix-shared FP8: all 128 sequences
    "prefill4": (4, "prefill"),      # chunked prefill, bf16: all 16,411 query rows
    "local4": (4, "chunked_local"),  # the same batch, chunked-local attention of 8192 tokens
}
LOCAL_CHUNK = 8192

# Inputs of the chunked-local job, inherited by its forked workers.
_LOCAL = None


def _local_seq(s):
    """Chunked-local attention of sequence s's query rows (the oracle's
    function on a one-sequence batch)."""
    from oracle import attention as A
    case, qb, kp, vp = _LOCAL
    qsl = case.query_start_loc.numpy()
    a, b = int(qsl[s]), int(qsl[s + 1])
    return A.prefill_chunked_local(qb[a:b], case.q_dtype, kp, vp, case.kv_dtype,
                                   case.block_tables.numpy()[s:s + 1], [0, b - a],
                                   case.context_lens.numpy()[s:s + 1], case.scale, LOCAL_CHUNK)


def _workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def compute(job: str):
    """The oracle's float64 output of one job (all sequences / all rows)."""
    sys.path.insert(0, ROOT)
    sys.path.insert(0, HERE)
    from oracle import attention as A
    from workloads import make_case, raw_bits
    from _util import oracle_pools
    idx, kind = JOBS[job]
    case = make_case(idx)
    kp, vp = oracle_pools(case)
    if kind == "decode":
        return A.decode(raw_bits(case.q), case.q_dtype, kp, vp, case.kv_dtype,
                        case.block_tables.numpy(), case.context_lens.numpy(), case.scale,
                        case.window, case.k_scale, case.v_scale, workers=_workers())
    if kind == "prefill":
        return A.prefill(raw_bits(case.q), case.q_dtype, kp, vp, case.kv_dtype,
                         case.block_tables.numpy(), case.query_start_loc.numpy(),
                         case.context_lens.numpy(), case.scale, case.window, workers=_workers())
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor
    import numpy as np
    global _LOCAL
    _LOCAL = (case, raw_bits(case.q), kp, vp)
    seqs = sorted(range(case.num_seqs), key=lambda j: -int(case.context_lens[j]))
    with ProcessPoolExecutor(_workers(), mp_context=multiprocessing.get_context("fork")) as ex:
        done = dict(zip(seqs, ex.map(_local_seq, seqs)))
    _LOCAL = None
    return np.concatenate([done[j] for j in range(case.num_seqs)], axis=0)


def _child(outdir: str, jobs: list) -> int:
    import numpy as np
    from threadpoolctl import threadpool_limits
    for job in jobs:
        t0 = time.time()
        try:
            # one BLAS thread in each forked worker (the host may default BLAS
            # to every core, which the workers would then oversubscribe)
            with threadpool_limits(limits=1, user_api="blas"):
                ref = compute(job)
        except Exception as e:                       # reported to the waiting test
            with open(os.path.join(outdir, job + ".err"), "w") as f:
                f.write(f"{type(e).__name__}: {e}\n")
            return 1
        tmp = os.path.join(outdir, job + ".tmp.npy")
        np.save(tmp, ref)
        os.replace(tmp, os.path.join(outdir, job + ".npy"))
        print(f"{job}: {ref.shape} in {time.time() - t0:.1f} s", flush=True)
    return 0


# ---- test-process side --------------------------------------------------------

_STATE = {"proc": None, "dir": None, "jobs": ()}


def start(jobs) -> None:
    """Start the child for ``jobs`` (no-op if already started)."""
    if _STATE["proc"] is not None or not jobs:
        return
    outdir = tempfile.mkdtemp(prefix="vllm_paged_oracle_")
    env = dict(os.environ)
    log = open(os.path.join(outdir, "child.log"), "w")
    _STATE["proc"] = subprocess.Popen([sys.executable, os.path.abspath(__file__), outdir, *jobs],
                                      stdout=log, stderr=subprocess.STDOUT, env=env, cwd=ROOT)
    _STATE["dir"] = outdir
    _STATE["jobs"] = tuple(jobs)


def result(job: str, timeout: float = 900.0):
    """Wait for and load one job's output (starting the child if needed)."""
    import numpy as np
    if _STATE["proc"] is None or job not in _STATE["jobs"]:
        stop()
        start([job])
    outdir, proc = _STATE["dir"], _STATE["proc"]
    path = os.path.join(outdir, job + ".npy")
    t0 = time.time()
    while not os.path.exists(path):
        if os.path.exists(os.path.join(outdir, job + ".err")) or proc.poll() not in (None, 0):
            log = open(os.path.join(outdir, "child.log")).read()[-2000:]
            err = os.path.join(outdir, job + ".err")
            msg = open(err).read() if os.path.exists(err) else ""
            raise RuntimeError(f"oracle child failed on {job}: {msg}{log}")
        if proc.poll() == 0 and not os.path.exists(path):
            raise RuntimeError(f"oracle child finished without {job}")
        if time.time() - t0 > timeout:
            raise TimeoutError(f"oracle reference {job} not ready after {timeout:.0f} s")
        time.sleep(0.2)
    return np.load(path)


def stop() -> None:
    """End the child (if running) and remove its files."""
    import shutil
    proc, outdir = _STATE["proc"], _STATE["dir"]
    if proc is not None and proc.poll() is None:
        proc.terminate()
        try:
            proc.wait(timeout=10)
        except subprocess.TimeoutExpired:
            proc.kill()
    if outdir:
        shutil.rmtree(outdir, ignore_errors=True)
    _STATE.update(proc=None, dir=None, jobs=())


if __name__ == "__main__":
    sys.exit(_child(sys.argv[1], sys.argv[2:]))
