"""CPU checks of the benchmark's own logic: the one-GPU guard and the
algorithmic byte / flop counts its roofline figures are priced on (counted
here by brute force over token positions)."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import make_case  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_decode_bytes_tiny_case():
    # 4 sequences of 1, 7, 16 and 33 tokens, 2 kv-heads of 64 fp16 values:
    # 57 tokens of K and V are 29,184 bytes
    case = make_case(0)
    by = bench.decode_bytes(case)
    assert by["kept_tokens"] == 57
    assert by["kv"] == 29184


def _kept_keys_decode(n, window):
    return sum(1 for t in range(n) if window == 0 or t > n - 1 - window)


def test_decode_bytes_window_brute_force():
    for window in (0, 1, 16, 17, 300):
        case = make_case(1, B=5, ctx_range=(1, 400), window=window)
        kept = sum(_kept_keys_decode(int(n), window) for n in case.context_lens.tolist())
        by = bench.decode_bytes(case)
        assert by["kept_tokens"] == kept
        assert by["kv"] == kept * case.num_kv_heads * case.head_dim * 2 * 2


def _prefill_pairs(case, chunk):
    qsl = case.query_start_loc.numpy()
    ctx = case.context_lens.numpy()
    pairs = 0
    for s in range(len(ctx)):
        Q, n = int(qsl[s + 1] - qsl[s]), int(ctx[s])
        for p in range(n - Q, n):
            for t in range(p + 1):
                if chunk:
                    keep = t >= (p // chunk) * chunk
                else:
                    keep = case.window == 0 or t > p - case.window
                pairs += keep
    return pairs


def test_prefill_work_brute_force():
    case = make_case(4, B=4, qlen_range=(1, 40), cached_range=(1, 150), window=64)
    for chunk in (0, 32, 48):
        w = bench.prefill_work(case, chunk)
        pairs = _prefill_pairs(case, chunk)
        assert w["pairs"] == pairs
        assert w["flops"] == pairs * case.num_q_heads * 4 * case.head_dim
        assert w["tokens"] == int(np.diff(case.query_start_loc.numpy()).sum())
