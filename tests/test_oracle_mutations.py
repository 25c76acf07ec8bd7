"""Planted mistakes: each plausible error in the oracle must trip a pin.

The mistakes are planted in the oracle (on the CPU, via monkeypatch) and the
pin tests of test_oracle_attention are re-run against the broken oracle."""
import numpy as np
import pytest

from oracle import attention as A
import test_oracle_attention as T


def _gqa_modulo(args):
    q, K, V, scale, window, want_w = args
    Hq, D = q.shape
    n, Hkv = K.shape[0], K.shape[1]
    out = np.zeros((Hq, D))
    lo, hi = A.decode_window(n, window)
    for h in range(Hq):
        kv = h % Hkv                                       # wrong head mapping
        p = A.softmax_rows(scale * (q[h:h + 1] @ K[lo:hi, kv, :].T))
        out[h] = (p @ V[lo:hi, kv, :])[0]
    return out


def _reassemble_untransposed(pool, fmt, scale, bt_row, n):
    npages = (n + 15) // 16
    pages = A.kv_bits_to_f64(pool[np.asarray(bt_row[:npages], np.int64)], fmt, scale)
    rows = pages.reshape(npages * 16, pool.shape[1], pool.shape[3])   # no transpose
    return rows[:n]


def _lse_wrong_sign(m, l, o):
    M = np.max(m, axis=-1, keepdims=True)
    w = np.where(l > 0, l * np.exp(M - np.where(l > 0, m, 0.0)), 0.0)
    return np.einsum("...p,...pd->...d", w, o) / w.sum(axis=-1)[..., None]


def test_window_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(A, "decode_window",
                        lambda n, w: ((max(0, n - w + 1) if w > 0 else 0), n))
    with pytest.raises(AssertionError):
        T.test_decode_vs_brute_force(*T.SMALL[1])
    with pytest.raises(AssertionError):
        T.test_golden_closed_form_fixture()


def test_gqa_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(A, "_decode_one", _gqa_modulo)
    with pytest.raises(AssertionError):
        T.test_closed_forms()
    with pytest.raises(AssertionError):
        T.test_decode_vs_torch_sdpa()


def test_dropped_scale_is_caught(monkeypatch):
    orig = A._decode_one
    monkeypatch.setattr(A, "_decode_one", lambda a: orig((a[0], a[1], a[2], 1.0) + tuple(a[4:])))
    with pytest.raises(AssertionError):
        T.test_decode_vs_brute_force(*T.SMALL[0])


def test_page_layout_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(A, "reassemble", _reassemble_untransposed)
    with pytest.raises(AssertionError):
        T.test_decode_vs_brute_force(*T.SMALL[0])


def test_lse_sign_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(A, "lse_combine", _lse_wrong_sign)
    with pytest.raises(AssertionError):
        T.test_splitk_lse_combine_equals_single_pass(32)


def test_causal_mask_mistake_is_caught(monkeypatch):
    orig = A.prefill_mask
    monkeypatch.setattr(A, "prefill_mask", lambda n, Q, w: orig(n, Q, w) | np.eye(Q, n, k=n - Q + 1, dtype=bool))
    with pytest.raises(AssertionError):
        T.test_prefill_causal_perturbation()


# ---- block manager ----------------------------------------------------------

from oracle import block_manager as BM  # noqa: E402
import test_oracle_block_manager as TB  # noqa: E402


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def _all_block_manager_pins():
    yield TB.test_walkthrough
    for seed, N, mb in [(1, 64, 16), (2, 40, 12), (3, 400, 24), (4, 24, 8)]:
        yield lambda seed=seed, N=N, mb=mb: TB.test_random_streams_hold_the_pins(seed, N, mb)
    yield TB.test_identical_prompts_in_one_batch_cache_once
    yield TB.test_a_fully_cached_prompt_still_computes_its_last_token


def _caught():
    return any(_fails(f) for f in _all_block_manager_pins())


def test_uncapped_hits_are_caught(monkeypatch):
    monkeypatch.setattr(BM, "max_hit_blocks", lambda n: n // BM.BLOCK)
    assert _caught()


def test_lru_tie_break_towards_parents_is_caught(monkeypatch):
    monkeypatch.setattr(BM.BlockManager, "eviction_key",
                        lambda self, b: (int(self.ts[b]), int(self.depth[b]), b))
    assert _caught()


def test_lru_newest_first_is_caught(monkeypatch):
    monkeypatch.setattr(BM.BlockManager, "eviction_key",
                        lambda self, b: (-int(self.ts[b]), -int(self.depth[b]), b))
    assert _caught()


def test_release_of_cached_blocks_to_the_free_stack_is_caught(monkeypatch):
    def release(self, block_tables, num_tokens, now):
        bt = np.asarray(block_tables, np.int64)
        for r, n in enumerate(np.asarray(num_tokens, np.int64)):
            for j in range(BM.ceil_blocks(int(n))):
                b = int(bt[r, j])
                self.ref[b] = max(0, self.ref[b] - 1)
                self.ts[b] = now
                if self.ref[b] == 0:                     # also pushes cached blocks
                    self.free.append(b)
    monkeypatch.setattr(BM.BlockManager, "release", release)
    assert _caught()


def test_hash_without_the_digit_offset_is_caught(monkeypatch):
    def chain_hash(parent_hash, block_tokens):
        h = parent_hash
        for t in block_tokens:
            h = (h * BM.HASH_BASE + (int(t) & 0xFFFFFFFF)) & BM.MASK64   # digit t, not t + 1
        return h
    monkeypatch.setattr(BM, "chain_hash", chain_hash)
    assert _fails(TB.test_chain_hash_is_the_prefix_polynomial)
