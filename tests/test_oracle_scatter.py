"""Pins for the oracle's cache write (oracle/scatter.py).

Pinned by invariants that do not restate the write: reading each sequence
back through its block table returns the contiguous fill rows; every slot not
named by the slot mapping keeps its NaN sentinel; the number of changed bytes
equals (valid tokens) x Hkv x D; a hand-checked tiny fixture."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import scatter
from oracle.formats import kv_bits_to_f64
from workloads import make_case, raw_bits, SENTINEL_BITS

from _util import oracle_pools, contiguous_kv


@pytest.mark.parametrize("idx,over", [
    (0, {}),
    (1, dict(B=3, ctx_range=(1, 70))),
    (2, dict(B=2, ctx_range=(40, 90), Hq=10, Hkv=2, D=64)),
    (3, dict(B=3, shared_tokens=32, suffix_range=(1, 40))),
    (4, dict(B=3, qlen_range=(1, 9), cached_range=(5, 40))),
])
def test_readback_through_tables(idx, over):
    case = make_case(idx, **over)
    kp, vp = oracle_pools(case)
    bt = case.block_tables.numpy()
    for s in range(case.num_seqs):
        n = int(case.context_lens[s])
        K = A.reassemble(kp, case.kv_dtype, case.k_scale, bt[s], n)
        V = A.reassemble(vp, case.kv_dtype, case.v_scale, bt[s], n)
        Kc, Vc = contiguous_kv(case, s)
        assert np.array_equal(K, Kc) and np.array_equal(V, Vc)


def test_untouched_slots_keep_sentinel():
    case = make_case(0)
    kp, _ = oracle_pools(case)
    written = np.zeros(kp.shape[0] * 16, bool)
    written[case.fill_slots.numpy()] = True
    written = written.reshape(kp.shape[0], 16)
    sent = SENTINEL_BITS["f16"]
    for b in range(kp.shape[0]):
        for off in range(16):
            page_row = kp[b, :, off, :]
            if written[b, off]:
                assert not np.any(page_row == sent)
            else:
                assert np.all(page_row == sent)


def test_changed_element_count_and_negative_slots():
    rng = np.random.default_rng(5)
    pool = np.full((6, 3, 16, 8), 0x7E00, np.uint16)
    bits = rng.integers(0, 0x3C00, size=(10, 3, 8)).astype(np.uint16)  # finite, non-sentinel
    slots = rng.permutation(6 * 16)[:10].astype(np.int64)
    slots[[2, 7]] = -1
    out = scatter.cache_write(pool, bits, slots, "f16", "f16")
    assert np.sum(out != pool) == 8 * 3 * 8
    for i, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(out[s // 16, :, s % 16, :], bits[i])
    assert np.array_equal(out, scatter.cache_write_fast(pool, bits, slots, "f16", "f16"))


def test_tiny_fixture_by_hand():
    # Pool of 2 pages, 1 head, D = 2.  Token 0 -> slot 17 = page 1 row 1;
    # token 1 skipped (-1); token 2 -> slot 3 = page 0 row 3.
    pool = np.zeros((2, 1, 16, 2), np.uint16)
    bits = np.array([[[1, 2]], [[3, 4]], [[5, 6]]], np.uint16)
    out = scatter.cache_write(pool, bits, np.array([17, -1, 3]), "f16", "f16")
    want = np.zeros_like(pool)
    want[1, 0, 1] = [1, 2]
    want[0, 0, 3] = [5, 6]
    assert np.array_equal(out, want)


def test_fp8_write_matches_codec_and_scale():
    case = make_case(3, B=2, shared_tokens=16, suffix_range=(3, 20))
    kp, vp = oracle_pools(case)
    assert kp.dtype == np.uint8
    # the value read back is code * scale, close to the fp16 input (|x| < 8
    # so x / 0.05 < 160 stays in range; relative step of E4M3 is 2^-3).
    Kc, _ = contiguous_kv(case, 0)
    x = raw_bits(case.fill_k)[case.seq_rows[0].numpy()]
    xf = kv_bits_to_f64(x, "f16")
    err = np.abs(Kc - xf)
    assert np.all(err <= np.abs(xf) * 2.0 ** -4 + 0.05 * 2.0 ** -10)


def test_fp8_code_table_equals_direct_encoder():
    rng = np.random.default_rng(7)
    for fmt in ("f16", "bf16"):
        for scale in (1.0, 0.05):
            bits = rng.integers(0, 65536, size=5000).astype(np.uint16)
            from oracle.formats import e4m3_quantize_bits
            assert np.array_equal(scatter.encode_rows(bits, fmt, "e4m3", scale),
                                  e4m3_quantize_bits(bits, fmt, scale))


def test_per_head_scales_pick_the_head():
    """With one scale per kv-head, head h of the pool equals a per-tensor
    write with scale[h] (for both FP8 formats)."""
    import numpy as np
    from workloads import make_case, raw_bits
    from oracle import scatter as S
    case = make_case(1, B=2, ctx_range=(20, 40), Hq=6, Hkv=3, kv="e4m3", q="f16", kv_src="f16")
    pool0 = raw_bits(case.sentinel_pool())
    fk, slots = raw_bits(case.fill_k), case.fill_slots.numpy()
    scales = (0.05, 0.7, 3.0)
    for fmt in ("e4m3", "e5m2"):
        got = S.cache_write_fast(pool0, fk, slots, "f16", fmt, scales)
        for h, sc in enumerate(scales):
            ref = S.cache_write(pool0, fk, slots, "f16", fmt, sc)
            assert np.array_equal(got[:, h], ref[:, h]), (fmt, h)
