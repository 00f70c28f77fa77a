"""Pins of the K/V append oracle (CPU only).

The oracle (oracle/append.py) copies new tokens into page slots through the
translation of "Week 3 Day 5: Paged FlashAttention", Task 1. It is pinned
here by a hand-worked example whose slots are written out by hand, by the
read half of the cache (gather_history, itself pinned in
test_oracle_pins.py), by composition of appends, and by the attention over a
pool rebuilt from nothing but appends.
"""

import numpy as np
import pytest

import oracle
from oracle import reference
from paged_flashattention_kv_amd import workloads as wl

NAN = np.uint16(0x7FC0)


def _bits(x):
    """bf16 bit patterns of float64 values that came from bf16 (exact)."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _history_bits(pages, row, ctx, ps):
    return _bits(reference.gather_history(pages, row, ctx, ps))


def test_hand_worked_slots():
    # 3 new tokens of a sequence whose context becomes 10, pages of 4 slots,
    # block table [5, 2, 7]: positions 7, 8, 9 -> (page 2, slot 3),
    # (page 7, slot 0), (page 7, slot 1); nothing else changes.
    kp = np.zeros((8, 1, 4, 2), dtype=np.uint16)
    vp = np.zeros((8, 1, 4, 2), dtype=np.uint16)
    kn = np.array([[[[11, 12], [21, 22], [31, 32]]]], dtype=np.uint16)
    vn = kn + 100
    bt = np.array([[5, 2, 7]], dtype=np.int32)
    k2, v2 = oracle.kv_append_ref(kn, vn, kp, vp, bt, np.array([10]), 4)
    want = np.zeros_like(kp)
    want[2, 0, 3] = [11, 12]
    want[7, 0, 0] = [21, 22]
    want[7, 0, 1] = [31, 32]
    assert np.array_equal(k2, want)
    want_v = np.where(want != 0, want + 100, 0).astype(np.uint16)
    assert np.array_equal(v2, want_v)
    assert not kp.any() and not vp.any()  # inputs untouched


def _blank_tail(p, n_new):
    """The problem's pools with the last n_new positions of every sequence set to NaN, and those tokens."""
    B, H, D = p.batch, p.num_kv_heads, p.head_dim
    kp, vp = p.key_pages.copy(), p.value_pages.copy()
    kn = np.zeros((B, H, n_new, D), dtype=np.uint16)
    vn = np.zeros_like(kn)
    for b in range(B):
        ctx = int(p.context_lens[b])
        hk = _history_bits(p.key_pages, p.block_table[b], ctx, p.page_size)
        hv = _history_bits(p.value_pages, p.block_table[b], ctx, p.page_size)
        kn[b] = hk[:, ctx - n_new:]
        vn[b] = hv[:, ctx - n_new:]
        for s in range(ctx - n_new, ctx):
            page = p.block_table[b, s // p.page_size]
            kp[page, :, s % p.page_size] = NAN
            vp[page, :, s % p.page_size] = NAN
    return kp, vp, kn, vn


@pytest.mark.parametrize("ps,n_new", [(1, 1), (3, 5), (4, 13), (16, 1), (16, 40), (128, 65)])
def test_append_restores_the_gathered_tail(ps, n_new):
    p = wl.make_problem(seed=300 + ps, batch=3, num_q_heads=4, num_kv_heads=2, query_len=1, head_dim=8,
                        page_size=ps, context_lens=[n_new + 7, n_new, n_new + 130], poison=True)
    kp, vp, kn, vn = _blank_tail(p, n_new)
    k2, v2 = oracle.kv_append_ref(kn, vn, kp, vp, p.block_table, p.context_lens, ps)
    assert np.array_equal(k2, p.key_pages) and np.array_equal(v2, p.value_pages)
    for b in range(p.batch):  # the read half sees the new tokens at the new positions
        ctx = int(p.context_lens[b])
        h = _history_bits(k2, p.block_table[b], ctx, ps)
        assert np.array_equal(h[:, ctx - n_new:], kn[b])


def test_two_appends_equal_one():
    p = wl.make_problem(seed=311, batch=2, num_q_heads=4, num_kv_heads=2, query_len=1, head_dim=8,
                        page_size=5, context_lens=[29, 41], poison=True)
    kp, vp, kn, vn = _blank_tail(p, 12)
    once = oracle.kv_append_ref(kn, vn, kp, vp, p.block_table, p.context_lens, 5)
    first = oracle.kv_append_ref(kn[:, :, :7], vn[:, :, :7], kp, vp, p.block_table, p.context_lens - 5, 5)
    twice = oracle.kv_append_ref(kn[:, :, 7:], vn[:, :, 7:], *first, p.block_table, p.context_lens, 5)
    assert np.array_equal(once[0], twice[0]) and np.array_equal(once[1], twice[1])


def test_attention_over_a_pool_built_by_appends():
    # a decode batch whose pool starts all-NaN and receives every token by append
    p = wl.make_problem(seed=312, batch=3, num_q_heads=8, num_kv_heads=2, query_len=1, head_dim=16,
                        page_size=4, context_lens=[9, 14, 3])
    kp = np.full_like(p.key_pages, NAN)
    vp = np.full_like(p.value_pages, NAN)
    for b in range(p.batch):
        ctx = int(p.context_lens[b])
        hk = _history_bits(p.key_pages, p.block_table[b], ctx, p.page_size)[None]
        hv = _history_bits(p.value_pages, p.block_table[b], ctx, p.page_size)[None]
        kp, vp = oracle.kv_append_ref(hk, hv, kp, vp, p.block_table[b:b + 1], p.context_lens[b:b + 1], 4)
    got = oracle.paged_attention_ref(p.query, kp, vp, p.block_table, p.context_lens, 4, p.scale, True)
    want = oracle.paged_attention_ref(p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens, 4,
                                      p.scale, True)
    assert np.array_equal(got, want)


def test_rejects_bad_metadata():
    kp = np.zeros((4, 1, 2, 2), dtype=np.uint16)
    kn = np.ones((1, 1, 3, 2), dtype=np.uint16)
    with pytest.raises(ValueError):  # fewer context positions than new tokens
        oracle.kv_append_ref(kn, kn, kp, kp, np.array([[0, 1]]), np.array([2]), 2)
    with pytest.raises(ValueError):  # position past the block table
        oracle.kv_append_ref(kn, kn, kp, kp, np.array([[0]]), np.array([3]), 2)
    with pytest.raises(ValueError):  # page not in the pool
        oracle.kv_append_ref(kn, kn, kp, kp, np.array([[0, 9]]), np.array([4]), 2)
    with pytest.raises(ValueError):  # two sequences sharing a slot
        kn2 = np.ones((2, 1, 1, 2), dtype=np.uint16)
        oracle.kv_append_ref(kn2, kn2, kp, kp, np.array([[1], [1]]), np.array([1, 1]), 2)
