"""Pins for the mixed-batch (per-sequence query length) oracle, no GPU.

``oracle.paged_attention_varlen_ref`` applies the definition to each
sequence of a token-major packed batch. It is tied to:

- brute force: every sequence's rows equal the scalar-loop oracle run on
  that sequence alone (a batch of one in the [1, H_q, L_b, D] layout);
- a closed form: with all keys zero every visible score is 0, so row l of
  sequence b is the mean of V over positions 0 .. ctx_b - L_b + l (causal)
  or over the whole context -- values chosen to be exact in bf16 and summed
  exactly in integers here, so a wrong per-sequence offset, a wrong head
  map or a row of the wrong sequence shows;
- invariants: reordering the sequences reorders the rows; a sequence with
  no query rows changes nothing (its table row and context are never read);
- planted mistakes (in the oracle, on the CPU): an off-by-one visibility
  rule and a batch-wide query length in place of L_b each fail the closed
  form.
"""

import numpy as np
import pytest

import oracle
from oracle import varlen as varlen_mod
from paged_flashattention_kv_amd import workloads as wl

D = 16


def _vr(p):
    return oracle.paged_attention_varlen_ref(
        p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens, p.query_start, p.page_size, p.scale,
        p.causal,
    )


def _small(seed, ql, ctx, Hq=4, Hkv=2, ps=4, causal=True, poison=True, pool=None):
    return wl.make_varlen_problem(seed=seed, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps,
                                  lens=(ql, ctx), causal=causal, poison=poison, pool_pages=pool)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("ql,ctx,ps", [
    ([3, 1, 5, 2], [7, 9, 5, 11], 4),
    ([1, 1, 1], [1, 6, 13], 3),
    ([6, 4], [6, 17], 5),
    ([2, 7, 1, 1, 3], [2, 8, 33, 4, 9], 8),
])
def test_each_sequence_matches_brute_force(ql, ctx, ps, causal):
    p = _small(11 + sum(ql), ql, ctx, ps=ps, causal=causal)
    got = _vr(p)
    qs = p.query_start
    for b in range(p.batch):
        t0, t1 = int(qs[b]), int(qs[b + 1])
        one = np.ascontiguousarray(p.query[t0:t1].transpose(1, 0, 2))[None]  # [1, H_q, L_b, D]
        want = oracle.paged_attention_brute(one, p.key_pages, p.value_pages, p.block_table[b:b + 1],
                                            p.context_lens[b:b + 1], p.page_size, p.scale, p.causal)[0]
        np.testing.assert_allclose(got[t0:t1], want.transpose(1, 0, 2), rtol=1e-12, atol=1e-12)


def _zero_key_problem(ql, ctx, Hq=4, Hkv=2, ps=4, causal=True):
    """K = 0 and V[page, g, slot, d] = ((7 * pos + 3 * g + d) % 13) - 6 at the logical position pos."""
    p = _small(5, ql, ctx, Hq=Hq, Hkv=Hkv, ps=ps, causal=causal, poison=True)
    k = p.key_pages.copy()
    v = p.value_pages.copy()
    val = {}
    for b in range(p.batch):
        for s in range(int(p.context_lens[b])):
            page, slot = p.block_table[b, s // ps], s % ps
            k[page, :, slot, :] = 0
            for g in range(Hkv):
                row = np.array([((7 * s + 3 * g + d) % 13) - 6 for d in range(D)], dtype=np.float32)
                v[page, g, slot, :] = wl.f32_to_bf16_bits(row)
                val[(b, g, s)] = row.astype(np.int64)
    p.key_pages, p.value_pages = k, v
    return p, val


def _zero_key_expected(p, val, Hq, Hkv):
    want = np.empty((p.total_query, Hq, D))
    qs = p.query_start
    for b in range(p.batch):
        L = int(qs[b + 1] - qs[b])
        c = int(p.context_lens[b])
        for l in range(L):
            last = c - L + l if p.causal else c - 1
            for h in range(Hq):
                g = h // (Hq // Hkv)
                tot = sum(val[(b, g, s)] for s in range(last + 1))  # exact integer sums
                want[qs[b] + l, h] = tot / (last + 1)
    return want


@pytest.mark.parametrize("causal", [True, False])
def test_zero_keys_give_mean_of_visible_values(causal):
    ql, ctx = [4, 1, 2, 1, 5], [9, 3, 14, 1, 5]
    p, val = _zero_key_problem(ql, ctx, causal=causal)
    np.testing.assert_allclose(_vr(p), _zero_key_expected(p, val, 4, 2), rtol=0, atol=1e-12)


def test_planted_off_by_one_visibility_is_caught(monkeypatch):
    ql, ctx = [4, 1, 2], [9, 3, 14]
    p, val = _zero_key_problem(ql, ctx)
    want = _zero_key_expected(p, val, 4, 2)

    def shifted(query_len, c, causal):
        s = np.arange(c)[None, :]
        l = np.arange(query_len)[:, None]
        return s <= l + c - query_len + 1

    monkeypatch.setattr(varlen_mod, "visible_mask", shifted)
    assert not np.allclose(_vr(p), want, atol=1e-6)


def test_planted_batch_wide_query_length_is_caught(monkeypatch):
    ql, ctx = [4, 1, 2], [9, 6, 14]
    p, val = _zero_key_problem(ql, ctx)
    want = _zero_key_expected(p, val, 4, 2)
    real = varlen_mod.visible_mask
    lmax = max(ql)

    def batch_wide(query_len, c, causal):
        # row l placed at c - lmax + l, as if every sequence had the longest query
        return real(lmax, c, causal)[:query_len]

    monkeypatch.setattr(varlen_mod, "visible_mask", batch_wide)
    # the rows of the longest sequence are unchanged; the short ones move
    assert not np.allclose(_vr(p), want, atol=1e-6)


def test_reordering_sequences_reorders_rows():
    p = _small(21, [3, 1, 6, 2], [5, 12, 6, 9], ps=4)
    got = _vr(p)
    order = [2, 0, 3, 1]
    qs = p.query_start
    rows = [np.arange(qs[b], qs[b + 1]) for b in order]
    ql = [int(qs[b + 1] - qs[b]) for b in order]
    q = p.query[np.concatenate(rows)]
    p2 = wl.VarlenProblem(name="perm", query=q, key_pages=p.key_pages, value_pages=p.value_pages,
                          block_table=p.block_table[order], context_lens=p.context_lens[order],
                          query_start=np.concatenate([[0], np.cumsum(ql)]).astype(np.int32),
                          page_size=p.page_size, scale=p.scale, causal=p.causal, seed=p.seed)
    got2 = _vr(p2)
    np.testing.assert_array_equal(got2, got[np.concatenate(rows)])


def test_sequence_without_queries_is_never_read():
    p = _small(31, [2, 3], [7, 4], ps=4)
    base = _vr(p)
    # insert a middle sequence with no query rows, a garbage table row and context 0
    bt = np.full((3, p.max_pages), -7, dtype=np.int32)
    bt[0], bt[2] = p.block_table[0], p.block_table[1]
    p2 = wl.VarlenProblem(name="gap", query=p.query, key_pages=p.key_pages, value_pages=p.value_pages,
                          block_table=bt, context_lens=np.array([7, 0, 4], dtype=np.int32),
                          query_start=np.array([0, 2, 2, 5], dtype=np.int32), page_size=4, scale=p.scale,
                          causal=True, seed=0)
    np.testing.assert_array_equal(_vr(p2), base)


def test_uniform_lengths_agree_with_the_uniform_layout():
    # consistency with the uniform oracle (itself pinned elsewhere): the same
    # sequences, queries moved from [B, H, L, D] to token-major [B * L, H, D]
    u = wl.make_problem(seed=41, batch=3, num_q_heads=4, num_kv_heads=2, query_len=3, head_dim=D, page_size=4,
                        context_lens=[5, 9, 3], poison=True)
    want = oracle.paged_attention_ref(u.query, u.key_pages, u.value_pages, u.block_table, u.context_lens,
                                      u.page_size, u.scale, True)
    q = np.ascontiguousarray(u.query.transpose(0, 2, 1, 3)).reshape(9, 4, D)
    got = oracle.paged_attention_varlen_ref(q, u.key_pages, u.value_pages, u.block_table, u.context_lens,
                                            np.array([0, 3, 6, 9]), 4, u.scale, True)
    np.testing.assert_array_equal(got, want.transpose(0, 2, 1, 3).reshape(9, 4, D))


@pytest.mark.parametrize("qs,ctx,causal", [
    ([1, 2, 3], [4, 4], True),    # does not start at 0
    ([0, 3, 2], [4, 4], True),    # decreases
    ([0, 2, 4], [4, 4], True),    # does not end at T = 3
    ([0, 1, 3], [4, 1], True),    # causal context shorter than the query
    ([0, 1, 3], [4, 0], False),   # context 0 for a sequence with queries
])
def test_rejects_inconsistent_metadata(qs, ctx, causal):
    p = _small(51, [1, 2], [4, 4], ps=4)
    with pytest.raises(ValueError):
        oracle.paged_attention_varlen_ref(p.query, p.key_pages, p.value_pages, p.block_table,
                                          np.array(ctx, dtype=np.int32), np.array(qs), 4, p.scale, causal)


def test_mixed_batch_workload_shape():
    p = wl.make_varlen_config("mixed_batch")
    ql = p.query_lens
    assert p.batch == 64 and int((ql > 1).sum()) <= 8 and int((ql == 1).sum()) >= 56
    assert ql.max() <= 128 and (p.context_lens >= ql).all() and p.context_lens.max() <= 1024 + 128
    assert int(p.query_start[-1]) == p.total_query == int(ql.sum())
