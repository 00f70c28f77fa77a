"""Pins for the CPU oracle (no GPU).

The oracle is the plain definition of paged attention (gather, then one
float64 softmax). These tests tie it to things other than itself:

- brute force: scalar loops with element-by-element page translation;
- a library special case: torch's scaled-dot-product attention in float64;
- closed forms: q = 0 gives the mean of the visible V rows; a row that sees
  one key returns that key's V row exactly;
- invariants: physical page permutation, NaN poisoning of never-read memory,
  repacking with another page size (all bit-identical); tile-size
  independence of the streaming model; chunked continuation equal to the
  tail rows of a full prefill; GQA group behaviour; needle probes;
- planted mistakes: a wrong head map, a dropped causal offset, an off-by-one
  visibility rule and swapped page/slot arithmetic are each caught.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import reference
from paged_flashattention_kv_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _grid():
    with open(os.path.join(GOLDEN, "test_grid.json")) as f:
        return json.load(f)


def _small(seed, B=2, Hq=4, Hkv=2, L=3, D=16, ps=4, ctx=(7, 11), causal=True, pool=None, poison=False):
    return wl.make_problem(
        seed=seed, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, query_len=L, head_dim=D,
        page_size=ps, context_lens=list(ctx), causal=causal, pool_pages=pool, poison=poison,
    )


def _ref(p, **kw):
    return oracle.paged_attention_ref(
        p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens, p.page_size, p.scale, p.causal, **kw
    )


def _brute(p):
    return oracle.paged_attention_brute(
        p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens, p.page_size, p.scale, p.causal
    )


def _online(p, tile, base2=False):
    return oracle.paged_attention_online(
        p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens, p.page_size, p.scale, p.causal,
        tile=tile, base2=base2,
    )


def _close(a, b, tol=1e-12):
    return np.max(np.abs(a - b)) <= tol * max(1.0, np.max(np.abs(b)))


# ---------------------------------------------------------------- brute force


@pytest.mark.parametrize("causal", [True, False])
def test_brute_force_tiny_prefill_config(causal):
    p = wl.make_config("tiny_prefill", causal=causal)
    assert _close(_ref(p), _brute(p))


def _grid_cases():
    g = _grid()["week2_decode_grid"]
    cases = []
    for L in g["query_lens"]:
        for ratio in g["gqa_ratios"]:
            for ctx in g["contexts"]:
                if ctx < L:
                    continue
                cases.append((L, ratio, ctx))
    return cases


@pytest.mark.parametrize("L,ratio,ctx", _grid_cases())
def test_brute_force_week2_grid(L, ratio, ctx):
    # Small head count and head_dim keep the scalar loops fast; the page size
    # (16) makes the longer contexts span several scattered pages.
    p = wl.make_problem(
        seed=100 + ctx + 7 * L + ratio, batch=1, num_q_heads=ratio, num_kv_heads=1, query_len=L,
        head_dim=8, page_size=16, context_lens=[ctx], causal=True, pool_pages=math.ceil(ctx / 16) + 3,
    )
    assert _close(_ref(p), _brute(p))


def test_brute_force_head_dim_128_mixed_batch():
    p = _small(7, B=3, Hq=4, Hkv=1, L=2, D=128, ps=5, ctx=(2, 9, 17), pool=12)
    assert _close(_ref(p), _brute(p))


# ------------------------------------------------------ library special case


def _dense_kv(p, b):
    ctx = int(p.context_lens[b])
    K = reference.gather_history(p.key_pages, p.block_table[b], ctx, p.page_size)
    V = reference.gather_history(p.value_pages, p.block_table[b], ctx, p.page_size)
    return K, V


def _sdpa(p):
    """torch float64 SDPA on the gathered history, K/V repeated per group."""
    B, Hq, L, D = p.query.shape
    G = Hq // p.num_kv_heads
    outs = []
    for b in range(B):
        ctx = int(p.context_lens[b])
        K, V = _dense_kv(p, b)
        Kt = torch.from_numpy(np.repeat(K, G, axis=0))[None]
        Vt = torch.from_numpy(np.repeat(V, G, axis=0))[None]
        q = torch.from_numpy(reference.bf16_bits_to_f64(p.query[b]))[None]
        if not p.causal:
            o = torch.nn.functional.scaled_dot_product_attention(q, Kt, Vt, scale=p.scale)
        elif L == ctx:
            o = torch.nn.functional.scaled_dot_product_attention(q, Kt, Vt, is_causal=True, scale=p.scale)
        else:
            # lower-right aligned causal mask written out explicitly
            mask = torch.ones(L, ctx, dtype=torch.bool).tril(diagonal=ctx - L)
            o = torch.nn.functional.scaled_dot_product_attention(q, Kt, Vt, attn_mask=mask, scale=p.scale)
        outs.append(o[0].numpy())
    return np.stack(outs)


@pytest.mark.parametrize(
    "kw",
    [
        dict(L=13, ctx=(13, 13), causal=True),
        dict(L=5, ctx=(40, 23), causal=True),
        dict(L=4, ctx=(9, 30), causal=False),
        dict(L=1, ctx=(1, 77), causal=True),
    ],
)
def test_matches_torch_sdpa_float64(kw):
    p = _small(11, Hq=8, Hkv=2, D=32, ps=4, **kw)
    assert _close(_ref(p), _sdpa(p))


# ------------------------------------------------------------- closed forms


def test_zero_query_gives_mean_of_visible_values():
    p = _small(12, B=2, Hq=4, Hkv=2, L=6, D=16, ps=3, ctx=(6, 20))
    p.query[:] = 0
    out = _ref(p)
    for b in range(p.batch):
        ctx = int(p.context_lens[b])
        _, V = _dense_kv(p, b)
        prefix = np.cumsum(V, axis=1)  # [H_kv, ctx, D]
        for h in range(p.num_q_heads):
            g = h // (p.num_q_heads // p.num_kv_heads)
            for l in range(p.query_len):
                n = l + ctx - p.query_len + 1
                assert np.allclose(out[b, h, l], prefix[g, n - 1] / n, rtol=0, atol=1e-13)


def test_single_visible_key_returns_its_value_row_exactly():
    p = wl.make_config("tiny_prefill")
    out = _ref(p)
    for h in range(p.num_q_heads):
        g = h // 2
        v0 = reference.bf16_bits_to_f64(p.value_pages[p.block_table[0, 0], g, 0])
        assert np.array_equal(out[0, h, 0], v0)


# --------------------------------------------------------------- invariants


def test_page_permutation_is_bit_identical():
    p = wl.make_config("tiny_prefill")
    q = wl.permute_pages(p, seed=99)
    assert not np.array_equal(p.block_table, q.block_table)
    assert np.array_equal(_ref(p), _ref(q))


def test_poisoned_unused_memory_is_bit_identical():
    clean = _small(13, B=3, L=2, ctx=(5, 9, 2), ps=4, pool=9)
    dirty = _small(13, B=3, L=2, ctx=(5, 9, 2), ps=4, pool=9, poison=True)
    assert np.isnan(wl.bf16_bits_to_f32(dirty.key_pages)).any()
    out = _ref(dirty)
    assert not np.isnan(out).any()
    assert np.array_equal(_ref(clean), out)


@pytest.mark.parametrize("new_ps", [1, 2, 4, 16, 128])
def test_repacking_page_size_is_bit_identical(new_ps):
    p = _small(14, B=2, L=4, ctx=(13, 29), ps=4)
    q = wl.repack_pages(p, new_ps, seed=5)
    assert np.array_equal(_ref(p), _ref(q))


def test_streaming_tile_plan_matches_diagram():
    with open(os.path.join(GOLDEN, "diagram_tiles.json")) as f:
        g = json.load(f)
    plan = oracle.tile_plan(g["history"], g["tile"])
    assert [(t0, v, m) for t0, v, m in plan] == [(t["start"], t["valid"], t["masked"]) for t in g["tiles"]]


def test_streaming_model_is_tile_size_independent():
    spec = _grid()["streaming_tile_sizes"]
    p = wl.make_config("tiny_prefill")
    assert int(p.context_lens[0]) == spec["history"]
    ref = _ref(p)
    outs = [_online(p, t) for t in spec["tile_sizes"]]
    for o in outs:
        assert _close(o, ref)
        assert _close(o, outs[0])
    assert _close(_online(p, 4, base2=True), ref)


def test_streaming_model_matches_oracle_on_ragged_batch():
    p = _small(15, B=3, Hq=4, Hkv=1, L=5, D=16, ps=3, ctx=(5, 31, 70), pool=40, poison=True)
    ref = _ref(p)
    for t in (1, 4, 32):
        assert _close(_online(p, t), ref)


def test_chunk_and_decode_equal_tail_of_full_prefill():
    ctx = 100
    full = _small(16, B=1, Hq=4, Hkv=2, L=ctx, D=16, ps=8, ctx=(ctx,))
    out_full = _ref(full)
    for L in (65, 1):
        chunk = wl.PagedProblem(**{**full.__dict__, "query": np.ascontiguousarray(full.query[:, :, ctx - L:, :])})
        assert _close(_ref(chunk), out_full[:, :, ctx - L:, :])


def test_gqa_equal_queries_in_group_give_equal_outputs():
    p = _small(17, B=1, Hq=8, Hkv=2, L=4, D=16, ps=4, ctx=(19,))
    for g in range(2):
        p.query[0, 4 * g + 1: 4 * g + 4] = p.query[0, 4 * g]
    out = _ref(p)
    for g in range(2):
        for j in range(1, 4):
            assert np.array_equal(out[0, 4 * g + j], out[0, 4 * g])
    assert not np.allclose(out[0, 0], out[0, 4])


def test_gqa_ratio_one_equals_explicitly_repeated_heads():
    p = _small(18, B=1, Hq=6, Hkv=2, L=3, D=16, ps=4, ctx=(10,))
    rep = wl.PagedProblem(**{
        **p.__dict__,
        "key_pages": np.ascontiguousarray(np.repeat(p.key_pages, 3, axis=1)),
        "value_pages": np.ascontiguousarray(np.repeat(p.value_pages, 3, axis=1)),
    })
    assert np.array_equal(_ref(p), _ref(rep))


def _needle(p, b, h, l, t):
    """Make q[b,h,l] = 8 * k_t so that key t dominates the softmax."""
    G = p.num_q_heads // p.num_kv_heads
    phys = p.block_table[b, t // p.page_size]
    k = wl.bf16_bits_to_f32(p.key_pages[phys, h // G, t % p.page_size])
    p.query[b, h, l] = wl.f32_to_bf16_bits(8.0 * k)
    return reference.bf16_bits_to_f64(p.value_pages[phys, h // G, t % p.page_size])


def test_needles_find_their_value_rows_and_invisible_needles_do_not():
    p = _small(19, B=2, Hq=4, Hkv=2, L=4, D=128, ps=4, ctx=(30, 45))
    want = {}
    for b in range(2):
        ctx = int(p.context_lens[b])
        for h in range(4):
            for l in range(4):
                last = l + ctx - 4
                t = (7 * b + 5 * h + 3 * l) % (last + 1)
                want[(b, h, l, True)] = _needle(p, b, h, l, t)
    out = _ref(p)
    for (b, h, l, _), v in want.items():
        assert np.allclose(out[b, h, l], v, atol=1e-9)
    # a needle one past the causal boundary must stay invisible
    q = _small(19, B=1, Hq=4, Hkv=2, L=4, D=128, ps=4, ctx=(30,))
    v_hidden = _needle(q, 0, 1, 0, 30 - 4 + 1)
    o = _ref(q)
    assert np.max(np.abs(o[0, 1, 0] - v_hidden)) > 0.5


# ---------------------------------------------------------- planted mistakes


def _pins_pass():
    """A compact pin suite; returns False as soon as one pin fails."""
    p = _small(21, B=2, Hq=4, Hkv=2, L=3, D=8, ps=3, ctx=(7, 10), pool=9)
    try:
        if not _close(_ref(p), _brute(p)):
            return False
        q = wl.make_config("tiny_prefill")
        if not _close(_ref(q), _sdpa(q)):
            return False
        if not _close(_ref(q), _online(q, 4)):
            return False
    except (IndexError, ValueError):
        return False
    return True


def test_pins_pass_on_the_real_oracle():
    assert _pins_pass()


@pytest.mark.parametrize("mistake", ["head_map_mod", "causal_offset_dropped", "causal_off_by_one", "page_slot_swapped"])
def test_planted_mistake_is_caught(monkeypatch, mistake):
    if mistake == "head_map_mod":
        monkeypatch.setattr(reference, "kv_head_of", lambda h, hq, hkv: h % hkv)
    elif mistake == "causal_offset_dropped":
        def vis(L, ctx, causal):
            s = np.arange(ctx)[None, :]
            l = np.arange(L)[:, None]
            return (s <= l) if causal else np.ones((L, ctx), bool)
        monkeypatch.setattr(reference, "visible_mask", vis)
    elif mistake == "causal_off_by_one":
        def vis(L, ctx, causal):
            s = np.arange(ctx)[None, :]
            l = np.arange(L)[:, None]
            return (s < l + ctx - L) | (s == 0) if causal else np.ones((L, ctx), bool)
        monkeypatch.setattr(reference, "visible_mask", vis)
    elif mistake == "page_slot_swapped":
        def gather(pages, row, ctx, ps):
            pos = np.arange(ctx)
            n = math.ceil(ctx / ps)
            phys = np.asarray(row)[pos % n]
            rows = pages[phys, :, np.minimum(pos // n, ps - 1), :]
            return reference.bf16_bits_to_f64(np.ascontiguousarray(rows.transpose(1, 0, 2)))
        monkeypatch.setattr(reference, "gather_history", gather)
    assert not _pins_pass()


@pytest.mark.parametrize("D", [8, 64, 80, 96, 112, 192, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_other_head_dims_match_brute_force(D, causal):
    # the definition has no head-dim-specific step; pin it at the other head dims the operator serves
    p = wl.make_problem(seed=90 + D, batch=2, num_q_heads=4, num_kv_heads=2, query_len=3, head_dim=D,
                        page_size=4, context_lens=[5, 9], causal=causal, poison=True)
    np.testing.assert_allclose(_ref(p), _brute(p), rtol=1e-12, atol=1e-12)
