"""Pins for the oracle's input validation (no GPU).

``oracle.reference.validate`` runs first in every oracle entry point. Each of
its checks is tied to something outside the oracle:

- H_q must be a multiple of H_kv: the pages require it before the grouped
  head map is used ("Week 2 Day 5: Fused Decode Attention", Task 1);
- 1 <= context_len <= max_pages * page_size: the block table row has to
  name a page for every logical position ("Week 3 Day 5: Paged
  FlashAttention", Task 1 translation);
- with causal, context_len >= L: query row 0 sits at position ctx - L, and
  below zero it would see no key at all, so its softmax is 0 / 0 (the
  mathematics, shown below by letting such a row through);
- every table entry a sequence uses names a page of the pool; an entry of -1
  would otherwise silently read the last page (NumPy's negative index).

The pins check each rejection, the boundary case just inside each limit, and
that dropping any one check (a planted mistake) is caught.
"""

import numpy as np
import pytest

import oracle
from oracle import reference
from paged_flashattention_kv_amd import workloads as wl


def _arrays(B=2, Hq=4, Hkv=2, L=3, D=16, ps=4, ctx=(7, 11), pool=None, seed=5):
    """Valid inputs as plain arrays (the tests break one property at a time)."""
    p = wl.make_problem(seed=seed, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, query_len=L, head_dim=D,
                        page_size=ps, context_lens=list(ctx), pool_pages=pool)
    return dict(query=p.query.copy(), key_pages=p.key_pages.copy(), value_pages=p.value_pages.copy(),
                block_table=p.block_table.copy(), context_lens=p.context_lens.copy(), page_size=ps,
                scale=p.scale)


def _run(a, causal=True):
    return oracle.paged_attention_ref(a["query"], a["key_pages"], a["value_pages"], a["block_table"],
                                      a["context_lens"], a["page_size"], a["scale"], causal)


def _cases():
    """(label, inputs, causal, must_raise) -- each invalid case next to its valid neighbour."""
    out = []
    # H_q % H_kv: 6 query heads over 4 kv heads is no grouping; 8 over 4 is
    a = _arrays()
    q6 = np.concatenate([a["query"], a["query"][:, :2]], axis=1)  # [B, 6, L, D]
    kv4 = np.concatenate([a["key_pages"], a["key_pages"]], axis=1)  # [P, 4, ps, D]
    out.append(("hq_not_multiple", {**a, "query": q6, "key_pages": kv4, "value_pages": kv4}, True, True))
    q8 = np.concatenate([a["query"], a["query"]], axis=1)
    out.append(("hq_multiple", {**a, "query": q8, "key_pages": kv4, "value_pages": kv4}, True, False))
    # causal ctx < L (row 0 would see nothing) -- the same context is fine without causal
    a = _arrays(L=3, ctx=(2, 11))
    out.append(("causal_ctx_below_L", a, True, True))
    out.append(("noncausal_ctx_below_L", a, False, False))
    out.append(("causal_ctx_equal_L", _arrays(L=3, ctx=(3, 11)), True, False))
    # ctx past what the table row can address (max_pages * page_size)
    a = _arrays(ctx=(7, 11))  # max_pages = 3 pages of 4 -> 12 positions
    over = {**a, "context_lens": np.array([7, 13], dtype=np.int32)}
    out.append(("ctx_past_table", over, True, True))
    at = {**a, "context_lens": np.array([7, 12], dtype=np.int32)}
    at["block_table"] = a["block_table"].copy()
    at["block_table"][1, 2] = a["block_table"][0, 0]  # a real page for the last logical page
    out.append(("ctx_at_table_end", at, True, False))
    zero = {**a, "context_lens": np.array([0, 11], dtype=np.int32)}
    out.append(("ctx_zero", zero, False, True))
    # a used table entry outside the pool: -1 and num_pages
    a = _arrays(ctx=(7, 11))
    P = a["key_pages"].shape[0]
    for bad in (-1, P):
        t = a["block_table"].copy()
        t[1, 1] = bad
        out.append((f"page_id_{bad}", {**a, "block_table": t}, True, True))
    # an unused entry may hold anything (sequence 0 uses 2 of its 3 entries)
    t = a["block_table"].copy()
    t[0, 2] = -1
    out.append(("unused_entry_minus_one", {**a, "block_table": t}, True, False))
    t = a["block_table"].copy()
    t[0, 2] = 10 ** 6
    out.append(("unused_entry_huge", {**a, "block_table": t}, True, False))
    return out


@pytest.mark.parametrize("label,inputs,causal,must_raise", _cases(), ids=[c[0] for c in _cases()])
def test_validate_branch(label, inputs, causal, must_raise):
    if must_raise:
        with pytest.raises(ValueError):
            _run(inputs, causal)
    else:
        out = _run(inputs, causal)
        assert np.isfinite(out).all()


def _validate_pins_pass() -> bool:
    """True when the oracle raises ValueError exactly on the invalid cases.

    Any other failure (an IndexError from a table entry or head index past an
    array's end) means an invalid input got past the checks.
    """
    for label, inputs, causal, must_raise in _cases():
        try:
            out = _run(inputs, causal)
        except ValueError:
            if not must_raise:
                return False
            continue
        except IndexError:
            return False
        if must_raise:
            return False
        if not np.isfinite(out).all():
            return False
    return True


def test_validate_pins_pass_on_the_real_oracle():
    assert _validate_pins_pass()


def _without(check):
    """``validate`` with one of its checks left out (a planted mistake)."""

    def patched(query_shape, pages_shape, block_table, context_lens, page_size, causal):
        B, Hq, L, D = (int(x) for x in query_shape)
        P, Hkv, ps, Dk = (int(x) for x in pages_shape)
        if min(B, Hq, L, D, P, Hkv, ps) <= 0 or ps != page_size or Dk != D:
            raise ValueError("shapes")
        if check != "group" and Hq % Hkv != 0:
            raise ValueError("group")
        bt = np.asarray(block_table)
        ctx = np.asarray(context_lens)
        for b in range(B):
            c = int(ctx[b])
            if check != "ctx_range" and (c < 1 or c > bt.shape[1] * ps):
                raise ValueError("ctx range")
            if check != "causal_ctx" and causal and c < L:
                raise ValueError("causal ctx")
            used = bt[b, : -(-c // ps)]
            if check != "page_range" and ((used < 0).any() or (used >= P).any()):
                raise ValueError("page range")

    return patched


@pytest.mark.parametrize("check", ["group", "causal_ctx", "ctx_range", "page_range"])
def test_planted_validation_mistake_is_caught(monkeypatch, check):
    monkeypatch.setattr(reference, "validate", _without(check))
    assert not _validate_pins_pass()


def test_row_without_visible_key_is_undefined():
    # Why causal needs ctx >= L: let a ctx < L case past validation and the first
    # query rows see no key, so their softmax is 0 / 0 (NaN) -- there is no value
    # to compare a kernel against, so the case is rejected instead.
    a = _arrays(L=3, ctx=(2, 11))
    ctx, L = 2, 3
    K = reference.gather_history(a["key_pages"][:, 0:1], a["block_table"][0], ctx, a["page_size"])[0]
    q = reference.bf16_bits_to_f64(a["query"][0, 0])
    S = np.where(reference.visible_mask(L, ctx, True), q @ K.T, -np.inf)
    with np.errstate(invalid="ignore"):
        P = np.exp(S - S.max(axis=1, keepdims=True))
        w = P / P.sum(axis=1, keepdims=True)
    assert np.isnan(w[0]).all() and np.isfinite(w[1:]).all()
