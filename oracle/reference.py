"""Plain float64 paged attention: gather the paged history, then one softmax.

TEST INFRASTRUCTURE ONLY (see the package docstring): the GPU path never
imports this module.

The method approximates nothing: it reaches plain scaled-dot-product
attention by another route through memory, and differs from it by rounding
alone ("Week 3 Day 5: Paged FlashAttention", section "Why Optimize the Paged
Path"). So the oracle is that definition written out:

1. translate every logical key position through the block table and gather
   the sequence's history into a dense ``[H_kv, ctx, D]`` buffer -- the
   gather-then-softmax reference of "Day 22: the fused paged-attention
   kernel" (section "What I added today"), with the translation of
   "Week 3 Day 5", Task 1 (logical page = position / page_size, slot =
   position % page_size, physical page = block_table[batch, logical page]);
2. map each query head to its K/V head, kv_head = q_head / (H_q / H_kv)
   ("Week 2 Day 5: Fused Decode Attention", Task 1);
3. score S = scale * Q K^T in float64;
4. hide key s from query row l unless s <= l + context_len - L when causal
   ("Week 3 Day 5", Task 2), by setting its score to -inf;
5. softmax over the visible keys and weight V.

All arithmetic is float64. bf16 inputs widen to float64 exactly.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly; other dtypes are cast."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def kv_head_of(q_head: int, num_q_heads: int, num_kv_heads: int) -> int:
    """GQA map: query head h reads K/V head h / (H_q / H_kv) ("Week 2 Day 5", Task 1)."""
    return q_head // (num_q_heads // num_kv_heads)


def validate(
    query_shape: Sequence[int],
    pages_shape: Sequence[int],
    block_table: np.ndarray,
    context_lens: np.ndarray,
    page_size: int,
    causal: bool,
) -> None:
    """Raise ``ValueError`` unless the inputs describe a well-defined attention.

    Checks: H_q divisible by H_kv ("Week 2 Day 5", Task 1); 1 <= ctx <=
    max_pages * page_size; ctx >= L when causal (otherwise some query row
    would see no key at all); every table entry a sequence uses is a valid
    page id. Entries past a sequence's last page are never read.
    """
    B, Hq, L, D = (int(x) for x in query_shape)
    P, Hkv, ps, Dk = (int(x) for x in pages_shape)
    if min(B, Hq, L, D, P, Hkv, ps) <= 0:
        raise ValueError("all dimensions must be positive")
    if ps != page_size:
        raise ValueError("page pool's slot dimension must equal page_size")
    if Dk != D:
        raise ValueError("query and pages disagree on head_dim")
    if Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    bt = np.asarray(block_table)
    ctx = np.asarray(context_lens)
    if bt.ndim != 2 or bt.shape[0] != B or ctx.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and context_lens [B]")
    max_pages = bt.shape[1]
    for b in range(B):
        c = int(ctx[b])
        if c < 1 or c > max_pages * ps:
            raise ValueError(f"context_lens[{b}]={c} outside [1, max_pages*page_size]")
        if causal and c < L:
            raise ValueError(f"causal attention needs context_lens[{b}] >= L")
        used = bt[b, : math.ceil(c / ps)]
        if (used < 0).any() or (used >= P).any():
            raise ValueError(f"block_table row {b} names a page outside the pool")


def gather_history(pages: np.ndarray, table_row: np.ndarray, ctx: int, page_size: int) -> np.ndarray:
    """Dense ``[H_kv, ctx, D]`` float64 history of one sequence.

    Position s lives in physical page table_row[s // page_size] at slot
    s % page_size ("Week 3 Day 5", Task 1). Only positions < ctx are read.
    """
    pos = np.arange(ctx)
    phys = np.asarray(table_row)[pos // page_size]
    slot = pos % page_size
    rows = pages[phys, :, slot, :]  # [ctx, H_kv, D]
    return bf16_bits_to_f64(np.ascontiguousarray(rows.transpose(1, 0, 2)))


def visible_mask(query_len: int, ctx: int, causal: bool) -> np.ndarray:
    """Boolean ``[L, ctx]``: key s is visible to query row l.

    Causal: s <= l + ctx - L ("Week 3 Day 5", Task 2); otherwise every key
    of the context is visible.
    """
    s = np.arange(ctx)[None, :]
    if not causal:
        return np.ones((query_len, ctx), dtype=bool)
    l = np.arange(query_len)[:, None]
    return s <= l + ctx - query_len


def paged_attention_ref(
    query: np.ndarray,
    key_pages: np.ndarray,
    value_pages: np.ndarray,
    block_table: np.ndarray,
    context_lens: np.ndarray,
    page_size: int,
    scale: float,
    causal: bool = True,
    pairs: Optional[Iterable[Tuple[int, int]]] = None,
) -> np.ndarray:
    """Exact paged attention in float64.

    Arguments follow the operator's contract: ``query [B, H_q, L, D]``,
    ``key_pages``/``value_pages [num_pages, H_kv, page_size, D]`` (bf16 bits
    as uint16, or any float dtype), ``block_table [B, max_pages]``,
    ``context_lens [B]``. ``scale`` is widened from float32.

    Returns float64 ``[B, H_q, L, D]``; with ``pairs`` (a list of (b, h)),
    only those rows are computed and the result is ``[len(pairs), L, D]``.
    One (batch, kv head) history is gathered at a time to bound memory.
    """
    query = np.asarray(query)
    validate(query.shape, key_pages.shape, block_table, context_lens, page_size, causal)
    B, Hq, L, D = query.shape
    Hkv = key_pages.shape[1]
    scale64 = float(np.float32(scale))
    want = None if pairs is None else [(int(b), int(h)) for b, h in pairs]
    if want is None:
        out = np.empty((B, Hq, L, D), dtype=np.float64)
        todo = [(b, h) for b in range(B) for h in range(Hq)]
    else:
        out = np.empty((len(want), L, D), dtype=np.float64)
        todo = want
    by_batch = {}
    for idx, (b, h) in enumerate(todo):
        by_batch.setdefault(b, []).append((idx, h))
    for b, items in by_batch.items():
        ctx = int(context_lens[b])
        vis = visible_mask(L, ctx, causal)
        by_group = {}
        for idx, h in items:
            by_group.setdefault(kv_head_of(h, Hq, Hkv), []).append((idx, h))
        for g, heads in by_group.items():
            K = gather_history(key_pages[:, g : g + 1], block_table[b], ctx, page_size)[0]  # [ctx, D]
            V = gather_history(value_pages[:, g : g + 1], block_table[b], ctx, page_size)[0]
            for idx, h in heads:
                q = bf16_bits_to_f64(query[b, h])  # [L, D]
                S = scale64 * (q @ K.T)  # [L, ctx]
                S = np.where(vis, S, -np.inf)
                m = S.max(axis=1, keepdims=True)
                P = np.exp(S - m)
                o = (P @ V) / P.sum(axis=1, keepdims=True)
                if want is None:
                    out[b, h] = o
                else:
                    out[idx] = o
    return out
