"""Plain float64 paged attention over a mixed batch: each sequence has its own query length.

TEST INFRASTRUCTURE ONLY (see the package docstring): the GPU path never
imports this module.

A continuous-batching step mixes sequences that prefill a chunk of their
prompt with sequences that decode one token ("Week 3 Day 5: Paged
FlashAttention", Task 4: long prefills take the tiled path, short queries
the vector decode path, and the result is measured on a continuous-serving
trace whose prefill proceeds in fixed-size steps). The attention of one
sequence does not depend on any other sequence of the batch, so the mixed
batch is the plain definition applied to every sequence on its own:

- the queries of all sequences are packed token-major, ``query[T, H_q, D]``;
  sequence b owns tokens ``[query_start[b], query_start[b + 1])``, so its
  query length is ``L_b = query_start[b + 1] - query_start[b]`` (0 allowed);
- query row l of sequence b sits at logical position ``context_lens[b] -
  L_b + l`` (the last L_b positions of its context, as for a uniform batch);
- with ``causal``, key s is visible to that row iff ``s <= context_lens[b] -
  L_b + l`` ("Week 3 Day 5", Task 2); otherwise every key of the context is;
- keys come from the pages through the block table ("Week 3 Day 5", Task 1),
  query head h reads K/V head h / (H_q / H_kv) ("Week 2 Day 5: Fused Decode
  Attention", Task 1).

Steps 1-5 of ``reference.paged_attention_ref`` are taken per sequence: the
history is gathered, scores and softmax are float64.
"""

from __future__ import annotations

import math

import numpy as np

from .reference import bf16_bits_to_f64, gather_history, kv_head_of, visible_mask


def validate_varlen(
    query_shape,
    pages_shape,
    block_table: np.ndarray,
    context_lens: np.ndarray,
    query_start: np.ndarray,
    page_size: int,
    causal: bool,
) -> None:
    """Raise ``ValueError`` unless the mixed batch is a well-defined attention.

    ``query_start`` is ``[B + 1]``, starts at 0, never decreases and ends at
    T. A sequence with at least one query row needs 1 <= ctx <= max_pages *
    page_size, ctx >= L_b when causal, and valid page ids for the pages it
    uses. A sequence with no query row is never read.
    """
    T, Hq, D = (int(x) for x in query_shape)
    P, Hkv, ps, Dk = (int(x) for x in pages_shape)
    if min(Hq, D, P, Hkv, ps) <= 0 or T < 0:
        raise ValueError("dimensions must be positive (T may be 0)")
    if ps != page_size or Dk != D:
        raise ValueError("page pool does not match page_size / head_dim")
    if Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    qs = np.asarray(query_start).astype(np.int64)
    bt = np.asarray(block_table)
    ctx = np.asarray(context_lens)
    B = ctx.shape[0]
    if qs.shape != (B + 1,) or bt.ndim != 2 or bt.shape[0] != B:
        raise ValueError("query_start must be [B + 1] and block_table [B, max_pages]")
    if qs[0] != 0 or qs[-1] != T or (np.diff(qs) < 0).any():
        raise ValueError("query_start must start at 0, never decrease and end at T")
    max_pages = bt.shape[1]
    for b in range(B):
        L = int(qs[b + 1] - qs[b])
        if L == 0:
            continue
        c = int(ctx[b])
        if c < 1 or c > max_pages * ps:
            raise ValueError(f"context_lens[{b}]={c} outside [1, max_pages*page_size]")
        if causal and c < L:
            raise ValueError(f"causal attention needs context_lens[{b}] >= its query length")
        used = bt[b, : math.ceil(c / ps)]
        if (used < 0).any() or (used >= P).any():
            raise ValueError(f"block_table row {b} names a page outside the pool")


def paged_attention_varlen_ref(
    query: np.ndarray,
    key_pages: np.ndarray,
    value_pages: np.ndarray,
    block_table: np.ndarray,
    context_lens: np.ndarray,
    query_start: np.ndarray,
    page_size: int,
    scale: float,
    causal: bool = True,
) -> np.ndarray:
    """Exact attention of a mixed batch in float64.

    ``query [T, H_q, D]`` (bf16 bits as uint16, or a float dtype), pools
    ``[num_pages, H_kv, page_size, D]``, ``block_table [B, max_pages]``,
    ``context_lens [B]``, ``query_start [B + 1]``. Returns float64
    ``[T, H_q, D]``: row t of sequence b (query_start[b] <= t <
    query_start[b + 1]) is query row t - query_start[b] of that sequence.
    """
    query = np.asarray(query)
    validate_varlen(query.shape, key_pages.shape, block_table, context_lens, query_start, page_size, causal)
    T, Hq, D = query.shape
    Hkv = key_pages.shape[1]
    scale64 = float(np.float32(scale))
    qs = np.asarray(query_start).astype(np.int64)
    out = np.empty((T, Hq, D), dtype=np.float64)
    for b in range(len(context_lens)):
        t0, t1 = int(qs[b]), int(qs[b + 1])
        L = t1 - t0
        if L == 0:
            continue
        ctx = int(context_lens[b])
        vis = visible_mask(L, ctx, causal)  # [L, ctx]
        for g in range(Hkv):
            K = gather_history(key_pages[:, g : g + 1], block_table[b], ctx, page_size)[0]  # [ctx, D]
            V = gather_history(value_pages[:, g : g + 1], block_table[b], ctx, page_size)[0]
            for h in range(Hq):
                if kv_head_of(h, Hq, Hkv) != g:
                    continue
                q = bf16_bits_to_f64(query[t0:t1, h])  # [L, D]
                S = np.where(vis, scale64 * (q @ K.T), -np.inf)
                m = S.max(axis=1, keepdims=True)
                P = np.exp(S - m)
                out[t0:t1, h] = (P @ V) / P.sum(axis=1, keepdims=True)
    return out
