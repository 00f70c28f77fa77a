"""Plain reference of the paged K/V write: new tokens' keys and values into their page slots.

TEST INFRASTRUCTURE ONLY (see the package docstring): the GPU path never
imports this module.

The write uses the same translation the reads do ("Week 3 Day 5: Paged
FlashAttention", Task 1: logical page = position / page_size, slot =
position % page_size, physical page = block_table[batch, logical page]).
Which positions the new tokens take is the convention of the attention
boundary: with context_lens counting the tokens after the append, token l
of a sequence with L new tokens sits at position context_len - L + l (the
position the attention gives query row l; the pages' causal decode after a
paged prefill appends the new token and then attends with the longer
context). Pure copies of bf16 bit patterns, so the result is exact.
"""

from __future__ import annotations

import numpy as np


def kv_append_ref(
    key_new: np.ndarray,
    value_new: np.ndarray,
    key_pages: np.ndarray,
    value_pages: np.ndarray,
    block_table: np.ndarray,
    context_lens: np.ndarray,
    page_size: int,
):
    """Returns copies of the two pools with the new tokens written.

    key_new / value_new: uint16 bf16 bits [B, H_kv, L, D]; key_pages /
    value_pages: uint16 [num_pages, H_kv, page_size, D]; block_table int
    [B, max_pages]; context_lens int [B] (after the append). Raises
    ValueError if a new position falls outside the block table or the pool,
    or if two new tokens would share a page slot.
    """
    B, H, L, D = key_new.shape
    if value_new.shape != key_new.shape or value_pages.shape != key_pages.shape:
        raise ValueError("keys and values must have matching shapes")
    num_pages, Hp, ps, Dp = key_pages.shape
    if Hp != H or Dp != D or ps != page_size:
        raise ValueError("pool shape does not match")
    kp = key_pages.copy()
    vp = value_pages.copy()
    seen = set()
    for b in range(B):
        ctx = int(context_lens[b])
        for l in range(L):
            pos = ctx - L + l
            if pos < 0:
                raise ValueError(f"sequence {b}: context length {ctx} < {L} new tokens")
            logical_page, slot = divmod(pos, page_size)
            if logical_page >= block_table.shape[1]:
                raise ValueError(f"sequence {b}: position {pos} past the block table")
            page = int(block_table[b, logical_page])
            if not 0 <= page < num_pages:
                raise ValueError(f"sequence {b}: page {page} not in the pool")
            if (page, slot) in seen:
                raise ValueError(f"page {page} slot {slot} written twice")
            seen.add((page, slot))
            kp[page, :, slot, :] = key_new[b, :, l, :]
            vp[page, :, slot, :] = value_new[b, :, l, :]
    return kp, vp
