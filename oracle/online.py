"""float64 tile-streaming model of the fused paged loop -- TEST INFRASTRUCTURE ONLY.

Follows the CPU model of "Day 22: the fused paged-attention kernel, modeled on
the CPU" (sections "What I added today" and "What I learned"): one program per
(sequence, query head, query row) walks the history one tile of ``tile`` keys
at a time. Each tile is read through the block table with a masked load (rows
past the context are not read and hold zero), scored against the query, then
-- as a second, separate mask -- every key that is past the context or hidden
by the causal rule gets score -inf. The tile is folded into the running
maximum, running denominator and running weighted-V sum; when the maximum
grows, the old state is rescaled by exp(m_old - m_new) first (the online
update of "Week 2 Day 5: Fused Decode Attention", Task 2). After the last tile
the sum is divided out.

``base2=True`` folds log2(e) into the scale once and uses 2**x instead of e**x
("Week 3 Day 5: Paged FlashAttention", Task 2) -- the same value up to
rounding. A tile whose keys are all hidden leaves the state untouched (the
whole-tile causal skip of the same task).
"""

from __future__ import annotations

import math
from typing import List, Tuple

import numpy as np


def _widen(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def tile_plan(ctx: int, tile: int) -> List[Tuple[int, List[int], List[int]]]:
    """Tiles covering a ``ctx``-key history: (start, loaded positions, masked positions).

    The last tile may be ragged: its positions at or past ``ctx`` are masked.
    """
    plan = []
    for t0 in range(0, ctx, tile):
        pos = list(range(t0, t0 + tile))
        plan.append((t0, [p for p in pos if p < ctx], [p for p in pos if p >= ctx]))
    return plan


def paged_attention_online(
    query,
    key_pages,
    value_pages,
    block_table,
    context_lens,
    page_size,
    scale,
    causal=True,
    tile=32,
    base2=False,
):
    """float64 ``[B, H_q, L, D]`` by the tile-streaming online softmax."""
    q_all = _widen(query)
    kp = np.asarray(key_pages)
    vp = np.asarray(value_pages)
    table = np.asarray(block_table)
    B, Hq, L, D = q_all.shape
    Hkv = kp.shape[1]
    group = Hq // Hkv
    sc = float(np.float32(scale))
    if base2:
        sc = sc * math.log2(math.e)
        expf = np.exp2
    else:
        expf = np.exp
    out = np.zeros((B, Hq, L, D), dtype=np.float64)
    for b in range(B):
        ctx = int(context_lens[b])
        for h in range(Hq):
            g = h // group
            for l in range(L):
                last = (l + ctx - L) if causal else (ctx - 1)
                m = -math.inf
                den = 0.0
                acc = np.zeros(D, dtype=np.float64)
                for t0 in range(0, ctx, tile):
                    if t0 > last:  # first key of the tile is past the last visible one
                        break
                    pos = np.arange(t0, t0 + tile)
                    in_ctx = pos < ctx
                    kt = np.zeros((tile, D), dtype=np.float64)
                    vt = np.zeros((tile, D), dtype=np.float64)
                    p_ok = pos[in_ctx]
                    phys = table[b, p_ok // page_size]
                    kt[in_ctx] = _widen(kp[phys, g, p_ok % page_size, :])
                    vt[in_ctx] = _widen(vp[phys, g, p_ok % page_size, :])
                    s = sc * (kt @ q_all[b, h, l])
                    s = np.where(in_ctx & (pos <= last), s, -np.inf)
                    tmax = s.max()
                    if tmax == -math.inf:
                        continue
                    new_m = max(m, tmax)
                    old = float(expf(m - new_m)) if m != -math.inf else 0.0
                    p = expf(s - new_m)
                    den = den * old + p.sum()
                    acc = acc * old + p @ vt
                    m = new_m
                out[b, h, l] = acc / den
    return out
