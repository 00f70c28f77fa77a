"""Plain float64 paged attention with an explicit additive mask -- TEST INFRASTRUCTURE ONLY.

The GPU path never imports this module.

The primitive of "Week 2 Day 5: Fused Decode Attention" (Task 1) accepts an
explicit mask normalised to ``[B * H_q, L, S]`` beside the causal flag, and
its per-position recurrence applies "the scale, optional mask, and causal
check" to each score (Task 2, step 3). Written out for paged K/V:

    score[b, h, l, s] = scale * q[b, h, l] . K_b[s] + mask[b, h, l, s]

for the keys s < context_lens[b] that the causal rule leaves visible (with
``causal``: s <= l + ctx - L); every other key is absent. The mask is in the
units of the score (natural-log weights): -inf removes a key, a finite value
multiplies its weight by exp(value). Readings where the pages are silent:

- the mask's last axis has ``S`` positions; a key at or past S has no mask
  entry and is absent (so a too-short mask can only hide keys, never read out
  of bounds);
- a row with no visible key has no softmax: its output is NaN, what 0 / 0
  gives in the definition.

Everything else follows ``reference.paged_attention_ref`` (gather through the
block table, GQA head map, float64 softmax).
"""

from __future__ import annotations

import numpy as np

from .reference import bf16_bits_to_f64, gather_history, kv_head_of, validate


def _scores(q: np.ndarray, K: np.ndarray, madd: np.ndarray, sc: float) -> np.ndarray:
    """scale * q K^T plus the mask entries (the mask is not scaled)."""
    return sc * (q @ K.T) + madd


def paged_attention_masked_ref(
    query: np.ndarray,
    key_pages: np.ndarray,
    value_pages: np.ndarray,
    block_table: np.ndarray,
    context_lens: np.ndarray,
    mask: np.ndarray,
    page_size: int,
    scale: float,
    causal: bool = True,
) -> np.ndarray:
    """float64 ``[B, H_q, L, D]``; ``mask`` is any float array broadcastable to ``[B, H_q, L, S]``."""
    query = np.asarray(query)
    B, Hq, L, D = query.shape
    # a context longer than L is required only for rows that must see a key:
    # a fully masked row is allowed (NaN), so validate without the causal check
    validate(query.shape, key_pages.shape, block_table, context_lens, page_size, False)
    m = np.asarray(mask, dtype=np.float64)
    if m.ndim != 4:
        raise ValueError("mask must have 4 axes (broadcastable to [B, H_q, L, S])")
    S = m.shape[3]
    m = np.broadcast_to(m, (B, Hq, L, S))
    Hkv = key_pages.shape[1]
    sc = float(np.float32(scale))
    out = np.empty((B, Hq, L, D), dtype=np.float64)
    for b in range(B):
        ctx = int(context_lens[b])
        s = np.arange(ctx)
        l = np.arange(L)[:, None]
        vis = (s[None, :] < S) & ((s[None, :] <= l + ctx - L) if causal else True)  # [L, ctx]
        madd = np.full((Hq, L, ctx), -np.inf)
        n = min(ctx, S)
        madd[:, :, :n] = m[b, :, :, :n]
        for g in range(Hkv):
            K = gather_history(key_pages[:, g : g + 1], block_table[b], ctx, page_size)[0]
            V = gather_history(value_pages[:, g : g + 1], block_table[b], ctx, page_size)[0]
            for h in range(Hq):
                if kv_head_of(h, Hq, Hkv) != g:
                    continue
                q = bf16_bits_to_f64(query[b, h])
                S_ = np.where(vis, _scores(q, K, madd[h], sc), -np.inf)
                mx = S_.max(axis=1, keepdims=True)
                with np.errstate(invalid="ignore"):
                    P = np.exp(S_ - mx)  # a row of -inf gives NaN weights, hence a NaN output
                    out[b, h] = (P @ V) / P.sum(axis=1, keepdims=True)
    return out
