"""Paged attention as explicit scalar loops -- TEST INFRASTRUCTURE ONLY.

The same definition as ``reference.py`` with no gather buffer, no matrix
products and no vectorisation: for each (sequence, query head, query row) it
walks the logical key positions one at a time, translates each through the
block table element by element ("Week 3 Day 5: Paged FlashAttention", Task 1),
applies the causal rule s <= l + context_len - L ("Week 3 Day 5", Task 2) and
the head map kv_head = q_head / (H_q / H_kv) ("Week 2 Day 5: Fused Decode
Attention", Task 1), and forms the softmax with ``math.exp`` and correctly
rounded ``math.fsum`` sums. Pure Python: tiny inputs only.
"""

from __future__ import annotations

import math

import numpy as np


def _widen(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def paged_attention_brute(query, key_pages, value_pages, block_table, context_lens, page_size, scale, causal=True):
    """float64 ``[B, H_q, L, D]`` from scalar loops (no validation beyond indexing)."""
    q = _widen(query).tolist()
    kp = _widen(key_pages)
    vp = _widen(value_pages)
    table = np.asarray(block_table).tolist()
    ctxs = [int(c) for c in np.asarray(context_lens).tolist()]
    B, Hq, L, D = np.asarray(query).shape
    Hkv = kp.shape[1]
    group = Hq // Hkv
    sc = float(np.float32(scale))
    out = np.zeros((B, Hq, L, D), dtype=np.float64)
    for b in range(B):
        ctx = ctxs[b]
        for h in range(Hq):
            g = h // group
            for l in range(L):
                last = (l + ctx - L) if causal else (ctx - 1)
                keys = []
                for s in range(ctx):
                    if s > last:
                        continue
                    phys = table[b][s // page_size]
                    slot = s % page_size
                    k = kp[phys, g, slot].tolist()
                    dot = math.fsum(q[b][h][l][d] * k[d] for d in range(D))
                    keys.append((sc * dot, phys, slot))
                mx = max(x for x, _, _ in keys)
                w = [math.exp(x - mx) for x, _, _ in keys]
                den = math.fsum(w)
                for d in range(D):
                    num = math.fsum(wi * vp[phys, g, slot, d] for wi, (_, phys, slot) in zip(w, keys))
                    out[b, h, l, d] = num / den
    return out


def paged_attention_masked_brute(query, key_pages, value_pages, block_table, context_lens, mask, page_size, scale,
                                 causal=True):
    """Scalar loops with an explicit additive mask ``mask[b][h][l][s]`` (natural-log units).

    A key is used when it is inside the context, allowed by the causal rule,
    has a mask entry (s < the mask's last axis) and that entry is not -inf;
    its score is scale * q.k plus the entry. A row with no usable key is NaN.
    """
    q = _widen(query).tolist()
    kp = _widen(key_pages)
    vp = _widen(value_pages)
    B, Hq, L, D = np.asarray(query).shape
    mk = np.broadcast_to(np.asarray(mask, dtype=np.float64), (B, Hq, L, np.asarray(mask).shape[3]))
    S = mk.shape[3]
    table = np.asarray(block_table).tolist()
    ctxs = [int(c) for c in np.asarray(context_lens).tolist()]
    Hkv = kp.shape[1]
    group = Hq // Hkv
    sc = float(np.float32(scale))
    out = np.zeros((B, Hq, L, D), dtype=np.float64)
    for b in range(B):
        ctx = ctxs[b]
        for h in range(Hq):
            g = h // group
            for l in range(L):
                last = (l + ctx - L) if causal else (ctx - 1)
                keys = []
                for s in range(min(ctx, S)):
                    add = float(mk[b, h, l, s])
                    if s > last or add == -math.inf:
                        continue
                    phys = table[b][s // page_size]
                    slot = s % page_size
                    k = kp[phys, g, slot].tolist()
                    dot = math.fsum(q[b][h][l][d] * k[d] for d in range(D))
                    keys.append((sc * dot + add, phys, slot))
                if not keys:
                    out[b, h, l, :] = math.nan
                    continue
                mx = max(x for x, _, _ in keys)
                w = [math.exp(x - mx) for x, _, _ in keys]
                den = math.fsum(w)
                for d in range(D):
                    num = math.fsum(wi * vp[phys, g, slot, d] for wi, (_, phys, slot) in zip(w, keys))
                    out[b, h, l, d] = num / den
    return out
