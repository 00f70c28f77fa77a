"""CPU oracle for paged attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package. The GPU product path
(``paged_flashattention_kv_amd``) never imports it, and this package imports
nothing from the product path: the two share no code.

Contents, each citing the passage it follows (pages: "Week 3 Day 5: Paged
FlashAttention" (tiny-llm), "Day 22: the fused paged-attention kernel, modeled
on the CPU" (nanoserve), "Week 2 Day 5: Fused Decode Attention" (tiny-llm)):

- ``reference.paged_attention_ref`` -- the plain definition: gather each
  sequence's paged history into a dense buffer, then one float64 softmax.
- ``brute.paged_attention_brute`` -- the same definition as explicit scalar
  loops (``math.exp``/``math.fsum``), for tiny inputs.
- ``online.paged_attention_online`` -- a float64 tile-streaming model of the
  fused loop (masked tile load through the block table, separate -inf score
  mask, running max / denominator / weighted-V fold).
- ``append.kv_append_ref`` -- the write half: new tokens' K/V copied into
  their page slots through the same translation.
- ``masked.paged_attention_masked_ref`` / ``brute.paged_attention_masked_brute``
  -- an explicit additive mask beside the causal flag ("Week 2 Day 5",
  Tasks 1 and 2), vectorised and as scalar loops.
- ``varlen.paged_attention_varlen_ref`` -- a mixed batch (each sequence its
  own query length, queries packed token-major): the definition applied to
  every sequence on its own.

Pins (tests marked ``not gpu``) tie these to brute force, a library special
case (torch scaled-dot-product attention in float64), closed forms and
invariants. Every function here is pinned; none is "parity unpinned".
"""

from .reference import (
    bf16_bits_to_f64,
    gather_history,
    kv_head_of,
    paged_attention_ref,
    validate,
    visible_mask,
)
from .brute import paged_attention_brute, paged_attention_masked_brute
from .masked import paged_attention_masked_ref
from .online import paged_attention_online, tile_plan
from .append import kv_append_ref
from .varlen import paged_attention_varlen_ref, validate_varlen

__all__ = [
    "kv_append_ref",
    "paged_attention_varlen_ref",
    "validate_varlen",
    "bf16_bits_to_f64",
    "gather_history",
    "kv_head_of",
    "paged_attention_ref",
    "paged_attention_brute",
    "paged_attention_masked_brute",
    "paged_attention_masked_ref",
    "paged_attention_online",
    "tile_plan",
    "validate",
    "visible_mask",
]
