"""MI355X-native paged attention operator.

The operator ``paged_attention``: exact scaled-dot-product attention over a
paged K/V pool (logical position -> block_table -> page slot), folded tile by
tile into an online softmax by hand-written gfx950 HIP kernels behind the C
ABI of ``include/paged_attention.h`` (``libpagedattn.so``), and its write
half ``kv_append`` (new tokens' K/V into their page slots);
``paged_attention_varlen`` runs a mixed batch (prefill chunks and decodes,
each sequence its own query length) in one call. PyTorch only provides
device memory and streams.

- ``native``    -- the ctypes binding (``paged_attention``,
  ``paged_attention_masked``, ``paged_attention_varlen``, ``kv_append``, ``workspace_bytes``,
  ``varlen_workspace_bytes``, ``schedule_for``, ``check_metadata``,
  ``check_varlen_metadata``)
- ``workloads`` -- seeded synthetic inputs of the measured configurations
- ``build``     -- hipcc build of the shared library
"""

from .native import (  # noqa: F401
    SCHEDULE_AUTO,
    SCHEDULE_DECODE,
    SCHEDULE_PREFILL,
    SCHEDULE_PREFILL_64X32,
    PagedAttentionError,
    check_metadata,
    check_varlen_metadata,
    kv_append,
    paged_attention,
    paged_attention_masked,
    paged_attention_varlen,
    schedule_for,
    varlen_workspace_bytes,
    workspace_bytes,
)
