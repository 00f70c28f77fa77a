"""MI355X-native paged attention operator.

The operator ``paged_attention``: exact scaled-dot-product attention over a
paged K/V pool (logical position -> block_table -> page slot), folded tile by
tile into an online softmax by hand-written gfx950 HIP kernels behind the C
ABI of ``include/paged_attention.h`` (``libpagedattn.so``), and its write
half ``kv_append`` (new tokens' K/V into their page slots). PyTorch only
provides device memory and streams.

- ``native``    -- the ctypes binding (``paged_attention``, ``kv_append``,
  ``workspace_bytes``, ``schedule_for``, ``check_metadata``)
- ``workloads`` -- seeded synthetic inputs of the five measured configurations
- ``build``     -- hipcc build of the shared library
"""

from .native import (  # noqa: F401
    SCHEDULE_AUTO,
    SCHEDULE_DECODE,
    SCHEDULE_PREFILL,
    PagedAttentionError,
    check_metadata,
    kv_append,
    paged_attention,
    schedule_for,
    workspace_bytes,
)
