"""ctypes binding of libpagedattn.so (the C ABI of include/paged_attention.h).

Argument marshalling only: every step of the operator runs in the library's
HIP kernels. PyTorch supplies device memory and the current stream. If the
library has not been built this module raises at first use -- there is no
fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

PA_OK = 0
PA_ERR_INVALID = -1
PA_ERR_UNSUPPORTED = -2
PA_ERR_WORKSPACE = -3
PA_ERR_LAUNCH = -4
PA_ERR_METADATA = -5

SCHEDULE_AUTO = 0
SCHEDULE_DECODE = 1
SCHEDULE_PREFILL = 2
SCHEDULE_PREFILL_64X32 = 3  # 64 query rows x 32 keys per tile; explicit only

# Every symbol include/paged_attention.h declares.
EXPORTED = (
    "paged_attention",
    "paged_attention_ex",
    "paged_attention_workspace_bytes",
    "paged_attention_workspace_bytes_ex",
    "paged_attention_schedule",
    "paged_attention_check_metadata",
    "paged_attention_last_error",
    "paged_kv_append",
    "paged_attention_varlen",
    "paged_attention_varlen_ex",
    "paged_attention_varlen_workspace_bytes",
    "paged_attention_varlen_check_metadata",
    "paged_attention_masked",
    "paged_attention_static",
    "paged_attention_static_scratch_bytes",
)

_lib = None
_lock = threading.Lock()


class PagedAttentionError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"paged_attention error {code}: {message}")
        self.code = code


def load() -> ctypes.CDLL:
    """Load the shared library (once) and declare argument types."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m paged_flashattention_kv_amd.build` "
                "(the operator has no non-HIP implementation)"
            )
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        ex_args = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp, sz]
        lib.paged_attention.argtypes = ex_args + [vp]
        lib.paged_attention.restype = ctypes.c_int
        lib.paged_attention_ex.argtypes = ex_args + [i32, i32, vp]
        lib.paged_attention_ex.restype = ctypes.c_int
        lib.paged_attention_workspace_bytes.argtypes = [i32] * 7
        lib.paged_attention_workspace_bytes.restype = sz
        lib.paged_attention_workspace_bytes_ex.argtypes = [i32] * 9
        lib.paged_attention_workspace_bytes_ex.restype = sz
        lib.paged_attention_schedule.argtypes = [i32] * 7
        lib.paged_attention_schedule.restype = ctypes.c_int
        lib.paged_attention_check_metadata.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp]
        lib.paged_attention_check_metadata.restype = ctypes.c_int
        lib.paged_kv_append.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
        lib.paged_kv_append.restype = ctypes.c_int
        var_args = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp, sz]
        lib.paged_attention_varlen.argtypes = var_args + [vp]
        lib.paged_attention_varlen.restype = ctypes.c_int
        lib.paged_attention_varlen_ex.argtypes = var_args + [i32, i32, vp]
        lib.paged_attention_varlen_ex.restype = ctypes.c_int
        lib.paged_attention_varlen_workspace_bytes.argtypes = [i32] * 9
        lib.paged_attention_varlen_workspace_bytes.restype = sz
        lib.paged_attention_varlen_check_metadata.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
        lib.paged_attention_varlen_check_metadata.restype = ctypes.c_int
        i64 = ctypes.c_int64
        lib.paged_attention_masked.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, i32, i32, i32, i32,
                                               i32, i32, i32, i32, f32, i32, vp, sz, i32, i32, vp]
        lib.paged_attention_masked.restype = ctypes.c_int
        lib.paged_attention_static.argtypes = ex_args[:16] + [vp]
        lib.paged_attention_static.restype = ctypes.c_int
        lib.paged_attention_static_scratch_bytes.argtypes = []
        lib.paged_attention_static_scratch_bytes.restype = sz
        lib.paged_attention_last_error.argtypes = []
        lib.paged_attention_last_error.restype = ctypes.c_char_p
        _lib = lib
        return lib


def last_error() -> str:
    return load().paged_attention_last_error().decode()


def _check(code: int) -> None:
    if code != PA_OK:
        raise PagedAttentionError(code, last_error())


def workspace_bytes(batch, num_q_heads, num_kv_heads, query_len, head_dim, page_size, max_pages,
                    schedule=SCHEDULE_AUTO, decode_work_items=0) -> int:
    n = load().paged_attention_workspace_bytes_ex(batch, num_q_heads, num_kv_heads, query_len, head_dim,
                                                  page_size, max_pages, schedule, decode_work_items)
    if n == ctypes.c_size_t(-1).value:
        raise PagedAttentionError(PA_ERR_INVALID, last_error())
    return int(n)


def schedule_for(batch, num_q_heads, num_kv_heads, query_len, head_dim, page_size, max_pages) -> int:
    r = load().paged_attention_schedule(batch, num_q_heads, num_kv_heads, query_len, head_dim, page_size, max_pages)
    if r < 0:
        raise PagedAttentionError(r, last_error())
    return int(r)


def _stream_ptr(stream: Optional[torch.cuda.Stream], device: torch.device) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return int(s.cuda_stream)


def _launch_stream(stream: Optional[torch.cuda.Stream], device: torch.device) -> torch.cuda.Stream:
    return stream if stream is not None else torch.cuda.current_stream(device)


def _temporaries(s: torch.cuda.Stream, out: Optional[torch.Tensor], like: torch.Tensor, ws_need: int,
                 workspace: Optional[torch.Tensor]):
    """``out`` and the workspace, allocated (and the workspace zero-filled) on the launch stream ``s``.

    Allocating on ``s`` orders the zero fill before the kernel that reads the
    counters, and ties the memory to ``s`` in torch's caching allocator: a
    local workspace freed on return is handed out again only to later work on
    ``s``, after the kernel, whichever stream the caller is on.
    """
    with torch.cuda.stream(s):
        if out is None:
            out = torch.empty_like(like)
        if ws_need > 0 and workspace is None:
            workspace = torch.zeros(ws_need, dtype=torch.uint8, device=like.device)
    return out, workspace


def _require(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int, device: torch.device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    if t.device != device:
        raise ValueError(f"{name} must live on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def paged_attention(
    query: torch.Tensor,
    key_pages: torch.Tensor,
    value_pages: torch.Tensor,
    block_table: torch.Tensor,
    context_lens: torch.Tensor,
    page_size: int,
    scale: Optional[float] = None,
    causal: bool = True,
    *,
    out: Optional[torch.Tensor] = None,
    workspace: Optional[torch.Tensor] = None,
    schedule: int = SCHEDULE_AUTO,
    decode_work_items: int = 0,
    stream: Optional[torch.cuda.Stream] = None,
) -> torch.Tensor:
    """Paged attention on the GPU ("Week 3 Day 5: Paged FlashAttention", "Keep the Day 4 Interface").

    query [B, H_q, L, D] bf16; key_pages / value_pages [num_pages, H_kv,
    page_size, D] bf16; block_table [B, max_pages] int32; context_lens [B]
    int32 -- all on one GPU. ``scale`` defaults to 1/sqrt(D). Returns
    ``out`` [B, H_q, L, D] bf16 (allocated when not given). A caller-owned
    ``workspace`` (uint8, at least ``workspace_bytes(...)``) must be
    zero-filled before its first use and can then be reused across calls on
    one stream. The call is asynchronous on ``stream`` (default: the current
    stream). Inputs must be ready on ``stream``; an ``out`` or workspace
    allocated here is allocated on ``stream``, so work on another stream that
    reads the returned ``out`` must first wait for ``stream``.
    """
    dev = query.device
    if dev.type != "cuda":
        raise ValueError("query must be a GPU tensor")
    _require(query, "query", torch.bfloat16, 4, dev)
    _require(key_pages, "key_pages", torch.bfloat16, 4, dev)
    _require(value_pages, "value_pages", torch.bfloat16, 4, dev)
    _require(block_table, "block_table", torch.int32, 2, dev)
    _require(context_lens, "context_lens", torch.int32, 1, dev)
    B, Hq, L, D = query.shape
    P, Hkv, ps, Dk = key_pages.shape
    if tuple(value_pages.shape) != tuple(key_pages.shape):
        raise ValueError("key_pages and value_pages must have the same shape")
    if ps != page_size or Dk != D:
        raise ValueError("page pool shape does not match page_size / head_dim")
    if block_table.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_table and context_lens need one row per sequence")
    max_pages = block_table.shape[1]
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if out is not None:
        _require(out, "out", torch.bfloat16, 4, dev)
        if tuple(out.shape) != tuple(query.shape):
            raise ValueError("out must have the query's shape")
    need = workspace_bytes(B, Hq, Hkv, L, D, ps, max_pages, schedule, decode_work_items)
    s = _launch_stream(stream, dev)
    out, workspace = _temporaries(s, out, query, need, workspace)
    ws_ptr, ws_len = None, 0
    if need > 0:
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the query's device")
        ws_ptr, ws_len = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    lib = load()
    rc = lib.paged_attention_ex(
        query.data_ptr(), key_pages.data_ptr(), value_pages.data_ptr(), block_table.data_ptr(),
        context_lens.data_ptr(), out.data_ptr(), B, Hq, Hkv, L, D, P, ps, max_pages, float(scale),
        1 if causal else 0, ws_ptr, ws_len, int(schedule), int(decode_work_items), int(s.cuda_stream),
    )
    _check(rc)
    return out


def kv_append(
    key_new: torch.Tensor,
    value_new: torch.Tensor,
    key_pages: torch.Tensor,
    value_pages: torch.Tensor,
    block_table: torch.Tensor,
    context_lens: torch.Tensor,
    page_size: int,
    *,
    stream: Optional[torch.cuda.Stream] = None,
) -> None:
    """Writes new tokens' K/V into their page slots, in place ("Week 3 Day 5: Paged FlashAttention").

    key_new / value_new [B, H_kv, L_new, D] bf16; key_pages / value_pages
    [num_pages, H_kv, page_size, D] bf16 (updated); block_table [B,
    max_pages] int32; context_lens [B] int32 = context lengths after the
    append, so token l of sequence b goes to position context_lens[b] -
    L_new + l. Asynchronous on ``stream`` (default: the current stream).
    """
    dev = key_new.device
    if dev.type != "cuda":
        raise ValueError("key_new must be a GPU tensor")
    _require(key_new, "key_new", torch.bfloat16, 4, dev)
    _require(value_new, "value_new", torch.bfloat16, 4, dev)
    _require(key_pages, "key_pages", torch.bfloat16, 4, dev)
    _require(value_pages, "value_pages", torch.bfloat16, 4, dev)
    _require(block_table, "block_table", torch.int32, 2, dev)
    _require(context_lens, "context_lens", torch.int32, 1, dev)
    B, Hkv, L, D = key_new.shape
    P, Hp, ps, Dp = key_pages.shape
    if tuple(value_new.shape) != tuple(key_new.shape) or tuple(value_pages.shape) != tuple(key_pages.shape):
        raise ValueError("keys and values must have matching shapes")
    if ps != page_size or Dp != D or Hp != Hkv:
        raise ValueError("page pool shape does not match page_size / kv heads / head_dim")
    if block_table.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_table and context_lens need one row per sequence")
    rc = load().paged_kv_append(
        key_new.data_ptr(), value_new.data_ptr(), key_pages.data_ptr(), value_pages.data_ptr(),
        block_table.data_ptr(), context_lens.data_ptr(), B, Hkv, L, D, P, ps, block_table.shape[1],
        _stream_ptr(stream, dev),
    )
    _check(rc)


def check_metadata(block_table: torch.Tensor, context_lens: torch.Tensor, num_pages: int, page_size: int,
                   query_len: int, causal: bool = True, stream: Optional[torch.cuda.Stream] = None) -> None:
    """Debug check of the device-side metadata preconditions (synchronises the stream)."""
    dev = block_table.device
    _require(block_table, "block_table", torch.int32, 2, dev)
    _require(context_lens, "context_lens", torch.int32, 1, dev)
    rc = load().paged_attention_check_metadata(
        block_table.data_ptr(), context_lens.data_ptr(), block_table.shape[0], block_table.shape[1],
        num_pages, page_size, query_len, 1 if causal else 0, _stream_ptr(stream, dev),
    )
    _check(rc)


def varlen_workspace_bytes(batch, num_q_heads, num_kv_heads, max_query_len, head_dim, page_size, max_pages,
                           decode_max_len=-1, decode_work_items=0) -> int:
    n = load().paged_attention_varlen_workspace_bytes(batch, num_q_heads, num_kv_heads, max_query_len, head_dim,
                                                      page_size, max_pages, decode_max_len, decode_work_items)
    if n == ctypes.c_size_t(-1).value:
        raise PagedAttentionError(PA_ERR_INVALID, last_error())
    return int(n)


def paged_attention_varlen(
    query: torch.Tensor,
    key_pages: torch.Tensor,
    value_pages: torch.Tensor,
    block_table: torch.Tensor,
    context_lens: torch.Tensor,
    query_start: torch.Tensor,
    max_query_len: int,
    page_size: int,
    scale: Optional[float] = None,
    causal: bool = True,
    *,
    out: Optional[torch.Tensor] = None,
    workspace: Optional[torch.Tensor] = None,
    decode_max_len: int = -1,
    decode_work_items: int = 0,
    stream: Optional[torch.cuda.Stream] = None,
) -> torch.Tensor:
    """Paged attention over a mixed batch: each sequence its own query length.

    query [T, H_q, D] bf16 packed token-major, sequence b owning tokens
    [query_start[b], query_start[b + 1]); query_start [B + 1] int32;
    ``max_query_len`` a host bound on every sequence's query length (no
    device read happens here). Pools, block_table, context_lens, scale and
    causal as for :func:`paged_attention`; query row l of sequence b sits at
    position context_lens[b] - L_b + l ("Week 3 Day 5: Paged
    FlashAttention", Task 4: short queries take the decode schedule, long
    ones the tiled prefill schedule -- chosen per sequence). Returns ``out``
    [T, H_q, D] bf16. ``decode_max_len`` / ``decode_work_items``: see
    paged_attention_varlen_ex in the C header.
    """
    dev = query.device
    if dev.type != "cuda":
        raise ValueError("query must be a GPU tensor")
    _require(query, "query", torch.bfloat16, 3, dev)
    _require(key_pages, "key_pages", torch.bfloat16, 4, dev)
    _require(value_pages, "value_pages", torch.bfloat16, 4, dev)
    _require(block_table, "block_table", torch.int32, 2, dev)
    _require(context_lens, "context_lens", torch.int32, 1, dev)
    _require(query_start, "query_start", torch.int32, 1, dev)
    T, Hq, D = query.shape
    P, Hkv, ps, Dk = key_pages.shape
    B = context_lens.shape[0]
    if tuple(value_pages.shape) != tuple(key_pages.shape):
        raise ValueError("key_pages and value_pages must have the same shape")
    if ps != page_size or Dk != D:
        raise ValueError("page pool shape does not match page_size / head_dim")
    if block_table.shape[0] != B or query_start.shape[0] != B + 1:
        raise ValueError("block_table needs one row per sequence and query_start B + 1 entries")
    max_pages = block_table.shape[1]
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if out is not None:
        _require(out, "out", torch.bfloat16, 3, dev)
        if tuple(out.shape) != tuple(query.shape):
            raise ValueError("out must have the query's shape")
    s = _launch_stream(stream, dev)
    if T == 0:
        return _temporaries(s, out, query, 0, None)[0]
    need = varlen_workspace_bytes(B, Hq, Hkv, max_query_len, D, ps, max_pages, decode_max_len, decode_work_items)
    out, workspace = _temporaries(s, out, query, need, workspace)
    ws_ptr, ws_len = None, 0
    if need > 0:
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the query's device")
        ws_ptr, ws_len = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    rc = load().paged_attention_varlen_ex(
        query.data_ptr(), key_pages.data_ptr(), value_pages.data_ptr(), block_table.data_ptr(),
        context_lens.data_ptr(), query_start.data_ptr(), out.data_ptr(), B, Hq, Hkv, T, int(max_query_len), D, P,
        ps, max_pages, float(scale), 1 if causal else 0, ws_ptr, ws_len, int(decode_max_len),
        int(decode_work_items), int(s.cuda_stream),
    )
    _check(rc)
    return out


def check_varlen_metadata(block_table: torch.Tensor, context_lens: torch.Tensor, query_start: torch.Tensor,
                          num_pages: int, page_size: int, total_query: int, max_query_len: int,
                          causal: bool = True, stream: Optional[torch.cuda.Stream] = None) -> None:
    """Debug check of a mixed batch's device-side metadata (synchronises the stream)."""
    dev = block_table.device
    _require(block_table, "block_table", torch.int32, 2, dev)
    _require(context_lens, "context_lens", torch.int32, 1, dev)
    _require(query_start, "query_start", torch.int32, 1, dev)
    rc = load().paged_attention_varlen_check_metadata(
        block_table.data_ptr(), context_lens.data_ptr(), query_start.data_ptr(), block_table.shape[0],
        block_table.shape[1], num_pages, page_size, total_query, max_query_len, 1 if causal else 0,
        _stream_ptr(stream, dev),
    )
    _check(rc)


def paged_attention_masked(
    query: torch.Tensor,
    key_pages: torch.Tensor,
    value_pages: torch.Tensor,
    block_table: torch.Tensor,
    context_lens: torch.Tensor,
    mask: torch.Tensor,
    page_size: int,
    scale: Optional[float] = None,
    causal: bool = True,
    *,
    out: Optional[torch.Tensor] = None,
    workspace: Optional[torch.Tensor] = None,
    schedule: int = SCHEDULE_AUTO,
    decode_work_items: int = 0,
    stream: Optional[torch.cuda.Stream] = None,
) -> torch.Tensor:
    """Paged attention with an explicit additive mask beside the causal flag.

    ``mask`` is a float32 GPU tensor of 4 axes [B or 1, H_q or 1, L or 1, S]
    (an axis of size 1 -- or an expanded view -- broadcasts), natural-log
    units, last axis contiguous: score = scale * q.k + mask; -inf removes a
    key, keys at or past S are absent ("Week 2 Day 5: Fused Decode
    Attention", Tasks 1-2). Other arguments as :func:`paged_attention`.
    """
    dev = query.device
    if dev.type != "cuda":
        raise ValueError("query must be a GPU tensor")
    _require(query, "query", torch.bfloat16, 4, dev)
    _require(key_pages, "key_pages", torch.bfloat16, 4, dev)
    _require(value_pages, "value_pages", torch.bfloat16, 4, dev)
    _require(block_table, "block_table", torch.int32, 2, dev)
    _require(context_lens, "context_lens", torch.int32, 1, dev)
    if not isinstance(mask, torch.Tensor) or mask.dtype != torch.float32 or mask.dim() != 4 or mask.device != dev:
        raise TypeError("mask must be a 4-axis float32 tensor on the query's device")
    B, Hq, L, D = query.shape
    for ax, (n, full) in enumerate(zip(mask.shape[:3], (B, Hq, L))):
        if n not in (1, full):
            raise ValueError(f"mask axis {ax} has size {n}, expected 1 or {full}")
    if mask.shape[3] < 1 or (mask.shape[3] > 1 and mask.stride(3) != 1):
        raise ValueError("the mask's last axis must be non-empty and contiguous")
    strides = [0 if mask.shape[i] == 1 else mask.stride(i) for i in range(3)]
    if min(strides) < 0:
        raise ValueError("negative mask strides are not supported")
    P, Hkv, ps, Dk = key_pages.shape
    if tuple(value_pages.shape) != tuple(key_pages.shape):
        raise ValueError("key_pages and value_pages must have the same shape")
    if ps != page_size or Dk != D:
        raise ValueError("page pool shape does not match page_size / head_dim")
    if block_table.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_table and context_lens need one row per sequence")
    max_pages = block_table.shape[1]
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if out is not None:
        _require(out, "out", torch.bfloat16, 4, dev)
        if tuple(out.shape) != tuple(query.shape):
            raise ValueError("out must have the query's shape")
    need = workspace_bytes(B, Hq, Hkv, L, D, ps, max_pages, schedule, decode_work_items)
    s = _launch_stream(stream, dev)
    out, workspace = _temporaries(s, out, query, need, workspace)
    ws_ptr, ws_len = None, 0
    if need > 0:
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the query's device")
        ws_ptr, ws_len = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    rc = load().paged_attention_masked(
        query.data_ptr(), key_pages.data_ptr(), value_pages.data_ptr(), block_table.data_ptr(),
        context_lens.data_ptr(), mask.data_ptr(), strides[0], strides[1], strides[2], int(mask.shape[3]),
        out.data_ptr(), B, Hq, Hkv, L, D, P, ps, max_pages, float(scale), 1 if causal else 0, ws_ptr, ws_len,
        int(schedule), int(decode_work_items), int(s.cuda_stream),
    )
    _check(rc)
    return out
