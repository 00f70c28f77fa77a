"""Seeded synthetic inputs for the paged attention operator.

This module holds none of the attention arithmetic. It draws random numbers,
rounds them to bf16 bit patterns, and lays out a page pool, a block table and
context lengths. The CPU oracle (through the tests) and the GPU binding both
consume the arrays it returns; neither of them is imported here.

Layouts (all row-major, C-contiguous):

- ``query``       uint16 bf16 bits ``[B, H_q, L, D]``
- ``key_pages``   uint16 bf16 bits ``[num_pages, H_kv, page_size, D]``
- ``value_pages`` uint16 bf16 bits ``[num_pages, H_kv, page_size, D]``
- ``block_table`` int32 ``[B, max_pages]``; entries past a sequence's last
  page are ``-1``
- ``context_lens`` int32 ``[B]``

Draw order for one problem: context lengths, then the page permutation, then
q, then k, then v, all from ``numpy.random.Generator(PCG64(seed))``. Values are
N(0, 1) drawn in float32 and rounded to bf16 with round-to-nearest-even.

The five named workloads follow the configurations the operator is measured
on: a tiny causal prefill, a decode batch at the Qwen3-4B attention shape, a
long causal prefill, a chunked-prefill continuation and a long-context decode
with page-crossing tiles.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Callable, Dict, Optional, Sequence, Union

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

_CHUNK = 1 << 24  # elements per rounding chunk (bounds temporaries)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    NaN inputs map to the canonical quiet NaN 0x7FC0. Works in chunks so that
    a 1 GiB pool needs no more than a few hundred MB of temporaries.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    for lo in range(0, flat.size, _CHUNK):
        u = flat[lo:lo + _CHUNK].view(np.uint32)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
        r = r.astype(np.uint16)
        nan = np.isnan(flat[lo:lo + _CHUNK])
        if nan.any():
            r[nan] = BF16_NAN
        out[lo:lo + _CHUNK] = r
    return out.reshape(x.shape)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape: Sequence[int]) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for lo in range(0, n, _CHUNK):
        m = min(_CHUNK, n - lo)
        out[lo:lo + m] = f32_to_bf16_bits(rng.standard_normal(m, dtype=np.float32))
    return out.reshape(tuple(shape))


@dataclasses.dataclass
class PagedProblem:
    """One synthetic paged-attention input set (host arrays)."""

    name: str
    query: np.ndarray
    key_pages: np.ndarray
    value_pages: np.ndarray
    block_table: np.ndarray
    context_lens: np.ndarray
    page_size: int
    scale: float
    causal: bool
    seed: int

    @property
    def batch(self) -> int:
        return int(self.query.shape[0])

    @property
    def num_q_heads(self) -> int:
        return int(self.query.shape[1])

    @property
    def query_len(self) -> int:
        return int(self.query.shape[2])

    @property
    def head_dim(self) -> int:
        return int(self.query.shape[3])

    @property
    def num_kv_heads(self) -> int:
        return int(self.key_pages.shape[1])

    @property
    def num_pages(self) -> int:
        return int(self.key_pages.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def kv_bytes(self) -> int:
        """K+V bytes the method must read: every visible logical position once."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_dim * 2 * 2

    def visible_pairs(self) -> int:
        """Number of (query row, key) pairs that are visible, summed over the batch."""
        L = self.query_len
        total = 0
        for c in self.context_lens.tolist():
            if self.causal:
                # row l sees keys 0 .. l + c - L  ->  (l + c - L + 1) keys
                total += L * (c - L) + L * (L + 1) // 2
            else:
                total += L * c
        return total

    def flops(self) -> int:
        """Algorithmic FLOPs: 2*D for Q.K and 2*D for P.V per visible pair per q head."""
        return 4 * self.head_dim * self.num_q_heads * self.visible_pairs()


def make_problem(
    seed: int,
    batch: int,
    num_q_heads: int,
    num_kv_heads: int,
    query_len: int,
    head_dim: int,
    page_size: int,
    context_lens: Union[Sequence[int], Callable[[np.random.Generator], Sequence[int]]],
    pool_pages: Optional[int] = None,
    causal: bool = True,
    scale: Optional[float] = None,
    poison: bool = False,
    name: str = "custom",
    max_pages: Optional[int] = None,
) -> PagedProblem:
    """Draw one problem.

    ``context_lens`` is either a fixed list or a function of the generator (so
    that random lengths are drawn first, as the draw order requires).
    ``pool_pages`` defaults to the total number of pages the batch needs; a
    larger pool leaves unused pages. With ``poison`` every unused page and
    every slot past a sequence's end holds bf16 NaN, so a read of them shows.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if callable(context_lens):
        ctx = np.asarray(context_lens(rng), dtype=np.int64)
    else:
        ctx = np.asarray(context_lens, dtype=np.int64)
    if ctx.shape != (batch,):
        raise ValueError("context_lens must have one entry per sequence")
    pages_per_seq = [int(math.ceil(c / page_size)) for c in ctx.tolist()]
    needed = int(sum(pages_per_seq))
    if pool_pages is None:
        pool_pages = needed
    if pool_pages < needed:
        raise ValueError("pool too small")
    width = max(pages_per_seq) if max_pages is None else int(max_pages)
    width = max(width, 1)
    perm = rng.permutation(pool_pages).astype(np.int32)
    table = np.full((batch, width), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(pages_per_seq):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    q = _normal_bf16(rng, (batch, num_q_heads, query_len, head_dim))
    k = _normal_bf16(rng, (pool_pages, num_kv_heads, page_size, head_dim))
    v = _normal_bf16(rng, (pool_pages, num_kv_heads, page_size, head_dim))
    if poison:
        used = np.zeros(pool_pages, dtype=bool)
        for b, n in enumerate(pages_per_seq):
            used[table[b, :n]] = True
            tail = int(ctx[b]) - (n - 1) * page_size  # valid slots in the last page
            if tail < page_size:
                last = table[b, n - 1]
                k[last, :, tail:, :] = BF16_NAN
                v[last, :, tail:, :] = BF16_NAN
        k[~used] = BF16_NAN
        v[~used] = BF16_NAN
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(head_dim)))
    return PagedProblem(
        name=name,
        query=q,
        key_pages=k,
        value_pages=v,
        block_table=table,
        context_lens=ctx.astype(np.int32),
        page_size=int(page_size),
        scale=float(np.float32(scale)),
        causal=bool(causal),
        seed=int(seed),
    )


def _uniform_not_multiple(lo: int, hi: int, n: int, tile: int = 32):
    """Uniform integers in [lo, hi] nudged off multiples of ``tile``."""

    def draw(rng: np.random.Generator):
        c = rng.integers(lo, hi + 1, size=n)
        bump = (c % tile) == 0
        c = np.where(bump & (c < hi), c + 1, np.where(bump, c - 1, c))
        return c

    return draw


def _continuation_lens(lo: int, hi: int, n: int, new: int, tile: int = 32):
    """History h ~ U[lo, hi] plus ``new`` queries; total nudged off tile multiples."""

    def draw(rng: np.random.Generator):
        h = rng.integers(lo, hi + 1, size=n)
        c = h + new
        bump = (c % tile) == 0
        return np.where(bump, c + 1, c)

    return draw


# name -> (seed, keyword arguments of make_problem)
CONFIGS: Dict[str, dict] = {
    # Tiny causal prefill: GQA 2:1, L = ctx = 13, page_size 4, 4 pages drawn
    # as scattered ids from a pool of 8.
    "tiny_prefill": dict(
        seed=1, batch=1, num_q_heads=4, num_kv_heads=2, query_len=13, head_dim=128,
        page_size=4, context_lens=[13], pool_pages=8, causal=True,
    ),
    # Decode batch at the Qwen3-4B attention shape: ctx ~ U[128, 4096], not
    # tile multiples, 128-token pages, pool = pages needed, random permutation.
    "decode_batch": dict(
        seed=2, batch=64, num_q_heads=32, num_kv_heads=8, query_len=1, head_dim=128,
        page_size=128, context_lens=_uniform_not_multiple(128, 4096, 64), causal=True,
    ),
    # Long causal prefill: L = ctx = 2048, 128-token shuffled pages.
    "long_prefill": dict(
        seed=3, batch=4, num_q_heads=32, num_kv_heads=8, query_len=2048, head_dim=128,
        page_size=128, context_lens=[2048] * 4, causal=True,
    ),
    # Chunked-prefill continuation: history h ~ U[1000, 3600] plus 65 new
    # queries, ctx = h + 65 (not a tile multiple), causal offset ctx - L.
    "chunked_continuation": dict(
        seed=4, batch=8, num_q_heads=32, num_kv_heads=8, query_len=65, head_dim=128,
        page_size=128, context_lens=_continuation_lens(1000, 3600, 8, 65), causal=True,
    ),
    # Long-context decode with page-crossing tiles: ctx = 32768, 16-token
    # pages, a random permutation over a 32768-page pool.
    "long_decode": dict(
        seed=5, batch=16, num_q_heads=32, num_kv_heads=8, query_len=1, head_dim=128,
        page_size=16, context_lens=[32768] * 16, causal=True,
    ),
}

CONFIG_ORDER = ["tiny_prefill", "decode_batch", "long_prefill", "chunked_continuation", "long_decode"]


def make_config(name: str, poison: bool = False, **overrides) -> PagedProblem:
    """Draw one of the five named workloads (``overrides`` replace arguments)."""
    kw = dict(CONFIGS[name])
    kw.update(overrides)
    seed = kw.pop("seed")
    return make_problem(seed=seed, poison=poison, name=name, **kw)


def permute_pages(p: PagedProblem, seed: int) -> PagedProblem:
    """Same logical K/V under a different physical page assignment.

    Moves every page to a new physical id and rewrites the block table to
    match, so the logical history of each sequence is unchanged.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    n = p.num_pages
    new_id = rng.permutation(n).astype(np.int32)  # old id -> new id
    k = np.empty_like(p.key_pages)
    v = np.empty_like(p.value_pages)
    k[new_id] = p.key_pages
    v[new_id] = p.value_pages
    table = p.block_table.copy()
    used = table >= 0
    table[used] = new_id[table[used]]
    return dataclasses.replace(p, key_pages=k, value_pages=v, block_table=table)


def repack_pages(p: PagedProblem, new_page_size: int, seed: int) -> PagedProblem:
    """Same logical K/V stored with another page size (fresh shuffled pool).

    Reads each sequence's history position by position through the old table
    and writes it into pages of ``new_page_size``. Slots past the end are NaN.
    """
    ctx = p.context_lens.astype(np.int64)
    pages_per_seq = [int(math.ceil(c / new_page_size)) for c in ctx.tolist()]
    needed = sum(pages_per_seq)
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(needed).astype(np.int32)
    H, D = p.num_kv_heads, p.head_dim
    k = np.full((needed, H, new_page_size, D), BF16_NAN, dtype=np.uint16)
    v = np.full((needed, H, new_page_size, D), BF16_NAN, dtype=np.uint16)
    table = np.full((p.batch, max(max(pages_per_seq), 1)), -1, dtype=np.int32)
    pos = 0
    ps = p.page_size
    for b, n in enumerate(pages_per_seq):
        table[b, :n] = perm[pos:pos + n]
        pos += n
        for s in range(int(ctx[b])):
            src = p.block_table[b, s // ps]
            dst = table[b, s // new_page_size]
            k[dst, :, s % new_page_size, :] = p.key_pages[src, :, s % ps, :]
            v[dst, :, s % new_page_size, :] = p.value_pages[src, :, s % ps, :]
    return dataclasses.replace(p, key_pages=k, value_pages=v, block_table=table, page_size=new_page_size)


@dataclasses.dataclass
class VarlenProblem:
    """A mixed batch: every sequence has its own number of query rows.

    ``query`` is packed token-major, uint16 bf16 bits ``[T, H_q, D]``;
    sequence b owns tokens ``[query_start[b], query_start[b + 1])``
    (``query_start`` int32 ``[B + 1]``). The pool, table and context lengths
    are laid out as in :class:`PagedProblem`.
    """

    name: str
    query: np.ndarray
    key_pages: np.ndarray
    value_pages: np.ndarray
    block_table: np.ndarray
    context_lens: np.ndarray
    query_start: np.ndarray
    page_size: int
    scale: float
    causal: bool
    seed: int

    @property
    def batch(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def total_query(self) -> int:
        return int(self.query.shape[0])

    @property
    def num_q_heads(self) -> int:
        return int(self.query.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.query.shape[2])

    @property
    def num_kv_heads(self) -> int:
        return int(self.key_pages.shape[1])

    @property
    def num_pages(self) -> int:
        return int(self.key_pages.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start.astype(np.int64))

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.batch else 0

    def kv_bytes(self) -> int:
        """K+V bytes the method must read: every position of a sequence with queries, once."""
        ctx = self.context_lens.astype(np.int64)[self.query_lens > 0]
        return int(ctx.sum()) * self.num_kv_heads * self.head_dim * 2 * 2

    def visible_pairs(self) -> int:
        total = 0
        for L, c in zip(self.query_lens.tolist(), self.context_lens.tolist()):
            if L == 0:
                continue
            total += L * (c - L) + L * (L + 1) // 2 if self.causal else L * c
        return total

    def flops(self) -> int:
        """Algorithmic FLOPs: 2*D for Q.K and 2*D for P.V per visible pair per q head."""
        return 4 * self.head_dim * self.num_q_heads * self.visible_pairs()


def make_varlen_problem(
    seed: int,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    page_size: int,
    lens: Union[Sequence[Sequence[int]], Callable[[np.random.Generator], Sequence[Sequence[int]]]],
    pool_pages: Optional[int] = None,
    causal: bool = True,
    scale: Optional[float] = None,
    poison: bool = False,
    name: str = "custom_varlen",
    max_pages: Optional[int] = None,
) -> VarlenProblem:
    """Draw one mixed batch.

    ``lens`` is ``(query_lens, context_lens)`` -- two equal-length lists --
    or a function of the generator returning them (drawn first). The rest of
    the draw order is that of :func:`make_problem`: page permutation, q, k,
    v. ``poison`` fills unused pages and slots past each context end with
    bf16 NaN.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    ql, cl = lens(rng) if callable(lens) else lens
    ql = np.asarray(ql, dtype=np.int64)
    ctx = np.asarray(cl, dtype=np.int64)
    if ql.shape != ctx.shape or ql.ndim != 1:
        raise ValueError("query_lens and context_lens must be equal-length lists")
    batch = int(ctx.shape[0])
    pages_per_seq = [int(math.ceil(c / page_size)) for c in ctx.tolist()]
    needed = int(sum(pages_per_seq))
    if pool_pages is None:
        pool_pages = max(needed, 1)
    if pool_pages < needed:
        raise ValueError("pool too small")
    width = max(max(pages_per_seq, default=1), 1) if max_pages is None else int(max_pages)
    perm = rng.permutation(pool_pages).astype(np.int32)
    table = np.full((batch, width), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(pages_per_seq):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    qs = np.zeros(batch + 1, dtype=np.int64)
    qs[1:] = np.cumsum(ql)
    T = int(qs[-1])
    q = _normal_bf16(rng, (T, num_q_heads, head_dim))
    k = _normal_bf16(rng, (pool_pages, num_kv_heads, page_size, head_dim))
    v = _normal_bf16(rng, (pool_pages, num_kv_heads, page_size, head_dim))
    if poison:
        used = np.zeros(pool_pages, dtype=bool)
        for b, n in enumerate(pages_per_seq):
            if n == 0:
                continue
            used[table[b, :n]] = True
            tail = int(ctx[b]) - (n - 1) * page_size
            if tail < page_size:
                last = table[b, n - 1]
                k[last, :, tail:, :] = BF16_NAN
                v[last, :, tail:, :] = BF16_NAN
        k[~used] = BF16_NAN
        v[~used] = BF16_NAN
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(head_dim)))
    return VarlenProblem(
        name=name,
        query=q,
        key_pages=k,
        value_pages=v,
        block_table=table,
        context_lens=ctx.astype(np.int32),
        query_start=qs.astype(np.int32),
        page_size=int(page_size),
        scale=float(np.float32(scale)),
        causal=bool(causal),
        seed=int(seed),
    )


def _serving_step(n: int, n_prefill: int, chunk: int, prompt, output):
    """Lengths of one continuous-batching step: n sequences, n_prefill of them
    prefilling one ``chunk``-token step of a prompt, the rest decoding one token.

    Prompt lengths ~ U[prompt], generated lengths ~ U[output]. A prefilling
    sequence is at a random chunk of its prompt (the last chunk may be
    shorter); a decoding one has its whole prompt plus some generated tokens
    (at least one: the token being decoded). Prefilling sequences sit at
    random places in the batch.
    """

    def draw(rng: np.random.Generator):
        ql = np.ones(n, dtype=np.int64)
        cl = np.empty(n, dtype=np.int64)
        pre = rng.permutation(n)[:n_prefill]
        is_pre = np.zeros(n, dtype=bool)
        is_pre[pre] = True
        for b in range(n):
            p = int(rng.integers(prompt[0], prompt[1] + 1))
            if is_pre[b]:
                k = int(rng.integers(0, (p + chunk - 1) // chunk))
                end = min((k + 1) * chunk, p)
                ql[b] = end - k * chunk
                cl[b] = end
            else:
                cl[b] = p + int(rng.integers(max(output[0], 1), output[1] + 1))
        return ql, cl

    return draw


# name -> (seed, keyword arguments of make_varlen_problem)
VARLEN_CONFIGS: Dict[str, dict] = {
    # One continuous-batching step at the Qwen3-4B attention shape with the
    # serving trace's length mix (prompts U[128, 1024], outputs U[32, 128],
    # 128-token prefill steps), widened to 64 sequences: 8 prefill one chunk,
    # 56 decode one token. 128-token shuffled pages.
    "mixed_batch": dict(
        seed=6, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=128,
        lens=_serving_step(64, 8, 128, (128, 1024), (32, 128)), causal=True,
    ),
}


def make_varlen_config(name: str, poison: bool = False, **overrides) -> VarlenProblem:
    """Draw a named mixed batch (``overrides`` replace arguments)."""
    kw = dict(VARLEN_CONFIGS[name])
    kw.update(overrides)
    seed = kw.pop("seed")
    return make_varlen_problem(seed=seed, poison=poison, name=name, **kw)
