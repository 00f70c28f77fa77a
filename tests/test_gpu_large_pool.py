"""GPU parity with page pools larger than 4 GiB.

The sequences' pages sit past the first 4 GiB of pools of several GiB, so
every K/V byte the kernels touch lies more than 2^32 bytes into its pool: the
decode's register loads, the prefill's tile loads (the buffer-form LDS DMA of
whole aligned tiles, whose base is the tile's first row, and the global LDS
DMA of the generic path) and the append's stores must all form page offsets
in 64-bit arithmetic. Every other page of the pools holds NaN, so a read of
a wrong page shows. The oracle runs the same small problem with its original
page ids ("Week 3 Day 5: Paged FlashAttention", Task 1: logical position ->
block_table -> page and slot; the page ids are opaque to the method).
"""

import numpy as np
import pytest

import oracle
from paged_flashattention_kv_amd import workloads as wl

from tests.helpers import parity, say

pytestmark = pytest.mark.gpu

FAR = 4.25 * 2**30  # byte offset of the first page the sequences use


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_flashattention_kv_amd import native

    native.load()


def _bf(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def _far_pools(p):
    """K/V pools with the problem's pages at page ids base .. base + n - 1, all else NaN."""
    import torch

    page_bytes = p.num_kv_heads * p.page_size * p.head_dim * 2
    base = int(FAR // page_bytes) + 1
    n = p.num_pages
    shape = (base + n + 1, p.num_kv_heads, p.page_size, p.head_dim)
    kb = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda:0")
    vb = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda:0")
    kb[base:base + n] = _bf(p.key_pages)
    vb[base:base + n] = _bf(p.value_pages)
    bt = torch.from_numpy(np.ascontiguousarray(p.block_table + base, dtype=np.int32)).cuda()
    ctx = torch.from_numpy(np.ascontiguousarray(p.context_lens, dtype=np.int32)).cuda()
    assert base * page_bytes > 2**32
    return kb, vb, bt, ctx, base


# (seed, B, H_q, H_kv, L, page size, contexts): decode (aligned register
# loads), prefill with page size 128 (whole aligned tiles: buffer form) and
# with page size 16 (generic path, tiles crossing pages)
CASES = [
    (1101, 3, 8, 2, 1, 128, (1, 700, 4097)),
    (1102, 2, 8, 2, 130, 128, (130, 1500)),
    (1103, 2, 8, 2, 65, 16, (65, 900)),
]


@pytest.mark.parametrize("seed,B,Hq,Hkv,L,ps,ctx", CASES)
def test_attention_pages_past_4gib(seed, B, Hq, Hkv, L, ps, ctx):
    import torch
    from paged_flashattention_kv_amd import native

    say(f"large pool seed={seed} B={B} Hq={Hq} Hkv={Hkv} L={L} ps={ps} ctx={ctx}")
    p = wl.make_problem(seed=seed, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, query_len=L, head_dim=128,
                        page_size=ps, context_lens=list(ctx), poison=True)
    want = oracle.paged_attention_ref(p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens,
                                      p.page_size, p.scale, p.causal)
    kb, vb, bt, cl, base = _far_pools(p)
    say(f"  pool {tuple(kb.shape)}: first used page {base} at byte {base * kb[0].numel() * 2:,}")
    o = native.paged_attention(_bf(p.query), kb, vb, bt, cl, ps, p.scale, p.causal)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy().astype(np.float64)
    del kb, vb
    torch.cuda.empty_cache()
    parity(got, want, f"large pool seed={seed}")


def test_append_pages_past_4gib():
    import torch
    from paged_flashattention_kv_amd import native

    B, H, L, ps, ctx = 3, 2, 65, 16, (65, 66, 700)
    say(f"large pool append B={B} Hkv={H} L={L} ps={ps} ctx={ctx}")
    p = wl.make_problem(seed=1104, batch=B, num_q_heads=H, num_kv_heads=H, query_len=1, head_dim=128,
                        page_size=ps, context_lens=list(ctx), poison=True)
    rng = np.random.Generator(np.random.PCG64(2104))
    kn = wl.f32_to_bf16_bits(rng.standard_normal((B, H, L, 128), dtype=np.float32))
    vn = wl.f32_to_bf16_bits(rng.standard_normal((B, H, L, 128), dtype=np.float32))
    want_k, want_v = oracle.kv_append_ref(kn, vn, p.key_pages, p.value_pages, p.block_table, p.context_lens, ps)
    kb, vb, bt, cl, base = _far_pools(p)
    native.kv_append(_bf(kn), _bf(vn), kb, vb, bt, cl, ps)
    torch.cuda.synchronize()
    n = p.num_pages
    got_k = kb[base:base + n].view(torch.int16).cpu().numpy().view(np.uint16)
    got_v = vb[base:base + n].view(torch.int16).cpu().numpy().view(np.uint16)
    # the pages on either side of the used range are untouched
    untouched = bool(torch.isnan(kb[base - 1]).all() and torch.isnan(kb[base + n]).all()
                     and torch.isnan(vb[base - 1]).all() and torch.isnan(vb[base + n]).all())
    del kb, vb
    torch.cuda.empty_cache()
    assert np.array_equal(got_k, want_k), "key pool differs from the oracle"
    assert np.array_equal(got_v, want_v), "value pool differs from the oracle"
    assert untouched, "a page outside the sequences' pages was written"
