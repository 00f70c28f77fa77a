"""paged_attention_static: the entry point that allocates nothing.

Its output must equal that of paged_attention with a caller workspace (the
same plan, the same kernels) bit for bit, and match the float64 oracle within
the parity bar, on two calls in a row, the second with a smaller input --
the scratch keeps the first call's contents, so stale counters and partials
must not leak into the second.
"""

import ctypes

import numpy as np
import pytest

import oracle
from paged_flashattention_kv_amd import workloads as wl
from tests.helpers import parity, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_flashattention_kv_amd import native

    native.load()


def _call_static(p, d, out):
    import torch
    from paged_flashattention_kv_amd import native

    lib = native.load()
    B, Hq, L, D = p.query.shape
    P, Hkv, ps, _ = p.key_pages.shape
    rc = lib.paged_attention_static(d["query"].data_ptr(), d["key_pages"].data_ptr(), d["value_pages"].data_ptr(),
                                    d["block_table"].data_ptr(), d["context_lens"].data_ptr(), out.data_ptr(), B, Hq,
                                    Hkv, L, D, P, ps, p.block_table.shape[1], ctypes.c_float(p.scale),
                                    1 if p.causal else 0, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, native.last_error()


def _call_with_workspace(p, d):
    import torch
    from paged_flashattention_kv_amd import native

    o = native.paged_attention(d["query"], d["key_pages"], d["value_pages"], d["block_table"], d["context_lens"],
                               p.page_size, p.scale, p.causal)
    torch.cuda.synchronize()
    return o


def _pair(seed, L, ctx_big, ctx_small, ps=16, Hq=32, Hkv=8):
    big = wl.make_problem(seed=seed, batch=len(ctx_big), num_q_heads=Hq, num_kv_heads=Hkv, query_len=L,
                          head_dim=128, page_size=ps, context_lens=list(ctx_big), poison=True)
    small = wl.make_problem(seed=seed + 1, batch=len(ctx_small), num_q_heads=Hq, num_kv_heads=Hkv, query_len=L,
                            head_dim=128, page_size=ps, context_lens=list(ctx_small), poison=True)
    return big, small


@pytest.mark.parametrize("L,ctx_big,ctx_small", [
    (1, (4000, 17, 2500, 999, 3000, 1, 128, 4096), (300, 70, 5)),      # decode schedule, shared segments
    (65, (1100, 3000, 2000, 1500), (200, 90)),                          # prefill, key-range split
])
def test_static_matches_workspace_entry_point_twice(L, ctx_big, ctx_small):
    import torch

    from paged_flashattention_kv_amd import native

    assert native.load().paged_attention_static_scratch_bytes() == 64 << 20
    for p in _pair(500 + L, L, ctx_big, ctx_small):
        say(f"static entry point L={L} B={p.batch} ctx={p.context_lens.tolist()}")
        d = to_device(p)
        want_ws = _call_with_workspace(p, d)
        out = torch.full_like(d["query"], float("nan"))
        _call_static(p, d, out)
        torch.cuda.synchronize()
        got = out.view(torch.int16).cpu().numpy()
        assert np.array_equal(got, want_ws.view(torch.int16).cpu().numpy()), "differs from paged_attention"
        want = oracle.paged_attention_ref(p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens,
                                          p.page_size, p.scale, p.causal)
        parity(out.float().cpu().numpy().astype(np.float64), want, f"static L={L} B={p.batch}")
