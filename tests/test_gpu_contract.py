"""GPU tests of the call contract itself, through the C ABI.

- the exact one-call entry point ``paged_attention`` and the 7-argument
  ``paged_attention_workspace_bytes`` (every other test goes through the
  ``_ex`` variants that add a schedule override);
- the binding on a side stream with no caller workspace: temporaries are made
  on the launch stream, results match the oracle;
- negative and zero ``scale`` (folded into the query's sign / a least-normal
  factor) on both schedules and with an explicit mask.
"""

import ctypes

import numpy as np
import pytest

import oracle
from paged_flashattention_kv_amd import workloads as wl
from tests.helpers import parity, say, to_device

pytestmark = pytest.mark.gpu

DECODE, PREFILL = 1, 2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_flashattention_kv_amd import native

    native.load()


def _ref(p, scale=None):
    return oracle.paged_attention_ref(p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens,
                                      p.page_size, p.scale if scale is None else scale, p.causal)


def _problem(seed, L, ctx, ps=16, Hq=8, Hkv=2, causal=True):
    return wl.make_problem(seed=seed, batch=len(ctx), num_q_heads=Hq, num_kv_heads=Hkv, query_len=L, head_dim=128,
                           page_size=ps, context_lens=list(ctx), causal=causal, poison=True)


@pytest.mark.parametrize("L,ctx", [(1, (5, 300, 1500, 4097)), (40, (40, 333, 1000))])
def test_exact_paged_attention_symbol(L, ctx):
    import torch
    from paged_flashattention_kv_amd import native

    p = _problem(71 + L, L, ctx)
    d = to_device(p)
    lib = native.load()
    B, Hq, _, D = p.query.shape
    P, Hkv, ps, _ = p.key_pages.shape
    mp = p.block_table.shape[1]
    need = lib.paged_attention_workspace_bytes(B, Hq, Hkv, L, D, ps, mp)
    assert need == native.workspace_bytes(B, Hq, Hkv, L, D, ps, mp)
    if L == 1:
        assert need > 0  # the decode schedule always needs its workspace
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(d["query"])
    stream = torch.cuda.current_stream().cuda_stream
    say(f"paged_attention symbol L={L} ctx={list(ctx)} workspace={need}")
    for _ in range(2):  # the second call reuses the workspace the first left zeroed
        rc = lib.paged_attention(d["query"].data_ptr(), d["key_pages"].data_ptr(), d["value_pages"].data_ptr(),
                                 d["block_table"].data_ptr(), d["context_lens"].data_ptr(), out.data_ptr(), B, Hq,
                                 Hkv, L, D, P, ps, mp, ctypes.c_float(p.scale), 1, ws.data_ptr(), need, stream)
        assert rc == 0, native.last_error()
        torch.cuda.synchronize()
        parity(out.float().cpu().numpy().astype(np.float64), _ref(p), f"paged_attention symbol L={L}")
    # a workspace one byte short is refused before any launch (decode needs it)
    if need > 0:
        rc = lib.paged_attention(d["query"].data_ptr(), d["key_pages"].data_ptr(), d["value_pages"].data_ptr(),
                                 d["block_table"].data_ptr(), d["context_lens"].data_ptr(), out.data_ptr(), B, Hq,
                                 Hkv, L, D, P, ps, mp, ctypes.c_float(p.scale), 1, ws.data_ptr(), need - 1, stream)
        assert rc == (native.PA_ERR_WORKSPACE if L == 1 else 0)


@pytest.mark.parametrize("schedule", [DECODE, PREFILL])
def test_side_stream_without_workspace(schedule):
    import torch
    from paged_flashattention_kv_amd import native

    p = _problem(83, 1, (700, 64, 2049, 1), ps=16)
    d = to_device(p)
    want = _ref(p)
    side = torch.cuda.Stream()
    # keep the current stream busy so that work wrongly ordered on it would lag
    x = torch.randn(4096, 4096, device="cuda:0")
    for _ in range(4):
        x = x @ x
        x = x / x.norm()
    outs = []
    for _ in range(3):
        outs.append(native.paged_attention(d["query"], d["key_pages"], d["value_pages"], d["block_table"],
                                           d["context_lens"], p.page_size, p.scale, True, schedule=schedule,
                                           stream=side))
    side.synchronize()
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        parity(o.float().cpu().numpy().astype(np.float64), want, f"side stream schedule={schedule} call {i}")


@pytest.mark.parametrize("scale_kind", ["negative", "zero"])
@pytest.mark.parametrize("L", [1, 2, 37])
def test_negative_and_zero_scale(scale_kind, L):
    from paged_flashattention_kv_amd import native

    p = _problem(97 + L, L, (37, 513, 2100), ps=16, Hq=8, Hkv=4)
    scale = -p.scale if scale_kind == "negative" else 0.0
    want = _ref(p, scale)
    assert np.isfinite(want).all()
    d = to_device(p)
    rows = L * 2
    for sched in ([DECODE, PREFILL] if rows <= 8 else [PREFILL]):
        import torch

        o = native.paged_attention(d["query"], d["key_pages"], d["value_pages"], d["block_table"],
                                   d["context_lens"], p.page_size, scale, True, schedule=sched)
        torch.cuda.synchronize()
        parity(o.float().cpu().numpy().astype(np.float64), want, f"scale={scale_kind} L={L} schedule={sched}")


@pytest.mark.parametrize("L", [1, 50])
def test_negative_scale_with_mask(L):
    import torch
    from paged_flashattention_kv_amd import native

    p = _problem(111 + L, L, (60, 777), ps=16, Hq=8, Hkv=2)
    rng = np.random.default_rng(5)
    S = int(p.context_lens.max())
    m = rng.normal(0.0, 1.0, size=(2, 8, L, S)).astype(np.float32)
    m[..., 0] = 0.0
    want = oracle.paged_attention_masked_ref(p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens, m,
                                             p.page_size, -p.scale, True)
    d = to_device(p)
    o = native.paged_attention_masked(d["query"], d["key_pages"], d["value_pages"], d["block_table"],
                                      d["context_lens"], torch.from_numpy(m).to("cuda:0"), p.page_size, -p.scale,
                                      True)
    torch.cuda.synchronize()
    parity(o.float().cpu().numpy().astype(np.float64), want, f"masked negative scale L={L}")
