"""GPU parity of the prefill schedule at 64 packed query rows x 32 keys per tile.

PA_SCHEDULE_PREFILL_64X32 runs the tiling of the matrix kernel in "Week 3 Day
5: Paged FlashAttention", Task 1 (a 64-row query block, 32 K/V positions per
iteration), kept beside the automatic 128 x 64 tiling so that the long causal
prefill can be measured at both. Same bar as every parity test: the float64
oracle, max-abs <= 2e-2 and mean-abs <= 2e-3 on the bf16 output.
"""

import numpy as np
import pytest

import oracle
from paged_flashattention_kv_amd import workloads as wl
from tests.helpers import parity, run_gpu, say, to_device

pytestmark = pytest.mark.gpu

T64 = 3  # PA_SCHEDULE_PREFILL_64X32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_flashattention_kv_amd import native

    native.load()
    assert native.SCHEDULE_PREFILL_64X32 == T64


def ref(p, **kw):
    return oracle.paged_attention_ref(
        p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens, p.page_size, p.scale, p.causal, **kw
    )


def test_config_long_prefill_64x32():
    p = wl.make_config("long_prefill")
    pairs = [(b, h) for b in range(4) for h in (0, 5, 14, 23, 31)]
    say(f"long_prefill at 64 x 32 tiles, {len(pairs)} (b, h) against the oracle")
    want = ref(p, pairs=pairs)
    got = run_gpu(p, schedule=T64)
    parity(np.stack([got[b, h] for b, h in pairs]), want, "long_prefill 64x32")
    for b in range(4):  # causal row 0 of every head sees only key 0, exactly
        for h in range(32):
            v0 = wl.bf16_bits_to_f32(p.value_pages[p.block_table[b, 0], h // 4, 0]).astype(np.float64)
            assert np.array_equal(got[b, h, 0], v0)


def test_config_tiny_and_chunked_64x32():
    for name in ("tiny_prefill", "chunked_continuation"):
        p = wl.make_config(name)
        say(f"{name} at 64 x 32 tiles")
        parity(run_gpu(p, schedule=T64), ref(p), f"{name} 64x32")


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("ps", [32, 128, 16, 5])
def test_ragged_64x32(D, ps):
    # query lengths and contexts that leave ragged row tiles (G*L not a multiple
    # of 64) and ragged key tiles (ctx not a multiple of 32), pages that hold a
    # whole 32-key tile (32, 128) or not (16, 5), a poisoned pool
    ctx = (37, 96, 161, 64 + 33)
    L = 33
    p = wl.make_problem(seed=700 + D + ps, batch=4, num_q_heads=8, num_kv_heads=2, query_len=L, head_dim=D,
                        page_size=ps, context_lens=list(ctx), causal=True, poison=True)
    say(f"ragged 64x32 D={D} ps={ps} L={L} ctx={list(ctx)}")
    parity(run_gpu(p, schedule=T64), ref(p), f"ragged D={D} ps={ps}")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("G,L", [(1, 1), (1, 64), (4, 17), (8, 40), (16, 4)])
def test_gqa_and_lengths_64x32(causal, G, L):
    ctx = (L + 90, L, L + 31)
    p = wl.make_problem(seed=800 + 10 * G + L, batch=3, num_q_heads=2 * G, num_kv_heads=2, query_len=L,
                        head_dim=128, page_size=32, context_lens=list(ctx), causal=causal)
    say(f"64x32 G={G} L={L} causal={causal}")
    parity(run_gpu(p, schedule=T64), ref(p), f"G={G} L={L} causal={causal}")


def test_page_permutation_bit_identical_64x32():
    p = wl.make_problem(seed=901, batch=2, num_q_heads=8, num_kv_heads=2, query_len=70, head_dim=128,
                        page_size=32, context_lens=[200, 133], causal=True, pool_pages=24)
    a = run_gpu(p, schedule=T64)
    q = wl.permute_pages(p, seed=5)
    b = run_gpu(q, schedule=T64)
    assert np.array_equal(a, b)


def test_refusals_64x32():
    """Through the C ABI: a head dim without an instance of its own, or an
    explicit mask, at this tiling returns PA_ERR_UNSUPPORTED and writes nothing."""
    import torch
    from paged_flashattention_kv_amd import native

    lib = native.load()
    stream = torch.cuda.current_stream().cuda_stream
    for D in (80, 128):
        p = wl.make_problem(seed=902 + D, batch=1, num_q_heads=4, num_kv_heads=2, query_len=8, head_dim=D,
                            page_size=32, context_lens=[40], causal=True)
        d = to_device(p)
        out = torch.full_like(d["query"], float("nan"))
        args = [d["query"].data_ptr(), d["key_pages"].data_ptr(), d["value_pages"].data_ptr(),
                d["block_table"].data_ptr(), d["context_lens"].data_ptr()]
        dims = [p.batch, p.num_q_heads, p.num_kv_heads, p.query_len, p.head_dim, p.num_pages, p.page_size,
                p.max_pages]
        if D == 80:
            rc = lib.paged_attention_ex(*args, out.data_ptr(), *dims, p.scale, 1, None, 0, T64, 0, stream)
        else:
            mask = torch.zeros(1, 1, 8, 40, dtype=torch.float32, device="cuda:0")
            rc = lib.paged_attention_masked(*args, mask.data_ptr(), 0, 0, 40, 40, out.data_ptr(), *dims, p.scale, 1,
                                            None, 0, T64, 0, stream)
        torch.cuda.synchronize()
        say(f"64x32 refusal D={D}: rc={rc} ({native.last_error()})")
        assert rc == native.PA_ERR_UNSUPPORTED
        assert torch.isnan(out.float()).all()
