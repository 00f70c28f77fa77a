"""GPU parity at head dims other than 128 (head dim 128 is covered by the other GPU tests).

64 and 256 have kernel instances of their own: the decode kernel holds D/16
lanes per key row, the prefill kernel takes D/16 contraction steps and D/32
output blocks per tile (one work item per CU at 256). Any other multiple of 8
up to 256 runs the next larger instance with the dims past it masked (zero
query, key/value chunks past the row re-read its first chunk, no stores past
it) -- the generic control beside the d128 kernel of "Week 3 Day 5: Paged
FlashAttention", Task 1. Each case runs through the C ABI and is compared with
the float64 oracle at the operator's bar (max abs <= 2e-2, mean abs <= 2e-3),
or bit for bit for the K/V append. Page sizes cover the aligned loaders (a
wave step or a 64-key tile inside one page) and the generic per-row ones.
"""

import numpy as np
import pytest

import oracle
from paged_flashattention_kv_amd import workloads as wl

from tests.helpers import parity, run_gpu, say, to_device

pytestmark = pytest.mark.gpu

DIMS = [64, 256, 8, 80, 96, 112, 160, 192, 248]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_flashattention_kv_amd import native

    native.load()


def _ref(p):
    return oracle.paged_attention_ref(p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens,
                                      p.page_size, p.scale, p.causal)


# (seed, B, H_q, H_kv, L, page size, contexts, causal)
CASES = [
    (701, 4, 8, 2, 1, 16, (1, 300, 4097, 64), True),       # decode, aligned at every D
    (702, 3, 8, 2, 1, 5, (7, 999, 130), True),             # decode, generic loader
    (703, 2, 16, 2, 1, 128, (2000, 33), True),             # decode, 8 rows per kv head
    (704, 3, 8, 2, 2, 8, (2, 70, 515), True),              # 2-token decode: 8 rows per kv head
    (705, 2, 8, 2, 65, 64, (65, 1000), True),              # prefill, aligned tiles
    (706, 2, 4, 2, 130, 16, (130, 700), True),             # prefill, tiles across pages, 2 query tiles
    (707, 2, 8, 8, 33, 3, (40, 500), True),                # prefill, MHA, 3-token pages
    (708, 3, 8, 2, 1, 32, (100, 1, 2049), False),          # non-causal decode
    (709, 2, 8, 4, 70, 64, (90, 333), False),              # non-causal prefill
]


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("seed,B,Hq,Hkv,L,ps,ctx,causal", CASES)
def test_parity_auto_schedule(D, seed, B, Hq, Hkv, L, ps, ctx, causal):
    say(f"head_dim={D} seed={seed} B={B} Hq={Hq} Hkv={Hkv} L={L} ps={ps} ctx={ctx} causal={causal}")
    p = wl.make_problem(seed=seed + D, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, query_len=L, head_dim=D,
                        page_size=ps, context_lens=list(ctx), causal=causal, poison=True)
    parity(run_gpu(p), _ref(p), f"D={D} seed={seed}")


@pytest.mark.parametrize("D", DIMS)
def test_both_schedules_on_one_short_query(D):
    # a 2-token query with GQA 2 fits the decode schedule (4 rows) and runs on both
    from paged_flashattention_kv_amd import native

    p = wl.make_problem(seed=720 + D, batch=3, num_q_heads=4, num_kv_heads=2, query_len=2, head_dim=D,
                        page_size=16, context_lens=[5, 400, 1500], poison=True)
    want = _ref(p)
    d = to_device(p)
    parity(run_gpu(p, schedule=native.SCHEDULE_DECODE, dev=d), want, f"D={D} decode")
    parity(run_gpu(p, schedule=native.SCHEDULE_PREFILL, dev=d), want, f"D={D} prefill")
    parity(run_gpu(p, schedule=native.SCHEDULE_DECODE, decode_work_items=5, dev=d), want, f"D={D} decode w=5")


@pytest.mark.parametrize("D", DIMS)
def test_chunked_continuation_matches_full_prefill_rows(D):
    # the pages' chunked-prefill continuation at another head dim: L = 65 new queries after a history
    p = wl.make_problem(seed=730 + D, batch=2, num_q_heads=8, num_kv_heads=2, query_len=65, head_dim=D,
                        page_size=128, context_lens=[65 + 1000, 65 + 2500], poison=True)
    parity(run_gpu(p), _ref(p), f"D={D} continuation")


@pytest.mark.parametrize("D", DIMS)
def test_varlen_mix(D):
    import torch
    from paged_flashattention_kv_amd import native

    p = wl.make_varlen_problem(seed=740 + D, num_q_heads=8, num_kv_heads=2, head_dim=D, page_size=16,
                               lens=([1, 70, 0, 1, 129, 2], [300, 70, 0, 2000, 400, 90]), poison=True)
    want = oracle.paged_attention_varlen_ref(p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens,
                                             p.query_start, p.page_size, p.scale, p.causal)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")

    q, kp, vp = bf(p.query), bf(p.key_pages), bf(p.value_pages)
    bt, cl, qs = i32(p.block_table), i32(p.context_lens), i32(p.query_start)
    for dml in (-1, 0, 2):
        out = native.paged_attention_varlen(q, kp, vp, bt, cl, qs, p.max_query_len, p.page_size, p.scale, True,
                                            decode_max_len=dml)
        torch.cuda.synchronize()
        parity(out.float().cpu().numpy().astype(np.float64), want, f"D={D} varlen dml={dml}")


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("L,ps", [(1, 16), (37, 5), (300, 128)])
def test_append_bit_exact(D, L, ps):
    import torch
    from paged_flashattention_kv_amd import native

    p = wl.make_problem(seed=750 + D + L, batch=3, num_q_heads=2, num_kv_heads=2, query_len=1, head_dim=D,
                        page_size=ps, context_lens=[L, L + 9, L + 400], poison=True)
    rng = np.random.Generator(np.random.PCG64(760 + D + L))
    kn = wl.f32_to_bf16_bits(rng.standard_normal((3, 2, L, D), dtype=np.float32))
    vn = wl.f32_to_bf16_bits(rng.standard_normal((3, 2, L, D), dtype=np.float32))
    want_k, want_v = oracle.kv_append_ref(kn, vn, p.key_pages, p.value_pages, p.block_table, p.context_lens, ps)
    d = to_device(p)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")

    native.kv_append(bf(kn), bf(vn), d["key_pages"], d["value_pages"], d["block_table"], d["context_lens"], ps)
    torch.cuda.synchronize()
    for name, got_t, want in (("key", d["key_pages"], want_k), ("value", d["value_pages"], want_v)):
        got = got_t.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want), f"D={D} L={L} ps={ps}: {name} pool differs"


@pytest.mark.parametrize("D", [96, 200])
@pytest.mark.parametrize("L", [1, 40])
def test_masked_generic_head_dim(D, L):
    import torch
    from paged_flashattention_kv_amd import native

    p = wl.make_problem(seed=770 + D + L, batch=2, num_q_heads=8, num_kv_heads=2, query_len=L, head_dim=D,
                        page_size=16, context_lens=[L + 30, L + 600], poison=True)
    rng = np.random.default_rng(771 + D)
    S = int(p.context_lens.max())
    m = rng.normal(0.0, 1.0, size=(2, 1, L, S)).astype(np.float32)
    m[..., 0] = 0.0
    m[rng.random(m.shape) < 0.1] = -np.inf
    m[..., 0] = 0.0
    want = oracle.paged_attention_masked_ref(p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens, m,
                                             p.page_size, p.scale, True)
    d = to_device(p)
    out = native.paged_attention_masked(d["query"], d["key_pages"], d["value_pages"], d["block_table"],
                                        d["context_lens"], torch.from_numpy(m).to("cuda:0"), p.page_size, p.scale,
                                        True)
    torch.cuda.synchronize()
    parity(out.float().cpu().numpy().astype(np.float64), want, f"masked D={D} L={L}")
