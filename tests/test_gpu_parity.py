"""GPU parity: the HIP operator (through the C ABI) against the float64 oracle.

Bar: max-abs error <= 2e-2 and mean-abs error <= 2e-3 of the bf16 output
against the float64 oracle; indexing and visibility exactly (needle probes,
page permutation and NaN poisoning are bit-identical or exact).
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from paged_flashattention_kv_amd import workloads as wl
from tests.helpers import parity, run_gpu, say, to_device

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DECODE, PREFILL = 1, 2


def ref(p, **kw):
    return oracle.paged_attention_ref(
        p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens, p.page_size, p.scale, p.causal, **kw
    )


def small(seed, B, Hq, Hkv, L, ctx, ps, causal=True, pool=None, poison=False, D=128):
    return wl.make_problem(
        seed=seed, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, query_len=L, head_dim=D, page_size=ps,
        context_lens=list(ctx), causal=causal, pool_pages=pool, poison=poison,
    )


def schedules_for(p):
    """Both schedules when the decode one accepts the shape (debugging ladder)."""
    rows = p.query_len * p.num_q_heads // p.num_kv_heads
    return [DECODE, PREFILL] if rows <= 8 else [PREFILL]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_flashattention_kv_amd import native

    native.load()


# ------------------------------------------------------------------ configs


def test_config_tiny_prefill():
    p = wl.make_config("tiny_prefill")
    say(f"tiny_prefill B=1 Hq=4 Hkv=2 L=13 ps=4 table={p.block_table.tolist()}")
    want = ref(p)
    got = run_gpu(p)
    parity(got, want, "tiny_prefill")
    # row 0 sees only key 0: the output is that key's value row, exactly
    for h in range(4):
        v0 = wl.bf16_bits_to_f32(p.value_pages[p.block_table[0, 0], h // 2, 0]).astype(np.float64)
        assert np.array_equal(got[0, h, 0], v0)


@pytest.fixture(scope="module")
def decode_batch():
    return wl.make_config("decode_batch")


def test_config_decode_batch(decode_batch):
    p = decode_batch
    say(f"decode_batch B=64 ctx in [{p.context_lens.min()},{p.context_lens.max()}] ps=128")
    want = ref(p)
    parity(run_gpu(p), want, "decode_batch auto")


@pytest.mark.parametrize("items", [1, 7, 100, 513, 4096])
def test_decode_batch_work_items(decode_batch, items):
    p = decode_batch
    pairs = [(b, h) for b in range(0, 64, 5) for h in (0, 13, 31)]
    want = ref(p, pairs=pairs)
    got = run_gpu(p, schedule=DECODE, decode_work_items=items)
    parity(np.stack([got[b, h] for b, h in pairs]), want, f"decode_batch items={items}")


@pytest.mark.parametrize("items", [1, 3, 64, 5000])
def test_decode_tiny_contexts_more_items_than_work(items):
    # contexts of 1..70 keys: a few granules in total, so most work items are empty
    p = small(44, B=9, Hq=8, Hkv=2, L=1, ctx=(1, 2, 63, 64, 65, 7, 70, 33, 1), ps=16, poison=True)
    parity(run_gpu(p, schedule=DECODE, decode_work_items=items), ref(p), f"tiny contexts items={items}")


def test_config_long_prefill():
    p = wl.make_config("long_prefill")
    say("long_prefill B=4 L=ctx=2048 ps=128, every (b, h) against the oracle")
    want = ref(p)
    got = run_gpu(p)
    parity(got, want, "long_prefill (all 128 (b, h))")
    for b in range(4):  # no (sequence, head) may hide behind the batch-wide mean
        for h in range(32):
            err = np.abs(got[b, h] - want[b, h])
            assert err.max() <= 2e-2 and err.mean() <= 2e-3, (b, h, err.max(), err.mean())
    # causal row 0 of every head sees only key 0
    for b in range(4):
        for h in range(32):
            v0 = wl.bf16_bits_to_f32(p.value_pages[p.block_table[b, 0], h // 4, 0]).astype(np.float64)
            assert np.array_equal(got[b, h, 0], v0)


def test_config_chunked_continuation():
    p = wl.make_config("chunked_continuation")
    say(f"chunked_continuation B=8 L=65 ctx={p.context_lens.tolist()}")
    parity(run_gpu(p), ref(p), "chunked_continuation")


@pytest.fixture(scope="module")
def long_decode():
    return wl.make_config("long_decode")


def test_config_long_decode(long_decode):
    p = long_decode
    say("long_decode B=16 ctx=32768 ps=16, every (b, h) against the oracle")
    want = ref(p)
    got = run_gpu(p)
    parity(got, want, "long_decode (all 512 (b, h))")
    for b in range(16):
        err = np.abs(got[b] - want[b])
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, (b, err.max(), err.mean())
    got3 = run_gpu(p, schedule=DECODE, decode_work_items=3)
    parity(got3, want, "long_decode items=3 (all 512 (b, h))")


# ------------------------------------------------------- needle probes


def _plant_needle(p, b, h, l, t):
    G = p.num_q_heads // p.num_kv_heads
    phys = p.block_table[b, t // p.page_size]
    k = wl.bf16_bits_to_f32(p.key_pages[phys, h // G, t % p.page_size])
    p.query[b, h, l] = wl.f32_to_bf16_bits(8.0 * k)
    return wl.bf16_bits_to_f32(p.value_pages[phys, h // G, t % p.page_size]).astype(np.float64)


def _plant_hidden(p, b, h, l, slot_pos):
    """q aimed at a slot that must stay invisible (past the context or causal bound)."""
    G = p.num_q_heads // p.num_kv_heads
    phys = p.block_table[b, slot_pos // p.page_size]
    k = wl.bf16_bits_to_f32(p.key_pages[phys, h // G, slot_pos % p.page_size])
    p.query[b, h, l] = wl.f32_to_bf16_bits(8.0 * k)
    return wl.bf16_bits_to_f32(p.value_pages[phys, h // G, slot_pos % p.page_size]).astype(np.float64)


def test_needles_decode_batch():
    p = wl.make_config("decode_batch")
    rng = np.random.default_rng(7)
    needles, hidden = {}, {}
    for b in range(64):
        ctx = int(p.context_lens[b])
        h = (5 * b) % 32
        t = int(rng.integers(0, ctx))
        needles[(b, h)] = _plant_needle(p, b, h, 0, t)
        if ctx % p.page_size:  # an unused slot in the last page
            h2 = (h + 16) % 32
            hidden[(b, h2)] = _plant_hidden(p, b, h2, 0, ctx)
    got = run_gpu(p)
    for (b, h), v in needles.items():
        assert np.max(np.abs(got[b, h, 0] - v)) <= 1e-2, (b, h)
    for (b, h), v in hidden.items():
        assert np.max(np.abs(got[b, h, 0] - v)) > 0.25, (b, h)
    pairs = list(hidden.keys())[:16]
    parity(np.stack([got[b, h] for b, h in pairs]), ref(p, pairs=pairs), "decode hidden needles")


def test_needles_long_decode_page_crossing(long_decode):
    p = wl.PagedProblem(**{**long_decode.__dict__, "query": long_decode.query.copy()})
    needles = {}
    targets = [0, 15, 16, 31, 32, 4095, 4096, 20000, 32767, 32752]
    for i, t in enumerate(targets):
        b, h = i % 16, (3 * i) % 32
        needles[(b, h)] = _plant_needle(p, b, h, 0, t)
    got = run_gpu(p)
    for (b, h), v in needles.items():
        assert np.max(np.abs(got[b, h, 0] - v)) <= 1e-2, (b, h)


def test_needles_prefill_diagonal():
    p = small(31, B=2, Hq=8, Hkv=2, L=300, ctx=(300, 421), ps=16)
    needles, hidden = {}, {}
    for b in range(2):
        ctx = int(p.context_lens[b])
        off = ctx - 300
        for i, l in enumerate([0, 5, 63, 64, 127, 128, 200, 299]):
            h = (i + 3 * b) % 8
            last = l + off
            t = last if i % 2 == 0 else (7 * l) % (last + 1)
            needles[(b, h, l)] = _plant_needle(p, b, h, l, t)
            if l < 299:
                h2 = (h + 4) % 8
                hidden[(b, h2, l)] = _plant_hidden(p, b, h2, l, last + 1)
    got = run_gpu(p)
    for (b, h, l), v in needles.items():
        assert np.max(np.abs(got[b, h, l] - v)) <= 1e-2, (b, h, l)
    for (b, h, l), v in hidden.items():
        assert np.max(np.abs(got[b, h, l] - v)) > 0.25, (b, h, l)
    parity(got, ref(p), "prefill needles")


# ------------------------------------------------- fixtures and the grid


def _fixture_cases():
    with open(os.path.join(GOLDEN, "test_grid.json")) as f:
        return json.load(f)["required_fixtures"]["cases"]


@pytest.mark.parametrize("case", _fixture_cases(), ids=lambda c: c["name"])
def test_required_fixtures(case):
    ps, ctx, L = case["page_size"], case["context"], case["query_len"]
    Hq, Hkv = (8, 2) if case["name"] == "gqa_group_of_4" else (4, 2)
    p = small(41, B=2, Hq=Hq, Hkv=Hkv, L=L, ctx=(ctx, ctx + 37), ps=ps, poison=True)
    want = ref(p)
    for sch in schedules_for(p):
        got = run_gpu(p, schedule=sch)
        parity(got, want, f"{case['name']} schedule={sch}")


def _grid():
    with open(os.path.join(GOLDEN, "test_grid.json")) as f:
        g = json.load(f)["week2_decode_grid"]
    cases = []
    for L in g["query_lens"] + [2]:
        for ratio in g["gqa_ratios"]:
            for ctx in g["contexts"]:
                if ctx >= L:
                    cases.append((L, ratio, ctx))
    return cases


@pytest.mark.parametrize("ps", [16, 128, 5])
@pytest.mark.parametrize("L,ratio,ctx", _grid())
def test_week2_grid(L, ratio, ctx, ps):
    p = small(1000 + ctx + 13 * L + ratio + ps, B=2, Hq=2 * ratio, Hkv=2, L=L, ctx=(ctx, max(L, ctx - 7)),
              ps=ps, poison=True)
    want = ref(p)
    for sch in schedules_for(p):
        parity(run_gpu(p, schedule=sch), want, f"L={L} G={ratio} ctx={ctx} ps={ps} sch={sch}")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("ps", [1, 3, 64, 256])
def test_ragged_batch_odd_page_sizes(causal, ps):
    p = small(77 + ps, B=5, Hq=6, Hkv=3, L=2, ctx=(2, 70, 129, 300, 555), ps=ps, causal=causal, poison=True)
    want = ref(p)
    for sch in schedules_for(p):
        parity(run_gpu(p, schedule=sch), want, f"ragged ps={ps} causal={causal} sch={sch}")


@pytest.mark.parametrize("L", [1, 33, 64, 65, 129, 200])
def test_prefill_query_tiles_and_offsets(L):
    p = small(90 + L, B=3, Hq=8, Hkv=2, L=L, ctx=(L, L + 100, L + 1000), ps=32, poison=True)
    parity(run_gpu(p, schedule=PREFILL), ref(p), f"prefill L={L}")


# Long queries: many 128-row query tiles with a ragged last one, both
# loaders, chunked continuations and non-causal attention.
@pytest.mark.parametrize("L,ctx,ps,causal,D", [
    (512, (512, 600), 128, True, 128),
    (700, (700, 1337), 64, True, 128),
    (777, (800, 2000), 16, True, 128),
    (530, (530, 531), 5, True, 128),
    (600, (650, 1200), 32, False, 128),
    (1000, (1000, 1100), 64, True, 64),
])
def test_prefill_long_queries(L, ctx, ps, causal, D):
    p = small(120 + L + ps, B=2, Hq=4, Hkv=2, L=L, ctx=ctx, ps=ps, causal=causal, poison=True, D=D)
    say(f"long query L={L} ctx={ctx} ps={ps} causal={causal} D={D}")
    parity(run_gpu(p), ref(p), f"long query L={L} ps={ps}")


def test_noncausal_prefill():
    p = small(95, B=2, Hq=4, Hkv=4, L=70, ctx=(30, 200), ps=16, causal=False, poison=True)
    parity(run_gpu(p), ref(p), "noncausal prefill")


# ------------------------------------------------------------ invariants


def test_page_permutation_bit_identical_on_gpu():
    for p in (small(51, B=3, Hq=8, Hkv=2, L=1, ctx=(100, 1000, 3000), ps=16),
              small(52, B=2, Hq=8, Hkv=2, L=100, ctx=(100, 700), ps=64)):
        q = wl.permute_pages(p, seed=3)
        for sch in schedules_for(p):
            a = run_gpu(p, schedule=sch)
            b = run_gpu(q, schedule=sch)
            assert np.array_equal(a, b), f"schedule {sch}"


def test_poisoned_memory_bit_identical_on_gpu():
    for kw in (dict(L=1, ctx=(77, 1000, 2001)), dict(L=40, ctx=(40, 333, 1000))):
        clean = small(61, B=3, Hq=8, Hkv=2, ps=32, pool=100, **kw)
        dirty = small(61, B=3, Hq=8, Hkv=2, ps=32, pool=100, poison=True, **kw)
        for sch in schedules_for(clean):
            a = run_gpu(clean, schedule=sch)
            b = run_gpu(dirty, schedule=sch)
            assert np.isfinite(b).all()
            assert np.array_equal(a, b), f"schedule {sch}"


def test_chunk_matches_tail_of_full_prefill():
    ctx = 777
    full = small(71, B=1, Hq=8, Hkv=2, L=ctx, ctx=(ctx,), ps=32)
    got_full = run_gpu(full)
    for L in (65, 2, 1):
        chunk = wl.PagedProblem(**{**full.__dict__, "query": np.ascontiguousarray(full.query[:, :, ctx - L:, :])})
        got = run_gpu(chunk)
        parity(got, ref(chunk), f"chunk L={L}")
        assert np.max(np.abs(got - got_full[:, :, ctx - L:, :])) <= 2e-2


def test_output_guard_regions_untouched():
    import torch
    from paged_flashattention_kv_amd import native

    p = small(81, B=3, Hq=8, Hkv=2, L=1, ctx=(50, 600, 3000), ps=16)
    d = to_device(p)
    n = p.query.size
    for sch in (DECODE, PREFILL):
        buf = torch.full((n + 2048,), 7.0, dtype=torch.bfloat16, device="cuda:0")
        out = buf[1024:1024 + n].view(p.query.shape)
        native.paged_attention(d["query"], d["key_pages"], d["value_pages"], d["block_table"], d["context_lens"],
                               p.page_size, p.scale, True, out=out, schedule=sch)
        torch.cuda.synchronize()
        assert (buf[:1024] == 7.0).all() and (buf[1024 + n:] == 7.0).all()


def test_metadata_check():
    import torch
    from paged_flashattention_kv_amd import native

    p = small(82, B=2, Hq=4, Hkv=2, L=4, ctx=(10, 30), ps=4)
    d = to_device(p)
    native.check_metadata(d["block_table"], d["context_lens"], p.num_pages, p.page_size, 4)
    bad = d["context_lens"].clone()
    bad[1] = 3  # shorter than L under causal
    with pytest.raises(native.PagedAttentionError):
        native.check_metadata(d["block_table"], bad, p.num_pages, p.page_size, 4)
    badt = d["block_table"].clone()
    badt[0, 1] = p.num_pages
    with pytest.raises(native.PagedAttentionError):
        native.check_metadata(badt, d["context_lens"], p.num_pages, p.page_size, 4)


def test_decode_workspace_reuse_and_stale_counters():
    import torch
    from paged_flashattention_kv_amd import native

    p = small(83, B=6, Hq=8, Hkv=2, L=1, ctx=(900, 3000, 70, 1500, 2222, 64), ps=32, poison=True)
    want = ref(p)
    d = to_device(p)
    need = native.workspace_bytes(p.batch, 8, 2, 1, 128, p.page_size, p.max_pages, DECODE, 37)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    ctr = ws[: p.batch * 2 * 8].view(torch.int64)
    for call in range(4):
        if call == 2:
            ctr.fill_(-(1 << 32) + 5)  # left by an interrupted call: another tag, count 5
        out = native.paged_attention(d["query"], d["key_pages"], d["value_pages"], d["block_table"],
                                     d["context_lens"], p.page_size, p.scale, True, workspace=ws,
                                     schedule=DECODE, decode_work_items=37)
        torch.cuda.synchronize()
        parity(out.float().cpu().numpy().astype(np.float64), want, f"workspace reuse call {call}")
        if call < 2:
            assert (ctr == 0).all(), "a clean workspace must be left at zero"
        else:
            # shared segments reset their counter; the others keep the stale tag, which is ignored
            assert ((ctr == 0) | (ctr == -(1 << 32) + 5)).all()


def _prefill_call(p, d, ws):
    import torch
    from paged_flashattention_kv_amd import native

    out = native.paged_attention(d["query"], d["key_pages"], d["value_pages"], d["block_table"],
                                 d["context_lens"], p.page_size, p.scale, p.causal, workspace=ws,
                                 schedule=PREFILL)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("L,ctx,ps,Hq,Hkv,causal", [
    (65, (1065, 3665, 2000), 128, 32, 8, True),   # chunked-continuation rows, ragged key ranges
    (150, (150, 700), 16, 4, 2, True),             # page-crossing tiles, a part with the diagonal
    (40, (40, 300, 5000), 64, 8, 1, False),        # group 8, non-causal, one long range
    (3, (3, 900), 32, 6, 2, True),                 # group 3: packed rows 3 positions x 3 heads
])
def test_prefill_key_range_split(L, ctx, ps, Hq, Hkv, causal):
    """Few work items: the key range splits over workgroups and merges through
    the workspace. Against the oracle, against the unsplit run (a workspace
    too small for the split), bit-identical across repeated calls."""
    import torch
    from paged_flashattention_kv_amd import native

    p = small(900 + L + ps, B=len(ctx), Hq=Hq, Hkv=Hkv, L=L, ctx=ctx, ps=ps, causal=causal, poison=True)
    max_pages = p.block_table.shape[1]
    need = native.workspace_bytes(p.batch, Hq, Hkv, L, 128, ps, max_pages, PREFILL, 0)
    assert need > 0, "the case must take the split"
    say(f"key-range split L={L} ctx={ctx} ps={ps} H={Hq}/{Hkv} causal={causal} workspace={need}")
    want = ref(p)
    d = to_device(p)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    split = _prefill_call(p, d, ws)
    parity(split, want, "split")
    again = _prefill_call(p, d, ws)
    assert np.array_equal(split, again), "the split run must be bit-reproducible"
    unsplit = _prefill_call(p, d, torch.zeros(1, dtype=torch.uint8, device="cuda:0"))
    parity(unsplit, want, "unsplit (no workspace)")
    n_items = len(ctx) * Hkv * ((Hq // Hkv * L + 127) // 128)  # batch x kv heads x packed row tiles
    ctr = ws[: 8 * n_items].view(torch.int64)
    assert (ctr == 0).all(), "the last part resets its counter"


@pytest.mark.parametrize("B,Hq,Hkv,L,D,seed", [
    (20, 6, 3, 70, 128, 1),   # 40 (sequence, row tile) pairs, 3 kv heads: list places not a multiple of 8
    (48, 8, 8, 17, 128, 2),   # 48 one-tile pairs, 8 kv heads: 384 work items, contexts 17 .. 4000
    (6, 4, 4, 130, 256, 3),   # head dim 256: one resident workgroup per CU
    (10, 8, 2, 40, 64, 4),    # head dim 64: three resident workgroups per CU
])
def test_prefill_split_assignment(B, Hq, Hkv, L, D, seed):
    """Key-range parts sized to the launch: pairs of very different lengths
    (one tile to dozens) get from one part to eight, all parts resident at
    once; every output row is written once and matches the oracle, and the
    run is bit-reproducible."""
    import torch
    from paged_flashattention_kv_amd import native

    rng = np.random.default_rng(seed)
    ctx = [int(L + x) for x in rng.integers(0, 4000, size=B)]
    ctx[0] = L  # a pair of one tile
    p = small(1200 + seed, B=B, Hq=Hq, Hkv=Hkv, L=L, ctx=ctx, ps=64, poison=True, D=D)
    max_pages = p.block_table.shape[1]
    need = native.workspace_bytes(B, Hq, Hkv, L, D, 64, max_pages, PREFILL, 0)
    assert need > 0, "the case must take the split"
    say(f"split assignment B={B} H={Hq}/{Hkv} L={L} D={D} workspace={need}")
    want = ref(p)
    d = to_device(p)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    out = torch.full_like(d["query"], float("nan"))  # a row left unwritten stays NaN
    native.paged_attention(d["query"], d["key_pages"], d["value_pages"], d["block_table"], d["context_lens"],
                           p.page_size, p.scale, p.causal, out=out, workspace=ws, schedule=PREFILL)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    parity(got, want, "split assignment")
    again = _prefill_call(p, d, ws)
    assert np.array_equal(got, again), "the split run must be bit-reproducible"


def test_prefill_split_stale_counters():
    """A workspace left by an interrupted call (counters tagged with another
    call, arbitrary partials) is safe to reuse."""
    import torch
    from paged_flashattention_kv_amd import native

    p = small(977, B=3, Hq=8, Hkv=2, L=70, ctx=(70, 1500, 2600), ps=64, poison=True)
    max_pages = p.block_table.shape[1]
    need = native.workspace_bytes(p.batch, 8, 2, 70, 128, 64, max_pages, PREFILL, 0)
    assert need > 0
    want = ref(p)
    d = to_device(p)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    n_items = 3 * 2 * ((4 * 70 + 127) // 128)  # batch x kv heads x packed row tiles
    for call in range(3):
        if call == 1:
            ws.view(torch.int8).random_(-128, 127)  # arbitrary partials and counter words ...
            ws[: 8 * n_items].view(torch.int64).fill_(-(1 << 32) + 1)  # ... counters: another tag, count 1
        got = _prefill_call(p, d, ws)
        parity(got, want, f"stale workspace call {call}")
