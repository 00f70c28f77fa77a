"""GPU parity of the mixed-batch entry point (paged_attention_varlen) against the oracle.

Each case packs sequences with different query lengths -- one-token decodes,
prefill chunks, multi-tile prompts, sequences with no query at all -- into
one call. The float64 oracle is ``oracle.paged_attention_varlen_ref``; the
bar is the operator's (max abs <= 2e-2, mean abs <= 2e-3 for bf16 outputs).
The same input also runs with the decode/prefill split forced (all prefill,
decode for length 1 only, decode for every length that fits one decode work
item) and with few and many decode work items, so both
schedules and the cross-work-item merge see every length mix. Rows of the
uniform entry point and of a uniform-length varlen call are compared bit for
bit (same kernels, only the addressing differs). Pools are NaN-poisoned past
every context end and on unused pages.
"""

import numpy as np
import pytest

import oracle
from paged_flashattention_kv_amd import workloads as wl

from tests.helpers import parity, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_flashattention_kv_amd import native

    native.load()


def _dev(p):
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")

    return dict(query=bf(p.query), key_pages=bf(p.key_pages), value_pages=bf(p.value_pages),
                block_table=i32(p.block_table), context_lens=i32(p.context_lens), query_start=i32(p.query_start))


def _run(p, d=None, max_query_len=None, **kw):
    import torch
    from paged_flashattention_kv_amd import native

    d = d or _dev(p)
    mq = p.max_query_len if max_query_len is None else max_query_len
    o = native.paged_attention_varlen(d["query"], d["key_pages"], d["value_pages"], d["block_table"],
                                      d["context_lens"], d["query_start"], mq, p.page_size, p.scale, p.causal, **kw)
    torch.cuda.synchronize()
    return o


def _f64(o):
    return o.float().cpu().numpy().astype(np.float64)


def _ref(p):
    return oracle.paged_attention_varlen_ref(p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens,
                                             p.query_start, p.page_size, p.scale, p.causal)


def _problem(seed, ql, ctx, Hq=8, Hkv=2, ps=16, causal=True):
    return wl.make_varlen_problem(seed=seed, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128, page_size=ps,
                                  lens=(ql, ctx), causal=causal, poison=True)


# (seed, query lengths, context lengths, H_q, H_kv, page size, causal)
CASES = [
    (601, [1, 37, 1, 2, 128, 1], [300, 37, 5, 1000, 500, 77], 8, 2, 16, True),
    (602, [3, 1, 129, 0, 65], [70, 2048, 129, 0, 1065], 32, 8, 128, True),
    (603, [1, 1, 1, 1], [1, 17, 64, 4097], 32, 8, 128, True),           # decodes only
    (604, [200, 13, 300], [200, 500, 301], 4, 2, 4, True),              # prefill only, 4-token pages
    (605, [2, 1, 50, 7], [33, 999, 50, 7], 16, 16, 5, True),            # MHA, ragged page size
    (606, [1, 9, 1, 130], [90, 600, 3, 200], 16, 1, 64, True),          # group 16: no decode part
    (607, [5, 1, 2, 1, 40], [400, 31, 800, 1, 40], 8, 8, 1, True),      # one-token pages
    (608, [1, 37, 2, 128, 1], [300, 900, 1000, 128, 77], 8, 2, 32, False),  # non-causal
    (609, [0, 1, 0, 64, 0], [0, 300, 0, 64, 0], 8, 2, 16, True),         # empty sequences between
]


@pytest.mark.parametrize("seed,ql,ctx,Hq,Hkv,ps,causal", CASES)
def test_varlen_parity(seed, ql, ctx, Hq, Hkv, ps, causal):
    say(f"varlen seed={seed} ql={ql} ctx={ctx} Hq={Hq} Hkv={Hkv} ps={ps} causal={causal}")
    p = _problem(seed, ql, ctx, Hq, Hkv, ps, causal)
    want = _ref(p)
    d = _dev(p)
    parity(_f64(_run(p, d)), want, f"auto seed={seed}")
    parity(_f64(_run(p, d, decode_max_len=0)), want, f"all-prefill seed={seed}")
    G = Hq // Hkv
    if G <= 8:
        parity(_f64(_run(p, d, decode_max_len=1, decode_work_items=7)), want, f"len1-decode w=7 seed={seed}")
        parity(_f64(_run(p, d, decode_work_items=1000)), want, f"auto w=1000 seed={seed}")
    if 8 // G >= 2:
        # the widest decode split: sequences of different row counts in one decode launch
        parity(_f64(_run(p, d, decode_max_len=8 // G, decode_work_items=300)), want, f"widest-decode seed={seed}")


def test_mixed_batch_workload_parity():
    p = wl.make_varlen_config("mixed_batch", poison=True)
    say(f"mixed_batch T={p.total_query} B={p.batch} max_L={p.max_query_len}")
    parity(_f64(_run(p)), _ref(p), "mixed_batch")


def test_long_prompt_with_decodes():
    p = _problem(611, [1024, 1, 1, 1, 3], [1024, 32768, 4000, 1, 1500], 32, 8, 16, True)
    say("long prompt + decodes")
    parity(_f64(_run(p)), _ref(p), "long prompt + decodes")


def test_uniform_lengths_bit_equal_uniform_entry_point():
    import torch
    from paged_flashattention_kv_amd import native

    for L, seed in ((1, 621), (2, 622), (65, 623), (300, 624)):
        say(f"uniform-vs-varlen L={L}")
        u = wl.make_problem(seed=seed, batch=5, num_q_heads=32, num_kv_heads=8, query_len=L, head_dim=128,
                            page_size=16, context_lens=[L + 7, L + 300, L, L + 1000, L + 64], poison=True)
        q = np.ascontiguousarray(u.query.transpose(0, 2, 1, 3)).reshape(5 * L, 32, 128)
        p = wl.VarlenProblem(name="uniform", query=q, key_pages=u.key_pages, value_pages=u.value_pages,
                             block_table=u.block_table, context_lens=u.context_lens,
                             query_start=(np.arange(6) * L).astype(np.int32), page_size=16, scale=u.scale,
                             causal=True, seed=seed)
        d = _dev(p)
        got = _run(p, d)
        uq = d["query"].view(5, L, 32, 128).transpose(1, 2).contiguous()
        ref = native.paged_attention(uq, d["key_pages"], d["value_pages"], d["block_table"], d["context_lens"], 16,
                                     u.scale, True)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.transpose(1, 2).reshape(5 * L, 32, 128).view(torch.int16))


def test_repeated_calls_are_bit_identical_and_reuse_the_workspace():
    import torch
    from paged_flashattention_kv_amd import native

    p = _problem(631, [1, 2, 70, 1, 1], [3000, 700, 900, 64, 129], 32, 8, 16, True)
    d = _dev(p)
    ws = torch.zeros(native.varlen_workspace_bytes(p.batch, 32, 8, p.max_query_len, 128, 16, p.max_pages),
                     dtype=torch.uint8, device="cuda:0")
    first = _run(p, d, workspace=ws)
    for _ in range(3):
        assert torch.equal(_run(p, d, workspace=ws).view(torch.int16), first.view(torch.int16))
    parity(_f64(first), _ref(p), "repeated")


def test_sequences_with_bad_offsets_are_skipped():
    # offsets past total_query or longer than max_query_len: the sequence is
    # not served (its rows keep what out held), the others are unaffected
    import torch

    p = _problem(641, [2, 3, 1, 4], [40, 50, 60, 70], 8, 2, 16, True)
    want = _ref(p)
    d = _dev(p)
    qs = d["query_start"].clone()
    qs[3] = 20  # sequence 2 now ends past T = 10, sequence 3 starts there
    sentinel = torch.full_like(d["query"], 7.0)
    import paged_flashattention_kv_amd.native as native
    native.paged_attention_varlen(d["query"], d["key_pages"], d["value_pages"], d["block_table"], d["context_lens"],
                                  qs, p.max_query_len, 16, p.scale, True, out=sentinel)
    torch.cuda.synchronize()
    got = _f64(sentinel)
    parity(got[:5], want[:5], "sequences before the bad offset")
    assert (got[5:] == 7.0).all()
    # a sequence longer than the max_query_len the caller passed is skipped too
    out = torch.full_like(d["query"], 7.0)
    native.paged_attention_varlen(d["query"], d["key_pages"], d["value_pages"], d["block_table"], d["context_lens"],
                                  d["query_start"], 3, 16, p.scale, True, out=out)
    torch.cuda.synchronize()
    got = _f64(out)
    parity(got[:6], want[:6], "sequences within max_query_len")
    assert (got[6:] == 7.0).all()


def test_check_varlen_metadata():
    from paged_flashattention_kv_amd import native

    p = _problem(651, [2, 0, 3], [40, 0, 50], 8, 2, 16, True)
    d = _dev(p)
    native.check_varlen_metadata(d["block_table"], d["context_lens"], d["query_start"], p.num_pages, 16,
                                 p.total_query, p.max_query_len)
    bad = d["context_lens"].clone()
    bad[2] = 2  # shorter than its 3 causal queries
    with pytest.raises(native.PagedAttentionError):
        native.check_varlen_metadata(d["block_table"], bad, d["query_start"], p.num_pages, 16, p.total_query,
                                     p.max_query_len)
    qs = d["query_start"].clone()
    qs[1] = 3  # decreases afterwards (3 -> 2)
    with pytest.raises(native.PagedAttentionError):
        native.check_varlen_metadata(d["block_table"], d["context_lens"], qs, p.num_pages, 16, p.total_query,
                                     p.max_query_len)
