"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments with an error code before any
launch. The planning code is also built alone under ASan/UBSan."""

import ctypes
import os
import re
import shutil
import subprocess

import pytest

from paged_flashattention_kv_amd import native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attention.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(paged_\w*)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(native.LIB_PATH):
        pytest.skip("library not built")
    return native.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) == 15
    assert sorted(native.EXPORTED) == names
    raw = ctypes.CDLL(native.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _call(lib, **kw):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, bt=FAKE + 0x300000, cl=FAKE + 0x400000,
             out=FAKE + 0x500000, B=1, Hq=4, Hkv=2, L=1, D=128, P=8, ps=16, mp=4, scale=0.088,
             causal=1, ws=None, wsb=0, sched=0, split=0)
    a.update(kw)
    return lib.paged_attention_ex(a["q"], a["k"], a["v"], a["bt"], a["cl"], a["out"], a["B"], a["Hq"], a["Hkv"],
                                  a["L"], a["D"], a["P"], a["ps"], a["mp"], a["scale"], a["causal"], a["ws"],
                                  a["wsb"], a["sched"], a["split"], None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(q=None), native.PA_ERR_INVALID),
        (dict(out=None), native.PA_ERR_INVALID),
        (dict(B=0), native.PA_ERR_INVALID),
        (dict(Hq=3), native.PA_ERR_INVALID),
        (dict(ps=0), native.PA_ERR_INVALID),
        (dict(L=200), native.PA_ERR_INVALID),
        (dict(causal=2), native.PA_ERR_INVALID),
        (dict(scale=float("nan")), native.PA_ERR_INVALID),
        (dict(D=100), native.PA_ERR_UNSUPPORTED),
        (dict(D=512), native.PA_ERR_UNSUPPORTED),
        (dict(D=0), native.PA_ERR_INVALID),
        (dict(sched=7), native.PA_ERR_INVALID),
        (dict(L=5, sched=1), native.PA_ERR_INVALID),  # 10 rows > 8
        (dict(sched=1, split=-1), native.PA_ERR_INVALID),
        (dict(sched=1, split=70000), native.PA_ERR_INVALID),
        (dict(out=FAKE, sched=2), native.PA_ERR_INVALID),  # aliases the query
        (dict(mp=400, ps=16, B=2, sched=1, split=256), native.PA_ERR_WORKSPACE),
        (dict(mp=400, ps=16, B=2), native.PA_ERR_WORKSPACE),
    ],
)
def test_invalid_arguments_return_codes(lib, kw, code):
    assert _call(lib, **kw) == code
    assert native.last_error() != ""


def _append(lib, **kw):
    a = dict(kn=FAKE, vn=FAKE + 0x100000, kp=FAKE + 0x200000, vp=FAKE + 0x300000, bt=FAKE + 0x400000,
             cl=FAKE + 0x500000, B=2, Hkv=2, L=3, D=128, P=8, ps=16, mp=4)
    a.update(kw)
    return lib.paged_kv_append(a["kn"], a["vn"], a["kp"], a["vp"], a["bt"], a["cl"], a["B"], a["Hkv"], a["L"],
                               a["D"], a["P"], a["ps"], a["mp"], None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(kn=None), native.PA_ERR_INVALID),
        (dict(vp=None), native.PA_ERR_INVALID),
        (dict(cl=None), native.PA_ERR_INVALID),
        (dict(B=0), native.PA_ERR_INVALID),
        (dict(L=0), native.PA_ERR_INVALID),
        (dict(ps=0), native.PA_ERR_INVALID),
        (dict(D=100), native.PA_ERR_UNSUPPORTED),
        (dict(L=65, ps=16, mp=4), native.PA_ERR_INVALID),  # 65 new tokens cannot fit 4 pages of 16
        (dict(mp=1 << 20, ps=1 << 12), native.PA_ERR_UNSUPPORTED),  # positions past int32
        (dict(vp=FAKE + 0x200000 + 4096), native.PA_ERR_INVALID),  # the two pools overlap
        (dict(kn=FAKE + 0x200000), native.PA_ERR_INVALID),  # new keys inside the key pool
    ],
)
def test_append_invalid_arguments_return_codes(lib, kw, code):
    assert _append(lib, **kw) == code
    assert native.last_error() != ""


def _varlen(lib, **kw):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, bt=FAKE + 0x300000, cl=FAKE + 0x400000,
             qs=FAKE + 0x480000, out=FAKE + 0x500000, B=2, Hq=4, Hkv=2, T=5, maxL=4, D=128, P=8, ps=16, mp=4,
             scale=0.088, causal=1, ws=None, wsb=0, dml=-1, split=0)
    a.update(kw)
    return lib.paged_attention_varlen_ex(a["q"], a["k"], a["v"], a["bt"], a["cl"], a["qs"], a["out"], a["B"],
                                         a["Hq"], a["Hkv"], a["T"], a["maxL"], a["D"], a["P"], a["ps"], a["mp"],
                                         a["scale"], a["causal"], a["ws"], a["wsb"], a["dml"], a["split"], None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(qs=None), native.PA_ERR_INVALID),
        (dict(bt=None), native.PA_ERR_INVALID),
        (dict(q=None), native.PA_ERR_INVALID),  # NULL query is allowed only when T == 0
        (dict(T=-1), native.PA_ERR_INVALID),
        (dict(maxL=0), native.PA_ERR_INVALID),
        (dict(maxL=6), native.PA_ERR_INVALID),  # longer than total_query
        (dict(B=0), native.PA_ERR_INVALID),
        (dict(Hq=3), native.PA_ERR_INVALID),
        (dict(causal=2), native.PA_ERR_INVALID),
        (dict(scale=float("inf")), native.PA_ERR_INVALID),
        (dict(D=100), native.PA_ERR_UNSUPPORTED),
        (dict(dml=5), native.PA_ERR_INVALID),  # 5 rows x group 2 > 8
        (dict(dml=-2), native.PA_ERR_INVALID),
        (dict(split=-1), native.PA_ERR_INVALID),
        (dict(T=100, maxL=100, mp=4, ps=16), native.PA_ERR_INVALID),  # causal query longer than any context
        (dict(out=FAKE + 2 * 4 * 128, dml=0), native.PA_ERR_INVALID),  # overlaps the query
        (dict(out=FAKE + 0x480000 - 64, dml=0), native.PA_ERR_INVALID),  # overlaps query_start
        (dict(), native.PA_ERR_WORKSPACE),  # length-1 sequences need the decode workspace
    ],
)
def test_varlen_invalid_arguments_return_codes(lib, kw, code):
    assert _varlen(lib, **kw) == code
    assert native.last_error() != ""


def _masked(lib, **kw):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, bt=FAKE + 0x300000, cl=FAKE + 0x400000,
             m=FAKE + 0x600000, sb=0, sh=0, sl=0, mlen=64, out=FAKE + 0x500000, B=1, Hq=4, Hkv=2, L=1, D=128, P=8,
             ps=16, mp=4, scale=0.088, causal=1, ws=None, wsb=0, sched=2, split=0)
    a.update(kw)
    return lib.paged_attention_masked(a["q"], a["k"], a["v"], a["bt"], a["cl"], a["m"], a["sb"], a["sh"], a["sl"],
                                      a["mlen"], a["out"], a["B"], a["Hq"], a["Hkv"], a["L"], a["D"], a["P"], a["ps"],
                                      a["mp"], a["scale"], a["causal"], a["ws"], a["wsb"], a["sched"], a["split"],
                                      None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(m=None), native.PA_ERR_INVALID),
        (dict(sb=-1), native.PA_ERR_INVALID),
        (dict(sl=-64), native.PA_ERR_INVALID),
        (dict(mlen=0), native.PA_ERR_INVALID),
        (dict(sh=1 << 41), native.PA_ERR_UNSUPPORTED),
        (dict(D=100), native.PA_ERR_UNSUPPORTED),
        (dict(q=None), native.PA_ERR_INVALID),
        (dict(out=FAKE + 0x600000 + 128), native.PA_ERR_INVALID),  # out inside the mask
        (dict(sched=0), native.PA_ERR_WORKSPACE),  # decode schedule without workspace
    ],
)
def test_masked_invalid_arguments_return_codes(lib, kw, code):
    assert _masked(lib, **kw) == code
    assert native.last_error() != ""


def test_varlen_empty_batch_is_a_no_op(lib):
    assert _varlen(lib, q=None, out=None, T=0, maxL=0) == native.PA_OK
    assert native.last_error() == ""


def test_varlen_workspace(lib):
    # a prefill chunk in the batch: only one-token queries take the decode part
    n = native.varlen_workspace_bytes(64, 32, 8, 128, 128, 128, 9)
    assert n == native.workspace_bytes(64, 32, 8, 1, 128, 128, 9, native.SCHEDULE_DECODE, 0)
    # every query within the automatic decode bound (4 rows per kv head): the uniform rule
    assert native.varlen_workspace_bytes(64, 32, 8, 1, 128, 128, 9) == native.workspace_bytes(64, 32, 8, 1, 128, 128, 9)
    assert native.varlen_workspace_bytes(64, 32, 16, 2, 128, 128, 9) == native.workspace_bytes(
        64, 32, 16, 2, 128, 128, 9) > 0
    # 2-token queries at GQA 4 (8 rows) take the prefill schedule; one-token ones the decode part
    assert native.varlen_workspace_bytes(64, 32, 8, 2, 128, 128, 9) == native.workspace_bytes(
        64, 32, 8, 1, 128, 128, 9, native.SCHEDULE_DECODE, 0)
    assert native.varlen_workspace_bytes(64, 32, 8, 128, 128, 128, 9, decode_max_len=0) == 0
    # group 16: no decode part; 256 prefill work items (16 heads x 128 positions = 2048 rows
    # per kv head) take the key-range split, whose workspace is the uniform prefill's
    assert native.varlen_workspace_bytes(4, 64, 4, 128, 128, 128, 9) == native.workspace_bytes(
        4, 64, 4, 128, 128, 128, 9, native.SCHEDULE_PREFILL, 0) > 0
    with pytest.raises(native.PagedAttentionError):
        native.varlen_workspace_bytes(64, 32, 8, 128, 128, 128, 9, decode_max_len=3)


def test_schedule_rule_and_workspace(lib):
    assert native.schedule_for(64, 32, 8, 1, 128, 128, 33) == native.SCHEDULE_DECODE
    assert native.schedule_for(64, 32, 8, 2, 128, 128, 33) == native.SCHEDULE_PREFILL  # 8 rows per kv head
    assert native.schedule_for(64, 32, 16, 2, 128, 128, 33) == native.SCHEDULE_DECODE  # 4 rows
    assert native.schedule_for(64, 32, 8, 3, 128, 128, 33) == native.SCHEDULE_PREFILL
    assert native.schedule_for(1, 8, 8, 4, 128, 128, 33) == native.SCHEDULE_DECODE
    assert native.schedule_for(1, 8, 8, 8, 128, 128, 33) == native.SCHEDULE_PREFILL
    assert native.schedule_for(4, 32, 8, 2048, 128, 128, 16) == native.SCHEDULE_PREFILL
    assert native.workspace_bytes(4, 32, 8, 2048, 128, 128, 16) == 0
    # the 64 x 32 prefill tiling: no workspace (never split), native head dims only
    assert native.workspace_bytes(8, 32, 8, 65, 128, 128, 30, native.SCHEDULE_PREFILL_64X32, 0) == 0
    with pytest.raises(native.PagedAttentionError):
        native.workspace_bytes(8, 32, 8, 65, 80, 128, 30, native.SCHEDULE_PREFILL_64X32, 0)
    with pytest.raises(native.PagedAttentionError):
        native.workspace_bytes(8, 32, 8, 65, 128, 128, 30, 4, 0)
    # decode: arrival counters plus two partial (max, sum, acc[D]) slots per work item and row
    n = native.workspace_bytes(16, 32, 8, 1, 128, 16, 2048)
    assert n >= 16 * 8 * 8 + 2048 * 2 * 4 * 130 * 4
    assert native.workspace_bytes(16, 32, 8, 1, 128, 16, 2048, native.SCHEDULE_DECODE, 100) < n
    with pytest.raises(native.PagedAttentionError):
        native.workspace_bytes(1, 3, 2, 1, 128, 16, 4)


def test_host_planning_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ missing")
    exe = str(tmp_path / "plan_check")
    csrc = os.path.join(ROOT, "paged_flashattention_kv_amd", "csrc")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{csrc}", os.path.join(ROOT, "tests", "host", "plan_check.cpp"), os.path.join(csrc, "pa_plan.cpp"),
           "-o", exe]
    subprocess.run(cmd, check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all passed" in r.stdout


def test_static_entry_point_rejects_before_any_launch(lib):
    # argument errors of the allocation-free entry point come back before it
    # touches a device (this host has none): NULL tensors, then a decode shape
    # whose counters and partials would not fit the 64 MiB scratch
    import torch

    if torch.cuda.is_available():
        pytest.skip("host-only error paths")
    assert lib.paged_attention_static_scratch_bytes() == 64 << 20
    rc = lib.paged_attention_static(None, None, None, None, None, None, 1, 32, 8, 1, 128, 10, 16, 4,
                                    ctypes.c_float(0.088), 1, None)
    assert rc == native.PA_ERR_INVALID
