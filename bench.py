"""Benchmark of the paged attention operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--repeats R]
                    [--no-cpu-baseline] [--no-extra] [--only CASES] [--inline]
    python bench.py --sweep dispatch [--out FILE]

A step is one call of the operator (one kernel launch of the schedule the
dispatcher picks) over one batch of synthetic input. The headline workload
is the decode batch at the Qwen3-4B attention shape (B=64, H_q=32, H_kv=8,
D=128, L=1, context lengths U[128, 4096] not tile multiples, 128-token
pages shuffled over a pool sized to what the batch needs). Inputs are
resident in HBM before the timed region. Each case first runs untimed for
--prewarm-seconds (0.3 s) so the engine clock has settled, then W warmup
calls, then exactly K timed calls between two HIP events on the launch
stream. Three independent copies of the K/V page pool are rotated step by
step so that the 256 MB Infinity Cache cannot serve repeated reads.

Measurement protocol ("Week 2 Day 5: Fused Decode Attention", "Benchmark
Analysis": repeated fresh-process passes in rotated order, every sample
kept, medians reported): this process draws every workload once on the CPU
and never touches the GPU; it then starts R fresh child processes (default
3), each timing every case once, child i in the case order rotated by i.
Every reported time is the median over the R children, with the quartiles
and all samples beside it. ``--inline`` times the cases once in this process
instead (for profilers, which must see the kernels in the process they
start).

Printed: one JSON line. ``value`` is decode K/V throughput in TB/s
(algorithmic bytes: 4096 B per visible context position = H_kv * D * 2
bytes * (K + V)). ``roofline`` compares the kernel against the 8 TB/s HBM
peak; its ``traffic`` field is the HBM byte count measured with rocprofv3
counters for this kernel source (null when the source changed since).
``cpu_baseline`` is the float64 CPU oracle timed on this host's cores over
whole passes of the same workload. ``extra`` holds the long causal prefill
(TFLOP/s against the dense bf16 MFMA peak), the chunked continuation, the
long-context decode, the K/V appends, the masked variants and a mixed batch.

``--sweep dispatch`` times both schedules over query lengths, context lengths
and GQA ratios (the crossover the host dispatch rule is set from) and prints
a markdown table.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import shutil
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode K/V TB/s (% HBM peak); causal prefill TFLOP/s (% bf16 MFMA peak)"
HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
POOL_COPIES = 3
PREWARM_SECONDS = 0.3  # untimed sustained load before each case's warmup calls (set by --prewarm-seconds)
KERNEL_SOURCES = {
    "pa_decode_work": ["paged_flashattention_kv_amd/csrc/pa_decode.hip", "paged_flashattention_kv_amd/csrc/pa_device.h"],
    "pa_prefill_mfma": ["paged_flashattention_kv_amd/csrc/pa_prefill.hip", "paged_flashattention_kv_amd/csrc/pa_device.h"],
    "pa_kv_append": ["paged_flashattention_kv_amd/csrc/pa_append.hip", "paged_flashattention_kv_amd/csrc/pa_device.h"],
}

# Workloads drawn once by the parent: name -> (generator, config name)
PROBLEMS = {
    "decode_batch": ("uniform", "decode_batch"),
    "long_prefill": ("uniform", "long_prefill"),
    "chunked_continuation": ("uniform", "chunked_continuation"),
    "long_decode": ("uniform", "long_decode"),
    "mixed_batch": ("varlen", "mixed_batch"),
}
EXTRA_CASES = [
    "long_prefill", "long_prefill_64x32", "chunked_continuation", "long_decode", "kv_append_prefill",
    "kv_append_decode", "masked_decode", "masked_prefill", "mixed_batch",
]
CASE_PROBLEM = {
    "decode_batch": "decode_batch", "long_prefill": "long_prefill", "long_prefill_64x32": "long_prefill",
    "chunked_continuation": "chunked_continuation",
    "long_decode": "long_decode", "kv_append_prefill": "long_prefill", "kv_append_decode": "decode_batch",
    "masked_decode": "decode_batch", "masked_prefill": "long_prefill", "mixed_batch": "mixed_batch",
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if still current.

    profiles/<kernel>__<workload>.md ends with a line
    ``traffic_bytes_per_launch: N source_sha: H``; the count is used only
    while the kernel's source still hashes to H.
    """
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}.md")
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch: (\d+) source_sha: ([0-9a-f]+)", text)
    if not m or m.group(2) != source_hash(kernel):
        return None
    return int(m.group(1))


# ------------------------------------------------------------------ problem cache (host only)


def draw_problem(name: str):
    from paged_flashattention_kv_amd import workloads as wl

    kind, cfg = PROBLEMS[name]
    return wl.make_config(cfg) if kind == "uniform" else wl.make_varlen_config(cfg)


def save_problem(p, directory: str) -> None:
    import numpy as np

    os.makedirs(directory, exist_ok=True)
    meta = {"class": type(p).__name__}
    for f in dataclasses.fields(p):
        v = getattr(p, f.name)
        if isinstance(v, np.ndarray):
            np.save(os.path.join(directory, f.name + ".npy"), v)
        else:
            meta[f.name] = v
    with open(os.path.join(directory, "meta.json"), "w") as fh:
        json.dump(meta, fh)


def load_problem(directory: str):
    import numpy as np

    from paged_flashattention_kv_amd import workloads as wl

    with open(os.path.join(directory, "meta.json")) as fh:
        meta = json.load(fh)
    cls = getattr(wl, meta.pop("class"))
    kw = dict(meta)
    for f in dataclasses.fields(cls):
        if f.name not in kw:
            kw[f.name] = np.load(os.path.join(directory, f.name + ".npy"), mmap_mode="r")
    return cls(**kw)


# ------------------------------------------------------------------ GPU cases (child / inline)


def _bf(a, dev="cuda:0"):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


class Case:
    """Device copies of a problem plus a callable that runs one step."""

    def __init__(self, p, copies: int, schedule: int = 0):
        import torch
        from paged_flashattention_kv_amd import native

        self.p = p
        self.schedule = schedule
        dev = "cuda:0"
        self.q = _bf(p.query)
        k = _bf(p.key_pages)
        v = _bf(p.value_pages)
        self.pools = [(k, v)] + [(k.clone(), v.clone()) for _ in range(copies - 1)]
        self.bt = torch.from_numpy(p.block_table.copy()).to(dev)
        self.ctx = torch.from_numpy(p.context_lens.copy()).to(dev)
        self.out = torch.empty_like(self.q)
        need = native.workspace_bytes(p.batch, p.num_q_heads, p.num_kv_heads, p.query_len, p.head_dim,
                                      p.page_size, p.max_pages, schedule, 0)
        self.ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
        self.i = 0
        self._native = native

    def step(self):
        k, v = self.pools[self.i % len(self.pools)]
        self.i += 1
        self._native.paged_attention(self.q, k, v, self.bt, self.ctx, self.p.page_size, self.p.scale, self.p.causal,
                                     out=self.out, workspace=self.ws, schedule=self.schedule)

    def time(self, steps: int, warmup: int):
        """ms per step over exactly ``steps`` calls, HIP events on the launch stream.

        Before the ``warmup`` calls the case runs untimed for PREWARM_SECONDS of
        wall time: the engine clock of the GPU settles only after sustained load
        (the first ~10 ms of a matrix-core-bound kernel run up to 20% slower),
        so the timed calls see the steady state a serving loop runs in.
        """
        import torch

        t_end = time.perf_counter() + PREWARM_SECONDS
        while time.perf_counter() < t_end:
            for _ in range(8):
                self.step()
            torch.cuda.synchronize()
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(stream)
        for _ in range(steps):
            self.step()
        stop.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return start.elapsed_time(stop) / steps, wall / steps * 1e3


class AppendCase:
    """The K/V append of ``new_len`` tokens per sequence into a problem's pools (the write half)."""

    def __init__(self, p, new_len: int, copies: int):
        import numpy as np
        import torch
        from paged_flashattention_kv_amd import native
        from paged_flashattention_kv_amd import workloads as wl

        dev = "cuda:0"
        rng = np.random.Generator(np.random.PCG64(1000 + p.seed))
        shape = (p.batch, p.num_kv_heads, new_len, p.head_dim)
        kn = _bf(wl.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32)))
        vn = _bf(wl.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32)))
        # sources rotated so that repeats are not served by the Infinity Cache
        self.src = [(kn, vn)] + [(kn.clone(), vn.clone()) for _ in range(copies - 1)]
        self.k = _bf(p.key_pages)
        self.v = _bf(p.value_pages)
        self.bt = torch.from_numpy(p.block_table.copy()).to(dev)
        self.ctx = torch.from_numpy(p.context_lens.copy()).to(dev)
        self.p = p
        self.i = 0
        self._native = native
        # bytes the method must move: every new K and V byte read once and written once
        self.bytes = 2 * 2 * p.batch * p.num_kv_heads * new_len * p.head_dim * 2

    def step(self):
        kn, vn = self.src[self.i % len(self.src)]
        self.i += 1
        self._native.kv_append(kn, vn, self.k, self.v, self.bt, self.ctx, self.p.page_size)

    time = Case.time


class VarlenCase:
    """A mixed batch (per-sequence query lengths) through paged_attention_varlen, pools rotated."""

    def __init__(self, p, copies: int):
        import torch
        from paged_flashattention_kv_amd import native

        dev = "cuda:0"
        self.p = p
        self.q = _bf(p.query)
        k = _bf(p.key_pages)
        v = _bf(p.value_pages)
        self.pools = [(k, v)] + [(k.clone(), v.clone()) for _ in range(copies - 1)]
        self.bt = torch.from_numpy(p.block_table.copy()).to(dev)
        self.ctx = torch.from_numpy(p.context_lens.copy()).to(dev)
        self.qs = torch.from_numpy(p.query_start.copy()).to(dev)
        self.out = torch.empty_like(self.q)
        need = native.varlen_workspace_bytes(p.batch, p.num_q_heads, p.num_kv_heads, p.max_query_len, p.head_dim,
                                             p.page_size, p.max_pages)
        self.ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
        self.i = 0
        self._native = native

    def step(self):
        k, v = self.pools[self.i % len(self.pools)]
        self.i += 1
        self._native.paged_attention_varlen(self.q, k, v, self.bt, self.ctx, self.qs, self.p.max_query_len,
                                            self.p.page_size, self.p.scale, self.p.causal, out=self.out,
                                            workspace=self.ws)

    time = Case.time


class MaskedCase(Case):
    """A problem through paged_attention_masked with a seeded additive mask of shape ``mshape``."""

    def __init__(self, p, copies: int, mshape):
        import numpy as np
        import torch

        super().__init__(p, copies)
        rng = np.random.Generator(np.random.PCG64(2000 + p.seed))
        m = rng.normal(0.0, 1.0, size=mshape).astype(np.float32)
        m[rng.random(mshape) < 0.1] = -np.inf
        m[..., 0] = 0.0
        self.mask = torch.from_numpy(m).to("cuda:0")
        # mask entries read: one per (row, head, visible key) for the axes the mask does not broadcast
        per_key = (mshape[1] if mshape[1] > 1 else 1) * (mshape[2] if mshape[2] > 1 else 1)
        self.mask_bytes = 4 * per_key * int(p.context_lens.astype(np.int64).sum()) if mshape[0] > 1 else None

    def step(self):
        k, v = self.pools[self.i % len(self.pools)]
        self.i += 1
        self._native.paged_attention_masked(self.q, k, v, self.bt, self.ctx, self.mask, self.p.page_size,
                                            self.p.scale, self.p.causal, out=self.out, workspace=self.ws)


def _case_steps(name: str, steps: int, warmup: int):
    if name == "decode_batch":
        return steps, warmup
    if name == "long_decode":  # 2 GiB per step
        return max(10, steps // 10), max(3, warmup // 10)
    if name == "mixed_batch":
        return max(20, steps // 2), max(5, warmup // 2)
    return max(20, steps // 4), max(5, warmup // 4)


def time_case(name: str, probs: dict, steps: int, warmup: int) -> dict:
    """One timing of one case on cuda:0: ms per call plus what the aggregate needs."""
    import torch

    p = probs[CASE_PROBLEM[name]]
    k, w = _case_steps(name, steps, warmup)
    info = {}
    if name in ("decode_batch", "chunked_continuation", "masked_decode", "masked_prefill"):
        c = (MaskedCase(p, POOL_COPIES, (64, 32, 1, 4096)) if name == "masked_decode" else
             MaskedCase(p, POOL_COPIES, (4, 1, 2048, 2048)) if name == "masked_prefill" else Case(p, POOL_COPIES))
        if name == "masked_decode":
            info["mask_bytes"] = c.mask_bytes
    elif name in ("long_prefill", "long_decode"):
        c = Case(p, 1)  # long_decode: 2 GiB per step already exceeds the Infinity Cache
    elif name == "long_prefill_64x32":
        from paged_flashattention_kv_amd import native

        c = Case(p, 1, schedule=native.SCHEDULE_PREFILL_64X32)
    elif name == "kv_append_prefill":
        c = AppendCase(p, 2048, 8)
        info["bytes"] = c.bytes
    elif name == "kv_append_decode":
        c = AppendCase(p, 1, 8)
        info["bytes"] = c.bytes
    elif name == "mixed_batch":
        c = VarlenCase(p, 8)
    else:
        raise KeyError(name)
    ms, wall_ms = c.time(k, w)
    del c
    torch.cuda.empty_cache()
    return {"ms": ms, "wall_ms": wall_ms, "steps": k, "warmup": w, **info}


def run_cases(names, probs, steps, warmup, rotate: int) -> dict:
    order = names[rotate % len(names):] + names[: rotate % len(names)]
    out = {}
    for n in order:
        out[n] = time_case(n, probs, steps, warmup)
        print(f"[bench] {n}: {out[n]['ms'] * 1e3:.2f} us", file=sys.stderr, flush=True)
    out["_order"] = order
    return out


def child_main(args) -> None:
    """Time every case once in this fresh process; print one JSON object."""
    import torch

    from paged_flashattention_kv_amd import native

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    native.load()
    torch.cuda.set_device(0)
    probs = {n: load_problem(os.path.join(args.cache, n)) for n in os.listdir(args.cache)}
    res = run_cases(args.cases.split(","), probs, args.steps, args.warmup, args.rotate)
    print(json.dumps(res), flush=True)


# ------------------------------------------------------------------ aggregate and report


def _stats(samples):
    import numpy as np

    a = np.asarray(samples, dtype=np.float64)
    q1, med, q3 = np.percentile(a, [25, 50, 75])
    return {"median": float(med), "q1": float(q1), "q3": float(q3), "samples": [round(float(x), 6) for x in a]}


def mixed_roofline_us(p) -> dict:
    """Lower bound of one mixed-batch call on this chip: the decode part's K/V bytes at HBM peak plus the
    prefill part's flops at the bf16 matrix peak (the two launches run one after the other)."""
    ql = p.query_lens
    group = p.num_q_heads // p.num_kv_heads
    if group * p.max_query_len <= 4:  # the library's automatic split (decode while G * L <= 4)
        dec_max = p.max_query_len
    else:
        dec_max = 1 if group <= 4 else 0
    dec = (ql >= 1) & (ql <= dec_max)
    pre = ql > dec_max
    ctx = p.context_lens.astype("int64")
    dec_bytes = int(ctx[dec].sum()) * p.num_kv_heads * p.head_dim * 4
    pre_pairs = 0
    for L, c in zip(ql[pre].tolist(), ctx[pre].tolist()):
        pre_pairs += L * (c - L) + L * (L + 1) // 2 if p.causal else L * c
    pre_flops = 4 * p.head_dim * p.num_q_heads * pre_pairs
    t = dec_bytes / (HBM_PEAK_GBPS * 1e9) + pre_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    return {"decode_kv_bytes": dec_bytes, "prefill_flops": pre_flops, "bound_us": round(t * 1e6, 3)}


def _traffic(spec, kernel, workload):
    """``traffic``: True = the profile of (kernel, workload); a (kernel, workload) pair = that profile."""
    if spec is True:
        return measured_traffic(kernel, workload)
    return measured_traffic(*spec) if spec else None


def _hbm_roofline(byt, ms, kernel, workload, traffic=True, **more):
    g = byt / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(g, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(g / HBM_PEAK_GBPS, 4),
            "traffic": _traffic(traffic, kernel, workload),
            "kernel": kernel, "algorithmic_bytes_per_launch": byt, **more}


def _mfma_roofline(flops, ms, kernel, workload, traffic=True):
    tf = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": _traffic(traffic, kernel, workload),
            "kernel": kernel, "algorithmic_flops_per_launch": flops}


def describe_extra(name: str, p, st: dict, info: dict) -> dict:
    ms = st["median"]
    timing = {"ms_per_step": round(ms, 5), "repeats": len(st["samples"]), "iqr_ms": [round(st["q1"], 5),
              round(st["q3"], 5)], "samples_ms": st["samples"], "steps": info["steps"], "warmup": info["warmup"]}
    if name == "long_prefill":
        tf = p.flops() / (ms * 1e-3) / 1e12
        return {"workload": "B=4 L=ctx=2048 H_q=32 H_kv=8 D=128 causal, page_size=128 shuffled", **timing,
                "value": round(tf, 2), "unit": "TFLOP/s",
                "roofline": _mfma_roofline(p.flops(), ms, "pa_prefill_mfma", "long_prefill")}
    if name == "long_prefill_64x32":
        tf = p.flops() / (ms * 1e-3) / 1e12
        return {"workload": "long_prefill at the stated tiling: 64 packed query rows x 32 keys per tile "
                            "(PA_SCHEDULE_PREFILL_64X32; the row above is the automatic 128 x 64 tiling)",
                **timing, "value": round(tf, 2), "unit": "TFLOP/s",
                "roofline": _mfma_roofline(p.flops(), ms, "pa_prefill_mfma (64x32)", "",
                                           traffic=("pa_prefill_mfma", "long_prefill_64x32"))}
    if name == "chunked_continuation":
        return {"workload": "B=8 L=65 history U[1000,3600] (seed 4) H_q=32 H_kv=8 D=128 causal, page_size=128",
                **timing, "tflops": round(p.flops() / (ms * 1e-3) / 1e12, 2),
                "kv_tbps": round(p.kv_bytes() / (ms * 1e-3) / 1e12, 4),
                "roofline_mfma": _mfma_roofline(p.flops(), ms, "pa_prefill_mfma", "chunked_continuation"),
                "roofline_hbm": _hbm_roofline(p.kv_bytes(), ms, "pa_prefill_mfma", "chunked_continuation")}
    if name == "long_decode":
        g = p.kv_bytes() / (ms * 1e-3) / 1e12
        return {"workload": "B=16 L=1 ctx=32768 H_q=32 H_kv=8 D=128, page_size=16 shuffled over 32768 pages",
                **timing, "value": round(g, 4), "unit": "TB/s",
                "roofline": _hbm_roofline(p.kv_bytes(), ms, "pa_decode_work", "long_decode")}
    if name in ("kv_append_prefill", "kv_append_decode"):
        new_len = 2048 if name == "kv_append_prefill" else 1
        byt = info["bytes"]
        return {"workload": f"append {new_len} new token(s) per sequence into the {CASE_PROBLEM[name]} pools "
                            f"(B={p.batch} H_kv={p.num_kv_heads} D=128, page_size={p.page_size})",
                **timing, "value": round(byt / (ms * 1e-3) / 1e12, 4), "unit": "TB/s",
                "roofline": _hbm_roofline(byt, ms, "pa_kv_append", name)}
    if name == "masked_decode":
        byt = p.kv_bytes() + info["mask_bytes"]
        return {"workload": "decode_batch with an explicit fp32 mask [64, 32, 1, 4096] (N(0,1) log-weights, 10% -inf)",
                **timing, "value": round(byt / (ms * 1e-3) / 1e12, 4), "unit": "TB/s",
                "roofline": _hbm_roofline(byt, ms, "pa_decode_work (masked)", "",
                                          traffic=("pa_decode_work", "masked_decode"), mask_bytes=info["mask_bytes"])}
    if name == "masked_prefill":
        tf = p.flops() / (ms * 1e-3) / 1e12
        return {"workload": "long_prefill with an explicit fp32 mask [4, 1, 2048, 2048] shared by the heads",
                **timing, "value": round(tf, 2), "unit": "TFLOP/s",
                "roofline": _mfma_roofline(p.flops(), ms, "pa_prefill_mfma (masked)", "",
                                           traffic=("pa_prefill_mfma", "masked_prefill"))}
    if name == "mixed_batch":
        rl = mixed_roofline_us(p)
        return {"workload": f"mixed_batch: B={p.batch}, {int((p.query_lens > 1).sum())} prefill chunks (<=128 "
                            f"tokens) + {int((p.query_lens == 1).sum())} one-token decodes, T={p.total_query} "
                            f"H_q=32 H_kv=8 D=128, prompts U[128,1024] outputs U[32,128] (seed 6), page_size=128 "
                            f"shuffled",
                **timing, "tokens_per_s": round(p.total_query / (ms * 1e-3), 1),
                "kv_tbps": round(p.kv_bytes() / (ms * 1e-3) / 1e12, 4),
                "tflops": round(p.flops() / (ms * 1e-3) / 1e12, 2),
                "roofline": {"bound": "hbm+mfma", "bound_us": rl["bound_us"], "achieved_us": round(ms * 1e3, 2),
                             "frac": round(rl["bound_us"] / (ms * 1e3), 4), "decode_kv_bytes": rl["decode_kv_bytes"],
                             "prefill_flops": rl["prefill_flops"], "kernels": ["pa_decode_work", "pa_prefill_mfma"]}}
    raise KeyError(name)


def cpu_baseline(p, min_seconds: float):
    """float64 oracle on whole passes over the workload; TB/s over the same algorithmic bytes."""
    import oracle

    threads = None
    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"), default=None)
    except Exception:
        threads = None
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.paged_attention_ref(p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens,
                                   p.page_size, p.scale, p.causal)
        passes += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {
        "value": round(p.kv_bytes() * passes / el / 1e12, 6),
        "unit": "TB/s",
        "cores": int(threads or os.cpu_count() or 1),
        "kind": "oracle",
        "sample": f"{passes} full passes over the {p.name} workload ({p.batch} sequences, "
                  f"{int(p.context_lens.sum())} context positions) in {el:.1f} s; float64 NumPy/BLAS, "
                  f"host has {os.cpu_count()} logical CPUs",
    }


def report(args, probs, runs) -> dict:
    """The JSON line: medians over the fresh-process runs."""
    names = [n for n in runs[0] if not n.startswith("_")]
    stats = {n: _stats([r[n]["ms"] for r in runs]) for n in names}
    p = probs["decode_batch"]
    st = stats["decode_batch"]
    ms = st["median"]
    kv = p.kv_bytes()
    result = {
        "metric": METRIC,
        "value": round(kv / (ms * 1e-3) / 1e12, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode_batch: B=64 L=1 H_q=32 H_kv=8 D=128, context U[128,4096] (seed 2), "
                        "page_size=128, shuffled pool",
            "batch": p.batch, "query_len": 1, "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128,
            "page_size": p.page_size, "context_positions": int(p.context_lens.sum()),
            "kv_bytes_per_step": kv, "pool_copies_rotated": POOL_COPIES, "schedule": "decode",
            "wall_ms_per_step": round(float(sorted(r["decode_batch"]["wall_ms"] for r in runs)[len(runs) // 2]), 5),
        },
        "stats": {"repeats": len(runs), "fresh_processes": not args.inline, "median_ms": round(ms, 5),
                  "iqr_ms": [round(st["q1"], 5), round(st["q3"], 5)], "samples_ms": st["samples"],
                  "case_orders": [r["_order"] for r in runs]},
        "roofline": _hbm_roofline(kv, ms, "pa_decode_work", "decode_batch"),
    }
    extra = {}
    for n in names:
        if n == "decode_batch":
            continue
        extra[n] = describe_extra(n, probs[CASE_PROBLEM[n]], stats[n], runs[0][n])
    if extra:
        result["extra"] = extra
    return result


def parent_main(args) -> None:
    """Draw the workloads (CPU only), time them in fresh child processes, report medians."""
    names = ["decode_batch"] + ([] if args.no_extra else EXTRA_CASES)
    if args.only:
        names = [n for n in args.only.split(",") if n]
        bad = [n for n in names if n not in CASE_PROBLEM]
        if bad:
            sys.exit(f"unknown case(s) {bad}; known: {sorted(CASE_PROBLEM)}")
        if "decode_batch" not in names:
            names = ["decode_batch"] + names  # the headline line is always measured
    need = sorted({CASE_PROBLEM[n] for n in names})
    t0 = time.perf_counter()
    probs = {n: draw_problem(n) for n in need}
    print(f"[bench] workloads drawn in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    if args.inline:
        import torch

        from paged_flashattention_kv_amd import native

        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(1)
        native.load()
        torch.cuda.set_device(0)
        if args.copy_calibration:
            n = 1 << 30
            a = torch.ones(n, dtype=torch.uint8, device="cuda:0")
            b = torch.empty_like(a)
            b.copy_(a)
            torch.cuda.synchronize()
            del a, b
        runs = [run_cases(names, probs, args.steps, args.warmup, 0)]
    else:
        cache = tempfile.mkdtemp(prefix="pa_bench_", dir="/tmp" if os.path.isdir("/tmp") else None)
        try:
            for n, p in probs.items():
                save_problem(p, os.path.join(cache, n))
            runs = []
            for i in range(args.repeats):
                cmd = [sys.executable, os.path.abspath(__file__), "--child", "--cache", cache, "--cases",
                       ",".join(names), "--rotate", str(i), "--steps", str(args.steps), "--warmup",
                       str(args.warmup), "--prewarm-seconds", str(PREWARM_SECONDS)]
                print(f"[bench] fresh process {i + 1}/{args.repeats}", file=sys.stderr, flush=True)
                r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
                if r.returncode != 0:
                    sys.exit(f"bench child {i} failed with exit status {r.returncode}")
                runs.append(json.loads(r.stdout.strip().splitlines()[-1]))
        finally:
            shutil.rmtree(cache, ignore_errors=True)
    result = report(args, probs, runs)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(probs["decode_batch"], args.cpu_seconds)
    print(json.dumps(result), flush=True)


# ------------------------------------------------------------------ dispatch sweep


def sweep_dispatch(args) -> None:
    """Both schedules over L x context x GQA ratio (decode only where G*L <= 8); markdown table."""
    import torch

    from paged_flashattention_kv_amd import native

    native.load()
    torch.cuda.set_device(0)
    dev = "cuda:0"
    B, Hq, D, ps = 16, 32, 128, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    rows_out = []
    for G in (1, 4, 8):
        Hkv = Hq // G
        for ctx in (128, 1024, 4096, 32768):
            pages = (ctx + ps - 1) // ps
            P = B * pages
            kp = torch.randn(P, Hkv, ps, D, device=dev, generator=gen).to(torch.bfloat16)
            vp = torch.randn(P, Hkv, ps, D, device=dev, generator=gen).to(torch.bfloat16)
            perm = torch.randperm(P, device=dev, generator=gen).to(torch.int32)
            bt = perm.view(B, pages).contiguous()
            cl = torch.full((B,), ctx, dtype=torch.int32, device=dev)
            for L in (1, 2, 3, 4, 6, 8, 16):
                q = torch.randn(B, Hq, L, D, device=dev, generator=gen).to(torch.bfloat16)
                out = torch.empty_like(q)
                times = {}
                for sched, label in ((1, "decode"), (2, "prefill")):
                    if sched == 1 and G * L > 8:
                        continue
                    need = native.workspace_bytes(B, Hq, Hkv, L, D, ps, pages, sched, 0)
                    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)

                    def step():
                        native.paged_attention(q, kp, vp, bt, cl, ps, None, True, out=out, workspace=ws,
                                               schedule=sched)

                    t_end = time.perf_counter() + 0.1
                    while time.perf_counter() < t_end:
                        for _ in range(4):
                            step()
                        torch.cuda.synchronize()
                    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    s0.record()
                    for _ in range(args.steps):
                        step()
                    s1.record()
                    torch.cuda.synchronize()
                    times[label] = s0.elapsed_time(s1) / args.steps * 1e3
                auto = native.schedule_for(B, Hq, Hkv, L, D, ps, pages)
                best = min(times, key=times.get)
                rows_out.append(dict(G=G, ctx=ctx, L=L, decode_us=times.get("decode"), prefill_us=times["prefill"],
                                     best=best, auto="decode" if auto == 1 else "prefill"))
                print(f"[sweep] G={G} ctx={ctx} L={L} " + " ".join(f"{k}={v:.1f}us" for k, v in times.items()),
                      file=sys.stderr, flush=True)
            del kp, vp
            torch.cuda.empty_cache()
    lines = ["| GQA | context | L | rows G*L | decode us | prefill us | faster | auto picks |",
             "|---|---|---|---|---|---|---|---|"]
    for r in rows_out:
        d = "-" if r["decode_us"] is None else f"{r['decode_us']:.1f}"
        lines.append(f"| {r['G']} | {r['ctx']} | {r['L']} | {r['G'] * r['L']} | {d} | {r['prefill_us']:.1f} | "
                     f"{r['best']} | {r['auto']} |")
    text = "\n".join(lines)
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            json.dump(rows_out, f)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=12)
    ap.add_argument("--repeats", type=int, default=3, help="fresh child processes, each timing every case once")
    ap.add_argument("--inline", action="store_true", help="time the cases once in this process (for profilers)")
    ap.add_argument("--only", default="", help="comma-separated cases (the headline case is always included)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--prewarm-seconds", type=float, default=PREWARM_SECONDS,
                    help="untimed sustained load before each case's warmup calls (the engine clock settles)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="with --inline: first run one 1 GiB device copy (reference for counter scaling)")
    ap.add_argument("--sweep", choices=["dispatch"], default=None)
    ap.add_argument("--out", default="")
    # internal: one fresh timing process started by the parent
    ap.add_argument("--child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--cache", default="", help=argparse.SUPPRESS)
    ap.add_argument("--cases", default="", help=argparse.SUPPRESS)
    ap.add_argument("--rotate", type=int, default=0, help=argparse.SUPPRESS)
    args = ap.parse_args()
    globals()["PREWARM_SECONDS"] = max(0.0, args.prewarm_seconds)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this operator build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.child:
        child_main(args)
    elif args.sweep == "dispatch":
        sweep_dispatch(args)
    else:
        if args.repeats < 1:
            sys.exit("--repeats must be >= 1")
        parent_main(args)


if __name__ == "__main__":
    main()
