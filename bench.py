"""Benchmark of the paged attention operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]

A step is one call of the operator (one kernel launch of the schedule the
dispatcher picks) over one batch of synthetic input. The headline workload
is the decode batch at the Qwen3-4B attention shape (B=64, H_q=32, H_kv=8,
D=128, L=1, context lengths U[128, 4096] not tile multiples, 128-token
pages shuffled over a pool sized to what the batch needs). Inputs are
resident in HBM before the timed region. Each case first runs untimed for
--prewarm-seconds (0.3 s) so the engine clock has settled, then W warmup
calls, then exactly K timed calls. Three independent copies of the
K/V page pool are rotated step by step so that the 256 MB Infinity Cache
cannot serve repeated reads.

Printed: one JSON line. ``value`` is decode K/V throughput in TB/s
(algorithmic bytes: 4096 B per visible context position = H_kv * D * 2
bytes * (K + V)). ``roofline`` compares the kernel against the 8 TB/s HBM
peak; its ``traffic`` field is the HBM byte count measured with rocprofv3
counters for this kernel source (null when the source changed since).
``cpu_baseline`` is the float64 CPU oracle timed on this host's cores over
whole passes of the same workload. ``extra`` holds the long causal prefill
(TFLOP/s against the dense bf16 MFMA peak) and the long-context decode.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
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


class Case:
    """Device copies of a problem plus a callable that runs one step."""

    def __init__(self, p, copies: int):
        import torch
        from paged_flashattention_kv_amd import native
        from paged_flashattention_kv_amd.workloads import PagedProblem  # noqa: F401

        self.p = p
        dev = "cuda:0"

        def bf(a):
            import numpy as np
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        self.q = bf(p.query)
        k = bf(p.key_pages)
        v = bf(p.value_pages)
        self.pools = [(k, v)] + [(k.clone(), v.clone()) for _ in range(copies - 1)]
        self.bt = torch.from_numpy(p.block_table).to(dev)
        self.ctx = torch.from_numpy(p.context_lens).to(dev)
        self.out = torch.empty_like(self.q)
        need = native.workspace_bytes(p.batch, p.num_q_heads, p.num_kv_heads, p.query_len, p.head_dim,
                                      p.page_size, p.max_pages)
        self.ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
        self.schedule = native.schedule_for(p.batch, p.num_q_heads, p.num_kv_heads, p.query_len, p.head_dim,
                                            p.page_size, p.max_pages)
        self.i = 0
        self._native = native

    def step(self):
        k, v = self.pools[self.i % len(self.pools)]
        self.i += 1
        self._native.paged_attention(self.q, k, v, self.bt, self.ctx, self.p.page_size, self.p.scale, self.p.causal,
                                     out=self.out, workspace=self.ws)

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

        def bf(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        shape = (p.batch, p.num_kv_heads, new_len, p.head_dim)
        kn = bf(wl.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32)))
        vn = bf(wl.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32)))
        # sources rotated so that repeats are not served by the Infinity Cache
        self.src = [(kn, vn)] + [(kn.clone(), vn.clone()) for _ in range(copies - 1)]
        self.k = bf(p.key_pages)
        self.v = bf(p.value_pages)
        self.bt = torch.from_numpy(p.block_table).to(dev)
        self.ctx = torch.from_numpy(p.context_lens).to(dev)
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
        import numpy as np
        import torch
        from paged_flashattention_kv_amd import native

        dev = "cuda:0"

        def bf(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        self.p = p
        self.q = bf(p.query)
        k = bf(p.key_pages)
        v = bf(p.value_pages)
        self.pools = [(k, v)] + [(k.clone(), v.clone()) for _ in range(copies - 1)]
        self.bt = torch.from_numpy(p.block_table).to(dev)
        self.ctx = torch.from_numpy(p.context_lens).to(dev)
        self.qs = torch.from_numpy(p.query_start).to(dev)
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
        B, Hq, L = p.batch, p.num_q_heads, p.query_len
        per_key = (mshape[1] if mshape[1] > 1 else 1) * (mshape[2] if mshape[2] > 1 else 1)
        self.mask_bytes = 4 * per_key * int(p.context_lens.astype(np.int64).sum()) if mshape[0] > 1 else None

    def step(self):
        k, v = self.pools[self.i % len(self.pools)]
        self.i += 1
        self._native.paged_attention_masked(self.q, k, v, self.bt, self.ctx, self.mask, self.p.page_size,
                                            self.p.scale, self.p.causal, out=self.out, workspace=self.ws)


def mixed_roofline_us(p) -> dict:
    """Lower bound of one mixed-batch call on this chip: the decode part's K/V bytes at HBM peak plus the
    prefill part's flops at the bf16 matrix peak (the two launches run one after the other)."""
    import numpy as np

    ql = p.query_lens
    group = p.num_q_heads // p.num_kv_heads
    if group * p.max_query_len <= 8:
        dec_max = p.max_query_len
    else:
        dec_max = 1 if group <= 8 else 0
    dec = (ql >= 1) & (ql <= dec_max)
    pre = ql > dec_max
    ctx = p.context_lens.astype(np.int64)
    dec_bytes = int(ctx[dec].sum()) * p.num_kv_heads * p.head_dim * 4
    pre_pairs = 0
    for L, c in zip(ql[pre].tolist(), ctx[pre].tolist()):
        pre_pairs += L * (c - L) + L * (L + 1) // 2 if p.causal else L * c
    pre_flops = 4 * p.head_dim * p.num_q_heads * pre_pairs
    t = dec_bytes / (HBM_PEAK_GBPS * 1e9) + pre_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    return {"decode_kv_bytes": dec_bytes, "prefill_flops": pre_flops, "bound_us": round(t * 1e6, 3)}


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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--prewarm-seconds", type=float, default=PREWARM_SECONDS,
                    help="untimed sustained load before each case's warmup calls (the engine clock settles)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one 1 GiB device copy (reference for counter scaling)")
    args = ap.parse_args()
    globals()["PREWARM_SECONDS"] = max(0.0, args.prewarm_seconds)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this operator build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from paged_flashattention_kv_amd import native, workloads as wl

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

    # ---- headline: decode batch ----
    p = wl.make_config("decode_batch")
    case = Case(p, POOL_COPIES)
    ms, wall_ms = case.time(args.steps, args.warmup)
    kv = p.kv_bytes()
    tbps = kv / (ms * 1e-3) / 1e12
    achieved_gbps = kv / (ms * 1e-3) / 1e9
    traffic = measured_traffic("pa_decode_work", "decode_batch")
    result = {
        "metric": METRIC,
        "value": round(tbps, 4),
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
            "wall_ms_per_step": round(wall_ms, 5),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": "pa_decode_work",
            "algorithmic_bytes_per_launch": kv,
        },
    }
    del case
    torch.cuda.empty_cache()

    if not args.no_extra:
        extra = {}
        pp = wl.make_config("long_prefill")
        c3 = Case(pp, 1)
        ms3, _ = c3.time(max(20, args.steps // 4), max(5, args.warmup // 4))
        tf = pp.flops() / (ms3 * 1e-3) / 1e12
        extra["long_prefill"] = {
            "workload": "B=4 L=ctx=2048 H_q=32 H_kv=8 D=128 causal, page_size=128 shuffled",
            "ms_per_step": round(ms3, 5), "value": round(tf, 2), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("pa_prefill_mfma", "long_prefill"),
                         "kernel": "pa_prefill_mfma", "algorithmic_flops_per_launch": pp.flops()},
        }
        del c3
        torch.cuda.empty_cache()
        pc = wl.make_config("chunked_continuation")
        c4 = Case(pc, POOL_COPIES)
        ms4, _ = c4.time(max(20, args.steps // 4), max(5, args.warmup // 4))
        extra["chunked_continuation"] = {
            "workload": "B=8 L=65 history U[1000,3600] (seed 4) H_q=32 H_kv=8 D=128 causal, page_size=128",
            "ms_per_step": round(ms4, 5),
            "tflops": round(pc.flops() / (ms4 * 1e-3) / 1e12, 2),
            "kv_tbps": round(pc.kv_bytes() / (ms4 * 1e-3) / 1e12, 4),
        }
        del c4
        torch.cuda.empty_cache()
        pl = wl.make_config("long_decode")
        c5 = Case(pl, 1)  # 2 GiB per step already exceeds the Infinity Cache
        ms5, _ = c5.time(max(10, args.steps // 10), max(3, args.warmup // 10))
        g5 = pl.kv_bytes() / (ms5 * 1e-3) / 1e9
        extra["long_decode"] = {
            "workload": "B=16 L=1 ctx=32768 H_q=32 H_kv=8 D=128, page_size=16 shuffled over 32768 pages",
            "ms_per_step": round(ms5, 5), "value": round(g5 / 1e3, 4), "unit": "TB/s",
            "roofline": {"bound": "hbm", "achieved": round(g5, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(g5 / HBM_PEAK_GBPS, 4),
                         "traffic": measured_traffic("pa_decode_work", "long_decode"),
                         "kernel": "pa_decode_work", "algorithmic_bytes_per_launch": pl.kv_bytes()},
        }
        del c5
        torch.cuda.empty_cache()
        for name, cfg, new_len, copies in (("kv_append_prefill", "long_prefill", 2048, 8),
                                           ("kv_append_decode", "decode_batch", 1, 8)):
            pa = wl.make_config(cfg)
            ca = AppendCase(pa, new_len, copies)
            msa, _ = ca.time(max(20, args.steps // 4), max(5, args.warmup // 4))
            ga = ca.bytes / (msa * 1e-3) / 1e9
            extra[name] = {
                "workload": f"append {new_len} new token(s) per sequence into the {cfg} pools "
                            f"(B={pa.batch} H_kv={pa.num_kv_heads} D=128, page_size={pa.page_size})",
                "ms_per_step": round(msa, 5), "value": round(ga / 1e3, 4), "unit": "TB/s",
                "roofline": {"bound": "hbm", "achieved": round(ga, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": round(ga / HBM_PEAK_GBPS, 4),
                             "traffic": measured_traffic("pa_kv_append", name), "kernel": "pa_kv_append",
                             "algorithmic_bytes_per_launch": ca.bytes},
            }
            del ca
            torch.cuda.empty_cache()
        pdm = wl.make_config("decode_batch")
        cdm = MaskedCase(pdm, POOL_COPIES, (64, 32, 1, 4096))
        msd, _ = cdm.time(max(20, args.steps // 4), max(5, args.warmup // 4))
        byt = pdm.kv_bytes() + cdm.mask_bytes
        gd = byt / (msd * 1e-3) / 1e9
        extra["masked_decode"] = {
            "workload": "decode_batch with an explicit fp32 mask [64, 32, 1, 4096] (N(0,1) log-weights, 10% -inf)",
            "ms_per_step": round(msd, 5), "value": round(gd / 1e3, 4), "unit": "TB/s",
            "roofline": {"bound": "hbm", "achieved": round(gd, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gd / HBM_PEAK_GBPS, 4), "traffic": None, "kernel": "pa_decode_work (masked)",
                         "algorithmic_bytes_per_launch": byt, "mask_bytes": cdm.mask_bytes},
        }
        del cdm
        torch.cuda.empty_cache()
        ppm = wl.make_config("long_prefill")
        cpm = MaskedCase(ppm, POOL_COPIES, (4, 1, 2048, 2048))
        msp, _ = cpm.time(max(20, args.steps // 4), max(5, args.warmup // 4))
        tfm = ppm.flops() / (msp * 1e-3) / 1e12
        extra["masked_prefill"] = {
            "workload": "long_prefill with an explicit fp32 mask [4, 1, 2048, 2048] shared by the heads",
            "ms_per_step": round(msp, 5), "value": round(tfm, 2), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(tfm, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tfm / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                         "kernel": "pa_prefill_mfma (masked)", "algorithmic_flops_per_launch": ppm.flops()},
        }
        del cpm
        torch.cuda.empty_cache()
        pm = wl.make_varlen_config("mixed_batch")
        cm = VarlenCase(pm, 8)
        msm, _ = cm.time(max(20, args.steps // 2), max(5, args.warmup // 2))
        rl = mixed_roofline_us(pm)
        extra["mixed_batch"] = {
            "workload": f"mixed_batch: B={pm.batch}, {int((pm.query_lens > 1).sum())} prefill chunks (<=128 tokens) "
                        f"+ {int((pm.query_lens == 1).sum())} one-token decodes, T={pm.total_query} H_q=32 H_kv=8 "
                        f"D=128, prompts U[128,1024] outputs U[32,128] (seed 6), page_size=128 shuffled",
            "ms_per_step": round(msm, 5),
            "tokens_per_s": round(pm.total_query / (msm * 1e-3), 1),
            "kv_tbps": round(pm.kv_bytes() / (msm * 1e-3) / 1e12, 4),
            "tflops": round(pm.flops() / (msm * 1e-3) / 1e12, 2),
            "roofline": {"bound": "hbm+mfma", "bound_us": rl["bound_us"], "achieved_us": round(msm * 1e3, 2),
                         "frac": round(rl["bound_us"] / (msm * 1e3), 4), "decode_kv_bytes": rl["decode_kv_bytes"],
                         "prefill_flops": rl["prefill_flops"], "kernels": ["pa_decode_work", "pa_prefill_mfma"]},
        }
        del cm
        torch.cuda.empty_cache()
        result["extra"] = extra

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
