"""Shared helpers for the tests: moving a seeded problem to the GPU, running
the operator through the C ABI binding, and the parity bar."""

from __future__ import annotations

import sys

import numpy as np

# spec tolerance for bf16 outputs against the float64 oracle
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def to_device(p, device="cuda:0"):
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    return dict(
        query=bf(p.query),
        key_pages=bf(p.key_pages),
        value_pages=bf(p.value_pages),
        block_table=torch.from_numpy(np.ascontiguousarray(p.block_table)).to(device),
        context_lens=torch.from_numpy(np.ascontiguousarray(p.context_lens)).to(device),
    )


def run_gpu(p, schedule=0, decode_work_items=0, dev=None, out=None):
    """Run the operator on problem ``p``; return float64 numpy [B, H_q, L, D]."""
    import torch
    from paged_flashattention_kv_amd import native

    d = dev if dev is not None else to_device(p)
    o = native.paged_attention(
        d["query"], d["key_pages"], d["value_pages"], d["block_table"], d["context_lens"],
        p.page_size, p.scale, p.causal, schedule=schedule, decode_work_items=decode_work_items, out=out,
    )
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64)


def parity(got, want, label=""):
    """Assert the bf16 output matches the float64 oracle within the bar."""
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    err = np.abs(got - want)
    mx, mean = float(err.max()), float(err.mean())
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    say(f"  parity {label}: max_abs={mx:.3e} mean_abs={mean:.3e} rel_l2={rel:.3e}")
    assert mx <= MAX_ABS, f"{label}: max abs error {mx} > {MAX_ABS}"
    assert mean <= MEAN_ABS, f"{label}: mean abs error {mean} > {MEAN_ABS}"
    return mx, mean, rel
