"""Pins for the explicit-mask oracle (no GPU).

``oracle.paged_attention_masked_ref`` adds an explicit additive mask to the
scaled scores beside the causal flag. It is tied to:

- brute force: ``oracle.paged_attention_masked_brute`` (scalar loops written
  separately) on random masks with -inf entries and broadcast axes;
- a library special case: torch's float64 scaled-dot-product attention with
  an additive ``attn_mask`` over the gathered history;
- closed forms: with all keys zero and mask = log(w) with integer weights,
  every row is sum(w V) / sum(w), summed exactly in integers here; a zero
  mask leaves the unmasked oracle unchanged;
- invariants: adding one constant to a whole mask row changes nothing; a
  -inf suffix (or a mask shorter than the context) equals a shorter context;
  a row with every key masked is NaN and leaves the other rows alone;
- a planted mistake (in the oracle): scaling the mask with the scores fails
  the closed form.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import masked as masked_mod
from paged_flashattention_kv_amd import workloads as wl

D = 16


def _p(seed, B=2, Hq=4, Hkv=2, L=3, ps=4, ctx=(7, 11), causal=True):
    return wl.make_problem(seed=seed, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, query_len=L, head_dim=D,
                           page_size=ps, context_lens=list(ctx), causal=causal, poison=True)


def _mref(p, m):
    return oracle.paged_attention_masked_ref(p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens, m,
                                             p.page_size, p.scale, p.causal)


def _rand_mask(seed, shape, frac_inf=0.2):
    rng = np.random.Generator(np.random.PCG64(seed))
    m = rng.normal(0.0, 2.0, size=shape)
    m[rng.random(shape) < frac_inf] = -np.inf
    return m


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("mshape", [(2, 4, 3, 11), (1, 4, 1, 11), (2, 1, 3, 12), (1, 1, 1, 9)])
def test_matches_brute_force(causal, mshape):
    p = _p(3, causal=causal)
    m = _rand_mask(7, mshape)
    # keep at least key 0 usable in every row so no row is empty
    m[..., 0] = 0.0
    got = _mref(p, m)
    want = oracle.paged_attention_masked_brute(p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens, m,
                                              p.page_size, p.scale, causal)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_zero_mask_is_the_unmasked_oracle():
    for causal in (True, False):
        p = _p(5, causal=causal)
        got = _mref(p, np.zeros((1, 1, 1, 11)))
        want = oracle.paged_attention_ref(p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens,
                                          p.page_size, p.scale, causal)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def test_torch_sdpa_with_additive_mask():
    p = _p(9, causal=False, ctx=(11, 11))
    m = _rand_mask(10, (2, 4, 3, 11), frac_inf=0.1)
    m[..., 3] = 0.0
    got = _mref(p, m)
    for b in range(2):
        K = oracle.gather_history(p.key_pages, p.block_table[b], 11, p.page_size)  # [H_kv, S, D]
        V = oracle.gather_history(p.value_pages, p.block_table[b], 11, p.page_size)
        q = torch.from_numpy(oracle.bf16_bits_to_f64(p.query[b]))  # [H_q, L, D]
        k = torch.from_numpy(np.repeat(K, 2, axis=0))
        v = torch.from_numpy(np.repeat(V, 2, axis=0))
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=torch.from_numpy(m[b]),
                                                               scale=float(np.float32(p.scale)))
        np.testing.assert_allclose(got[b], ref.numpy(), rtol=1e-12, atol=1e-12)


def _zero_key_weighted(causal):
    """K = 0, V = small integers, mask = log(w) with integer weights w in 1..5 (and -inf where w = 0)."""
    p = _p(11, causal=causal, ctx=(9, 6))
    k = p.key_pages.copy()
    v = p.value_pages.copy()
    vals = {}
    for b in range(p.batch):
        for s in range(int(p.context_lens[b])):
            page, slot = p.block_table[b, s // p.page_size], s % p.page_size
            k[page, :, slot, :] = 0
            for g in range(2):
                row = np.array([((5 * s + 2 * g + d) % 9) - 4 for d in range(D)], dtype=np.float32)
                v[page, g, slot, :] = wl.f32_to_bf16_bits(row)
                vals[(b, g, s)] = row.astype(np.int64)
    p.key_pages, p.value_pages = k, v
    rng = np.random.Generator(np.random.PCG64(12))
    w = rng.integers(0, 6, size=(2, 4, 3, 9))
    w[..., 0] = 1
    with np.errstate(divide="ignore"):
        m = np.log(w.astype(np.float64))
    want = np.zeros((2, 4, 3, D))
    for b in range(2):
        c = int(p.context_lens[b])
        for h in range(4):
            for l in range(3):
                last = c - 3 + l if causal else c - 1
                num = sum(int(w[b, h, l, s]) * vals[(b, h // 2, s)] for s in range(last + 1))
                den = sum(int(w[b, h, l, s]) for s in range(last + 1))
                want[b, h, l] = num / den
    return p, m, want


@pytest.mark.parametrize("causal", [True, False])
def test_log_weights_give_the_weighted_mean(causal):
    p, m, want = _zero_key_weighted(causal)
    np.testing.assert_allclose(_mref(p, m), want, rtol=0, atol=1e-12)


def test_planted_scaled_mask_is_caught(monkeypatch):
    p, m, want = _zero_key_weighted(True)
    monkeypatch.setattr(masked_mod, "_scores", lambda q, K, madd, sc: sc * (q @ K.T + madd))
    assert not np.allclose(_mref(p, m), want, atol=1e-6)


def test_row_constant_shift_changes_nothing():
    p = _p(13)
    m = _rand_mask(14, (2, 4, 3, 11))
    m[..., 0] = 0.0
    shift = np.random.Generator(np.random.PCG64(15)).normal(0, 50, size=(2, 4, 3, 1))
    np.testing.assert_allclose(_mref(p, m + shift), _mref(p, m), rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("short_axis", [False, True])
def test_masked_suffix_equals_shorter_context(short_axis):
    p = _p(17, causal=False, ctx=(10, 10))
    cut = 6
    if short_axis:
        m = np.zeros((1, 1, 1, cut))  # keys at or past the mask's last axis are absent
    else:
        m = np.zeros((1, 1, 1, 10))
        m[..., cut:] = -np.inf
    short = oracle.paged_attention_ref(p.query, p.key_pages, p.value_pages, p.block_table,
                                       np.array([cut, cut], dtype=np.int32), p.page_size, p.scale, False)
    np.testing.assert_allclose(_mref(p, m), short, rtol=0, atol=1e-14)


def test_fully_masked_row_is_nan_and_isolated():
    p = _p(19)
    m = np.zeros((2, 4, 3, 11))
    m[1, 2, 0, :] = -np.inf
    got = _mref(p, m)
    assert np.isnan(got[1, 2, 0]).all()
    ok = np.ones(got.shape[:3], dtype=bool)
    ok[1, 2, 0] = False
    assert np.isfinite(got[ok]).all()
    base = _mref(p, np.zeros((1, 1, 1, 11)))
    np.testing.assert_array_equal(got[ok], base[ok])
    brute = oracle.paged_attention_masked_brute(p.query, p.key_pages, p.value_pages, p.block_table, p.context_lens,
                                                m, p.page_size, p.scale, True)
    assert np.isnan(brute[1, 2, 0]).all() and math.isfinite(brute[0, 0, 0, 0])
