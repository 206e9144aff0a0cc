"""Pins for the oracle's attention (CPU only).

PagedAttention computes plain softmax attention over the gathered context
(Colossal-Inference release post, section "分页注意力算法 (PagedAttention)";
LLM inference optimisation overview, section 2.1.2); GQA shares each KV head
among a group of query heads (same overview, section 2.2.2); split-KV relies
on reducing softmax without the whole input at once (section 2.2.1).

Pins used: a hand-worked case, closed forms, torch's scaled_dot_product_attention
in float64 on repeated KV heads (a library routine), 50-digit brute force with
mpmath, and invariants.
"""
import math
import os

import mpmath
import numpy as np
import pytest
import torch

from conftest import GOLDEN
from oracle import attend, attend_partitioned, combine_partials


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa(q, k, v, scale, mask=None):
    """torch SDPA (float64, CPU) on KV heads repeated over each query group."""
    nq, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]  # [1, Hq, nq, D]
    kt = torch.from_numpy(np.repeat(k, g, axis=1)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.repeat(v, g, axis=1)).permute(1, 0, 2)[None]
    am = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def test_hand_worked_case():
    rows = {"q": [], "k": [], "v": [], "o": []}
    with open(os.path.join(GOLDEN, "attention_hand.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            tag, *vals = line.split()
            rows[tag].append([float(x) for x in vals])
    q = np.array(rows["q"])[:, None, :]
    k = np.array(rows["k"])[:, None, :]
    v = np.array(rows["v"])[:, None, :]
    o = attend(q, k, v, scale=1.0)
    np.testing.assert_allclose(o[0, 0], rows["o"][0], rtol=0, atol=1e-14)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (8, 8), (8, 1), (32, 8), (64, 8)])
@pytest.mark.parametrize("L", [1, 2, 17, 100])
def test_matches_library_sdpa(hq, hkv, L):
    rng = np.random.default_rng(hq * 1000 + hkv * 10 + L)
    d = 16
    q = _rand(rng, 1, hq, d)
    k = _rand(rng, L, hkv, d)
    v = _rand(rng, L, hkv, d)
    scale = 1 / math.sqrt(d)
    np.testing.assert_allclose(attend(q, k, v, scale), _sdpa(q, k, v, scale), rtol=0, atol=1e-12)


def test_causal_varlen_mask_matches_sdpa_with_end_aligned_mask():
    rng = np.random.default_rng(7)
    n, L, hq, hkv, d = 5, 12, 4, 2, 8
    q = _rand(rng, n, hq, d)
    k = _rand(rng, L, hkv, d)
    v = _rand(rng, L, hkv, d)
    pos = L - n + np.arange(n)
    mask = np.arange(L)[None, :] <= pos[:, None]  # query i sees keys 0..L-n+i
    np.testing.assert_allclose(attend(q, k, v, 0.3, pos), _sdpa(q, k, v, 0.3, mask), rtol=0, atol=1e-12)
    # the last query of the chunk sees the whole context: same as decode
    np.testing.assert_array_equal(attend(q[-1:], k, v, 0.3, pos[-1:]), attend(q[-1:], k, v, 0.3))


def test_single_token_returns_its_value_row_exactly():
    rng = np.random.default_rng(1)
    q = _rand(rng, 1, 4, 8)
    k = _rand(rng, 1, 2, 8)
    v = _rand(rng, 1, 2, 8)
    o = attend(q, k, v, 0.125)
    for h in range(4):
        assert np.array_equal(o[0, h], v[0, h // 2])


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    L = 37
    q = _rand(rng, 1, 2, 8)
    k = np.repeat(_rand(rng, 1, 1, 8), L, axis=0)
    v = _rand(rng, L, 1, 8)
    o = attend(q, k, v, 0.5)
    np.testing.assert_allclose(o[0, 0], v[:, 0].mean(axis=0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0, 1], v[:, 0].mean(axis=0), rtol=0, atol=1e-14)


def test_two_tokens_closed_form():
    rng = np.random.default_rng(3)
    q = _rand(rng, 1, 1, 6)
    k = _rand(rng, 2, 1, 6)
    v = _rand(rng, 2, 1, 6)
    sc = 0.7
    s0 = sc * q[0, 0] @ k[0, 0]
    s1 = sc * q[0, 0] @ k[1, 0]
    sig = 1 / (1 + math.exp(-(s1 - s0)))
    np.testing.assert_allclose(attend(q, k, v, sc)[0, 0], v[0, 0] + sig * (v[1, 0] - v[0, 0]), atol=1e-14)


def test_gqa_special_cases():
    rng = np.random.default_rng(4)
    L, d = 20, 8
    q = _rand(rng, 1, 8, d)
    k1 = _rand(rng, L, 1, d)
    v1 = _rand(rng, L, 1, d)
    # one group (MQA): every query head reads the single KV head
    o = attend(q, k1, v1, 0.3)
    for h in range(8):
        np.testing.assert_array_equal(o[0, h], attend(q[:, h : h + 1], k1, v1, 0.3)[0, 0])
    # GQA == MHA with each KV head repeated over its group
    k2 = _rand(rng, L, 2, d)
    v2 = _rand(rng, L, 2, d)
    np.testing.assert_allclose(attend(q, k2, v2, 0.3), attend(q, np.repeat(k2, 4, 1), np.repeat(v2, 4, 1), 0.3),
                               rtol=0, atol=1e-15)
    # heads 0-3 use KV head 0, heads 4-7 KV head 1 (contiguous grouping)
    np.testing.assert_array_equal(attend(q[:, :4], k2[:, :1], v2[:, :1], 0.3), attend(q, k2, v2, 0.3)[:, :4])


def test_affine_in_values_and_token_order_invariance():
    rng = np.random.default_rng(5)
    L = 33
    q = _rand(rng, 1, 4, 8)
    k = _rand(rng, L, 2, 8)
    v = _rand(rng, L, 2, 8)
    o = attend(q, k, v, 0.35)
    np.testing.assert_allclose(attend(q, k, 2.5 * v - 1.0, 0.35), 2.5 * o - 1.0, atol=1e-13)
    p = rng.permutation(L)
    np.testing.assert_allclose(attend(q, k[p], v[p], 0.35), o, atol=1e-14)


def test_empty_context_gives_zeros():
    q = np.ones((1, 2, 4))
    o = attend(q, np.zeros((0, 1, 4)), np.zeros((0, 1, 4)), 1.0)
    assert np.array_equal(o, np.zeros((1, 2, 4)))


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_50_digits(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(1, 6))
    d = int(rng.integers(1, 5))
    hkv = int(rng.integers(1, 3))
    hq = hkv * int(rng.integers(1, 3))
    q = _rand(rng, 1, hq, d)
    k = _rand(rng, L, hkv, d)
    v = _rand(rng, L, hkv, d)
    sc = float(rng.uniform(0.1, 2.0))
    got = attend(q, k, v, sc)
    mpmath.mp.dps = 50
    g = hq // hkv
    for h in range(hq):
        kh = h // g
        s = [mpmath.mpf(sc) * mpmath.fsum(mpmath.mpf(q[0, h, i]) * mpmath.mpf(k[t, kh, i]) for i in range(d))
             for t in range(L)]
        e = [mpmath.exp(x) for x in s]  # no max shift: exact arithmetic does not need it
        z = mpmath.fsum(e)
        for i in range(d):
            want = mpmath.fsum(e[t] * mpmath.mpf(v[t, kh, i]) for t in range(L)) / z
            assert abs(float(want) - got[0, h, i]) <= 1e-14 * max(1.0, abs(float(want)))


@pytest.mark.parametrize("part", [1, 5, 16, 512])
def test_partitioned_softmax_recombines_to_full(part):
    rng = np.random.default_rng(part)
    L = 100
    q = _rand(rng, 3, 4, 8)
    k = 3 * _rand(rng, L, 2, 8)
    v = _rand(rng, L, 2, 8)
    pos = np.array([L - 1, 40, 0])
    m, l, o = attend_partitioned(q, k, v, 0.4, part, pos)
    np.testing.assert_allclose(combine_partials(m, l, o), attend(q, k, v, 0.4, pos), rtol=0, atol=1e-13)
    # one partition reproduces the unsplit state exactly up to rounding
    m1, l1, o1 = attend_partitioned(q[:1], k, v, 0.4, L)
    np.testing.assert_allclose(o1[0], attend(q[:1], k, v, 0.4), atol=1e-15)
