"""Pins for the oracle's fp64 decode attention.

Attention here is the plain definition (page "Open Weights: from files to tokens /
second", section "03 / The inference loop"): one query token per sequence, scaled dot products with
every cached token of its sequence reached through the page table, softmax, weighted sum of V;
grouped-query heads share one KV head.  The pins are closed forms (one token, zero query,
equal keys, a dominating logit, a two-token weight), a brute-force computation with library
primitives (matmul + scipy softmax) on tiny inputs, the grouped-query head mapping, and
invariance under any physical page permutation.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth


def bits(x):
    """float -> bf16 bits (values used here are exact in bf16)."""
    a = np.asarray(x, np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def f(b):
    return synth.bf16_to_f32(b).astype(np.float64)


def make_cache(rng, B, H, D, T, lens, extra_pages=3):
    npages = sum(-(-int(L) // T) for L in lens) + extra_pages
    perm = rng.permutation(npages).astype(np.int32)
    maxp = max(1, max(-(-int(L) // T) for L in lens))
    pt = np.full((B, maxp), -1, np.int32)
    nxt = 0
    for b, L in enumerate(lens):
        n = -(-int(L) // T)
        pt[b, :n] = perm[nxt:nxt + n]
        nxt += n
    vals = rng.standard_normal((npages, H, 2, T, D)).astype(np.float32)
    return pt, bits(vals), npages


def gather(raw, pt, b, L, h, kv, T):
    return np.stack([f(raw[pt[b, t // T], h, kv, t % T]) for t in range(L)]) if L else np.zeros((0, raw.shape[-1]))


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(0)
    B, H, D, T = 2, 2, 64, 16
    lens = np.array([1, 1], np.int32)
    pt, raw, _ = make_cache(rng, B, H, D, T, lens)
    q = bits(rng.standard_normal((B, 4, D)))
    st, out = oracle.attention(raw, lens, pt, q)
    assert st == 0
    for b in range(B):
        for hq in range(4):
            assert np.array_equal(out[b, hq], f(raw[pt[b, 0], hq // 2, 1, 0]))


def test_zero_query_or_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(1)
    B, H, D, T = 1, 1, 64, 16
    lens = np.array([37], np.int32)
    pt, raw, _ = make_cache(rng, B, H, D, T, lens)
    q = np.zeros((B, 2, D), np.uint16)
    _, out = oracle.attention(raw, lens, pt, q)
    V = gather(raw, pt, 0, 37, 0, 1, T)
    np.testing.assert_allclose(out[0, 0], V.mean(0), rtol=1e-13, atol=1e-13)
    raw2 = raw.copy()
    for t in range(37):
        raw2[pt[0, t // T], 0, 0, t % T] = raw[pt[0, 0], 0, 0, 0]
    q = bits(rng.standard_normal((B, 2, D)))
    _, out = oracle.attention(raw2, lens, pt, q)
    np.testing.assert_allclose(out[0, 1], V.mean(0), rtol=1e-13, atol=1e-13)


def test_dominating_logit_selects_its_value():
    rng = np.random.default_rng(2)
    B, H, D, T = 1, 1, 64, 16
    lens = np.array([40], np.int32)
    pt, raw, _ = make_cache(rng, B, H, D, T, lens)
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 5] = 1.0
    hot = 23
    raw[pt[0, hot // T], 0, 0, hot % T, 5] = bits(2.0 ** 14)  # logit 16384/8 = 2048 above others
    _, out = oracle.attention(raw, lens, pt, bits(q))
    assert np.array_equal(out[0, 0], f(raw[pt[0, hot // T], 0, 1, hot % T]))


def test_two_token_closed_form_pins_the_scale():
    """out = (v0 + e^d v1) / (1 + e^d) with d = (q.k1 - q.k0) / sqrt(D)."""
    D, T = 128, 16
    pt = np.array([[0]], np.int32)
    raw = np.zeros((1, 1, 2, T, D), np.uint16)
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, :4] = [1.0, 2.0, -1.0, 0.5]
    raw[0, 0, 0, 0, :4] = bits([0.5, 0.25, 0.0, 1.0])   # q.k0 = 0.5+0.5+0+0.5 = 1.5
    raw[0, 0, 0, 1, :4] = bits([2.0, 1.0, -1.0, 2.0])   # q.k1 = 2+2+1+1 = 6
    raw[0, 0, 1, 0, :3] = bits([1.0, -2.0, 4.0])
    raw[0, 0, 1, 1, :3] = bits([3.0, 0.5, -8.0])
    _, out = oracle.attention(raw, np.array([2], np.int32), pt, bits(q))
    d = (6.0 - 1.5) / math.sqrt(128.0)
    w1 = math.exp(d) / (1.0 + math.exp(d))
    expect = (1 - w1) * np.array([1.0, -2.0, 4.0]) + w1 * np.array([3.0, 0.5, -8.0])
    np.testing.assert_allclose(out[0, 0, :3], expect, rtol=1e-14)
    assert not out[0, 0, 3:].any()


def test_empty_sequence_gives_zeros():
    rng = np.random.default_rng(3)
    lens = np.array([0, 5], np.int32)
    pt, raw, _ = make_cache(rng, 2, 1, 64, 16, [1, 5])
    _, out = oracle.attention(raw, lens, pt, bits(rng.standard_normal((2, 1, 64))))
    assert not out[0].any() and out[1].any()


@pytest.mark.parametrize("seed", [4, 5, 6])
def test_brute_force_against_library_softmax(seed):
    rng = np.random.default_rng(seed)
    B, H, G, D, T = 3, 2, 3, 64, 16
    lens = rng.integers(1, 70, B).astype(np.int32)
    pt, raw, _ = make_cache(rng, B, H, D, T, lens)
    q = bits(rng.standard_normal((B, H * G, D)) * 2)
    _, out = oracle.attention(raw, lens, pt, q)
    for b in range(B):
        for hq in range(H * G):
            K = gather(raw, pt, b, int(lens[b]), hq // G, 0, T)
            V = gather(raw, pt, b, int(lens[b]), hq // G, 1, T)
            p = softmax(K @ f(q[b, hq]) / math.sqrt(D))
            np.testing.assert_allclose(out[b, hq], p @ V, rtol=1e-12, atol=1e-12)


def test_grouped_query_heads_share_their_kv_head():
    """V of kv head g set to the constant g+1: every q head of group g must return g+1."""
    rng = np.random.default_rng(7)
    B, H, G, D, T = 2, 4, 4, 64, 16
    lens = np.array([19, 33], np.int32)
    pt, raw, _ = make_cache(rng, B, H, D, T, lens)
    for g in range(H):
        raw[:, g, 1] = bits(float(g + 1))
    _, out = oracle.attention(raw, lens, pt, bits(rng.standard_normal((B, H * G, D))))
    for hq in range(H * G):
        np.testing.assert_allclose(out[:, hq], hq // G + 1, rtol=1e-14)


def test_physical_page_permutation_is_invisible():
    rng = np.random.default_rng(8)
    B, H, D, T = 2, 2, 64, 16
    lens = np.array([50, 29], np.int32)
    pt, raw, npages = make_cache(rng, B, H, D, T, lens)
    q = bits(rng.standard_normal((B, 8, D)))
    _, out = oracle.attention(raw, lens, pt, q)
    perm = rng.permutation(npages)
    raw2 = np.empty_like(raw)
    raw2[perm] = raw
    pt2 = np.where(pt >= 0, perm[np.maximum(pt, 0)], -1).astype(np.int32)
    _, out2 = oracle.attention(raw2, lens, pt2, q)
    assert np.array_equal(out, out2)


def test_want_mask_computes_only_selected_rows():
    rng = np.random.default_rng(9)
    lens = np.array([20], np.int32)
    pt, raw, _ = make_cache(rng, 1, 2, 64, 16, lens)
    q = bits(rng.standard_normal((1, 4, 64)))
    _, full = oracle.attention(raw, lens, pt, q)
    want = np.array([[0, 1, 0, 1]], np.uint8)
    _, part = oracle.attention(raw, lens, pt, q, want=want)
    assert np.array_equal(part[0, 1], full[0, 1]) and np.array_equal(part[0, 3], full[0, 3])
    assert not part[0, 0].any() and not part[0, 2].any()


def test_effective_token_count_closed_forms():
    """neff = (sum w)^2 / sum w^2: 1 for a dominating logit, L for equal keys, and for two
    tokens with logit gap d, (1 + e^d)^2 / (1 + e^(2d))."""
    rng = np.random.default_rng(10)
    D, T = 64, 16
    lens = np.array([37, 40], np.int32)
    pt, raw, _ = make_cache(rng, 2, 1, D, T, lens)
    for t in range(37):  # sequence 0: every key equal
        raw[pt[0, t // T], 0, 0, t % T] = raw[pt[0, 0], 0, 0, 0]
    hot = 23             # sequence 1: one key 2048 logits above the rest on dim 5
    raw[pt[1, hot // T], 0, 0, hot % T, :] = 0
    raw[pt[1, hot // T], 0, 0, hot % T, 5] = bits(2.0 ** 14)
    q = bits(rng.standard_normal((2, 1, D)))
    q[1, 0, :] = 0
    q[1, 0, 5] = bits(1.0)
    st, _, neff = oracle.attention(raw, lens, pt, q, with_neff=True)
    assert st == 0
    np.testing.assert_allclose(neff[0, 0], 37.0, rtol=1e-13)
    assert neff[1, 0] == 1.0
    # two tokens: the scale-pinning case above
    pt2 = np.array([[0]], np.int32)
    raw2 = np.zeros((1, 1, 2, T, 128), np.uint16)
    q2 = np.zeros((1, 1, 128), np.float32)
    q2[0, 0, :4] = [1.0, 2.0, -1.0, 0.5]
    raw2[0, 0, 0, 0, :4] = bits([0.5, 0.25, 0.0, 1.0])
    raw2[0, 0, 0, 1, :4] = bits([2.0, 1.0, -1.0, 2.0])
    _, _, n2 = oracle.attention(raw2, np.array([2], np.int32), pt2, bits(q2), with_neff=True)
    d = (6.0 - 1.5) / math.sqrt(128.0)
    np.testing.assert_allclose(n2[0, 0], (1 + math.exp(d)) ** 2 / (1 + math.exp(2 * d)), rtol=1e-14)
    _, _, n0 = oracle.attention(raw, np.array([0, 40], np.int32), pt, q, with_neff=True)
    assert n0[0, 0] == 0.0


def test_threaded_slices_equal_one_call_bit_for_bit():
    rng = np.random.default_rng(11)
    B, H, G, D, T = 5, 2, 4, 64, 16
    lens = rng.integers(0, 90, B).astype(np.int32)
    pt, raw, _ = make_cache(rng, B, H, D, T, np.maximum(lens, 1))
    q = bits(rng.standard_normal((B, H * G, D)))
    _, one, n1 = oracle.attention(raw, lens, pt, q, with_neff=True)
    _, many, n2 = oracle.attention(raw, lens, pt, q, threads=7, with_neff=True)
    assert np.array_equal(one, many) and np.array_equal(n1, n2)
    want = (rng.random((B, H * G)) < 0.5).astype(np.uint8)
    _, part = oracle.attention(raw, lens, pt, q, want=want, threads=3)
    sel = want.astype(bool)
    assert np.array_equal(part[sel], one[sel]) and not part[~sel].any()
