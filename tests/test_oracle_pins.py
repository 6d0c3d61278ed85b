"""Pins for the double-precision oracle, independent of the oracle itself.

Each test ties the oracle to something it does not compute the same way:
brute force without the max shift, closed forms, special cases, invariants of
exact attention and of its tree reduction, the energy-gradient identity, and
the format definitions as implemented by torch's own dtypes.

Sources: exact softmax attention as the glossary page "Attention" describes it
(section on Query/Key/Value); the tree reduction along the sequence axis and its
exactness ("Tree Attention: Topology-aware Decoding for Long-Context Attention
on GPU Clusters", explainer sections 1-3); max subtraction for stability
("Attention in SRAM on Tenstorrent Grayskull", explainer section 3).
"""
import math
import random

import numpy as np
import pytest
import torch

import datagen
import oracle

RNG = np.random.default_rng(12345)


def rand_f32(*shape, scale=1.0):
    return (RNG.standard_normal(shape) * scale).astype(np.float32)


def brute_row(qrow, krows, vrows, scale):
    """Textbook softmax with no max shift, in plain Python floats."""
    s = [scale * math.fsum(float(a) * float(b) for a, b in zip(qrow, k)) for k in krows]
    e = [math.exp(x) for x in s]
    z = math.fsum(e)
    d = len(qrow)
    out = [math.fsum(e[j] * float(vrows[j][c]) for j in range(len(krows))) / z for c in range(d)]
    return np.array(out), math.log(z)


def run(prob):
    out, lse = oracle.attention(prob)
    return out.reshape(prob.B, prob.Hq, prob.Lq, prob.d), lse.reshape(prob.B, prob.Hq, prob.Lq)


# ---------------------------------------------------------------- brute force

def test_bruteforce_mha_noncausal():
    B, H, Lq, L, d = 2, 3, 2, 7, 5
    q, k, v = rand_f32(B, H, Lq, d), rand_f32(B, H, L, d), rand_f32(B, H, L, d)
    prob = oracle.Problem(q, k, v, scale=0.37)
    out, lse = run(prob)
    for b in range(B):
        for h in range(H):
            for i in range(Lq):
                o_ref, lse_ref = brute_row(q[b, h, i], k[b, h], v[b, h], 0.37)
                np.testing.assert_allclose(out[b, h, i], o_ref, rtol=1e-12, atol=1e-14)
                assert abs(lse[b, h, i] - lse_ref) < 1e-12


def test_default_scale_is_inverse_sqrt_d():
    q, k, v = rand_f32(1, 1, 1, 16), rand_f32(1, 1, 9, 16), rand_f32(1, 1, 9, 16)
    out, lse = run(oracle.Problem(q, k, v))
    o_ref, lse_ref = brute_row(q[0, 0, 0], k[0, 0], v[0, 0], 0.25)
    np.testing.assert_allclose(out[0, 0, 0], o_ref, rtol=1e-12, atol=1e-14)
    assert abs(lse[0, 0, 0] - lse_ref) < 1e-12


# ---------------------------------------------------------------- closed forms

def test_two_keys_closed_form():
    # O = logistic(s1 - s2) v1 + logistic(s2 - s1) v2, lse = ln(e^s1 + e^s2)
    q = np.array([[[[1.0, -2.0, 0.5]]]], dtype=np.float32)
    k = np.array([[[[0.5, 0.25, 2.0], [-1.0, 1.0, 0.0]]]], dtype=np.float32)
    v = np.array([[[[1.0, 2.0, 3.0], [-4.0, 0.5, 8.0]]]], dtype=np.float32)
    out, lse = run(oracle.Problem(q, k, v, scale=1.0))
    s1, s2 = 0.5 - 0.5 + 1.0, -1.0 - 2.0
    w1 = 1.0 / (1.0 + math.exp(-(s1 - s2)))
    w2 = 1.0 / (1.0 + math.exp(-(s2 - s1)))
    np.testing.assert_allclose(out[0, 0, 0], w1 * v[0, 0, 0].astype(np.float64) + w2 * v[0, 0, 1].astype(np.float64), rtol=1e-14)
    assert abs(lse[0, 0, 0] - math.log(math.exp(s1) + math.exp(s2))) < 1e-14


def test_single_key_returns_its_value():
    q, k, v = rand_f32(1, 2, 1, 8), rand_f32(1, 2, 1, 8), rand_f32(1, 2, 1, 8)
    out, lse = run(oracle.Problem(q, k, v, scale=0.5))
    for h in range(2):
        np.testing.assert_array_equal(out[0, h, 0], v[0, h, 0].astype(np.float64))
        s0 = 0.5 * float(np.dot(q[0, h, 0].astype(np.float64), k[0, h, 0].astype(np.float64)))
        assert abs(lse[0, h, 0] - s0) < 1e-14


def test_uniform_scores_give_mean_of_v():
    n, d = 37, 6
    v = rand_f32(1, 1, n, d)
    # zero query: every score is 0
    out, lse = run(oracle.Problem(np.zeros((1, 1, 1, d), np.float32), rand_f32(1, 1, n, d), v))
    np.testing.assert_allclose(out[0, 0, 0], v[0, 0].astype(np.float64).mean(axis=0), rtol=1e-13, atol=1e-15)
    assert abs(lse[0, 0, 0] - math.log(n)) < 1e-13
    # all keys equal: every score equals s
    krow = rand_f32(d)
    k = np.broadcast_to(krow, (1, 1, n, d)).copy()
    q = rand_f32(1, 1, 1, d)
    out, lse = run(oracle.Problem(q, k, v, scale=0.3))
    s = 0.3 * float(np.dot(q[0, 0, 0].astype(np.float64), krow.astype(np.float64)))
    np.testing.assert_allclose(out[0, 0, 0], v[0, 0].astype(np.float64).mean(axis=0), rtol=1e-13, atol=1e-15)
    assert abs(lse[0, 0, 0] - (s + math.log(n))) < 1e-12


def test_huge_scores_stay_finite():
    # Scores around 1e4: exp without the max shift overflows; the oracle must not.
    d, n = 4, 9
    q = np.array([[[[100.0, 0.0, 0.0, 0.0]]]], dtype=np.float32)
    k = np.zeros((1, 1, n, d), np.float32)
    k[0, 0, :, 0] = np.arange(n, dtype=np.float32) * 10.0 + 50.0  # scores 5000 .. 13000, spaced by 1000
    v = rand_f32(1, 1, n, d)
    out, lse = run(oracle.Problem(q, k, v, scale=1.0))
    assert np.all(np.isfinite(out)) and np.isfinite(lse).all()
    np.testing.assert_array_equal(out[0, 0, 0], v[0, 0, n - 1].astype(np.float64))
    assert lse[0, 0, 0] == pytest.approx(100.0 * (50.0 + 10.0 * (n - 1)), rel=1e-15)
    # two tied maxima: the mean of their values
    k[0, 0, 3, 0] = k[0, 0, n - 1, 0]
    out, lse = run(oracle.Problem(q, k, v, scale=1.0))
    np.testing.assert_allclose(out[0, 0, 0], 0.5 * (v[0, 0, 3].astype(np.float64) + v[0, 0, n - 1]), rtol=1e-15)
    assert lse[0, 0, 0] == pytest.approx(13000.0 + math.log(2.0), rel=1e-15)


# ---------------------------------------------------------------- invariants

def test_weights_sum_to_one():
    q, k = rand_f32(2, 2, 3, 8, scale=3.0), rand_f32(2, 2, 50, 8, scale=3.0)
    out, _ = run(oracle.Problem(q, k, np.ones((2, 2, 50, 8), np.float32)))
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-13)


def test_linear_in_v():
    q, k = rand_f32(1, 2, 2, 8), rand_f32(1, 2, 20, 8)
    v1, v2 = rand_f32(1, 2, 20, 8), rand_f32(1, 2, 20, 8)
    o1, _ = run(oracle.Problem(q, k, v1))
    o2, _ = run(oracle.Problem(q, k, v2))
    o3, _ = run(oracle.Problem(q, k, (2.0 * v1 - 0.5 * v2).astype(np.float32)))
    # 2 v1 - 0.5 v2 is exact in fp32 for these magnitudes only up to rounding; compare in f64 terms
    v3 = (2.0 * v1 - 0.5 * v2).astype(np.float32).astype(np.float64)
    o3_ref, _ = run(oracle.Problem(q, k, v3.astype(np.float32)))
    np.testing.assert_allclose(o3, o3_ref, rtol=0, atol=0)
    np.testing.assert_allclose(o3, 2.0 * o1 - 0.5 * o2, rtol=0, atol=2e-6)


def test_key_permutation_invariance():
    q, k, v = rand_f32(1, 1, 2, 8), rand_f32(1, 1, 31, 8), rand_f32(1, 1, 31, 8)
    perm = RNG.permutation(31)
    o1, l1 = run(oracle.Problem(q, k, v))
    o2, l2 = run(oracle.Problem(q, k[:, :, perm].copy(), v[:, :, perm].copy()))
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)


def test_gqa_equals_mha_with_repeated_kv():
    B, Hq, Hkv, Lq, L, d = 2, 8, 2, 3, 19, 8
    q, k, v = rand_f32(B, Hq, Lq, d), rand_f32(B, Hkv, L, d), rand_f32(B, Hkv, L, d)
    G = Hq // Hkv
    o1, l1 = run(oracle.Problem(q, k, v))
    o2, l2 = run(oracle.Problem(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    # and a mapping h -> h % Hkv would differ
    o3, _ = run(oracle.Problem(q, np.tile(k, (1, G, 1, 1)), np.tile(v, (1, G, 1, 1))))
    assert not np.allclose(o1, o3)


@pytest.mark.parametrize("Lq,L", [(6, 6), (3, 10), (1, 9)])
def test_causal_row_equals_its_prefix(Lq, L):
    B, H, d = 1, 2, 8
    q, k, v = rand_f32(B, H, Lq, d), rand_f32(B, H, L, d), rand_f32(B, H, L, d)
    out, lse = run(oracle.Problem(q, k, v, causal=True))
    for h in range(H):
        for i in range(Lq):
            n = L - Lq + i + 1  # bottom-right alignment, self included
            o_ref, lse_ref = brute_row(q[0, h, i], k[0, h, :n], v[0, h, :n], 1 / math.sqrt(d))
            np.testing.assert_allclose(out[0, h, i], o_ref, rtol=1e-12, atol=1e-14)
            assert abs(lse[0, h, i] - lse_ref) < 1e-12


def test_ragged_row_equals_sequence_alone():
    B, Hq, Hkv, Lcap, d = 3, 4, 2, 16, 8
    q, k, v = rand_f32(B, Hq, 1, d), rand_f32(B, Hkv, Lcap, d), rand_f32(B, Hkv, Lcap, d)
    lens = np.array([16, 5, 0], np.int32)
    out, lse = run(oracle.Problem(q, k, v, kv_lens=lens, causal=True))
    for b in range(2):
        n = int(lens[b])
        o_ref, l_ref = run(oracle.Problem(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n]))
        np.testing.assert_array_equal(out[b], o_ref[0])
        np.testing.assert_array_equal(lse[b], l_ref[0])
    # an empty sequence: O = 0, lse = -inf
    assert np.all(out[2] == 0.0) and np.all(np.isneginf(lse[2]))


# ---------------------------------------------------------------- tree reduction

def _chunks(n, S):
    bounds = [n * s // S for s in range(S + 1)]
    return list(zip(bounds[:-1], bounds[1:]))


def _reduce(parts, shape, rnd):
    if shape == "left":
        acc = parts[0]
        for p in parts[1:]:
            acc = oracle.merge(acc, p)
        return acc
    if shape == "right":
        acc = parts[-1]
        for p in reversed(parts[:-1]):
            acc = oracle.merge(p, acc)
        return acc
    if shape == "balanced":
        level = list(parts)
        while len(level) > 1:
            nxt = [oracle.merge(level[i], level[i + 1]) for i in range(0, len(level) - 1, 2)]
            if len(level) % 2:
                nxt.append(level[-1])
            level = nxt
        return level[0]
    # random tree: merge random neighbours (any order: merge is commutative too)
    level = list(parts)
    while len(level) > 1:
        i = rnd.randrange(len(level) - 1)
        a, b = level[i], level[i + 1]
        m = oracle.merge(b, a) if rnd.random() < 0.5 else oracle.merge(a, b)
        level[i:i + 2] = [m]
    return level[0]


@pytest.mark.parametrize("shape", ["left", "right", "balanced", "random"])
def test_tree_combine_equals_single_pass_for_every_split(shape):
    n, d = 13, 6
    q, k, v = rand_f32(1, 2, 1, d, scale=2.0), rand_f32(1, 2, n, d), rand_f32(1, 2, n, d)
    prob = oracle.Problem(q, k, v)
    out, lse = run(prob)
    rnd = random.Random(7)
    for h in range(2):
        for S in range(1, n + 1):
            parts = [oracle.partial(prob, 0, h, 0, a, b) for a, b in _chunks(n, S)]
            o, lse_t = oracle.finalize(_reduce(parts, shape, rnd))
            np.testing.assert_allclose(o, out[0, h, 0], rtol=1e-12, atol=1e-14)
            assert abs(lse_t - lse[0, h, 0]) < 1e-12


def test_tree_with_empty_chunks_and_identity():
    n, d = 8, 4
    q, k, v = rand_f32(1, 1, 1, d), rand_f32(1, 1, n, d), rand_f32(1, 1, n, d)
    prob = oracle.Problem(q, k, v)
    out, lse = run(prob)
    ident = (np.zeros(d), -math.inf, 0.0)
    parts = [ident, oracle.partial(prob, 0, 0, 0, 0, 3), oracle.partial(prob, 0, 0, 0, 3, 3), ident,
             oracle.partial(prob, 0, 0, 0, 3, 8), ident]
    o, l = oracle.finalize(_reduce(parts, "balanced", None))
    np.testing.assert_allclose(o, out[0, 0, 0], rtol=1e-12)
    assert abs(l - lse[0, 0, 0]) < 1e-12
    o, l = oracle.finalize(oracle.merge(ident, ident))
    assert np.all(o == 0) and l == -math.inf


def test_combine_of_fp32_partials_matches_single_pass():
    R, n, d, S = 3, 40, 8, 6
    q, k, v = rand_f32(1, R, 1, d), rand_f32(1, R, n, d), rand_f32(1, R, n, d)
    prob = oracle.Problem(q, k, v)
    out, lse = run(prob)
    o_p = np.zeros((R, S, d), np.float32)
    m_p = np.full((R, S), -np.inf, np.float32)
    l_p = np.zeros((R, S), np.float32)
    for r in range(R):
        for s, (a, b) in enumerate(_chunks(n, S)):
            o, m, l = oracle.partial(prob, 0, r, 0, a, b)
            o_p[r, s], m_p[r, s], l_p[r, s] = o, m, l
    o_c, lse_c = oracle.combine(o_p, m_p, l_p)
    np.testing.assert_allclose(o_c, out[0, :, 0], rtol=0, atol=1e-6)
    np.testing.assert_allclose(lse_c, lse[0, :, 0], rtol=0, atol=1e-6)
    # a normalised (O, lse) pair is the partial (O, lse, 1)
    o_n, l_n = oracle.combine(out[0, :, 0][:, None, :].astype(np.float32), lse[0, :, 0][:, None].astype(np.float32),
                              np.ones((R, 1), np.float32))
    np.testing.assert_allclose(o_n, out[0, :, 0], rtol=0, atol=1e-6)
    # counts limit what is read; zero partials -> O = 0, lse = -inf
    o_z, l_z = oracle.combine(o_p, m_p, l_p, count=np.array([0, 1, S], np.int32))
    assert np.all(o_z[0] == 0) and np.isneginf(l_z[0])
    np.testing.assert_allclose(o_z[1], o_p[1, 0] / l_p[1, 0], rtol=1e-6)


# ---------------------------------------------------------------- energy view

def test_output_is_gradient_of_energy():
    d, n = 6, 25
    q, k, v = rand_f32(1, 1, 1, d), rand_f32(1, 1, n, d), rand_f32(1, 1, n, d)
    prob = oracle.Problem(q, k, v)
    out, lse = run(prob)
    assert abs(oracle.energy(prob, 0, 0, 0, np.zeros(d)) - lse[0, 0, 0]) < 1e-13
    h = 1e-5
    grad = np.zeros(d)
    for c in range(d):
        e = np.zeros(d)
        e[c] = h
        grad[c] = (oracle.energy(prob, 0, 0, 0, e) - oracle.energy(prob, 0, 0, 0, -e)) / (2 * h)
    np.testing.assert_allclose(grad, out[0, 0, 0], rtol=0, atol=1e-8)


def test_energy_of_union_is_logsumexp():
    d, n = 4, 10
    q, k, v = rand_f32(1, 1, 1, d), rand_f32(1, 1, n, d), rand_f32(1, 1, n, d)
    zeta = rand_f32(d).astype(np.float64) * 0.1
    full = oracle.energy(oracle.Problem(q, k, v), 0, 0, 0, zeta)
    fa = oracle.energy(oracle.Problem(q, k[:, :, :4].copy(), v[:, :, :4].copy()), 0, 0, 0, zeta)
    fb = oracle.energy(oracle.Problem(q, k[:, :, 4:].copy(), v[:, :, 4:].copy()), 0, 0, 0, zeta)
    assert abs(full - np.logaddexp(fa, fb)) < 1e-13


# ---------------------------------------------------------------- storage formats

def test_bf16_decoder_matches_torch_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_e4m3_decoder_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_bf16_inputs_match_bruteforce_on_decoded_values():
    B, Hq, Hkv, L, d = 1, 4, 2, 11, 8
    tq = torch.randn(B, Hq, 1, d, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    tk = torch.randn(B, Hkv, L, d, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    tv = torch.randn(B, Hkv, L, d, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    out, lse = run(oracle.Problem(bits(tq), bits(tk), bits(tv)))
    qd, kd, vd = (t.to(torch.float64).numpy() for t in (tq, tk, tv))
    for h in range(Hq):
        o_ref, l_ref = brute_row(qd[0, h, 0], kd[0, h // 2], vd[0, h // 2], 1 / math.sqrt(d))
        np.testing.assert_allclose(out[0, h, 0], o_ref, rtol=1e-12, atol=1e-14)
        assert abs(lse[0, h, 0] - l_ref) < 1e-12


def test_e4m3_inputs_apply_their_scale():
    B, Hq, Hkv, L, d = 1, 2, 1, 9, 8
    q = rand_f32(B, Hq, 1, d)
    kc = RNG.integers(0, 0x7E, size=(B, Hkv, L, d), dtype=np.uint8) | (RNG.integers(0, 2, size=(B, Hkv, L, d), dtype=np.uint8) << 7)
    vc = RNG.integers(0, 0x7E, size=(B, Hkv, L, d), dtype=np.uint8)
    ks, vs = np.array([0.0125], np.float32), np.array([3.5], np.float32)
    out, lse = run(oracle.Problem(q, kc, vc, k_scale=ks, v_scale=vs))
    kd = torch.from_numpy(kc).view(torch.float8_e4m3fn).to(torch.float64).numpy() * float(ks[0])
    vd = torch.from_numpy(vc).view(torch.float8_e4m3fn).to(torch.float64).numpy() * float(vs[0])
    for h in range(Hq):
        o_ref, l_ref = brute_row(q[0, h, 0], kd[0, 0], vd[0, 0], 1 / math.sqrt(d))
        np.testing.assert_allclose(out[0, h, 0], o_ref, rtol=1e-12, atol=1e-14)
        assert abs(lse[0, h, 0] - l_ref) < 1e-12


# ------------------------------------------------ two-precision cache (union)
# A cache that keeps some keys in bf16 and the rest in fp8 (the ThriftAttention
# page, introduction and Physical AI Stack section) is, for one query, exact
# attention over the union of both key sets at their real values.

def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def _mixed_case(B, Hq, Hkv, L_hi, L_lo, d, seed):
    g = torch.Generator().manual_seed(seed)
    tq = torch.randn(B, Hq, 1, d, generator=g).to(torch.bfloat16)
    khi = torch.randn(B, Hkv, L_hi, d, generator=g).to(torch.bfloat16)
    vhi = torch.randn(B, Hkv, L_hi, d, generator=g).to(torch.bfloat16)
    klo = (torch.randn(B, Hkv, L_lo, d, generator=g) * 40).to(torch.float8_e4m3fn)
    vlo = (torch.randn(B, Hkv, L_lo, d, generator=g) * 40).to(torch.float8_e4m3fn)
    ks = (torch.rand(B * Hkv, generator=g) * 0.05 + 0.01).numpy().astype(np.float32)
    vs = (torch.rand(B * Hkv, generator=g) * 0.05 + 0.01).numpy().astype(np.float32)
    return tq, khi, vhi, klo, vlo, ks, vs


def test_mixed_matches_bruteforce_over_the_union():
    B, Hq, Hkv, L_hi, L_lo, d = 2, 4, 2, 6, 9, 8
    tq, khi, vhi, klo, vlo, ks, vs = _mixed_case(B, Hq, Hkv, L_hi, L_lo, d, 7)
    hl = np.array([6, 0, 3, 5], np.int32)  # per (sequence, KV head); one head has no bf16 key
    ll = np.array([9, 4, 0, 2], np.int32)  # and one no fp8 key
    out, lse = oracle.decode_mixed(_bits(tq), _bits(khi), _bits(vhi), klo.view(torch.uint8).numpy(),
                                   vlo.view(torch.uint8).numpy(), ks, vs, hl, ll)
    qd = tq.to(torch.float64).numpy()
    khd, vhd = khi.to(torch.float64).numpy(), vhi.to(torch.float64).numpy()
    kld, vld = klo.to(torch.float64).numpy(), vlo.to(torch.float64).numpy()
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            bg = b * Hkv + h // G
            krows = list(khd[b, h // G, :hl[bg]]) + list(kld[b, h // G, :ll[bg]] * float(ks[bg]))
            vrows = list(vhd[b, h // G, :hl[bg]]) + list(vld[b, h // G, :ll[bg]] * float(vs[bg]))
            o_ref, l_ref = brute_row(qd[b, h, 0], krows, vrows, 1 / math.sqrt(d))
            np.testing.assert_allclose(out[b * Hq + h], o_ref, rtol=1e-12, atol=1e-14)
            assert abs(lse[b * Hq + h] - l_ref) < 1e-12


def test_mixed_with_no_fp8_keys_is_the_bf16_decode():
    B, Hq, Hkv, L_hi, L_lo, d = 3, 8, 2, 40, 16, 16
    tq, khi, vhi, klo, vlo, ks, vs = _mixed_case(B, Hq, Hkv, L_hi, L_lo, d, 8)
    lens = np.array([40, 17, 1], np.int32)
    out, lse = oracle.decode_mixed(_bits(tq), _bits(khi), _bits(vhi), klo.view(torch.uint8).numpy(),
                                   vlo.view(torch.uint8).numpy(), ks, vs, np.repeat(lens, Hkv),
                                   np.zeros(B * Hkv, np.int32))
    ref, ref_lse = oracle.attention(oracle.Problem(_bits(tq), _bits(khi), _bits(vhi), kv_lens=lens))
    np.testing.assert_array_equal(out, ref)
    np.testing.assert_array_equal(lse, ref_lse)


def test_mixed_with_no_bf16_keys_is_the_fp8_decode():
    B, Hq, Hkv, L_hi, L_lo, d = 2, 8, 2, 8, 50, 16
    tq, khi, vhi, klo, vlo, ks, vs = _mixed_case(B, Hq, Hkv, L_hi, L_lo, d, 9)
    kc, vc = klo.view(torch.uint8).numpy(), vlo.view(torch.uint8).numpy()
    out, lse = oracle.decode_mixed(_bits(tq), None, None, kc, vc, ks, vs, None, None)
    ref, ref_lse = oracle.attention(oracle.Problem(_bits(tq), kc, vc, k_scale=ks, v_scale=vs))
    np.testing.assert_array_equal(out, ref)
    np.testing.assert_array_equal(lse, ref_lse)


def test_mixed_does_not_depend_on_which_span_holds_a_key():
    # fp8 values times a power-of-two scale are exact bf16 values, so any key can
    # move between the spans without changing its real value; the result may
    # only move by rounding.
    B, Hq, Hkv, L, d = 1, 4, 1, 24, 8
    g = torch.Generator().manual_seed(10)
    tq = torch.randn(B, Hq, 1, d, generator=g).to(torch.bfloat16)
    kf = (torch.randn(B, Hkv, L, d, generator=g) * 30).to(torch.float8_e4m3fn)
    vf = (torch.randn(B, Hkv, L, d, generator=g) * 30).to(torch.float8_e4m3fn)
    ks, vs = np.array([2.0 ** -4], np.float32), np.array([2.0 ** -3], np.float32)
    kb = (kf.to(torch.float32) * float(ks[0])).to(torch.bfloat16)
    vb = (vf.to(torch.float32) * float(vs[0])).to(torch.bfloat16)
    kc, vc = kf.view(torch.uint8).numpy(), vf.view(torch.uint8).numpy()
    ref, ref_lse = oracle.decode_mixed(_bits(tq), _bits(kb), _bits(vb), None, None, None, None)
    for cut in (0, 5, 13, 24):
        # keys [cut, L) stored in bf16 first, keys [0, cut) in fp8
        out, lse = oracle.decode_mixed(_bits(tq), _bits(kb[:, :, cut:]), _bits(vb[:, :, cut:]), kc[:, :, :cut],
                                       vc[:, :, :cut], ks, vs)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-13)


def test_mixed_with_no_key_at_all_is_empty():
    tq, khi, vhi, klo, vlo, ks, vs = _mixed_case(1, 4, 1, 4, 4, 8, 11)
    out, lse = oracle.decode_mixed(_bits(tq), _bits(khi), _bits(vhi), klo.view(torch.uint8).numpy(),
                                   vlo.view(torch.uint8).numpy(), ks, vs, np.zeros(1, np.int32),
                                   np.zeros(1, np.int32))
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_f64_inputs_are_taken_as_given():
    B, Hq, Hkv, L, d = 1, 2, 1, 7, 8
    q, k, v = rand_f32(B, Hq, 1, d), rand_f32(B, Hkv, L, d), rand_f32(B, Hkv, L, d)
    out32, lse32 = oracle.attention(oracle.Problem(q, k, v))
    out64, lse64 = oracle.attention(oracle.Problem(q, k.astype(np.float64), v.astype(np.float64)))
    np.testing.assert_array_equal(out32, out64)
    np.testing.assert_array_equal(lse32, lse64)


# ------------------------------------------------------------- pi-Attention
# The pi-Attention explainer (method section A): a ring-local window of k
# tokens on either side, skip keys a whole number of periods pi away (past
# only when causal), and a gate alpha used as a log-prior in the one softmax.

def _pi_keys(pos, n, window, period, causal):
    """Local and skip key lists written out with ranges (not the oracle's
    modular test)."""
    hi_local = pos if causal else min(n - 1, pos + window)
    local = list(range(max(0, pos - window), hi_local + 1)) if pos >= 0 else []
    skip = []
    if period > 0:
        skip = [j for j in range(pos - period, -1, -period) if j < pos - window]
        if not causal:
            skip += [j for j in range(pos + period, n, period) if j > pos + window]
    return [j for j in local if 0 <= j < n], skip


def _brute_biased(qrow, keys, vals, biases, scale):
    s = [scale * math.fsum(float(a) * float(b) for a, b in zip(qrow, k)) + bb for k, bb in zip(keys, biases)]
    fin = [x for x in s if x != -math.inf]
    if not fin:
        return np.zeros(len(qrow)), -math.inf
    e = [math.exp(x) if x != -math.inf else 0.0 for x in s]
    z = math.fsum(e)
    out = [math.fsum(e[j] * float(vals[j][c]) for j in range(len(keys))) / z for c in range(len(qrow))]
    return np.array(out), math.log(z)


@pytest.mark.parametrize("window,period,causal,Lq", [(2, 3, True, 1), (0, 4, True, 1), (3, 2, True, 9),
                                                     (1, 5, False, 9), (4, 1, True, 6), (2, 0, True, 9),
                                                     (30, 3, True, 9)])
def test_pi_matches_bruteforce_on_explicit_key_lists(window, period, causal, Lq):
    B, Hq, Hkv, L, d = 2, 4, 2, 23, 6
    q, k, v = rand_f32(B, Hq, Lq, d), rand_f32(B, Hkv, L, d), rand_f32(B, Hkv, L, d)
    lens = np.array([23, 14], np.int32)
    alpha = RNG.uniform(0.05, 0.95, size=(B, Hq, Lq)).astype(np.float32)
    alpha[0, 0, 0] = 1.0  # skip keys switched off
    alpha[1, 1, -1] = 0.0  # local keys switched off
    prob = oracle.Problem(q, k, v, kv_lens=lens, scale=0.41, causal=causal)
    out, lse = oracle.pi_attention(prob, window, period, alpha)
    out = out.reshape(B, Hq, Lq, d)
    lse = lse.reshape(B, Hq, Lq)
    for b in range(B):
        n = int(lens[b])
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(Lq):
                pos = n - Lq + i
                local, skip = _pi_keys(pos, n, window, period, causal)
                a = float(alpha[b, h, i])
                bl = math.log(a) if a > 0 else -math.inf
                bs = math.log(1 - a) if a < 1 else -math.inf
                keys = [k[b, g, j] for j in local + skip]
                vals = [v[b, g, j] for j in local + skip]
                o_ref, l_ref = _brute_biased(q[b, h, i], keys, vals, [bl] * len(local) + [bs] * len(skip), 0.41)
                np.testing.assert_allclose(out[b, h, i], o_ref, rtol=1e-12, atol=1e-14)
                if l_ref == -math.inf:
                    assert lse[b, h, i] == -math.inf
                else:
                    assert abs(lse[b, h, i] - l_ref) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_pi_with_period_one_is_full_attention(causal):
    # every key is a whole number of periods away: the union is every key
    B, Hq, Hkv, L, d = 1, 4, 2, 40, 8
    q, k, v = rand_f32(B, Hq, 12, d), rand_f32(B, Hkv, L, d), rand_f32(B, Hkv, L, d)
    prob = oracle.Problem(q, k, v, causal=causal)
    ref, ref_lse = oracle.attention(prob)
    for window in (0, 5, 100):
        out, lse = oracle.pi_attention(prob, window, 1)
        np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-13)


def test_pi_alpha_one_is_the_window_and_alpha_zero_the_strided_slice():
    B, Hq, Hkv, L, d = 1, 4, 1, 50, 8
    q, k, v = rand_f32(B, Hq, 1, d), rand_f32(B, Hkv, L, d), rand_f32(B, Hkv, L, d)
    window, period = 6, 7
    prob = oracle.Problem(q, k, v, causal=True)
    pos = L - 1
    ones = np.ones((B, Hq, 1), np.float32)
    out, lse = oracle.pi_attention(prob, window, period, ones)
    win = oracle.Problem(q, k[:, :, pos - window:], v[:, :, pos - window:])
    ref, ref_lse = oracle.attention(win)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13)
    out, lse = oracle.pi_attention(prob, window, period, np.zeros_like(ones))
    r = pos % period
    last = pos - window - 1
    sl = slice(r, last + 1, period)
    ref, ref_lse = oracle.attention(oracle.Problem(q, np.ascontiguousarray(k[:, :, sl]),
                                                   np.ascontiguousarray(v[:, :, sl])))
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13)


def test_pi_half_alpha_changes_only_lse():
    B, Hq, Hkv, L, d = 1, 2, 1, 30, 8
    q, k, v = rand_f32(B, Hq, 5, d), rand_f32(B, Hkv, L, d), rand_f32(B, Hkv, L, d)
    prob = oracle.Problem(q, k, v, causal=True)
    out0, lse0 = oracle.pi_attention(prob, 3, 4)
    out1, lse1 = oracle.pi_attention(prob, 3, 4, np.full((B, Hq, 5), 0.5, np.float32))
    np.testing.assert_allclose(out1, out0, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse1, lse0 + math.log(0.5), rtol=1e-13)


def test_pi_is_the_merge_of_its_window_and_its_skip_keys():
    # the prior shifts each part's log-sum-exp; the tree merge of the two
    # shifted parts is the whole (the Tree Attention explainer, section 3)
    B, Hq, Hkv, L, d = 1, 4, 1, 64, 8
    q, k, v = rand_f32(B, Hq, 1, d), rand_f32(B, Hkv, L, d), rand_f32(B, Hkv, L, d)
    alpha = np.array([0.2, 0.5, 0.7, 0.9], np.float32).reshape(B, Hq, 1)
    window, period = 9, 5
    prob = oracle.Problem(q, k, v, causal=True)
    out, lse = oracle.pi_attention(prob, window, period, alpha)
    pos = L - 1
    for h in range(Hq):
        a = float(alpha[0, h, 0])
        o_l, m_l, l_l = oracle.partial(prob, 0, h, 0, pos - window, pos + 1)
        sk = oracle.Problem(q, np.ascontiguousarray(k[:, :, pos % period:pos - window:period]),
                            np.ascontiguousarray(v[:, :, pos % period:pos - window:period]))
        o_s, m_s, l_s = oracle.partial(sk, 0, h, 0, 0, L)
        merged = oracle.finalize(oracle.merge((o_l, m_l + math.log(a), l_l), (o_s, m_s + math.log(1 - a), l_s)))
        np.testing.assert_allclose(out[h], merged[0], rtol=1e-12, atol=1e-14)
        assert abs(lse[h] - merged[1]) < 1e-12


# ------------------------------------------------------------- backward
# Gradients of a loss L = sum(dO * O) with respect to q, k and v.

def _loss(q, k, v, dout, **kw):
    out, _ = oracle.attention(oracle.Problem(q, k, v, **kw))
    return float((out.reshape(dout.shape) * dout).sum())


@pytest.mark.parametrize("causal,Lq,lens", [(True, 6, None), (False, 6, None), (True, 3, None), (True, 6, [4])])
def test_backward_matches_central_differences(causal, Lq, lens):
    B, Hq, Hkv, L, d = 1, 4, 2, 6, 5
    rng = np.random.default_rng(3)
    q = rng.standard_normal((B, Hq, Lq, d))
    k = rng.standard_normal((B, Hkv, L, d))
    v = rng.standard_normal((B, Hkv, L, d))
    dout = rng.standard_normal((B, Hq, Lq, d))
    kw = dict(causal=causal, scale=0.6, kv_lens=None if lens is None else np.array(lens, np.int32))
    dq, dk, dv = oracle.backward(oracle.Problem(q, k, v, **kw), dout)
    h = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], dout, **kw)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], dout, **kw)
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


def test_backward_key_gradients_sum_to_zero():
    # adding a constant to every logit of a row changes nothing, so the logit
    # gradients of a row sum to zero, and so do the key gradients of a head
    B, Hq, Hkv, L, d = 2, 8, 2, 40, 16
    q, k, v = rand_f32(B, Hq, 40, d), rand_f32(B, Hkv, L, d), rand_f32(B, Hkv, L, d)
    dout = rand_f32(B, Hq, 40, d)
    dq, dk, dv = oracle.backward(oracle.Problem(q, k, v, causal=True), dout)
    assert np.abs(dk.sum(axis=2)).max() < 1e-10
    # and the value gradients of a head add up to the sum of its rows' dO
    np.testing.assert_allclose(dv.sum(axis=2), dout.astype(np.float64).reshape(B, Hkv, -1, d).sum(axis=2),
                               rtol=1e-12, atol=1e-10)


@pytest.mark.parametrize("B,Hq,Hkv,Lq,L,causal,lens", [
    (1, 4, 2, 6, 6, True, None), (2, 8, 2, 37, 50, True, [50, 23]), (1, 4, 1, 20, 33, False, None),
    (1, 8, 2, 1, 40, True, None), (2, 4, 4, 30, 30, True, [0, 30])])
def test_backward_subset_equals_the_full_backward(B, Hq, Hkv, Lq, L, causal, lens):
    # the full backward is pinned by central differences above; the subset
    # must give the same rows and keys, in any order and with repeats
    rng = np.random.default_rng(B * 100 + Lq)
    q, k, v = rand_f32(B, Hq, Lq, 16), rand_f32(B, Hkv, L, 16), rand_f32(B, Hkv, L, 16)
    dout = rand_f32(B, Hq, Lq, 16)
    prob = oracle.Problem(q, k, v, causal=causal, kv_lens=None if lens is None else np.array(lens, np.int32))
    dq, dk, dv = oracle.backward(prob, dout)
    rows = rng.permutation(B * Hq * Lq)[:max(1, B * Hq * Lq // 2)]
    rows = np.concatenate([rows, rows[:2]])
    keys = rng.permutation(B * Hkv * L)[:max(1, B * Hkv * L // 3)]
    keys = np.concatenate([keys, keys[:1]])
    sq, sk, sv = oracle.backward_subset(prob, dout, q_rows=rows, keys=keys)
    np.testing.assert_allclose(sq, dq.reshape(-1, 16)[rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sk, dk.reshape(-1, 16)[keys], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sv, dv.reshape(-1, 16)[keys], rtol=1e-12, atol=1e-13)


def test_backward_subset_matches_central_differences_directly():
    B, Hq, Hkv, L, d = 1, 4, 2, 7, 4
    rng = np.random.default_rng(11)
    q, k, v = rng.standard_normal((B, Hq, L, d)), rng.standard_normal((B, Hkv, L, d)), rng.standard_normal((B, Hkv, L, d))
    dout = rng.standard_normal((B, Hq, L, d))
    kw = dict(causal=True, scale=0.7)
    rows, keys = [3, 9, 27], [0, 5, 13]
    sq, sk, sv = oracle.backward_subset(oracle.Problem(q, k, v, **kw), dout, q_rows=rows, keys=keys)
    h = 1e-5
    for name, x, got, ids in (("q", q, sq, rows), ("k", k, sk, keys), ("v", v, sv, keys)):
        for n, flat in enumerate(ids):
            for c in range(d):
                idx = np.unravel_index(flat, x.shape[:3]) + (c,)
                args = {"q": q, "k": k, "v": v}
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args[name] = xp
                lp = _loss(args["q"], args["k"], args["v"], dout, **kw)
                args[name] = xm
                lm = _loss(args["q"], args["k"], args["v"], dout, **kw)
                assert abs(got[n, c] - (lp - lm) / (2 * h)) <= 1e-6 * max(1.0, abs(got[n, c])), (name, flat, c)


def test_backward_subset_rejects_ids_out_of_range():
    q, k, v = rand_f32(1, 2, 4, 8), rand_f32(1, 1, 4, 8), rand_f32(1, 1, 4, 8)
    prob = oracle.Problem(q, k, v, causal=True)
    with pytest.raises(ValueError):
        oracle.backward_subset(prob, q, q_rows=[8])
    with pytest.raises(ValueError):
        oracle.backward_subset(prob, q, keys=[-1])


# ------------------------------------------------ MX FP4 low-precision span
# The page's FP4 (a 4-bit float with a 2-bit exponent) held as OCP MX FP4:
# E2M1 elements, one E8M0 power-of-two scale per 32 consecutive elements of a
# row, two elements per byte with the first in the low nibble.

def _e2m1_table(code):
    # the magnitudes OCP MX v1.0 lists for E2M1 codes 0..7; bit 3 is the sign
    mag = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0][code & 7]
    return -mag if code & 8 else mag


def test_e2m1_decoder_is_the_ocp_table():
    got = oracle.e2m1_to_f64(np.arange(16, dtype=np.uint8))
    assert [float(x) for x in got] == [_e2m1_table(c) for c in range(16)]
    assert math.copysign(1.0, float(got[8])) == -1.0  # code 8 is negative zero


def test_e8m0_decoder_is_a_power_of_two():
    got = oracle.e8m0_to_f64(np.arange(256, dtype=np.uint8))
    assert all(float(got[e]) == math.ldexp(1.0, e - 127) for e in range(255))
    assert math.isnan(float(got[255]))


def test_mxfp4_rows_low_nibble_first_one_scale_per_32():
    codes = np.zeros((2, 32), np.uint8)
    scales = np.array([[127, 130], [120, 127]], np.uint8)
    codes[0, 0] = 0x71   # element 0: code 1 (0.5); element 1: code 7 (6)
    codes[0, 16] = 0x0A  # element 32: code 10 (-1), in the second block (scale 2^3)
    codes[1, 31] = 0xF0  # element 62: 0; element 63: code 15 (-6)
    out = oracle.mxfp4_to_f64(codes, scales)
    assert out[0, 0] == 0.5 and out[0, 1] == 6.0 and out[0, 32] == -8.0 and out[1, 63] == -6.0
    assert np.count_nonzero(out) == 4


def test_mxfp4_codes_of_the_input_generator_decode_to_their_values():
    # the generator's encoder (OCP MX conversion) and the oracle's decoder are
    # separate code: decoded values are the drawn values to within half a grid
    # step of the block, or the block's +-6 * scale where the value saturates
    shape = (3, 5, 128)
    f = datagen.normal_f32(7, 4, shape, 0.5).astype(np.float64)
    codes, sc = datagen.normal_mxfp4(7, 4, shape, 0.5)
    got = oracle.mxfp4_to_f64(codes, sc)
    s = np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=-1)
    y = f / s
    blk = np.abs(y).reshape(-1, 32).max(axis=1)
    assert np.all((blk >= 4) & (blk < 8))  # the shared exponent is floor(log2 amax) - 2
    sat = np.abs(y) > 6
    assert np.all(got[sat] == np.sign(f[sat]) * 6 * s[sat])
    step = np.where(np.abs(y) < 2, 0.5, np.where(np.abs(y) < 4, 1.0, 2.0))
    assert np.all(np.abs(got - f)[~sat] <= 0.5 * step[~sat] * s[~sat])


def test_mixed_fp4_span_is_attention_over_the_decoded_union():
    B, Hq, Hkv, L_hi, L_lo, d = 2, 4, 2, 5, 9, 64
    rng = np.random.default_rng(11)
    tq = torch.from_numpy(rng.standard_normal((B, Hq, 1, d)).astype(np.float32)).to(torch.bfloat16)
    khi = torch.from_numpy(rng.standard_normal((B, Hkv, L_hi, d)).astype(np.float32)).to(torch.bfloat16)
    vhi = torch.from_numpy(rng.standard_normal((B, Hkv, L_hi, d)).astype(np.float32)).to(torch.bfloat16)
    klo = rng.integers(0, 256, (B, Hkv, L_lo, d // 2), dtype=np.uint8)
    vlo = rng.integers(0, 256, (B, Hkv, L_lo, d // 2), dtype=np.uint8)
    ksc = rng.integers(121, 129, (B, Hkv, L_lo, d // 32), dtype=np.uint8)
    vsc = rng.integers(121, 129, (B, Hkv, L_lo, d // 32), dtype=np.uint8)
    hl = np.array([5, 0, 2, 4], np.int32)  # per (sequence, KV head); one head has no bf16 key
    ll = np.array([9, 3, 0, 1], np.int32)  # and one no fp4 key
    out, lse = oracle.decode_mixed(_bits(tq), _bits(khi), _bits(vhi), klo, vlo, ksc, vsc, hl, ll,
                                   lo_format="mxfp4")

    def dec(codes, scales):  # test-side decode: the table above, ldexp for the scale
        vals = np.empty(codes.shape[:-1] + (d,))
        for idx in np.ndindex(*codes.shape[:-1]):
            for c in range(d):
                byte = int(codes[idx + (c // 2,)])
                code = byte >> 4 if c & 1 else byte & 15
                vals[idx + (c,)] = math.ldexp(_e2m1_table(code), int(scales[idx + (c // 32,)]) - 127)
        return vals

    kld, vld = dec(klo, ksc), dec(vlo, vsc)
    qd = tq.to(torch.float64).numpy()
    khd, vhd = khi.to(torch.float64).numpy(), vhi.to(torch.float64).numpy()
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            g = h // G
            bg = b * Hkv + g
            krows = list(khd[b, g, :hl[bg]]) + list(kld[b, g, :ll[bg]])
            vrows = list(vhd[b, g, :hl[bg]]) + list(vld[b, g, :ll[bg]])
            o_ref, l_ref = brute_row(qd[b, h, 0], krows, vrows, 1 / math.sqrt(d))
            np.testing.assert_allclose(out[b * Hq + h], o_ref, rtol=1e-12, atol=1e-14)
            assert abs(lse[b * Hq + h] - l_ref) < 1e-12


# ------------------------------------------- three precisions in one cache
# The ThriftAttention page switches among FP4, FP8 and BF16 within one kernel
# (COMPUTE layer of its Physical AI Stack section): one query's attention over
# a cache whose keys are kept in all three formats is attention over the union.

def _fp4_test_decode(codes, scales, d):
    vals = np.empty(codes.shape[:-1] + (d,))
    for idx in np.ndindex(*codes.shape[:-1]):
        for c in range(d):
            byte = int(codes[idx + (c // 2,)])
            code = byte >> 4 if c & 1 else byte & 15
            vals[idx + (c,)] = math.ldexp(_e2m1_table(code), int(scales[idx + (c // 32,)]) - 127)
    return vals


def _three_span_case(B, Hq, Hkv, L3, d, seed):
    rng = np.random.default_rng(seed)
    tq = torch.from_numpy(rng.standard_normal((B, Hq, 1, d)).astype(np.float32)).to(torch.bfloat16)
    kb = torch.from_numpy(rng.standard_normal((B, Hkv, L3[0], d)).astype(np.float32)).to(torch.bfloat16)
    vb = torch.from_numpy(rng.standard_normal((B, Hkv, L3[0], d)).astype(np.float32)).to(torch.bfloat16)
    k8 = (torch.from_numpy(rng.standard_normal((B, Hkv, L3[1], d)).astype(np.float32)) * 40).to(torch.float8_e4m3fn)
    v8 = (torch.from_numpy(rng.standard_normal((B, Hkv, L3[1], d)).astype(np.float32)) * 40).to(torch.float8_e4m3fn)
    ks8 = rng.uniform(0.01, 0.06, B * Hkv).astype(np.float32)
    vs8 = rng.uniform(0.01, 0.06, B * Hkv).astype(np.float32)
    k4 = rng.integers(0, 256, (B, Hkv, L3[2], d // 2), dtype=np.uint8)
    v4 = rng.integers(0, 256, (B, Hkv, L3[2], d // 2), dtype=np.uint8)
    ks4 = rng.integers(121, 129, (B, Hkv, L3[2], d // 32), dtype=np.uint8)
    vs4 = rng.integers(121, 129, (B, Hkv, L3[2], d // 32), dtype=np.uint8)
    return tq, (kb, vb), (k8, v8, ks8, vs8), (k4, v4, ks4, vs4)


def _spans(c, lens):
    tq, (kb, vb), (k8, v8, ks8, vs8), (k4, v4, ks4, vs4) = c
    return [dict(k=_bits(kb), v=_bits(vb), format="bf16", lens=lens[0]),
            dict(k=k8.view(torch.uint8).numpy(), v=v8.view(torch.uint8).numpy(), format="e4m3", k_scale=ks8,
                 v_scale=vs8, lens=lens[1]),
            dict(k=k4, v=v4, format="mxfp4", k_scale=ks4, v_scale=vs4, lens=lens[2])]


def test_three_span_cache_is_attention_over_the_decoded_union():
    B, Hq, Hkv, d = 2, 4, 2, 64
    c = _three_span_case(B, Hq, Hkv, (5, 7, 9), d, 21)
    lens = (np.array([5, 0, 2, 3], np.int32), np.array([7, 4, 0, 1], np.int32), np.array([9, 3, 0, 0], np.int32))
    out, lse = oracle.decode_spans(_bits(c[0]), _spans(c, lens))
    tq, (kb, vb), (k8, v8, ks8, vs8), (k4, v4, ks4, vs4) = c
    qd = tq.to(torch.float64).numpy()
    kbd, vbd = kb.to(torch.float64).numpy(), vb.to(torch.float64).numpy()
    k8d, v8d = k8.to(torch.float64).numpy(), v8.to(torch.float64).numpy()
    k4d, v4d = _fp4_test_decode(k4, ks4, d), _fp4_test_decode(v4, vs4, d)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            g = h // G
            bg = b * Hkv + g
            krows = (list(kbd[b, g, :lens[0][bg]]) + list(k8d[b, g, :lens[1][bg]] * float(ks8[bg])) +
                     list(k4d[b, g, :lens[2][bg]]))
            vrows = (list(vbd[b, g, :lens[0][bg]]) + list(v8d[b, g, :lens[1][bg]] * float(vs8[bg])) +
                     list(v4d[b, g, :lens[2][bg]]))
            if not krows:  # (b=1, g=1) has no key in any span
                assert np.all(out[b * Hq + h] == 0) and np.isneginf(lse[b * Hq + h])
                continue
            o_ref, l_ref = brute_row(qd[b, h, 0], krows, vrows, 1 / math.sqrt(d))
            np.testing.assert_allclose(out[b * Hq + h], o_ref, rtol=1e-12, atol=1e-14)
            assert abs(lse[b * Hq + h] - l_ref) < 1e-12


def test_three_span_cache_does_not_depend_on_span_order():
    c = _three_span_case(1, 8, 2, (30, 20, 40), 64, 22)
    lens = (None, np.array([20, 11], np.int32), np.array([3, 40], np.int32))
    sp = _spans(c, lens)
    ref, ref_lse = oracle.decode_spans(_bits(c[0]), sp)
    for order in ((2, 0, 1), (1, 2, 0), (2, 1, 0)):
        out, lse = oracle.decode_spans(_bits(c[0]), [sp[i] for i in order])
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-13)
    # and two of the spans alone are the two-precision decode
    two, two_lse = oracle.decode_mixed(_bits(c[0]), sp[0]["k"], sp[0]["v"], sp[2]["k"], sp[2]["v"], sp[2]["k_scale"],
                                       sp[2]["v_scale"], None, lens[2], lo_format="mxfp4")
    out, lse = oracle.decode_spans(_bits(c[0]), [sp[0], dict(sp[1], lens=np.zeros(2, np.int32)), sp[2]])
    np.testing.assert_array_equal(out, two)
    np.testing.assert_array_equal(lse, two_lse)
