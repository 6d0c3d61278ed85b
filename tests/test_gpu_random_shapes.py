"""GPU parity against the oracle on seeded random shapes: batch sizes, head
ratios (1, 2, 4, 8 query heads per KV head), head dims 64 and 128, lengths
that are multiples of nothing in particular, ragged per-sequence or per-head
lengths (zero included), causal or not, automatic or explicit split counts,
for the plain, two-precision (bf16 + fp8, bf16 + MX fp4), three-precision and
pi-Attention decodes, the plain and pi-Attention prefills and the prefill's
backward. The shapes come from a fixed generator, so every run checks the
same cases; each case prints its parameters before it runs."""
import numpy as np
import pytest
import torch

import oracle
from _gpu import (assert_close, assert_lse_close, decode_on_gpu, from_dev, mixed_fp4_on_gpu, mixed_on_gpu, needs_gpu,
                  oracle_decode, oracle_mixed, oracle_pi, pi_on_gpu)
from datagen.workloads import make_inputs, make_mixed3_inputs, make_mixed_inputs, mixed3_spans
from test_gpu_backward import _check as check_grad
from test_gpu_backward import _run as backward_on_gpu
from test_gpu_mixed3 import _run as mixed3_on_gpu
from test_gpu_pi_prefill import oracle_pi_rows, pi_prefill_on_gpu
from test_gpu_prefill import oracle_rows, prefill_on_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]


def _decode_cases(n=60):
    r = np.random.default_rng(2024)
    out = []
    for _ in range(n):
        fmt = ["bf16", "bf16", "e4m3", "f32"][r.integers(4)]
        d = int(r.choice([64, 128]))
        G = int(r.choice([1, 2, 4, 8]))
        Hkv = int(r.integers(1, 4))
        B = int(r.integers(1, 5))
        L = int(r.integers(1, 3001))
        ragged = bool(r.integers(2))
        causal = bool(r.integers(2))
        S = int(r.choice([0, int(r.integers(1, 41))]))
        out.append((fmt, d, G, Hkv, B, L, ragged, causal, S, int(r.integers(1 << 30))))
    return out


@pytest.mark.parametrize("fmt,d,G,Hkv,B,L,ragged,causal,S,seed", _decode_cases())
def test_random_decode(fmt, d, G, Hkv, B, L, ragged, causal, S, seed):
    print("decode", fmt, "d", d, "G", G, "Hkv", Hkv, "B", B, "L", L, "ragged", ragged, "causal", causal, "S", S,
          flush=True)
    wl = {"bf16": 2, "e4m3": 5, "f32": 1}[fmt]
    inp = make_inputs(wl, B=B, Hq=G * Hkv, Hkv=Hkv, d=d, L=L, seed=seed % 100000)
    if ragged:
        inp["kv_lens"] = np.random.default_rng(seed).integers(0, L + 1, size=B).astype(np.int32)
    out, lse = decode_on_gpu(inp, num_splits=S, causal=causal)
    ref, ref_lse = oracle_decode(inp, causal=causal)
    kind = "f32" if fmt == "f32" else "bf16"
    assert_close(from_dev(out)[:, :, 0, :], ref, kind, what="random decode")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, 1e-5 if kind == "f32" else 2e-3)


def _mixed_cases(n=24):
    r = np.random.default_rng(2025)
    out = []
    for _ in range(n):
        d = int(r.choice([64, 128]))
        G = int(r.choice([1, 2, 4, 8]))
        Hkv = int(r.integers(1, 3))
        B = int(r.integers(1, 4))
        L_hi = int(r.choice([0, int(r.integers(1, 1500))]))
        L_lo = int(r.integers(1, 3000)) if L_hi == 0 else int(r.choice([0, int(r.integers(1, 3000))]))
        ragged = bool(r.integers(2))
        S = (0, 0) if r.integers(2) else (int(r.integers(1, 9)), int(r.integers(1, 17)))
        out.append((d, G, Hkv, B, L_hi, L_lo, ragged, S, int(r.integers(1 << 30))))
    return out


@pytest.mark.parametrize("d,G,Hkv,B,L_hi,L_lo,ragged,S,seed", _mixed_cases())
def test_random_mixed_decode(d, G, Hkv, B, L_hi, L_lo, ragged, S, seed):
    print("mixed d", d, "G", G, "Hkv", Hkv, "B", B, "L_hi", L_hi, "L_lo", L_lo, "ragged", ragged, "S", S, flush=True)
    inp = make_mixed_inputs(B=B, Hq=G * Hkv, Hkv=Hkv, d=d, L_hi=L_hi, L_lo=L_lo, lens=(0.0, 1.0) if ragged else None,
                            seed=seed % 100000)
    S_hi, S_lo = S
    out, lse = mixed_on_gpu(inp, num_splits_hi=S_hi if L_hi else 0, num_splits_lo=S_lo if L_lo else 0)
    ref, ref_lse = oracle_mixed(inp)
    assert_close(from_dev(out)[:, :, 0, :], ref, "bf16", what="random mixed")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, 2e-3)


def _pi_cases(n=24):
    r = np.random.default_rng(2026)
    out = []
    for _ in range(n):
        kv = ["bf16", "e4m3"][r.integers(2)]
        d = int(r.choice([64, 128]))
        G = int(r.choice([1, 2, 4, 8]))
        Hkv = int(r.integers(1, 3))
        B = int(r.integers(1, 4))
        L = int(r.integers(2, 4000))
        window = int(r.integers(0, L))
        period = int(r.choice([0, int(r.integers(1, 300))]))
        alpha = bool(r.integers(2))
        ragged = bool(r.integers(2))
        out.append((kv, d, G, Hkv, B, L, window, period, alpha, ragged, int(r.integers(1 << 30))))
    return out


@pytest.mark.parametrize("kv,d,G,Hkv,B,L,window,period,alpha,ragged,seed", _pi_cases())
def test_random_pi_decode(kv, d, G, Hkv, B, L, window, period, alpha, ragged, seed):
    print("pi decode", kv, "d", d, "G", G, "Hkv", Hkv, "B", B, "L", L, "window", window, "period", period, "alpha",
          alpha, "ragged", ragged, flush=True)
    inp = make_inputs(2 if kv == "bf16" else 5, B=B, Hq=G * Hkv, Hkv=Hkv, d=d, L=L, seed=seed % 100000)
    rng = np.random.default_rng(seed)
    if ragged:
        inp["kv_lens"] = rng.integers(0, L + 1, size=B).astype(np.int32)
    a = rng.uniform(0.0, 1.0, size=(B, G * Hkv, 1)).astype(np.float32) if alpha else None
    out, lse = pi_on_gpu(inp, window, period, alpha=a)
    ref, ref_lse = oracle_pi(inp, window, period, a)
    assert_close(from_dev(out)[:, :, 0, :], ref, "bf16", what="random pi decode")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, 2e-3)


def _prefill_cases(n=24):
    r = np.random.default_rng(2027)
    out = []
    for _ in range(n):
        G = int(r.choice([1, 2, 4, 8]))
        Hkv = int(r.integers(1, 3))
        B = int(r.integers(1, 3))
        Lkv = int(r.integers(1, 700))
        causal = bool(r.integers(2))
        Lq = int(r.integers(1, Lkv + 1)) if causal else int(r.integers(1, 700))
        out.append((G, Hkv, B, Lq, Lkv, causal, int(r.integers(1 << 30))))
    return out


@pytest.mark.parametrize("G,Hkv,B,Lq,Lkv,causal,seed", _prefill_cases())
def test_random_prefill(G, Hkv, B, Lq, Lkv, causal, seed):
    print("prefill G", G, "Hkv", Hkv, "B", B, "Lq", Lq, "Lkv", Lkv, "causal", causal, flush=True)
    inp = make_inputs(4, B=B, Hq=G * Hkv, Hkv=Hkv, L=Lkv, Lq=Lq, seed=seed % 100000)
    out, lse = prefill_on_gpu(inp, causal)
    ref, ref_lse = oracle_rows(inp, causal)
    assert_close(from_dev(out).reshape(-1, 128), ref, "bf16", what="random prefill")
    assert_lse_close(lse.cpu().numpy().astype(np.float64).ravel(), ref_lse, 2e-3)


def _pi_prefill_cases(n=20):
    r = np.random.default_rng(2028)
    out = []
    for _ in range(n):
        G = int(r.choice([1, 2, 4, 8]))
        Hkv = int(r.integers(1, 3))
        B = int(r.integers(1, 3))
        L = int(r.integers(2, 800))
        window = int(r.integers(0, L))
        period = int(r.choice([0, int(r.integers(1, 100))]))
        causal = bool(r.integers(2))
        alpha = bool(r.integers(2))
        out.append((G, Hkv, B, L, window, period, causal, alpha, int(r.integers(1 << 30))))
    return out


@pytest.mark.parametrize("G,Hkv,B,L,window,period,causal,alpha,seed", _pi_prefill_cases())
def test_random_pi_prefill(G, Hkv, B, L, window, period, causal, alpha, seed):
    print("pi prefill G", G, "Hkv", Hkv, "B", B, "L", L, "window", window, "period", period, "causal", causal,
          "alpha", alpha, flush=True)
    inp = make_inputs(4, B=B, Hq=G * Hkv, Hkv=Hkv, L=L, seed=seed % 100000)
    a = np.random.default_rng(seed).uniform(0.0, 1.0, size=(B, G * Hkv, L)).astype(np.float32) if alpha else None
    out, lse = pi_prefill_on_gpu(inp, window, period, a, causal=causal)
    ref, ref_lse = oracle_pi_rows(inp, window, period, a, causal=causal)
    assert_close(from_dev(out).reshape(-1, 128), ref, "bf16", what="random pi prefill")
    assert_lse_close(lse.cpu().numpy().astype(np.float64).ravel(), ref_lse, 2e-3)


def _fp4_cases(n=16):
    r = np.random.default_rng(2029)
    out = []
    for _ in range(n):
        G = int(r.choice([1, 2, 4, 8]))
        Hkv = int(r.integers(1, 3))
        B = int(r.integers(1, 4))
        L_hi = int(r.choice([0, int(r.integers(1, 1500))]))
        L_lo = int(r.integers(1, 3000)) if L_hi == 0 else int(r.choice([0, int(r.integers(1, 3000))]))
        ragged = bool(r.integers(2))
        S = (0, 0) if r.integers(2) else (int(r.integers(1, 9)), int(r.integers(1, 17)))
        out.append((G, Hkv, B, L_hi, L_lo, ragged, S, int(r.integers(1 << 30))))
    return out


@pytest.mark.parametrize("G,Hkv,B,L_hi,L_lo,ragged,S,seed", _fp4_cases())
def test_random_mixed_fp4_decode(G, Hkv, B, L_hi, L_lo, ragged, S, seed):
    print("mixed fp4 G", G, "Hkv", Hkv, "B", B, "L_hi", L_hi, "L_lo", L_lo, "ragged", ragged, "S", S, flush=True)
    inp = make_mixed_inputs(9, B=B, Hq=G * Hkv, Hkv=Hkv, L_hi=L_hi, L_lo=L_lo, lens=(0.0, 1.0) if ragged else None,
                            seed=seed % 100000)
    out, lse = mixed_fp4_on_gpu(inp, S[0] if L_hi else 0, S[1] if L_lo else 0)
    ref, ref_lse = oracle_mixed(inp)
    assert_close(from_dev(out)[:, :, 0, :], ref, "bf16", what="random mixed fp4")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, 2e-3)


def _mixed3_cases(n=12):
    r = np.random.default_rng(2030)
    out = []
    for _ in range(n):
        G = int(r.choice([1, 2, 4, 8]))
        Hkv = int(r.integers(1, 3))
        B = int(r.integers(1, 4))
        L = [int(r.choice([0, int(r.integers(1, 1500))])) for _ in range(3)]
        if not any(L):
            L[int(r.integers(3))] = int(r.integers(1, 1500))
        ragged = bool(r.integers(2))
        S = (0, 0, 0) if r.integers(2) else tuple(int(r.integers(1, 9)) for _ in range(3))
        out.append((G, Hkv, B, tuple(L), ragged, S, int(r.integers(1 << 30))))
    return out


@pytest.mark.parametrize("G,Hkv,B,L,ragged,S,seed", _mixed3_cases())
def test_random_mixed3_decode(G, Hkv, B, L, ragged, S, seed):
    print("mixed3 G", G, "Hkv", Hkv, "B", B, "L", L, "ragged", ragged, "S", S, flush=True)
    inp = make_mixed3_inputs(B=B, Hq=G * Hkv, Hkv=Hkv, L=sum(L), L_hi=L[0], L_mid=L[1], L_lo=L[2],
                             lens=(0.0, 1.0) if ragged else None, seed=seed % 100000)
    out, lse = mixed3_on_gpu(inp, tuple(s if n else 0 for s, n in zip(S, L)))
    ref, ref_lse = oracle.decode_spans(inp["q"], mixed3_spans(inp))
    assert_close(from_dev(out).reshape(B * G * Hkv, -1), ref, "bf16", what="random mixed3")
    assert_lse_close(lse.cpu().numpy().astype(np.float64).ravel(), ref_lse, 2e-3)


def _backward_cases(n=10):
    r = np.random.default_rng(2031)
    out = []
    for _ in range(n):
        G = int(r.choice([1, 2, 4, 8]))
        Hkv = int(r.integers(1, 3))
        B = int(r.integers(1, 3))
        Lkv = int(r.integers(1, 400))
        causal = bool(r.integers(2))
        Lq = int(r.integers(1, Lkv + 1)) if causal else int(r.integers(1, 400))
        out.append((G, Hkv, B, Lq, Lkv, causal, int(r.integers(1 << 30))))
    return out


@pytest.mark.parametrize("G,Hkv,B,Lq,Lkv,causal,seed", _backward_cases())
def test_random_backward(G, Hkv, B, Lq, Lkv, causal, seed):
    print("backward G", G, "Hkv", Hkv, "B", B, "Lq", Lq, "Lkv", Lkv, "causal", causal, flush=True)
    inp = make_inputs(4, B=B, Hq=G * Hkv, Hkv=Hkv, L=Lkv, Lq=Lq, seed=seed % 100000)
    (dq, dk, dv), dout_bits, _, _ = backward_on_gpu(inp, causal, seed=seed % 1000)
    rq, rk, rv = oracle.backward(oracle.Problem(inp["q"], inp["k"], inp["v"], causal=causal), dout_bits)
    what = "random bwd %s" % ((G, Hkv, B, Lq, Lkv, causal),)
    check_grad(dq, rq, what + " dq")
    check_grad(dk, rk, what + " dk")
    check_grad(dv, rv, what + " dv")


def _prefill_d64_cases(n=12):
    r = np.random.default_rng(2032)
    out = []
    for _ in range(n):
        G = int(r.choice([1, 2, 4, 8]))
        Hkv = int(r.integers(1, 3))
        B = int(r.integers(1, 3))
        Lkv = int(r.integers(1, 700))
        causal = bool(r.integers(2))
        Lq = int(r.integers(1, Lkv + 1)) if causal else int(r.integers(1, 700))
        out.append((G, Hkv, B, Lq, Lkv, causal, int(r.integers(1 << 30))))
    return out


@pytest.mark.parametrize("G,Hkv,B,Lq,Lkv,causal,seed", _prefill_d64_cases())
def test_random_prefill_d64(G, Hkv, B, Lq, Lkv, causal, seed):
    print("prefill d64 G", G, "Hkv", Hkv, "B", B, "Lq", Lq, "Lkv", Lkv, "causal", causal, flush=True)
    inp = make_inputs(4, B=B, Hq=G * Hkv, Hkv=Hkv, d=64, L=Lkv, Lq=Lq, seed=seed % 100000)
    out, lse = prefill_on_gpu(inp, causal)
    ref, ref_lse = oracle_rows(inp, causal)
    assert_close(from_dev(out).reshape(-1, 64), ref, "bf16", what="random prefill d64")
    assert_lse_close(lse.cpu().numpy().astype(np.float64).ravel(), ref_lse, 2e-3)
