"""GPU parity of attn_prefill (fused causal / non-causal prefill) against the
double-precision oracle: full comparisons on shapes spanning several tiles with
ragged tails, bottom-right causal alignment with Lq < Lkv, grouped heads, and
the 16K-token causal workload on a sampled set of rows per head."""
import numpy as np
import pytest
import torch

import oracle
from _gpu import assert_close, assert_lse_close, from_dev, needs_gpu, to_dev
from datagen.workloads import make_inputs

pytestmark = [pytest.mark.gpu, needs_gpu]


def prefill_on_gpu(inp, causal, dev=None, scale=0.0):
    import long_context_decode_kv_amd as lib
    dev = dev or {k: to_dev(inp[k]) for k in ("q", "k", "v")}
    out, lse = lib.attn_prefill(dev["q"], dev["k"], dev["v"], causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return out, lse


def oracle_rows(inp, causal, rows=None, scale=None):
    prob = oracle.Problem(inp["q"], inp["k"], inp["v"], causal=causal, scale=scale)
    return oracle.attention(prob, rows=rows)


@pytest.mark.parametrize("B,Hq,Hkv,Lq,Lkv,causal", [
    (1, 8, 2, 300, 300, True),
    (2, 4, 4, 129, 129, True),
    (1, 8, 1, 200, 200, False),
    (1, 8, 2, 130, 400, True),
    (1, 4, 2, 64, 1000, False),
    (1, 16, 2, 513, 513, True),
    (1, 4, 4, 1, 77, True),
    (1, 4, 2, 257, 300, True),
    (1, 8, 2, 200, 777, False),
])
def test_prefill_small(B, Hq, Hkv, Lq, Lkv, causal):
    inp = make_inputs(4, B=B, Hq=Hq, Hkv=Hkv, L=Lkv, Lq=Lq, seed=80 + Lq + Lkv)
    out, lse = prefill_on_gpu(inp, causal)
    ref, ref_lse = oracle_rows(inp, causal)
    got = from_dev(out).reshape(-1, 128)
    res = assert_close(got, ref, "bf16", what="prefill")
    assert_lse_close(lse.cpu().numpy().astype(np.float64).ravel(), ref_lse, 2e-3)
    print("prefill %s max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % ((B, Hq, Hkv, Lq, Lkv, causal), *res), flush=True)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("Lq,Lkv,causal", [
    (1024, 1024, True),   # every workgroup walks at most 1024 keys: four-wave workgroups
    (1025, 1025, True),   # one key more: eight-wave workgroups
    (1000, 1089, True),
    (300, 1024, False),
    (300, 1025, False),
])
def test_prefill_both_workgroup_shapes(Lq, Lkv, causal, d):
    # At d = 128, launches whose workgroups walk at most 1024 keys take
    # four-wave workgroups (two per compute unit), longer ones eight-wave
    # workgroups: every row on both sides of the boundary against the oracle
    # (d = 64 always takes four-wave workgroups).
    inp = make_inputs(4, B=1, Hq=4, Hkv=2, d=d, L=Lkv, Lq=Lq, seed=7000 + Lq + Lkv + d)
    out, lse = prefill_on_gpu(inp, causal)
    ref, ref_lse = oracle_rows(inp, causal)
    res = assert_close(from_dev(out).reshape(-1, d), ref, "bf16", what="prefill")
    assert_lse_close(lse.cpu().numpy().astype(np.float64).ravel(), ref_lse, 2e-3)
    print("prefill d=%d %s max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % (d, (Lq, Lkv, causal), *res), flush=True)


def test_prefill_scale_override_and_determinism():
    inp = make_inputs(4, B=1, Hq=4, Hkv=2, L=700, seed=90)
    dev = {k: to_dev(inp[k]) for k in ("q", "k", "v")}
    o1, l1 = prefill_on_gpu(inp, True, dev=dev, scale=0.05)
    o2, l2 = prefill_on_gpu(inp, True, dev=dev, scale=0.05)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    ref, ref_lse = oracle_rows(inp, True, scale=0.05)
    assert_close(from_dev(o1).reshape(-1, 128), ref, "bf16")
    assert_lse_close(l1.cpu().numpy().astype(np.float64).ravel(), ref_lse, 2e-3)


def _sample_rows(Hq, L):
    # every head: the first 256 rows, the last 256 and 512 spread over the sequence
    per_head = np.unique(np.concatenate([np.arange(256), np.arange(L - 256, L), np.linspace(0, L - 1, 512).astype(int)]))
    return np.concatenate([h * L + per_head for h in range(Hq)]), per_head


def test_workload4_causal_16k_sampled_rows():
    inp = make_inputs(4)
    L = inp["q"].shape[2]
    out, lse = prefill_on_gpu(inp, True)
    got_all = out.view(torch.int16).cpu().numpy()
    rows, per_head = _sample_rows(32, L)
    ref, ref_lse = oracle_rows(inp, True, rows=rows)
    got = (got_all.reshape(-1, 128)[rows].astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    res = assert_close(got, ref, "bf16", what="wl4 sampled")
    assert_lse_close(lse.cpu().numpy().astype(np.float64).ravel()[rows], ref_lse, 2e-3)
    # properties at every row: finite, and each output is an average of V rows
    o = from_dev(out)
    vmax = np.abs((inp["v"].astype(np.uint32) << 16).view(np.float32)).max()
    assert np.isfinite(o).all() and np.abs(o).max() <= vmax * (1 + 1e-2)
    print("wl4 sampled rows=%d max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % (rows.size, *res), flush=True)


def test_prefill_strided_bshd_kv_and_q():
    # K/V stored [B, L, Hkv, d] (the cache layout of a running model) and Q
    # [B, Lq, Hq, d], passed as strided views; results must not depend on layout.
    B, Hq, Hkv, L = 2, 8, 2, 333
    inp = make_inputs(4, B=B, Hq=Hq, Hkv=Hkv, L=L, seed=97)
    dev = {}
    for name in ("q", "k", "v"):
        t = to_dev(inp[name])
        dev[name] = t.transpose(1, 2).contiguous().transpose(1, 2)
        assert not dev[name].is_contiguous()
    out, lse = prefill_on_gpu(inp, True, dev=dev)
    ref, ref_lse = oracle_rows(inp, True)
    assert_close(from_dev(out).reshape(-1, 128), ref, "bf16", what="strided prefill")
    assert_lse_close(lse.cpu().numpy().astype(np.float64).ravel(), ref_lse, 2e-3)


def test_prefill_repeats_are_bit_identical():
    # The K/V ring in LDS is filled asynchronously; a missing wait would show
    # up as results that change from run to run. Ten runs must agree bit for bit
    # and match the oracle on sampled rows.
    inp = make_inputs(4, B=1, Hq=32, Hkv=8, L=4096, seed=98)
    dev = {k: to_dev(inp[k]) for k in ("q", "k", "v")}
    first, first_lse = prefill_on_gpu(inp, True, dev=dev)
    for _ in range(9):
        o, l = prefill_on_gpu(inp, True, dev=dev)
        assert torch.equal(o.view(torch.int16), first.view(torch.int16)) and torch.equal(l, first_lse)
    rows, _ = _sample_rows(32, 4096)
    ref, ref_lse = oracle_rows(inp, True, rows=rows)
    got = from_dev(first).reshape(-1, 128)[rows]
    assert_close(got, ref, "bf16", what="repeats")
    assert_lse_close(first_lse.cpu().numpy().astype(np.float64).ravel()[rows], ref_lse, 2e-3)


# ------------------------------------------------------------ vector-ALU prefill (fp32, head dim 64 or 128)

@pytest.mark.parametrize("wl,B,Hq,Hkv,d,Lq,Lkv,causal,kind", [
    (1, 1, 4, 2, 128, 150, 150, True, "f32"),
    (1, 2, 2, 2, 64, 100, 230, True, "f32"),
    (1, 1, 8, 1, 64, 77, 77, False, "f32"),
])
def test_prefill_valu_path(wl, B, Hq, Hkv, d, Lq, Lkv, causal, kind):
    inp = make_inputs(wl, B=B, Hq=Hq, Hkv=Hkv, d=d, L=Lkv, Lq=Lq, seed=140 + Lq + d)
    out, lse = prefill_on_gpu(inp, causal)
    ref, ref_lse = oracle_rows(inp, causal)
    got = from_dev(out).reshape(-1, d)
    res = assert_close(got, ref, kind, what="prefill valu")
    assert_lse_close(lse.cpu().numpy().astype(np.float64).ravel(), ref_lse, 1e-5 if kind == "f32" else 2e-3)
    print("prefill valu %s max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % ((wl, B, Hq, Hkv, d, Lq, Lkv, causal), *res),
          flush=True)


def _scale_key_rows(bits, exponents):
    """bf16 K rows times 2^e per row (exact: only the exponent changes)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32) * (2.0 ** exponents).astype(np.float32)[None, None, :, None]
    return (f.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("direction", ["rising", "falling"])
def test_prefill_score_ramp(causal, direction):
    # keys of 64-key tile t scaled by 2^(t // 2) (rising: the scores' scale
    # grows up to 32x, so the running max passes the lazy headroom on tile
    # after tile and the accumulators are rescaled each time) or by
    # 2^-(t // 2) (falling: the first tile holds the max and the later
    # weights underflow towards zero)
    inp = make_inputs(4, B=1, Hq=8, Hkv=2, L=700, seed=140)
    t = np.arange(700) // 64
    inp["k"] = _scale_key_rows(inp["k"], (t // 2) if direction == "rising" else -(t // 2))
    out, lse = prefill_on_gpu(inp, causal)
    ref, ref_lse = oracle_rows(inp, causal)
    res = assert_close(from_dev(out).reshape(-1, 128), ref, "bf16", what="prefill ramp %s" % direction)
    assert_lse_close(lse.cpu().numpy().astype(np.float64).ravel(), ref_lse, 2e-3)
    print("prefill ramp %s causal %s max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % (direction, causal, *res), flush=True)


def test_prefill_sharp_softmax_and_needles():
    # Q scaled x4 (a sharp softmax), and for a few rows of every head a key
    # planted along the row's query, at or before the row, so that one key
    # dominates it
    inp = make_inputs(4, B=1, Hq=8, Hkv=2, L=600, q_mul=4.0, seed=141)
    q = (inp["q"].astype(np.uint32) << 16).view(np.float32)
    k = inp["k"].copy()
    rng = np.random.default_rng(141)
    import datagen
    for g in range(2):
        for i in rng.choice(600, size=4, replace=False):
            j = int(rng.integers(0, i + 1))
            qd = q[0, 4 * g, i]
            k[0, g, j] = datagen.f32_to_bf16_bits((2.0 * qd / np.linalg.norm(qd) * np.sqrt(128)).astype(np.float32))
    inp["k"] = k
    for causal in (True, False):
        out, lse = prefill_on_gpu(inp, causal)
        ref, ref_lse = oracle_rows(inp, causal)
        res = assert_close(from_dev(out).reshape(-1, 128), ref, "bf16", what="prefill sharp/needles")
        assert_lse_close(lse.cpu().numpy().astype(np.float64).ravel(), ref_lse, 2e-3)
        print("prefill sharp/needles causal %s max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % (causal, *res), flush=True)


# ------------------------------------------------------------ MFMA prefill at head dim 64

@pytest.mark.parametrize("B,Hq,Hkv,Lq,Lkv,causal", [
    (1, 8, 2, 300, 300, True),
    (2, 4, 4, 129, 129, True),
    (1, 8, 1, 200, 200, False),
    (1, 8, 2, 130, 400, True),
    (1, 4, 2, 64, 1000, False),
    (1, 16, 2, 513, 513, True),
    (1, 4, 4, 1, 90, True),
    (1, 6, 3, 257, 300, True),
])
def test_prefill_d64(B, Hq, Hkv, Lq, Lkv, causal):
    # the same kernel with 128-byte K/V rows: its own LDS swizzles, half the
    # score steps and output blocks, and the 8 KB output staging per wave
    inp = make_inputs(4, B=B, Hq=Hq, Hkv=Hkv, d=64, L=Lkv, Lq=Lq, seed=160 + Lq + Lkv)
    out, lse = prefill_on_gpu(inp, causal)
    ref, ref_lse = oracle_rows(inp, causal)
    res = assert_close(from_dev(out).reshape(-1, 64), ref, "bf16", what="prefill d64")
    assert_lse_close(lse.cpu().numpy().astype(np.float64).ravel(), ref_lse, 2e-3)
    print("prefill d64 %s max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % ((B, Hq, Hkv, Lq, Lkv, causal), *res), flush=True)


def test_prefill_d64_4k_sampled_rows_and_repeats():
    # 4096 tokens, 32 query / 8 KV heads, causal: sampled rows of every head
    # against the oracle, and a second call bit-identical to the first
    inp = make_inputs(4, L=4096, d=64, seed=170)
    dev = {k: to_dev(inp[k]) for k in ("q", "k", "v")}
    o1, l1 = prefill_on_gpu(inp, True, dev=dev)
    o2, l2 = prefill_on_gpu(inp, True, dev=dev)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    rows, _ = _sample_rows(32, 4096)
    ref, ref_lse = oracle_rows(inp, True, rows=rows)
    res = assert_close(from_dev(o1).reshape(-1, 64)[rows], ref, "bf16", what="prefill d64 4K")
    assert_lse_close(l1.cpu().numpy().astype(np.float64).ravel()[rows], ref_lse, 2e-3)
    print("prefill d64 4K max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % res, flush=True)
