"""GPU parity of attn_decode_mixed_fp4 (a cache with the first and last tenth
of the tokens in bf16 and the rest in OCP MX fp4, the ThriftAttention page's
FP4 on this hardware) against the oracle's attention over the union of both
spans at their decoded values: small shapes with several tiles and ragged
tails, per-head ragged lengths with empty spans, both merge paths, every E2M1
code and a wide range of E8M0 scales, either span absent, strided views, the
full 128K-token workload (also with per-head ragged lengths), and
bit-identical repeats."""
import numpy as np
import pytest
import torch

from _gpu import assert_close, assert_lse_close, from_dev, mixed_fp4_on_gpu, needs_gpu, oracle_mixed, to_dev
from datagen.workloads import make_mixed_inputs

pytestmark = [pytest.mark.gpu, needs_gpu]


def _dev(inp):
    return {k: to_dev(v) for k, v in inp.items() if k != "lo_format"}


def _check(inp, S_hi=0, S_lo=0, what="", dev=None):
    out, lse = mixed_fp4_on_gpu(inp, S_hi, S_lo, dev=dev)
    ref, ref_lse = oracle_mixed(inp)
    res = assert_close(from_dev(out)[:, :, 0, :], ref, "bf16", what="%s S=(%d,%d)" % (what, S_hi, S_lo))
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, 2e-3)
    print("%s S=(%d,%d) max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % (what, S_hi, S_lo, *res), flush=True)
    return out, lse


@pytest.mark.parametrize("S_hi,S_lo", [(1, 1), (2, 5), (3, 7), (0, 0), (10, 38)])
def test_mixed_fp4_small(S_hi, S_lo):
    # L_hi = 600, L_lo = 2400: several 64-key tiles per split and ragged tails
    inp = make_mixed_inputs(9, B=2, Hq=8, Hkv=2, L=3000, seed=90)
    _check(inp, S_hi, S_lo, what="fp4 L=3000")


@pytest.mark.parametrize("G", [1, 8])
def test_mixed_fp4_other_head_ratios(G):
    inp = make_mixed_inputs(9, B=2, Hq=2 * G, Hkv=2, L=3000, seed=98 + G)
    _check(inp, 3, 7, what="mixed fp4 G=%d" % G)


def test_mixed_fp4_per_head_ragged_lengths_and_empty_spans():
    inp = make_mixed_inputs(9, B=3, Hq=8, Hkv=2, L=4000, lens=(0.0, 1.0), seed=91)
    inp["hi_lens"][0] = 0  # a head with fp4 keys only
    inp["lo_lens"][1] = 0  # a head with bf16 keys only
    inp["hi_lens"][2] = inp["lo_lens"][2] = 0  # a head with no key at all
    inp["lo_lens"][3] = 17  # a ragged tail inside one tile
    out, lse = _check(inp, 4, 9, what="fp4 ragged")
    o = from_dev(out)
    assert np.all(o[1, 0:4] == 0) and np.all(np.isneginf(lse.cpu().numpy()[1, 0:4]))


def test_mixed_fp4_fused_and_separate_merge():
    # 4 (sequence, KV head) groups: 2 + 5 splits merge inside the decode
    # kernel; 100 + 100 and 200 + 300 in the second kernel
    inp = make_mixed_inputs(9, B=2, Hq=8, Hkv=2, L_hi=12800, L_lo=38400, lens=(0.3, 1.0), seed=92)
    dev = _dev(inp)
    for S_hi, S_lo in ((2, 5), (100, 100), (200, 300)):
        _check(inp, S_hi, S_lo, what="fp4 merge", dev=dev)


def test_mixed_fp4_every_code_and_wide_scales():
    # every E2M1 code in K and V, block scales 2^-20 .. 2^3 for K and
    # 2^-17 .. 2^-3 for V (so the output stays of order 1)
    inp = make_mixed_inputs(9, B=1, Hq=8, Hkv=2, L_hi=64, L_lo=1024, seed=93)
    n = inp["k_lo"].size
    inp["k_lo"] = (np.arange(n, dtype=np.int64) * 37 % 256).astype(np.uint8).reshape(inp["k_lo"].shape)
    inp["v_lo"] = (np.arange(n, dtype=np.int64) * 91 % 256).astype(np.uint8).reshape(inp["v_lo"].shape)
    m = inp["k_scale"].size
    inp["k_scale"] = (107 + np.arange(m) % 24).astype(np.uint8).reshape(inp["k_scale"].shape)   # 2^-20 .. 2^3
    inp["v_scale"] = (110 + np.arange(m) * 7 % 15).astype(np.uint8).reshape(inp["v_scale"].shape)  # 2^-17 .. 2^-3
    _check(inp, 1, 5, what="fp4 all codes")


def test_mixed_fp4_without_fp4_span_matches_bf16_decode():
    import long_context_decode_kv_amd as lib
    inp = make_mixed_inputs(9, B=1, Hq=8, Hkv=2, L_hi=2048, L_lo=0, seed=94)
    assert inp["k_lo"] is None
    out, lse = _check(inp, 3, 0, what="fp4 bf16 only")
    dev = _dev(inp)
    ref_out, ref_lse = lib.attn_decode(dev["q"], dev["k_hi"], dev["v_hi"], num_splits=3)
    assert (out.float() - ref_out.float()).abs().max().item() <= 2 ** -7
    assert (lse - ref_lse).abs().max().item() <= 1e-5


def test_mixed_fp4_without_bf16_span():
    inp = make_mixed_inputs(9, B=2, Hq=8, Hkv=2, L_hi=0, L_lo=3000, seed=95)
    assert inp["k_hi"] is None
    _check(inp, 0, 6, what="fp4 only")


def test_mixed_fp4_strided_views():
    # codes and scales as slices of larger tensors ([B, L, Hkv, .] storage)
    import long_context_decode_kv_amd as lib
    inp = make_mixed_inputs(9, B=2, Hq=8, Hkv=2, L=2000, seed=96)
    dev = _dev(inp)
    big = lambda t, w: torch.zeros((t.shape[0], t.shape[2], t.shape[1], w), dtype=t.dtype, device=t.device)
    views = {}
    for name, width in (("k_lo", 80), ("v_lo", 96), ("k_scale", 8), ("v_scale", 12)):
        t = dev[name]
        store = big(t, width)
        store[..., :t.shape[3]] = t.permute(0, 2, 1, 3)
        views[name] = store.permute(0, 2, 1, 3)[..., :t.shape[3]]
    out, lse = lib.attn_decode_mixed_fp4(dev["q"], dev["k_hi"], dev["v_hi"], views["k_lo"], views["v_lo"],
                                         k_lo_scale=views["k_scale"], v_lo_scale=views["v_scale"], num_splits_hi=2,
                                         num_splits_lo=5)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_mixed(inp)
    assert_close(from_dev(out)[:, :, 0, :], ref, "bf16", what="fp4 strided")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, 2e-3)


def test_workload9_full_size_auto_plan_and_repeats():
    import long_context_decode_kv_amd as lib
    inp = make_mixed_inputs(9)
    dev = _dev(inp)
    outs = [mixed_fp4_on_gpu(inp, dev=dev) for _ in range(2)]
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))
    B, Hq = inp["q"].shape[:2]
    heads = np.arange(B * Hq)
    ref, ref_lse = oracle_mixed(inp, heads=heads)
    res = assert_close(from_dev(outs[0][0]).reshape(B * Hq, -1), ref, "bf16", what="wl9 auto")
    assert_lse_close(outs[0][1].cpu().numpy().astype(np.float64).ravel(), ref_lse, 2e-3)
    print("wl9 auto %s max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % (lib.attn_decode_mixed_fp4_splits(1, 8, 26214 * 1, 104858), *res), flush=True)
    out2, _ = mixed_fp4_on_gpu(inp, 64, 128, dev=dev)
    assert_close(from_dev(out2).reshape(B * Hq, -1), ref, "bf16", what="wl9 64+128")


def test_workload9_full_size_ragged_heads():
    # each (sequence, KV head) keeps between half and all of each span's capacity
    inp = make_mixed_inputs(9, lens=(0.5, 1.0))
    assert inp["hi_lens"].min() < inp["hi_lens"].max() and inp["lo_lens"].min() < inp["lo_lens"].max()
    _check(inp, 0, 0, what="wl9 ragged")


def test_mixed_fp4_scale_extremes_and_nan_scale():
    # E8M0 bytes at the low end (1, 2: 2^-126, 2^-125) in K and V blocks, and
    # 140 (2^13) in V blocks: all exact in fp32. Byte 255 is NaN: the V block
    # that carries it makes its 32 output dims NaN for the heads of that KV
    # group, in the kernel as in the definition, and leaves the rest finite.
    inp = make_mixed_inputs(9, B=1, Hq=8, Hkv=2, L_hi=128, L_lo=1000, seed=97)
    ks, vs = inp["k_scale"], inp["v_scale"]
    ks[0, 0, 0:300:3, 1] = 1
    ks[0, 1, 5:200:7, 2] = 2
    vs[0, 0, 10:400:5, 0] = 1
    vs[0, 1, 3:900:11, 3] = 140
    vs[0, 1, 123, 2] = 255  # NaN scale: dims 64..95 of KV head 1
    out, lse = mixed_fp4_on_gpu(inp, 2, 5)
    ref, ref_lse = oracle_mixed(inp)
    got = from_dev(out)[:, :, 0, :]
    nan_ref = np.isnan(ref)
    assert nan_ref[0, 4:8, 64:96].all() and nan_ref.sum() == 4 * 32
    assert np.array_equal(np.isnan(got), nan_ref)
    fin = ~nan_ref
    err = np.abs(got[fin] - ref[fin])
    rel = np.linalg.norm(got[fin] - ref[fin]) / np.linalg.norm(ref[fin])
    print("fp4 scale extremes max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % (err.max(), err.mean(), rel), flush=True)
    assert err.max() <= 2e-2 * max(1.0, np.abs(ref[fin]).max()) and rel <= 1e-2
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, 2e-3)
