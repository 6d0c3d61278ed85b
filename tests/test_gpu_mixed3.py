"""GPU parity of attn_decode_mixed3 (a cache kept in bf16, fp8-e4m3 and OCP MX
fp4 at once: the ThriftAttention page's three precisions in one kernel)
against the oracle's attention over the union of the three spans at their
decoded values: split triples with several tiles and ragged tails, per-head
ragged lengths with empty spans and an empty head, both merge paths, each span
absent, equality with the two-precision entry points when one span is empty,
and the full 128K-token workload with bit-identical repeats."""
import numpy as np
import pytest
import torch

import oracle
from _gpu import assert_close, assert_lse_close, from_dev, needs_gpu, to_dev
from datagen.workloads import make_mixed3_inputs, mixed3_spans

pytestmark = [pytest.mark.gpu, needs_gpu]


def _dev(inp):
    return {k: to_dev(v) for k, v in inp.items()}


def _run(inp, S=(0, 0, 0), dev=None):
    import long_context_decode_kv_amd as lib
    dev = dev or _dev(inp)
    out, lse = lib.attn_decode_mixed3(dev["q"], dev["k_hi"], dev["v_hi"], dev["k_mid"], dev["v_mid"], dev["k_lo"],
                                      dev["v_lo"], k_mid_scale=dev["k_mid_scale"], v_mid_scale=dev["v_mid_scale"],
                                      k_lo_scale=dev["k_lo_scale"], v_lo_scale=dev["v_lo_scale"],
                                      hi_lens=dev["hi_lens"], mid_lens=dev["mid_lens"], lo_lens=dev["lo_lens"],
                                      num_splits_hi=S[0], num_splits_mid=S[1], num_splits_lo=S[2])
    torch.cuda.synchronize()
    return out, lse


def _check(inp, S=(0, 0, 0), what="", dev=None):
    out, lse = _run(inp, S, dev)
    ref, ref_lse = oracle.decode_spans(inp["q"], mixed3_spans(inp))
    B, Hq = inp["q"].shape[:2]
    res = assert_close(from_dev(out).reshape(B * Hq, -1), ref, "bf16", what="%s S=%s" % (what, S))
    assert_lse_close(lse.cpu().numpy().astype(np.float64).ravel(), ref_lse, 2e-3)
    print("%s S=%s max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % (what, S, *res), flush=True)
    return out, lse


@pytest.mark.parametrize("S", [(1, 1, 1), (2, 3, 5), (3, 1, 7), (0, 0, 0), (6, 6, 20)])
def test_mixed3_small(S):
    # 600 bf16, 600 fp8 and 1800 fp4 keys: several tiles per split and ragged tails
    inp = make_mixed3_inputs(B=2, Hq=8, Hkv=2, L=3000, seed=100)
    _check(inp, S, what="mixed3 L=3000")


@pytest.mark.parametrize("G", [2, 8])
def test_mixed3_other_head_ratios(G):
    inp = make_mixed3_inputs(B=2, Hq=2 * G, Hkv=2, L=3000, seed=104 + G)
    _check(inp, (2, 2, 4), what="mixed3 G=%d" % G)


def test_mixed3_per_head_ragged_lengths_and_empty_spans():
    inp = make_mixed3_inputs(B=3, Hq=8, Hkv=2, L=5000, lens=(0.0, 1.0), seed=101)
    inp["hi_lens"][0] = 0                     # no bf16 key
    inp["mid_lens"][1] = inp["lo_lens"][1] = 0  # bf16 keys only
    inp["hi_lens"][2] = inp["mid_lens"][2] = inp["lo_lens"][2] = 0  # no key at all
    inp["lo_lens"][3] = 17                    # a ragged tail inside one fp4 tile
    inp["mid_lens"][4] = 1
    out, lse = _check(inp, (2, 3, 4), what="mixed3 ragged")
    o = from_dev(out)
    assert np.all(o[1, 0:4] == 0) and np.all(np.isneginf(lse.cpu().numpy()[1, 0:4]))


def test_mixed3_fused_and_separate_merge():
    # 4 (sequence, KV head) groups: 2 + 3 + 5 splits merge inside the decode
    # kernel; 60 + 60 + 100 in the second kernel
    inp = make_mixed3_inputs(B=2, Hq=8, Hkv=2, L_hi=12800, L_mid=12800, L_lo=38400, lens=(0.3, 1.0), seed=102)
    dev = _dev(inp)
    for S in ((2, 3, 5), (60, 60, 100)):
        _check(inp, S, what="mixed3 merge", dev=dev)


@pytest.mark.parametrize("absent", ["hi", "mid", "lo"])
def test_mixed3_with_one_span_absent(absent):
    caps = dict(L_hi=700, L_mid=900, L_lo=1500)
    caps["L_" + absent] = 0
    inp = make_mixed3_inputs(B=1, Hq=8, Hkv=2, seed=103, **caps)
    _check(inp, (2, 2, 3), what="mixed3 without %s" % absent)


def test_mixed3_with_empty_fp8_span_equals_the_bf16_fp4_decode():
    # same split plan and the same workgroup order: the same kernels' bits
    import long_context_decode_kv_amd as lib
    inp = make_mixed3_inputs(B=2, Hq=8, Hkv=2, L_hi=900, L_mid=0, L_lo=3000, seed=104)
    dev = _dev(inp)
    out, lse = _run(inp, (3, 0, 7), dev)
    ref, ref_lse = lib.attn_decode_mixed_fp4(dev["q"], dev["k_hi"], dev["v_hi"], dev["k_lo"], dev["v_lo"],
                                             k_lo_scale=dev["k_lo_scale"], v_lo_scale=dev["v_lo_scale"],
                                             num_splits_hi=3, num_splits_lo=7)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))


def test_workload10_full_size_auto_plan_and_repeats():
    import long_context_decode_kv_amd as lib
    inp = make_mixed3_inputs()
    dev = _dev(inp)
    outs = [_run(inp, dev=dev) for _ in range(2)]
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))
    ref, ref_lse = oracle.decode_spans(inp["q"], mixed3_spans(inp))
    res = assert_close(from_dev(outs[0][0]).reshape(32, -1), ref, "bf16", what="wl10 auto")
    assert_lse_close(outs[0][1].cpu().numpy().astype(np.float64).ravel(), ref_lse, 2e-3)
    caps = [inp[k].shape[2] for k in ("k_hi", "k_mid", "k_lo")]
    print("wl10 auto %s max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % (lib.attn_decode_mixed3_splits(1, 8, *caps), *res),
          flush=True)
    out2, _ = _run(inp, (16, 24, 88), dev)
    assert_close(from_dev(out2).reshape(32, -1), ref, "bf16", what="wl10 16+24+88")
