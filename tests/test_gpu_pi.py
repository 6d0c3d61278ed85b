"""GPU parity of attn_decode_pi (the pi-Attention explainer's ring-local window,
periodic skip keys and alpha log-prior, as one decode launch over two spans of
the same cache) against the oracle's masked definition: window and period
combinations that leave the skip set empty, sparse or total, with and without
the prior (including alpha = 0 and 1), ragged lengths shorter than the window,
fp8 caches, both merge paths, and the 128K-key cache."""
import numpy as np
import pytest

from _gpu import assert_close, assert_lse_close, from_dev, needs_gpu, oracle_pi, pi_on_gpu, to_dev
from datagen.workloads import make_inputs

pytestmark = [pytest.mark.gpu, needs_gpu]


def _alpha(B, Hq, seed):
    return np.random.default_rng(seed).uniform(0.05, 0.95, size=(B, Hq, 1)).astype(np.float32)


def _check(inp, window, period, alpha, sw=0, ss=0, what="", dev=None, kind="bf16"):
    out, lse = pi_on_gpu(inp, window, period, alpha, sw, ss, dev=dev)
    ref, ref_lse = oracle_pi(inp, window, period, alpha)
    got = from_dev(out)[:, :, 0, :]
    res = assert_close(got, ref, kind, what="%s w=%d pi=%d S=(%d,%d)" % (what, window, period, sw, ss))
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, 2e-3)
    print("%s w=%d pi=%d S=(%d,%d) max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % (what, window, period, sw, ss, *res),
          flush=True)
    return out, lse


@pytest.mark.parametrize("window,period", [(256, 64), (0, 7), (100, 1), (2999, 3), (50, 0), (640, 13)])
@pytest.mark.parametrize("with_alpha", [False, True])
def test_pi_small(window, period, with_alpha):
    inp = make_inputs(2, B=2, Hq=8, Hkv=2, L=3000, seed=70)
    alpha = _alpha(2, 8, 71) if with_alpha else None
    _check(inp, window, period, alpha, what="pi")


@pytest.mark.parametrize("sw,ss", [(1, 1), (3, 5), (1, 40)])
def test_pi_split_counts(sw, ss):
    inp = make_inputs(2, B=1, Hq=8, Hkv=2, L=5000, seed=72)
    _check(inp, 700, 9, _alpha(1, 8, 73), sw, ss, what="pi splits")


def test_pi_ragged_lengths_below_and_above_the_window():
    inp = make_inputs(2, B=6, Hq=8, Hkv=2, L=4000, seed=74)
    inp["kv_lens"] = np.array([0, 1, 2, 300, 1537, 4000], np.int32)
    alpha = _alpha(6, 8, 75)
    alpha[2, 0, 0] = 1.0  # skip keys weighted zero
    alpha[3, 1, 0] = 0.0  # window weighted zero
    alpha[1, 2, 0] = 0.0  # one key, in the window, weighted zero: empty row
    out, lse = _check(inp, 500, 16, alpha, what="pi ragged")
    assert np.all(from_dev(out)[0] == 0) and np.all(np.isneginf(lse.cpu().numpy()[0]))
    assert np.isneginf(lse.cpu().numpy()[1, 2])


@pytest.mark.parametrize("G,kv", [(1, "bf16"), (8, "bf16"), (2, "e4m3")])
def test_pi_other_head_ratios(G, kv):
    inp = make_inputs(2 if kv == "bf16" else 5, B=2, Hq=2 * G, Hkv=2, L=3000, seed=78 + G)
    _check(inp, 256, 16, _alpha(2, 2 * G, 79 + G), what="pi G=%d %s" % (G, kv), kind=kv)


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_pi_head_dim_64(kv):
    inp = make_inputs(2 if kv == "bf16" else 5, B=2, Hq=8, Hkv=2, d=64, L=3000, seed=88)
    _check(inp, 256, 16, _alpha(2, 8, 89), what="pi d=64 %s" % kv, kind=kv)


def test_pi_fp8_cache():
    inp = make_inputs(5, B=2, Hq=8, Hkv=2, L=6000, seed=76)
    _check(inp, 1024, 32, _alpha(2, 8, 77), what="pi fp8", kind="e4m3")


def test_pi_separate_merge_path():
    # 2 sequences x 8 KV heads x (60 + 90) splits: more workgroups than stay
    # resident, so the merge runs as its own kernel
    inp = make_inputs(2, B=2, Hq=32, Hkv=8, L=40000, seed=78)
    _check(inp, 15000, 3, _alpha(2, 32, 79), 60, 90, what="pi separate merge")


def test_pi_full_size_cache():
    inp = make_inputs(2)
    dev = {k: to_dev(v) for k, v in inp.items()}
    alpha = _alpha(1, 32, 80)
    out1, lse1 = _check(inp, 4096, 64, alpha, what="pi 128K", dev=dev)
    out2, lse2 = pi_on_gpu(inp, 4096, 64, alpha, dev=dev)
    import torch
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32))
    _check(inp, 16384, 8, None, what="pi 128K dense skips", dev=dev)
