"""GPU parity of attn_prefill_pi (pi-Attention prefill: the ring-local window,
the periodic skip keys of each residue class as strided views, and the alpha
log-prior, merged per row; causal, and two-sided with keys on both sides)
against the oracle's masked definition: window / period combinations on
lengths that are multiples of neither the tile nor the period, alpha 0 and 1,
skip sets that are empty for every row, period 1 (every key), strided BSHD
views, and the 16K-token cache on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
from _gpu import assert_close, assert_lse_close, from_dev, needs_gpu, to_dev
from datagen.workloads import make_inputs

pytestmark = [pytest.mark.gpu, needs_gpu]


def pi_prefill_on_gpu(inp, window, period, alpha=None, dev=None, causal=True):
    import long_context_decode_kv_amd as lib
    dev = dev or {k: to_dev(inp[k]) for k in ("q", "k", "v")}
    a = None if alpha is None else torch.from_numpy(np.ascontiguousarray(alpha, np.float32)).cuda()
    out, lse = lib.attn_prefill_pi(dev["q"], dev["k"], dev["v"], window, period, alpha=a, causal=causal)
    torch.cuda.synchronize()
    return out, lse


def oracle_pi_rows(inp, window, period, alpha=None, rows=None, causal=True):
    prob = oracle.Problem(inp["q"], inp["k"], inp["v"], causal=causal)
    return oracle.pi_attention(prob, window, period, alpha, rows=rows)


def _check(inp, window, period, alpha, what, dev=None, rows=None, causal=True):
    out, lse = pi_prefill_on_gpu(inp, window, period, alpha, dev=dev, causal=causal)
    ref, ref_lse = oracle_pi_rows(inp, window, period, alpha, rows=rows, causal=causal)
    got = from_dev(out).reshape(-1, inp["q"].shape[-1])
    gl = lse.cpu().numpy().astype(np.float64).ravel()
    if rows is not None:
        got, gl = got[rows], gl[rows]
    res = assert_close(got, ref, "bf16", what="%s w=%d pi=%d" % (what, window, period))
    assert_lse_close(gl, ref_lse, 2e-3)
    print("%s w=%d pi=%d max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % (what, window, period, *res), flush=True)
    return out, lse


@pytest.mark.parametrize("window,period", [(128, 16), (0, 3), (300, 1), (999, 5), (64, 0), (100, 7), (37, 200)])
@pytest.mark.parametrize("with_alpha", [False, True])
def test_pi_prefill_small(window, period, with_alpha):
    B, Hq, Hkv, L = 2, 8, 2, 1000
    inp = make_inputs(4, B=B, Hq=Hq, Hkv=Hkv, L=L, seed=100 + window + period)
    alpha = np.random.default_rng(101).uniform(0.05, 0.95, size=(B, Hq, L)).astype(np.float32) if with_alpha else None
    _check(inp, window, period, alpha, "pi prefill")


def test_pi_prefill_alpha_extremes_and_empty_rows():
    B, Hq, Hkv, L = 1, 4, 1, 700
    inp = make_inputs(4, B=B, Hq=Hq, Hkv=Hkv, L=L, seed=102)
    alpha = np.full((B, Hq, L), 0.5, np.float32)
    alpha[0, 0] = 1.0  # head 0: window only
    alpha[0, 1] = 0.0  # head 1: skip keys only; rows below 56 have none -> empty
    out, lse = _check(inp, 50, 8, alpha, "pi prefill alpha 0/1")
    l = lse.cpu().numpy()
    # the first skip key of position i is i - 56 (7 periods of 8 clear the window of 50)
    assert np.all(np.isneginf(l[0, 1, :56])) and np.all(np.isfinite(l[0, 1, 56:]))
    assert np.all(from_dev(out)[0, 1, :56] == 0)


def test_pi_prefill_period_one_window_zero_is_causal_prefill():
    import long_context_decode_kv_amd as lib
    inp = make_inputs(4, B=1, Hq=8, Hkv=2, L=777, seed=103)
    dev = {k: to_dev(inp[k]) for k in ("q", "k", "v")}
    out, lse = pi_prefill_on_gpu(inp, 0, 1, dev=dev)
    ref_out, ref_lse = lib.attn_prefill(dev["q"], dev["k"], dev["v"], causal=True)
    torch.cuda.synchronize()
    # two bf16 parts merged vs one pass: agree to bf16 rounding
    assert (out.float() - ref_out.float()).abs().max().item() < 2e-2
    assert (lse - ref_lse).abs().max().item() < 1e-3


def test_pi_prefill_strided_bshd_views():
    B, Hq, Hkv, L = 1, 8, 2, 600
    inp = make_inputs(4, B=B, Hq=Hq, Hkv=Hkv, L=L, seed=104)
    dev = {}
    for name in ("q", "k", "v"):
        t = to_dev(inp[name])
        bshd = torch.empty((t.shape[0], t.shape[2], t.shape[1], t.shape[3]), dtype=t.dtype, device=t.device)
        bshd.copy_(t.permute(0, 2, 1, 3))
        dev[name] = bshd.permute(0, 2, 1, 3)
    _check(inp, 90, 6, None, "pi prefill bshd", dev=dev)


def test_pi_prefill_medium():
    inp = make_inputs(4, B=1, Hq=32, Hkv=8, L=5000, seed=105)
    alpha = np.random.default_rng(106).uniform(0.05, 0.95, size=(1, 32, 5000)).astype(np.float32)
    _check(inp, 512, 64, alpha, "pi prefill 5000")


def test_pi_prefill_16k_sampled_rows():
    inp = make_inputs(4)
    B, Hq, L = 1, 32, 16384
    alpha = np.random.default_rng(107).uniform(0.05, 0.95, size=(B, Hq, L)).astype(np.float32)
    per_head = np.unique(np.concatenate([np.arange(64), np.arange(L - 64, L), np.linspace(0, L - 1, 64).astype(int)]))
    rows = np.concatenate([h * L + per_head for h in (0, 5, 17, 31)])
    _check(inp, 512, 64, alpha, "pi prefill 16K", rows=rows)


# ---------------------------------------------------------------- two-sided
# Keys on both sides of the query: the window i - w .. i + w, skip keys
# i +- m * period outside it (the page's bidirectional case).

@pytest.mark.parametrize("window,period", [(128, 16), (0, 3), (300, 1), (999, 5), (64, 0), (100, 7), (37, 200),
                                           (450, 64)])
@pytest.mark.parametrize("with_alpha", [False, True])
def test_pi_prefill_two_sided_small(window, period, with_alpha):
    B, Hq, Hkv, L = 2, 8, 2, 1000
    inp = make_inputs(4, B=B, Hq=Hq, Hkv=Hkv, L=L, seed=200 + window + period)
    alpha = np.random.default_rng(201).uniform(0.05, 0.95, size=(B, Hq, L)).astype(np.float32) if with_alpha else None
    _check(inp, window, period, alpha, "pi prefill two-sided", causal=False)


def test_pi_prefill_two_sided_alpha_extremes():
    B, Hq, Hkv, L = 1, 4, 1, 700
    inp = make_inputs(4, B=B, Hq=Hq, Hkv=Hkv, L=L, seed=202)
    alpha = np.full((B, Hq, L), 0.5, np.float32)
    alpha[0, 0] = 1.0  # head 0: the window only
    alpha[0, 1] = 0.0  # head 1: the skip keys only, on both sides
    out, lse = _check(inp, 50, 8, alpha, "pi prefill two-sided alpha 0/1", causal=False)
    assert np.all(np.isfinite(lse.cpu().numpy()))


def test_pi_prefill_two_sided_period_one_is_full_prefill():
    import long_context_decode_kv_amd as lib
    inp = make_inputs(4, B=1, Hq=8, Hkv=2, L=777, seed=203)
    dev = {k: to_dev(inp[k]) for k in ("q", "k", "v")}
    out, lse = pi_prefill_on_gpu(inp, 10, 1, dev=dev, causal=False)
    ref_out, ref_lse = lib.attn_prefill(dev["q"], dev["k"], dev["v"], causal=False)
    torch.cuda.synchronize()
    assert (out.float() - ref_out.float()).abs().max().item() < 2e-2
    assert (lse - ref_lse).abs().max().item() < 1e-3


def test_pi_prefill_two_sided_16k_sampled_rows():
    inp = make_inputs(4)
    B, Hq, L = 1, 32, 16384
    alpha = np.random.default_rng(204).uniform(0.05, 0.95, size=(B, Hq, L)).astype(np.float32)
    per_head = np.unique(np.concatenate([np.arange(64), np.arange(L - 64, L), np.linspace(0, L - 1, 64).astype(int)]))
    rows = np.concatenate([h * L + per_head for h in (0, 5, 17, 31)])
    _check(inp, 512, 64, alpha, "pi prefill two-sided 16K", rows=rows, causal=False)


@pytest.mark.parametrize("causal", [True, False])
def test_pi_prefill_rising_score_ramp(causal):
    # keys of 64-key tile t scaled by 2^(t // 2): the banded kernel's running
    # max passes its lazy headroom on tile after tile, in the window launch
    # and in the strided skip-class launches
    from test_gpu_prefill import _scale_key_rows
    inp = make_inputs(4, B=1, Hq=8, Hkv=2, L=700, seed=142)
    inp["k"] = _scale_key_rows(inp["k"], (np.arange(700) // 64) // 2)
    alpha = np.random.default_rng(142).uniform(0.0, 1.0, size=(1, 8, 700)).astype(np.float32)
    _check(inp, 100, 16, alpha, "pi ramp causal %s" % causal, causal=causal)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window,period", [(128, 16), (37, 5), (0, 1)])
def test_pi_prefill_d64(window, period, causal):
    # head dim 64 through the same window and skip-class launches
    inp = make_inputs(4, B=1, Hq=8, Hkv=2, d=64, L=700, seed=180 + window + period)
    alpha = np.random.default_rng(180).uniform(0.0, 1.0, size=(1, 8, 700)).astype(np.float32)
    _check(inp, window, period, alpha, "pi d64 causal %s" % causal, causal=causal)


@pytest.mark.parametrize("window,causal", [(960, True), (961, True), (470, False), (500, False)])
def test_pi_prefill_window_launch_both_workgroup_shapes(window, causal):
    # The window launch takes four-wave workgroups while a workgroup walks at
    # most 1024 keys (window + 64 <= 1024 causal; two-sided the band is
    # 2 window + 1 keys) and eight-wave workgroups past that; the skip-class
    # launches (94 rows a class here) take four-wave workgroups. Every row.
    inp = make_inputs(4, B=1, Hq=4, Hkv=2, L=1500, seed=7100 + window)
    alpha = np.random.default_rng(window).uniform(0.0, 1.0, size=(1, 4, 1500))
    _check(inp, window, 16, alpha, "pi prefill boundary", causal=causal)

