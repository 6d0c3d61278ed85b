"""GPU parity of attn_prefill_backward (dq, dk, dv of causal or full attention)
against the oracle's backward: causal and full, Lq < Lkv alignment, grouped
heads (G = 1, 4, 8), lengths that are not multiples of the 64-row blocks, one
query row, bf16 and fp32 gradient outputs, determinism, and at the 16K-token
size element-wise parity on sampled rows and keys plus two sum invariants.

Tolerance. P and dz enter the MFMAs rounded to bf16 (relative error 2^-9 each)
and D = dO . O uses the forward's bf16 output, so each gradient element carries
a few 2^-9-relative terms that do not cancel: the bound is relative L2 error
<= 2e-2 and max |error| <= 2e-2 * max |reference| per tensor.
"""
import numpy as np
import pytest
import torch

import oracle
from _gpu import from_dev, needs_gpu, to_dev
from datagen import TID_DOUT, normal_bf16_bits
from datagen.workloads import make_inputs

pytestmark = [pytest.mark.gpu, needs_gpu]


def _run(inp, causal, grad_dtype=torch.float32, scale=0.0, seed=0):
    import long_context_decode_kv_amd as lib
    dev = {k: to_dev(inp[k]) for k in ("q", "k", "v")}
    dout_bits = normal_bf16_bits(seed, TID_DOUT, inp["q"].shape, 1.0)
    dout = to_dev(dout_bits)
    out, lse = lib.attn_prefill(dev["q"], dev["k"], dev["v"], causal=causal, softmax_scale=scale)
    dq, dk, dv = lib.attn_prefill_backward(dev["q"], dev["k"], dev["v"], out, lse, dout, causal=causal,
                                           softmax_scale=scale, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return (dq, dk, dv), dout_bits, dev, (out, lse, dout)


def _check(got, ref, what):
    got = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    scale = np.abs(ref).max()
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    msg = "%s max_abs=%.3g (ref max %.3g) rel_l2=%.3g" % (what, err.max(), scale, rel)
    print(msg, flush=True)
    assert rel <= 2e-2 and err.max() <= 2e-2 * scale, msg


@pytest.mark.parametrize("B,Hq,Hkv,Lq,Lkv,causal", [
    (1, 8, 2, 300, 300, True),
    (2, 4, 4, 129, 129, True),
    (1, 8, 1, 200, 200, False),
    (1, 8, 2, 130, 400, True),
    (1, 4, 2, 64, 1000, False),
    (1, 16, 2, 513, 513, True),
    (1, 4, 4, 1, 77, True),
])
def test_backward_small(B, Hq, Hkv, Lq, Lkv, causal):
    inp = make_inputs(4, B=B, Hq=Hq, Hkv=Hkv, L=Lkv, Lq=Lq, seed=120 + Lq + Lkv)
    (dq, dk, dv), dout_bits, _, _ = _run(inp, causal, seed=121)
    rq, rk, rv = oracle.backward(oracle.Problem(inp["q"], inp["k"], inp["v"], causal=causal), dout_bits)
    what = "bwd %s" % ((B, Hq, Hkv, Lq, Lkv, causal),)
    _check(dq, rq, what + " dq")
    _check(dk, rk, what + " dk")
    _check(dv, rv, what + " dv")


def test_backward_bf16_gradients_and_scale():
    inp = make_inputs(4, B=1, Hq=8, Hkv=2, L=700, seed=130)
    (dq, dk, dv), dout_bits, _, _ = _run(inp, True, grad_dtype=torch.bfloat16, scale=0.05, seed=131)
    assert dq.dtype == torch.bfloat16
    rq, rk, rv = oracle.backward(oracle.Problem(inp["q"], inp["k"], inp["v"], causal=True, scale=0.05), dout_bits)
    _check(dq, rq, "bwd bf16 dq")
    _check(dk, rk, "bwd bf16 dk")
    _check(dv, rv, "bwd bf16 dv")


def test_backward_1024_tokens_all_heads_and_determinism():
    import long_context_decode_kv_amd as lib
    inp = make_inputs(4, L=1024, seed=132)
    (dq, dk, dv), dout_bits, dev, (out, lse, dout) = _run(inp, True, seed=133)
    rq, rk, rv = oracle.backward(oracle.Problem(inp["q"], inp["k"], inp["v"], causal=True), dout_bits)
    _check(dq, rq, "bwd 1024 dq")
    _check(dk, rk, "bwd 1024 dk")
    _check(dv, rv, "bwd 1024 dv")
    again = lib.attn_prefill_backward(dev["q"], dev["k"], dev["v"], out, lse, dout, causal=True,
                                      grad_dtype=torch.float32)
    torch.cuda.synchronize()
    for a, b_ in zip((dq, dk, dv), again):
        assert torch.equal(a.view(torch.int32), b_.view(torch.int32))


def _row_sample(L):
    """The prefill's row sample: the first and last 256 rows and 512 rows spread between them."""
    return np.unique(np.concatenate([np.arange(256), np.arange(L - 256, L),
                                     np.linspace(256, L - 257, 512).astype(np.int64)]))


def test_backward_16k_sampled_rows_and_keys():
    # the timed size (16K causal, 32q/8kv): dq element by element on the row
    # sample of every query head, dk and dv on 512 keys of each of two KV heads
    # (the first and last 64 keys and 384 spread between), against the oracle
    # computed at those places only; then the two sum invariants over all keys
    inp = make_inputs(4)
    (dq, dk, dv), dout_bits, _, _ = _run(inp, True, seed=134)
    B, Hq, L, d = inp["q"].shape
    Hkv = inp["k"].shape[1]
    rows_i = _row_sample(L)
    q_rows = (np.arange(Hq)[:, None] * L + rows_i[None, :]).ravel()
    keys_j = np.unique(np.concatenate([np.arange(64), np.arange(L - 64, L),
                                       np.linspace(64, L - 65, 384).astype(np.int64)]))
    keys = np.concatenate([g * L + keys_j for g in (0, 5)])
    prob = oracle.Problem(inp["q"], inp["k"], inp["v"], causal=True)
    rq, rk, rv = oracle.backward_subset(prob, dout_bits, q_rows=q_rows, keys=keys)
    _check(dq.reshape(-1, d)[torch.from_numpy(q_rows).cuda()], rq, "bwd 16k dq (%d rows)" % q_rows.size)
    kidx = torch.from_numpy(keys).cuda()
    _check(dk.reshape(-1, d)[kidx], rk, "bwd 16k dk (%d keys)" % keys.size)
    _check(dv.reshape(-1, d)[kidx], rv, "bwd 16k dv (%d keys)" % keys.size)
    # each KV head's key gradients sum to zero (a row's logit gradients do),
    # and its value gradients sum to the dO of its query rows
    dk64 = dk.double().sum(dim=2)
    assert dk64.abs().max().item() <= 1e-3 * dk.double().abs().sum(dim=2).max().item()
    do = torch.from_numpy(dout_bits.view(np.int16)).view(torch.bfloat16).double()
    ref_sum = do.reshape(B, Hkv, Hq // Hkv * L, d).sum(dim=2)
    got_sum = dv.double().sum(dim=2).cpu()
    rel = (got_sum - ref_sum).norm() / ref_sum.norm()
    print("16k: dk column sums max %.3g, dv sums rel %.3g" % (dk64.abs().max().item(), rel.item()), flush=True)
    assert rel.item() <= 1e-2
    assert torch.isfinite(dq).all()


@pytest.mark.parametrize("causal", [True, False])
def test_backward_rising_score_ramp(causal):
    # keys of 64-key tile t scaled by 2^(t // 2) (scores up to 32x their usual
    # size, so each row's softmax is dominated by the latest tiles it sees):
    # P recomputed from the forward's lse, dz and the three gradients against
    # the oracle's backward
    from test_gpu_prefill import _scale_key_rows
    inp = make_inputs(4, B=1, Hq=8, Hkv=2, L=600, seed=150)
    inp["k"] = _scale_key_rows(inp["k"], (np.arange(600) // 64) // 2)
    (dq, dk, dv), dout_bits, _, _ = _run(inp, causal, seed=151)
    rq, rk, rv = oracle.backward(oracle.Problem(inp["q"], inp["k"], inp["v"], causal=causal), dout_bits)
    what = "bwd ramp causal %s" % causal
    _check(dq, rq, what + " dq")
    _check(dk, rk, what + " dk")
    _check(dv, rv, what + " dv")
