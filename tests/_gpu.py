"""Helpers shared by the GPU parity tests: device upload of the seeded inputs,
calls through the C ABI (via the thin binding) and the tolerance checks.

Tolerances: fp32 inputs, max |err| <= 1e-5; bf16 / fp8 inputs, max |err| <=
2e-2 and mean |err| <= 2e-3, plus a relative L2 bound of 1e-2, because with
nearly uniform softmax weights the outputs are small enough that an all-zero
answer would pass the absolute bounds alone.
"""
import numpy as np
import pytest
import torch

import oracle

HAS_GPU = torch.cuda.is_available()
needs_gpu = pytest.mark.skipif(not HAS_GPU, reason="no GPU")


def to_dev(x):
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def from_dev(t):
    return t.float().cpu().numpy().astype(np.float64)


def decode_on_gpu(inp, num_splits=0, causal=False, softmax_scale=0.0, dev=None):
    import long_context_decode_kv_amd as lib
    dev = dev or {k: to_dev(v) for k, v in inp.items()}
    out, lse = lib.attn_decode(dev["q"], dev["k"], dev["v"], k_scale=dev.get("k_scale"),
                               v_scale=dev.get("v_scale"), kv_lens=dev.get("kv_lens"),
                               softmax_scale=softmax_scale, causal=causal, num_splits=num_splits)
    torch.cuda.synchronize()
    return out, lse


def oracle_decode(inp, causal=False, scale=None):
    prob = oracle.Problem(inp["q"], inp["k"], inp["v"], k_scale=inp.get("k_scale"), v_scale=inp.get("v_scale"),
                          kv_lens=inp.get("kv_lens"), scale=scale, causal=causal)
    out, lse = oracle.attention(prob)
    B, Hq = inp["q"].shape[:2]
    return out.reshape(B, Hq, -1), lse.reshape(B, Hq)


def errors(got, ref):
    err = np.abs(got - ref)
    den = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / den if den > 0 else np.linalg.norm(got - ref)
    return float(err.max()), float(err.mean()), float(rel)


def assert_close(got, ref, kind, what=""):
    mx, mean, rel = errors(got, ref)
    msg = "%s max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % (what, mx, mean, rel)
    if kind == "f32":
        assert mx <= 1e-5, msg
    else:
        assert mx <= 2e-2 and mean <= 2e-3 and rel <= 1e-2, msg
    return mx, mean, rel


def assert_lse_close(got, ref, tol):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), "lse finiteness differs"
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "-inf lse differs"
    if fin.any():
        assert np.abs(got[fin] - ref[fin]).max() <= tol, np.abs(got[fin] - ref[fin]).max()


def mixed_on_gpu(inp, num_splits_hi=0, num_splits_lo=0, dev=None, softmax_scale=0.0):
    import long_context_decode_kv_amd as lib
    dev = dev or {k: to_dev(v) for k, v in inp.items()}
    out, lse = lib.attn_decode_mixed(dev["q"], dev["k_hi"], dev["v_hi"], dev["k_lo"], dev["v_lo"],
                                     k_scale=dev["k_scale"], v_scale=dev["v_scale"], hi_lens=dev["hi_lens"],
                                     lo_lens=dev["lo_lens"], softmax_scale=softmax_scale,
                                     num_splits_hi=num_splits_hi, num_splits_lo=num_splits_lo)
    torch.cuda.synchronize()
    return out, lse


def mixed_fp4_on_gpu(inp, num_splits_hi=0, num_splits_lo=0, dev=None):
    import long_context_decode_kv_amd as lib
    dev = dev or {k: to_dev(v) for k, v in inp.items() if k != "lo_format"}
    out, lse = lib.attn_decode_mixed_fp4(dev["q"], dev["k_hi"], dev["v_hi"], dev["k_lo"], dev["v_lo"],
                                         k_lo_scale=dev["k_scale"], v_lo_scale=dev["v_scale"], hi_lens=dev["hi_lens"],
                                         lo_lens=dev["lo_lens"], num_splits_hi=num_splits_hi,
                                         num_splits_lo=num_splits_lo)
    torch.cuda.synchronize()
    return out, lse


def oracle_mixed(inp, heads=None, scale=None):
    out, lse = oracle.decode_mixed(inp["q"], inp["k_hi"], inp["v_hi"], inp["k_lo"], inp["v_lo"], inp["k_scale"],
                                   inp["v_scale"], inp["hi_lens"], inp["lo_lens"], scale=scale, heads=heads,
                                   lo_format=inp.get("lo_format", "e4m3"))
    if heads is not None:
        return out, lse
    B, Hq = inp["q"].shape[:2]
    return out.reshape(B, Hq, -1), lse.reshape(B, Hq)


def pi_on_gpu(inp, window, period, alpha=None, num_splits_window=0, num_splits_skip=0, dev=None):
    import long_context_decode_kv_amd as lib
    dev = dev or {k: to_dev(v) for k, v in inp.items()}
    a = None if alpha is None else torch.from_numpy(np.ascontiguousarray(alpha, np.float32).ravel()).cuda()
    out, lse = lib.attn_decode_pi(dev["q"], dev["k"], dev["v"], window, period, alpha=a, k_scale=dev.get("k_scale"),
                                  v_scale=dev.get("v_scale"), kv_lens=dev.get("kv_lens"),
                                  num_splits_window=num_splits_window, num_splits_skip=num_splits_skip)
    torch.cuda.synchronize()
    return out, lse


def oracle_pi(inp, window, period, alpha=None):
    prob = oracle.Problem(inp["q"], inp["k"], inp["v"], k_scale=inp.get("k_scale"), v_scale=inp.get("v_scale"),
                          kv_lens=inp.get("kv_lens"), causal=True)
    out, lse = oracle.pi_attention(prob, window, period, alpha)
    B, Hq = inp["q"].shape[:2]
    return out.reshape(B, Hq, -1), lse.reshape(B, Hq)
