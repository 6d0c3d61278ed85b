"""The nine synthetic workloads: shapes and input recipes (no arithmetic of the
method). Shapes follow Llama-3.1-8B's attention (32 query heads, 8 KV heads,
head dim 128), the model the Tree Attention explainer evaluates on (section 4);
no weights, prompts or datasets are involved -- every tensor is drawn from the
seeded generator.

Recipe: seed = workload number; tensor ids Q=0, K=1, V=2, lengths=3. Values are
N(0,1) * mul rounded to the storage format; fp8 tensors get one amax/448 scale
per (batch, KV head); MX fp4 tensors get one power-of-two (e8m0) scale per 32
consecutive elements of a row, chosen from the block's largest magnitude.
"""
import numpy as np

from . import (TID_K, TID_K_LO, TID_K_MID, TID_LENS, TID_LENS_LO, TID_LENS_MID, TID_Q, TID_V, TID_V_LO,
               TID_V_MID, normal_bf16_bits, normal_e4m3, normal_f32, normal_mxfp4, uniform_int)

WORKLOADS = {
    1: dict(name="single-head decode, fp32, L=1024, d=64, 4 splits", kind="decode", B=1, Hq=1, Hkv=1, d=64,
            L=1024, q="f32", kv="f32", mul=1.0, causal=False, splits=4),
    2: dict(name="GQA decode, bf16, L=131072, 32q/8kv, d=128", kind="decode", B=1, Hq=32, Hkv=8, d=128,
            L=131072, q="bf16", kv="bf16", mul=0.5, causal=False, splits=(64, 128, 256)),
    3: dict(name="batched ragged GQA decode, bf16, B=16, L_b~U[4096,65536]", kind="decode", B=16, Hq=32, Hkv=8,
            d=128, L=65536, lens=(4096, 65536), q="bf16", kv="bf16", mul=0.5, causal=True, splits=0),
    4: dict(name="causal prefill, bf16, L=16384, 32q/8kv, d=128", kind="prefill", B=1, Hq=32, Hkv=8, d=128,
            L=16384, q="bf16", kv="bf16", mul=1.0, causal=True),
    5: dict(name="fp8-e4m3 KV decode, L=1048576, 32q/8kv, d=128", kind="decode", B=1, Hq=32, Hkv=8, d=128,
            L=1048576, q="bf16", kv="e4m3", mul=1.0, causal=False, splits=1024),
    6: dict(name="two-precision KV decode, L=131072: first and last 10% bf16, the rest fp8-e4m3, 32q/8kv, d=128",
            kind="mixed", B=1, Hq=32, Hkv=8, d=128, L=131072, hi_frac=0.1, q="bf16", mul=0.5, causal=False),
    7: dict(name="pi-Attention decode, bf16, L=131072, window 4096, period 64, 32q/8kv, d=128", kind="decode", B=1,
            Hq=32, Hkv=8, d=128, L=131072, q="bf16", kv="bf16", mul=0.5, causal=True, window=4096, period=64),
    8: dict(name="pi-Attention causal prefill, bf16, L=16384, window 512, period 64, 32q/8kv, d=128", kind="prefill",
            B=1, Hq=32, Hkv=8, d=128, L=16384, q="bf16", kv="bf16", mul=1.0, causal=True, window=512, period=64),
    9: dict(name="two-precision KV decode, L=131072: first and last 10% bf16, the rest MX fp4 (e2m1, one e8m0 scale "
                 "per 32), 32q/8kv, d=128",
            kind="mixed", B=1, Hq=32, Hkv=8, d=128, L=131072, hi_frac=0.1, q="bf16", mul=0.5, causal=False,
            lo="mxfp4"),
    10: dict(name="three-precision KV decode, L=131072: first and last 10% bf16, 20% fp8-e4m3, 60% MX fp4, "
                  "32q/8kv, d=128",
             kind="mixed3", B=1, Hq=32, Hkv=8, d=128, L=131072, hi_frac=0.1, mid_frac=0.2, q="bf16", mul=0.5,
             causal=False),
}

# Tensor id of the pi-Attention gate alpha (one value per query row, uniform in
# [0.05, 0.95]; a trained gate is not available, so any value in (0, 1) serves).
TID_ALPHA = 7


def _draw(fmt, seed, tid, shape, mul):
    if fmt == "f32":
        return normal_f32(seed, tid, shape, mul), None
    if fmt == "bf16":
        return normal_bf16_bits(seed, tid, shape, mul), None
    if fmt == "e4m3":
        return normal_e4m3(seed, tid, shape, mul)
    raise ValueError(fmt)


def make_inputs(wl, seed=None, B=None, Hq=None, Hkv=None, d=None, L=None, Lq=None, mul=None, q_mul=None,
                lens=None):
    """Host inputs of a workload (any field overridable for smaller variants).

    Returns dict(q, k, v, k_scale, v_scale, kv_lens) as numpy arrays: bf16 as
    uint16 bit patterns, e4m3 as uint8 codes, kv_lens int32 or None."""
    cfg = WORKLOADS[wl] if isinstance(wl, int) else wl
    seed = cfg.get("seed", wl if isinstance(wl, int) else 0) if seed is None else seed
    B = B or cfg["B"]
    Hq = Hq or cfg["Hq"]
    Hkv = Hkv or cfg["Hkv"]
    d = d or cfg["d"]
    L = L or cfg["L"]
    mul = cfg["mul"] if mul is None else mul
    if Lq is None:
        Lq = L if cfg["kind"] == "prefill" else 1
    q, _ = _draw(cfg["q"], seed, TID_Q, (B, Hq, Lq, d), mul if q_mul is None else q_mul)
    k, ks = _draw(cfg["kv"], seed, TID_K, (B, Hkv, L, d), mul)
    v, vs = _draw(cfg["kv"], seed, TID_V, (B, Hkv, L, d), mul)
    kv_lens = None
    rng = lens if lens is not None else cfg.get("lens")
    if rng is not None:
        kv_lens = uniform_int(seed, TID_LENS, B, int(rng[0]), int(min(rng[1], L)))
    return dict(q=q, k=k, v=v, k_scale=None if ks is None else ks.ravel(),
                v_scale=None if vs is None else vs.ravel(), kv_lens=kv_lens)


def make_mixed_inputs(wl=6, seed=None, B=None, Hq=None, Hkv=None, d=None, L=None, hi_frac=None, L_hi=None,
                      L_lo=None, lens=None):
    """Host inputs of a two-precision cache: the first and the last hi_frac of
    the L tokens (2 * round(hi_frac * L) keys) in bf16, the others in fp8-e4m3.

    Key order does not change single-query attention, so the bf16 keys are
    stored as one span k_hi/v_hi [B,Hkv,L_hi,d] and the fp8 keys as another,
    k_lo/v_lo [B,Hkv,L_lo,d] with one amax/448 scale per (batch, KV head).
    A workload with lo="mxfp4" keeps the low span as MX fp4 instead: k_lo/v_lo
    are codes [B,Hkv,L_lo,d/2] and k_scale/v_scale their E8M0 block scales
    [B,Hkv,L_lo,d/32].
    `lens` = (lo, hi) draws a valid length per (batch, KV head) for each span
    uniformly from [lo*cap, hi*cap] (ragged per head); None = full spans.
    Returns dict(q, k_hi, v_hi, k_lo, v_lo, k_scale, v_scale, hi_lens, lo_lens)."""
    cfg = WORKLOADS[wl]
    seed = wl if seed is None else seed
    B = B or cfg["B"]
    Hq = Hq or cfg["Hq"]
    Hkv = Hkv or cfg["Hkv"]
    d = d or cfg["d"]
    L = L or cfg["L"]
    frac = cfg["hi_frac"] if hi_frac is None else hi_frac
    if L_hi is None:
        L_hi = 2 * int(round(frac * L))
    if L_lo is None:
        L_lo = L - L_hi
    mul = cfg["mul"]
    q = normal_bf16_bits(seed, TID_Q, (B, Hq, 1, d), mul)
    k_hi = normal_bf16_bits(seed, TID_K, (B, Hkv, L_hi, d), mul) if L_hi else None
    v_hi = normal_bf16_bits(seed, TID_V, (B, Hkv, L_hi, d), mul) if L_hi else None
    mx = cfg.get("lo") == "mxfp4"
    lo_fill = normal_mxfp4 if mx else normal_e4m3
    k_lo, ks = lo_fill(seed, TID_K_LO, (B, Hkv, L_lo, d), mul) if L_lo else (None, None)
    v_lo, vs = lo_fill(seed, TID_V_LO, (B, Hkv, L_lo, d), mul) if L_lo else (None, None)
    hi_lens = lo_lens = None
    if lens is not None:
        lo_f, hi_f = lens
        hi_lens = uniform_int(seed, TID_LENS, B * Hkv, int(lo_f * L_hi), int(hi_f * L_hi))
        lo_lens = uniform_int(seed, TID_LENS_LO, B * Hkv, int(lo_f * L_lo), int(hi_f * L_lo))
    if mx:
        return dict(q=q, k_hi=k_hi, v_hi=v_hi, k_lo=k_lo, v_lo=v_lo, k_scale=ks, v_scale=vs, hi_lens=hi_lens,
                    lo_lens=lo_lens, lo_format="mxfp4")
    return dict(q=q, k_hi=k_hi, v_hi=v_hi, k_lo=k_lo, v_lo=v_lo, k_scale=None if ks is None else ks.ravel(),
                v_scale=None if vs is None else vs.ravel(), hi_lens=hi_lens, lo_lens=lo_lens)


def make_alpha(wl, shape, seed=None):
    """The gate alpha of a pi-Attention workload: uniform in [0.05, 0.95]."""
    from . import uniform_f32
    seed = wl if seed is None else seed
    return uniform_f32(seed, TID_ALPHA, shape, 0.05, 0.95)


def make_mixed3_inputs(wl=10, seed=None, B=None, Hq=None, Hkv=None, d=None, L=None, L_hi=None, L_mid=None,
                       L_lo=None, lens=None):
    """Host inputs of a three-precision cache: the first and the last tenth of
    the L tokens (2 * round(0.1 * L) keys) in bf16, 2 * round(0.1 * L) more in
    fp8-e4m3 (one amax/448 scale per (batch, KV head)) and the rest in MX fp4
    (one e8m0 scale per 32 elements of a row). Key order does not change
    single-query attention, so each precision is one span. `lens` = (lo, hi)
    draws a valid length per (batch, KV head) for each span uniformly from
    [lo*cap, hi*cap]. Returns dict(q, k_hi, v_hi, k_mid, v_mid, k_mid_scale,
    v_mid_scale, k_lo, v_lo, k_lo_scale, v_lo_scale, hi_lens, mid_lens,
    lo_lens)."""
    cfg = WORKLOADS[wl]
    seed = wl if seed is None else seed
    B = B or cfg["B"]
    Hq = Hq or cfg["Hq"]
    Hkv = Hkv or cfg["Hkv"]
    d = d or cfg["d"]
    L = L or cfg["L"]
    if L_hi is None:
        L_hi = 2 * int(round(cfg["hi_frac"] * L))
    if L_mid is None:
        L_mid = 2 * int(round((cfg["mid_frac"] / 2) * L))
    if L_lo is None:
        L_lo = L - L_hi - L_mid
    mul = cfg["mul"]
    out = dict(q=normal_bf16_bits(seed, TID_Q, (B, Hq, 1, d), mul))
    out["k_hi"] = normal_bf16_bits(seed, TID_K, (B, Hkv, L_hi, d), mul) if L_hi else None
    out["v_hi"] = normal_bf16_bits(seed, TID_V, (B, Hkv, L_hi, d), mul) if L_hi else None
    k8, ks8 = normal_e4m3(seed, TID_K_MID, (B, Hkv, L_mid, d), mul) if L_mid else (None, None)
    v8, vs8 = normal_e4m3(seed, TID_V_MID, (B, Hkv, L_mid, d), mul) if L_mid else (None, None)
    out.update(k_mid=k8, v_mid=v8, k_mid_scale=None if ks8 is None else ks8.ravel(),
               v_mid_scale=None if vs8 is None else vs8.ravel())
    k4, ks4 = normal_mxfp4(seed, TID_K_LO, (B, Hkv, L_lo, d), mul) if L_lo else (None, None)
    v4, vs4 = normal_mxfp4(seed, TID_V_LO, (B, Hkv, L_lo, d), mul) if L_lo else (None, None)
    out.update(k_lo=k4, v_lo=v4, k_lo_scale=ks4, v_lo_scale=vs4)
    out["hi_lens"] = out["mid_lens"] = out["lo_lens"] = None
    if lens is not None:
        lo_f, hi_f = lens
        out["hi_lens"] = uniform_int(seed, TID_LENS, B * Hkv, int(lo_f * L_hi), int(hi_f * L_hi))
        out["mid_lens"] = uniform_int(seed, TID_LENS_MID, B * Hkv, int(lo_f * L_mid), int(hi_f * L_mid))
        out["lo_lens"] = uniform_int(seed, TID_LENS_LO, B * Hkv, int(lo_f * L_lo), int(hi_f * L_lo))
    return out


def mixed3_spans(inp):
    """The three spans of make_mixed3_inputs() in the form oracle.decode_spans takes."""
    return [dict(k=inp["k_hi"], v=inp["v_hi"], format="bf16", lens=inp["hi_lens"]),
            dict(k=inp["k_mid"], v=inp["v_mid"], format="e4m3", k_scale=inp["k_mid_scale"],
                 v_scale=inp["v_mid_scale"], lens=inp["mid_lens"]),
            dict(k=inp["k_lo"], v=inp["v_lo"], format="mxfp4", k_scale=inp["k_lo_scale"],
                 v_scale=inp["v_lo_scale"], lens=inp["lo_lens"])]
