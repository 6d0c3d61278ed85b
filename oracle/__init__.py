"""ORACLE -- test infrastructure only.

A plain double-precision CPU implementation of exact softmax attention
(``oracle.c``), used to check the HIP library. Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
it. The library (``long_context_decode_kv_amd``) never imports it and shares no
code with it.

Everything here is argument marshalling around ``oracle.c``; the arithmetic and
its citations live in that file.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, E4M3, F64 = 0, 1, 2, 3
_DTYPE_OF_NUMPY = {np.dtype(np.float32): F32, np.dtype(np.uint16): BF16, np.dtype(np.uint8): E4M3,
                   np.dtype(np.float64): F64}


def build():
    """Compile ``oracle.c`` with plain gcc (no fast-math, no contraction)."""
    src = os.path.join(_HERE, "oracle.c")
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-o", _LIB_PATH, src,
           "-lm", "-lpthread"]
    subprocess.check_call(cmd)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    src = os.path.join(_HERE, "oracle.c")
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    common = [vp, i32, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32, dbl, i32]
    lib.oracle_attention.argtypes = common + [vp, i64, vp, vp, i32]
    lib.oracle_attention.restype = i32
    lib.oracle_pi_attention.argtypes = common + [i32, i32, vp, vp, i64, vp, vp, i32]
    lib.oracle_pi_attention.restype = i32
    lib.oracle_backward.argtypes = common + [vp, vp, vp, vp, i32]
    lib.oracle_backward.restype = i32
    lib.oracle_backward_subset.argtypes = common + [vp, vp, i64, vp, i64, vp, vp, vp, i32]
    lib.oracle_backward_subset.restype = i32
    lib.oracle_partial.argtypes = common + [i32, i32, i32, i64, i64, vp, vp, vp]
    lib.oracle_partial.restype = i32
    lib.oracle_energy.argtypes = common + [i32, i32, i32, vp]
    lib.oracle_energy.restype = dbl
    lib.oracle_merge.argtypes = [vp, dbl, dbl, vp, dbl, dbl, i32, vp, vp, vp]
    lib.oracle_finalize.argtypes = [vp, dbl, dbl, i32, vp, vp]
    lib.oracle_combine.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, vp]
    lib.oracle_combine.restype = i32
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = dbl
    lib.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_f64.restype = dbl
    lib.oracle_decode_elems.argtypes = [vp, i32, i64, vp]
    lib.oracle_decode_elems.restype = None
    lib.oracle_e2m1_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1_to_f64.restype = dbl
    lib.oracle_e8m0_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_to_f64.restype = dbl
    lib.oracle_mxfp4_decode.argtypes = [vp, vp, i64, i32, vp]
    lib.oracle_mxfp4_decode.restype = None
    _lib = lib
    return lib


def _threads():
    return max(1, min(os.cpu_count() or 1, 16))


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


class Problem:
    """Inputs of one attention call, exactly as stored for the GPU.

    q: [B,Hq,Lq,d] float32 / uint16 (bf16 bits); k, v: [B,Hkv,Lcap,d] float32 /
    uint16 (bf16) / uint8 (e4m3 codes) / float64 (values already decoded);
    k_scale, v_scale: float32 [B*Hkv] for e4m3; kv_lens: int32 [B] or None.
    """

    def __init__(self, q, k, v, k_scale=None, v_scale=None, kv_lens=None, scale=None, causal=False):
        self.q = np.ascontiguousarray(q)
        self.k = np.ascontiguousarray(k)
        self.v = np.ascontiguousarray(v)
        assert self.k.dtype == self.v.dtype and self.k.shape == self.v.shape
        self.B, self.Hq, self.Lq, self.d = self.q.shape
        _, self.Hkv, self.Lcap, _ = self.k.shape
        self.q_dtype = _DTYPE_OF_NUMPY[self.q.dtype]
        self.kv_dtype = _DTYPE_OF_NUMPY[self.k.dtype]
        self.k_scale = None if k_scale is None else np.ascontiguousarray(k_scale, dtype=np.float32).ravel()
        self.v_scale = None if v_scale is None else np.ascontiguousarray(v_scale, dtype=np.float32).ravel()
        self.kv_lens = None if kv_lens is None else np.ascontiguousarray(kv_lens, dtype=np.int32)
        self.scale = float(scale) if scale is not None else 1.0 / np.sqrt(self.d)
        self.causal = int(bool(causal))

    def _common(self):
        return [_p(self.q), self.q_dtype, _p(self.k), _p(self.v), self.kv_dtype, _p(self.k_scale),
                _p(self.v_scale), _p(self.kv_lens), self.B, self.Hq, self.Hkv, self.Lq, self.Lcap, self.d,
                self.scale, self.causal]


def attention(prob, rows=None, nthreads=None):
    """Exact attention. Returns (out [nrows,d] f64, lse [nrows] f64); rows are
    flat ids (b*Hq + h)*Lq + i, or every row in that order when None."""
    lib = _load()
    if rows is None:
        n = prob.B * prob.Hq * prob.Lq
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows_arr.size
    out = np.zeros((n, prob.d), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    rc = lib.oracle_attention(*prob._common(), _p(rows_arr), n, _p(out), _p(lse), nthreads or _threads())
    if rc != 0:
        raise ValueError("oracle_attention: bad arguments")
    return out, lse


def pi_attention(prob, window, period, alpha=None, rows=None, nthreads=None):
    """pi-Attention: the ring-local window, the period-pi skip keys and the
    log-prior alpha (float32 [B, Hq, Lq] or None), as defined in oracle.c.
    Returns (out [nrows, d], lse [nrows]) like attention()."""
    lib = _load()
    if rows is None:
        n = prob.B * prob.Hq * prob.Lq
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows_arr.size
    a = None if alpha is None else np.ascontiguousarray(alpha, dtype=np.float32).ravel()
    if a is not None and a.size != prob.B * prob.Hq * prob.Lq:
        raise ValueError("alpha needs one value per (batch, query head, query)")
    out = np.zeros((n, prob.d), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    rc = lib.oracle_pi_attention(*prob._common(), int(window), int(period), _p(a), _p(rows_arr), n, _p(out),
                                 _p(lse), nthreads or _threads())
    if rc != 0:
        raise ValueError("oracle_pi_attention: bad arguments")
    return out, lse


def backward(prob, dout, nthreads=None):
    """Gradients of exact attention for output gradient dout (same layout and
    dtype as q): returns (dq [B,Hq,Lq,d], dk [B,Hkv,Lcap,d], dv) in float64."""
    lib = _load()
    dout = np.ascontiguousarray(dout)
    if dout.dtype != prob.q.dtype or dout.shape != prob.q.shape:
        raise ValueError("dout must match q in shape and dtype")
    dq = np.zeros(prob.q.shape, dtype=np.float64)
    dk = np.zeros(prob.k.shape, dtype=np.float64)
    dv = np.zeros(prob.k.shape, dtype=np.float64)
    rc = lib.oracle_backward(*prob._common(), _p(dout), _p(dq), _p(dk), _p(dv), nthreads or _threads())
    if rc != 0:
        raise ValueError("oracle_backward: bad arguments")
    return dq, dk, dv


def backward_subset(prob, dout, q_rows=(), keys=(), nthreads=None):
    """The gradients of backward() at chosen places only: dq of the query rows
    q_rows (flat ids (b*Hq + h)*Lq + i) and dk, dv of the keys `keys` (flat
    ids (b*Hkv + g)*Lcap + j). Returns (dq [len(q_rows), d], dk [len(keys), d],
    dv [len(keys), d]) in float64."""
    lib = _load()
    dout = np.ascontiguousarray(dout)
    if dout.dtype != prob.q.dtype or dout.shape != prob.q.shape:
        raise ValueError("dout must match q in shape and dtype")
    qr = np.ascontiguousarray(q_rows, dtype=np.int64).ravel()
    ky = np.ascontiguousarray(keys, dtype=np.int64).ravel()
    dq = np.zeros((qr.size, prob.d), dtype=np.float64)
    dk = np.zeros((ky.size, prob.d), dtype=np.float64)
    dv = np.zeros((ky.size, prob.d), dtype=np.float64)
    rc = lib.oracle_backward_subset(*prob._common(), _p(dout), _p(qr), qr.size, _p(ky), ky.size, _p(dq), _p(dk),
                                    _p(dv), nthreads or _threads())
    if rc != 0:
        raise ValueError("oracle_backward_subset: bad arguments")
    return dq, dk, dv


def partial(prob, b, h, i, j0, j1):
    """Partial (o, m, l) of one row over keys [j0, j1)."""
    lib = _load()
    o = np.zeros(prob.d, dtype=np.float64)
    m = ctypes.c_double()
    l = ctypes.c_double()
    rc = lib.oracle_partial(*prob._common(), b, h, i, j0, j1, _p(o), ctypes.byref(m), ctypes.byref(l))
    if rc != 0:
        raise ValueError("oracle_partial: bad arguments")
    return o, m.value, l.value


def merge(a, b):
    lib = _load()
    oa, ma, la = a
    ob, mb, lb = b
    oa = np.ascontiguousarray(oa, dtype=np.float64)
    ob = np.ascontiguousarray(ob, dtype=np.float64)
    o = np.zeros_like(oa)
    m = ctypes.c_double()
    l = ctypes.c_double()
    lib.oracle_merge(_p(oa), ma, la, _p(ob), mb, lb, oa.size, _p(o), ctypes.byref(m), ctypes.byref(l))
    return o, m.value, l.value


def finalize(part):
    lib = _load()
    o, m, l = part
    o = np.ascontiguousarray(o, dtype=np.float64)
    out = np.zeros_like(o)
    lse = ctypes.c_double()
    lib.oracle_finalize(_p(o), m, l, o.size, _p(out), ctypes.byref(lse))
    return out, lse.value


def combine(o_part, m_part, l_part, count=None):
    """Normalised output of fp32 partials o [R,S,d], m [R,S], l [R,S]."""
    lib = _load()
    o_part = np.ascontiguousarray(o_part, dtype=np.float32)
    m_part = np.ascontiguousarray(m_part, dtype=np.float32)
    l_part = np.ascontiguousarray(l_part, dtype=np.float32)
    R, S, d = o_part.shape
    cnt = None if count is None else np.ascontiguousarray(count, dtype=np.int32)
    out = np.zeros((R, d), dtype=np.float64)
    lse = np.zeros(R, dtype=np.float64)
    rc = lib.oracle_combine(_p(o_part), _p(m_part), _p(l_part), R, S, d, _p(cnt), _p(out), _p(lse))
    if rc != 0:
        raise ValueError("oracle_combine: bad arguments")
    return out, lse


def energy(prob, b, h, i, zeta):
    lib = _load()
    z = np.ascontiguousarray(zeta, dtype=np.float64)
    return lib.oracle_energy(*prob._common(), b, h, i, _p(z))


def bf16_to_f64(bits):
    lib = _load()
    bits = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.oracle_bf16_to_f64(int(b)) for b in bits.ravel()]).reshape(bits.shape)


def e4m3_to_f64(codes):
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e4m3_to_f64(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def e2m1_to_f64(codes):
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e2m1_to_f64(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def e8m0_to_f64(codes):
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e8m0_to_f64(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def mxfp4_to_f64(codes, scales):
    """Real values (float64) of MX FP4 rows: codes (..., d/2) uint8 (element 2i
    in the low nibble of byte i), scales (..., d/32) uint8 E8M0."""
    lib = _load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    d = codes.shape[-1] * 2
    assert scales.shape[-1] * 32 == d and codes.shape[:-1] == scales.shape[:-1]
    rows = int(np.prod(codes.shape[:-1])) if codes.ndim > 1 else 1
    out = np.empty(codes.shape[:-1] + (d,), dtype=np.float64)
    if out.size:
        lib.oracle_mxfp4_decode(_p(codes), _p(scales), rows, d, _p(out))
    return out


def decode_elems(a):
    """Real values (float64) of stored elements: float32, bf16 bits (uint16),
    e4m3 codes (uint8) or float64, with no scale applied."""
    lib = _load()
    a = np.ascontiguousarray(a)
    out = np.empty(a.shape, dtype=np.float64)
    if a.size:
        lib.oracle_decode_elems(_p(a), _DTYPE_OF_NUMPY[a.dtype], a.size, _p(out))
    return out


def decode_spans(q, spans, scale=None, heads=None):
    """Single-query decode over a cache kept as several key spans, each in its
    own storage format (a cache kept in several precisions).

    q [B,Hq,1,d] (bf16 bits or float32). Each span is a dict with k, v and
    "format": "bf16" (k, v [B,Hkv,L,d] bf16 bits), "e4m3" (codes
    [B,Hkv,L,d] with "k_scale", "v_scale" float32 [B*Hkv]) or "mxfp4" (codes
    [B,Hkv,L,d/2] with E8M0 "k_scale", "v_scale" [B,Hkv,L,d/32]); "lens" int32
    [B*Hkv] (valid keys per (sequence, KV head), clamped to the capacity) or
    None = the capacity. A span with k None has no keys. Each query head sees
    the union of its group's valid keys of every span at their real values,
    built in float64 (spans in the order given) and handed to the plain
    attention above. `heads` lists flat query heads b*Hq + h (all when None).
    Returns (out [n,d], lse [n]) in float64."""
    q = np.ascontiguousarray(q)
    B, Hq, Lq, d = q.shape
    assert Lq == 1
    present = [sp for sp in spans if sp.get("k") is not None]
    Hkv = present[0]["k"].shape[1] if present else Hq
    G = Hq // Hkv
    caps, lens = [], []
    for sp in spans:
        cap = 0 if sp.get("k") is None else sp["k"].shape[2]
        caps.append(cap)
        ln = sp.get("lens")
        lens.append(np.full(B * Hkv, cap, np.int64) if ln is None else np.clip(np.asarray(ln).ravel(), 0, cap))
    heads = np.arange(B * Hq) if heads is None else np.asarray(heads).ravel()
    out = np.zeros((heads.size, d), np.float64)
    lse = np.zeros(heads.size, np.float64)
    by_group = {}
    for i, r in enumerate(heads):
        by_group.setdefault((int(r) // Hq, (int(r) % Hq) // G), []).append((i, int(r) % Hq))
    for (b, g), items in by_group.items():
        bg = b * Hkv + g
        kparts, vparts = [], []
        for sp, ln in zip(spans, lens):
            n_s = int(ln[bg]) if sp.get("k") is not None else 0
            if not n_s:
                continue
            fmt = sp["format"]
            if fmt == "mxfp4":
                kparts.append(mxfp4_to_f64(sp["k"][b, g, :n_s], sp["k_scale"][b, g, :n_s]))
                vparts.append(mxfp4_to_f64(sp["v"][b, g, :n_s], sp["v_scale"][b, g, :n_s]))
            elif fmt == "e4m3":
                ks = np.asarray(sp["k_scale"], np.float32).ravel()
                vs = np.asarray(sp["v_scale"], np.float32).ravel()
                kparts.append(decode_elems(sp["k"][b, g, :n_s]) * np.float64(ks[bg]))
                vparts.append(decode_elems(sp["v"][b, g, :n_s]) * np.float64(vs[bg]))
            elif fmt == "bf16":
                kparts.append(decode_elems(sp["k"][b, g, :n_s]))
                vparts.append(decode_elems(sp["v"][b, g, :n_s]))
            else:
                raise ValueError("unknown span format %r" % (fmt,))
        n = sum(x.shape[0] for x in kparts)
        kk = np.concatenate(kparts) if n else np.zeros((1, d))
        vv = np.concatenate(vparts) if n else np.zeros((1, d))
        prob = Problem(q[b:b + 1, g * G:(g + 1) * G], kk[None, None], vv[None, None],
                       kv_lens=np.array([n], np.int32), scale=scale)
        o, l_ = attention(prob, rows=[h - g * G for _, h in items])
        for j, (i, _) in enumerate(items):
            out[i] = o[j]
            lse[i] = l_[j]
    return out, lse


def decode_mixed(q, k_hi, v_hi, k_lo, v_lo, k_scale, v_scale, hi_lens=None, lo_lens=None, scale=None,
                 heads=None, lo_format="e4m3"):
    """Single-query decode over a cache kept in two precisions: decode_spans
    with a bf16 span and a low-precision span.

    q [B,Hq,1,d] (bf16 bits or float32); k_hi, v_hi [B,Hkv,L_hi,d] bf16 bits
    (or None: no such keys); k_lo, v_lo [B,Hkv,L_lo,d] e4m3 codes (or None)
    with k_scale, v_scale float32 [B*Hkv]; hi_lens, lo_lens int32 [B*Hkv]
    (valid keys per (sequence, KV head), clamped to the capacity) or None =
    the capacity. With lo_format="mxfp4" the low span is MX FP4: k_lo, v_lo
    are codes [B,Hkv,L_lo,d/2] and k_scale, v_scale their E8M0 scales
    [B,Hkv,L_lo,d/32]. Returns (out [n,d], lse [n]) in float64.
    """
    spans = [dict(k=k_hi, v=v_hi, format="bf16", lens=hi_lens),
             dict(k=k_lo, v=v_lo, format="mxfp4" if lo_format == "mxfp4" else "e4m3", k_scale=k_scale,
                  v_scale=v_scale, lens=lo_lens)]
    return decode_spans(q, spans, scale=scale, heads=heads)
