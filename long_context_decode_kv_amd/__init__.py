"""Python binding of libattn.so (exact attention for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/attn.h``. torch provides device
memory (outputs and the decode workspace are allocated here as torch tensors
when the caller does not pass them) and the current HIP stream.

There is no fallback: if ``libattn.so`` is missing the calls raise.
"""
import ctypes
import os

import torch

__all__ = [
    "AttnError", "ATTN_F32", "ATTN_BF16", "ATTN_FP8_E4M3", "ATTN_MXFP4", "ATTN_E8M0", "library_path", "load_library",
    "attn_status_string", "attn_decode_auto_splits", "attn_decode_workspace_size", "attn_decode_workspace_init",
    "attn_decode_plan",
    "attn_decode", "attn_decode_noalloc", "attn_decode_partials", "attn_decode_workspace", "attn_prefill", "attn_combine_partials",
    "attn_decode_mixed", "attn_decode_mixed_splits", "attn_decode_mixed_fp4", "attn_decode_mixed_fp4_splits",
    "attn_decode_mixed3", "attn_decode_mixed3_splits",
    "attn_decode_pi", "attn_decode_pi_splits", "attn_prefill_pi",
    "attn_prefill_pi_workspace_size", "attn_prefill_backward", "attn_prefill_backward_workspace_size",
]

ATTN_F32, ATTN_BF16, ATTN_FP8_E4M3, ATTN_MXFP4, ATTN_E8M0 = 0, 1, 2, 3, 4
_STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED", 3: "ATTN_ERR_WORKSPACE",
           4: "ATTN_ERR_HIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libattn.so")
_lib = None


class AttnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (_STATUS.get(status, str(status)), message))
        self.status = status


class attn_tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_s", ctypes.c_int64)]


def load_library():
    """Load libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError("libattn.so not found at %s; build it with __graft_entry__.build()" % library_path)
    lib = ctypes.CDLL(library_path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    tp = ctypes.POINTER(attn_tensor)
    lib.attn_status_string.argtypes = [i32]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_decode_auto_splits.argtypes = [i32, i32, i32, i32, i32]
    lib.attn_decode_auto_splits.restype = i32
    lib.attn_decode_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.attn_decode_workspace_size.restype = ctypes.c_size_t
    lib.attn_decode_workspace_init.argtypes = [vp, ctypes.c_size_t, vp]
    lib.attn_decode_workspace_init.restype = i32
    lib.attn_decode.argtypes = [tp, tp, tp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32, tp, vp, vp,
                                ctypes.c_size_t, vp]
    lib.attn_decode.restype = i32
    lib.attn_decode_noalloc.argtypes = [tp, tp, tp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32, tp, vp, vp]
    lib.attn_decode_noalloc.restype = i32
    lib.attn_decode_plan.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_int)]
    lib.attn_decode_plan.restype = i32
    lib.attn_decode_partials.argtypes = [tp, tp, tp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32, vp, vp, vp,
                                         ctypes.POINTER(ctypes.c_int), vp]
    lib.attn_decode_partials.restype = i32
    lib.attn_prefill.argtypes = [tp, tp, tp, i32, i32, i32, i32, i32, i32, f32, i32, tp, vp, vp]
    lib.attn_prefill.restype = i32
    lib.attn_combine_partials.argtypes = [vp, vp, vp, i32, i32, i32, tp, vp, vp]
    lib.attn_combine_partials.restype = i32
    lib.attn_decode_mixed.argtypes = [tp, tp, tp, vp, i32, tp, tp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32,
                                      tp, vp, vp, ctypes.c_size_t, vp]
    lib.attn_decode_mixed.restype = i32
    ip = ctypes.POINTER(ctypes.c_int)
    lib.attn_decode_mixed_splits.argtypes = [i32, i32, i32, i32, ip, ip]
    lib.attn_decode_mixed_splits.restype = i32
    lib.attn_decode_mixed_fp4.argtypes = [tp, tp, tp, vp, i32, tp, tp, tp, tp, vp, i32, i32, i32, i32, i32, f32, i32,
                                          i32, tp, vp, vp, ctypes.c_size_t, vp]
    lib.attn_decode_mixed_fp4.restype = i32
    lib.attn_decode_mixed_fp4_splits.argtypes = [i32, i32, i32, i32, ip, ip]
    lib.attn_decode_mixed_fp4_splits.restype = i32
    lib.attn_decode_mixed3.argtypes = [tp, tp, tp, vp, i32, tp, tp, vp, vp, vp, i32, tp, tp, tp, tp, vp, i32, i32, i32,
                                       i32, i32, f32, i32, i32, i32, tp, vp, vp, ctypes.c_size_t, vp]
    lib.attn_decode_mixed3.restype = i32
    lib.attn_decode_mixed3_splits.argtypes = [i32, i32, i32, i32, i32, ip, ip, ip]
    lib.attn_decode_mixed3_splits.restype = i32
    lib.attn_decode_pi.argtypes = [tp, tp, tp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32, vp, i32, i32, tp, vp,
                                   vp, ctypes.c_size_t, vp]
    lib.attn_decode_pi.restype = i32
    lib.attn_decode_pi_splits.argtypes = [i32, i32, i32, i32, i32, i32, ip, ip]
    lib.attn_decode_pi_splits.restype = i32
    lib.attn_prefill_pi.argtypes = [tp, tp, tp, i32, i32, i32, i32, i32, f32, i32, i32, i32, vp, tp, vp, vp,
                                    ctypes.c_size_t, vp]
    lib.attn_prefill_pi.restype = i32
    lib.attn_prefill_pi_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.attn_prefill_pi_workspace_size.restype = ctypes.c_size_t
    lib.attn_prefill_backward.argtypes = [tp, tp, tp, tp, vp, tp, i32, i32, i32, i32, i32, i32, f32, i32, tp, tp, tp, vp,
                                          ctypes.c_size_t, vp]
    lib.attn_prefill_backward.restype = i32
    lib.attn_prefill_backward_workspace_size.argtypes = [i32, i32, i32]
    lib.attn_prefill_backward_workspace_size.restype = ctypes.c_size_t
    _lib = lib
    return lib


def _dtype_code(t):
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return ATTN_FP8_E4M3
    raise TypeError("unsupported dtype %s" % t.dtype)


def _tensor(t, dtype=None):
    """attn_tensor view of a 4-D tensor; `dtype` overrides the code taken from
    t.dtype (uint8 tensors holding MX fp4 codes or E8M0 scales)."""
    if t.dim() != 4:
        raise ValueError("expected a 4-D [batch, heads, seq, d] tensor, got shape %s" % (tuple(t.shape),))
    if t.stride(3) != 1:
        raise ValueError("the last dimension must be contiguous")
    if dtype is not None and t.dtype != torch.uint8:
        raise TypeError("MX fp4 codes and E8M0 scales are uint8 tensors")
    code = _dtype_code(t) if dtype is None else dtype
    return attn_tensor(t.data_ptr(), code, t.stride(0), t.stride(1), t.stride(2))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(status):
    if status != 0:
        raise AttnError(status, load_library().attn_last_error().decode())


def attn_status_string(status):
    return load_library().attn_status_string(int(status)).decode()


def attn_decode_auto_splits(B, Hkv, L_cap, kv_dtype=ATTN_BF16, ragged=False):
    return load_library().attn_decode_auto_splits(B, Hkv, L_cap, kv_dtype, int(bool(ragged)))


def attn_decode_workspace_size(B, Hq, d, num_splits):
    return load_library().attn_decode_workspace_size(B, Hq, d, num_splits)


def attn_decode_workspace_init(workspace, stream=None):
    """Zero the merge counters of a freshly allocated decode workspace."""
    st = load_library().attn_decode_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                                   _stream(stream, workspace.device))
    _check(st)
    return workspace


def attn_decode_workspace(B, Hq, d, num_splits, device="cuda"):
    """Allocate and prepare a decode workspace for up to `num_splits` splits."""
    need = load_library().attn_decode_workspace_size(B, Hq, d, num_splits)
    return attn_decode_workspace_init(torch.empty(need, dtype=torch.uint8, device=device))


def attn_decode_plan(L_cap, num_splits):
    """(S, chunk): splits used and keys per split for a requested split count."""
    chunk = ctypes.c_int(0)
    S = load_library().attn_decode_plan(L_cap, num_splits, ctypes.byref(chunk))
    return S, chunk.value


def attn_decode(q, k, v, k_scale=None, v_scale=None, kv_lens=None, softmax_scale=0.0, causal=False, num_splits=0,
                out=None, lse=None, workspace=None, stream=None):
    """Single-query decode. q [B,Hq,1,d]; k, v [B,Hkv,L_cap,d]. Returns (out, lse)."""
    lib = load_library()
    B, Hq, Lq, d = q.shape
    Hkv, L_cap = k.shape[1], k.shape[2]
    if Lq != 1:
        raise ValueError("attn_decode takes one query per sequence (q.shape[2] == 1)")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    S = num_splits if num_splits > 0 else lib.attn_decode_auto_splits(B, Hkv, L_cap, _dtype_code(k),
                                                                      int(kv_lens is not None))
    if S <= 0:
        raise AttnError(4, "could not plan splits")
    if workspace is None:
        workspace = attn_decode_workspace(B, Hq, d, S, device=q.device)
    qt, kt, vt, ot = _tensor(q), _tensor(k), _tensor(v), _tensor(out)
    st = lib.attn_decode(ctypes.byref(qt), ctypes.byref(kt), ctypes.byref(vt), _ptr(k_scale), _ptr(v_scale),
                         _ptr(kv_lens), B, Hq, Hkv, d, L_cap, float(softmax_scale), int(bool(causal)), int(S),
                         ctypes.byref(ot), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
                         _stream(stream, q.device))
    _check(st)
    return out, lse


def attn_decode_noalloc(q, k, v, k_scale=None, v_scale=None, kv_lens=None, softmax_scale=0.0, causal=False,
                        num_splits=0, out=None, lse=None, stream=None):
    """attn_decode without a workspace: the library's fixed per-GPU scratch
    array holds the merge counters and partials (up to 32 MiB; larger requests
    raise). Pass `out` and `lse` to make the call allocate nothing at all."""
    lib = load_library()
    B, Hq, Lq, d = q.shape
    Hkv, L_cap = k.shape[1], k.shape[2]
    if Lq != 1:
        raise ValueError("attn_decode_noalloc takes one query per sequence (q.shape[2] == 1)")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    qt, kt, vt, ot = _tensor(q), _tensor(k), _tensor(v), _tensor(out)
    st = lib.attn_decode_noalloc(ctypes.byref(qt), ctypes.byref(kt), ctypes.byref(vt), _ptr(k_scale), _ptr(v_scale),
                                 _ptr(kv_lens), B, Hq, Hkv, d, L_cap, float(softmax_scale), int(bool(causal)),
                                 int(num_splits), ctypes.byref(ot), _ptr(lse), _stream(stream, q.device))
    _check(st)
    return out, lse


def attn_decode_partials(q, k, v, k_scale=None, v_scale=None, kv_lens=None, softmax_scale=0.0, causal=False,
                         num_splits=0, o_part=None, m_part=None, l_part=None, stream=None):
    """First level of the decode: returns (o_part [B*Hq,S,d], m_part [B*Hq,S], l_part [B*Hq,S])."""
    lib = load_library()
    B, Hq, Lq, d = q.shape
    Hkv, L_cap = k.shape[1], k.shape[2]
    if Lq != 1:
        raise ValueError("attn_decode_partials takes one query per sequence (q.shape[2] == 1)")
    req = num_splits if num_splits > 0 else lib.attn_decode_auto_splits(B, Hkv, L_cap, _dtype_code(k),
                                                                        int(kv_lens is not None))
    S, _ = attn_decode_plan(L_cap, req)
    if S <= 0:
        raise AttnError(4, "could not plan splits")
    dev = q.device
    o_part = torch.empty((B * Hq, S, d), dtype=torch.float32, device=dev) if o_part is None else o_part
    m_part = torch.empty((B * Hq, S), dtype=torch.float32, device=dev) if m_part is None else m_part
    l_part = torch.empty((B * Hq, S), dtype=torch.float32, device=dev) if l_part is None else l_part
    for t, shape in ((o_part, (B * Hq, S, d)), (m_part, (B * Hq, S)), (l_part, (B * Hq, S))):
        if tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("partials must be contiguous fp32 of shape %s" % (shape,))
    used = ctypes.c_int(0)
    qt, kt, vt = _tensor(q), _tensor(k), _tensor(v)
    st = lib.attn_decode_partials(ctypes.byref(qt), ctypes.byref(kt), ctypes.byref(vt), _ptr(k_scale),
                                  _ptr(v_scale), _ptr(kv_lens), B, Hq, Hkv, d, L_cap, float(softmax_scale),
                                  int(bool(causal)), int(req), _ptr(o_part), _ptr(m_part), _ptr(l_part),
                                  ctypes.byref(used), _stream(stream, dev))
    _check(st)
    return o_part, m_part, l_part


def attn_prefill(q, k, v, softmax_scale=0.0, causal=True, out=None, lse=None, stream=None):
    """Prefill attention. q [B,Hq,Lq,d]; k, v [B,Hkv,Lkv,d] (bf16). Returns (out, lse [B,Hq,Lq])."""
    lib = load_library()
    B, Hq, Lq, d = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    qt, kt, vt, ot = _tensor(q), _tensor(k), _tensor(v), _tensor(out)
    st = lib.attn_prefill(ctypes.byref(qt), ctypes.byref(kt), ctypes.byref(vt), B, Hq, Hkv, d, Lq, Lkv,
                          float(softmax_scale), int(bool(causal)), ctypes.byref(ot), _ptr(lse),
                          _stream(stream, q.device))
    _check(st)
    return out, lse


def attn_combine_partials(o_part, m_part, l_part, out=None, lse=None, out_dtype=torch.float32, stream=None):
    """Merge partials o [R,S,d], m [R,S], l [R,S] (fp32) into (out [R,d], lse [R])."""
    lib = load_library()
    R, S, d = o_part.shape
    for t in (o_part, m_part, l_part):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("partials must be contiguous fp32")
    if out is None:
        out = torch.empty((R, d), dtype=out_dtype, device=o_part.device)
    if lse is None:
        lse = torch.empty((R,), dtype=torch.float32, device=o_part.device)
    if out.stride(1) != 1:
        raise ValueError("out rows must be contiguous")
    ot = attn_tensor(out.data_ptr(), _dtype_code(out), 0, 0, out.stride(0))
    st = lib.attn_combine_partials(_ptr(o_part), _ptr(m_part), _ptr(l_part), R, S, d, ctypes.byref(ot), _ptr(lse),
                                   _stream(stream, o_part.device))
    _check(st)
    return out, lse


def attn_decode_mixed_splits(B, Hkv, L_hi_cap, L_lo_cap):
    """(S_hi, S_lo): the automatic split plan of attn_decode_mixed."""
    hi, lo = ctypes.c_int(0), ctypes.c_int(0)
    total = load_library().attn_decode_mixed_splits(B, Hkv, L_hi_cap, L_lo_cap, ctypes.byref(hi), ctypes.byref(lo))
    if total <= 0:
        raise AttnError(4, "could not plan splits")
    return hi.value, lo.value


def attn_decode_mixed(q, k_hi, v_hi, k_lo, v_lo, k_scale=None, v_scale=None, hi_lens=None, lo_lens=None,
                      softmax_scale=0.0, num_splits_hi=0, num_splits_lo=0, out=None, lse=None, workspace=None,
                      stream=None):
    """Decode over a two-precision KV cache: a bf16 span (k_hi, v_hi [B,Hkv,L_hi,d]) and an fp8 span (k_lo,
    v_lo [B,Hkv,L_lo,d] with k_scale, v_scale [B*Hkv]); hi_lens / lo_lens are int32 [B,Hkv] or None. Either
    span may be None (no keys). Returns (out [B,Hq,1,d] bf16, lse [B,Hq])."""
    lib = load_library()
    B, Hq, Lq, d = q.shape
    if Lq != 1:
        raise ValueError("attn_decode_mixed takes one query per sequence (q.shape[2] == 1)")
    L_hi = 0 if k_hi is None else k_hi.shape[2]
    L_lo = 0 if k_lo is None else k_lo.shape[2]
    Hkv = (k_hi if k_hi is not None else k_lo).shape[1]
    for lens in (hi_lens, lo_lens):
        if lens is not None and (lens.dtype != torch.int32 or lens.numel() != B * Hkv or not lens.is_contiguous()):
            raise ValueError("span lengths must be contiguous int32 with B*Hkv entries")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    S_hi, S_lo = num_splits_hi, num_splits_lo
    if (S_hi <= 0 and L_hi) or (S_lo <= 0 and L_lo):
        auto_hi, auto_lo = attn_decode_mixed_splits(B, Hkv, L_hi, L_lo)
        S_hi = S_hi if S_hi > 0 else auto_hi
        S_lo = S_lo if S_lo > 0 else auto_lo
    if workspace is None:
        used = (attn_decode_plan(L_hi, S_hi)[0] if L_hi else 0) + (attn_decode_plan(L_lo, S_lo)[0] if L_lo else 0)
        workspace = attn_decode_workspace(B, Hq, d, used, device=q.device)

    def view(t):
        return None if t is None else ctypes.byref(_tensor(t))

    qt, ot = _tensor(q), _tensor(out)
    st = lib.attn_decode_mixed(ctypes.byref(qt), view(k_hi), view(v_hi), _ptr(hi_lens), L_hi, view(k_lo), view(v_lo),
                               _ptr(k_scale), _ptr(v_scale), _ptr(lo_lens), L_lo, B, Hq, Hkv, d,
                               float(softmax_scale), int(S_hi), int(S_lo), ctypes.byref(ot), _ptr(lse), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    _check(st)
    return out, lse


def attn_decode_mixed_fp4_splits(B, Hkv, L_hi_cap, L_lo_cap):
    """(S_hi, S_lo): the automatic split plan of attn_decode_mixed_fp4."""
    hi, lo = ctypes.c_int(0), ctypes.c_int(0)
    total = load_library().attn_decode_mixed_fp4_splits(B, Hkv, L_hi_cap, L_lo_cap, ctypes.byref(hi),
                                                        ctypes.byref(lo))
    if total <= 0:
        raise AttnError(4, "could not plan splits")
    return hi.value, lo.value


def attn_decode_mixed_fp4(q, k_hi, v_hi, k_lo, v_lo, k_lo_scale=None, v_lo_scale=None, hi_lens=None, lo_lens=None,
                          softmax_scale=0.0, num_splits_hi=0, num_splits_lo=0, out=None, lse=None, workspace=None,
                          stream=None):
    """Decode over a cache with a bf16 span (k_hi, v_hi [B,Hkv,L_hi,d]) and an MX fp4 span: k_lo, v_lo uint8
    [B,Hkv,L_lo,d/2] (E2M1 codes, first of a pair in the low nibble) with k_lo_scale, v_lo_scale uint8
    [B,Hkv,L_lo,d/32] (E8M0). hi_lens / lo_lens are int32 [B,Hkv] or None; either span may be None. Returns
    (out [B,Hq,1,d] bf16, lse [B,Hq]). Scale bytes 1..252 are exact for every code; 253-254 can overflow to inf,
    0 gives fp32 subnormals (may flush to zero), 255 is NaN."""
    lib = load_library()
    B, Hq, Lq, d = q.shape
    if Lq != 1:
        raise ValueError("attn_decode_mixed_fp4 takes one query per sequence (q.shape[2] == 1)")
    L_hi = 0 if k_hi is None else k_hi.shape[2]
    L_lo = 0 if k_lo is None else k_lo.shape[2]
    Hkv = (k_hi if k_hi is not None else k_lo).shape[1]
    for lens in (hi_lens, lo_lens):
        if lens is not None and (lens.dtype != torch.int32 or lens.numel() != B * Hkv or not lens.is_contiguous()):
            raise ValueError("span lengths must be contiguous int32 with B*Hkv entries")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    S_hi, S_lo = num_splits_hi, num_splits_lo
    if workspace is None:
        if (S_hi <= 0 and L_hi) or (S_lo <= 0 and L_lo):
            auto_hi, auto_lo = attn_decode_mixed_fp4_splits(B, Hkv, L_hi, L_lo)
            S_hi = S_hi if S_hi > 0 else auto_hi
            S_lo = S_lo if S_lo > 0 else auto_lo
        used = (attn_decode_plan(L_hi, S_hi)[0] if L_hi else 0) + (attn_decode_plan(L_lo, S_lo)[0] if L_lo else 0)
        workspace = attn_decode_workspace(B, Hq, d, used, device=q.device)

    def view(t, dtype=None):
        return None if t is None else ctypes.byref(_tensor(t, dtype))

    qt, ot = _tensor(q), _tensor(out)
    st = lib.attn_decode_mixed_fp4(ctypes.byref(qt), view(k_hi), view(v_hi), _ptr(hi_lens), L_hi,
                                   view(k_lo, ATTN_MXFP4), view(v_lo, ATTN_MXFP4), view(k_lo_scale, ATTN_E8M0),
                                   view(v_lo_scale, ATTN_E8M0), _ptr(lo_lens), L_lo, B, Hq, Hkv, d,
                                   float(softmax_scale), int(max(S_hi, 0)), int(max(S_lo, 0)), ctypes.byref(ot),
                                   _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream, q.device))
    _check(st)
    return out, lse


def attn_decode_mixed3_splits(B, Hkv, L_hi_cap, L_mid_cap, L_lo_cap):
    """(S_hi, S_mid, S_lo): the automatic split plan of attn_decode_mixed3."""
    hi, mid, lo = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    total = load_library().attn_decode_mixed3_splits(B, Hkv, L_hi_cap, L_mid_cap, L_lo_cap, ctypes.byref(hi),
                                                     ctypes.byref(mid), ctypes.byref(lo))
    if total <= 0:
        raise AttnError(4, "could not plan splits")
    return hi.value, mid.value, lo.value


def attn_decode_mixed3(q, k_hi, v_hi, k_mid, v_mid, k_lo, v_lo, k_mid_scale=None, v_mid_scale=None, k_lo_scale=None,
                       v_lo_scale=None, hi_lens=None, mid_lens=None, lo_lens=None, softmax_scale=0.0,
                       num_splits_hi=0, num_splits_mid=0, num_splits_lo=0, out=None, lse=None, workspace=None,
                       stream=None):
    """Decode over a cache with a bf16 span (k_hi, v_hi [B,Hkv,L_hi,d]), an fp8-e4m3 span (k_mid, v_mid uint8
    [B,Hkv,L_mid,d] with k_mid_scale, v_mid_scale float32 [B*Hkv]) and an MX fp4 span (k_lo, v_lo uint8
    [B,Hkv,L_lo,d/2] with E8M0 k_lo_scale, v_lo_scale uint8 [B,Hkv,L_lo,d/32]); *_lens int32 [B,Hkv] or None; any
    span may be None. Returns (out [B,Hq,1,d] bf16, lse [B,Hq])."""
    lib = load_library()
    B, Hq, Lq, d = q.shape
    if Lq != 1:
        raise ValueError("attn_decode_mixed3 takes one query per sequence (q.shape[2] == 1)")
    caps = [0 if t is None else t.shape[2] for t in (k_hi, k_mid, k_lo)]
    Hkv = next(t for t in (k_hi, k_mid, k_lo) if t is not None).shape[1]
    for lens in (hi_lens, mid_lens, lo_lens):
        if lens is not None and (lens.dtype != torch.int32 or lens.numel() != B * Hkv or not lens.is_contiguous()):
            raise ValueError("span lengths must be contiguous int32 with B*Hkv entries")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    S = [num_splits_hi, num_splits_mid, num_splits_lo]
    if workspace is None:
        if any(s <= 0 and c for s, c in zip(S, caps)):
            auto = attn_decode_mixed3_splits(B, Hkv, *caps)
            S = [s if s > 0 else a for s, a in zip(S, auto)]
        used = sum(attn_decode_plan(c, s)[0] for s, c in zip(S, caps) if c)
        workspace = attn_decode_workspace(B, Hq, d, used, device=q.device)

    def view(t, dtype=None):
        return None if t is None else ctypes.byref(_tensor(t, dtype))

    qt, ot = _tensor(q), _tensor(out)
    st = lib.attn_decode_mixed3(ctypes.byref(qt), view(k_hi), view(v_hi), _ptr(hi_lens), caps[0],
                                view(k_mid), view(v_mid), _ptr(k_mid_scale),
                                _ptr(v_mid_scale), _ptr(mid_lens), caps[1], view(k_lo, ATTN_MXFP4),
                                view(v_lo, ATTN_MXFP4), view(k_lo_scale, ATTN_E8M0), view(v_lo_scale, ATTN_E8M0),
                                _ptr(lo_lens), caps[2], B, Hq, Hkv, d, float(softmax_scale), int(max(S[0], 0)),
                                int(max(S[1], 0)), int(max(S[2], 0)), ctypes.byref(ot), _ptr(lse), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    _check(st)
    return out, lse


def attn_decode_pi_splits(B, Hkv, L_cap, window, period, kv_dtype=ATTN_BF16):
    """(S_window, S_skip): the automatic split plan of attn_decode_pi."""
    sw, ss = ctypes.c_int(0), ctypes.c_int(0)
    total = load_library().attn_decode_pi_splits(B, Hkv, L_cap, window, period, kv_dtype, ctypes.byref(sw),
                                                 ctypes.byref(ss))
    if total <= 0:
        raise AttnError(4, "could not plan splits")
    return sw.value, ss.value


def attn_decode_pi(q, k, v, window, period, alpha=None, k_scale=None, v_scale=None, kv_lens=None,
                   softmax_scale=0.0, num_splits_window=0, num_splits_skip=0, out=None, lse=None, workspace=None,
                   stream=None):
    """pi-Attention decode: the window of `window` keys before each sequence's query, the keys a whole number of
    `period`s further back, and the gate alpha (float [B*Hq] or None) as a log-prior. q [B,Hq,1,d]; k, v
    [B,Hkv,L_cap,d]. Returns (out, lse)."""
    lib = load_library()
    B, Hq, Lq, d = q.shape
    Hkv, L_cap = k.shape[1], k.shape[2]
    if Lq != 1:
        raise ValueError("attn_decode_pi takes one query per sequence (q.shape[2] == 1)")
    if alpha is not None and (alpha.dtype != torch.float32 or alpha.numel() != B * Hq or not alpha.is_contiguous()):
        raise ValueError("alpha must be contiguous float32 with B*Hq entries")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    sw, ss = num_splits_window, num_splits_skip
    if sw <= 0 or ss <= 0:
        aw, as_ = attn_decode_pi_splits(B, Hkv, L_cap, window, period, _dtype_code(k))
        sw = sw if sw > 0 else aw
        ss = ss if ss > 0 else as_
    if workspace is None:
        cap_w = min(window + 1, L_cap)
        last = L_cap - 2 - window
        cap_s = last // period + 1 if period > 0 and last >= 0 else 0
        S = attn_decode_plan(cap_w, sw)[0] + (attn_decode_plan(cap_s, ss)[0] if cap_s else 0)
        workspace = attn_decode_workspace(B, Hq, d, S, device=q.device)
    qt, kt, vt, ot = _tensor(q), _tensor(k), _tensor(v), _tensor(out)
    st = lib.attn_decode_pi(ctypes.byref(qt), ctypes.byref(kt), ctypes.byref(vt), _ptr(k_scale), _ptr(v_scale),
                            _ptr(kv_lens), B, Hq, Hkv, d, L_cap, float(softmax_scale), int(window), int(period),
                            _ptr(alpha), int(sw), int(ss), ctypes.byref(ot), _ptr(lse), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    _check(st)
    return out, lse


def attn_prefill_pi_workspace_size(B, Hq, L, d):
    return load_library().attn_prefill_pi_workspace_size(B, Hq, L, d)


def attn_prefill_pi(q, k, v, window, period, alpha=None, softmax_scale=0.0, causal=True, out=None, lse=None,
                    workspace=None, stream=None):
    """pi-Attention prefill: window keys i-window..i, skip keys a whole number of `period`s below the window
    (causal=False: window i-window..i+window, skip keys on both sides), alpha (float [B,Hq,L] or None) as a
    log-prior. q [B,Hq,L,d]; k, v [B,Hkv,L,d] bf16. Returns (out, lse)."""
    lib = load_library()
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    if k.shape[2] != L:
        raise ValueError("attn_prefill_pi takes as many keys as queries")
    if alpha is not None and (alpha.dtype != torch.float32 or alpha.numel() != B * Hq * L or not alpha.is_contiguous()):
        raise ValueError("alpha must be contiguous float32 with B*Hq*L entries")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(lib.attn_prefill_pi_workspace_size(B, Hq, L, d), dtype=torch.uint8, device=q.device)
    qt, kt, vt, ot = _tensor(q), _tensor(k), _tensor(v), _tensor(out)
    st = lib.attn_prefill_pi(ctypes.byref(qt), ctypes.byref(kt), ctypes.byref(vt), B, Hq, Hkv, d, L,
                             float(softmax_scale), int(bool(causal)), int(window), int(period), _ptr(alpha),
                             ctypes.byref(ot), _ptr(lse),
                             _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    _check(st)
    return out, lse


def attn_prefill_backward_workspace_size(B, Hq, Lq):
    return load_library().attn_prefill_backward_workspace_size(B, Hq, Lq)


def attn_prefill_backward(q, k, v, out, lse, dout, causal=True, softmax_scale=0.0, dq=None, dk=None, dv=None,
                          grad_dtype=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of attn_prefill for output gradient dout; out and lse are the forward's results."""
    lib = load_library()
    B, Hq, Lq, d = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    gd = grad_dtype or q.dtype
    if dq is None:
        dq = torch.empty(q.shape, dtype=gd, device=q.device)
    if dk is None:
        dk = torch.empty(k.shape, dtype=gd, device=q.device)
    if dv is None:
        dv = torch.empty(v.shape, dtype=gd, device=q.device)
    if not lse.is_contiguous() or lse.dtype != torch.float32 or lse.numel() != B * Hq * Lq:
        raise ValueError("lse must be the forward's contiguous float32 [B, Hq, Lq]")
    if workspace is None:
        workspace = torch.empty(lib.attn_prefill_backward_workspace_size(B, Hq, Lq), dtype=torch.uint8, device=q.device)
    ts = [_tensor(t) for t in (q, k, v, out, dout, dq, dk, dv)]
    st = lib.attn_prefill_backward(ctypes.byref(ts[0]), ctypes.byref(ts[1]), ctypes.byref(ts[2]), ctypes.byref(ts[3]),
                                   _ptr(lse), ctypes.byref(ts[4]), B, Hq, Hkv, d, Lq, Lkv, float(softmax_scale),
                                   int(bool(causal)), ctypes.byref(ts[5]), ctypes.byref(ts[6]), ctypes.byref(ts[7]),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream, q.device))
    _check(st)
    return dq, dk, dv
