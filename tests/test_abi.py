"""The C ABI on the CPU: libattn.so loads, exports every function that
include/attn.h declares, and rejects bad arguments with the documented status
codes before touching the GPU (so these run without one)."""
import ctypes
import os
import re
import subprocess

import pytest

import long_context_decode_kv_amd as lib
from long_context_decode_kv_amd import attn_tensor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, 1, 2, 3, 4
F32, BF16, FP8, MXFP4, E8M0 = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def so():
    if not os.path.exists(lib.library_path):
        from long_context_decode_kv_amd import build
        build.build()
    return lib.load_library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    return re.findall(r"ATTN_API\s+[\w\s\*]+?\b(attn_\w+)\s*\(", text)


def test_every_declared_symbol_is_exported(so):
    names = declared_functions()
    assert set(names) == {"attn_status_string", "attn_last_error", "attn_decode_auto_splits",
                          "attn_decode_workspace_size", "attn_decode_workspace_init", "attn_decode_plan",
                          "attn_decode", "attn_decode_partials", "attn_prefill", "attn_combine_partials",
                          "attn_decode_mixed", "attn_decode_mixed_splits", "attn_decode_mixed_fp4",
                          "attn_decode_mixed_fp4_splits", "attn_decode_pi",
                          "attn_decode_pi_splits", "attn_prefill_pi", "attn_prefill_pi_workspace_size",
                          "attn_prefill_backward", "attn_prefill_backward_workspace_size",
                          "attn_decode_noalloc", "attn_decode_mixed3", "attn_decode_mixed3_splits"}
    nm = subprocess.run(["nm", "-D", "--defined-only", lib.library_path], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in nm.splitlines() if line.strip()}
    for n in names:
        assert n in exported, n
        assert getattr(so, n) is not None
    # nothing else named attn_* leaks out
    assert {e for e in exported if e.startswith("attn_")} == set(names)


def test_no_undefined_library_symbols(so):
    # Every symbol of the library's own namespace is defined in it: a kernel
    # template whose host-side launch stub was not emitted would otherwise
    # link and only fail when the library is loaded (with RTLD_NOW) or launched.
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib.library_path], capture_output=True, text=True).stdout
    undefined = [line.split()[-1] for line in nm.splitlines() if line.strip()]
    assert not [u for u in undefined if "4attn" in u or u.startswith("attn_")], undefined


def test_status_strings(so):
    assert [lib.attn_status_string(s) for s in range(5)] == [
        "ATTN_OK", "ATTN_ERR_INVALID_ARG", "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_WORKSPACE", "ATTN_ERR_HIP"]


def test_split_plan(so):
    # chunk = roundup(ceil(L/S), 64); S_used = ceil(L/chunk)
    assert lib.attn_decode_plan(131072, 256) == (256, 512)
    assert lib.attn_decode_plan(131072, 100) == (98, 1344)
    assert lib.attn_decode_plan(1024, 4) == (4, 256)
    assert lib.attn_decode_plan(1000, 7) == (6, 192)
    assert lib.attn_decode_plan(100, 64) == (2, 64)
    assert lib.attn_decode_plan(0, 4)[0] == 0 and lib.attn_decode_plan(10, 0)[0] == 0
    for L in (1, 63, 64, 65, 1000, 65536, 1 << 20):
        for S in (1, 2, 3, 7, 64, 1000):
            used, chunk = lib.attn_decode_plan(L, S)
            assert chunk % 64 == 0 and used <= S and (used - 1) * chunk < L <= used * chunk


def test_workspace_size(so):
    # a fixed 4 MiB block of merge counters, then the fp32 partials
    assert lib.attn_decode_workspace_size(1, 32, 128, 256) == (4 << 20) + 32 * 256 * 130 * 4 + 32 * 16 * 130 * 4
    assert lib.attn_decode_workspace_size(16, 32, 128, 0) == 0
    assert lib.attn_decode_workspace_size(0, 32, 128, 4) == 0


FAKE = 0x100000  # never dereferenced: validation fails first


def T(dtype, sb, sh, ss, data=FAKE):
    return attn_tensor(data, dtype, sb, sh, ss)


def decode(so, q=None, k=None, v=None, ks=None, vs=None, B=1, Hq=8, Hkv=2, d=128, L=1024, S=4, out=None,
           ws=FAKE, ws_bytes=1 << 30, scale=0.0):
    q = q or T(BF16, Hq * d, d, d)
    k = k or T(BF16, Hkv * L * d, L * d, d)
    v = v or T(BF16, Hkv * L * d, L * d, d)
    out = out or T(BF16, Hq * d, d, d)
    return so.attn_decode(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ks, vs, None, B, Hq, Hkv, d, L,
                          scale, 0, S, ctypes.byref(out), None, ws, ws_bytes, None)


def test_decode_argument_errors(so):
    assert decode(so, q=T(BF16, 1024, 128, 128, data=0)) == INVALID
    assert decode(so, Hq=6, Hkv=4) == INVALID
    assert decode(so, B=0) == INVALID
    assert decode(so, S=-1) == INVALID
    assert decode(so, scale=float("nan")) == INVALID
    assert decode(so, d=96) == UNSUPPORTED
    assert decode(so, Hq=6, Hkv=2) == UNSUPPORTED  # 3 query heads per KV head
    assert decode(so, k=T(FP8, 2 * 1024 * 128, 1024 * 128, 128), v=T(FP8, 2 * 1024 * 128, 1024 * 128, 128)) == INVALID
    assert decode(so, ks=FAKE, vs=FAKE) == INVALID  # scales with bf16 k/v
    # rows are read in 32-row tiles with 32-bit byte offsets on the grouped-query path
    big8 = T(FP8, 2 * 1024 * (1 << 26), 1024 * (1 << 26), 1 << 26)
    assert decode(so, k=big8, v=big8, ks=FAKE, vs=FAKE) == INVALID
    assert "2^26" in lib.load_library().attn_last_error().decode()
    big16 = T(BF16, 2 * 1024 * (1 << 25), 1024 * (1 << 25), 1 << 25)  # 2^26 bytes a row
    assert decode(so, k=big16, v=big16) == INVALID
    assert decode(so, k=T(F32, 2 * 1024 * 128, 1024 * 128, 128)) == INVALID  # k and v dtypes differ
    assert decode(so, q=T(BF16, 1024, 128, 128, data=FAKE + 2)) == INVALID  # misaligned
    assert decode(so, k=T(BF16, 2 * 1024 * 129, 1024 * 129, 129)) == INVALID
    assert decode(so, ws=None) == WORKSPACE
    assert decode(so, ws_bytes=100) == WORKSPACE
    assert decode(so, ws_bytes=(4 << 20) + 8 * 16 * 130 * 4 + 100) == WORKSPACE
    assert decode(so, ws=FAKE + 4) == WORKSPACE
    assert decode(so, out=T(F32, 1024, 128, 128)) == INVALID  # out dtype must equal q dtype
    # MX fp4 codes and E8M0 scales are not decode inputs: rejected before any launch
    fp4 = T(MXFP4, 2 * 1024 * 64, 1024 * 64, 64)
    assert decode(so, k=fp4, v=fp4) == UNSUPPORTED
    e8 = T(E8M0, 2 * 1024 * 16, 1024 * 16, 16)
    assert decode(so, k=e8, v=e8) == UNSUPPORTED
    assert decode(so, q=T(MXFP4, 1024, 128, 128), out=T(MXFP4, 1024, 128, 128)) == UNSUPPORTED
    assert decode(so, q=T(E8M0, 1024, 128, 128), out=T(E8M0, 1024, 128, 128)) == UNSUPPORTED


def noalloc(so, B=1, Hq=8, Hkv=2, d=128, L=1024, S=4):
    q = T(BF16, Hq * d, d, d)
    k = T(BF16, Hkv * L * d, L * d, d)
    out = T(BF16, Hq * d, d, d)
    return so.attn_decode_noalloc(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), None, None, None, B, Hq, Hkv, d,
                                  L, 0.0, 0, S, ctypes.byref(out), None, None)


def test_decode_noalloc_argument_errors(so):
    assert noalloc(so, B=0) == INVALID
    assert noalloc(so, S=-1) == INVALID
    # the fixed array holds 32 MiB: 4 MiB of counters, then (S + 16) partials of d + 2 floats per query row
    limit = 32 << 20
    assert lib.attn_decode_workspace_size(1, 32, 128, 1024) <= limit
    assert lib.attn_decode_workspace_size(1, 32, 128, 2048) > limit
    assert noalloc(so, Hq=32, Hkv=8, L=1 << 20, S=2048) == WORKSPACE  # before any device query or launch
    msg = lib.load_library().attn_last_error().decode()
    assert "2048 splits" in msg and "scratch" in msg
    assert noalloc(so, B=16, Hq=32, Hkv=8, L=65536, S=128) == WORKSPACE


def partials(so, q=None, k=None, B=1, Hq=8, Hkv=2, d=128, L=1024, S=4):
    q = q or T(BF16, Hq * d, d, d)
    k = k or T(BF16, Hkv * L * d, L * d, d)
    used = ctypes.c_int(0)
    return so.attn_decode_partials(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), None, None, None, B, Hq, Hkv,
                                   d, L, 0.0, 0, S, FAKE, FAKE, FAKE, ctypes.byref(used), None)


def test_decode_partials_argument_errors(so):
    assert partials(so, B=0) == INVALID
    assert partials(so, d=96) == UNSUPPORTED
    assert partials(so, k=T(MXFP4, 2 * 1024 * 64, 1024 * 64, 64)) == UNSUPPORTED
    assert partials(so, k=T(E8M0, 2 * 1024 * 16, 1024 * 16, 16)) == UNSUPPORTED
    assert partials(so, q=T(MXFP4, 1024, 128, 128)) == UNSUPPORTED
    assert partials(so, q=T(E8M0, 1024, 128, 128)) == UNSUPPORTED


def test_workspace_init_errors(so):
    assert so.attn_decode_workspace_init(None, 1 << 20, None) == WORKSPACE
    assert so.attn_decode_workspace_init(FAKE, 1000, None) == WORKSPACE


def test_error_message_names_the_problem(so):
    assert decode(so, ws_bytes=(4 << 20) + 8 * 16 * 130 * 4 + 100) == WORKSPACE
    msg = lib.load_library().attn_last_error().decode()
    assert "workspace" in msg and "need" in msg


def prefill(so, dtype=BF16, d=128, Lq=256, Lkv=256, causal=1, Hq=8, Hkv=2, q_ss=None):
    q = T(dtype, Hq * Lq * d, Lq * d, q_ss or d)
    k = T(dtype, Hkv * Lkv * d, Lkv * d, d)
    o = T(dtype, Hq * Lq * d, Lq * d, d)
    return so.attn_prefill(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), 1, Hq, Hkv, d, Lq, Lkv, 0.0, causal,
                           ctypes.byref(o), None, None)


def test_prefill_argument_errors(so):
    assert prefill(so, Lq=300, Lkv=200, causal=1) == INVALID
    assert prefill(so, dtype=FP8) == UNSUPPORTED
    assert prefill(so, d=96) == UNSUPPORTED
    assert prefill(so, Hq=6, Hkv=4) == INVALID
    assert prefill(so, Lq=0) == INVALID
    assert prefill(so, q_ss=1 << 24) == UNSUPPORTED  # Q rows are read through 32-bit buffer offsets


def test_combine_argument_errors(so):
    out = T(BF16, 0, 0, 128)
    assert so.attn_combine_partials(None, FAKE, FAKE, 4, 2, 128, ctypes.byref(out), None, None) == INVALID
    assert so.attn_combine_partials(FAKE, FAKE, FAKE, 0, 2, 128, ctypes.byref(out), None, None) == INVALID
    bad = T(FP8, 0, 0, 128)
    assert so.attn_combine_partials(FAKE, FAKE, FAKE, 4, 2, 128, ctypes.byref(bad), None, None) == UNSUPPORTED


def mixed(so, q=None, khi=None, klo=None, ks=FAKE, vs=FAKE, B=1, Hq=8, Hkv=2, d=128, L_hi=256, L_lo=1024, S_hi=2,
          S_lo=4, out=None, ws=FAKE, ws_bytes=1 << 30, no_hi=False):
    q = q or T(BF16, Hq * d, d, d)
    khi = None if no_hi else (khi or T(BF16, Hkv * L_hi * d, L_hi * d, d))
    klo = klo or T(FP8, Hkv * L_lo * d, L_lo * d, d)
    out = out or T(BF16, Hq * d, d, d)
    ref = lambda t: None if t is None else ctypes.byref(t)
    return so.attn_decode_mixed(ctypes.byref(q), ref(khi), ref(khi), None, L_hi, ref(klo), ref(klo), ks, vs, None,
                                L_lo, B, Hq, Hkv, d, 0.0, S_hi, S_lo, ctypes.byref(out), None, ws, ws_bytes, None)


def test_mixed_decode_argument_errors(so):
    assert mixed(so, L_hi=0, L_lo=0) == INVALID
    assert mixed(so, L_hi=-1) == INVALID
    assert mixed(so, S_hi=-1) == INVALID
    assert mixed(so, ks=None) == INVALID  # the fp8 span needs its scales
    assert mixed(so, khi=T(FP8, 2 * 256 * 128, 256 * 128, 128)) == UNSUPPORTED  # bf16 span holds fp8
    assert mixed(so, klo=T(BF16, 2 * 1024 * 128, 1024 * 128, 128)) == UNSUPPORTED  # fp8 span holds bf16
    assert mixed(so, Hq=6, Hkv=2) == UNSUPPORTED  # 3 query heads per KV head
    assert mixed(so, d=96) == UNSUPPORTED
    assert mixed(so, out=T(F32, 1024, 128, 128)) == UNSUPPORTED
    assert mixed(so, Hq=6, Hkv=4) == INVALID
    assert mixed(so, klo=T(FP8, 2 * 1024 * (1 << 26), 1024 * (1 << 26), 1 << 26)) == INVALID  # 32-row tile offsets
    assert mixed(so, ws=None) == WORKSPACE
    # 2 + 4 splits: counters, then (d + 2) floats per split and per block partial
    need = (4 << 20) + 8 * 6 * 130 * 4 + 8 * 16 * 130 * 4
    assert lib.attn_decode_workspace_size(1, 8, 128, 6) == need
    assert mixed(so, ws_bytes=need - 1) == WORKSPACE
    assert "6 splits" in lib.load_library().attn_last_error().decode()
    # an empty span may come without tensors
    assert mixed(so, L_hi=0, S_hi=0, no_hi=True, ws=None) == WORKSPACE  # validation reaches the workspace check
    assert mixed(so, L_hi=16, no_hi=True) == INVALID


_DEFAULT = object()


def mixed_fp4(so, klo=_DEFAULT, ksc=_DEFAULT, vsc=_DEFAULT, B=1, Hq=8, Hkv=2, d=128, L_hi=256, L_lo=1024, S_hi=2,
              S_lo=4, out=None, ws=FAKE, ws_bytes=1 << 30, no_lo=False):
    q = T(BF16, Hq * d, d, d)
    khi = T(BF16, Hkv * L_hi * d, L_hi * d, d)
    pick = lambda x, dflt: None if no_lo else (dflt if x is _DEFAULT else x)
    klo = pick(klo, T(MXFP4, Hkv * L_lo * d // 2, L_lo * d // 2, d // 2))
    ksc = pick(ksc, T(E8M0, Hkv * L_lo * 4, L_lo * 4, 4))
    vsc = pick(vsc, T(E8M0, Hkv * L_lo * 4, L_lo * 4, 4))
    out = out or T(BF16, Hq * d, d, d)
    ref = lambda t: None if t is None else ctypes.byref(t)
    return so.attn_decode_mixed_fp4(ctypes.byref(q), ref(khi), ref(khi), None, L_hi, ref(klo), ref(klo), ref(ksc),
                                    ref(vsc), None, L_lo, B, Hq, Hkv, d, 0.0, S_hi, S_lo, ctypes.byref(out), None, ws,
                                    ws_bytes, None)


def test_mixed_fp4_decode_argument_errors(so):
    assert mixed_fp4(so, L_hi=0, L_lo=0) == INVALID
    assert mixed_fp4(so, S_lo=-1) == INVALID
    assert mixed_fp4(so, ksc=None) == INVALID  # the fp4 span needs its scales
    assert mixed_fp4(so, ksc=T(FP8, 2 * 1024 * 4, 1024 * 4, 4)) == INVALID  # scales of the wrong dtype
    assert mixed_fp4(so, vsc=T(E8M0, 2 * 1024 * 4, 1024 * 4, 6)) == INVALID  # row stride not a multiple of 4
    assert mixed_fp4(so, ksc=T(E8M0, 0, 0, 4, data=FAKE + 2)) == INVALID  # misaligned scales
    assert mixed_fp4(so, klo=T(FP8, 2 * 1024 * 128, 1024 * 128, 128)) == UNSUPPORTED  # fp4 span holds fp8
    assert mixed_fp4(so, klo=T(MXFP4, 0, 0, 72)) == INVALID  # code rows must be 16-byte multiples
    assert mixed_fp4(so, klo=T(MXFP4, 0, 0, 1 << 26)) == INVALID  # row stride too large for the tile offsets
    assert mixed_fp4(so, d=64) == UNSUPPORTED
    assert mixed_fp4(so, Hq=6, Hkv=2) == UNSUPPORTED
    assert mixed_fp4(so, ws=None) == WORKSPACE
    assert mixed_fp4(so, ws_bytes=lib.attn_decode_workspace_size(1, 8, 128, 6) - 1) == WORKSPACE
    assert "6 splits" in lib.load_library().attn_last_error().decode()
    assert mixed_fp4(so, L_lo=0, S_lo=0, no_lo=True, ws=None) == WORKSPACE  # no fp4 span: bf16 only
    assert mixed_fp4(so, L_lo=16, no_lo=True) == INVALID


def pi(so, kv=BF16, ks=None, vs=None, B=1, Hq=8, Hkv=2, d=128, L=4096, window=512, period=16, Sw=2, Ss=2, out=None,
       ws=FAKE, ws_bytes=1 << 30):
    q = T(BF16, Hq * d, d, d)
    k = T(kv, Hkv * L * d, L * d, d)
    out = out or T(BF16, Hq * d, d, d)
    return so.attn_decode_pi(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), ks, vs, None, B, Hq, Hkv, d, L, 0.0,
                             window, period, None, Sw, Ss, ctypes.byref(out), None, ws, ws_bytes, None)


def test_pi_decode_argument_errors(so):
    assert pi(so, window=-1) == INVALID
    assert pi(so, period=-2) == INVALID
    assert pi(so, Sw=-1) == INVALID
    assert pi(so, L=0) == INVALID
    assert pi(so, kv=FP8) == INVALID  # fp8 without scales
    assert pi(so, ks=FAKE, vs=FAKE) == INVALID  # scales with bf16
    assert pi(so, kv=F32) == UNSUPPORTED
    # fp8 skip keys are read 32 at a time, period rows apart, with 32-bit byte offsets
    assert pi(so, kv=FP8, ks=FAKE, vs=FAKE, period=1 << 19) == INVALID
    assert "2^26" in lib.load_library().attn_last_error().decode()
    assert pi(so, kv=FP8, ks=FAKE, vs=FAKE, period=(1 << 19) - 1, ws=None) == WORKSPACE  # within the limit
    assert pi(so, period=1 << 18) == INVALID  # bf16: 256-byte rows
    assert pi(so, period=(1 << 18) - 1, ws=None) == WORKSPACE
    assert pi(so, d=96) == UNSUPPORTED
    assert pi(so, Hq=6) == UNSUPPORTED
    assert pi(so, out=T(F32, 1024, 128, 128)) == UNSUPPORTED
    assert pi(so, ws=None) == WORKSPACE
    # window 513 keys in 2 splits, (4096 - 2 - 512) // 16 + 1 = 224 skip keys in 2 splits
    need = lib.attn_decode_workspace_size(1, 8, 128, 4)
    assert pi(so, ws_bytes=need - 1) == WORKSPACE
    assert "4 splits" in lib.load_library().attn_last_error().decode()
    # no skip keys at all (period 0, or a window covering the cache): one span
    assert pi(so, period=0, ws_bytes=lib.attn_decode_workspace_size(1, 8, 128, 2) - 1) == WORKSPACE
    assert "2 splits" in lib.load_library().attn_last_error().decode()
    assert pi(so, window=5000, ws_bytes=lib.attn_decode_workspace_size(1, 8, 128, 2) - 1) == WORKSPACE
    # a window far past the cache is the whole cache (no overflow in the plan)
    assert pi(so, window=2 ** 31 - 1, ws_bytes=lib.attn_decode_workspace_size(1, 8, 128, 2) - 1) == WORKSPACE


def pi_prefill(so, dtype=BF16, d=128, L=256, Hq=8, Hkv=2, window=16, period=4, ws=FAKE, ws_bytes=1 << 30, causal=1):
    q = T(dtype, Hq * L * d, L * d, d)
    k = T(dtype, Hkv * L * d, L * d, d)
    o = T(dtype, Hq * L * d, L * d, d)
    return so.attn_prefill_pi(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), 1, Hq, Hkv, d, L, 0.0, causal,
                              window, period, None, ctypes.byref(o), None, ws, ws_bytes, None)


def test_pi_prefill_argument_errors(so):
    assert pi_prefill(so, window=-1) == INVALID
    assert pi_prefill(so, period=-1) == INVALID
    assert pi_prefill(so, L=0) == INVALID
    assert pi_prefill(so, dtype=F32) == UNSUPPORTED
    assert pi_prefill(so, d=96) == UNSUPPORTED  # head dims 64 and 128 run (not launched here)
    assert pi_prefill(so, period=1 << 17) == UNSUPPORTED  # strided rows past the 32-bit buffer offsets
    assert pi_prefill(so, ws=None) == WORKSPACE
    # the window part's lse, rounded up to 256 bytes
    need = lib.attn_prefill_pi_workspace_size(1, 8, 256, 128)
    assert need == 8 * 256 * 4
    assert pi_prefill(so, ws_bytes=need - 1) == WORKSPACE
    assert lib.attn_prefill_pi_workspace_size(0, 8, 256, 128) == 0
    assert pi_prefill(so, causal=0, window=-1) == INVALID
    assert pi_prefill(so, causal=0, ws=None) == WORKSPACE
    assert pi_prefill(so, causal=0, ws_bytes=need - 1) == WORKSPACE


def backward(so, dtype=BF16, gdt=F32, d=128, Lq=256, Lkv=256, causal=1, Hq=8, Hkv=2, lse=FAKE, ws=FAKE,
             ws_bytes=1 << 30):
    q = T(dtype, Hq * Lq * d, Lq * d, d)
    k = T(dtype, Hkv * Lkv * d, Lkv * d, d)
    g = T(gdt, Hq * Lq * d, Lq * d, d)
    gk = T(gdt, Hkv * Lkv * d, Lkv * d, d)
    return so.attn_prefill_backward(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), ctypes.byref(q), lse,
                                    ctypes.byref(q), 1, Hq, Hkv, d, Lq, Lkv, 0.0, causal, ctypes.byref(g),
                                    ctypes.byref(gk), ctypes.byref(gk), ws, ws_bytes, None)


def test_backward_argument_errors(so):
    assert backward(so, lse=None) == INVALID
    assert backward(so, Lq=300, Lkv=200) == INVALID
    assert backward(so, dtype=F32) == UNSUPPORTED
    assert backward(so, d=64) == UNSUPPORTED
    assert backward(so, gdt=FP8) == UNSUPPORTED
    assert backward(so, ws=None) == WORKSPACE
    need = lib.attn_prefill_backward_workspace_size(1, 8, 256)
    assert need == 8 * 256 * 4
    assert backward(so, ws_bytes=need - 1) == WORKSPACE


def mixed3(so, L_hi=256, L_mid=512, L_lo=1024, mid_dtype=FP8, lo_dtype=MXFP4, ks=FAKE, ksc=True, S=(2, 2, 4), B=1,
           Hq=8, Hkv=2, d=128, out=None, ws=FAKE, ws_bytes=1 << 30):
    q = T(BF16, Hq * d, d, d)
    khi = T(BF16, Hkv * L_hi * d, L_hi * d, d)
    kmid = T(mid_dtype, Hkv * L_mid * d, L_mid * d, d)
    klo = T(lo_dtype, Hkv * L_lo * d // 2, L_lo * d // 2, d // 2)
    sc = T(E8M0, Hkv * L_lo * 4, L_lo * 4, 4) if ksc else None
    out = out or T(BF16, Hq * d, d, d)
    ref = lambda t: None if t is None else ctypes.byref(t)
    return so.attn_decode_mixed3(ctypes.byref(q), ref(khi), ref(khi), None, L_hi, ref(kmid), ref(kmid), ks, ks, None,
                                 L_mid, ref(klo), ref(klo), ref(sc), ref(sc), None, L_lo, B, Hq, Hkv, d, 0.0, S[0], S[1],
                                 S[2], ctypes.byref(out), None, ws, ws_bytes, None)


def test_mixed3_decode_argument_errors(so):
    assert mixed3(so, L_hi=0, L_mid=0, L_lo=0) == INVALID
    assert mixed3(so, L_mid=-1) == INVALID
    assert mixed3(so, S=(1, -1, 1)) == INVALID
    assert mixed3(so, ks=None) == INVALID  # the fp8 span needs its scales
    assert mixed3(so, ksc=False) == INVALID  # the fp4 span needs its scales
    assert mixed3(so, mid_dtype=BF16) == UNSUPPORTED
    assert mixed3(so, lo_dtype=FP8) == UNSUPPORTED
    assert mixed3(so, Hq=6) == UNSUPPORTED
    assert mixed3(so, d=64) == UNSUPPORTED
    assert mixed3(so, out=T(F32, 1024, 128, 128)) == UNSUPPORTED
    assert mixed3(so, ws=None) == WORKSPACE
    need = lib.attn_decode_workspace_size(1, 8, 128, 8)  # 2 + 2 + 4 splits
    assert mixed3(so, ws_bytes=need - 1) == WORKSPACE
    assert "8 splits" in lib.load_library().attn_last_error().decode()
    # a span without keys takes no splits
    assert mixed3(so, L_mid=0, ws_bytes=lib.attn_decode_workspace_size(1, 8, 128, 6) - 1) == WORKSPACE
    assert "6 splits" in lib.load_library().attn_last_error().decode()
