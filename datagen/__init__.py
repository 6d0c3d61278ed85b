"""Seeded synthetic inputs shared by the tests, ``smoke()`` and ``bench.py``.

Holds no attention arithmetic: it only draws numbers (counter-based SplitMix64
stream + Box-Muller, see ``datagen.c``) and encodes them into the storage
formats the library reads. Random numbers never come from the GPU path.

Tensor ids used by the workloads: Q=0, K=1, V=2, per-sequence lengths=3; the
low-precision span of a two-precision cache: K=4, V=5, its lengths=6; the
pi-Attention gate alpha=7; the output gradient of the backward pass=9; the
fp8 span of a three-precision cache: K=10, V=11, its lengths=12.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdatagen.so")
_lib = None

TID_Q, TID_K, TID_V, TID_LENS = 0, 1, 2, 3
TID_K_LO, TID_V_LO, TID_LENS_LO = 4, 5, 6
TID_DOUT = 9
TID_K_MID, TID_V_MID, TID_LENS_MID = 10, 11, 12


def build():
    """Compile ``datagen.c`` into ``libdatagen.so`` (plain gcc)."""
    src = os.path.join(_HERE, "datagen.c")
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-o", _LIB_PATH, src, "-lm", "-lpthread"]
    subprocess.check_call(cmd)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    src = os.path.join(_HERE, "datagen.c")
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.dg_normal_f64.argtypes = [u64, u64, u64, dbl, vp, i32]
    lib.dg_fill_f32.argtypes = [u64, u64, u64, dbl, vp, i32]
    lib.dg_fill_bf16.argtypes = [u64, u64, u64, dbl, vp, i32]
    lib.dg_fill_e4m3.argtypes = [u64, u64, u64, u64, dbl, vp, vp, i32]
    lib.dg_uniform_int.argtypes = [u64, u64, u64, ctypes.c_int32, ctypes.c_int32, vp]
    lib.dg_words.argtypes = [u64, u64, u64, vp]
    lib.dg_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.dg_f32_to_bf16.restype = ctypes.c_uint16
    lib.dg_f32_to_e4m3.argtypes = [ctypes.c_float]
    lib.dg_f32_to_e4m3.restype = ctypes.c_uint8
    lib.dg_f32_to_e2m1.argtypes = [ctypes.c_float]
    lib.dg_f32_to_e2m1.restype = ctypes.c_uint8
    lib.dg_fill_mxfp4.argtypes = [u64, u64, u64, u64, dbl, vp, vp, i32]
    _lib = lib
    return lib


def _threads():
    n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def normal_f64(seed, tensor_id, shape, mul=1.0):
    out = np.empty(shape, dtype=np.float64)
    _load().dg_normal_f64(seed, tensor_id, out.size, mul, _ptr(out), _threads())
    return out


def normal_f32(seed, tensor_id, shape, mul=1.0):
    out = np.empty(shape, dtype=np.float32)
    _load().dg_fill_f32(seed, tensor_id, out.size, mul, _ptr(out), _threads())
    return out


def normal_bf16_bits(seed, tensor_id, shape, mul=1.0):
    """bf16 bit patterns (uint16) of N(0,1)*mul."""
    out = np.empty(shape, dtype=np.uint16)
    _load().dg_fill_bf16(seed, tensor_id, out.size, mul, _ptr(out), _threads())
    return out


def normal_e4m3(seed, tensor_id, shape, mul=1.0):
    """fp8-e4m3 codes (uint8) of N(0,1)*mul, one fp32 scale per leading slice.

    ``shape`` is (..., L, d); every (…) index (one batch row and KV head) is a
    group with scale = amax/448 over its L*d values. Returns (codes, scales)."""
    per_group = int(shape[-1]) * int(shape[-2])
    groups = int(np.prod(shape[:-2])) if len(shape) > 2 else 1
    out = np.empty(shape, dtype=np.uint8)
    scales = np.empty(shape[:-2] if len(shape) > 2 else (1,), dtype=np.float32)
    _load().dg_fill_e4m3(seed, tensor_id, groups, per_group, mul, _ptr(out), _ptr(scales), _threads())
    return out, scales


def normal_mxfp4(seed, tensor_id, shape, mul=1.0):
    """OCP MX fp4 of N(0,1)*mul (the values normal_f32 draws for ``shape``):
    ``shape`` is (..., d) with d a multiple of 32; every 32 consecutive values
    of the last dimension share a power-of-two scale 2^X, X = floor(log2 amax)
    - 2, stored as the E8M0 byte X + 127, and each value is the E2M1 code of
    x / 2^X (nearest, ties to even, saturating to 6), two codes per byte with
    element 2i in the low nibble of byte i. Returns (codes (..., d/2) uint8,
    scales (..., d/32) uint8)."""
    d = int(shape[-1])
    if d % 32:
        raise ValueError("d must be a multiple of 32")
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    codes = np.empty(tuple(shape[:-1]) + (d // 2,), dtype=np.uint8)
    scales = np.empty(tuple(shape[:-1]) + (d // 32,), dtype=np.uint8)
    if rows:
        _load().dg_fill_mxfp4(seed, tensor_id, rows, d, mul, _ptr(codes), _ptr(scales), _threads())
    return codes, scales


def uniform_int(seed, tensor_id, n, lo, hi):
    out = np.empty(n, dtype=np.int32)
    _load().dg_uniform_int(seed, tensor_id, n, lo, hi, _ptr(out))
    return out


def uniform_f32(seed, tensor_id, shape, lo, hi):
    """float32 uniform in [lo, hi): the top 53 bits of each stream word as a
    fraction in [0, 1)."""
    n = int(np.prod(shape))
    u = (words(seed, tensor_id, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    return (lo + (hi - lo) * u).astype(np.float32).reshape(shape)


def words(seed, tensor_id, n):
    out = np.empty(n, dtype=np.uint64)
    _load().dg_words(seed, tensor_id, n, _ptr(out))
    return out


def f32_to_bf16_bits(x):
    """Encode an fp32 array into bf16 bit patterns (RNE)."""
    lib = _load()
    x = np.asarray(x, dtype=np.float32)
    return np.array([lib.dg_f32_to_bf16(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def f32_to_e2m1(x):
    """Encode an fp32 array into E2M1 codes (0..15; nearest, ties to even,
    saturating to +-6)."""
    lib = _load()
    x = np.asarray(x, dtype=np.float32)
    return np.array([lib.dg_f32_to_e2m1(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def f32_to_e4m3(x):
    """Encode an fp32 array into e4m3 codes (RNE, saturating to +-448)."""
    lib = _load()
    x = np.asarray(x, dtype=np.float32)
    return np.array([lib.dg_f32_to_e4m3(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)
