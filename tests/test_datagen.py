"""The seeded input generator: reproducible, independent of thread count, and
its encoders agree with torch's own storage-format conversions."""
import numpy as np
import torch

import datagen

MASK = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15


def _mix(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def test_words_are_the_splitmix64_stream():
    # SplitMix64 (Steele, Lea, Flood 2014): state += golden gamma, output = mix(state).
    seed, tid = 5, 2
    state = _mix(_mix(seed) ^ (((tid + 1) * GOLDEN) & MASK))
    ref = []
    for _ in range(64):
        state = (state + GOLDEN) & MASK
        ref.append(_mix(state))
    assert datagen.words(seed, tid, 64).tolist() == ref


def test_normals_have_unit_moments_and_are_reproducible():
    x = datagen.normal_f64(3, 1, (1 << 20,))
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3
    assert np.array_equal(x, datagen.normal_f64(3, 1, (1 << 20,)))
    assert not np.array_equal(x[:1000], datagen.normal_f64(3, 2, (1000,)))
    assert not np.array_equal(x[:1000], datagen.normal_f64(4, 1, (1000,)))


def test_thread_count_does_not_change_values():
    lib = datagen._load()
    a = np.empty(100003, np.uint16)
    b = np.empty(100003, np.uint16)
    lib.dg_fill_bf16(9, 1, a.size, 0.5, datagen._ptr(a), 1)
    lib.dg_fill_bf16(9, 1, b.size, 0.5, datagen._ptr(b), 7)
    assert np.array_equal(a, b)


def test_fills_are_roundings_of_the_normals():
    x = datagen.normal_f64(11, 0, (4096,), mul=0.5)
    f = datagen.normal_f32(11, 0, (4096,), mul=0.5)
    assert np.array_equal(f, x.astype(np.float32))
    b = datagen.normal_bf16_bits(11, 0, (4096,), mul=0.5)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_bf16_encoder_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(5000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 5000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 3.0e38, 1e-40], np.float32)])
    x = x.astype(np.float32)
    ours = datagen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_encoder_matches_torch_in_range_and_saturates():
    rng = np.random.default_rng(1)
    grid = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    finite = np.sort(grid[np.isfinite(grid)])
    mids = ((finite[1:].astype(np.float64) + finite[:-1]) / 2).astype(np.float32)  # ties: exactly representable
    x = np.concatenate([finite, mids, rng.uniform(-464, 464, 20000).astype(np.float32),
                        rng.standard_normal(5000).astype(np.float32) * 1e-2]).astype(np.float32)
    ours = datagen.f32_to_e4m3(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps the sign of zero; so do we
    assert np.array_equal(ours, ref)
    sat = datagen.f32_to_e4m3(np.array([470.0, 1e6, -500.0], np.float32))
    assert sat.tolist() == [0x7E, 0x7E, 0xFE]


def test_e4m3_groups_use_amax_scale():
    codes, scales = datagen.normal_e4m3(5, 1, (2, 3, 64, 16))
    assert codes.shape == (2, 3, 64, 16) and scales.shape == (2, 3)
    f = datagen.normal_f32(5, 1, (2, 3, 64, 16))
    amax = np.abs(f).reshape(6, -1).max(axis=1)
    np.testing.assert_array_equal(scales.ravel(), (amax / np.float32(448.0)).astype(np.float32))
    # the largest magnitude of each group lands on the top code
    top = (codes.reshape(6, -1) & 0x7F).max(axis=1)
    assert np.all(top == 0x7E)


def test_uniform_int_range():
    x = datagen.uniform_int(3, 3, 10000, 4096, 65536)
    assert x.min() >= 4096 and x.max() <= 65536
    assert abs(x.mean() - (4096 + 65536) / 2) < 1500


def test_bf16_encoder_rounds_midpoints_to_even():
    # every midpoint between adjacent bf16 values of one binade per exponent
    # (mantissas 0..126 and their successors) is a tie: the even neighbour wins
    lo = np.arange(0x0080, 0x7F00, 1, dtype=np.uint32)  # positive normal bf16 patterns below the top binade
    lo = lo[(lo & 0x7F) != 0x7F]
    mid = ((lo << 16) | 0x8000).view(np.float32)        # exactly halfway to the next pattern
    enc = datagen.f32_to_bf16_bits(mid).astype(np.uint32)
    want = np.where(lo & 1, lo + 1, lo)
    assert np.array_equal(enc, want)
    # just above and just below a midpoint go to the nearer neighbour
    assert np.array_equal(datagen.f32_to_bf16_bits(((lo << 16) | 0x8001).view(np.float32)).astype(np.uint32), lo + 1)
    assert np.array_equal(datagen.f32_to_bf16_bits(((lo << 16) | 0x7FFF).view(np.float32)).astype(np.uint32), lo)


def test_e2m1_encoder_rounds_ties_to_even_and_saturates():
    # midpoints between neighbouring E2M1 magnitudes go to the code whose
    # mantissa bit is 0; magnitudes past 6 saturate; the sign is bit 3
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    assert datagen.f32_to_e2m1(mids).tolist() == [0, 2, 2, 4, 4, 6, 6]
    assert datagen.f32_to_e2m1(-mids).tolist() == [8, 10, 10, 12, 12, 14, 14]
    assert datagen.f32_to_e2m1(np.array([6.0, 6.5, 1e30, -7.0], np.float32)).tolist() == [7, 7, 7, 15]
    # just off a midpoint goes to the nearer neighbour
    assert datagen.f32_to_e2m1(np.array([0.2501, 0.7499, 4.99, 5.01], np.float32)).tolist() == [1, 1, 6, 7]


def test_mxfp4_fill_is_reproducible_and_thread_independent():
    a = datagen.normal_mxfp4(5, 4, (7, 3, 128), 0.5)
    b = datagen.normal_mxfp4(5, 4, (7, 3, 128), 0.5)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    lib = datagen._load()
    c1 = np.empty((21, 64), np.uint8); s1 = np.empty((21, 4), np.uint8)
    c7 = np.empty((21, 64), np.uint8); s7 = np.empty((21, 4), np.uint8)
    lib.dg_fill_mxfp4(5, 4, 21, 128, 0.5, datagen._ptr(c1), datagen._ptr(s1), 1)
    lib.dg_fill_mxfp4(5, 4, 21, 128, 0.5, datagen._ptr(c7), datagen._ptr(s7), 7)
    assert np.array_equal(c1, c7) and np.array_equal(s1, s7)
    assert np.array_equal(c1.reshape(a[0].shape), a[0]) and np.array_equal(s1.reshape(a[1].shape), a[1])
