"""The byte and flop models bench.py divides by, checked against counts made
another way (the per-head KV size the ThriftAttention page prints for a
128K-token FP16 cache, brute-force enumeration of pi-Attention's visible
pairs)."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402


def test_kv_bytes_per_head_at_128k():
    # 131072 keys x 128 dims x 2 (K and V) x 2 bytes = 67,108,864 bytes (about 67 MB per head)
    assert bench.kv_bytes(131072, 1, 128, 2) == 67108864
    assert bench.decode_algorithmic_bytes(1, 32, 8, 128, 131072) == 8 * 67108864 + 2 * 32 * 128 * 2


def test_prefill_flops_count_the_causal_pairs():
    L = 37
    pairs = sum(i + 1 for i in range(L))
    assert bench.prefill_flops(3, 16, L) == 4 * 3 * 16 * pairs
    assert bench.prefill_flops(32, 128, 16384) == 2199157473280


def test_mixed_bytes():
    assert bench.mixed_algorithmic_bytes(1, 32, 8, 128, 26214, 104858) == \
        2 * 8 * 26214 * 128 * 2 + 2 * 8 * 104858 * 128 + 2 * 4 * 8 + 2 * 32 * 128 * 2


def test_mixed_fp4_bytes():
    # per key and KV head: bf16 K + V rows (2 x 256 B); fp4 K + V codes (2 x 64 B) and e8m0 scales (2 x 4 B)
    per_bf16, per_fp4 = 2 * 128 * 2, 2 * (128 // 2 + 128 // 32)
    assert bench.mixed_fp4_algorithmic_bytes(1, 32, 8, 128, 26214, 104858) == \
        8 * (26214 * per_bf16 + 104858 * per_fp4) + 2 * 32 * 128 * 2 == 221474432


def test_pi_counts_by_enumeration():
    for L, w, per in ((300, 37, 11), (129, 0, 1), (200, 250, 7), (64, 5, 0), (1000, 64, 64)):
        pairs = 0
        for i in range(L):
            for j in range(i + 1):
                d = i - j
                if d <= w or (per > 0 and d % per == 0):
                    pairs += 1
        assert bench.pi_prefill_pairs(L, w, per) == pairs
        i = L - 1
        keys = sum(1 for j in range(L) if (i - j) <= w or (per > 0 and (i - j) % per == 0))
        assert bench.pi_decode_keys(L, w, per) == keys


def test_two_sided_pi_counts_by_enumeration():
    for L, w, per in ((300, 37, 11), (129, 0, 1), (200, 250, 7), (64, 5, 0), (500, 64, 64)):
        pairs = sum(1 for i in range(L) for j in range(L)
                    if abs(i - j) <= w or (per > 0 and (i - j) % per == 0))
        assert bench.pi_prefill_pairs(L, w, per, causal=False) == pairs


def test_ragged_fp8_and_three_precision_bytes():
    # per key and KV head: bf16 2 x 256 B, fp8 2 x 128 B, fp4 2 x (64 + 4) B
    assert bench.ragged_bytes([4096, 100], 32, 8, 128) == 8 * 4196 * 512 + 2 * 2 * 32 * 128 * 2
    assert bench.fp8_decode_bytes(1, 32, 8, 128, 1 << 20) == (1 << 31) + 64 + 2 * 32 * 128 * 2
    assert bench.mixed3_algorithmic_bytes(1, 32, 8, 128, 26214, 26214, 78644) == \
        8 * (26214 * 512 + 26214 * 256 + 78644 * 136) + 64 + 2 * 32 * 128 * 2
