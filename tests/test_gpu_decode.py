"""GPU parity of attn_decode (split-KV decode + level-2 combine) against the
double-precision oracle, element by element, on seeded inputs: the five
workloads' decode shapes at full size, small shapes spanning several tiles with
ragged tails, edge lengths, every fp8 code, strided views, all split counts of a
sweep, and bit-identical repeats for a fixed split plan."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from _gpu import (assert_close, assert_lse_close, decode_on_gpu, errors, from_dev, needs_gpu, oracle_decode,
                  to_dev)
from datagen.workloads import make_inputs

pytestmark = [pytest.mark.gpu, needs_gpu]


def _check(inp, S, kind, causal=False, lse_tol=None, scale=None, what=""):
    out, lse = decode_on_gpu(inp, num_splits=S, causal=causal, softmax_scale=scale or 0.0)
    ref, ref_lse = oracle_decode(inp, causal=causal, scale=scale)
    got = from_dev(out)[:, :, 0, :]
    res = assert_close(got, ref, kind, what="%s S=%s" % (what, S))
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, lse_tol or (1e-5 if kind == "f32" else 2e-3))
    print("%s S=%s max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % (what, S, *res), flush=True)
    return out, lse


# ------------------------------------------------------------ workload 1 (fp32)

def test_workload1_single_head_fp32_four_splits():
    _check(make_inputs(1), 4, "f32", what="wl1")


@pytest.mark.parametrize("S", [1, 2, 3, 5, 8, 16])
def test_fp32_split_count_sweep(S):
    _check(make_inputs(1), S, "f32", what="wl1-sweep")


# ------------------------------------------------------------ MFMA path, small shapes

@pytest.mark.parametrize("L,S", [(1000, 1), (1000, 3), (1000, 7), (77, 2), (17, 1), (5, 1), (4096, 16), (4096, 64)])
def test_gqa_bf16_small(L, S):
    inp = make_inputs(2, B=2, Hq=8, Hkv=2, L=L, seed=20 + L)
    _check(inp, S, "bf16", what="gqa-bf16 L=%d" % L)


def test_gqa_bf16_peaked_queries():
    # Q scaled x8: a much sharper softmax, running max moves often
    inp = make_inputs(2, B=1, Hq=8, Hkv=2, L=3000, q_mul=4.0, seed=31)
    _check(inp, 5, "bf16", what="gqa-bf16 q*8")


def test_gqa_bf16_needles():
    # Keys planted along head 0's query make single keys dominate (needle case)
    inp = make_inputs(2, B=1, Hq=8, Hkv=2, L=5000, seed=32)
    q = datagen_bf16_to_f32(inp["q"])
    k = inp["k"].copy()
    rng = np.random.default_rng(5)
    for g in range(2):
        qd = q[0, 4 * g, 0]
        needle = (6.0 * qd / np.linalg.norm(qd) * np.sqrt(128)).astype(np.float32)
        for pos in rng.choice(5000, size=3, replace=False):
            k[0, g, pos] = datagen.f32_to_bf16_bits(needle)
    inp["k"] = k
    ref, _ = oracle_decode(inp)
    assert np.abs(ref).max() > 0.3  # the needles really dominate
    _check(inp, 7, "bf16", what="gqa-bf16 needles")


def datagen_bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_softmax_scale_override():
    inp = make_inputs(2, B=1, Hq=4, Hkv=1, L=700, seed=33)
    _check(inp, 3, "bf16", scale=0.02, what="scale=0.02")


# ------------------------------------------------------------ ragged batches

def test_ragged_edge_lengths():
    lens = np.array([0, 1, 15, 16, 17, 63, 64, 65, 300, 129], np.int32)
    inp = make_inputs(3, B=10, Hq=8, Hkv=2, L=300, seed=34)
    inp["kv_lens"] = lens
    out, lse = _check(inp, 5, "bf16", causal=True, what="ragged edges")
    got = from_dev(out)
    assert np.all(got[0] == 0.0) and np.all(np.isneginf(lse.cpu().numpy()[0]))


@pytest.mark.parametrize("S", [1, 5])
def test_fp8_ragged_edge_lengths(S):
    # fp8 spans are read in 32-key tiles: lengths at and around the tile and
    # the 64-key split quantum, a split holding a single key, an empty row
    lens = np.array([0, 1, 31, 32, 33, 63, 64, 65, 96, 97, 300, 129], np.int32)
    inp = make_inputs(5, B=12, Hq=8, Hkv=2, L=300, seed=36 + S)
    inp["kv_lens"] = lens
    out, lse = _check(inp, S, "e4m3", causal=True, what="fp8 ragged edges")
    got = from_dev(out)
    assert np.all(got[0] == 0.0) and np.all(np.isneginf(lse.cpu().numpy()[0]))


def test_ragged_lengths_beyond_capacity_are_clamped():
    inp = make_inputs(3, B=3, Hq=4, Hkv=1, L=256, seed=35)
    inp["kv_lens"] = np.array([-5, 1000, 100], np.int32)
    ref_inp = dict(inp, kv_lens=np.array([0, 256, 100], np.int32))
    out, lse = decode_on_gpu(inp, num_splits=2, causal=True)
    ref, ref_lse = oracle_decode(ref_inp, causal=True)
    assert_close(from_dev(out)[:, :, 0], ref, "bf16")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, 2e-3)


def test_workload3_ragged_batch_full_size():
    inp = make_inputs(3)
    print("lengths", inp["kv_lens"].tolist(), flush=True)
    _check(inp, 0, "bf16", causal=True, what="wl3")


# ------------------------------------------------------------ workload 2, full size

@pytest.mark.parametrize("S", [64, 128, 256])
def test_workload2_full_size(S):
    _check(make_inputs(2), S, "bf16", what="wl2")


def test_workload2_auto_splits_and_determinism():
    inp = make_inputs(2)
    dev = {k: to_dev(v) for k, v in inp.items()}
    outs = [decode_on_gpu(inp, num_splits=128, dev=dev) for _ in range(3)]
    b0 = outs[0][0].view(torch.int16).cpu().numpy()
    l0 = outs[0][1].cpu().numpy()
    for o, l in outs[1:]:
        assert np.array_equal(o.view(torch.int16).cpu().numpy(), b0)
        assert np.array_equal(l.cpu().numpy().view(np.uint32), l0.view(np.uint32))
    out, _ = decode_on_gpu(inp, num_splits=0, dev=dev)
    ref, _ = oracle_decode(inp)
    assert_close(from_dev(out)[:, :, 0], ref, "bf16", what="wl2 auto")


# ------------------------------------------------------------ many splits

@pytest.mark.parametrize("wl,B,L,S", [(2, 2, 65436, 256), (2, 1, 100000, 521), (5, 1, 100000, 521)])
def test_many_splits_several_rounds_of_workgroups(wl, B, L, S):
    # Several rounds of workgroups, merged by the second kernel. Covers a short
    # last split ending mid-tile, an odd split count and 192-key chunks.
    inp = make_inputs(wl, B=B, Hq=32, Hkv=8, L=L, seed=60 + S)
    dev = {k: to_dev(v) for k, v in inp.items()}
    out, lse = decode_on_gpu(inp, num_splits=S, dev=dev)
    ref, ref_lse = oracle_decode(inp)
    res = assert_close(from_dev(out)[:, :, 0, :], ref, "bf16" if wl == 2 else "e4m3", what="multi L=%d S=%d" % (L, S))
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, 2e-3)
    print("multi wl%d L=%d S=%d max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % (wl, L, S, *res), flush=True)
    out2, lse2 = decode_on_gpu(inp, num_splits=S, dev=dev)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))


# ------------------------------------------------------------ fp8 KV

@pytest.mark.parametrize("S", [1, 3, 16])
def test_fp8_small(S):
    inp = make_inputs(5, B=2, Hq=8, Hkv=2, L=2000, seed=40)
    _check(inp, S, "e4m3", what="fp8")


def test_fp8_every_code():
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    B, Hkv, L, d = 1, 2, 256, 128
    idx = np.arange(B * Hkv * L * d).reshape(B, Hkv, L, d)
    inp = make_inputs(5, B=B, Hq=8, Hkv=Hkv, L=L, seed=41)
    inp["k"] = finite[idx % finite.size]
    inp["v"] = finite[(idx * 7 + 3) % finite.size]
    # scales keep |V| <= 2 (outputs of order 1, where the absolute bounds apply);
    # every code still passes through the decoders
    inp["k_scale"] = np.array([0.003, 0.0011], np.float32)
    inp["v_scale"] = np.array([0.004, 0.0025], np.float32)
    _check(inp, 2, "e4m3", lse_tol=5e-3, what="fp8 all codes")


def test_workload5_fp8_1m_full_size():
    inp = make_inputs(5)
    dev = {k: to_dev(v) for k, v in inp.items()}
    out1, lse1 = decode_on_gpu(inp, num_splits=1024, dev=dev)
    out2, lse2 = decode_on_gpu(inp, num_splits=1024, dev=dev)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32))
    ref, ref_lse = oracle_decode(inp)
    res = assert_close(from_dev(out1)[:, :, 0], ref, "e4m3", what="wl5")
    assert_lse_close(lse1.cpu().numpy().astype(np.float64), ref_lse, 2e-3)
    print("wl5 max_abs=%.3g mean_abs=%.3g rel_l2=%.3g" % res, flush=True)
    del dev


# ------------------------------------------------------------ MFMA path, other head ratios

@pytest.mark.parametrize("G,fmt,S", [(1, "bf16", 3), (2, "bf16", 5), (8, "bf16", 7), (8, "e4m3", 4), (1, "e4m3", 2),
                                     (2, "e4m3", 1)])
def test_mfma_head_ratios(G, fmt, S):
    wl = 2 if fmt == "bf16" else 5
    inp = make_inputs(wl, B=2, Hq=2 * G, Hkv=2, L=1500, seed=70 + G + S)
    _check(inp, S, fmt, what="mfma G=%d %s" % (G, fmt))


@pytest.mark.parametrize("G", [1, 8])
def test_mfma_head_ratios_ragged_edges(G):
    lens = np.array([0, 1, 31, 33, 64, 65, 300, 129], np.int32)
    inp = make_inputs(3, B=8, Hq=2 * G, Hkv=2, L=300, seed=80 + G)
    inp["kv_lens"] = lens
    out, lse = _check(inp, 5, "bf16", causal=True, what="mfma G=%d ragged" % G)
    assert np.all(from_dev(out)[0] == 0.0) and np.all(np.isneginf(lse.cpu().numpy()[0]))


@pytest.mark.parametrize("fmt", ["bf16", "e4m3"])
def test_d64_ragged_edges(fmt):
    lens = np.array([0, 1, 31, 32, 33, 65, 300, 129], np.int32)
    inp = make_inputs(3 if fmt == "bf16" else 5, B=8, Hq=8, Hkv=2, d=64, L=300, seed=84)
    inp["kv_lens"] = lens
    out, lse = _check(inp, 5, fmt, causal=True, what="d=64 %s ragged" % fmt)
    assert np.all(from_dev(out)[0] == 0.0) and np.all(np.isneginf(lse.cpu().numpy()[0]))


def test_d64_long_cache():
    inp = make_inputs(2, B=1, Hq=32, Hkv=8, d=64, L=65536, seed=85)
    _check(inp, 64, "bf16", what="d=64 64K")


def test_g8_full_size_128k():
    # 64 query heads over 8 KV heads (eight per group), 128K bf16 keys
    inp = make_inputs(2, Hq=64, Hkv=8, seed=82)
    _check(inp, 64, "bf16", what="G=8 128K")


# ------------------------------------------------------------ head dim 64 (MFMA) and fp32 (vector ALU)

@pytest.mark.parametrize("G,d,fmt", [(1, 64, "bf16"), (2, 64, "bf16"), (8, 64, "bf16"), (4, 64, "bf16"),
                                     (1, 128, "f32"), (8, 64, "f32"), (2, 64, "e4m3"), (4, 64, "e4m3"),
                                     (8, 64, "e4m3")])
def test_d64_and_fp32_paths(G, d, fmt):
    wl = {"bf16": 2, "f32": 1, "e4m3": 5}[fmt]
    inp = make_inputs(wl, B=2, Hq=2 * G, Hkv=2, d=d, L=1111, seed=50 + G + d)
    kind = "f32" if fmt == "f32" else "bf16"
    _check(inp, 4, kind, what="valu G=%d d=%d %s" % (G, d, fmt))


# ------------------------------------------------------------ strided views

def test_strided_bshd_cache_and_padded_q():
    B, Hq, Hkv, L, d = 2, 8, 2, 900, 128
    inp = make_inputs(2, B=B, Hq=Hq, Hkv=Hkv, L=L, seed=60)
    # K/V stored as [B, L, Hkv, d] (sequence-major) and viewed as [B, Hkv, L, d]
    k_bshd = to_dev(np.ascontiguousarray(inp["k"].transpose(0, 2, 1, 3)))
    v_bshd = to_dev(np.ascontiguousarray(inp["v"].transpose(0, 2, 1, 3)))
    # Q inside a larger buffer: [B, Hq, 1, 2d], first half used
    qbig = np.zeros((B, Hq, 1, 2 * d), np.uint16)
    qbig[..., :d] = inp["q"]
    qdev = to_dev(qbig)[..., :d]
    dev = dict(q=qdev, k=k_bshd.permute(0, 2, 1, 3), v=v_bshd.permute(0, 2, 1, 3))
    out, lse = decode_on_gpu(inp, num_splits=3, dev=dev)
    ref, ref_lse = oracle_decode(inp)
    assert_close(from_dev(out)[:, :, 0], ref, "bf16", what="strided")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, 2e-3)


# ------------------------------------------------------------ split sweep agreement

def test_split_counts_agree_with_each_other():
    inp = make_inputs(2, B=1, Hq=8, Hkv=2, L=8192, seed=70)
    dev = {k: to_dev(v) for k, v in inp.items()}
    ref, _ = oracle_decode(inp)
    worst = 0.0
    for S in (1, 2, 3, 4, 7, 16, 33, 64, 128):
        out, _ = decode_on_gpu(inp, num_splits=S, dev=dev)
        mx, _, _ = assert_close(from_dev(out)[:, :, 0], ref, "bf16", what="S=%d" % S)
        worst = max(worst, mx)
    print("worst max_abs over splits %.3g" % worst, flush=True)


# ------------------------------------------------------------ workspace reuse and the two-level API

def test_workspace_reused_across_shapes_and_split_counts():
    import long_context_decode_kv_amd as lib
    ws = lib.attn_decode_workspace(16, 32, 128, 512)
    cases = [(make_inputs(2, B=1, Hq=32, Hkv=8, L=20000, seed=101), 64, False),
             (make_inputs(3, B=6, Hq=8, Hkv=2, L=3000, seed=102), 7, True),
             (make_inputs(2, B=2, Hq=16, Hkv=4, L=999, seed=103), 3, False),
             (make_inputs(5, B=1, Hq=8, Hkv=2, L=5000, seed=104), 16, False),
             (make_inputs(2, B=1, Hq=32, Hkv=8, L=20000, seed=101), 64, False)]
    for inp, S, causal in cases:
        d = {k: to_dev(v) for k, v in inp.items()}
        out, lse = lib.attn_decode(d["q"], d["k"], d["v"], k_scale=d.get("k_scale"), v_scale=d.get("v_scale"),
                                   kv_lens=d.get("kv_lens"), causal=causal, num_splits=S, workspace=ws)
        torch.cuda.synchronize()
        ref, ref_lse = oracle_decode(inp, causal=causal)
        assert_close(from_dev(out)[:, :, 0], ref, "bf16", what="reuse S=%d" % S)
        assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, 2e-3)
        # the merge counters are left at zero for the next call
        assert int(ws[:4 << 20].view(torch.int32).abs().sum()) == 0


def test_workspace_init_clears_a_dirty_workspace():
    # attn_decode_workspace_init must zero the counter block whatever it held
    import long_context_decode_kv_amd as lib
    inp = make_inputs(2, B=1, Hq=32, Hkv=8, L=8192, seed=105)
    S = 32
    ws = torch.full((lib.attn_decode_workspace_size(1, 32, 128, S),), 0x5A, dtype=torch.uint8, device="cuda")
    lib.attn_decode_workspace_init(ws)
    torch.cuda.synchronize()
    assert int(ws[:4 << 20].view(torch.int32).abs().sum()) == 0
    assert int(ws[4 << 20].item()) == 0x5A  # only the counter block is touched
    d = {k: to_dev(v) for k, v in inp.items()}
    out, lse = lib.attn_decode(d["q"], d["k"], d["v"], num_splits=S, workspace=ws)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_decode(inp)
    assert_close(from_dev(out)[:, :, 0], ref, "bf16", what="after init")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, 2e-3)


@pytest.mark.parametrize("wl,S", [(2, 64), (5, 128), (3, 0)])
def test_two_level_api_matches_fused_decode(wl, S):
    import long_context_decode_kv_amd as lib
    kw = dict(B=2, Hq=8, Hkv=2, L=6000) if wl != 3 else dict(B=4, Hq=8, Hkv=2, L=6000)
    inp = make_inputs(wl, seed=110 + wl, **kw)
    d = {k: to_dev(v) for k, v in inp.items()}
    out, lse = lib.attn_decode(d["q"], d["k"], d["v"], k_scale=d.get("k_scale"), v_scale=d.get("v_scale"),
                               kv_lens=d.get("kv_lens"), num_splits=S)
    o_p, m_p, l_p = lib.attn_decode_partials(d["q"], d["k"], d["v"], k_scale=d.get("k_scale"),
                                             v_scale=d.get("v_scale"), kv_lens=d.get("kv_lens"), num_splits=S)
    o2, lse2 = lib.attn_combine_partials(o_p, m_p, l_p, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_decode(inp)
    B, Hq = inp["q"].shape[:2]
    assert_close(from_dev(o2).reshape(B, Hq, -1), ref, "bf16", what="two-level")
    assert_lse_close(lse2.cpu().numpy().astype(np.float64).reshape(B, Hq), ref_lse, 2e-3)
    # both paths agree to within one bf16 rounding of the output: bf16 keeps 8
    # significant bits, so one unit in the last place at x is at most 2^-7 |x|
    a, b = from_dev(out).reshape(B * Hq, -1), from_dev(o2)
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-6)


# (R, S, d): one column block of 64 lanes; a deep merge over few rows (32- and
# 16-lane slots, three column blocks); odd d (4-byte loads); one partial
@pytest.mark.parametrize("R,S,d", [(5, 37, 96), (4, 300, 96), (3, 200, 7), (4, 1, 128)])
def test_combine_partials_api_against_oracle(R, S, d):
    import long_context_decode_kv_amd as lib
    rng = np.random.default_rng(9 + S)
    o = rng.standard_normal((R, S, d)).astype(np.float32)
    m = (rng.standard_normal((R, S)) * 3).astype(np.float32)
    l = rng.uniform(0.5, 20, (R, S)).astype(np.float32)
    m[1, :] = -np.inf
    l[1, :] = 0.0
    if S > 5:
        m[2, 5:] = -np.inf
        l[2, 5:] = 0.0
    if R > 3:
        m[3] = np.arange(S, dtype=np.float32) * 0.25  # the max moves with every batch
    for dt, kind in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        out, lse = lib.attn_combine_partials(to_dev(o), to_dev(m), to_dev(l), out_dtype=dt)
        torch.cuda.synchronize()
        ref, ref_lse = oracle.combine(o, m, l)
        got = from_dev(out)
        if kind == "f32":
            assert np.abs(got - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())
        else:
            assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
        assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, 1e-5)
        assert np.all(got[1] == 0) and np.isneginf(lse.cpu().numpy()[1])


def test_decode_captured_in_a_graph_matches_eager_on_every_replay():
    # A decode step replayed from a HIP graph (as a serving loop would run it):
    # no memset is recorded (the merge counters are left zero by each call),
    # and every replay, with eager work in between, must equal the eager call.
    import long_context_decode_kv_amd as lib
    inp = make_inputs(2, B=1, Hq=32, Hkv=8, L=20000, seed=106)
    d = {k: to_dev(v) for k, v in inp.items()}
    S = 32
    ws = lib.attn_decode_workspace(1, 32, 128, S)
    out = torch.empty_like(d["q"])
    lse = torch.empty((1, 32), dtype=torch.float32, device="cuda")
    ref_out, ref_lse = lib.attn_decode(d["q"], d["k"], d["v"], num_splits=S, workspace=ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lib.attn_decode(d["q"], d["k"], d["v"], num_splits=S, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lib.attn_decode(d["q"], d["k"], d["v"], num_splits=S, out=out, lse=lse, workspace=ws)
    for i in range(5):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "replay %d" % i
        assert torch.equal(lse, ref_lse), "replay %d" % i
        # eager work between replays, on the same workspace
        o2, _ = lib.attn_decode(d["q"], d["k"], d["v"], num_splits=S, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o2.view(torch.int16), ref_out.view(torch.int16))
    assert int(ws[:4 << 20].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("S", [1, 5, 0])
def test_gqa_bf16_rising_score_ramp(S):
    # keys of 64-key block t scaled by 2^(t // 8) (up to 32x at 3000 keys): the
    # running max of each wave moves past its lazy headroom again and again,
    # and the splits' partials differ in scale by orders of magnitude
    inp = make_inputs(2, B=2, Hq=8, Hkv=2, L=3000, seed=34)
    t = np.arange(3000) // 64
    f = (inp["k"].astype(np.uint32) << 16).view(np.float32) * (2.0 ** (t // 8)).astype(np.float32)[None, None, :, None]
    inp["k"] = (f.view(np.uint32) >> 16).astype(np.uint16)
    _check(inp, S, "bf16", what="gqa-bf16 ramp S=%d" % S)
