"""Every entry point replayed from a HIP graph, as a serving loop would run it.

Each call is captured once with fixed inputs, outputs and workspace, then
replayed several times with the outputs poisoned before each replay and an
eager call of the same entry point (on the same workspace) between replays;
every replay must reproduce the eager result bit for bit. No entry point
records a memset: the merge counters a call uses are left zero by that call,
and nothing else needs clearing. The eager results themselves are checked
against the oracle by the other GPU tests.
"""
import numpy as np
import pytest
import torch

from _gpu import needs_gpu, to_dev
from datagen.workloads import make_inputs, make_mixed3_inputs, make_mixed_inputs

pytestmark = [pytest.mark.gpu, needs_gpu]


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _replays_match_eager(call, outs, replays=4):
    """call() writes into the tensors of `outs`; the graph of one call must
    reproduce the eager outputs on every replay."""
    cur = torch.cuda.current_stream()
    call()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        call()
    cur.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for i in range(replays):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for j, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(_bits(o), _bits(r)), "replay %d, output %d" % (i, j)
        call()  # eager work between replays, same workspace
        torch.cuda.synchronize()
        for j, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(_bits(o), _bits(r)), "eager call after replay %d, output %d" % (i, j)
    del graph


def _decode_outs(q):
    B, Hq = q.shape[:2]
    return torch.empty_like(q), torch.empty((B, Hq), dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("wl,S", [(2, 64), (2, 0), (2, 16), (5, 0), (1, 4)])
def test_graph_decode(wl, S):
    # bf16 with the merge kernel (64 splits x 8 KV heads x 2 sequences), the
    # automatic plan, the fused merge (16 x 8 x 2: one workgroup per CU), fp8,
    # fp32
    import long_context_decode_kv_amd as lib
    print("graph decode workload", wl, "splits", S, flush=True)
    if wl == 1:
        inp = make_inputs(1, B=1, Hq=1, Hkv=1, d=64, L=1024, seed=300)
    else:
        inp = make_inputs(wl, B=2, Hq=32, Hkv=8, L=20000, seed=301 + S)
        inp["kv_lens"] = np.array([20000, 13457], dtype=np.int32)
    d = {k: to_dev(v) for k, v in inp.items()}
    B, Hq, _, hd = d["q"].shape
    Hkv, L = d["k"].shape[1], d["k"].shape[2]
    S_ws = S if S > 0 else lib.attn_decode_auto_splits(B, Hkv, L, lib._dtype_code(d["k"]), d.get("kv_lens") is not None)
    ws = lib.attn_decode_workspace(B, Hq, hd, S_ws)
    out, lse = _decode_outs(d["q"])

    def call():
        lib.attn_decode(d["q"], d["k"], d["v"], k_scale=d.get("k_scale"), v_scale=d.get("v_scale"),
                        kv_lens=d.get("kv_lens"), num_splits=S, out=out, lse=lse, workspace=ws)

    _replays_match_eager(call, [out, lse])


@pytest.mark.parametrize("S", [(0, 0), (8, 24)])
def test_graph_decode_mixed_fp8(S):
    import long_context_decode_kv_amd as lib
    print("graph mixed fp8 splits", S, flush=True)
    inp = make_mixed_inputs(6, B=1, Hq=32, Hkv=8, L=20000, seed=310)
    d = {k: to_dev(v) for k, v in inp.items()}
    L_hi, L_lo = d["k_hi"].shape[2], d["k_lo"].shape[2]
    S_hi, S_lo = S if S[0] else lib.attn_decode_mixed_splits(1, 8, L_hi, L_lo)
    used = lib.attn_decode_plan(L_hi, S_hi)[0] + lib.attn_decode_plan(L_lo, S_lo)[0]
    ws = lib.attn_decode_workspace(1, 32, 128, used)
    out, lse = _decode_outs(d["q"])

    def call():
        lib.attn_decode_mixed(d["q"], d["k_hi"], d["v_hi"], d["k_lo"], d["v_lo"], k_scale=d["k_scale"],
                              v_scale=d["v_scale"], hi_lens=d["hi_lens"], lo_lens=d["lo_lens"],
                              num_splits_hi=S_hi, num_splits_lo=S_lo, out=out, lse=lse, workspace=ws)

    _replays_match_eager(call, [out, lse])


def test_graph_decode_mixed_fp4():
    import long_context_decode_kv_amd as lib
    print("graph mixed fp4", flush=True)
    inp = make_mixed_inputs(9, B=1, Hq=32, Hkv=8, L=20000, seed=311)
    d = {k: to_dev(v) for k, v in inp.items() if k != "lo_format"}
    L_hi, L_lo = d["k_hi"].shape[2], d["k_lo"].shape[2]
    S_hi, S_lo = lib.attn_decode_mixed_fp4_splits(1, 8, L_hi, L_lo)
    used = lib.attn_decode_plan(L_hi, S_hi)[0] + lib.attn_decode_plan(L_lo, S_lo)[0]
    ws = lib.attn_decode_workspace(1, 32, 128, used)
    out, lse = _decode_outs(d["q"])

    def call():
        lib.attn_decode_mixed_fp4(d["q"], d["k_hi"], d["v_hi"], d["k_lo"], d["v_lo"], k_lo_scale=d["k_scale"],
                                  v_lo_scale=d["v_scale"], hi_lens=d["hi_lens"], lo_lens=d["lo_lens"],
                                  num_splits_hi=S_hi, num_splits_lo=S_lo, out=out, lse=lse, workspace=ws)

    _replays_match_eager(call, [out, lse])


def test_graph_decode_mixed3():
    import long_context_decode_kv_amd as lib
    print("graph mixed3", flush=True)
    inp = make_mixed3_inputs(B=1, Hq=32, Hkv=8, L=20000, seed=312)
    d = {k: to_dev(v) for k, v in inp.items()}
    caps = [d[k].shape[2] for k in ("k_hi", "k_mid", "k_lo")]
    S = lib.attn_decode_mixed3_splits(1, 8, *caps)
    used = sum(lib.attn_decode_plan(c, s)[0] for c, s in zip(caps, S))
    ws = lib.attn_decode_workspace(1, 32, 128, used)
    out, lse = _decode_outs(d["q"])

    def call():
        lib.attn_decode_mixed3(d["q"], d["k_hi"], d["v_hi"], d["k_mid"], d["v_mid"], d["k_lo"], d["v_lo"],
                               k_mid_scale=d["k_mid_scale"], v_mid_scale=d["v_mid_scale"],
                               k_lo_scale=d["k_lo_scale"], v_lo_scale=d["v_lo_scale"], hi_lens=d["hi_lens"],
                               mid_lens=d["mid_lens"], lo_lens=d["lo_lens"], num_splits_hi=S[0],
                               num_splits_mid=S[1], num_splits_lo=S[2], out=out, lse=lse, workspace=ws)

    _replays_match_eager(call, [out, lse])


def test_graph_decode_pi():
    import long_context_decode_kv_amd as lib
    print("graph pi decode", flush=True)
    inp = make_inputs(2, B=2, Hq=32, Hkv=8, L=20000, seed=313)
    d = {k: to_dev(v) for k, v in inp.items()}
    d["kv_lens"] = torch.tensor([20000, 9001], dtype=torch.int32, device="cuda")
    alpha = torch.rand(2 * 32, generator=torch.Generator().manual_seed(5)).cuda()
    window, period = 1000, 64
    sw, ss = lib.attn_decode_pi_splits(2, 8, 20000, window, period)
    cap_s = (20000 - 2 - window) // period + 1
    used = lib.attn_decode_plan(window + 1, sw)[0] + lib.attn_decode_plan(cap_s, ss)[0]
    ws = lib.attn_decode_workspace(2, 32, 128, used)
    out, lse = _decode_outs(d["q"])

    def call():
        lib.attn_decode_pi(d["q"], d["k"], d["v"], window, period, alpha=alpha, kv_lens=d["kv_lens"],
                           num_splits_window=sw, num_splits_skip=ss, out=out, lse=lse, workspace=ws)

    _replays_match_eager(call, [out, lse])


def test_graph_combine_partials():
    import long_context_decode_kv_amd as lib
    print("graph combine", flush=True)
    g = torch.Generator().manual_seed(6)
    R, S, d = 32, 8, 128
    o = torch.randn(R, S, d, generator=g).cuda()
    m = torch.randn(R, S, generator=g).cuda()
    m[3, 2] = float("-inf")
    l = (torch.rand(R, S, generator=g) + 0.5).cuda()
    l[3, 2] = 0.0
    out = torch.empty(R, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(R, dtype=torch.float32, device="cuda")

    def call():
        lib.attn_combine_partials(o, m, l, out=out, lse=lse)

    _replays_match_eager(call, [out, lse])


@pytest.mark.parametrize("causal", [True, False])
def test_graph_prefill(causal):
    import long_context_decode_kv_amd as lib
    print("graph prefill causal", causal, flush=True)
    inp = make_inputs(4, B=1, Hq=8, Hkv=2, L=1000, Lq=1000 if causal else 700, seed=314)
    d = {k: to_dev(v) for k, v in inp.items()}
    out = torch.empty_like(d["q"])
    lse = torch.empty(d["q"].shape[:3], dtype=torch.float32, device="cuda")

    def call():
        lib.attn_prefill(d["q"], d["k"], d["v"], causal=causal, out=out, lse=lse)

    _replays_match_eager(call, [out, lse])


@pytest.mark.parametrize("causal", [True, False])
def test_graph_prefill_pi(causal):
    import long_context_decode_kv_amd as lib
    print("graph pi prefill causal", causal, flush=True)
    inp = make_inputs(4, B=1, Hq=8, Hkv=2, L=1000, seed=315)
    d = {k: to_dev(v) for k, v in inp.items()}
    alpha = torch.rand(1, 8, 1000, generator=torch.Generator().manual_seed(7)).cuda()
    out = torch.empty_like(d["q"])
    lse = torch.empty(d["q"].shape[:3], dtype=torch.float32, device="cuda")
    ws = torch.empty(lib.attn_prefill_pi_workspace_size(1, 8, 1000, 128), dtype=torch.uint8, device="cuda")

    def call():
        lib.attn_prefill_pi(d["q"], d["k"], d["v"], 100, 16, alpha=alpha, causal=causal, out=out, lse=lse,
                            workspace=ws)

    _replays_match_eager(call, [out, lse])


def test_graph_prefill_backward():
    import long_context_decode_kv_amd as lib
    print("graph backward", flush=True)
    inp = make_inputs(4, B=1, Hq=8, Hkv=2, L=700, seed=316)
    d = {k: to_dev(v) for k, v in inp.items()}
    o, lse = lib.attn_prefill(d["q"], d["k"], d["v"], causal=True)
    dout = torch.randn(d["q"].shape, generator=torch.Generator().manual_seed(8)).to(torch.bfloat16).cuda()
    dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
    ws = torch.empty(lib.attn_prefill_backward_workspace_size(1, 8, 700), dtype=torch.uint8, device="cuda")

    def call():
        lib.attn_prefill_backward(d["q"], d["k"], d["v"], o, lse, dout, causal=True, dq=dq, dk=dk, dv=dv,
                                  workspace=ws)

    _replays_match_eager(call, [dq, dk, dv])
