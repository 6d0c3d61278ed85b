"""attn_decode_noalloc (the decode for callers that cannot allocate) against
attn_decode: the same kernels and split plan on the library's fixed scratch
array instead of a workspace, so the outputs must be bit-identical, and both
within the bf16 tolerance of the oracle. Two calls in a row on the same array,
the second on a smaller input. (A request too large for the array is
rejected on the host before any launch: tests/test_abi.py.)"""
import numpy as np
import pytest
import torch

from _gpu import assert_close, assert_lse_close, needs_gpu, oracle_decode, to_dev
from datagen.workloads import make_inputs

pytestmark = [pytest.mark.gpu, needs_gpu]


def _both(inp, num_splits):
    import long_context_decode_kv_amd as lib
    dev = {k: to_dev(v) for k, v in inp.items() if v is not None}
    args = (dev["q"], dev["k"], dev["v"])
    kw = dict(k_scale=dev.get("k_scale"), v_scale=dev.get("v_scale"), kv_lens=dev.get("kv_lens"),
              num_splits=num_splits)
    ref, ref_lse = lib.attn_decode(*args, **kw)
    out = torch.full_like(dev["q"], float("nan"))
    lse = torch.full((dev["q"].shape[0], dev["q"].shape[1]), float("nan"), device="cuda")
    lib.attn_decode_noalloc(*args, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    return (out, lse), (ref, ref_lse)


def _check(inp, num_splits, what):
    (out, lse), (ref, ref_lse) = _both(inp, num_splits)
    print("%s: splits %s" % (what, num_splits), flush=True)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), what
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), what
    o, l = oracle_decode(inp)
    B, Hq = inp["q"].shape[:2]
    assert_close(out.float().cpu().numpy().astype(np.float64).reshape(B, Hq, -1), o, "bf16", what)
    assert_lse_close(lse.cpu().numpy().astype(np.float64), l, 2e-3)


def test_noalloc_twice_second_smaller():
    # fused merge (one workgroup per CU or fewer): 8 KV heads x 16 splits
    _check(make_inputs(2, L=40000, seed=301), 16, "noalloc 40000 keys")
    # a smaller input right after, on the same array (counters left by the first)
    _check(make_inputs(2, L=3000, Hq=8, Hkv=2, seed=302), 5, "noalloc 3000 keys")


def test_noalloc_second_kernel_merge_and_auto_plan():
    # more workgroups than CUs: partials in the array, merged by the second kernel
    _check(make_inputs(2, L=70000, seed=303), 100, "noalloc 70000 keys, 100 splits")
    _check(make_inputs(2, L=20000, seed=304), 0, "noalloc 20000 keys, automatic plan")
    inp = make_inputs(3, B=4, L=9000, lens=(1, 9000), seed=305)
    _check(inp, 0, "noalloc ragged batch")
