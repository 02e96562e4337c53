"""kda_prefill_noalloc: the prefill with its operand records in the library's
static device scratch instead of a caller workspace.

It runs the same kernels as kda_prefill; only the segment length differs (the
records of one segment must fit the 64 MiB scratch), and the state passes
between segments in fp32, so its outputs must equal kda_prefill's bitwise.
Two calls in a row, the second smaller than the first (the scratch keeps the
first call's records), then fp32 (no scratch), the size limit, and a
graph-captured call replayed.
"""
import numpy as np
import pytest
import torch

import kda_inputs
import kimi_delta_attention_chunked_amd as kda

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCRATCH = 64 << 20
REC = {128: 72704, 64: 39936}


def dev(a, dtype=torch.float32):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dtype)


def inputs(dtype, seed, **kw):
    dt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    d = kda_inputs.prefill_inputs(1, dtype=dtype, seed=seed, **kw)
    return [dev(d[x], dt) for x in ("q", "k", "v")] + [dev(d["g"]), dev(d["beta"]), dev(d["S0"])]


def same(a, b, what):
    for name, x, y in zip(("o", "S_T", "ckpt"), a, b):
        assert (x is None) == (y is None), what + " " + name
        if x is not None:
            assert torch.equal(x, y), "%s: %s differs from kda_prefill" % (what, name)


def test_noalloc_equals_prefill_two_calls_then_smaller():
    # First call: B=1, H=32, T=4096 -> 64 chunks of 32 heads = 149 MB of
    # records, so the 64 MiB scratch runs it in 3 segments (kda_prefill: 1).
    q, k, v, g, b, S0 = inputs("bf16", 101, B=1, H=32, T=4096, D=128)
    assert 32 * 64 * REC[128] > 2 * SCRATCH
    ref = kda.prefill(q, k, v, g, b, S0=S0, checkpoint_every=1024)
    got = kda.prefill_noalloc(q, k, v, g, b, S0=S0, checkpoint_every=1024)
    torch.cuda.synchronize()
    same(got, ref, "call 1 (B=1, H=32, T=4096)")
    # Second call, smaller: a ragged tail, one segment, other heads.
    q, k, v, g, b, S0 = inputs("bf16", 102, B=2, H=3, T=333, D=64)
    ref = kda.prefill(q, k, v, g, b, S0=S0, checkpoint_every=128)
    got = kda.prefill_noalloc(q, k, v, g, b, S0=S0, checkpoint_every=128)
    torch.cuda.synchronize()
    same(got, ref, "call 2 (B=2, H=3, T=333)")


def test_noalloc_fp32_and_empty():
    q, k, v, g, b, S0 = inputs("fp32", 103, B=1, H=2, T=200, D=64)
    same(kda.prefill_noalloc(q, k, v, g, b, S0=S0), kda.prefill(q, k, v, g, b, S0=S0), "fp32")
    q, k, v, g, b, S0 = inputs("bf16", 104, B=1, H=2, T=0, D=128)
    o, S_T, _ = kda.prefill_noalloc(q, k, v, g, b, S0=S0)
    torch.cuda.synchronize()
    assert torch.equal(S_T, S0)


def test_noalloc_rejects_more_heads_than_the_scratch_holds():
    H = SCRATCH // REC[128] + 1  # one chunk of every head no longer fits
    q = torch.zeros((1, 64, H, 128), dtype=torch.bfloat16, device=DEV)
    g = torch.zeros((1, 64, H, 128), device=DEV)
    b = torch.zeros((1, 64, H), device=DEV)
    S_T = torch.full((1, H, 128, 128), 7.0, device=DEV)
    with pytest.raises(kda.KDAError) as e:
        kda.prefill_noalloc(q, q, q, g, b, S_T=S_T)
    assert e.value.code == 6  # KDA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((S_T == 7.0).all()), "a rejected call must write nothing"


def test_noalloc_graph_replays_equal_eager():
    q, k, v, g, b, S0 = inputs("bf16", 105, B=1, H=32, T=2048, D=128)
    ref = kda.prefill(q, k, v, g, b, S0=S0, checkpoint_every=512)
    o, S_T, ck = (torch.empty_like(x) for x in ref)
    kda.prefill_noalloc(q, k, v, g, b, S0=S0, checkpoint_every=512, o=o, S_T=S_T, ckpt=ck)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.prefill_noalloc(q, k, v, g, b, S0=S0, checkpoint_every=512, o=o, S_T=S_T, ckpt=ck)
    for r in range(3):
        for x in (o, S_T, ck):
            x.fill_(float("nan"))
        kda.prefill_noalloc(*inputs("bf16", 106 + r, B=1, H=4, T=300, D=128))  # eager use of the scratch
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same((o, S_T, ck), ref, "replay %d" % r)
