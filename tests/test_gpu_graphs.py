"""HIP-graph capture of the prefill entry points.

A serving loop records its launches once and replays them.  Each test here
captures one call of a prefill entry point (through the C ABI, on the
capturing stream) and replays the graph three times, with eager launches of
the same kernels and host synchronisations in between; every replay must be
bitwise equal to the eager call on the same inputs.  The workloads are sized so
that the bf16 calls run in more than one segment (several launches of each
kernel, the state carried between them).
"""
import numpy as np
import pytest
import torch

import kda_inputs
import kimi_delta_attention_chunked_amd as kda

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a, dtype=torch.float32):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dtype)


def replay_and_compare(graph, outs, refs, eager_between):
    for r in range(3):
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        eager_between()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("o", "S_T", "ckpt"), outs, refs):
            assert torch.equal(got, ref), "replay %d: %s differs from the eager call" % (r, name)


@pytest.mark.parametrize("dtype,H,T,D", [("bf16", 32, 8192, 128), ("fp32", 2, 700, 64)])
def test_prefill_graph_replays_equal_eager(dtype, H, T, D):
    dt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    d = kda_inputs.prefill_inputs(1, B=1, H=H, T=T, D=D, dtype=dtype, seed=91)
    q, k, v = (dev(d[x], dt) for x in ("q", "k", "v"))
    g, beta, S0 = dev(d["g"]), dev(d["beta"]), dev(d["S0"])
    N = 1024 if dtype == "bf16" else 256
    if dtype == "bf16":
        assert kda.segment_tokens(q, v) < T, "the workload should run in several segments"
    o_e, S_e, ck_e = kda.prefill(q, k, v, g, beta, S0=S0, checkpoint_every=N)
    o, S_T, ck = torch.empty_like(o_e), torch.empty_like(S_e), torch.empty_like(ck_e)
    ws = kda.prefill_workspace(q, v)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.prefill(q, k, v, g, beta, S0=S0, checkpoint_every=N, o=o, S_T=S_T, ckpt=ck, ws=ws)

    def eager():  # the same kernels, eagerly, on other buffers
        kda.prefill(q, k, v, g, beta, S0=S0, checkpoint_every=N)

    replay_and_compare(graph, (o, S_T, ck), (o_e, S_e, ck_e), eager)


def test_prefill_varlen_graph_replays_equal_eager():
    lens = [1000, 0, 3000, 65, 4000, 1]
    H, D = 32, 128
    cu = [0] + list(np.cumsum(lens))
    total = cu[-1]
    d = kda_inputs.prefill_inputs(1, B=1, T=total, H=H, D=D, seed=92)
    s0 = kda_inputs.prefill_inputs(1, B=len(lens), T=0, H=H, D=D, seed=93)["S0"]
    bf = torch.bfloat16
    q, k, v = (dev(d[x][0], bf) for x in ("q", "k", "v"))
    g, beta, S0 = dev(d["g"][0]), dev(d["beta"][0]), dev(s0)
    o_e, S_e, ck_e = kda.prefill_varlen(q, k, v, g, beta, cu, S0=S0, checkpoint_every=512)
    o, S_T, ck = torch.empty_like(o_e), torch.empty_like(S_e), torch.empty_like(ck_e)
    ws = kda.varlen_workspace(q, v, cu)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cu_host = list(cu)  # a host list that the call reads; changed after capture
    with torch.cuda.graph(graph):
        kda.prefill_varlen(q, k, v, g, beta, cu_host, S0=S0, checkpoint_every=512, o=o, S_T=S_T, ckpt=ck,
                           ws=ws)
    cu_host[1:] = [0] * len(lens)  # the captured call keeps the offsets it was recorded with

    def eager():  # other offsets through the same kernels, on other buffers
        kda.prefill_varlen(q, k, v, g, beta, [0, total // 2, total], checkpoint_every=512)

    replay_and_compare(graph, (o, S_T, ck), (o_e, S_e, ck_e), eager)
