"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Error metric: Frobenius-relative error ||X - X_ref|| / ||X_ref||, in fp64, per
output tensor.  Bounds: 1e-4 when q/k/v are fp32, 1e-2 when they are bf16 (the
kernels then use bf16 MFMA operands with fp32 accumulation).  Full-size
workloads run completely on the GPU, in the configuration the benchmark times;
the oracle then checks a sample of (batch, head) chains, each of which is an
independent recurrence.
"""
import ctypes

import numpy as np
import pytest
import torch

import kda_inputs
import kimi_delta_attention_chunked_amd as kda
import oracle

pytestmark = pytest.mark.gpu

DT = {"fp32": torch.float32, "bf16": torch.bfloat16}
TOL = {"fp32": 1e-4, "bf16": 1e-2}
DEV = "cuda:0"


def dev(a, dtype=torch.float32):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dtype)


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def check(name, got, ref, tol):
    err = rel(got, ref)
    print("%s: rel err %.3e (bound %.0e)" % (name, err, tol), flush=True)
    assert err <= tol, "%s: %.3e > %.0e" % (name, err, tol)


def gpu_prefill(d, ckpt_every=0, S0="input"):
    dt = DT[d["dtype"]]
    S0 = d["S0"] if isinstance(S0, str) else S0
    o, S_T, ck = kda.prefill(dev(d["q"], dt), dev(d["k"], dt), dev(d["v"], dt), dev(d["g"]),
                             dev(d["beta"]), dev(S0), checkpoint_every=ckpt_every)
    torch.cuda.synchronize()
    return (o.float().cpu().numpy(), S_T.cpu().numpy(),
            None if ck is None else ck.cpu().numpy())


def head_slice(d, heads, keys=("q", "k", "v", "g", "beta")):
    """Inputs of a subset of heads (each head is an independent chain)."""
    out = {key: np.ascontiguousarray(d[key][:, :, heads]) for key in keys}
    out["S0"] = None if d["S0"] is None else np.ascontiguousarray(d["S0"][:, heads])
    return out


def compare_prefill(d, ckpt_every=0, heads=None, label=""):
    tol = TOL[d["dtype"]]
    o, S_T, ck = gpu_prefill(d, ckpt_every)
    ref_in = d if heads is None else head_slice(d, heads)
    o_ref, S_ref, ck_ref = oracle.prefill(ref_in["q"], ref_in["k"], ref_in["v"], ref_in["g"],
                                          ref_in["beta"], ref_in["S0"], ckpt_every=ckpt_every)
    sel = np.s_[:] if heads is None else np.s_[:, :, heads]
    check(label + " o", o[sel], o_ref, tol)
    check(label + " S_T", S_T[:, heads] if heads is not None else S_T, S_ref, tol)
    if ckpt_every:
        assert ck.shape[0] == ck_ref.shape[0]
        for j in range(ck.shape[0]):
            got = ck[j][:, heads] if heads is not None else ck[j]
            check(label + " ckpt[%d]" % j, got, ck_ref[j], tol)
    return o, S_T, ck


# -- the workloads -------------------------------------------------------------

def test_prefill_tiny_fp32():
    compare_prefill(kda_inputs.prefill_inputs(0), label="tiny fp32")


def test_prefill_mid_bf16_all_heads():
    compare_prefill(kda_inputs.prefill_inputs(1), label="mid bf16")


def test_prefill_fp32_dk128_with_state_and_checkpoints():
    # The mid workload's distributions (S0 included) in fp32 at a size the
    # oracle finishes in seconds: many chunks, a ragged tail, 4 checkpoints.
    d = kda_inputs.prefill_inputs(1, B=2, H=4, T=1000, D=128, dtype="fp32", seed=5)
    compare_prefill(d, ckpt_every=256, label="fp32 D=128")


def test_prefill_long_bf16_sampled_heads():
    compare_prefill(kda_inputs.prefill_inputs(2), heads=[0, 13, 31], label="long bf16")


def test_prefill_agentic_checkpoints_sampled_heads():
    d = kda_inputs.prefill_inputs(3)
    compare_prefill(d, ckpt_every=d["ckpt_every"], heads=[3, 28], label="agentic bf16")


def test_prefill_beyond_2_31_elements_per_tensor():
    # T = 600,037 tokens of 32 heads: q, k, v, g and o each hold 2.46e9
    # elements, so every element offset past token 524,288 exceeds 2^31.  The
    # tokens before the last 3,000 have k = 0 and g = 0 and leave the state
    # exactly S0: the checkpoints there must equal S0 bitwise, the outputs
    # there are S0^T q, and the oracle runs only the last 3,000 tokens (which
    # cross a segment boundary) from S0.
    d = kda_inputs.huge_prefill_inputs(device=DEV)
    T, H, D, tail = d["T"], d["H"], d["D"], d["tail"]
    assert T * H * D > 2 ** 31
    o, S_T, ck = kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"],
                             checkpoint_every=131072)
    torch.cuda.synchronize()
    assert ck.shape[0] == 5
    for j in range(4):
        assert torch.equal(ck[j], d["S0"]), "checkpoint %d differs from S0" % j
    S0 = d["S0"].cpu().numpy().astype(np.float64)
    ts = [0, 1, 2 ** 31 // (H * D) - 1, 2 ** 31 // (H * D), T - tail - 1]
    qs = d["q"][0, ts].float().cpu().numpy().astype(np.float64)      # [token, head, dk]
    o_ref = np.einsum("hij,thi->thj", S0[0], qs)
    check("prefix o (sampled tokens)", o[0, ts].float().cpu().numpy(), o_ref, TOL["bf16"])
    heads, sl = [0, 31], slice(T - tail, T)

    def host(x):
        return np.ascontiguousarray(x[:, sl][:, :, heads].float().cpu().numpy())

    o_t, S_t, _ = oracle.prefill(host(d["q"]), host(d["k"]), host(d["v"]), host(d["g"]),
                                 host(d["beta"]), np.ascontiguousarray(S0[:, heads]))
    check("tail o", host(o), o_t, TOL["bf16"])
    check("S_T", S_T[:, heads].cpu().numpy(), S_t, TOL["bf16"])
    check("last checkpoint", ck[4][:, heads].cpu().numpy(), S_t, TOL["bf16"])
    del d, o, S_T, ck
    torch.cuda.empty_cache()


def test_decode_444_steps_sampled_sequences():
    d = kda_inputs.decode_inputs(4)
    dt = DT[d["dtype"]]
    seqs = [0, 21, 63]
    S = dev(d["S0"])
    q, k, v = (dev(d[x], dt) for x in ("q", "k", "v"))
    g, beta = dev(d["g"]), dev(d["beta"])
    outs = []
    for s in range(d["steps"]):
        outs.append(kda.decode_step(q[s], k[s], v[s], g[s], beta[s], S))
    torch.cuda.synchronize()
    o = torch.stack(outs).float().cpu().numpy()
    S_ref = d["S0"][seqs]
    o_ref = []
    for s in range(d["steps"]):
        o_s, S_ref = oracle.decode_step(d["q"][s, seqs], d["k"][s, seqs], d["v"][s, seqs],
                                        d["g"][s, seqs], d["beta"][s, seqs], S_ref)
        o_ref.append(o_s)
    check("decode o (444 steps)", o[:, seqs], np.stack(o_ref), TOL["bf16"])
    check("decode S (444 steps)", S.cpu().numpy()[seqs], S_ref, TOL["bf16"])


# -- edge cases ----------------------------------------------------------------

@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("fp32", 128), ("fp32", 64)])
@pytest.mark.parametrize("T,ckpt_every", [(1, 0), (63, 64), (64, 64), (65, 64), (200, 128),
                                          (300, 64)])
def test_prefill_ragged_lengths_and_checkpoints(dtype, D, T, ckpt_every):
    d = kda_inputs.prefill_inputs(1, B=2, H=3, T=T, D=D, dtype=dtype, seed=7 + T)
    compare_prefill(d, ckpt_every=ckpt_every, label="%s D=%d T=%d" % (dtype, D, T))


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 128), ("fp32", 64)])
@pytest.mark.parametrize("case", ["no_decay", "strong_decay", "beta0", "beta1", "q_equals_k"])
def test_prefill_special_cases(dtype, D, case):
    d = kda_inputs.prefill_inputs(1, B=1, H=2, T=200, D=D, dtype=dtype, seed=11)
    if case == "no_decay":
        d["g"] = np.zeros_like(d["g"])
    elif case == "strong_decay":          # the documented edge of the domain
        d["g"] = np.full_like(d["g"], -1.0)
    elif case == "beta0":
        d["beta"] = np.zeros_like(d["beta"])
    elif case == "beta1":
        d["beta"] = np.ones_like(d["beta"])
    elif case == "q_equals_k":
        d["q"] = d["k"].copy()
    compare_prefill(d, ckpt_every=64, label="%s %s" % (dtype, case))


def test_prefill_zero_length_returns_initial_state():
    d = kda_inputs.prefill_inputs(1, B=1, H=2, T=0)
    o, S_T, ck = gpu_prefill(d, ckpt_every=64)
    assert o.shape == (1, 0, 2, 128) and ck is None
    assert np.array_equal(S_T, d["S0"])


def test_prefill_null_state_equals_zero_state_bitwise():
    d = kda_inputs.prefill_inputs(1, B=1, H=4, T=333, seed=3)
    a = gpu_prefill(d, S0=None)
    b = gpu_prefill(d, S0=np.zeros_like(d["S0"]))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_prefill_final_state_may_alias_initial_state():
    d = kda_inputs.prefill_inputs(1, B=2, H=3, T=250, seed=4)
    o1, S1, _ = gpu_prefill(d)
    dt = DT[d["dtype"]]
    S = dev(d["S0"])
    o2, S2, _ = kda.prefill(dev(d["q"], dt), dev(d["k"], dt), dev(d["v"], dt), dev(d["g"]),
                            dev(d["beta"]), S, S_T=S)
    torch.cuda.synchronize()
    assert S2.data_ptr() == S.data_ptr()
    assert np.array_equal(S2.cpu().numpy(), S1) and np.array_equal(o2.float().cpu().numpy(), o1)


def test_prefill_resume_from_checkpoint():
    """Checkpoint j passed back as S0 reproduces the rest of the sequence."""
    d = kda_inputs.prefill_inputs(1, B=1, H=2, T=320, seed=5)
    o, S_T, ck = gpu_prefill(d, ckpt_every=128)
    rest = {key: np.ascontiguousarray(d[key][:, 128:]) for key in ("q", "k", "v", "g", "beta")}
    rest.update(dtype=d["dtype"], S0=ck[0])
    o2, S2, _ = gpu_prefill(rest)
    check("resume o", o2, o[:, 128:], 1e-2)
    check("resume S_T", S2, S_T, 1e-2)


def test_prefill_deterministic():
    d = kda_inputs.prefill_inputs(1, B=1, H=8, T=1000, seed=6)
    a = gpu_prefill(d, ckpt_every=256)
    b = gpu_prefill(d, ckpt_every=256)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("dtype,D", [("fp32", 64), ("fp32", 128), ("bf16", 64), ("bf16", 128)])
def test_decode_steps_match_oracle(dtype, D):
    d = kda_inputs.decode_inputs(4, N=5, H=3, D=D, steps=20, dtype=dtype, seed=8)
    dt = DT[dtype]
    S = dev(d["S0"])
    S_ref = d["S0"]
    for s in range(20):
        o = kda.decode_step(dev(d["q"][s], dt), dev(d["k"][s], dt), dev(d["v"][s], dt),
                            dev(d["g"][s]), dev(d["beta"][s]), S)
        o_ref, S_ref = oracle.decode_step(d["q"][s], d["k"][s], d["v"][s], d["g"][s],
                                          d["beta"][s], S_ref)
        check("decode %s D=%d o[%d]" % (dtype, D, s), o.float().cpu().numpy(), o_ref, TOL[dtype])
    check("decode %s D=%d S" % (dtype, D), S.cpu().numpy(), S_ref, TOL[dtype])


def test_decode_graph_replays_equal_eager_steps():
    # Six decode steps captured in a HIP graph, replayed three times, each
    # from a different state set eagerly before the replay (with eager steps
    # of the same kernels in between): every replay equals the eager steps
    # from that state, bitwise.
    N, H, D, T = 8, 4, 128, 6
    d = kda_inputs.decode_inputs(4, N=N, H=H, D=D, steps=T, seed=81)
    bf = torch.bfloat16
    q, k, v = dev(d["q"], bf), dev(d["k"], bf), dev(d["v"], bf)
    g, b = dev(d["g"]), dev(d["beta"])
    S = torch.empty((N, H, D, D), device=DEV)
    o = torch.empty((T, N, H, D), dtype=bf, device=DEV)
    S.copy_(dev(d["S0"]))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(T):
            kda.decode_step(q[t], k[t], v[t], g[t], b[t], S, o=o[t])
    for r in range(3):
        start = dev(d["S0"]) * (1.0 + 0.5 * r)
        S.copy_(start)
        o.zero_()
        graph.replay()
        Se = start.clone()
        oe = torch.stack([kda.decode_step(q[t], k[t], v[t], g[t], b[t], Se) for t in range(T)])
        torch.cuda.synchronize()
        assert torch.equal(S, Se) and torch.equal(o, oe), "replay %d differs from the eager steps" % r


def test_decode_steps_equal_prefill_on_gpu():
    d = kda_inputs.prefill_inputs(1, B=2, H=2, T=70, seed=9)
    o, S_T, _ = gpu_prefill(d)
    dt = DT[d["dtype"]]
    S = dev(d["S0"])
    for t in range(70):
        od = kda.decode_step(dev(d["q"][:, t], dt), dev(d["k"][:, t], dt), dev(d["v"][:, t], dt),
                             dev(d["g"][:, t]), dev(d["beta"][:, t]), S)
        check("decode vs prefill o[%d]" % t, od.float().cpu().numpy(), o[:, t], 1e-2)
    check("decode vs prefill S", S.cpu().numpy(), S_T, 1e-2)


def test_invalid_arguments_raise_before_launch():
    q = torch.zeros((1, 64, 1, 96), dtype=torch.bfloat16, device=DEV)
    g = torch.zeros((1, 64, 1, 96), device=DEV)
    beta = torch.zeros((1, 64, 1), device=DEV)
    with pytest.raises(kda.KDAError) as e:
        kda.prefill(q, q, q, g, beta)
    assert e.value.code == 5  # KDA_ERR_UNSUPPORTED


@pytest.mark.parametrize("D", [128, 64])
def test_prefill_stages_equal_prefill_bitwise(D):
    """kda_prefill_chunk_prep then kda_prefill_chunk_recur == kda_prefill."""
    d = kda_inputs.prefill_inputs(1, B=2, H=3, T=333, D=D, seed=10)
    o, S_T, ck = gpu_prefill(d, ckpt_every=128)
    q, k, v = (dev(d[x], torch.bfloat16) for x in ("q", "k", "v"))
    ws = kda.workspace(q, v)
    kda.prefill_chunk_prep(q, k, v, dev(d["g"]), dev(d["beta"]), ws)
    o2, S2, ck2 = kda.prefill_chunk_recur(ws, q, v, dev(d["S0"]), checkpoint_every=128)
    torch.cuda.synchronize()
    assert np.array_equal(o2.float().cpu().numpy(), o)
    assert np.array_equal(S2.cpu().numpy(), S_T)
    assert np.array_equal(ck2.cpu().numpy(), ck)


def test_prefill_recur_zero_length_writes_initial_state():
    d = kda_inputs.prefill_inputs(1, B=1, H=2, T=0)
    q, v = dev(d["q"], torch.bfloat16), dev(d["v"], torch.bfloat16)
    assert kda.workspace(q, v) is None
    o, S_T, _ = kda.prefill_chunk_recur(None, q, v, dev(d["S0"]))
    torch.cuda.synchronize()
    assert np.array_equal(S_T.cpu().numpy(), d["S0"])


# -- packed sequences of different lengths (kda_prefill_varlen) ---------------

def packed_inputs(lens, H, D, seed):
    """One seeded B=1 token stream cut into consecutive sequences of the given
    lengths, plus per-sequence initial states."""
    total = int(sum(lens))
    d = kda_inputs.prefill_inputs(1, B=1, T=total, H=H, D=D, seed=seed)
    s0 = kda_inputs.prefill_inputs(1, B=len(lens), T=0, H=H, D=D, seed=seed + 1)["S0"]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return d, s0, [int(x) for x in cu]


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("ckpt_every", [0, 64, 128])
def test_prefill_varlen_matches_oracle_per_sequence(D, ckpt_every):
    lens = [1, 63, 64, 65, 0, 200, 130, 7]
    H = 3
    d, s0, cu = packed_inputs(lens, H, D, seed=20 + D + ckpt_every)
    bf = torch.bfloat16
    o, S_T, ck = kda.prefill_varlen(dev(d["q"][0], bf), dev(d["k"][0], bf), dev(d["v"][0], bf),
                                    dev(d["g"][0]), dev(d["beta"][0]), cu, S0=dev(s0),
                                    checkpoint_every=ckpt_every)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    S_T = S_T.cpu().numpy()
    ck = None if ck is None else ck.cpu().numpy()
    c = 0
    for i, L in enumerate(lens):
        a, b = cu[i], cu[i + 1]
        sl = lambda x: np.ascontiguousarray(x[:, a:b])
        o_ref, S_ref, ck_ref = oracle.prefill(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]),
                                              sl(d["beta"]), s0[i:i + 1], ckpt_every=ckpt_every)
        if L:
            check("varlen D=%d seq %d o" % (D, i), o[a:b], o_ref[0], 1e-2)
        check("varlen D=%d seq %d S_T" % (D, i), S_T[i], S_ref[0], 1e-2)
        n = -(-L // ckpt_every) if ckpt_every else 0
        for j in range(n):
            check("varlen D=%d seq %d ckpt[%d]" % (D, i, j), ck[c + j], ck_ref[j][0], 1e-2)
        c += n
    assert c == (0 if ck is None else ck.shape[0])


def test_prefill_varlen_equal_lengths_equal_batched_prefill_bitwise():
    """B sequences of T tokens packed end to end == the [B,T,H] prefill."""
    B, T, H = 3, 257, 4
    d = kda_inputs.prefill_inputs(1, B=B, T=T, H=H, seed=30)
    bf = torch.bfloat16
    o, S_T, ck = kda.prefill(dev(d["q"], bf), dev(d["k"], bf), dev(d["v"], bf), dev(d["g"]),
                             dev(d["beta"]), dev(d["S0"]), checkpoint_every=128)
    pk = lambda x: x.reshape((B * T,) + x.shape[2:])
    o2, S2, ck2 = kda.prefill_varlen(pk(dev(d["q"], bf)), pk(dev(d["k"], bf)), pk(dev(d["v"], bf)),
                                     pk(dev(d["g"])), pk(dev(d["beta"])), [0, T, 2 * T, 3 * T],
                                     S0=dev(d["S0"]), checkpoint_every=128)
    torch.cuda.synchronize()
    assert torch.equal(o2.reshape(o.shape), o)
    assert torch.equal(S2, S_T)
    # uniform checkpoints are [n, B, H, ...]; packed ones are per sequence, consecutive
    n = ck.shape[0]
    for b in range(B):
        assert torch.equal(ck2[b * n:(b + 1) * n], ck[:, b])


def varlen_segments(cu, H, D):
    """Whether kda_prefill_varlen splits these sequences into segments: its
    workspace then holds fewer records than the sequences have chunks."""
    lib = kda.library()
    arr = (ctypes.c_int * len(cu))(*cu)
    ws = lib.kda_prefill_varlen_workspace_size(arr, len(cu) - 1, H, D, D, 1)
    chunks = sum(-(-(b - a) // 64) for a, b in zip(cu, cu[1:]))
    return ws < H * chunks * {128: 72704, 64: 39936}[D]


@pytest.mark.parametrize("with_s0", [True, False], ids=["S0", "zero-state"])
def test_prefill_varlen_segmented_equals_batched_prefill_bitwise(with_s0):
    """Four 8190-token sequences of 32 heads: the packed prefill runs them in
    segments of 103 chunks (boundaries inside sequences, the state carried
    between segments), the batched prefill in segments of its own; results are bitwise
    equal, checkpoints included, from given initial states or from zeros."""
    B, T, H = 4, 8190, 32
    d = kda_inputs.prefill_inputs(1, B=B, T=T, H=H, seed=32)
    cu = [0, T, 2 * T, 3 * T, 4 * T]
    assert varlen_segments(cu, H, 128)
    bf = torch.bfloat16
    q, k, v, g, b = dev(d["q"], bf), dev(d["k"], bf), dev(d["v"], bf), dev(d["g"]), dev(d["beta"])
    S0 = dev(d["S0"]) if with_s0 else None
    o, S_T, ck = kda.prefill(q, k, v, g, b, S0, checkpoint_every=4096)
    pk = lambda x: x.reshape((B * T,) + x.shape[2:])
    o2, S2, ck2 = kda.prefill_varlen(pk(q), pk(k), pk(v), pk(g), pk(b), cu, S0=S0, checkpoint_every=4096)
    torch.cuda.synchronize()
    assert torch.equal(o2.reshape(o.shape), o)
    assert torch.equal(S2, S_T)
    n = ck.shape[0]
    for i in range(B):
        assert torch.equal(ck2[i * n:(i + 1) * n], ck[:, i])


def test_prefill_varlen_many_heads_short_segments_bitwise():
    """Four 500-token sequences of 256 heads: the packed prefill's records
    allow segments of at most 13 chunks (three of 11, boundaries inside
    sequences), while
    the batched prefill runs in one pass; results are bitwise equal."""
    B, T, H = 4, 500, 256
    d = kda_inputs.prefill_inputs(1, B=B, T=T, H=H, seed=36)
    cu = [0, T, 2 * T, 3 * T, 4 * T]
    assert varlen_segments(cu, H, 128)
    bf = torch.bfloat16
    q, k, v, g, b = dev(d["q"], bf), dev(d["k"], bf), dev(d["v"], bf), dev(d["g"]), dev(d["beta"])
    S0 = dev(d["S0"])
    assert kda.segment_tokens(q, v) == T
    o, S_T, ck = kda.prefill(q, k, v, g, b, S0, checkpoint_every=128)
    pk = lambda x: x.reshape((B * T,) + x.shape[2:])
    o2, S2, ck2 = kda.prefill_varlen(pk(q), pk(k), pk(v), pk(g), pk(b), cu, S0=S0, checkpoint_every=128)
    torch.cuda.synchronize()
    assert torch.equal(o2.reshape(o.shape), o)
    assert torch.equal(S2, S_T)
    n = ck.shape[0]
    for i in range(B):
        assert torch.equal(ck2[i * n:(i + 1) * n], ck[:, i])


def test_prefill_varlen_segmented_mixed_lengths_sampled_heads():
    """Sequences of mixed length, empty and one-token ones among them, with 32
    heads, so the packed prefill runs in segments: every sequence's outputs,
    final state and checkpoints on two heads against the oracle."""
    lens = [0, 5000, 1, 0, 64, 3001, 0, 7000, 130, 2048, 65, 0, 1700]
    H, D, ckpt_every = 32, 128, 2048
    heads = [0, 21]
    d, s0, cu = packed_inputs(lens, H, D, seed=33)
    assert varlen_segments(cu, H, D)
    bf = torch.bfloat16
    o, S_T, ck = kda.prefill_varlen(dev(d["q"][0], bf), dev(d["k"][0], bf), dev(d["v"][0], bf),
                                    dev(d["g"][0]), dev(d["beta"][0]), cu, S0=dev(s0),
                                    checkpoint_every=ckpt_every)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()[:, heads]
    S_T = S_T.cpu().numpy()[:, heads]
    ck = ck.cpu().numpy()[:, heads]
    c = 0
    for i, L in enumerate(lens):
        a, b = cu[i], cu[i + 1]
        sl = lambda x: np.ascontiguousarray(x[:, a:b][:, :, heads])
        o_ref, S_ref, ck_ref = oracle.prefill(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]),
                                              sl(d["beta"]), np.ascontiguousarray(s0[i:i + 1, heads]),
                                              ckpt_every=ckpt_every)
        if L:
            check("segmented varlen seq %d o" % i, o[a:b], o_ref[0], 1e-2)
        check("segmented varlen seq %d S_T" % i, S_T[i], S_ref[0], 1e-2)
        n = -(-L // ckpt_every)
        for j in range(n):
            check("segmented varlen seq %d ckpt[%d]" % (i, j), ck[c + j], ck_ref[j][0], 1e-2)
        c += n
    assert c == ck.shape[0]


def test_prefill_varlen_all_empty_sequences_return_initial_states():
    H, D = 2, 128
    s0 = kda_inputs.prefill_inputs(1, B=3, T=0, H=H, D=D, seed=31)["S0"]
    z = torch.zeros((0, H, D), dtype=torch.bfloat16, device=DEV)
    zf = torch.zeros((0, H, D), device=DEV)
    o, S_T, ck = kda.prefill_varlen(z, z, z, zf, torch.zeros((0, H), device=DEV), [0, 0, 0, 0],
                                    S0=dev(s0), checkpoint_every=64)
    torch.cuda.synchronize()
    assert o.shape == (0, H, D) and ck is None
    assert np.array_equal(S_T.cpu().numpy(), s0)


# -- several tokens per sequence: speculative verification and commit --------

def multi_inputs(N, T, H, D, dtype, seed):
    """Seeded [N,T,H,.] token inputs and a seeded state (the decode recipe)."""
    d = kda_inputs.decode_inputs(4, N=N, H=H, D=D, steps=T, dtype=dtype, seed=seed)
    tr = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1))  # [T,N,...] -> [N,T,...]
    return {x: tr(d[x]) for x in ("q", "k", "v", "g", "beta")}, d["S0"]


def oracle_multi(x, S0, counts):
    """The oracle's prefill of each sequence's first counts[n] tokens from S0[n]."""
    N = S0.shape[0]
    outs, states = [], []
    for n in range(N):
        c = counts[n]
        sl = lambda a: np.ascontiguousarray(a[n:n + 1, :c])
        o_ref, S_ref, _ = oracle.prefill(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]),
                                         S0[n:n + 1])
        outs.append(o_ref[0])
        states.append(S_ref[0])
    return outs, states


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("fp32", 128), ("fp32", 64)])
def test_decode_multi_verify_then_commit(dtype, D):
    N, T, H = 6, 9, 3
    x, S0 = multi_inputs(N, T, H, D, dtype, seed=40 + D)
    dt = DT[dtype]
    tol = TOL[dtype]
    args = [dev(x["q"], dt), dev(x["k"], dt), dev(x["v"], dt), dev(x["g"]), dev(x["beta"])]
    S = dev(S0)
    # verification: outputs of all T drafts, state untouched
    o = kda.decode_multi(*args, S, update_state=False)
    torch.cuda.synchronize()
    assert np.array_equal(S.cpu().numpy(), S0)
    outs, _ = oracle_multi(x, S0, [T] * N)
    for n in range(N):
        check("verify %s D=%d seq %d o" % (dtype, D, n), o[n].float().cpu().numpy(), outs[n], tol)
    # commit of per-sequence accepted counts (out-of-range counts clamp to [0, T])
    acc = [0, 1, 4, T, -2, 99]
    cnt = [min(max(a, 0), T) for a in acc]
    kda.decode_multi(*args, S, n_tokens=torch.tensor(acc, dtype=torch.int32, device=DEV), want_output=False)
    torch.cuda.synchronize()
    _, states = oracle_multi(x, S0, cnt)
    Sg = S.cpu().numpy()
    for n in range(N):
        if cnt[n] == 0:
            assert np.array_equal(Sg[n], S0[n])
        else:
            check("commit %s D=%d seq %d (%d tokens) S" % (dtype, D, n, cnt[n]), Sg[n], states[n], tol)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decode_multi_strong_decay(dtype):
    # Decays far beyond the prefill's domain (g down to -60 per token, so
    # e^{G} underflows within two tokens): the pairwise factors stay <= 1.
    N, T, H, D = 3, 12, 2, 128
    x, S0 = multi_inputs(N, T, H, D, dtype, seed=60)
    x["g"] = np.random.default_rng(61).uniform(-60.0, -0.001, x["g"].shape).astype(np.float32)
    dt = DT[dtype]
    args = [dev(x["q"], dt), dev(x["k"], dt), dev(x["v"], dt), dev(x["g"]), dev(x["beta"])]
    S = dev(S0)
    o = kda.decode_multi(*args, S, update_state=False)
    acc = [T, 5, 1]
    kda.decode_multi(*args, S, n_tokens=torch.tensor(acc, dtype=torch.int32, device=DEV), want_output=False)
    torch.cuda.synchronize()
    outs, _ = oracle_multi(x, S0, [T] * N)
    _, states = oracle_multi(x, S0, acc)
    Sg = S.cpu().numpy()
    for n in range(N):
        check("strong decay %s seq %d o" % (dtype, n), o[n].float().cpu().numpy(), outs[n], TOL[dtype])
        check("strong decay %s seq %d S" % (dtype, n), Sg[n], states[n], TOL[dtype])


def test_decode_multi_equals_repeated_decode_steps():
    N, T, H, D = 4, 16, 2, 128
    x, S0 = multi_inputs(N, T, H, D, "bf16", seed=50)
    bf = torch.bfloat16
    S1 = dev(S0)
    o1 = kda.decode_multi(dev(x["q"], bf), dev(x["k"], bf), dev(x["v"], bf), dev(x["g"]), dev(x["beta"]), S1)
    S2 = dev(S0)
    o2 = []
    for t in range(T):
        o2.append(kda.decode_step(dev(x["q"][:, t], bf), dev(x["k"][:, t], bf), dev(x["v"][:, t], bf),
                                  dev(x["g"][:, t]), dev(x["beta"][:, t]), S2))
    torch.cuda.synchronize()
    check("multi vs steps S", S1.cpu().numpy(), S2.cpu().numpy(), 1e-5)
    check("multi vs steps o", o1.float().cpu().numpy(), torch.stack(o2, 1).float().cpu().numpy(), 1e-2)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("case", ["uniform", "mixed_channels", "near_limit"])
def test_prefill_decays_beyond_a_chunk_span(dtype, D, case):
    """Decays summing far below -88 over a 64-token chunk, on both prefill
    paths: every factor the kernels form spans at most 16 tokens, so the
    result stays finite and matches the oracle (1e-2 for bf16, 1e-4 for fp32).
    near_limit: g in [-4.9, -3], close to the documented domain (the sum over
    16 tokens above -80)."""
    d = kda_inputs.prefill_inputs(1, B=1, H=2, T=300, D=D, dtype=dtype, seed=12)
    rng = np.random.Generator(np.random.PCG64(13))
    lo, hi = (-4.9, -3.0) if case == "near_limit" else (-4.5, -2.0)
    strong = rng.uniform(lo, hi, size=d["g"].shape).astype(np.float32)
    if case != "mixed_channels":
        d["g"] = strong
    else:  # fast-forgetting channels beside slow ones
        d["g"] = np.where(np.arange(D) % 3 == 0, strong, d["g"]).astype(np.float32)
    o, S_T, _ = gpu_prefill(d, ckpt_every=64)
    assert np.isfinite(o).all() and np.isfinite(S_T).all()
    compare_prefill(d, ckpt_every=64, label="strong decay %s %s D=%d" % (case, dtype, D))



# -- segmented prefill ----------------------------------------------------------

def test_prefill_segments_equal_one_pass_long():
    """kda_prefill runs the long workload in segments whose records stay
    within 232 MiB (the state carried between them); the result
    equals one pass of the two stages over all tokens, bitwise, checkpoints
    included (their interval does not align with the segments)."""
    d = kda_inputs.prefill_inputs(2)
    dt = torch.bfloat16
    q, k, v = dev(d["q"], dt), dev(d["k"], dt), dev(d["v"], dt)
    g, b = dev(d["g"]), dev(d["beta"])
    T = q.shape[1]
    assert 1024 <= kda.segment_tokens(q, v) < T
    o1, S1, c1 = kda.prefill(q, k, v, g, b, checkpoint_every=4096)
    ws = kda.workspace(q, v)
    kda.prefill_chunk_prep(q, k, v, g, b, ws)
    o2, S2, c2 = kda.prefill_chunk_recur(ws, q, v, checkpoint_every=4096)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(c1, c2)


def test_prefill_many_heads_short_segments_equal_one_pass():
    """16 sequences of 1000 tokens, 32 heads each, from nonzero states: the
    records of 512 heads allow 384-token segments (three, the last 232 tokens
    long), and the recurrence runs 4096 workgroups, more than fit at once.
    Equal to one pass of the two stages, bitwise, checkpoints every 256 tokens
    across the segment boundaries included; sampled heads against the oracle."""
    d = kda_inputs.prefill_inputs(1, B=16, T=1000, H=32, seed=71)
    dt = torch.bfloat16
    q, k, v = dev(d["q"], dt), dev(d["k"], dt), dev(d["v"], dt)
    g, b, S0 = dev(d["g"]), dev(d["beta"]), dev(d["S0"])
    assert kda.segment_tokens(q, v) == 384
    o1, S1, c1 = kda.prefill(q, k, v, g, b, S0, checkpoint_every=256)
    ws = kda.workspace(q, v)
    kda.prefill_chunk_prep(q, k, v, g, b, ws)
    o2, S2, c2 = kda.prefill_chunk_recur(ws, q, v, S0=S0, checkpoint_every=256)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(c1, c2)
    seqs, heads = [0, 15], [0, 31]
    sub = {x: np.ascontiguousarray(d[x][seqs][:, :, heads]) for x in ("q", "k", "v", "g", "beta")}
    o_ref, S_ref, ck_ref = oracle.prefill(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"],
                                          np.ascontiguousarray(d["S0"][seqs][:, heads]), ckpt_every=256)
    check("short segments o", o1.float().cpu().numpy()[seqs][:, :, heads], o_ref, TOL["bf16"])
    check("short segments S_T", S1.cpu().numpy()[seqs][:, heads], S_ref, TOL["bf16"])
    check("short segments ckpt", c1.cpu().numpy()[:, seqs][:, :, heads], ck_ref, TOL["bf16"])


@pytest.mark.parametrize("D", [128, 64])
def test_segment_stages_equal_one_pass(D):
    """The segment entry points over [0,128) [128,192) [192,300), from a nonzero
    S0 with checkpoints every 64 tokens, equal one pass over all 300 tokens."""
    d = kda_inputs.prefill_inputs(1, B=2, T=300, H=2, D=D, s0_std=0.01)
    dt = torch.bfloat16
    q, k, v = dev(d["q"], dt), dev(d["k"], dt), dev(d["v"], dt)
    g, b, S0 = dev(d["g"]), dev(d["beta"]), dev(d["S0"])
    ws = kda.workspace(q, v)
    kda.prefill_chunk_prep(q, k, v, g, b, ws)
    o_ref, S_ref, c_ref = kda.prefill_chunk_recur(ws, q, v, S0=S0, checkpoint_every=64)
    wseg = kda.workspace(q, v, 128)
    o = torch.full_like(o_ref, float("nan"))
    S_T = torch.empty_like(S_ref)
    ck = torch.full_like(c_ref, float("nan"))
    S_prev = S0
    for t0, tl in ((0, 128), (128, 64), (192, 108)):
        kda.prefill_segment_prep(q, k, v, g, b, t0, tl, wseg)
        kda.prefill_segment_recur(wseg, q, v, t0, tl, S0=S_prev, checkpoint_every=64, o=o, S_T=S_T, ckpt=ck)
        S_prev = S_T
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S_T, S_ref) and torch.equal(ck, c_ref)
