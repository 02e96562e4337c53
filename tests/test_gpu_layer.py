"""Parity of the layer entry points (kda_prefill_layer, kda_decode_layer_step,
kda_output_norm_gate; the short convolution, L2 norm, gates and output
norm/gate of the primer's section 3) with the fp64 oracle in oracle/layer.py.

Error metric and bounds as in test_gpu_parity.py: Frobenius-relative error per
tensor, 1e-2 for bf16 q/k/v, 1e-4 for fp32.  Convolution states hold raw
inputs and are compared exactly.  The oracle takes the taps as [H, 2dk+dv, W];
the library takes [H, W, 2dk+dv]."""
import numpy as np
import pytest
import torch

import kda_inputs
import kimi_delta_attention_chunked_amd as kda
import oracle.layer as layer_oracle

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


def taps_for_oracle(conv_w):
    return None if conv_w is None else np.ascontiguousarray(np.transpose(conv_w, (0, 2, 1)))


def run_prefill_layer(d, W, silu, use_state, use_z, ckpt_every=0, heads=None, S0=None, conv_state=None):
    dt = DT[d["dtype"]]
    conv_w = d["conv_w"] if W > 0 else None
    cs = conv_state if conv_state is not None else (d["conv_state"] if (use_state and W > 1) else None)
    S0 = d["S0"] if S0 is None else S0
    o, S_T, ck, cs_out = kda.prefill_layer(
        dev(d["q"], dt), dev(d["k"], dt), dev(d["v"], dt), dev(d["a"]), dev(d["b"]),
        conv_w=dev(conv_w), conv_state=dev(cs), silu=silu, S0=dev(S0), checkpoint_every=ckpt_every,
        z=dev(d["z"], dt) if use_z else None, norm_w=dev(d["norm_w"]) if use_z else None, eps=1e-6)
    torch.cuda.synchronize()
    return (o.float().cpu().numpy(), S_T.cpu().numpy(), None if ck is None else ck.cpu().numpy(),
            None if cs_out is None else cs_out.cpu().numpy(), cs)


def oracle_prefill_layer(d, W, silu, cs, use_z, ckpt_every=0, heads=None, S0=None):
    hs = np.s_[:] if heads is None else heads
    S0 = d["S0"] if S0 is None else S0
    return layer_oracle.prefill_layer(
        d["q"][:, :, hs], d["k"][:, :, hs], d["v"][:, :, hs], d["a"][:, :, hs], d["b"][:, :, hs],
        conv_w=taps_for_oracle(d["conv_w"][hs]) if W > 0 else None,
        conv_state=None if cs is None else cs[:, hs], silu=silu,
        S0=None if S0 is None else S0[:, hs], ckpt_every=ckpt_every,
        z=d["z"][:, :, hs] if use_z else None, norm_w=d["norm_w"] if use_z else None, eps=1e-6)


# (D, W, silu, carried conv state, output gate, checkpoint interval)
CASES = [
    (128, 4, True, True, True, 64),
    (128, 3, False, False, False, 0),
    (128, 0, False, False, True, 0),
    (128, 2, True, False, False, 128),
    (64, 4, True, True, True, 0),
    (64, 1, False, False, True, 64),
]


@pytest.mark.parametrize("D,W,silu,use_state,use_z,ck", CASES,
                         ids=["D%d-W%d-silu%d-state%d-z%d-ck%d" % c for c in CASES])
def test_prefill_layer_matches_oracle(D, W, silu, use_state, use_z, ck):
    d = kda_inputs.layer_inputs(1, W=max(W, 1), B=2, T=200, H=2, D=D, s0_std=0.01)
    tol = TOL["bf16"]
    o, S_T, cko, cs_out, cs = run_prefill_layer(d, W, silu, use_state, use_z, ck)
    o_ref, S_ref, ck_ref, cs_ref = oracle_prefill_layer(d, W, silu, cs, use_z, ck)
    label = "layer D%d W%d" % (D, W)
    check(label + " o", o, o_ref, tol)
    check(label + " S_T", S_T, S_ref, tol)
    if ck:
        assert cko.shape[0] == ck_ref.shape[0]
        for j in range(ck_ref.shape[0]):
            check(label + " ckpt[%d]" % j, cko[j], ck_ref[j], tol)
    if W > 1:
        np.testing.assert_array_equal(cs_out, cs_ref)
    else:
        assert cs_out is None


def test_prefill_layer_continues_a_sequence():
    """Two calls carrying S and the convolution state = one call over the whole
    sequence (checked against the oracle of the whole sequence)."""
    d = kda_inputs.layer_inputs(1, W=4, B=1, T=300, H=2, D=128, s0_std=0.01)
    dt = DT["bf16"]
    T1 = 130  # not a chunk multiple: the second call's chunks start mid-way
    parts = []
    S, cs = dev(d["S0"]), dev(d["conv_state"])
    for lo, hi in ((0, T1), (T1, 300)):
        o, S, _, cs = kda.prefill_layer(dev(d["q"][:, lo:hi], dt), dev(d["k"][:, lo:hi], dt),
                                        dev(d["v"][:, lo:hi], dt), dev(d["a"][:, lo:hi]),
                                        dev(d["b"][:, lo:hi]), conv_w=dev(d["conv_w"]), conv_state=cs,
                                        silu=True, S0=S, z=dev(d["z"][:, lo:hi], dt),
                                        norm_w=dev(d["norm_w"]))
        parts.append(o.float().cpu().numpy())
    torch.cuda.synchronize()
    o_ref, S_ref, _, cs_ref = oracle_prefill_layer(d, 4, True, d["conv_state"], True)
    check("split o", np.concatenate(parts, axis=1), o_ref, TOL["bf16"])
    check("split S_T", S.cpu().numpy(), S_ref, TOL["bf16"])
    np.testing.assert_array_equal(cs.cpu().numpy(), cs_ref)


def test_prefill_layer_empty_sequence():
    d = kda_inputs.layer_inputs(1, W=3, B=2, T=0, H=2, D=64, s0_std=0.01)
    o, S_T, _, cs_out, cs = run_prefill_layer(d, 3, True, True, True)
    assert o.shape == (2, 0, 2, 64)
    np.testing.assert_array_equal(S_T, d["S0"])
    np.testing.assert_array_equal(cs_out, cs)
    # without a carried state the state after no tokens is zeros
    o, S_T, _, cs_out, _ = run_prefill_layer(d, 3, True, False, False)
    assert np.all(cs_out == 0.0)


def test_prefill_layer_long_sampled_heads():
    """The long workload (B=1, H=32, T=32768, D=128) with a width-4 convolution,
    SiLU and the output gate, as the benchmark runs it; two heads checked."""
    d = kda_inputs.layer_inputs(2, W=4)
    heads = [0, 21]
    o, S_T, _, cs_out, _ = run_prefill_layer(d, 4, True, False, True)
    o_ref, S_ref, _, cs_ref = oracle_prefill_layer(d, 4, True, None, True, heads=heads)
    check("long layer o (heads 0, 21)", o[:, :, heads], o_ref, TOL["bf16"])
    check("long layer S_T (heads 0, 21)", S_T[:, heads], S_ref, TOL["bf16"])
    np.testing.assert_array_equal(cs_out[:, heads], cs_ref)


def test_prefill_layer_segments_two_sequences_sampled_heads():
    """Two sequences of 4096 tokens, 32 heads: the layer runs in two
    segments (the convolution halos and the state carried across segment
    boundaries in both sequences); checked on two heads."""
    d = kda_inputs.layer_inputs(1, W=4, B=2, T=4096, H=32, D=128, s0_std=0.01)
    q = dev(d["q"], torch.bfloat16)
    assert kda.segment_tokens(q, q) < 4096
    heads = [5, 30]
    o, S_T, _, cs_out, cs = run_prefill_layer(d, 4, True, True, True)
    o_ref, S_ref, _, cs_ref = oracle_prefill_layer(d, 4, True, cs, True, heads=heads)
    check("2-sequence segmented layer o (heads 5, 30)", o[:, :, heads], o_ref, TOL["bf16"])
    check("2-sequence segmented layer S_T (heads 5, 30)", S_T[:, heads], S_ref, TOL["bf16"])
    np.testing.assert_array_equal(cs_out[:, heads], cs_ref)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("full", [True, False], ids=["conv-gate", "plain"])
def test_decode_layer_matches_oracle(dtype, D, full):
    """Token-by-token layer decode = the oracle's layer over those tokens."""
    W = 4 if full else 1
    d = kda_inputs.layer_inputs(1, W=W, B=5, T=6, H=3, D=D, dtype=dtype, s0_std=0.02)
    dt = DT[dtype]
    tol = TOL[dtype]
    S = dev(d["S0"])
    cs = dev(d["conv_state"]) if full else None
    outs = []
    for t in range(d["T"]):
        o = kda.decode_layer_step(dev(d["q"][:, t], dt), dev(d["k"][:, t], dt), dev(d["v"][:, t], dt),
                                  dev(d["a"][:, t]), dev(d["b"][:, t]), S, conv_state=cs,
                                  conv_w=dev(d["conv_w"]) if full else None, silu=full,
                                  z=dev(d["z"][:, t], dt) if full else None,
                                  norm_w=dev(d["norm_w"]) if full else None, eps=1e-6)
        outs.append(o.float().cpu().numpy())
    torch.cuda.synchronize()
    o_ref, S_ref, _, cs_ref = layer_oracle.prefill_layer(
        d["q"], d["k"], d["v"], d["a"], d["b"], conv_w=taps_for_oracle(d["conv_w"]) if full else None,
        conv_state=d["conv_state"] if full else None, silu=full, S0=d["S0"],
        z=d["z"] if full else None, norm_w=d["norm_w"] if full else None, eps=1e-6)
    check("decode layer o", np.stack(outs, axis=1), o_ref, tol)
    check("decode layer S", S.cpu().numpy(), S_ref, tol)
    if full:
        np.testing.assert_array_equal(cs.cpu().numpy(), cs_ref)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("dv", [128, 64])
@pytest.mark.parametrize("weighted", [True, False])
@pytest.mark.parametrize("inplace", [True, False])
def test_output_norm_gate_matches_oracle(dtype, dv, weighted, inplace):
    r = np.random.default_rng(77)
    rows = 1001  # not a multiple of the rows a wave covers per step
    dt = DT[dtype]
    o_np = kda_inputs.round_bf16(r.standard_normal((rows, dv)).astype(np.float32) * 3.0)
    z_np = kda_inputs.round_bf16(r.standard_normal((rows, dv)).astype(np.float32))
    w_np = (1.0 + 0.1 * r.standard_normal(dv)).astype(np.float32) if weighted else None
    o = dev(o_np, dt)
    y = kda.output_norm_gate(o, dev(z_np, dt), norm_w=dev(w_np), eps=1e-5, y=o if inplace else None)
    torch.cuda.synchronize()
    ref = layer_oracle.output_norm_gate(o_np, z_np, w_np, 1e-5)
    check("norm/gate %s dv%d" % (dtype, dv), y.float().cpu().numpy(), ref, TOL[dtype])
