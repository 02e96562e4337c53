"""The seeded input generator: deterministic, right shapes and distributions."""
import numpy as np

import kda_inputs


def test_prefill_inputs_deterministic_and_shaped():
    a = kda_inputs.prefill_inputs(1, B=2, H=3, T=100)
    b = kda_inputs.prefill_inputs(1, B=2, H=3, T=100)
    for key in ("q", "k", "v", "g", "beta", "S0"):
        assert np.array_equal(a[key], b[key]), key
    assert a["q"].shape == (2, 100, 3, 128) and a["beta"].shape == (2, 100, 3)
    assert a["S0"].shape == (2, 3, 128, 128)
    c = kda_inputs.prefill_inputs(1, seed=5, B=2, H=3, T=100)
    assert not np.array_equal(a["q"], c["q"])


def test_prefill_distributions():
    d = kda_inputs.prefill_inputs(2, T=4096, H=4)
    for key in ("q", "k", "v"):  # bf16-representable
        assert np.array_equal(kda_inputs.round_bf16(d[key]), d[key])
    n = np.linalg.norm(d["q"].astype(np.float64), axis=-1)
    assert np.abs(n - 1).max() < 4e-3  # unit rows up to bf16 rounding
    assert d["g"].min() >= -0.05 - 1e-7 and d["g"].max() <= -0.0005 + 1e-7
    assert 0 < d["beta"].min() and d["beta"].max() < 1
    assert abs(d["v"].std() - 1) < 0.01 and d["S0"] is None


def test_tiny_is_fp32_and_decode_shapes():
    d = kda_inputs.prefill_inputs(0)
    assert d["dtype"] == "fp32" and d["q"].shape == (1, 256, 2, 64)
    n = np.linalg.norm(d["k"].astype(np.float64), axis=-1)
    assert np.abs(n - 1).max() < 1e-6
    dd = kda_inputs.decode_inputs(4, N=3, H=2, steps=5)
    assert dd["S0"].shape == (3, 2, 128, 128) and dd["q"].shape == (5, 3, 2, 128)
    assert dd["beta"].shape == (5, 3, 2)
    assert abs(dd["S0"].std() - 0.02) < 1e-3


def test_round_bf16_ties_to_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], dtype=np.float32)
    r = kda_inputs.round_bf16(x)
    assert r.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0]


def test_packed_lengths_recipe():
    lens, cu = kda_inputs.packed_lengths()
    assert len(lens) == 16 and sum(lens) == 32768 and cu[0] == 0 and cu[-1] == 32768
    assert all(b - a == L for a, b, L in zip(cu, cu[1:], lens))
    assert min(lens) > 0 and len(set(lens)) > 8          # mixed lengths
    assert any(L % 64 for L in lens)                      # ragged last chunks
    assert kda_inputs.packed_lengths() == (lens, cu)     # seeded



def test_huge_prefill_inputs_recipe_on_cpu():
    # The maximum-size recipe at a small size on the CPU: deterministic, k = 0
    # and g = 0 before the tail, the long workload's distributions in it.
    import torch
    a = kda_inputs.huge_prefill_inputs(T=3000, H=2, D=64, tail=500, device="cpu")
    b = kda_inputs.huge_prefill_inputs(T=3000, H=2, D=64, tail=500, device="cpu")
    for key in ("q", "k", "v", "g", "beta", "S0"):
        assert torch.equal(a[key], b[key]), key
    assert a["q"].dtype == torch.bfloat16 and a["g"].dtype == torch.float32
    assert a["q"].shape == (1, 3000, 2, 64) and a["beta"].shape == (1, 3000, 2)
    assert a["S0"].shape == (1, 2, 64, 64)
    assert not a["k"][:, :2500].any() and not a["g"][:, :2500].any()
    tail_g = a["g"][:, 2500:]
    assert tail_g.min() >= -0.05 - 1e-7 and tail_g.max() <= -0.0005 + 1e-7
    n = torch.linalg.vector_norm(a["k"][:, 2500:].double(), dim=-1)
    assert (n - 1).abs().max() < 4e-3
    n = torch.linalg.vector_norm(a["q"].double(), dim=-1)
    assert (n - 1).abs().max() < 4e-3
