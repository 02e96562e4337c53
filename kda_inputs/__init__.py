"""Seeded synthetic inputs for KDA prefill and decode.

This module is shared by the tests, the smoke check and the benchmark.  It only
draws random numbers and shapes them the way the workloads are specified; it
holds none of the recurrence's arithmetic and imports neither the oracle nor
the HIP library.

Workloads (sizes from the Kimi K3 primer's serving section: a 142k-token median
prompt and a 444-token median answer per agentic turn; state checkpoints every
32K tokens from its prefix-cache section):

  0 tiny     B=1,  H=2,  T=256,    D=64,  fp32 everything
  1 mid      B=2,  H=16, T=4096,   D=128, bf16 q/k/v, S0 ~ N(0, 0.01)
  2 long     B=1,  H=32, T=32768,  D=128, bf16 q/k/v, g ~ U(-0.05, -0.0005)
  3 agentic  B=1,  H=32, T=142000, D=128, bf16 q/k/v, checkpoints every 32768
  4 decode   N=64, H=32, D=128, 444 steps, bf16 q/k/v, S0 ~ N(0, 0.02)

Distributions: q, k ~ N(0,1) then L2-normalised per token and head (in fp32),
v ~ N(0,1), beta = sigmoid(N(0,1)), g ~ U(lo, hi) per key channel (a natural-log
decay, alpha = exp(g)).  The second parameter of N(.,.) is a standard
deviation.  bf16 tensors are rounded to nearest-even from fp32; the arrays
returned here hold those rounded values as float32, so every consumer sees
exactly the same numbers.  RNG: numpy PCG64 seeded with 1000 + config id by
default; draw order q, k, v, beta-logits, g, S0 (decode: S0 first, then per
step q, k, v, beta-logits, g).
"""
from __future__ import annotations

import numpy as np

CONFIGS = {
    0: dict(name="tiny", kind="prefill", B=1, H=2, T=256, D=64, dtype="fp32",
            g_range=(-0.1, -0.001), s0_std=None, ckpt_every=0),
    1: dict(name="mid", kind="prefill", B=2, H=16, T=4096, D=128, dtype="bf16",
            g_range=(-0.1, -0.001), s0_std=0.01, ckpt_every=0),
    2: dict(name="long", kind="prefill", B=1, H=32, T=32768, D=128, dtype="bf16",
            g_range=(-0.05, -0.0005), s0_std=None, ckpt_every=0),
    3: dict(name="agentic", kind="prefill", B=1, H=32, T=142000, D=128, dtype="bf16",
            g_range=(-0.05, -0.0005), s0_std=None, ckpt_every=32768),
    4: dict(name="decode", kind="decode", N=64, H=32, D=128, steps=444, dtype="bf16",
            g_range=(-0.1, -0.001), s0_std=0.02),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def prefill_inputs(config: int = 0, seed: int | None = None, **override) -> dict:
    """Inputs for one prefill call.

    ``override`` may replace B, H, T, D, dtype, g_range, s0_std or ckpt_every
    to make smaller cases with the same distributions.  Returns a dict with
    q, k, g [B,T,H,D], v [B,T,H,D], beta [B,T,H] (float32), S0 [B,H,D,D] or
    None, and the metadata keys of the config.
    """
    c = dict(CONFIGS[config])
    assert c["kind"] == "prefill"
    c.update(override)
    rng = np.random.Generator(np.random.PCG64(1000 + config if seed is None else seed))
    B, H, T, D, dt = c["B"], c["H"], c["T"], c["D"], c["dtype"]
    shape = (B, T, H, D)
    q = _cast(_unit_rows(rng.standard_normal(shape, dtype=np.float32)), dt)
    k = _cast(_unit_rows(rng.standard_normal(shape, dtype=np.float32)), dt)
    v = _cast(rng.standard_normal(shape, dtype=np.float32), dt)
    beta = _sigmoid(rng.standard_normal((B, T, H), dtype=np.float32))
    lo, hi = c["g_range"]
    g = (np.float32(lo) + np.float32(hi - lo) * rng.random(shape, dtype=np.float32))
    S0 = None
    if c["s0_std"]:
        S0 = (rng.standard_normal((B, H, D, D), dtype=np.float32) * np.float32(c["s0_std"]))
    c.update(q=q, k=k, v=v, g=g, beta=beta, S0=S0)
    return c


def decode_inputs(config: int = 4, seed: int | None = None, **override) -> dict:
    """Inputs for ``steps`` sequential decode steps of N sequences.

    Returns S0 [N,H,D,D] float32 and per-step stacks q, k, g, v [steps,N,H,D]
    and beta [steps,N,H] (float32 arrays; q/k/v hold bf16-rounded values).
    """
    c = dict(CONFIGS[config])
    assert c["kind"] == "decode"
    c.update(override)
    rng = np.random.Generator(np.random.PCG64(1000 + config if seed is None else seed))
    N, H, D, steps, dt = c["N"], c["H"], c["D"], c["steps"], c["dtype"]
    S0 = rng.standard_normal((N, H, D, D), dtype=np.float32) * np.float32(c["s0_std"])
    shape = (steps, N, H, D)
    q = _cast(_unit_rows(rng.standard_normal(shape, dtype=np.float32)), dt)
    k = _cast(_unit_rows(rng.standard_normal(shape, dtype=np.float32)), dt)
    v = _cast(rng.standard_normal(shape, dtype=np.float32), dt)
    beta = _sigmoid(rng.standard_normal((steps, N, H), dtype=np.float32))
    lo, hi = c["g_range"]
    g = (np.float32(lo) + np.float32(hi - lo) * rng.random(shape, dtype=np.float32))
    c.update(q=q, k=k, v=v, g=g, beta=beta, S0=S0)
    return c
