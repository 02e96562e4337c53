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
exactly the same numbers.

RNG: numpy SeedSequence(1000 + config id) by default (or the given seed)
spawns one child per tensor, in the order q, k, v, beta-logits, g, S0 (decode:
S0, q, k, v, beta-logits, g).  Each tensor is filled in fixed blocks of 2^20
elements; block i draws from PCG64 seeded with the i-th child of that tensor's
seed sequence.  Blocks are generated on worker threads, and the values do not
depend on the thread count.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

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


BLOCK = 1 << 20  # elements per independently seeded block (a multiple of D)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw(shape, seq: np.random.SeedSequence, kind: str, D: int = 1, dtype: str = "fp32",
          lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    """Fill a float32 array block by block.  kind: 'normal', 'unit' (normal
    rows L2-normalised over the last axis of length D), 'uniform' (U(lo, hi))."""
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    nblk = -(-flat.size // BLOCK)
    kids = seq.spawn(nblk)

    def work(i):
        sl = flat[i * BLOCK:(i + 1) * BLOCK]
        gen = np.random.Generator(np.random.PCG64(kids[i]))
        if kind == "uniform":
            gen.random(out=sl, dtype=np.float32)
            sl *= np.float32(hi - lo)
            sl += np.float32(lo)
            return
        gen.standard_normal(out=sl, dtype=np.float32)
        if kind == "unit":
            rows = sl.reshape(-1, D)
            n = np.sqrt(np.sum(rows * rows, axis=-1, keepdims=True, dtype=np.float32))
            rows /= n
        if dtype == "bf16":
            sl[:] = round_bf16(sl)

    if nblk == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nblk)))
    return out


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
    root = np.random.SeedSequence(1000 + config if seed is None else seed)
    sq, sk, sv, sb, sg, ss = root.spawn(6)
    B, H, T, D, dt = c["B"], c["H"], c["T"], c["D"], c["dtype"]
    shape = (B, T, H, D)
    lo, hi = c["g_range"]
    q = _draw(shape, sq, "unit", D, dt)
    k = _draw(shape, sk, "unit", D, dt)
    v = _draw(shape, sv, "normal", D, dt)
    beta = _sigmoid(_draw((B, T, H), sb, "normal"))
    g = _draw(shape, sg, "uniform", lo=lo, hi=hi)
    S0 = None
    if c["s0_std"]:
        S0 = _draw((B, H, D, D), ss, "normal") * np.float32(c["s0_std"])
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
    root = np.random.SeedSequence(1000 + config if seed is None else seed)
    ss, sq, sk, sv, sb, sg = root.spawn(6)
    N, H, D, steps, dt = c["N"], c["H"], c["D"], c["steps"], c["dtype"]
    lo, hi = c["g_range"]
    S0 = _draw((N, H, D, D), ss, "normal") * np.float32(c["s0_std"])
    shape = (steps, N, H, D)
    q = _draw(shape, sq, "unit", D, dt)
    k = _draw(shape, sk, "unit", D, dt)
    v = _draw(shape, sv, "normal", D, dt)
    beta = _sigmoid(_draw((steps, N, H), sb, "normal"))
    g = _draw(shape, sg, "uniform", lo=lo, hi=hi)
    c.update(q=q, k=k, v=v, g=g, beta=beta, S0=S0)
    return c


def layer_inputs(config: int = 2, seed: int | None = None, W: int = 4, **override) -> dict:
    """Inputs of the layer core (raw q, k, v before the short convolution and
    the L2 norm; gate logits instead of g and beta).

    Distributions: q, k, v ~ N(0,1) (bf16-rounded when the config is bf16);
    decay-gate logits a ~ U(3.0, 7.6) per key channel; write-gate logits
    b ~ N(0,1); output-gate logits z ~ N(0,1) (bf16-rounded); convolution taps
    conv_w [H, W, 3D] ~ N(0, 1/W) (standard deviation 1/sqrt(W)); output-norm
    weight norm_w [D] = 1 + N(0, 0.1); a carried convolution state conv_state
    [B, H, 3D, W-1] ~ N(0,1) (bf16-rounded), for tests that continue a
    sequence; S0 as the config.  RNG: SeedSequence(5000 + config) (or seed)
    spawns q, k, v, b, a, S0, z, conv_w, norm_w, conv_state in that order.
    """
    c = dict(CONFIGS[config])
    assert c["kind"] == "prefill"
    c.update(override)
    root = np.random.SeedSequence(5000 + config if seed is None else seed)
    sq, sk, sv, sb, sa, ss, sz, sw, sn, sc = root.spawn(10)
    B, H, T, D, dt = c["B"], c["H"], c["T"], c["D"], c["dtype"]
    shape = (B, T, H, D)
    q = _draw(shape, sq, "normal", D, dt)
    k = _draw(shape, sk, "normal", D, dt)
    v = _draw(shape, sv, "normal", D, dt)
    b = _draw((B, T, H), sb, "normal")
    a = _draw(shape, sa, "uniform", lo=3.0, hi=7.6)
    S0 = None
    if c["s0_std"]:
        S0 = _draw((B, H, D, D), ss, "normal") * np.float32(c["s0_std"])
    z = _draw(shape, sz, "normal", D, dt)
    conv_w = _draw((H, W, 3 * D), sw, "normal") * np.float32(1.0 / np.sqrt(W))
    norm_w = np.float32(1.0) + _draw((D,), sn, "normal") * np.float32(0.1)
    conv_state = _draw((B, H, 3 * D, max(W - 1, 0)), sc, "normal", 1, dt) if W > 1 else None
    c.update(q=q, k=k, v=v, a=a, b=b, S0=S0, z=z, conv_w=conv_w, norm_w=norm_w, conv_state=conv_state, W=W)
    return c


def packed_lengths(n: int = 16, total: int = 32768, lo: int = 256, hi: int = 8192, seed: int = 2000):
    """Lengths of n prompts packed into one prefill of `total` tokens: drawn
    log-uniformly in [lo, hi] (numpy PCG64 seeded with `seed`), scaled to sum
    to `total`, floored, the remainder added to the last prompt.  Returns the
    lengths and the offsets cu_seqlens [n + 1]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    raw = np.exp(rng.uniform(np.log(lo), np.log(hi), size=n))
    lens = np.floor(raw / raw.sum() * total).astype(np.int64)
    lens[-1] += total - int(lens.sum())
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return [int(x) for x in lens], [int(x) for x in cu]



def huge_prefill_inputs(T: int = 600_037, H: int = 32, D: int = 128, tail: int = 3000,
                        seed: int = 77, s0_std: float = 0.02, device: str = "cuda:0") -> dict:
    """Device tensors of one bf16 prefill (B = 1) large enough that q, k, v, g
    and o each hold more than 2^31 elements at the default sizes.

    Tokens [0, T - tail) carry k = 0 and g = 0, so they neither decay nor
    write the state; q, v and beta are drawn there as usual.  The last `tail`
    tokens follow the long workload's distributions (q, k L2-normalised
    N(0,1) rows, v ~ N(0,1), beta = sigmoid(N(0,1)), g ~ U(-0.05, -0.0005)).
    S0 ~ N(0, s0_std).  q, k, v are rounded to bf16 (nearest even) from fp32.

    RNG: a torch.Generator on `device` seeded with `seed`, drawing q, v,
    beta-logits, the tail's k, the tail's g, then S0.  Returns torch tensors
    on `device`: q, k, v [1,T,H,D] bf16, g [1,T,H,D] and beta [1,T,H] fp32,
    S0 [1,H,D,D] fp32, and the sizes.
    """
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def unit_rows(n):
        x = torch.randn((1, n, H, D), generator=gen, device=device, dtype=torch.float32)
        x /= torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        return x.to(torch.bfloat16)

    q = unit_rows(T)
    v = torch.randn((1, T, H, D), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    beta = torch.sigmoid(torch.randn((1, T, H), generator=gen, device=device, dtype=torch.float32))
    k = torch.zeros((1, T, H, D), device=device, dtype=torch.bfloat16)
    k[:, T - tail:] = unit_rows(tail)
    g = torch.zeros((1, T, H, D), device=device, dtype=torch.float32)
    lo, hi = CONFIGS[2]["g_range"]
    g[:, T - tail:] = torch.rand((1, tail, H, D), generator=gen, device=device,
                                 dtype=torch.float32) * (hi - lo) + lo
    S0 = torch.randn((1, H, D, D), generator=gen, device=device, dtype=torch.float32) * s0_std
    return dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0, T=T, H=H, D=D, tail=tail)
