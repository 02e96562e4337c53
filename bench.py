"""Benchmark: KDA prefill tokens/s and decode us/step on one MI355X.

A step is one kda_prefill call over the long-prefill workload (B=1, H=32,
T=32768, dk=dv=128, chunk 64, bf16 q/k/v, fp32 g/beta/state) with inputs
resident in HBM.  The decode workload (64 sequences x 32 heads, 444 one-token
steps from a seeded fp32 state) is timed in the same run and reported beside
it.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0   # MI355X dense bf16 MFMA
C = 64

PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "kda_prefill_long_traffic.json")
KERNEL_SOURCES = ["kda_device.h", "kda_prefill.hip", "kda_decode.hip"]


def prefill_flops_per_token_head(D: int, C: int = C) -> int:
    """Per-chunk count 12C^3 + 8C^2 D + 6 C D^2 of the primer's FlashKDA
    analysis (bayesiansapien wiki page, section 2), divided by C."""
    return 12 * C * C + 8 * C * D + 6 * D * D


def prefill_min_bytes(B, T, H, D, elem_bytes, s0: bool, n_ckpt: int) -> int:
    """Compulsory HBM bytes of one prefill call: q, k, v read and o written
    once in the input dtype, g (fp32, per channel) and beta (fp32) read once,
    the states read/written once."""
    per_token_head = 3 * D * elem_bytes + 4 * D + 4 + D * elem_bytes
    state = 4 * D * D
    return B * T * H * per_token_head + B * H * state * (1 + n_ckpt + (1 if s0 else 0))


def kernel_sources_sha() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "kimi_delta_attention_chunked_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per prefill launch from committed rocprofv3 counters, or None
    when the counters are missing or were taken on different kernel sources."""
    try:
        with open(PREFILL_COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_sha") != kernel_sources_sha():
        return None
    return c.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the KDA path here is single-GPU (heads and "
              "sequences shard across GPUs with no communication); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import kda_inputs
    import kimi_delta_attention_chunked_amd as kda

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- prefill, long workload ----
    d = kda_inputs.prefill_inputs(2)
    B, T, H, D = d["B"], d["T"], d["H"], d["D"]
    t = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    q, k, v = (t(d[x], torch.bfloat16) for x in ("q", "k", "v"))
    g, beta = t(d["g"]), t(d["beta"])
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
    S_T = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        kda.prefill(q, k, v, g, beta, None, o=o, S_T=S_T)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        kda.prefill(q, k, v, g, beta, None, o=o, S_T=S_T)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    tok_s = B * T / (ms_per_step * 1e-3)

    flops = prefill_flops_per_token_head(D) * B * T * H
    min_bytes = prefill_min_bytes(B, T, H, D, 2, s0=False, n_ckpt=0)
    t_s = ms_per_step * 1e-3
    achieved_gbs = min_bytes / t_s / 1e9
    tflops = flops / t_s / 1e12
    traffic = measured_traffic()

    result = {
        "metric": "KDA prefill tokens/s @H=32,D=128,T=32K (+% MFMA peak); decode us/step",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised, v~N(0,1), beta=sigmoid(N(0,1)), "
                "g~U(-0.05,-0.0005))",
        "config": {"workload": "KDA chunked prefill, long: B=1, H=32, T=32768, dk=dv=128, "
                               "C=64, bf16 q/k/v/o, fp32 g/beta/state, S0=0",
                   "B": B, "T": T, "H": H, "dk": D, "dv": D, "chunk": C,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "kda_prefill_kernel<OpBF16, InBF16, 128>",
                     "algorithmic_bytes_per_launch": min_bytes},
        "prefill_tflops": round(tflops, 2),
        "prefill_mfma_frac": round(tflops / MFMA_BF16_PEAK_TFS, 4),
        "prefill_flops_per_launch": flops,
        "wall_s_timed": round(wall, 3),
    }

    # ---- decode, 444 steps of 64 x 32 heads ----
    if not args.no_decode:
        dd = kda_inputs.decode_inputs(4)
        steps = dd["steps"]
        N, Hd, Dd = dd["N"], dd["H"], dd["D"]
        dq, dk_, dv_ = (t(dd[x], torch.bfloat16) for x in ("q", "k", "v"))
        dg, db = t(dd["g"]), t(dd["beta"])
        S0 = t(dd["S0"])
        S = S0.clone()
        od = torch.empty((steps, N, Hd, Dd), dtype=torch.bfloat16, device=dev)
        for s in range(min(steps, 20)):  # warm-up
            kda.decode_step(dq[s], dk_[s], dv_[s], dg[s], db[s], S, o=od[s])
        S.copy_(S0)
        torch.cuda.synchronize()
        ev0.record(stream)
        for s in range(steps):
            kda.decode_step(dq[s], dk_[s], dv_[s], dg[s], db[s], S, o=od[s])
        ev1.record(stream)
        torch.cuda.synchronize()
        us_step = ev0.elapsed_time(ev1) * 1e3 / steps
        state_bytes = 8 * Dd * Dd * N * Hd
        io_bytes = N * Hd * (3 * Dd * 2 + 4 * Dd + 4 + Dd * 2)
        gbs = (state_bytes + io_bytes) / (us_step * 1e-6) / 1e9
        result["decode"] = {
            "workload": "KDA decode: N=64 sequences, H=32, dk=dv=128, 444 steps, bf16 q/k/v/o, "
                        "fp32 g/beta/state",
            "us_per_step": round(us_step, 3),
            "tokens_per_s": round(N / (us_step * 1e-6), 1),
            "state_gbs": round(gbs, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "kernel": "kda_decode_kernel<InBF16, 128>",
                         "algorithmic_bytes_per_launch": state_bytes + io_bytes},
            "note": "the 128 MiB state can be served partly by the 256 MB Infinity Cache",
        }

    # ---- CPU baseline: the fp64 oracle on the same prefill inputs ----
    if not args.no_cpu:
        import oracle
        threads = oracle.default_threads()
        heads = list(range(H))
        T_s = T
        sl = lambda a: np.ascontiguousarray(a[:, :T_s])
        c0 = time.perf_counter()
        o_ref, S_ref, _ = oracle.prefill(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]),
                                         sl(d["beta"]), None, threads=threads)
        cpu_s = time.perf_counter() - c0
        o_gpu = o.float().cpu().numpy()
        err_o = float(np.linalg.norm(o_gpu - o_ref) / np.linalg.norm(o_ref))
        err_s = float(np.linalg.norm(S_T.cpu().numpy() - S_ref) / np.linalg.norm(S_ref))
        result["cpu_baseline"] = {
            "value": round(B * T_s / cpu_s, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": "the whole long-prefill workload (B=1, T=%d, all %d heads), fp64 "
                      "token-by-token recurrence, OpenMP over heads; %.1f s" % (T_s, len(heads),
                                                                              cpu_s)}
        result["parity_vs_oracle"] = {"o_rel_err": err_o, "S_T_rel_err": err_s, "bound": 1e-2}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
