"""Benchmark: KDA prefill tokens/s and decode us/step on one MI355X.

A step is one bf16 chunked prefill over the long workload (B=1, H=32,
T=32768, dk=dv=128, chunk 64, bf16 q/k/v/o, fp32 g/beta/state, S0 = 0) with
every input resident in HBM: the chunk-preparation kernel, then the
chunk-recurrence kernel over each segment of kda_prefill's schedule, launched
through the segment entry points of the C ABI (together exactly kda_prefill).
In each timed step HIP events on the launch stream bracket the two launches of
one segment, cycling through the segments from step to step, so the
per-kernel average launch durations are measured live at a cost of three
events per step.  Beside
it, the same tokens cut into 16 prompts of mixed length run through the packed
prefill (kda_prefill_varlen), and the decode workload (64 sequences x 32 heads,
444 one-token steps from a seeded fp32 state) is timed in the same run, and
so is the layer core on the long workload (kda_prefill_layer: short causal
convolution, L2 norm and gates fused into the chunk preparation, then the
output norm/gate pass) with its one-token decode; then the fp64 CPU oracle runs
on the long prefill's inputs as the CPU baseline.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-varlen] [--no-decode] [--no-cpu] [--no-layer]

Counter support (HBM traffic and MFMA use of each kernel):

    rocprofv3 --pmc FETCH_SIZE -f csv -d DIR1 -o run -- python3 bench.py --counters-run
    rocprofv3 --pmc WRITE_SIZE -f csv -d DIR2 -o run -- python3 bench.py --counters-run
    python bench.py --write-traffic DIR1/run_counter_collection.csv DIR2/run_counter_collection.csv
    rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 SQ_INSTS_VALU_MFMA_BF16 GRBM_GUI_ACTIVE -f csv -d DIR3 -o run -- python3 bench.py --counters-run
    python bench.py --write-mfma DIR3/run_counter_collection.csv

--counters-run does 2 prefill steps, one 1 GiB device-to-device copy (the
plain copy kernel that calibrates the traffic counters) and 3 decode steps;
--write-traffic turns the two traffic files into
profiles/kda_prefill_long_traffic.json, which later runs report as
roofline.traffic (and decode.traffic), and --write-mfma turns the MFMA file
into profiles/kda_prefill_long_mfma.json, reported as mfma_counters, both
while the kernel sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0   # MI355X dense bf16 MFMA
C = 64
COPY_BYTES = 1 << 30          # calibration copy: 1 GiB read, 1 GiB written

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kda_prefill_long_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "kda_prefill_long_mfma.json")
# The files that define the kernels and their launch geometry (segment rule,
# grid sizes): a change to any of them invalidates the committed counters.
KERNEL_SOURCES = ["kda_device.h", "kda_prefill.hip", "kda_decode.hip", "kda_api.hip", "kda_launch.h",
                  "kda_layer.hip"]
PREP_KERNEL = "kda_chunk_prep"
RECUR_KERNEL = "kda_chunk_recur"
DECODE_KERNEL = "kda_decode_kernel"
COPY_KERNEL = "copyBuffer"
FAMILIES = (PREP_KERNEL, RECUR_KERNEL, DECODE_KERNEL, COPY_KERNEL)

# Bytes of one operand record (per batch, head and 64-token chunk) at dk = 128.
RECORD_BYTES = {128: 72704, 64: 39936}


def prefill_flops_per_token_head(D: int, C: int = C) -> int:
    """Per-chunk count 12C^3 + 8C^2 D + 6 C D^2 of the primer's FlashKDA
    analysis (bayesiansapien wiki page, section 2), divided by C."""
    return 12 * C * C + 8 * C * D + 6 * D * D


def pages_bytes_per_chunk(D: int, C: int = C) -> int:
    """Bytes a two-kernel chunked step moves per chunk and head by the primer's
    count for FlashKDA (bayesiansapien wiki page, section 2): 8C^2 + 22CD, its
    preparation kernel's intermediates included."""
    return 8 * C * C + 22 * C * D


def prefill_min_bytes(B, T, H, D, elem_bytes, s0: bool, n_ckpt: int) -> int:
    """Compulsory HBM bytes of one prefill call: q, k, v read and o written
    once in the input dtype, g (fp32, per channel) and beta (fp32) read once,
    the states read/written once."""
    per_token_head = 3 * D * elem_bytes + 4 * D + 4 + D * elem_bytes
    state = 4 * D * D
    return B * T * H * per_token_head + B * H * state * (1 + n_ckpt + (1 if s0 else 0))


def kernel_traffic_bytes(B, T, H, D, segs):
    """Bytes each kernel moves per step in this design, records included: the
    preparation reads q, k, v (bf16), g and beta once and writes one record per
    chunk; the recurrence reads every record once, writes o (bf16), and writes
    the state after each segment (reading it back at the next).  The records
    are this implementation's own hand-over, not algorithmic bytes: the
    roofline of the step uses prefill_min_bytes."""
    n = sum((tl + C - 1) // C for _, tl in segs)
    rec = B * H * n * RECORD_BYTES[D]
    tok = B * T * H
    prep = tok * (3 * D * 2 + 4 * D + 4) + rec
    recur = rec + tok * D * 2 + B * H * D * D * 4 * (2 * len(segs) - 1)
    return {PREP_KERNEL: prep, RECUR_KERNEL: recur}


def kernel_sources_sha() -> str:
    """Hash of the kernel sources' code: comments and whitespace are left out,
    so that an edit of the explanations alone keeps the counters valid."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "kimi_delta_attention_chunked_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def committed_counters(path):
    """Per-kernel figures from a committed counter file, or None when it is
    missing or was taken on different kernel sources."""
    try:
        with open(path) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_sha") != kernel_sources_sha():
        return None
    return c.get("kernels")


def measured_traffic():
    """Per-kernel HBM bytes per launch (see committed_counters)."""
    return committed_counters(TRAFFIC_FILE)


def _counter_means(path, counter):
    """Average counter value per dispatch of each kernel family in a rocprofv3
    counter_collection.csv (KiB for the traffic counters).  For the copy
    family, the largest dispatch: the 1 GiB calibration copy, not torch's
    small copies around it."""
    vals = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            fam = next((k for k in FAMILIES if k in name), None)
            if fam is not None:
                vals.setdefault(fam, []).append(float(row["Counter_Value"]))
    return {k: (max(v) if k == COPY_KERNEL else sum(v) / len(v)) for k, v in vals.items()}


def write_traffic(fetch_csv, write_csv):
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    # The calibration copy moves COPY_BYTES each way; scale each counter so it
    # reads exactly that for the copy.
    f_scale = COPY_BYTES / (fetch[COPY_KERNEL] * 1024.0)
    w_scale = COPY_BYTES / (write[COPY_KERNEL] * 1024.0)
    out = {"kernel_sha": kernel_sources_sha(),
           "workload": "long prefill, B=1 H=32 T=32768 dk=dv=128 bf16",
           "fetch_scale": f_scale, "write_scale": w_scale,
           "raw_kib_per_dispatch": {"FETCH_SIZE": fetch, "WRITE_SIZE": write},
           "kernels": {}}
    for k in (PREP_KERNEL, RECUR_KERNEL, DECODE_KERNEL):
        if k not in fetch or k not in write:
            continue
        rd = fetch[k] * 1024.0 * f_scale
        wr = write[k] * 1024.0 * w_scale
        out["kernels"][k] = {"read_bytes": round(rd), "write_bytes": round(wr),
                             "hbm_bytes": round(rd + wr)}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


class HipEvent:
    """A HIP timing event on one stream, created with hipEventDisableSystemFence:
    recording it then issues no system-scope release, which would otherwise add
    about 2 us to every bracketed launch (nothing here reads device memory from
    the host at an event).  Uses the HIP runtime torch has loaded."""
    _hip = None

    def __init__(self, stream):
        import ctypes
        if HipEvent._hip is None:
            with open("/proc/self/maps") as f:
                path = next(l.split()[-1] for l in f if "libamdhip64" in l)
            HipEvent._hip = ctypes.CDLL(path)
        self._ct = ctypes
        self.h = ctypes.c_void_p()
        self.s = ctypes.c_void_p(stream.cuda_stream)
        self._check(HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.h), 0x20000000))

    @staticmethod
    def _check(rc):
        if rc != 0:
            raise RuntimeError("HIP event call failed: %d" % rc)

    def record(self):
        self._check(HipEvent._hip.hipEventRecord(self.h, self.s))

    def elapsed_ms(self, later) -> float:
        f = self._ct.c_float()
        self._check(HipEvent._hip.hipEventElapsedTime(self._ct.byref(f), self.h, later.h))
        return f.value

    def __del__(self):
        if HipEvent._hip is not None and self.h:
            HipEvent._hip.hipEventDestroy(self.h)


def write_mfma(csv_path):
    """Per-dispatch averages of the MFMA counters of each prefill kernel:
    MfmaUtil (percent of the SIMDs' cycles with the MFMA unit busy while the
    kernel runs), MfmaFlopsBF16 (bf16 MFMA FLOPs), SQ_INSTS_VALU_MFMA_BF16
    (MFMA instructions) and GRBM_GUI_ACTIVE (GPU-active cycles)."""
    names = ("MfmaUtil", "MfmaFlopsBF16", "SQ_INSTS_VALU_MFMA_BF16", "GRBM_GUI_ACTIVE")
    out = {"kernel_sha": kernel_sources_sha(),
           "workload": "long prefill, B=1 H=32 T=32768 dk=dv=128 bf16, per segment launch",
           "kernels": {}}
    for k in (PREP_KERNEL, RECUR_KERNEL):
        out["kernels"][k] = {}
    for n in names:
        for k, v in _counter_means(csv_path, n).items():
            if k in out["kernels"]:
                out["kernels"][k][n] = v
    with open(MFMA_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def time_region(fn, reps, stream):
    """Milliseconds per call of fn, from HIP events on the launch stream around
    reps back-to-back calls."""
    import torch
    torch.cuda.synchronize()
    e0, e1 = HipEvent(stream), HipEvent(stream)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_ms(e1) / reps


def rel_err(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


# Heads the oracle checks on the bench's larger workloads (each (batch, head)
# chain is an independent recurrence).
CONFIG_HEADS = {1: None, 3: [3, 28]}


def config_line(torch, kda, cid, args, stream):
    """One prefill workload of the inputs recipe: kda_prefill timed per call
    (HIP events on the launch stream), the compulsory-bytes roofline, the
    pages' FLOP count, one pass through the segment entry points with events
    around every launch (per-kernel times; the recurrence's launches that
    store checkpoints apart), and parity against the oracle on sampled heads."""
    import kda_inputs
    import oracle
    dev = torch.device("cuda:0")
    d = kda_inputs.prefill_inputs(cid)
    B, T, H, D = d["B"], d["T"], d["H"], d["D"]
    N = d["ckpt_every"]
    t = lambda a, dt=torch.float32: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    q, k, v = (t(d[x], torch.bfloat16) for x in ("q", "k", "v"))
    g, beta, S0 = t(d["g"]), t(d["beta"]), t(d["S0"])
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
    S_T = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    n_ck = -(-T // N) if N else 0
    ck = torch.empty((n_ck, B, H, D, D), dtype=torch.float32, device=dev) if n_ck else None
    ws = kda.prefill_workspace(q, v)

    def call():
        kda.prefill(q, k, v, g, beta, S0=S0, checkpoint_every=N, o=o, S_T=S_T, ckpt=ck, ws=ws)

    reps = max(2, args.steps // (4 if T > 100000 else 1))
    for _ in range(max(1, args.warmup // 2)):
        call()
    ms = time_region(call, reps, stream)
    o_keep, S_keep = o.clone(), S_T.clone()
    ck_keep = None if ck is None else ck.clone()

    # Per-kernel times: one pass through the segment entry points, events
    # around every launch.
    L = kda.segment_tokens(q, v)
    segs = [(t0, min(L, T - t0)) for t0 in range(0, T, L)]
    wss = kda.workspace(q, v, L)
    ev = [HipEvent(stream) for _ in range(2 * len(segs) + 1)]
    passes = 3
    prep_us = np.zeros(len(segs))
    recur_us = np.zeros(len(segs))
    for p in range(passes + 1):  # the first pass warms up, the others are averaged
        torch.cuda.synchronize()
        ev[0].record()
        for i, (t0, tl) in enumerate(segs):
            kda.prefill_segment_prep(q, k, v, g, beta, t0, tl, wss)
            ev[2 * i + 1].record()
            kda.prefill_segment_recur(wss, q, v, t0, tl, S0=S0 if t0 == 0 else S_T, checkpoint_every=N,
                                      o=o, S_T=S_T, ckpt=ck)
            ev[2 * i + 2].record()
        torch.cuda.synchronize()
        if p:
            prep_us += [1e3 * ev[2 * i].elapsed_ms(ev[2 * i + 1]) / passes for i in range(len(segs))]
            recur_us += [1e3 * ev[2 * i + 1].elapsed_ms(ev[2 * i + 2]) / passes for i in range(len(segs))]
    with_ck = [i for i, (t0, tl) in enumerate(segs) if N and ((t0 + tl) // N > t0 // N or t0 + tl == T)]
    bitwise = bool(torch.equal(o, o_keep) and torch.equal(S_T, S_keep)
                   and (ck is None or torch.equal(ck, ck_keep)))

    flops = prefill_flops_per_token_head(D) * B * T * H
    mb = prefill_min_bytes(B, T, H, D, 2, s0=S0 is not None, n_ckpt=n_ck)
    line = {
        "workload": "KDA chunked prefill, %s: B=%d, H=%d, T=%d, dk=dv=%d, C=64, bf16 q/k/v/o, fp32 "
                    "g/beta/state, S0 %s, checkpoints %s" % (d["name"], B, H, T, D,
                                                             "~N(0,0.01)" if S0 is not None else "= 0",
                                                             "every %d tokens (%d)" % (N, n_ck) if N else "none"),
        "entry_point": "kda_prefill", "calls_timed": reps, "ms_per_step": round(ms, 4),
        "tokens_per_s": round(B * T / (ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "algorithmic_bytes_per_step": mb,
                     "achieved": round(mb / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(mb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "prefill_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "prefill_mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
        "segments": len(segs), "segment_tokens": L,
        "kernels_us_per_pass": {PREP_KERNEL: round(float(sum(prep_us)), 1),
                                RECUR_KERNEL: round(float(sum(recur_us)), 1),
                                "passes": passes, "note": "segment entry points, events around every launch"},
        "segment_entry_points_bitwise_equal_to_call": bitwise,
    }
    if N:
        wo = [recur_us[i] for i in range(len(segs)) if i not in with_ck]
        line["recur_us_per_segment"] = {
            "with_checkpoint": round(float(np.mean([recur_us[i] for i in with_ck])), 2),
            "without": round(float(np.mean(wo)), 2) if wo else None,
            "segments_with_checkpoint": len(with_ck)}
    # Parity on the sampled heads.
    heads = CONFIG_HEADS[cid]
    sl = (lambda a: a) if heads is None else (lambda a: np.ascontiguousarray(a[:, :, heads]))
    s0r = None if d["S0"] is None else (d["S0"] if heads is None else np.ascontiguousarray(d["S0"][:, heads]))
    c0 = time.perf_counter()
    o_ref, S_ref, ck_ref = oracle.prefill(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]), sl(d["beta"]), s0r,
                                          ckpt_every=N, threads=oracle.default_threads())
    cpu_s = time.perf_counter() - c0
    hs = np.s_[:] if heads is None else heads
    par = {"heads": "all" if heads is None else heads, "bound": 1e-2,
           "o_rel_err": rel_err(o_keep.float().cpu().numpy()[:, :, hs], o_ref),
           "S_T_rel_err": rel_err(S_keep.cpu().numpy()[:, hs], S_ref), "oracle_s": round(cpu_s, 2)}
    if N:
        cg = ck_keep.cpu().numpy()
        par["ckpt_rel_err_max"] = max(rel_err(cg[j][:, hs], ck_ref[j]) for j in range(n_ck))
    line["parity_vs_oracle"] = par
    del q, k, v, g, beta, S0, o, S_T, ck, ws, wss, o_keep, S_keep, ck_keep
    return line


def prefill_workload(torch, dev):
    import kda_inputs
    d = kda_inputs.prefill_inputs(2)
    t = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    q, k, v = (t(d[x], torch.bfloat16) for x in ("q", "k", "v"))
    return d, q, k, v, t(d["g"]), t(d["beta"])


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-varlen", action="store_true", help="skip the packed-prompts prefill")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the mid and agentic prefill workloads")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the layer-core lines (short convolution, L2 norm, gates, output norm/gate)")
    ap.add_argument("--counters-run", action="store_true",
                    help="2 prefill steps and the 1 GiB calibration copy, for rocprofv3 --pmc")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--write-mfma", metavar="MFMA_CSV")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.write_mfma:
        write_mfma(args.write_mfma)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the KDA path here is single-GPU (heads and "
              "sequences shard across GPUs with no communication); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import kimi_delta_attention_chunked_amd as kda

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- prefill, long workload ----
    d, q, k, v, g, beta = prefill_workload(torch, dev)
    B, T, H, D = d["B"], d["T"], d["H"], d["D"]
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
    S_T = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    # kda_prefill's schedule: segments of L tokens through one workspace, the
    # state carried in S_T (run through the segment entry points so that each
    # kernel launch can be bracketed by events).
    L = kda.segment_tokens(q, v)
    segs = [(t0, min(L, T - t0)) for t0 in range(0, T, L)]
    ws = kda.workspace(q, v, L)

    def step():
        for t0, tl in segs:
            kda.prefill_segment_prep(q, k, v, g, beta, t0, tl, ws)
            kda.prefill_segment_recur(ws, q, v, t0, tl, S0=None if t0 == 0 else S_T, o=o, S_T=S_T)

    if args.counters_run:
        for _ in range(2):
            step()
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        del src, dst
        import kda_inputs
        dd = kda_inputs.decode_inputs(4, steps=3)
        td = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
        Sd = td(dd["S0"])
        for j in range(3):
            kda.decode_step(td(dd["q"][j], torch.bfloat16), td(dd["k"][j], torch.bfloat16),
                            td(dd["v"][j], torch.bfloat16), td(dd["g"][j]), td(dd["beta"][j]), Sd)
        torch.cuda.synchronize()
        print("counters run done", flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()   # the stream the library launches on
    ns = len(segs)
    # Timed step j brackets the launches of segment j % ns with three events.
    mark = [[HipEvent(stream) for _ in range(3)] for _ in range(args.steps)]
    e_start, e_end = HipEvent(stream), HipEvent(stream)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e_start.record()
    for j in range(args.steps):
        sj = j % ns
        for i, (t0, tl) in enumerate(segs):
            if i == sj:
                mark[j][0].record()
            kda.prefill_segment_prep(q, k, v, g, beta, t0, tl, ws)
            if i == sj:
                mark[j][1].record()
            kda.prefill_segment_recur(ws, q, v, t0, tl, S0=None if t0 == 0 else S_T, o=o, S_T=S_T)
            if i == sj:
                mark[j][2].record()
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = e_start.elapsed_ms(e_end) / args.steps
    # Per segment, the mean of its sampled launches; per launch, the mean over
    # the sampled segments; per step, the sum over all segments (each segment's
    # own mean once every segment has been sampled).
    samples = {}
    for j in range(args.steps):
        samples.setdefault(j % ns, []).append((mark[j][0].elapsed_ms(mark[j][1]), mark[j][1].elapsed_ms(mark[j][2])))
    seg_mean = {i: np.mean(np.array(x), axis=0) for i, x in samples.items()}
    per_launch = np.mean(np.array(list(seg_mean.values())), axis=0)
    per_step = (np.sum(np.array(list(seg_mean.values())), axis=0) if len(seg_mean) == ns
                else per_launch * ns)
    launch_us = {PREP_KERNEL: 1e3 * per_launch[0], RECUR_KERNEL: 1e3 * per_launch[1]}
    kernel_us = {PREP_KERNEL: 1e3 * per_step[0], RECUR_KERNEL: 1e3 * per_step[1]}
    tok_s = B * T / (ms_per_step * 1e-3)

    flops = prefill_flops_per_token_head(D) * B * T * H
    min_bytes = prefill_min_bytes(B, T, H, D, 2, s0=False, n_ckpt=0)
    t_s = ms_per_step * 1e-3
    tflops = flops / t_s / 1e12
    ktraffic = kernel_traffic_bytes(B, T, H, D, segs)
    dom = max(kernel_us, key=kernel_us.get)
    traffic = measured_traffic()
    kernels = {}
    for name, us in kernel_us.items():
        gbs = ktraffic[name] / (us * 1e-6) / 1e9
        kernels[name] = {"avg_us": round(launch_us[name], 2), "launches_per_step": ns, "us_per_step": round(us, 2),
                         "timed_launches": args.steps, "segments_sampled": len(seg_mean),
                         "design_bytes_per_launch": ktraffic[name] // ns,
                         "design_gbs": round(gbs, 1),
                         "counter_bytes_per_launch": None if traffic is None else traffic[name]["hbm_bytes"],
                         "note": "design bytes include the per-chunk operand records this implementation "
                                 "hands from one kernel to the other; they are not algorithmic bytes"}
    # Counter bytes of the whole step: each kernel's calibrated L2<->memory
    # bytes per launch times its launches per step.
    step_traffic = None if traffic is None else sum(traffic[n]["hbm_bytes"] * ns for n in kernel_us)
    achieved = min_bytes / t_s / 1e9
    pages_bytes = B * H * ((T + C - 1) // C) * pages_bytes_per_chunk(D)

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
                   "B": B, "T": T, "H": H, "dk": D, "dv": D, "chunk": C, "segment_tokens": L},
        # The step's compulsory bytes (1540 B per token-head: q, k, v, o in
        # bf16, g and beta in fp32, plus the final state) over the step time.
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": step_traffic,
                     "traffic_ratio": None if step_traffic is None else round(step_traffic / min_bytes, 3),
                     "kernel": "whole prefill step: %d x (%s + %s)" % (ns, PREP_KERNEL, RECUR_KERNEL),
                     "algorithmic_bytes_per_step": min_bytes, "avg_us": round(ms_per_step * 1e3, 2),
                     "dominant_kernel": dom, "dominant_kernel_avg_us": round(launch_us[dom], 2),
                     # Beside it: the primer's own byte count for a two-kernel step
                     # (intermediates included), over the same time.
                     "pages_traffic_model": {
                         "bytes_per_chunk_head": pages_bytes_per_chunk(D),
                         "bytes_per_step": pages_bytes,
                         "achieved": round(pages_bytes / t_s / 1e9, 1),
                         "frac": round(pages_bytes / t_s / 1e9 / HBM_PEAK_GBS, 4)}},
        "kernels": kernels,
        "mfma_counters": committed_counters(MFMA_FILE),
        "prefill_tflops": round(tflops, 2),
        "prefill_mfma_frac": round(tflops / MFMA_BF16_PEAK_TFS, 4),
        "prefill_flops_per_step": flops,
        "wall_s_timed": round(wall, 3),
    }

    # ---- the public call: one kda_prefill per step on the same inputs ----
    def call():
        kda.prefill(q, k, v, g, beta, o=o, S_T=S_T, ws=ws_call)

    ws_call = kda.prefill_workspace(q, v)
    for _ in range(args.warmup):
        call()
    cms = time_region(call, args.steps, stream)
    result["prefill_call"] = {
        "entry_point": "kda_prefill", "ms_per_step": round(cms, 4),
        "tokens_per_s": round(B * T / (cms * 1e-3), 1),
        "hbm_min_frac": round(min_bytes / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "vs_segment_entry_points_ms": round(ms_per_step, 4)}
    del ws_call

    if not args.no_configs:
        # (the long workload's tensors stay resident: 288 GB of HBM holds both)
        result["configs"] = {}
        for cid, name in ((1, "mid"), (3, "agentic")):
            result["configs"][name] = config_line(torch, kda, cid, args, stream)
            torch.cuda.empty_cache()

    # ---- packed prompts: the same 32768 tokens cut into 16 prompts of mixed length ----
    if not args.no_varlen:
        import kda_inputs
        lens, cu = kda_inputs.packed_lengths()
        pq, pk, pv = (x.reshape(T, H, D) for x in (q, k, v))
        pg, pb = g.reshape(T, H, D), beta.reshape(T, H)
        po = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
        pS = torch.empty((len(lens), H, D, D), dtype=torch.float32, device=dev)
        for _ in range(args.warmup):
            kda.prefill_varlen(pq, pk, pv, pg, pb, cu, o=po, S_T=pS)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            kda.prefill_varlen(pq, pk, pv, pg, pb, cu, o=po, S_T=pS)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        result["varlen"] = {
            "workload": "KDA packed prefill: 16 prompts of seeded log-uniform lengths in [256, 8192] "
                        "summing to 32768 tokens (longest %d), H=32, dk=dv=128, bf16, S0=0" % max(lens),
            "ms_per_step": round(ms, 4),
            "tokens_per_s": round(T / (ms * 1e-3), 1),
            "note": "the recurrence of each prompt is serial, so the longest prompt sets its time",
        }

    # ---- the layer core on the long workload: convolution, L2 norm and gates
    # fused into the chunk preparation, then the output norm/gate pass ----
    if not args.no_layer:
        import kda_inputs
        ld = kda_inputs.layer_inputs(2, W=4)
        lt = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
        lq, lk, lv, lz = (lt(ld[x], torch.bfloat16) for x in ("q", "k", "v", "z"))
        la_, lb_, lw, lnw = lt(ld["a"]), lt(ld["b"]), lt(ld["conv_w"]), lt(ld["norm_w"])
        del ld
        lo = torch.empty_like(lq)
        lS = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
        lcs = torch.empty((B, H, 3 * D, 3), dtype=torch.float32, device=dev)

        def layer_step():
            kda.prefill_layer(lq, lk, lv, la_, lb_, conv_w=lw, silu=True, z=lz, norm_w=lnw, o=lo, S_T=lS,
                              conv_state_out=lcs, ws=ws)

        for _ in range(args.warmup):
            layer_step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            layer_step()
        e1.record(stream)
        torch.cuda.synchronize()
        lms = e0.elapsed_time(e1) / args.steps
        # the output step alone (in place, as the layer runs it)
        e0.record(stream)
        for _ in range(args.steps):
            kda.output_norm_gate(lo, lz, norm_w=lnw, y=lo)
        e1.record(stream)
        torch.cuda.synchronize()
        ong_us = e0.elapsed_time(e1) * 1e3 / args.steps
        ong_bytes = B * T * H * D * 2 * 3
        ong_gbs = ong_bytes / (ong_us * 1e-6) / 1e9
        result["layer"] = {
            "workload": "KDA layer core, long: B=1, H=32, T=32768, dk=dv=128, bf16; raw q/k/v through a "
                        "width-4 causal convolution with SiLU, L2 norm of q/k, alpha=sigmoid(a), "
                        "beta=sigmoid(b), output RMS norm under a sigmoid output gate",
            "ms_per_step": round(lms, 4),
            "tokens_per_s": round(B * T / (lms * 1e-3), 1),
            "vs_core_prefill_ms": round(ms_per_step, 4),
            "output_norm_gate": {"avg_us": round(ong_us, 2), "algorithmic_bytes_per_launch": ong_bytes,
                                 "achieved_gbs": round(ong_gbs, 1), "frac": round(ong_gbs / HBM_PEAK_GBS, 4)},
        }
        del lq, lk, lv, lz, la_, lb_, lo, lS, lcs

    # ---- decode, 444 steps of 64 x 32 heads ----
    if not args.no_decode:
        import kda_inputs
        dd = kda_inputs.decode_inputs(4)
        t = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
        steps = dd["steps"]
        N, Hd, Dd = dd["N"], dd["H"], dd["D"]
        dq, dk2, dv2 = (t(dd[x], torch.bfloat16) for x in ("q", "k", "v"))
        dg, db = t(dd["g"]), t(dd["beta"])
        S0 = t(dd["S0"])
        S = S0.clone()
        od = torch.empty((steps, N, Hd, Dd), dtype=torch.bfloat16, device=dev)
        for s in range(min(steps, 20)):  # warm-up
            kda.decode_step(dq[s], dk2[s], dv2[s], dg[s], db[s], S, o=od[s])
        S.copy_(S0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(steps):
            kda.decode_step(dq[s], dk2[s], dv2[s], dg[s], db[s], S, o=od[s])
        e1.record(stream)
        torch.cuda.synchronize()
        us_step = e0.elapsed_time(e1) * 1e3 / steps
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
                         "kernel": "kda_decode_kernel", "avg_us": round(us_step, 3),
                         "algorithmic_bytes_per_launch": state_bytes + io_bytes,
                         "traffic": (traffic or {}).get(DECODE_KERNEL, {}).get("hbm_bytes")},
            "note": "cache-assisted: the 128 MiB state fits the 256 MB Infinity Cache, so part of the "
                    "stream can be served from it; decode.past_cache is the HBM-bound line",
        }

        # The same decode with 256 sequences: a 512 MiB state, twice the
        # Infinity Cache, so the state stream is HBM traffic.  Beside it, the
        # same bytes moved by a plain device copy (512 MiB read + 512 MiB
        # written) and by an in-place elementwise update of a 512 MiB buffer,
        # as the practical roofs.
        NB, SB = 256, 50
        db_ = kda_inputs.decode_inputs(4, N=NB, steps=SB)
        bq, bk, bv = (t(db_[x], torch.bfloat16) for x in ("q", "k", "v"))
        bg, bb, bS = t(db_["g"]), t(db_["beta"]), t(db_["S0"])
        del db_
        bo = torch.empty((NB, Hd, Dd), dtype=torch.bfloat16, device=dev)
        for s in range(5):
            kda.decode_step(bq[s], bk[s], bv[s], bg[s], bb[s], bS, o=bo)
        it = iter(range(10**9))

        def big_step():
            s = next(it) % SB
            kda.decode_step(bq[s], bk[s], bv[s], bg[s], bb[s], bS, o=bo)

        bus = 1e3 * time_region(big_step, SB, stream)
        b_state = 8 * Dd * Dd * NB * Hd
        b_io = NB * Hd * (3 * Dd * 2 + 4 * Dd + 4 + Dd * 2)
        bgbs = (b_state + b_io) / (bus * 1e-6) / 1e9
        src = torch.empty(b_state // 2, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        dst.copy_(src)
        cus = 1e3 * time_region(lambda: dst.copy_(src), 20, stream)
        xbuf = torch.ones(b_state // 8, dtype=torch.float32, device=dev)
        xbuf.mul_(1.0)
        ius = 1e3 * time_region(lambda: xbuf.mul_(1.0), 20, stream)
        copy_gbs = b_state / (cus * 1e-6) / 1e9
        inplace_gbs = b_state / (ius * 1e-6) / 1e9
        result["decode"]["past_cache"] = {
            "workload": "KDA decode: N=256 sequences, H=32, dk=dv=128, %d steps, bf16 q/k/v/o, fp32 "
                        "g/beta/state (512 MiB state, twice the 256 MB Infinity Cache)" % SB,
            "us_per_step": round(bus, 3),
            "tokens_per_s": round(NB / (bus * 1e-6), 1),
            "roofline": {"bound": "hbm", "achieved": round(bgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(bgbs / HBM_PEAK_GBS, 4), "kernel": "kda_decode_kernel",
                         "avg_us": round(bus, 3), "algorithmic_bytes_per_launch": b_state + b_io},
            "copy_roof": {"what": "device copy of 512 MiB (read + write)", "us": round(cus, 2),
                          "gbs": round(copy_gbs, 1)},
            "inplace_roof": {"what": "in-place elementwise update of a 512 MiB fp32 buffer", "us": round(ius, 2),
                             "gbs": round(inplace_gbs, 1)},
            "frac_of_inplace_roof": round(bgbs / inplace_gbs, 4),
        }
        del bq, bk, bv, bg, bb, bS, bo, src, dst, xbuf

        # The same 444 launches captured once in a HIP graph and replayed
        # (the state reset eagerly before each replay), checked bitwise
        # against the launch loop above.
        S_loop, o_loop = S.clone(), od.clone()
        S.copy_(S0)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for s in range(steps):
                kda.decode_step(dq[s], dk2[s], dv2[s], dg[s], db[s], S, o=od[s])
        gus = []
        equal = True
        for _ in range(3):
            S.copy_(S0)
            od.zero_()
            torch.cuda.synchronize()
            e0.record(stream)
            graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            gus.append(e0.elapsed_time(e1) * 1e3 / steps)
            equal = equal and torch.equal(S, S_loop) and torch.equal(od, o_loop)
        del graph
        result["decode"]["graph"] = {"us_per_step": round(float(np.median(gus)), 3),
                                     "replays": len(gus), "bitwise_equal_to_loop": bool(equal)}

        # ---- speculative decoding: verify 8 drafts, commit the accepted ones ----
        TS = 8
        tq = lambda a: a[:TS].transpose(0, 1).contiguous()  # [T,N,...] -> [N,T,...]
        sq_, sk_, sv_, sg_, sb_ = (tq(x) for x in (dq, dk2, dv2, dg, db))
        acc = torch.from_numpy(np.random.Generator(np.random.PCG64(3000)).integers(0, TS + 1, N)
                               .astype(np.int32)).to(dev)
        so = torch.empty((N, TS, Hd, Dd), dtype=torch.bfloat16, device=dev)
        S.copy_(S0)
        for _ in range(args.warmup):
            kda.decode_multi(sq_, sk_, sv_, sg_, sb_, S, update_state=False, o=so)
        torch.cuda.synchronize()
        ev3 = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        vs, cs = [], []
        for _ in range(args.steps):
            S.copy_(S0)
            ev3[0].record(stream)
            kda.decode_multi(sq_, sk_, sv_, sg_, sb_, S, update_state=False, o=so)
            ev3[1].record(stream)
            kda.decode_multi(sq_, sk_, sv_, sg_, sb_, S, n_tokens=acc, want_output=False)
            ev3[2].record(stream)
            torch.cuda.synchronize()
            vs.append(ev3[0].elapsed_time(ev3[1]) * 1e3)
            cs.append(ev3[1].elapsed_time(ev3[2]) * 1e3)
        v_us, c_us = float(np.mean(vs)), float(np.mean(cs))
        result["decode"]["speculative"] = {
            "workload": "verify 8 draft tokens per sequence (outputs, state untouched), then commit "
                        "a seeded accepted count in [0, 8] per sequence; N=64, H=32, dk=dv=128, bf16",
            "verify_us": round(v_us, 3),
            "commit_us": round(c_us, 3),
            "mean_accepted": round(float(acc.float().mean()), 3),
            "vs_8_decode_steps_us": round(TS * us_step, 3),
        }

        if not args.no_layer:
            # one decode token of the layer core (convolution state, norms, gates, output gate)
            rr = np.random.Generator(np.random.PCG64(3001))
            da = torch.from_numpy(rr.uniform(3.0, 7.6, (N, Hd, Dd)).astype(np.float32)).to(dev)
            dbl = torch.from_numpy(rr.standard_normal((N, Hd)).astype(np.float32)).to(dev)
            dz = torch.from_numpy(rr.standard_normal((N, Hd, Dd)).astype(np.float32)).to(dev, torch.bfloat16)
            dw = torch.from_numpy((rr.standard_normal((Hd, 4, 3 * Dd)) * 0.5).astype(np.float32)).to(dev)
            dcs = torch.zeros((N, Hd, 3 * Dd, 3), dtype=torch.float32, device=dev)
            dol = torch.empty((N, Hd, Dd), dtype=torch.bfloat16, device=dev)
            S.copy_(S0)
            nls = min(steps, 100)
            for s_ in range(args.warmup):
                kda.decode_layer_step(dq[s_], dk2[s_], dv2[s_], da, dbl, S, conv_state=dcs, conv_w=dw,
                                      silu=True, z=dz, o=dol)
            torch.cuda.synchronize()
            e0.record(stream)
            for s_ in range(nls):
                kda.decode_layer_step(dq[s_], dk2[s_], dv2[s_], da, dbl, S, conv_state=dcs, conv_w=dw,
                                      silu=True, z=dz, o=dol)
            e1.record(stream)
            torch.cuda.synchronize()
            result["decode"]["layer_step"] = {
                "workload": "one token of the layer core per sequence: width-4 convolution state, L2 "
                            "norms, sigmoid gates, output norm/gate; N=64, H=32, dk=dv=128, bf16",
                "us_per_step": round(e0.elapsed_time(e1) * 1e3 / nls, 3),
                "vs_decode_step_us": round(us_step, 3),
            }

    # ---- CPU baseline: the fp64 oracle on the same prefill inputs ----
    if not args.no_cpu:
        import oracle
        threads = oracle.default_threads()
        c0 = time.perf_counter()
        o_ref, S_ref, _ = oracle.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], None,
                                         threads=threads)
        cpu_s = time.perf_counter() - c0
        o_gpu = o.float().cpu().numpy()
        err_o = float(np.linalg.norm(o_gpu - o_ref) / np.linalg.norm(o_ref))
        err_s = float(np.linalg.norm(S_T.cpu().numpy() - S_ref) / np.linalg.norm(S_ref))
        result["cpu_baseline"] = {
            "value": round(B * T / cpu_s, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": "the whole long-prefill workload (B=1, T=%d, all %d heads), fp64 "
                      "token-by-token recurrence, OpenMP over heads; %.1f s" % (T, H, cpu_s)}
        # One thread on one head of the same inputs, scaled to the whole layer.
        one = {x: np.ascontiguousarray(d[x][:, :, :1]) for x in ("q", "k", "v", "g", "beta")}
        c0 = time.perf_counter()
        oracle.prefill(one["q"], one["k"], one["v"], one["g"], one["beta"], None, threads=1)
        one_s = time.perf_counter() - c0
        result["cpu_baseline"]["single_thread"] = {
            "value": round(B * T / (one_s * H), 1), "unit": "tokens/s", "cores": 1,
            "sample": "head 0 of the same inputs (T=%d) on one thread, %.2f s, scaled by %d heads"
                      % (T, one_s, H)}
        result["parity_vs_oracle"] = {"o_rel_err": err_o, "S_T_rel_err": err_s, "bound": 1e-2}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
