#!/usr/bin/env python3
"""Benchmark of the KDA chunked forward (prefill) on one MI355X.

One step = one kda_chunk_fwd call (every kernel of the path) over one batch of seeded synthetic
inputs already resident in HBM.  Default workload: B=1, Nqk=Nv=3, S=8192, D=128, BNSD, strong
decay g = -5*sigmoid(N(0,1)), fp32 initial state N(0, 0.1^2) -- the 8K-token prefill the metric
is quoted on.  Prints one JSON line.

Timing: W untimed warm-up steps, then K steps bracketed by torch.cuda.synchronize() (the timed
region: `value`, `ms_per_step`); the input set rotates over enough copies that the step's
inputs exceed the 256 MB last-level cache, so the bytes really come from HBM.  The same K steps
then run again through kda_chunk_fwd_timed, whose kernels' own dispatches record HIP events at
each kernel's start and end on the launch stream: those give the per-kernel durations
(`stages_ms`; they agree with rocprofv3's kernel trace).  A third pass puts an event pair
around every call: `per_call_ms` (median, min, mean).

Roofline: `roofline` is the dominant kernel's: the call's algorithmic bytes (1,538 B per
token-head at Nqk = Nv plus the states; `path_bytes`) over that kernel's average duration,
against the 8 TB/s HBM peak; `traffic` is that kernel's HBM bytes per launch from the committed
rocprofv3 counter summary (profiles/), null when the kernel sources changed since; and
`traffic_ratio` the counter bytes of all launched kernels over the algorithmic bytes; `l2_read`
each kernel's L1-to-L2 read bytes per launch (from the same summary) and their rate, the bound
of the chunk walks (about 26 B per clock per compute unit).
`path_roofline` uses the whole step time.  `copy_ceiling` times a plain device copy of the
algorithmic bytes (the practical bandwidth of a transfer that size).  The CPU baseline times the
fp64 oracle on the host cores on the full workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
MALL_BYTES = 256 << 20     # last-level (Infinity) cache

METRIC = "KDA prefill tokens/s (all heads) at D=128, T=8K; % of MFMA/HBM roofline"


def head_dim(inp) -> int:
    return int(inp.q.shape[-1])


def gate_bytes(inp) -> int:
    """Bytes of g per token-head: D fp32 per-channel gates, one fp32 with the scalar gate, or
    D bf16 raw gates (activated in the kernel)."""
    if inp.raw_gate:
        return head_dim(inp) * 2
    return 4 if inp.scalar_gate else head_dim(inp) * 4


def path_bytes(inp) -> int:
    """Algorithmic bytes of one call: q,k (bf16) per q/k head, v (bf16), g (fp32), beta (bf16),
    out (bf16) per value head, plus one fp32 state read and one written per (sequence, head)."""
    t, d = inp.tokens, head_dim(inp)
    b = t * inp.n_qk * d * 2 * 2 + t * inp.n_v * (d * 2 + gate_bytes(inp) + 2 + d * 2)
    states = inp.batch * inp.n_v * d * d * 4
    gate_params = inp.n_v * (d + 1) * 4 if inp.raw_gate else 0   # dt_bias and A_log
    return b + states * ((inp.initial_state is not None) + 1) + gate_params


def shape_of(inp):
    from kimi_delta_attention_chunk_amd import make_shape
    d = head_dim(inp)
    return make_shape(inp.layout, inp.batch, inp.seq_len, inp.n_qk, inp.n_v, inp.scale,
                      inp.qk_l2norm, inp.beta_sigmoid, d, d, inp.scalar_gate,
                      raw_gate=inp.raw_gate)


def seg_p_of(inp) -> int:
    """Segments per sequence of the library's plan for this shape (kda_chunk_fwd_plan)."""
    from kimi_delta_attention_chunk_amd import kda_chunk_fwd_plan
    return kda_chunk_fwd_plan(shape_of(inp))[1]


def record_bytes(d: int) -> int:
    """Workspace record per (chunk, value head): W, Q' (bf16), K_dec, U (fp16), O_intra
    (bf16), gamma (fp32 per channel)."""
    return 64 * d * (2 + 2 + 2 + 2 + 2) + d * 4


def chunk_counts(inp, sp: int, seg1: bool = False):
    """(chunks in segment 0, chunks in later segments) over all sequences, per value head; with
    seg1, the chunks of segment 1 alone as a third entry."""
    first = later = one = 0
    for L in inp.lengths:
        nc = (L + 63) // 64
        n0 = min(-(-nc // sp), nc)
        first += n0
        later += nc - n0
        one += min(n0, nc - n0)
    return (first, later, one) if seg1 else (first, later)


def scan_bytes(inp) -> int:
    """Compulsory bytes of the one-level scan: the record of every (chunk, value head), the
    output, and the initial and final states."""
    if seg_p_of(inp) > 1:
        return 0
    d = head_dim(inp)
    chunks = sum((L + 63) // 64 for L in inp.lengths)
    out = inp.tokens * inp.n_v * d * 2
    states = inp.batch * inp.n_v * d * d * 4
    return (chunks * inp.n_v * record_bytes(d) + out
            + states * ((inp.initial_state is not None) + 1))


def intra_bytes(inp) -> int:
    """Compulsory bytes of the intra kernel: q,k,v,g,beta in, the per-chunk record out."""
    d = head_dim(inp)
    chunks = sum((L + 63) // 64 for L in inp.lengths)
    rd = inp.tokens * inp.n_v * (d * 2 * 3 + gate_bytes(inp) + 2)   # q,k re-read per value head
    return rd + chunks * inp.n_v * record_bytes(d)


def seg_bytes(inp) -> int:
    """Compulsory bytes of the segment pass: every record, the initial states, the final
    outputs of segment 0, O0 and R of the later segments' chunks (all bf16), the N (fp32)
    and P (fp16) matrices of every segment, and S_in(1) = N_0 in bf16."""
    sp = seg_p_of(inp)
    if sp == 1:
        return 0
    d = head_dim(inp)
    first, later = chunk_counts(inp, sp)
    states = inp.batch * inp.n_v * d * d * 4
    mats = inp.batch * inp.n_v * sp * d * d * (4 + 2)
    return (inp.n_v * ((first + later) * record_bytes(d) + first * 64 * d * 2
                       + later * 64 * d * 2 * 2)
            + states * (inp.initial_state is not None) + mats + inp.batch * inp.n_v * d * d * 2)


def combine_bytes(inp) -> int:
    """Compulsory bytes of the combine pass: N_0 and the N (fp32) and P (fp16) of segments
    1 .. seg_p-2 in, S_in of segments 2.. out (bf16) and S_in of the last segment out in fp32
    (for the final-state step of the completion pass); and the completion of segment 1's
    chunks: their O0 and R and S_in(1) in, their outputs out (all bf16)."""
    sp = seg_p_of(inp)
    if sp == 1:
        return 0
    d = head_dim(inp)
    m = inp.batch * inp.n_v * d * d * 4
    _, _, one = chunk_counts(inp, sp, seg1=True)
    return (m * (sp - 1) + m // 2 * (sp - 2) + m // 2 * (sp - 2) + m
            + inp.n_v * one * 64 * d * (2 * 2 + 2) + m // 2)


def out_bytes(inp) -> int:
    """Compulsory bytes of the completion pass: O0 and R of every chunk of segments 2.. and
    S_in of those segments in, the outputs out (all bf16); for the final state, S_in of the last
    segment and its N (fp32) and P (fp16) in and the state (fp32) out."""
    sp = seg_p_of(inp)
    if sp == 1:
        return 0
    d = head_dim(inp)
    _, later, one = chunk_counts(inp, sp, seg1=True)
    m = inp.batch * inp.n_v * d * d * 4
    return (inp.n_v * (later - one) * 64 * d * (2 * 2 + 2)
            + inp.batch * inp.n_v * (sp - 2) * d * d * 2 + 3 * m + m // 2)


KERNEL_BYTES = {"kda_intra_kernel": intra_bytes, "kda_seg_kernel": seg_bytes,
                "kda_combine_kernel": combine_bytes, "kda_out_kernel": out_bytes,
                "kda_scan_kernel": scan_bytes}


def source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("kda_kernels.hip", "kda_plan.cpp", "kda_plan.h"):
        h.update(open(os.path.join(ROOT, "kimi_delta_attention_chunk_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def counter_summary(workload: str):
    """The committed rocprofv3 counter summary of this workload (FETCH_SIZE and WRITE_SIZE per
    dispatch and the copy-kernel calibration), or None when there is none or the kernel sources
    changed since the counters were taken."""
    import re
    path = os.path.join(ROOT, "profiles", f"kda_kernels_{workload}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)```", open(path).read(), re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("source_hash") != source_hash():
        return None
    return d


def measured_traffic(summary, kernel: str):
    """HBM bytes per launch of `kernel` from a counter summary (scaled FETCH_SIZE + WRITE_SIZE)."""
    if summary is None or kernel not in summary.get("kernels", {}):
        return None
    k = summary["kernels"][kernel]
    return (k["fetch_kib"] * summary["fetch_scale"] + k["write_kib"] * summary["write_scale"]) * 1024


def measured_l2_read(summary, kernel: str):
    """Bytes the kernel's vector L1s read from L2 per launch (TCP_TCC_READ_REQ x 128 B) from a
    counter summary, or None."""
    if summary is None or kernel not in summary.get("kernels", {}):
        return None
    return summary["kernels"][kernel].get("l2_read_bytes")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, min_seconds: float = 10.0) -> dict:
    """The fp64 oracle on the host cores, on the full workload, repeated for about
    `min_seconds`; its median run gives tokens/s."""
    from oracle import kda_oracle, oracle_threads, QK_L2NORM, BETA_SIGMOID, SCALAR_GATE
    flags = ((QK_L2NORM if inp.qk_l2norm else 0) | (BETA_SIGMOID if inp.beta_sigmoid else 0)
             | (SCALAR_GATE if inp.scalar_gate else 0))
    times = []
    t_start = time.perf_counter()
    while len(times) < 3 or time.perf_counter() - t_start < min_seconds:
        t0 = time.perf_counter()
        kda_oracle(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.initial_state,
                   inp.cu_seqlens, inp.layout, flags, raw_gate=inp.gate_args)
        times.append(time.perf_counter() - t0)
        if len(times) >= 200:
            break
    times.sort()
    med = times[len(times) // 2]
    threads = oracle_threads()
    affinity = len(os.sched_getaffinity(0))
    return {"value": inp.tokens / med, "unit": "tokens/s", "cores": min(threads, affinity),
            "kind": "oracle", "omp_threads": threads, "affinity_cores": affinity,
            "cpu_model": cpu_model(),
            "sample": f"full workload ({inp.tokens} tokens x {inp.n_v} heads), fp64 token "
                      f"recurrence, median of {len(times)} runs over "
                      f"{time.perf_counter() - t_start:.1f} s"}


def copy_ceiling(nbytes: int, reps: int = 20) -> dict:
    """A plain device-to-device copy moving `nbytes` in all (nbytes / 2 read, nbytes / 2
    written): the practical bandwidth ceiling for a kernel of that size."""
    import torch
    half = max(nbytes // 2, 1)
    src = torch.ones(half, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return {"bytes": 2 * half, "median_ms": ms[reps // 2], "min_ms": ms[0],
            "GB/s": 2 * half / (ms[reps // 2] * 1e-3) / 1e9}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill_s8k_n3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copies", type=int, default=0, help="input copies rotated (0 = auto)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the reference "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by whole heads with no communication; see the design notes)",
              file=sys.stderr)
        return 2

    import torch
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / 5
        print(json.dumps({"copy_bytes": n, "ms": dt * 1e3, "GB/s (read+write)": 2 * n / dt / 1e9}))
        return 0
    from kimi_delta_attention_chunk_amd import (chunk_fwd, kda_chunk_fwd_workspace,
                                                kda_num_stages, kda_stage_name, make_shape,
                                                kda_chunk_fwd_plan, kda_chunk_fwd_plan_kernels)
    from kimi_delta_attention_chunk_amd.workloads import workload_inputs, BY_NAME

    wl = BY_NAME[args.workload]
    host = workload_inputs(wl)
    in_bytes = (host.q.numel() * 4 + host.v.numel() * 2 +
                host.g.numel() * host.g.element_size() + host.beta.numel() * 2)
    copies = args.copies or max(1, min(16, math.ceil(2 * MALL_BYTES / max(in_bytes, 1))))
    dev = torch.device("cuda", 0)
    sets = [host.to(dev) for _ in range(copies)]
    out = torch.empty_like(sets[0].v)
    d = head_dim(host)
    fin = torch.empty((host.batch, host.n_v, d, d), dtype=torch.float32, device=dev)
    shape = shape_of(host)
    ws = torch.empty(kda_chunk_fwd_workspace(shape), dtype=torch.uint8, device=dev)
    nst = kda_num_stages()

    for i in range(args.warmup):
        chunk_fwd(sets[i % copies], out=out, final_state=fin, workspace=ws)
    torch.cuda.synchronize()

    # timed region: K plain steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        chunk_fwd(sets[i % copies], out=out, final_state=fin, workspace=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    # the same K steps again, each kernel's dispatch recording its own start and end
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nst)]
              for _ in range(args.steps)]
    for evs in events:          # torch creates the HIP event on its first record
        for e in evs:
            e.record()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(args.steps):
        chunk_fwd(sets[i % copies], out=out, final_state=fin, workspace=ws,
                  stage_events=[e.cuda_event for e in events[i]])
    torch.cuda.synchronize()
    t3 = time.perf_counter()

    # the same K steps a third time, an event pair around each call: per-call median and min
    calls = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    for i in range(args.steps):
        calls[i][0].record()
        chunk_fwd(sets[i % copies], out=out, final_state=fin, workspace=ws)
        calls[i][1].record()
    torch.cuda.synchronize()
    call_ms = sorted(a.elapsed_time(b) for a, b in calls)

    ms_step = (t1 - t0) * 1e3 / args.steps
    stage_ms = [sum(events[i][2 * s].elapsed_time(events[i][2 * s + 1]) for i in range(args.steps))
                / args.steps for s in range(nst)]
    # stages the plan enqueues (an empty stage's two back-to-back events measure only the
    # marker packets between them)
    mask, segments = kda_chunk_fwd_plan(shape)
    live = [s for s in range(nst) if mask >> s & 1]
    dom = max(live, key=lambda s: stage_ms[s])
    kbytes = [KERNEL_BYTES[kda_stage_name(s)](host) for s in range(nst)]
    pbytes = path_bytes(host)
    value = host.tokens / (ms_step * 1e-3)
    summary = counter_summary(wl.name)
    traffic = {kda_stage_name(s): measured_traffic(summary, kda_stage_name(s)) for s in live}
    all_traffic = (sum(traffic.values()) if all(t is not None for t in traffic.values())
                   else None)
    # roofline of the dominant kernel: the call's algorithmic bytes (1,538 B per token-head at
    # Nqk = Nv, plus the states) over that kernel's average launch duration
    achieved = pbytes / (stage_ms[dom] * 1e-3)

    res = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": wl.name, "layout": host.layout, "batch": host.batch,
                   "seq_len": host.seq_len, "tokens": host.tokens, "n_qk": host.n_qk,
                   "n_v": host.n_v, "head_dim": d, "scalar_gate": host.scalar_gate,
                   "raw_gate": host.raw_gate,
                   "input_copies": copies,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": kda_stage_name(dom), "achieved": achieved / 1e9,
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": achieved / HBM_PEAK,
                     "traffic": traffic[kda_stage_name(dom)],
                     "algorithmic_bytes": pbytes, "avg_launch_ms": stage_ms[dom]},
        "path_roofline": {"bound": "hbm", "algorithmic_bytes": pbytes,
                          "achieved": pbytes / (ms_step * 1e-3) / 1e9, "unit": "GB/s",
                          "frac": pbytes / (ms_step * 1e-3) / HBM_PEAK},
        "traffic_ratio": None if all_traffic is None else all_traffic / pbytes,
        "kernel_traffic": traffic,
        # what bounds the chunk walks: the bytes each kernel's L1s pull from L2 per launch, and
        # that rate per compute unit (256 units; the two-level segment pass runs on fewer)
        "l2_read": {kda_stage_name(s): None if measured_l2_read(summary, kda_stage_name(s)) is None
                    else {"bytes": measured_l2_read(summary, kda_stage_name(s)),
                          "GB/s": measured_l2_read(summary, kda_stage_name(s))
                          / (stage_ms[s] * 1e-3) / 1e9}
                    for s in live},
        "per_call_ms": {"median": call_ms[len(call_ms) // 2], "min": call_ms[0],
                        "mean": sum(call_ms) / len(call_ms)},
        "copy_ceiling": copy_ceiling(pbytes),
        "stages_ms": {kda_stage_name(s): stage_ms[s] for s in live},
        "stage_workspace_bytes": {kda_stage_name(s): kbytes[s] for s in live},
        "kernels": kda_chunk_fwd_plan_kernels(shape),
        "segments": segments,
        "ms_per_step_with_stage_events": (t3 - t2) * 1e3 / args.steps,
        "token_heads_per_s": host.tokens * host.n_v / (ms_step * 1e-3),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(host)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
