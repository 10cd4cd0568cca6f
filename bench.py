#!/usr/bin/env python3
"""Benchmark of one rank's ring block-attention steps on one MI355X.

Headline (value): the forward ring replay of one rank of the 512K-token
causal zigzag workload (524288 tokens over 8 virtual ranks, rank 0 = pieces
0 and 15, 65536 queries; 32 query / 8 KV heads, d = 128, bf16, inputs
N(0,1) * 0.5): 8 steps of 65536 keys, rba_fwd_step for the first and
rba_fwd_step_acc (the LSE merge fused into the step) for the other 7, the
last one writing the bf16 output.  A bench "step" is one such replay.

value = effective forward FLOPs of the replay (4*d per allowed (query, key,
head) triple; masked and skipped work is not counted) / wall time of the
replay, with all inputs resident in HBM.  roofline.achieved is the same
flops / the summed launch times of the step kernels (HIP events on the
launch stream around every launch of the timed replays).

The breakdown reports, in the same run:
  * measured ceilings: a dense bf16 MFMA loop and an HBM copy
    (librba_probe.so), and the headline against both;
  * the 32K causal zigzag forward replay (rank 3);
  * the 64K packed-document forward replay of all 16 ranks (256 calls, the
    host skips the empty ones) through rba_fwd_step_ws, whose steps with few
    rows of work split their key ranges over more workgroups, and without
    the workspace;
  * the 32K backward replay (preprocess + 8 rba_bwd_step) and the
    forward + backward step it belongs to;
  * the stand-alone merge (rba_merge) in GB/s.
The CPU baseline is the fp64 oracle on a bounded sample of the headline
workload (sampled query rows of rank 0 against all 524288 keys).

Prints ONE JSON line.  Usage:
    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--headline-only] [--extra] [--flush-mib 512]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "per-rank block-attention TFLOP/s (effective, 1 GPU) and % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the 512K forward replay only (no breakdown workloads, probes or CPU baseline)")
    ap.add_argument("--part", choices=("fwd_32k", "fwd_64k_packed", "bwd_32k", "merge_32k", "probes"),
                    default=None,
                    help="run one breakdown part alone and print its figures (for profiler runs that "
                         "must see one workload's kernels only)")
    ap.add_argument("--extra", action="store_true",
                    help="also time the 32K forward replay under TASP's schedule and under the striped layout")
    ap.add_argument("--cpu-rows", type=int, default=96, help="query rows in the CPU-oracle sample")
    ap.add_argument("--flush-mib", type=int, default=0, metavar="MIB",
                    help="also time replays with the last-level cache flushed before each one "
                         "(a MIB-sized device buffer is overwritten between replays, outside the timing)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 4 device-to-device copies of MIB MiB (calibrates HBM byte counters) and exit")
    return ap.parse_args()


def copy_probe(mib):
    """A plain copy of known size: reads and writes mib MiB per launch."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_launch": n * 4, "launches": 4}), flush=True)


class LaunchTimer:
    """Events recorded on the launch stream before every launch (and once at the end)."""

    def __init__(self, torch):
        self.torch = torch
        self.marks = []          # (label, step index, event)

    def __call__(self, kind, i):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record()
        self.marks.append((kind, i, ev))

    def close(self):
        self("end", -1)

    def durations(self):
        out = []
        for (kind, i, a), (_, _, b) in zip(self.marks[:-1], self.marks[1:]):
            out.append((kind, i, a.elapsed_time(b)))
        return out


# ---------------------------------------------------------------------------
# HBM traffic of the headline kernel, from the committed counter summary

TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "fwd_step_512k_zigzag_hbm_traffic.md")
# Sources that make up a forward step (host planning and launch, the kernel
# and the headers it includes): the counters only hold for the code they
# were taken on.
FWD_SOURCES = ("rba_host.cpp", "rba_fwd.hip", "rba_qtile.h", "rba_device.h", "rba_kernels.h", "rba_addr.h")


def kernel_sources_sha256(files=FWD_SOURCES):
    src = os.path.join(ROOT, "ring_sequence_parallelism_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(files):
        h.update(f.encode())
        with open(os.path.join(src, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(path=None, files=FWD_SOURCES):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None when the kernel sources changed since those counters were taken."""
    path = path or TRAFFIC_PROFILE
    try:
        with open(path) as f:
            kv = dict(l.split(": ", 1) for l in f.read().splitlines() if l.startswith(("traffic_", "sources_")))
        if kv["sources_sha256"].strip() != kernel_sources_sha256(files):
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# timing helpers

def fwd_launch_stats(rr, timer, d, hq):
    """(flops, ms) summed over the forward launches a LaunchTimer saw."""
    fl, ms = 0, 0.0
    for kind, i, t in timer.durations():
        if kind == "fwd":
            fl += 4 * d * hq * rr.steps[i].pairs
            ms += t
    return fl, ms


def warm(torch, fn, min_ms=150.0):
    """Runs fn untimed until about min_ms of GPU time has passed (the shader
    clock ramps up over the first tens of milliseconds of load after the
    host-side setup of a workload); returns the ms of one call."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    fn()
    b.record()
    torch.cuda.synchronize()
    one = max(a.elapsed_time(b), 1e-3)
    for _ in range(int(min_ms / one)):
        fn()
    torch.cuda.synchronize()
    return one


_SPACER = {}


def spacer(torch, ms=100.0):
    """Queues about `ms` of GPU work (librba_probe's MFMA loop) ahead of a
    timed region, so that the host enqueues the timed launches while the GPU
    is still busy: they then run back to back, and the events around each
    launch time the GPU's work rather than the host's launch overhead (which
    exceeds the run time of the smallest steps when each launch is also
    bracketed by event records)."""
    from ring_sequence_parallelism_amd import probe
    if "out" not in _SPACER:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        _SPACER["wgs"] = 2 * cus
        _SPACER["out"] = torch.empty(2 * cus * 256, dtype=torch.float32, device="cuda")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        probe.rba_probe_mfma_bf16(_SPACER["wgs"], 20000, _SPACER["out"])
        b.record()
        torch.cuda.synchronize()
        _SPACER["iters_per_ms"] = 20000 / max(a.elapsed_time(b), 1e-3)
    probe.rba_probe_mfma_bf16(_SPACER["wgs"], max(1, int(ms * _SPACER["iters_per_ms"])), _SPACER["out"])


def forward_replay_rate(torch, replays, reps=10):
    """Effective forward TFLOP/s of ring replays (the step launches' summed
    time, events on the launch stream), after untimed warm-up replays."""
    fl, ms_tot, calls = 0, 0.0, 0

    def all_replays():
        for rr in replays:
            rr.forward()
    warm(torch, all_replays)
    spacer(torch)
    tm = LaunchTimer(torch)
    for _ in range(reps):
        for rr in replays:
            rr.forward(on_step=tm)
    tm.close()
    torch.cuda.synchronize()
    for kind, i, t in tm.durations():
        if kind == "fwd":
            ms_tot += t
    for rr in replays:
        fl += rr.fwd_flops()
        calls += sum(1 for s in rr.steps if s.status == 0)
    ms = ms_tot / reps
    t = fl / (ms * 1e-3) / 1e12
    return {"fwd_step_tflops": round(t, 2), "frac_peak": round(t / PEAK_BF16_TFLOPS, 4),
            "fwd_ms": round(ms, 4), "launches": calls, "replays": len(replays)}


def mfma_probe(torch):
    """Dense bf16 MFMA rate of librba_probe's loop (2 workgroups of 4 waves per CU)."""
    from ring_sequence_parallelism_amd import probe
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = 2 * cus
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    iters = 20000
    warm(torch, lambda: probe.rba_probe_mfma_bf16(wgs, iters, out))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps, fl = 5, 0.0
    a.record()
    for _ in range(reps):
        fl += probe.rba_probe_mfma_bf16(wgs, iters, out)
    b.record()
    torch.cuda.synchronize()
    t = fl / (a.elapsed_time(b) * 1e-3) / 1e12
    return {"tflops": round(t, 1), "frac_datasheet": round(t / PEAK_BF16_TFLOPS, 4),
            "workgroups": wgs, "launch_ms": round(a.elapsed_time(b) / reps, 3)}


def hbm_probe(torch, mib=2048):
    """HBM bandwidth of librba_probe's copy: 2 * bytes moved per launch."""
    from ring_sequence_parallelism_amd import probe
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nbytes = mib << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    wgs = 8 * cus
    warm(torch, lambda: probe.rba_probe_copy(src, dst, nbytes, wgs))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    a.record()
    for _ in range(reps):
        probe.rba_probe_copy(src, dst, nbytes, wgs)
    b.record()
    torch.cuda.synchronize()
    ok = bool(torch.equal(src[:1 << 20], dst[:1 << 20]))
    gbs = 2 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"gbs": round(gbs, 1), "frac_datasheet": round(gbs / PEAK_HBM_GBS, 4), "copy_mib": mib,
            "copied_ok": ok}


def cpu_baseline(w, rows_n):
    """The oracle's forward on a bounded sample of the headline workload:
    sampled query rows of the rank against all keys of the sequence."""
    import numpy as np
    import oracle
    from ring_sequence_parallelism_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    rows = W.gen_sampled_rows(w, rows_n, w.chunk_len)
    qpos = oracle.zigzag_positions(w.seq, w.n_ranks, w.rank)[rows]
    q = W.to_f64(W.gen_rank_chunk(w, W.T_Q, w.rank), w.dtype)[rows]
    k = W.to_f64(W.gen_pieces(w, W.T_K, range(w.n_pieces)), w.dtype)
    v = W.to_f64(W.gen_pieces(w, W.T_V, range(w.n_pieces)), w.dtype)
    kpos = np.arange(w.seq)
    t0 = time.perf_counter()
    oracle.attention(q, k, v, qpos, kpos, w.mask, w.scale)
    secs = time.perf_counter() - t0
    pairs = int((qpos + 1).sum())          # causal: the row at position p sees p + 1 keys
    flops = 4 * w.d * w.hq * pairs
    cores = len(os.sched_getaffinity(0))
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": blas_threads or cores,
            "kind": "oracle",
            "sample": f"fp64 numpy oracle forward of {rows_n} sampled query rows of rank {w.rank} of the "
                      f"524288-token causal zigzag workload (all {w.hq} heads) against all {w.seq} keys; "
                      f"{secs:.1f} s on {cores} visible host cores, BLAS threads {blas_threads}; effective "
                      f"flops counted as on the GPU (4*d per allowed pair and head)"}


# ---------------------------------------------------------------------------

def headline(torch, args, RingReplay, W):
    """The timed region: K forward replays of the 512K zigzag rank."""
    w = W.WORKLOADS["c4"]
    rr = RingReplay(w, None, "cuda")
    flops = rr.fwd_flops()
    for _ in range(args.warmup):
        rr.forward()
    torch.cuda.synchronize()
    timer = LaunchTimer(torch)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for k in range(args.steps):
        marks[k].record()
        rr.forward(on_step=timer)
    marks[-1].record()
    timer.close()
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    step_ms = sorted(marks[k].elapsed_time(marks[k + 1]) for k in range(args.steps))
    kfl, kms = fwd_launch_stats(rr, timer, w.d, w.hq)
    per_step = {}
    for kind, i, t in timer.durations():
        if kind == "fwd":
            per_step.setdefault(i, []).append(t)
    res = {
        "w": w, "flops": flops, "ms_per_step": total_ms / args.steps, "step_ms": step_ms,
        "kernel_flops": kfl, "kernel_ms": kms, "launches": sum(len(v) for v in per_step.values()),
        "per_step_us": {f"step{i}_src{rr.steps[i].src}": round(1e3 * sum(v) / len(v), 1)
                        for i, v in sorted(per_step.items())},
        "pairs": rr.effective_pairs,
    }
    if args.flush_mib > 0:
        buf = torch.empty(args.flush_mib * (1 << 18), dtype=torch.float32, device="cuda")
        cold = []
        for k in range(max(3, args.steps // 4)):
            buf.fill_(float(k))
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            rr.forward()
            b.record()
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b))
        cold.sort()
        med = cold[len(cold) // 2]
        res["cold_cache"] = {"flush_mib": args.flush_mib, "step_ms_median": round(med, 3),
                             "tflops_at_median": round(flops / (med * 1e-3) / 1e12, 2)}
        del buf
    del rr
    torch.cuda.empty_cache()
    return res


def backward_breakdown(torch, RingReplay, W, reps=10):
    """The 32K forward + backward step (c5 layout): backward launch rates and
    the end-to-end step."""
    w = W.WORKLOADS["c5"]
    rr = RingReplay(w, None, "cuda", with_grad=True)
    fwd_fl, bwd_fl = rr.fwd_flops(), rr.bwd_flops()

    def step():
        rr.forward()
        rr.backward()
    warm(torch, step)
    spacer(torch)
    tm = LaunchTimer(torch)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        rr.forward(on_step=tm)
        rr.backward(on_step=tm)
    tm.close()
    b.record()
    torch.cuda.synchronize()
    per = {}
    for kind, i, t in tm.durations():
        per.setdefault(kind, []).append((i, t))
    d, hq = w.d, w.hq
    bwd_ms = sum(t for _, t in per["bwd"])
    bwd_work = sum(10 * d * hq * rr.steps[i].pairs for i, _ in per["bwd"])
    fwd_ms = sum(t for _, t in per["fwd"])
    prep_ms = sum(t for _, t in per["prep"])
    step_ms = a.elapsed_time(b) / reps
    bt = bwd_work / (bwd_ms * 1e-3) / 1e12
    out = {"bwd_step_tflops": round(bt, 2), "bwd_step_frac_peak": round(bt / PEAK_BF16_TFLOPS, 4),
           "bwd_avg_launch_us": round(1e3 * bwd_ms / len(per["bwd"]), 1),
           "prep_us": round(1e3 * prep_ms / len(per["prep"]), 1),
           "fwd_plus_bwd_step_ms": round(step_ms, 4),
           "fwd_plus_bwd_tflops": round((fwd_fl + bwd_fl) / (step_ms * 1e-3) / 1e12, 2),
           "fwd_kernel_ms": round(fwd_ms / reps, 4), "bwd_kernel_ms": round(bwd_ms / reps, 4)}
    del rr
    torch.cuda.empty_cache()
    return out


def merge_breakdown(torch, RingReplay, W, reps=10):
    """rba_merge alone: the 32K replay through o_part and separate merges."""
    w = W.WORKLOADS["c2"]
    rr = RingReplay(w, None, "cuda")
    warm(torch, lambda: rr.forward(fused_merge=False))
    spacer(torch)
    mt = LaunchTimer(torch)
    for _ in range(reps):
        rr.forward(on_step=mt, fused_merge=False)
    mt.close()
    torch.cuda.synchronize()
    items = [t for kind, _, t in mt.durations() if kind == "merge"]
    sq, hq, d = rr.q.shape[0], w.hq, w.d
    # 12d+12 bytes per (row, head); the last merge of each replay also writes bf16 O
    work = len(items) * (12 * d + 12) * sq * hq + reps * 2 * d * sq * hq
    gbs = work / (sum(items) * 1e-3) / 1e9
    del rr
    torch.cuda.empty_cache()
    return {"merge_gbs": round(gbs, 1), "merge_frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
            "merge_avg_us": round(1e3 * sum(items) / len(items), 2)}


def packed_docs_breakdown(torch, RingReplay, W, reps=10):
    """All 16 ranks of the 64K packed-document workload (K / V shared), with
    a workspace (steps with few rows of work split their key ranges,
    rba_fwd_step_ws) and without."""
    from ring_sequence_parallelism_amd import rba
    from ring_sequence_parallelism_amd.ring import to_device
    w = W.WORKLOADS["c3"]
    shared = {"k": {j: to_device(W.gen_rank_chunk(w, W.T_K, j), w.dtype, "cuda") for j in range(w.n_ranks)},
              "v": {j: to_device(W.gen_rank_chunk(w, W.T_V, j), w.dtype, "cuda") for j in range(w.n_ranks)}}
    ws = torch.empty((32 << 20) // 4, dtype=torch.float32, device="cuda")
    replays = [RingReplay(w, r, "cuda", kv=shared, workspace=ws) for r in range(w.n_ranks)]
    out = forward_replay_rate(torch, replays, reps=reps)
    out["split_launches"] = sum(
        1 for rr in replays for s_ in rr.steps
        if s_.status == rba.RBA_OK and rba.rba_fwd_workspace_size(
            rr.attn, rr.q.shape[0], rr.q_segs, rr.k[s_.src].shape[0], rr.kv_segs[s_.src]) > 0)
    out["documents"] = int(replays[0].attn.n_docs)
    for rr in replays:
        rr.workspace = None
    out["unsplit"] = forward_replay_rate(torch, replays, reps=reps)
    del replays, shared, ws
    torch.cuda.empty_cache()
    return out


def extra_breakdown(torch, RingReplay, W):
    import dataclasses
    from ring_sequence_parallelism_amd.ring import TaspReplay
    extra = {}
    tx = TaspReplay(W.WORKLOADS["c2"], None, "cuda")
    extra["c2_tasp_schedule_fwd"] = forward_replay_rate(torch, [tx])
    extra["c2_tasp_schedule_fwd"]["max_segments_per_step"] = max(tx.kv_segs[i].n for i in tx.kv_segs)
    del tx
    wst = dataclasses.replace(W.WORKLOADS["c2"], layout="striped", name="c2_bf16_causal_striped_32k")
    sx = RingReplay(wst, None, "cuda")
    extra[wst.name] = forward_replay_rate(torch, [sx])
    del sx
    torch.cuda.empty_cache()
    return extra


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the ring is replayed on a single MI355X "
              f"(got --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    from ring_sequence_parallelism_amd import rba
    from ring_sequence_parallelism_amd import workloads as W
    from ring_sequence_parallelism_amd.ring import RingReplay

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    rba.load()
    if args.part:
        parts = {
            "fwd_32k": lambda: forward_replay_rate(torch, [RingReplay(W.WORKLOADS["c2"], None, "cuda")],
                                                   reps=max(1, args.steps)),
            "fwd_64k_packed": lambda: packed_docs_breakdown(torch, RingReplay, W, reps=max(1, args.steps)),
            "bwd_32k": lambda: backward_breakdown(torch, RingReplay, W, reps=max(1, args.steps)),
            "merge_32k": lambda: merge_breakdown(torch, RingReplay, W, reps=max(1, args.steps)),
            "probes": lambda: {"mfma_bf16": mfma_probe(torch), "hbm_copy": hbm_probe(torch)},
        }
        print(json.dumps({"part": args.part, "steps": args.steps, "result": parts[args.part]()}), flush=True)
        return
    h = headline(torch, args, RingReplay, W)
    w = h["w"]
    value = h["flops"] / (h["ms_per_step"] * 1e-3) / 1e12
    achieved = h["kernel_flops"] / (h["kernel_ms"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(),
                "kernel": "rba_fwd_step / rba_fwd_step_acc (fwd_bf16_kernel), 512K causal zigzag steps",
                "avg_launch_us": round(1e3 * h["kernel_ms"] / h["launches"], 1)}
    breakdown = {
        "value_frac_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "step_ms_median": round(h["step_ms"][len(h["step_ms"]) // 2], 3),
        "step_ms_min": round(h["step_ms"][0], 3),
        "effective_pairs_per_head": h["pairs"],
        "step_effective_flops": h["flops"],
        "fwd_launch_us": h["per_step_us"],
    }
    if "cold_cache" in h:
        breakdown["cold_cache"] = h["cold_cache"]
    extra = {}
    cpu = None
    if not args.headline_only:
        mp = mfma_probe(torch)
        hp = hbm_probe(torch)
        breakdown["measured_peaks"] = {"mfma_bf16": mp, "hbm_copy": hp}
        breakdown["value_frac_measured_mfma"] = round(value / mp["tflops"], 4)
        breakdown["achieved_frac_measured_mfma"] = round(achieved / mp["tflops"], 4)
        c2 = W.WORKLOADS["c2"]
        breakdown["fwd_32k_zigzag"] = forward_replay_rate(torch, [RingReplay(c2, None, "cuda")])
        torch.cuda.empty_cache()
        breakdown["fwd_64k_packed_docs"] = packed_docs_breakdown(torch, RingReplay, W)
        breakdown["bwd_32k_zigzag"] = backward_breakdown(torch, RingReplay, W)
        mg = merge_breakdown(torch, RingReplay, W)
        mg["merge_frac_measured_hbm"] = round(mg["merge_gbs"] / hp["gbs"], 4)
        breakdown["merge_32k"] = mg
        if args.extra:
            extra = extra_breakdown(torch, RingReplay, W)
        if not args.no_cpu_baseline:
            cpu = cpu_baseline(w, args.cpu_rows)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(h["ms_per_step"], 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal zigzag 524288 tokens over 8 virtual ranks, rank 0 (65536 queries, "
                               "pieces 0 and 15), 32 q / 8 kv heads, d=128, bf16: forward ring replay "
                               "(8 steps of 65536 keys, LSE merges fused into steps 2-8)",
                   "seq_len": w.seq, "ranks": w.n_ranks, "rank": w.rank, "hq": w.hq, "hkv": w.hkv,
                   "head_dim": w.d, "mask": "causal-zigzag"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "breakdown": breakdown,
    }
    if extra:
        line["extra_workloads"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
