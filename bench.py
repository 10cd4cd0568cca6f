#!/usr/bin/env python3
"""Benchmark of one rank's ring block-attention step on one MI355X.

A bench "step" is one pass of the whole hot path over one batch of
synthetic input: the forward ring replay (rba_fwd_step for the first step,
then rba_fwd_step_acc, which merges each later step's partial into the
running result in the same launch, the last one writing the bf16 output)
followed by the backward ring replay (rba_bwd_preprocess on the merged fp32
output, then 8 rba_bwd_step launches).  The stand-alone rba_merge is timed
on a separate replay for the breakdown.
Workload: causal zigzag split of a 32768-token sequence over 8 virtual
ranks, rank 3 (pieces 3 and 12, 4096 queries), 32 query / 8 KV heads,
d = 128, bf16, inputs N(0,1) plus a seeded dO.

value = effective FLOPs of the step (4*d per allowed (query, key, head)
triple in the forward, 10*d in the backward; masked and skipped work is not
counted) / time of the step, with all inputs resident in HBM.  The
breakdown also reports the forward replay of one rank of a 524288-token
causal zigzag split (8 steps of 65536 keys; --no-long-forward skips it).

Prints ONE JSON line.  Usage:
    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-long-forward] [--extra] [--flush-mib 512]
"""
from __future__ import annotations

import argparse
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
    ap.add_argument("--extra", action="store_true",
                    help="also time the forward replays of the 64K packed-document and 512K zigzag workloads")
    ap.add_argument("--no-long-forward", action="store_true",
                    help="skip the 512K zigzag forward replay reported in the breakdown")
    ap.add_argument("--cpu-rows", type=int, default=1024,
                    help="query rows in the CPU-oracle sample")
    ap.add_argument("--flush-mib", type=int, default=0, metavar="MIB",
                    help="also time steps with the last-level cache flushed before each one "
                         "(a MIB-sized device buffer is overwritten between steps, outside the timing)")
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


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "bwd_step_32k_zigzag_hbm_traffic.md")


# Sources that make up rba_bwd_step (host planning and launch, the fused
# backward kernel and the headers it includes): the counter summary is only
# valid for the code it was measured on.
BWD_SOURCES = ("rba_host.cpp", "rba_bwd.hip", "rba_bwd_dq.h", "rba_qtile.h", "rba_device.h", "rba_kernels.h")


def kernel_sources_sha256():
    import hashlib
    src = os.path.join(ROOT, "ring_sequence_parallelism_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(BWD_SOURCES):
        h.update(f.encode())
        with open(os.path.join(src, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per rba_bwd_step from the committed rocprofv3 counter summary,
    or None when the kernel sources changed since those counters were taken."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            kv = dict(l.split(": ", 1) for l in f.read().splitlines() if l.startswith(("traffic_", "sources_")))
        if kv["sources_sha256"].strip() != kernel_sources_sha256():
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def run_step(rr, timer=None):
    rr.forward(on_step=timer)
    rr.backward(on_step=timer)


def cpu_baseline(w, rows_n):
    """The oracle's forward + backward on a bounded sample of the same workload."""
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
    do = W.to_f64(W.gen_rank_chunk(w, W.T_DO, w.rank), w.dtype)[rows]
    k = W.to_f64(W.gen_pieces(w, W.T_K, range(w.n_pieces)), w.dtype)
    v = W.to_f64(W.gen_pieces(w, W.T_V, range(w.n_pieces)), w.dtype)
    kpos = np.arange(w.seq)
    t0 = time.perf_counter()
    oracle.attention_backward(q, k, v, do, qpos, kpos, w.mask, w.scale)
    secs = time.perf_counter() - t0
    pairs = int((qpos + 1).sum())          # causal: the row at position p sees p + 1 keys
    flops = 14 * w.d * w.hq * pairs
    cores = len(os.sched_getaffinity(0))
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": blas_threads or cores,
            "kind": "oracle",
            "sample": f"fp64 numpy oracle forward+backward of {rows_n} sampled query rows of rank "
                      f"{w.rank} (all {w.hq} heads) against all {w.seq} keys; {secs:.1f} s on "
                      f"{cores} visible host cores, BLAS threads {blas_threads}; effective flops "
                      f"counted as on the GPU (14*d per allowed pair and head)"}


def forward_replay_rate(torch, RingReplay, wx, ranks, reps=2):
    """Effective forward TFLOP/s of the ring replays of `ranks` (sum of the
    rba_fwd_step / rba_fwd_step_acc launch times, events on the launch stream)."""
    fl, ms_tot = 0, 0.0
    for r in ranks:
        rx = RingReplay(wx, r, "cuda")
        rx.forward()
        torch.cuda.synchronize()
        tm = LaunchTimer(torch)
        for _ in range(reps):
            rx.forward(on_step=tm)
        tm.close()
        torch.cuda.synchronize()
        ms_tot += sum(ms for kind, _, ms in tm.durations() if kind == "fwd") / reps
        fl += rx.fwd_flops()
        del rx
        torch.cuda.empty_cache()
    t = fl / (ms_tot * 1e-3) / 1e12
    return {"fwd_step_tflops": round(t, 2), "frac_peak": round(t / PEAK_BF16_TFLOPS, 4),
            "fwd_ms": round(ms_tot, 3), "ranks": len(ranks)}


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
    w = W.WORKLOADS["c5"]
    rr = RingReplay(w, None, "cuda", with_grad=True)
    fwd_flops, bwd_flops = rr.fwd_flops(), rr.bwd_flops()
    step_flops = fwd_flops + bwd_flops

    for _ in range(args.warmup):
        run_step(rr)
    torch.cuda.synchronize()

    timer = LaunchTimer(torch)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t_start.record()
    for k in range(args.steps):
        marks[k].record()
        run_step(rr, timer)
    marks[-1].record()
    timer.close()
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    step_ms = sorted(marks[k].elapsed_time(marks[k + 1]) for k in range(args.steps))

    # per-kernel time over the timed region
    per = {}
    for kind, i, ms in timer.durations():
        per.setdefault(kind, []).append((i, ms))
    d, hq, sq = w.d, w.hq, rr.q.shape[0]
    kern = {}
    for kind, items in per.items():
        tot = sum(ms for _, ms in items)
        if kind == "fwd":
            work = sum(4 * d * hq * rr.steps[i].pairs for i, _ in items)
        elif kind == "bwd":
            work = sum(10 * d * hq * rr.steps[i].pairs for i, _ in items)
        else:   # preprocess: reads O (fp32 accumulator) and dO (bf16), writes delta
            work = len(items) * (6 * d + 4) * sq * hq
        kern[kind] = {"launches": len(items), "total_ms": tot, "avg_us": 1e3 * tot / len(items), "work": work}
    # The timed replay merges each step inside rba_fwd_step_acc.  The stand-alone
    # merge (rba_merge) is timed on a separate replay that goes through o_part.
    mt = LaunchTimer(torch)
    for _ in range(3):
        rr.forward(on_step=mt, fused_merge=False)
    mt.close()
    torch.cuda.synchronize()
    m_items = [(i, ms) for kind, i, ms in mt.durations() if kind == "merge"]
    m_tot = sum(ms for _, ms in m_items)
    # 12d+12 bytes per (row, head); the last merge of each replay also writes bf16 O
    m_work = len(m_items) * (12 * d + 12) * sq * hq + 3 * 2 * d * sq * hq
    kern["merge"] = {"launches": len(m_items), "total_ms": m_tot, "avg_us": 1e3 * m_tot / len(m_items),
                     "work": m_work}
    dom = max(("fwd", "bwd"), key=lambda k: kern[k]["total_ms"])
    dk = kern[dom]
    achieved = dk["work"] / (dk["total_ms"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic() if dom == "bwd" else None,
                "kernel": ("rba_bwd_step (dK/dV zero fill, dK/dV and dQ kernels)" if dom == "bwd"
                           else "rba_fwd_step"),
                "avg_launch_us": round(dk["avg_us"], 2)}
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    fwd_t = kern["fwd"]["work"] / (kern["fwd"]["total_ms"] * 1e-3) / 1e12
    bwd_t = kern["bwd"]["work"] / (kern["bwd"]["total_ms"] * 1e-3) / 1e12
    merge_gbs = kern["merge"]["work"] / (kern["merge"]["total_ms"] * 1e-3) / 1e9
    breakdown = {
        "fwd_step_tflops": round(fwd_t, 2), "fwd_step_frac_peak": round(fwd_t / PEAK_BF16_TFLOPS, 4),
        "bwd_step_tflops": round(bwd_t, 2), "bwd_step_frac_peak": round(bwd_t / PEAK_BF16_TFLOPS, 4),
        "merge_gbs": round(merge_gbs, 1), "merge_frac_hbm": round(merge_gbs / PEAK_HBM_GBS, 4),
        "value_frac_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "kernel_ms_per_step": {k: round(v["total_ms"] / args.steps, 4) for k, v in kern.items() if k != "merge"},
        "kernel_avg_us": {k: round(v["avg_us"], 2) for k, v in kern.items()},
        "effective_pairs_per_head": rr.effective_pairs,
        "step_effective_flops": step_flops,
        "step_ms_median": round(step_ms[len(step_ms) // 2], 4),
        "step_ms_min": round(step_ms[0], 4),
    }
    if args.flush_mib > 0:
        # cold last-level cache: overwrite a buffer larger than the 256 MB
        # Infinity Cache before each step, then time the step alone
        buf = torch.empty(args.flush_mib * (1 << 18), dtype=torch.float32, device="cuda")
        cold = []
        for k in range(args.steps):
            buf.fill_(float(k))
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            run_step(rr)
            b.record()
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b))
        cold.sort()
        med = cold[len(cold) // 2]
        breakdown["cold_cache"] = {"flush_mib": args.flush_mib, "step_ms_median": round(med, 4),
                                   "step_ms_min": round(cold[0], 4),
                                   "tflops_at_median": round(step_flops / (med * 1e-3) / 1e12, 2)}
        del buf
        torch.cuda.empty_cache()
    extra = {}
    if args.extra:
        # the same 32K zigzag forward under TASP's decomposed schedule: steps
        # are unions of 7 slices from different source ranks
        from ring_sequence_parallelism_amd.ring import TaspReplay
        tx = TaspReplay(W.WORKLOADS["c2"], None, "cuda")
        tx.forward()
        torch.cuda.synchronize()
        tm = LaunchTimer(torch)
        for _ in range(3):
            tx.forward(on_step=tm)
        tm.close()
        torch.cuda.synchronize()
        f_ms = sum(ms for kind, _, ms in tm.durations() if kind == "fwd") / 3
        t = tx.fwd_flops() / (f_ms * 1e-3) / 1e12
        extra["c2_tasp_schedule_fwd"] = {"fwd_step_tflops": round(t, 2), "frac_peak": round(t / PEAK_BF16_TFLOPS, 4),
                                         "fwd_ms": round(f_ms, 3),
                                         "max_segments_per_step": max(tx.kv_segs[i].n for i in tx.kv_segs)}
        del tx
        torch.cuda.empty_cache()
        # the 32K causal replay under the striped layout (token i on rank i mod 8)
        import dataclasses
        wst = dataclasses.replace(W.WORKLOADS["c2"], layout="striped", name="c2_bf16_causal_striped_32k")
        sx = RingReplay(wst, None, "cuda")
        sx.forward()
        torch.cuda.synchronize()
        tm = LaunchTimer(torch)
        for _ in range(3):
            sx.forward(on_step=tm)
        tm.close()
        torch.cuda.synchronize()
        f_ms = sum(ms for kind, _, ms in tm.durations() if kind == "fwd") / 3
        t = sx.fwd_flops() / (f_ms * 1e-3) / 1e12
        extra[wst.name] = {"fwd_step_tflops": round(t, 2), "frac_peak": round(t / PEAK_BF16_TFLOPS, 4),
                           "fwd_ms": round(f_ms, 3)}
        del sx
        torch.cuda.empty_cache()
        wx = W.WORKLOADS["c3"]
        extra[wx.name] = forward_replay_rate(torch, RingReplay, wx, range(wx.n_ranks))
    # The 512K causal zigzag forward (one rank's 8 steps of 65536 keys) is the
    # long-sequence forward figure; it is reported on every run (about 10 s).
    if not args.no_long_forward:
        wx = W.WORKLOADS["c4"]
        breakdown["fwd_512k_zigzag"] = forward_replay_rate(torch, RingReplay, wx, [wx.rank])

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_rows)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal zigzag 32768 tokens over 8 virtual ranks, rank 3 (4096 queries), "
                               "32 q / 8 kv heads, d=128, bf16: forward ring replay (8 steps, LSE merges fused "
                               "into steps 2-8) + backward ring replay (preprocess + 8 steps)",
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
