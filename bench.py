"""Benchmark: packed varlen block-causal attention, forward + backward, one MI355X.

Default workload: best-fit-decreasing packing of 20,000 log-normal sample
lengths (median 600, sigma 1, clipped to [8, 8192]) at budget 8192, then
attention on the first pack (T = 8192, one 8192-token segment), H = 32,
head_dim = 128, bf16 Q/K/V ~ N(0,1)*0.5 and dO ~ N(0,1).

One step is one pass of the whole hot path over that batch:
  host   pack_plan_bfd over the 20,000 lengths; the first pack's lengths are
         copied to the device (pinned ring buffer, asynchronous),
  device build_packed_row (cu_seqlens, position_ids, segment_ids),
         varlen_attn_fwd (O bf16, LSE), varlen_attn_bwd (dQ, dK, dV fp32).
Host planning of step i+1 overlaps the device work of step i.

Useful work: F = sum over segments of H * 4 * d * L(L+1)/2 for the forward;
the backward counts 2.5 F (five matrix products over the permitted edges),
so a step is 3.5 F.  Printed as one JSON line.

python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-hbm-case]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


T_START = time.perf_counter()


def note(msg):
    """One progress line on stderr (stdout carries only the JSON result)."""
    print(f"bench: {msg} ({time.perf_counter() - T_START:.1f} s)", file=sys.stderr, flush=True)


def useful_fwd_flops(lengths, H, d):
    return float(sum(H * 4.0 * d * L * (L + 1) / 2.0 for L in (int(x) for x in lengths)))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hbm-case", action="store_true")
    ap.add_argument("--no-long-case", action="store_true")
    ap.add_argument("--no-meta-case", action="store_true")
    ap.add_argument("--no-loss-case", action="store_true")
    ap.add_argument("--no-gqa-case", action="store_true")
    ap.add_argument("--no-band-case", action="store_true")
    ap.add_argument("--no-gdn-case", action="store_true")
    ap.add_argument("--no-calls-case", action="store_true")
    ap.add_argument("--no-edge-case", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration)")
    return ap.parse_args()


KERNEL_SOURCES = ("pvb_device.hpp", "attn_common.hip", "attn_fwd.hip", "attn_bwd.hip")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "packed_varlen_block_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(here, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch from the committed counter runs, if the kernels
    they were taken on are the ones built now; else None."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_info():
    """(library, threads) of numpy's BLAS as threadpoolctl reports it."""
    try:
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                return f"{p.get('internal_api')} ({os.path.basename(p.get('filepath', ''))})", int(p["num_threads"])
    except Exception:
        pass
    return "unknown", 0


def oracle_per_config(seed, raw, first, budget_s=10.0):
    """The fp64 oracle's wall time per workload, on one head of each (the
    head count is scaled out: full = one head x H, every head costing the
    same), forward for the forward-only workloads and forward + backward for
    the others; with the useful GFLOP/s on the same count as the GPU's."""
    from oracle import attention as A
    import workloads as W
    res = {}
    t_all = time.perf_counter()
    for cfg in (1, 2, 3, 5, 4):
        if cfg == 4 and time.perf_counter() - t_all > budget_s:
            res[f"cfg{cfg}"] = {"skipped": "time budget"}
            continue
        H_full = W.HEADS[cfg]
        w1 = W.make(cfg, seed=seed, first_pack_lengths=first if cfg == 3 else None, H=1)
        f = W.bf16_bits_to_f64
        q, k, v = f(w1.q), f(w1.k), f(w1.v)
        cu = np.concatenate([[0], np.cumsum(w1.lengths)]).astype(np.int64)
        t0 = time.perf_counter()
        A.varlen_forward(q, k, v, cu)
        t_f = time.perf_counter() - t0
        rec = {"T": int(w1.T), "H": H_full, "head_dim": w1.d, "heads_timed": 1,
               "fwd_s_per_head": round(t_f, 4), "fwd_s_full": round(t_f * H_full, 3)}
        F1 = useful_fwd_flops(w1.lengths, 1, w1.d)
        if w1.backward:
            t0 = time.perf_counter()
            A.varlen_backward(q, k, v, f(w1.do), cu)
            t_b = time.perf_counter() - t0
            rec.update({"bwd_s_per_head": round(t_b, 4), "fwd_bwd_s_full": round((t_f + t_b) * H_full, 3),
                        "useful_gflops": round(3.5 * F1 / (t_f + t_b) / 1e9, 2)})
        else:
            rec["useful_gflops"] = round(F1 / t_f / 1e9, 2)
        res[f"cfg{cfg}"] = rec
    # host planners at n = 20,000: the oracle's BFD against the library's
    from oracle import packing as P
    import packed_varlen_block_amd as pvb
    t0 = time.perf_counter()
    P.best_fit_decreasing(raw.tolist(), 8192)
    t_py = time.perf_counter() - t0
    t0 = time.perf_counter()
    for _ in range(10):
        pvb.pack_plan_bfd(raw, 8192)
    t_c = (time.perf_counter() - t0) / 10
    res["bfd_n20000"] = {"oracle_python_ms": round(t_py * 1e3, 2), "library_cpp_ms": round(t_c * 1e3, 3)}
    return res


def cpu_baseline(wl, budget_s):
    """Time the fp64 oracle (as it stands) on whole heads of the same workload."""
    from oracle import attention as A
    import workloads as W
    cores = len(os.sched_getaffinity(0))
    blas, blas_threads = blas_info()
    q = W.bf16_bits_to_f64(wl.q)
    k = W.bf16_bits_to_f64(wl.k)
    v = W.bf16_bits_to_f64(wl.v)
    do = W.bf16_bits_to_f64(wl.do)
    cu = np.concatenate([[0], np.cumsum(wl.lengths)]).astype(np.int64)
    heads = 0
    t0 = time.perf_counter()
    while heads < wl.H and time.perf_counter() - t0 < budget_s:
        A.varlen_forward(q, k, v, cu, heads=[heads])
        A.varlen_backward(q, k, v, do, cu, heads=[heads])
        heads += 1
    el = time.perf_counter() - t0
    flops = 3.5 * useful_fwd_flops(wl.lengths, heads, wl.d)
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"fp64 numpy oracle forward+backward on {heads} of {wl.H} heads of the same "
                      f"pack, {el:.1f} s; useful causal FLOP counted as on the GPU",
            "cpu_model": cpu_model(), "blas": blas, "blas_threads": blas_threads}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}); this build has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import packed_varlen_block_amd as pvb
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # ---- workload: BFD first pack of the 20,000 lengths
    raw = W.raw_lengths_cfg3(a.seed)
    _, _, n_bins, order, offs = pvb.pack_plan_bfd(raw, 8192)
    first = raw[order[offs[0]:offs[1]]]
    wl = W.make(3, seed=a.seed, first_pack_lengths=first)
    T, H, d = wl.T, wl.H, wl.d
    B = len(wl.lengths)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = up(wl.q), up(wl.k), up(wl.v), up(wl.do)
    o = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    dq = torch.empty((T, H, d), dtype=torch.float32, device=dev)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    ws_f = torch.empty(pvb.workspace_bytes(T, H, d, B, False), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(pvb.workspace_bytes(T, H, d, B, True, pvb.PVB_F32), dtype=torch.uint8, device=dev)
    st_row = torch.zeros(1, dtype=torch.int32, device=dev)
    st_f = torch.zeros(1, dtype=torch.int32, device=dev)
    st_b = torch.zeros(1, dtype=torch.int32, device=dev)
    # Each step's pack lengths are planned on the host and uploaded on a copy
    # stream one step ahead, while the previous step runs, so that the upload's
    # latency stays off the compute stream; four pinned and device slots rotate.
    ring = [torch.empty(B, dtype=torch.int32).pin_memory() for _ in range(4)]
    ring_ev = [None] * 4                              # the slot's last upload
    use_ev = [None] * 4                               # the slot's last packed-row build
    len_dev = [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(4)]
    copy_stream = torch.cuda.Stream(dev)

    ev = {name: [] for name in ("row", "fwd", "bwd")}

    def plan_and_upload(i):
        # host: plan, take the first pack, stage its lengths for step i
        _, _, _, order_i, offs_i = pvb.pack_plan_bfd(raw, 8192)
        slot = i % 4
        if ring_ev[slot] is not None:
            ring_ev[slot].synchronize()               # step i - 4 is done with the slot
        ring[slot].numpy()[:] = raw[order_i[offs_i[0]:offs_i[1]]]
        if use_ev[slot] is not None:
            copy_stream.wait_event(use_ev[slot])      # step i - 4's packed-row build has read it
        with torch.cuda.stream(copy_stream):
            len_dev[slot].copy_(ring[slot], non_blocking=True)
        e = torch.cuda.Event()
        e.record(copy_stream)
        ring_ev[slot] = e

    def step(i, timed):
        slot = i % 4
        stream.wait_event(ring_ev[slot])              # step i's lengths have landed
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if timed else None
        if timed:
            marks[0].record(stream)
        row = pvb.build_packed_row(len_dev[slot], capacity=T, status=st_row)
        # one event after the build: the timing mark, which also frees the slot
        use_ev[slot] = marks[1] if timed else torch.cuda.Event()
        use_ev[slot].record(stream)
        pvb.varlen_attn_fwd(q, k, v, row["cu"], out=o, lse=lse, workspace=ws_f, status=st_f)
        if timed:
            marks[2].record(stream)
        pvb.varlen_attn_bwd(q, k, v, o, do, lse, row["cu"], dq=dq, dk=dk, dv=dv, workspace=ws_b,
                            status=st_b)
        if timed:
            marks[3].record(stream)
            ev["row"].append((marks[0], marks[1]))
            ev["fwd"].append((marks[1], marks[2]))
            ev["bwd"].append((marks[2], marks[3]))
        plan_and_upload(i + 1)                        # the next step's pack, while this one runs

    if a.copy_mb > 0:
        src = torch.empty(a.copy_mb << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    plan_and_upload(0)
    for i in range(a.warmup):
        step(i, False)
    torch.cuda.synchronize()
    for s in (st_row, st_f, st_b):
        pvb.check_status(s)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(a.warmup + i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    for s in (st_row, st_f, st_b):
        pvb.check_status(s)

    def avg_ms(name):
        return float(np.mean([s.elapsed_time(e) for s, e in ev[name]]))

    # each timed step's device time, packed-row build to the end of the
    # backward (its host planning runs before and overlaps the previous step)
    dev_ms = np.array([r[0].elapsed_time(b[1]) for r, b in zip(ev["row"], ev["bwd"])])
    step_spread = {"median": round(float(np.median(dev_ms)), 4), "p10": round(float(np.percentile(dev_ms, 10)), 4),
                   "p90": round(float(np.percentile(dev_ms, 90)), 4)}

    ms_step = elapsed / a.steps * 1e3
    F = useful_fwd_flops(wl.lengths, H, d)
    value = 3.5 * F / (ms_step * 1e-3) / 1e12
    fwd_ms, bwd_ms, row_ms = avg_ms("fwd"), avg_ms("bwd"), avg_ms("row")
    bwd_tflops = 2.5 * F / (bwd_ms * 1e-3) / 1e12
    fwd_tflops = F / (fwd_ms * 1e-3) / 1e12
    # host planner time alone
    tp = time.perf_counter()
    for _ in range(5):
        pvb.pack_plan_bfd(raw, 8192)
    plan_ms = (time.perf_counter() - tp) / 5 * 1e3

    out = {
        "metric": "varlen causal attn fwd+bwd useful TFLOP/s and % bf16 MFMA peak, T=8192 pack",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bfd_first_pack_T8192_H32_d128", "T": T, "H": H, "head_dim": d,
                   "segments": B, "samples_planned": int(raw.size), "packs": int(n_bins),
                   "passes": "fwd+bwd", "o_dtype": "bf16", "grad_dtype": "f32",
                   "precision": "bf16", "seed": a.seed},
        "pct_bf16_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "useful_flop_per_step": 3.5 * F,
        "breakdown_ms": {"host_bfd_plan": round(plan_ms, 4), "build_packed_row": round(row_ms, 4),
                         "varlen_attn_fwd": round(fwd_ms, 4), "varlen_attn_bwd": round(bwd_ms, 4)},
        "step_device_ms": step_spread,
        "fwd_tflops": round(fwd_tflops, 2),
        "bwd_tflops": round(bwd_tflops, 2),
        "roofline": {"kernel": "varlen_attn_bwd", "bound": "mfma", "achieved": round(bwd_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("varlen_attn_bwd")},
    }

    note(f"main step: {ms_step:.3f} ms per step over {a.steps} steps")
    if not a.no_calls_case:
        c3 = attn_calls(torch, pvb, W, dev, stream, wl, torch.bfloat16, torch.float32, "bf16")
        c3.update({"workload": "bfd_first_pack_T8192_H32_d128", "o_dtype": "bf16", "grad_dtype": "f32",
                   "precision": "bf16"})
        out["first_pack_calls"] = c3
        note("first pack calls done")
    if not a.no_edge_case:
        w5 = W.make(5, seed=a.seed)
        c5 = attn_calls(torch, pvb, W, dev, stream, w5, torch.float32, torch.float32, "split")
        c5.update({"workload": "edge_case_T16384_H16_d128", "seed_used": int(w5.extra["seed_used"]),
                   "o_dtype": "f32", "grad_dtype": "f32", "precision": "split"})
        out["edge_case_pack"] = c5
        note("edge-case pack done")
    if not a.no_hbm_case:
        out["short_pack_fwd"] = short_pack_forward(torch, pvb, W, dev, stream, a.seed)
        note("short pack done")
    if not a.no_long_case:
        out["long_mixed_pack"] = long_mixed_pack(torch, pvb, W, dev, stream, a.seed)
        note("long mixed pack done")
    if not a.no_meta_case:
        out["boundaries_from_positions"] = boundary_compilation(torch, pvb, W, dev, stream, a.seed)
        note("boundaries from positions done")
    if not a.no_loss_case:
        out["packed_loss"] = packed_loss(torch, pvb, dev, stream, a.seed)
        note("packed loss done")
    if not a.no_gqa_case:
        out["grouped_heads"] = grouped_heads(torch, pvb, dev, stream, a.seed)
        note("grouped heads done")
    if not a.no_band_case:
        out["cross_and_window"] = cross_and_window(torch, pvb, dev, stream, a.seed)
        note("cross and window done")
    if not a.no_gdn_case:
        out["gated_delta"] = gated_delta(torch, pvb, W, dev, stream, a.seed)
        out["gated_delta_grouped"] = gated_delta(torch, pvb, W, dev, stream, a.seed, Hk=16)
        note("gated delta done")
        out["gated_delta_backward"] = gated_delta_backward(torch, pvb, W, dev, stream, a.seed)
        note("gated delta backward done")

    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, a.cpu_seconds)
        out["cpu_baseline"]["per_config"] = oracle_per_config(a.seed, raw, first)
        note("cpu baseline done")
    print(json.dumps(out), flush=True)


def short_pack_forward(torch, pvb, W, dev, stream, seed, n_sets=8, reps=200):
    """The short-segment pack (T=4096, 16 segments in [64,512], H=16, d=128,
    forward, O bf16): achieved HBM GB/s of algorithmic bytes.  n_sets input
    sets (536 MB in total, more than the 256 MB last-level cache) rotate so
    that each call starts cold in the caches.  Each timed call is preceded by
    a 30 us spin kernel on the stream, so the GPU is busy while the host
    enqueues the events and the call: the events then bracket device work
    only, not the host's launch latency.  The call passes the host mirror of
    cu_seqlens (the work list is then built on the host and passed with the
    launch); `device_planned` times the same calls without it (items decoded
    from the device cu_seqlens in the kernel)."""
    w = W.make(2, seed=seed)
    T, H, d = w.T, w.H, w.d
    B = len(w.lengths)
    sets = []
    for s in range(n_sets):
        ws = W.random_small(seed * 100 + s, w.lengths, H, d, scale=0.5, backward=False, cfg_tag=2)
        up = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
        sets.append((up(ws.q), up(ws.k), up(ws.v), torch.empty((T, H, d), dtype=torch.bfloat16, device=dev),
                     torch.empty((H, T), dtype=torch.float32, device=dev)))
    hcu = np.concatenate([[0], np.cumsum(w.lengths)]).astype(np.int32)
    cu = torch.tensor(hcu, device=dev)
    wsp = torch.empty(pvb.workspace_bytes(T, H, d, B, False), dtype=torch.uint8, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)

    def run(h_cu):
        for i in range(10):
            q, k, v, o, l = sets[i % n_sets]
            pvb.varlen_attn_fwd(q, k, v, cu, h_cu=h_cu, out=o, lse=l, workspace=wsp, status=st)
        torch.cuda.synchronize()
        times = []
        for i in range(reps):
            q, k, v, o, l = sets[i % n_sets]
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(60_000)
            e0.record(stream)
            pvb.varlen_attn_fwd(q, k, v, cu, h_cu=h_cu, out=o, lse=l, workspace=wsp, status=st)
            e1.record(stream)
            times.append((e0, e1))
        torch.cuda.synchronize()
        pvb.check_status(st)
        return np.array([a.elapsed_time(b) for a, b in times]) * 1e3

    us = run(hcu)
    us_dev = run(None)
    byts = 3 * T * H * d * 2 + T * H * d * 2 + 4 * T * H + 4 * (B + 1)
    F = useful_fwd_flops(w.lengths, H, d)
    med = float(np.median(us))
    return {"workload": "pack_T4096_16seg_H16_d128", "pass": "fwd", "calls": reps, "median_us": round(med, 2),
            "p10_us": round(float(np.percentile(us, 10)), 2), "p90_us": round(float(np.percentile(us, 90)), 2),
            "algorithmic_bytes": byts, "achieved_GBs": round(byts / (med * 1e-6) / 1e9, 1),
            "hbm_frac": round(byts / (med * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "useful_tflops": round(F / (med * 1e-6) / 1e12, 2),
            "traffic": measured_traffic("short_pack_fwd"),
            "device_planned": {"median_us": round(float(np.median(us_dev)), 2),
                               "p10_us": round(float(np.percentile(us_dev, 10)), 2),
                               "p90_us": round(float(np.percentile(us_dev, 90)), 2)}}


def long_mixed_pack(torch, pvb, W, dev, stream, seed, reps=50):
    """The long mixed pack (T=32768: one 16384-token segment, then segments of
    16-1024, H=32, d=128), forward and backward as in the main step (O bf16,
    fp32 gradients, bf16 P/dS): median, p10 and p90 over reps calls, useful
    TFLOP/s at the medians."""
    w = W.make(4, seed=seed)
    r = attn_calls(torch, pvb, W, dev, stream, w, torch.bfloat16, torch.float32, "bf16", reps=reps)
    r.update({"workload": "long_mixed_T32768_H32_d128", "pass": "fwd+bwd",
              "fwd_ms": r["fwd"]["median_ms"], "bwd_ms": r["bwd"]["median_ms"],
              "fwd_bwd_ms": r["fwd_bwd"]["median_ms"]})
    return r


def queued_us(torch, stream, fn, reps):
    """Device time per call with the queue kept full: a spin kernel holds the
    GPU while the calls are enqueued, so they run back to back and the events
    around them see no host launch gaps."""
    torch.cuda.synchronize()
    torch.cuda._sleep(20_000_000)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def timed_calls(torch, stream, parts, warmup=10, reps=50):
    """Median, p10 and p90 (ms) of each part of a call sequence over reps timed
    repetitions after warmup untimed ones; parts is a list of (name, fn), the
    parts run back to back and each is bracketed by HIP events on the launch
    stream."""
    for _ in range(warmup):
        for _, fn in parts:
            fn()
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)]
        marks[0].record(stream)
        for i, (_, fn) in enumerate(parts):
            fn()
            marks[i + 1].record(stream)
        ev.append(marks)
    torch.cuda.synchronize()
    out = {}
    for i, (name, _) in enumerate(parts):
        ms = np.array([m[i].elapsed_time(m[i + 1]) for m in ev])
        out[name] = ms
    out["total"] = np.array([m[0].elapsed_time(m[-1]) for m in ev])
    return out


def pct(ms):
    return {"median_ms": round(float(np.median(ms)), 4), "p10_ms": round(float(np.percentile(ms, 10)), 4),
            "p90_ms": round(float(np.percentile(ms, 90)), 4)}


def attn_calls(torch, pvb, W, dev, stream, w, o_dtype, g_dtype, precision, reps=50):
    """One workload's forward and backward calls timed alone: median, p10 and
    p90 over reps calls after 10 warmups, and useful TFLOP/s at the medians."""
    T, H, d = w.T, w.H, w.d
    B = len(w.lengths)
    up = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v, do = up(w.q), up(w.k), up(w.v), up(w.do)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(w.lengths)]).astype(np.int32), device=dev)
    o = torch.empty((T, H, d), dtype=o_dtype, device=dev)
    lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    grads = [torch.empty((T, H, d), dtype=g_dtype, device=dev) for _ in range(3)]
    gcode = pvb.PVB_F32 if g_dtype == torch.float32 else pvb.PVB_BF16
    wf = torch.empty(pvb.workspace_bytes(T, H, d, B, False), dtype=torch.uint8, device=dev)
    wb = torch.empty(pvb.workspace_bytes(T, H, d, B, True, gcode), dtype=torch.uint8, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    r = timed_calls(torch, stream, [
        ("fwd", lambda: pvb.varlen_attn_fwd(q, k, v, cu, out=o, lse=lse, workspace=wf, status=st,
                                            precision=precision)),
        ("bwd", lambda: pvb.varlen_attn_bwd(q, k, v, o, do, lse, cu, dq=grads[0], dk=grads[1], dv=grads[2],
                                            workspace=wb, status=st, precision=precision))], reps=reps)
    pvb.check_status(st)
    F = useful_fwd_flops(w.lengths, H, d)
    fwd, bwd, tot = (float(np.median(r[n])) for n in ("fwd", "bwd", "total"))
    return {"segments": B, "T": T, "H": H, "head_dim": d, "calls": reps,
            "fwd": pct(r["fwd"]), "bwd": pct(r["bwd"]), "fwd_bwd": pct(r["total"]),
            "fwd_tflops": round(F / (fwd * 1e-3) / 1e12, 2), "bwd_tflops": round(2.5 * F / (bwd * 1e-3) / 1e12, 2),
            "useful_tflops": round(3.5 * F / (tot * 1e-3) / 1e12, 2),
            "pct_bf16_mfma_peak": round(100.0 * 3.5 * F / (tot * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}


def boundary_compilation(torch, pvb, W, dev, stream, seed, reps=50):
    """cu_seqlens compiled back from the long mixed pack's position stream
    (T=32768, one 16384-token segment then segments of 16-1024): one
    single-workgroup launch (128 KB of positions: launch- and latency-bound).
    median_us: one call on an idle GPU, host launch included; queued_us: per
    call with the queue full (outputs reused, nothing allocated)."""
    w = W.make(4, seed=seed)
    T = w.T
    L = torch.tensor(np.asarray(w.lengths, dtype=np.int32), device=dev)
    row = pvb.build_packed_row(L, capacity=T)
    pvb.check_status(row["status"])
    pos = row["pos"]
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    out = pvb.boundaries_from_positions(pos, "zero", status=st)
    for _ in range(5):
        out = pvb.boundaries_from_positions(pos, "zero", status=st, out=out)
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        out = pvb.boundaries_from_positions(pos, "zero", status=st, out=out)
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    q_us = queued_us(torch, stream, lambda i: pvb.boundaries_from_positions(pos, "zero", status=st, out=out), reps)
    pvb.check_status(st)
    n = int(out["n_seg"].item())
    if out["cu"][:n + 1].cpu().tolist() != [0] + np.cumsum(w.lengths).tolist():
        raise RuntimeError("boundaries_from_positions: wrong cu_seqlens")
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    return {"workload": "positions_T32768_long_mixed", "segments": n,
            "median_us": round(float(np.median(ms)) * 1e3, 2),
            "p90_us": round(float(np.percentile(ms, 90)) * 1e3, 2), "queued_us": round(q_us, 2)}


def grouped_heads(torch, pvb, dev, stream, seed, T=8192, H=32, Hk=8, d=128, reps=5):
    """The T=8192 pack (one segment) with 32 query heads over 8 key/value heads
    (grouped heads; the pages give no grouped configuration, this ratio is a
    common one): forward and backward as in the main step (O bf16, fp32
    gradients), useful TFLOP/s counted on the query heads, median of reps."""
    g = torch.Generator(device=dev).manual_seed(seed + 7)
    rnd = lambda *shape: (torch.randn(shape, generator=g, device=dev) * 0.5).to(torch.bfloat16)
    q, k, v, do = rnd(T, H, d), rnd(T, Hk, d), rnd(T, Hk, d), (torch.randn((T, H, d), generator=g, device=dev)).to(torch.bfloat16)
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    o = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    dq = torch.empty((T, H, d), dtype=torch.float32, device=dev)
    dk, dv = (torch.empty((T, Hk, d), dtype=torch.float32, device=dev) for _ in range(2))
    wf = torch.empty(pvb.workspace_bytes(T, H, d, 1, False), dtype=torch.uint8, device=dev)
    wb = torch.empty(pvb.workspace_bytes(T, H, d, 1, True, pvb.PVB_F32), dtype=torch.uint8, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ev = []
    for i in range(2 + reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        pvb.varlen_attn_fwd(q, k, v, cu, out=o, lse=lse, workspace=wf, status=st)
        e[1].record(stream)
        pvb.varlen_attn_bwd(q, k, v, o, do, lse, cu, dq=dq, dk=dk, dv=dv, workspace=wb, status=st)
        e[2].record(stream)
        if i >= 2:
            ev.append(e)
    torch.cuda.synchronize()
    pvb.check_status(st)
    fwd = float(np.median([a.elapsed_time(b) for a, b, _ in ev]))
    bwd = float(np.median([b.elapsed_time(c) for _, b, c in ev]))
    F = useful_fwd_flops([T], H, d)
    return {"workload": "gqa_T8192_H32_Hkv8_d128", "pass": "fwd+bwd", "fwd_ms": round(fwd, 4),
            "bwd_ms": round(bwd, 4), "useful_tflops": round(3.5 * F / ((fwd + bwd) * 1e-3) / 1e12, 2)}


def band_pairs(Lq, Lk, wl, wr):
    """(query, key) pairs a slice of Lq queries over Lk keys uses: query r takes
    keys max(0, r + Lk - Lq - wl) .. min(Lk - 1, r + Lk - Lq + wr), a negative
    bound being open."""
    r = np.arange(Lq, dtype=np.int64)
    hi = np.full(Lq, Lk - 1) if wr < 0 else np.minimum(Lk - 1, r + Lk - Lq + wr)
    lo = np.zeros(Lq, dtype=np.int64) if wl < 0 else np.maximum(0, r + Lk - Lq - wl)
    return float(np.maximum(hi - lo + 1, 0).sum())


def cross_and_window(torch, pvb, dev, stream, seed, H=32, d=128, reps=5):
    """Two band shapes at H=32, d=128 (O bf16, fp32 gradients), forward and
    backward, useful TFLOP/s from the (query, key) pairs each uses (4 d flops
    per pair forward, 2.5 times that backward), median of reps:
      - local causal window of 1024 keys over the T=8192 single-segment pack
        (window (1023, 0), keys = queries);
      - chunked prefill: 4 slices whose last 2048 queries attend to all 8192 of
        their keys with the causal clamp aligned to the bottom right."""
    g = torch.Generator(device=dev).manual_seed(seed + 9)
    res = {}
    for name, lq, lk, win in (("window1024_T8192", [8192], [8192], (1023, 0)),
                              ("prefill_q2048_k8192_x4", [2048] * 4, [8192] * 4, (-1, 0))):
        Tq, Tk = sum(lq), sum(lk)
        rnd = lambda *shape: (torch.randn(shape, generator=g, device=dev) * 0.5).to(torch.bfloat16)
        q, k, v, do = rnd(Tq, H, d), rnd(Tk, H, d), rnd(Tk, H, d), rnd(Tq, H, d) * 2
        hq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
        hk = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
        cq, ck = torch.from_numpy(hq).to(dev), torch.from_numpy(hk).to(dev)
        o = torch.empty((Tq, H, d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((H, Tq), dtype=torch.float32, device=dev)
        dq = torch.empty((Tq, H, d), dtype=torch.float32, device=dev)
        dk, dv = (torch.empty((Tk, H, d), dtype=torch.float32, device=dev) for _ in range(2))
        n = len(lq)
        wf = torch.empty(pvb.cross_workspace_bytes(Tq, Tk, H, d, n, False), dtype=torch.uint8, device=dev)
        wb = torch.empty(pvb.cross_workspace_bytes(Tq, Tk, H, d, n, True), dtype=torch.uint8, device=dev)
        st = torch.zeros(1, dtype=torch.int32, device=dev)
        ev = []
        for i in range(2 + reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            pvb.varlen_cross_attn_fwd(q, k, v, cq, ck, hq, hk, window=win, out=o, lse=lse, workspace=wf, status=st)
            e[1].record(stream)
            pvb.varlen_cross_attn_bwd(q, k, v, o, do, lse, cq, ck, hq, hk, window=win, dq=dq, dk=dk, dv=dv,
                                      workspace=wb, status=st)
            e[2].record(stream)
            if i >= 2:
                ev.append(e)
        torch.cuda.synchronize()
        pvb.check_status(st)
        fwd = float(np.median([a.elapsed_time(b) for a, b, _ in ev]))
        bwd = float(np.median([b.elapsed_time(c) for _, b, c in ev]))
        F = sum(band_pairs(a, b, *win) for a, b in zip(lq, lk)) * 4.0 * d * H
        res[name] = {"window": list(win), "fwd_ms": round(fwd, 4), "bwd_ms": round(bwd, 4),
                     "fwd_tflops": round(F / (fwd * 1e-3) / 1e12, 2),
                     "bwd_tflops": round(2.5 * F / (bwd * 1e-3) / 1e12, 2),
                     "useful_tflops": round(3.5 * F / ((fwd + bwd) * 1e-3) / 1e12, 2)}
    return res


def gated_delta(torch, pvb, W, dev, stream, seed, H=32, d=128, reps=5, Hk=None):
    """Gated delta rule over the long mixed pack (T=32768: one 16384-token
    slice, then slices of 16-1024), H=32, d=128, bf16 O and fp32 final states,
    the state reset at every boundary; g ~ U(-0.1, 0), beta ~ U(0.05, 1), unit
    q and k (Hk query/key heads: H when None, else value heads share them in
    groups).  Each (slice, head) is a chain of 64-token chunks; the default
    evaluation cuts it into groups of 1024 tokens (the workspace call), and
    `one_chain_ms` times the call without a workspace, one chain per (slice,
    head), whose time is set by the longest slice.  Reported per chunk of that
    slice, beside the HBM rate of the algorithmic bytes (q, k, v, g, beta read
    once, O and the final states written once).  Median of reps."""
    lengths = W.lengths_cfg4(seed)
    T, B = int(lengths.sum()), len(lengths)
    g = torch.Generator(device=dev).manual_seed(seed + 11)

    def unit(*shape):
        x = torch.randn(shape, generator=g, device=dev)
        return (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    Hk = H if Hk is None else Hk
    q, k = unit(T, Hk, d), unit(T, Hk, d)
    v = torch.randn((T, H, d), generator=g, device=dev).to(torch.bfloat16)
    gg = torch.rand((T, H), generator=g, device=dev) * -0.1
    bb = torch.rand((T, H), generator=g, device=dev) * 0.95 + 0.05
    hc = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cu = torch.from_numpy(hc).to(dev)
    o = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    ht = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = torch.empty(pvb.gated_delta_fwd_workspace_bytes(T, H, B), dtype=torch.uint8, device=dev)

    def timed(chain):
        for _ in range(2):
            pvb.gated_delta_fwd(q, k, v, gg, bb, cu, out=o, state_out=ht, workspace=ws, chain=chain, status=st)
        torch.cuda.synchronize()
        ev = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pvb.gated_delta_fwd(q, k, v, gg, bb, cu, out=o, state_out=ht, workspace=ws, chain=chain, status=st)
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        pvb.check_status(st)
        return float(np.median([a.elapsed_time(b) for a, b in ev]))
    chain_ms = timed(True)
    ms = timed(False)
    byts = (2 * Hk + 2 * H) * T * d * 2 + 2 * T * H * 4 + B * H * d * d * 4
    chain = int(-(-int(lengths.max()) // 64))
    name = "gdn_long_mixed_T32768_H32_d128" if Hk == H else f"gdn_long_mixed_T32768_H32_Hk{Hk}_d128"
    return {"workload": name, "segments": B, "ms": round(ms, 4), "one_chain_ms": round(chain_ms, 4),
            "workspace_bytes": int(ws.numel()),
            "longest_chain_chunks": chain, "us_per_chunk": round(ms * 1e3 / chain, 3),
            "algorithmic_bytes": byts, "achieved_GBs": round(byts / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def gated_delta_backward(torch, pvb, W, dev, stream, seed, H=32, d=128, reps=5):
    """Backward of the gated delta rule over the long mixed pack (T=32768: one
    16384-token slice, then slices of 16-1024), H=32, d=128, fp32 gradients,
    dO ~ N(0,1) bf16 and a final-state gradient; inputs as in gated_delta.  One
    call recomputes the forward (storing chunk checkpoints) and walks the
    chunks back; reported per chunk of the longest slice's chain, median of reps.
    The training pair is timed beside it: the training forward, which leaves
    the checkpoints in the backward's workspace, and the backward that reads
    them (`train_forward_ms`, `after_forward_ms`), against the plain forward
    (with its workspace) and backward, each pair run back to back
    (`plain_pair_ms`, `train_pair_ms`)."""
    lengths = W.lengths_cfg4(seed)
    T, B = int(lengths.sum()), len(lengths)
    g = torch.Generator(device=dev).manual_seed(seed + 13)

    def unit(*shape):
        x = torch.randn(shape, generator=g, device=dev)
        return (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    q, k = unit(T, H, d), unit(T, H, d)
    v = torch.randn((T, H, d), generator=g, device=dev).to(torch.bfloat16)
    gg = torch.rand((T, H), generator=g, device=dev) * -0.1
    bb = torch.rand((T, H), generator=g, device=dev) * 0.95 + 0.05
    do = torch.randn((T, H, d), generator=g, device=dev).to(torch.bfloat16)
    dht = torch.randn((B, H, d, d), generator=g, device=dev) * 0.1
    hc = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cu = torch.from_numpy(hc).to(dev)
    ws = torch.empty(pvb.gated_delta_bwd_workspace_bytes(T, H, B), dtype=torch.uint8, device=dev)
    wsf = torch.empty(pvb.gated_delta_fwd_workspace_bytes(T, H, B), dtype=torch.uint8, device=dev)
    o = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    ht = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)

    def plain_fwd():
        pvb.gated_delta_fwd(q, k, v, gg, bb, cu, out=o, state_out=ht, workspace=wsf, status=st)

    def plain_bwd():
        pvb.gated_delta_bwd(q, k, v, gg, bb, cu, do, dht=dht, workspace=ws, status=st)

    def train_fwd():
        pvb.gated_delta_fwd(q, k, v, gg, bb, cu, out=o, state_out=ht, workspace=ws, train=True, status=st)

    def after_fwd():
        pvb.gated_delta_bwd(q, k, v, gg, bb, cu, do, dht=dht, workspace=ws, after_fwd=True, status=st)

    def timed(*fns):
        for _ in range(2):
            for fn in fns:
                fn()
        torch.cuda.synchronize()
        ev = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for fn in fns:
                fn()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        pvb.check_status(st)
        return float(np.median([a.elapsed_time(b) for a, b in ev]))
    ms = timed(plain_bwd)
    plain_pair = timed(plain_fwd, plain_bwd)
    train_pair = timed(train_fwd, after_fwd)
    train_f = timed(train_fwd)
    after_b = timed(after_fwd)              # the workspace holds the last training forward's checkpoints
    chain = int(-(-int(lengths.max()) // 64))
    return {"workload": "gdn_bwd_long_mixed_T32768_H32_d128", "segments": B, "ms": round(ms, 4),
            "longest_chain_chunks": chain, "us_per_chunk": round(ms * 1e3 / chain, 3),
            "workspace_bytes": int(ws.numel()), "train_forward_ms": round(train_f, 4),
            "after_forward_ms": round(after_b, 4), "plain_pair_ms": round(plain_pair, 4),
            "train_pair_ms": round(train_pair, 4)}


def packed_loss(torch, pvb, dev, stream, seed, C=8192, V=32768, reps=20):
    """Token-weighted NLL and its logit gradient over the cells of one 8192-token
    row (bf16 logits N(0,1)*2, a vocabulary of 32768 -- the pages fix no model
    vocabulary -- and about 1% of cells excluded): achieved HBM GB/s of
    algorithmic bytes (logits read once, gradient written once, targets, row
    NLL) per call with the queue full and the outputs reused; two 512 MB input
    sets alternate so each call starts cold.  median_us: one call on an idle
    GPU, host launch included."""
    g = torch.Generator(device=dev).manual_seed(seed + 5)
    sets = [(torch.randn((C, V), generator=g, device=dev) * 2).to(torch.bfloat16) for _ in range(2)]
    tg = torch.randint(0, V, (C,), generator=g, device=dev, dtype=torch.int64).to(torch.int32)
    tg[torch.rand((C,), generator=g, device=dev) < 0.01] = -100
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    out = pvb.packed_nll(sets[0], tg, status=st)
    for i in range(3):
        out = pvb.packed_nll(sets[i % 2], tg, status=st, out=out)
    torch.cuda.synchronize()
    ev = []
    for i in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        out = pvb.packed_nll(sets[i % 2], tg, status=st, out=out)
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    q_us = queued_us(torch, stream, lambda i: pvb.packed_nll(sets[i % 2], tg, status=st, out=out), reps)
    pvb.check_status(st)
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    byts = 2 * C * V * 2 + 4 * C + 4 * C
    return {"workload": "nll_C8192_V32768_bf16", "median_us": round(ms * 1e3, 2), "queued_us": round(q_us, 2),
            "algorithmic_bytes": byts, "achieved_GBs": round(byts / (q_us * 1e-6) / 1e9, 1),
            "hbm_frac": round(byts / (q_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}


if __name__ == "__main__":
    main()
