#!/usr/bin/env python3
"""Throughput of the Summaryformer per-block memory on one MI355X.

Workload: the served rollout in steady state -- 28 blocks, 16 heads of 64,
24x42 = 1008 raw tokens + 96 summary tokens per record, Y = 2, W = 24, so
every attention reads 6,528 keys (model card "GTA world model: weights and
inference code": the caption at the top and section "One buffer, no mask").
One step is one frame through all 28 blocks: the all-block eviction, then per
block the record write and the dense attention read, through the C-ABI.
Inputs are seeded N(0,1) bf16 tensors already resident in HBM; the session is
prefilled through frames 0..25 (untimed) and timed frames cycle through 8
seeded frames' inputs while frame ids, slots and evictions advance normally.

Prints one JSON line.  `value` comes from the first timed region; per-kernel
durations come from a second timed region of the same length in which the
library has each kernel it launches stamp two HIP events (its own start and end) on this stream.
The cpu_baseline leg times the fp64 oracle on a bounded sample (rank 0, N=1).
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Summaryformer attn TFLOP/s + frames/s (28 blocks, 6528 keys) vs MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PREFILL = 26                # frames 0..25: from frame 25 on, every read has the full 6,528 keys
RING = 8
SINK_GAP = 5                # Z0 follows the window: rotated when the gap reaches 5 (model card)


def profiled_traffic(profile, source):
    """HBM bytes per launch of a kernel from its committed counter summary, or None.

    The summary records the sha256 of the kernel source it was measured on; a
    kernel changed since then has no valid counter figure."""
    import hashlib
    try:
        text = open(os.path.join(ROOT, profile)).read()
        fields = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line and not line.startswith(" "))
        want = hashlib.sha256(open(os.path.join(ROOT, source), "rb").read()).hexdigest()
        if fields.get("kernel_source_sha256", "").strip() != want:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-sink", action="store_true", help="leave Z0's keys where they are (no streaming sink)")
    ap.add_argument("--no-rope-leg", action="store_true",
                    help="skip the second leg (the same rollout with the library applying the temporal band)")
    ap.add_argument("--no-bias-leg", action="store_true",
                    help="skip the third leg (the same rollout with a recency bias on summary keys)")
    ap.add_argument("--no-long-leg", action="store_true",
                    help="skip the long-horizon leg (24 heads of 128, 46,688 keys per read)")
    ap.add_argument("--no-batched-leg", action="store_true",
                    help="skip the batched leg (8 sessions at fill levels 0..31, one sf_attend per block)")
    ap.add_argument("--no-evict-sweep", action="store_true",
                    help="skip the eviction at 1..112 blocks (fixed cost and streaming rate of the copy)")
    ap.add_argument("--no-heads-leg", action="store_true",
                    help="skip the head-count leg (2/4/8 heads: one GPU's share under head sharding; 20 heads)")
    ap.add_argument("--long-steps", type=int, default=4, help="timed frames of the long-horizon leg")
    return ap.parse_args()


def host_cpu():
    """(logical CPUs this process may run on, CPU model name) of the host."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def cpu_long_block_step(rows_small=16, rows_large=64):
    """The oracle's long-horizon block-step (24 heads of 128, 3,856 query rows, 46,688 keys)
    timed on two subsamples of query rows; the read's fixed part (gathering the 46,688 keys in
    fp64) and its per-row part are fitted from the two and extrapolated to all rows.  The
    buffer is replayed to frame 100 with one frame's K/V written every frame (the read's cost
    does not depend on the values)."""
    import numpy as np
    import sf_inputs
    from oracle import sf_oracle as so
    wl = dict(sf_inputs.WORKLOADS["long"], n_blocks=1)
    g = so.Geometry.from_workload(wl)
    orc = so.MemoryReplay(g)
    q, k, v = (sf_inputs.to_host_bytes(x) for x in sf_inputs.frame_tensors(wl, 0, 0, 0))
    for t in range(101):
        orc.step(t, {0: (k, v)})
    assert orc.n_keys() == 46688
    timing = {}
    for n in (rows_small, rows_large):
        rows = np.arange(0, g.r, g.r // n)[:n]
        start = time.perf_counter()
        orc.attend(0, q, rows=rows)
        timing[n] = time.perf_counter() - start
    per_row = max((timing[rows_large] - timing[rows_small]) / (rows_large - rows_small), 0.0)
    fixed = max(timing[rows_small] - per_row * rows_small, 0.0)
    whole = fixed + per_row * g.r
    return {"seconds_per_block_step": whole, "sample_rows": [rows_small, rows_large],
            "sample_seconds": [round(timing[rows_small], 3), round(timing[rows_large], 3)],
            "flop_per_block_step": 4.0 * g.r * 46688 * 24 * 128, "gflops": 4.0 * g.r * 46688 * 24 * 128 / whole / 1e9,
            "note": f"fp64 attention of {rows_small} and {rows_large} of {g.r} query rows x 24 heads x 128 "
                    f"against 46,688 keys; the fixed part (keys gathered in fp64, {fixed:.2f} s) plus "
                    f"{g.r} x the per-row part ({per_row * 1e3:.1f} ms) extrapolate a whole block-step"}


def cpu_baseline(wl, target_s, sink_gap, long_sample=True):
    """Times the oracle (fp64, numpy) on served block-steps at 6,528 keys; frames/s extrapolated to 28 blocks."""
    import numpy as np
    import sf_inputs
    from oracle import sf_oracle as so
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    nproc, model = host_cpu()
    one = dict(wl, n_blocks=1)
    g = so.Geometry.from_workload(one)
    orc = so.MemoryReplay(g, sink_gap=sink_gap)
    for t in range(PREFILL):
        _, k, v = sf_inputs.frame_tensors(one, 0, 0, t)
        orc.step(t, {0: (sf_inputs.to_host_bytes(k), sf_inputs.to_host_bytes(v))})
    t = PREFILL
    q, k, v = (sf_inputs.to_host_bytes(x) for x in sf_inputs.frame_tensors(one, 0, 0, t))
    start = time.perf_counter()
    n = 0
    while True:
        orc.step(t, {0: (k, v)})
        orc.attend(0, q)
        n += 1
        t += 1
        el = time.perf_counter() - start
        if el >= target_s or n >= 64:
            break
    assert orc.n_keys() == 6528
    per_block_step = el / n
    result = {
        "value": 1.0 / (per_block_step * wl["n_blocks"]),
        "unit": "frames/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{n} served block-steps at 6528 keys (eviction + record copy + fp64 attention of 1104 "
                  f"query rows x 16 heads x 64), {el:.1f} s; frames/s extrapolated to 28 blocks",
        "seconds_per_block_step": per_block_step,
        "gflops": 4.0 * 1104 * 6528 * 16 * 64 / per_block_step / 1e9,
        "threads_used": int(threads),
        "host_logical_cpus": int(nproc),
        "host_cpu_model": model,
    }
    # the same oracle on one core: one more block-step with the BLAS pool held to one thread
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            s1 = time.perf_counter()
            orc.step(t, {0: (k, v)})
            orc.attend(0, q)
            one_core = time.perf_counter() - s1
        result["one_core"] = {"seconds_per_block_step": one_core, "frames_per_s": 1.0 / (one_core * wl["n_blocks"]),
                              "gflops": 4.0 * 1104 * 6528 * 16 * 64 / one_core / 1e9}
    except ImportError:
        pass
    if long_sample:
        result["long_horizon"] = cpu_long_block_step()
    return result


def run_leg(sf, sf_inputs, torch, wl, steps, warmup, setup=None, **cfg_kw):
    """The served rollout on one session of the workload's shape with extra config fields:
    (ms of `steps` timed frames, per-kind kernel times of `steps` more frames, traced)."""
    import ctypes
    nb, R, H, D = wl["n_blocks"], wl["hw"] + wl["x"], wl["n_heads"], wl["head_dim"]
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    sess = sf.Session(sf.make_config(**dict(wl, **cfg_kw)), device=dev)
    if setup is not None:
        setup(sess)
    h = sess.handle
    out = torch.empty((R, H, D), dtype=torch.float32, device=dev)
    for t in range(PREFILL):
        for b in range(nb):
            q, k, v = sf_inputs.frame_tensors(wl, 0, b, t, device=dev)
            sf.sf_step(h, b, t, q, k, v, out, 0.0, stream)
    ring = [[sf_inputs.frame_tensors(wl, 0, b, PREFILL + i, device=dev) for b in range(nb)] for i in range(RING)]
    ptrs = [[(q.data_ptr(), k.data_ptr(), v.data_ptr()) for (q, k, v) in fr] for fr in ring]
    lib, sptr, optr = sf._lib, stream.cuda_stream, out.data_ptr()
    t = PREFILL

    def frames(n):
        nonlocal t
        for _ in range(n):
            fr = ptrs[(t - PREFILL) % RING]
            rc = 0
            for b in range(nb):
                rc |= lib.sf_step(h, b, t, fr[b][0], fr[b][1], fr[b][2], optr, ctypes.c_float(0.0), sptr)
            if rc != 0:
                raise RuntimeError("libsf call failed: " + sf.sf_last_error(h))
            t += 1

    frames(warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    frames(steps)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    sf.sf_profile_enable(h, True)
    frames(steps)
    kt = sf.sf_kernel_times_read(h)
    sf.sf_profile_enable(h, False)
    sess.close()
    return ms, kt


def rope_leg(sf, sf_inputs, torch, wl, sink_gap, steps, warmup, mode="replace"):
    """The same served rollout with the library turning keys at the write and queries at the
    read (level planes, `mode` reading): frames/s and the rotating kernels' durations."""
    R, H, D = wl["hw"] + wl["x"], wl["n_heads"], wl["head_dim"]
    ms, kt = run_leg(sf, sf_inputs, torch, wl, steps, warmup, sink_gap=sink_gap, rope_mode=mode)
    avg = lambda kind: kt[kind][0] / max(kt[kind][1], 1)
    rec_bytes = R * H * D * 2
    write_bytes = 6 * rec_bytes   # K, V and Q read from the caller; K, V written to the slot, Q to the session
    return {
        "rope_mode": mode,
        "frames_per_s": round(steps / (ms * 1e-3), 2),
        "ms_per_step": round(ms / steps, 4),
        "write_kernel": "rope_rows_kernel<true, 12> (K and Q turned, V copied; one launch per sf_step)",
        "write_bytes": write_bytes,
        "write_avg_us": round(avg("write") * 1e3, 3),
        "write_gbps": round(write_bytes / (avg("write") * 1e-3) / 1e9, 1),
        "write_frac_hbm": round(write_bytes / (avg("write") * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "attend_call_us": round((kt["attend"][0] + kt["tail"][0] + kt["combine"][0]) / max(kt["attend"][1], 1) * 1e3,
                                3),
        "write_launches": kt["write"][1], "separate_query_turns": kt["rope"][1],
    }


def bias_leg(sf, sf_inputs, torch, wl, sink_gap, steps, warmup):
    """The same served rollout with a recency bias on summary keys (a seeded N(0, 0.5^2) table
    per head and age): frames/s and the biased read's durations.  That read goes through the
    split-key kernel, after a separate record write."""
    R, H, D = wl["hw"] + wl["x"], wl["n_heads"], wl["head_dim"]
    C = R * (wl["y"] + 2) + (wl["w"] - wl["y"]) * wl["x"]
    tab = sf_inputs.bias_table(wl, 0, 0, 0.5, device="cuda").contiguous()
    ms, kt = run_leg(sf, sf_inputs, torch, wl, steps, warmup, setup=lambda s: s.set_recency_bias(tab),
                     sink_gap=sink_gap, recency_bias=True)
    avg = lambda kind: kt[kind][0] / max(kt[kind][1], 1)
    flop = 4.0 * R * C * H * D
    return {
        "frames_per_s": round(steps / (ms * 1e-3), 2),
        "ms_per_step": round(ms / steps, 4),
        "attn_kernel": "attn_bf16_kernel<64, true> (split-key, per-key bias in the score FMA)",
        "attn_avg_us": round(avg("attend") * 1e3, 3),
        "attn_tflops": round(flop / (avg("attend") * 1e-3) / 1e12, 2),
        "attn_frac_mfma": round(flop / (avg("attend") * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "combine_avg_us": round(avg("combine") * 1e3, 3),
        "write_avg_us": round(avg("write") * 1e3, 3),
        "bias_rows_avg_us": round(avg("bias") * 1e3, 3),
        "bias_rows_launches": kt["bias"][1],
        "attend_launches": kt["attend"][1],
    }


def heads_leg(sf, sf_inputs, torch, wl, sink_gap, steps, warmup, heads=(2, 4, 8, 20)):
    """The served rollout (28 blocks, 6,528 keys per read) with other head counts: 2, 4 and 8
    heads are one GPU's share of the 16 heads under 8-, 4- and 2-way head sharding (every head's
    memory, writes and read stay on its GPU); 20 heads of 64 is the width the model card gives
    its model.  Per head count: frames/s of the share and the stream-K read's durations."""
    R, D = wl["hw"] + wl["x"], wl["head_dim"]
    res = {}
    for H in heads:
        ms, kt = run_leg(sf, sf_inputs, torch, dict(wl, n_heads=H), steps, warmup, sink_gap=sink_gap)
        avg = lambda kind: kt[kind][0] / max(kt[kind][1], 1)
        flop = 4.0 * R * 6528 * H * D
        call = (kt["attend"][0] + kt["tail"][0] + kt["combine"][0]) / max(kt["attend"][1], 1)
        res[str(H)] = {
            "frames_per_s": round(steps / (ms * 1e-3), 2),
            "attn_avg_us": round(avg("attend") * 1e3, 3),
            "attn_tflops": round(flop / (avg("attend") * 1e-3) / 1e12, 2),
            "attn_frac_mfma": round(flop / (avg("attend") * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "attend_call_us": round(call * 1e3, 3),
            "attend_call_frac_mfma": round(flop / (call * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        }
    return {"workload": "served rollout with H heads of 64 (2/4/8: one GPU's share under 8/4/2-way head "
                        "sharding; 20: the model card's width); step = 28 x sf_step", "by_heads": res}


def evict_sweep(sf, sf_inputs, torch, frames=12, blocks=(1, 4, 14, 28, 56, 112)):
    """The all-block eviction at the served shape with 1 to 112 blocks (0.79 to 88 MB moved
    per launch): its duration against its bytes, fitted as a fixed part plus bytes over a
    streaming rate, which shows how much of the 28-block eviction is launch and ramp."""
    wl = sf_inputs.WORKLOADS["rollout"]
    R, H, D, X = wl["hw"] + wl["x"], wl["n_heads"], wl["head_dim"], wl["x"]
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    _, k, v = sf_inputs.frame_tensors(wl, 0, 0, 0, device=dev)
    pts = []
    for nb in blocks:
        sess = sf.Session(sf.make_config(**dict(wl, n_blocks=nb)), device=dev)
        h = sess.handle
        n_t = wl["y"] + 2 + frames
        for t in range(n_t):
            if t == wl["y"] + 2:
                torch.cuda.synchronize()
                sf.sf_profile_enable(h, True)
            if t >= 1:
                sf.sf_evict(h, t, stream)
            for b in range(nb):
                sf.sf_write_record(h, b, t, k, v, stream)
        kt = sf.sf_kernel_times_read(h)
        sf.sf_profile_enable(h, False)
        sess.close()
        us = kt["evict"][0] / max(kt["evict"][1], 1) * 1e3
        pts.append((nb * 2 * 2 * X * H * D * 2, us, kt["evict"][1]))
    # least squares: us = a + bytes / rate
    n = len(pts)
    mx = sum(b for b, _, _ in pts) / n
    my = sum(u for _, u, _ in pts) / n
    sxx = sum((b - mx) ** 2 for b, _, _ in pts)
    slope = sum((b - mx) * (u - my) for b, u, _ in pts) / sxx
    fixed = my - slope * mx
    return {
        "points": [{"blocks": nb, "bytes": b, "avg_us": round(u, 3), "launches": c,
                    "gbps": round(b / (u * 1e-6) / 1e9, 1), "frac_hbm": round(b / (u * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
                   for nb, (b, u, c) in zip(blocks, pts)],
        "fit_fixed_us": round(fixed, 3),
        "fit_stream_gbps": round(1e-3 / slope, 1) if slope > 0 else None,
        "fit_stream_frac_hbm": round(1e-3 / slope / PEAK_HBM_GBPS, 4) if slope > 0 else None,
    }


def long_leg(sf, sf_inputs, torch, steps, warmup=1):
    """The long-horizon workload in steady state: 28 blocks, 24 heads of 128, 45x80 = 3,600 raw
    + 256 summary tokens per record, Y = 4, W = 96, so every read has 46,688 keys.  The session
    is filled through frame 99 with evictions and record writes only (no reads), then each timed
    frame is the all-block eviction plus 28 x sf_step (separate record write, split-key read,
    combine).  Inputs cycle through two seeded frames per block."""
    wl = sf_inputs.WORKLOADS["long"]
    nb, R, H, D, X = wl["n_blocks"], wl["hw"] + wl["x"], wl["n_heads"], wl["head_dim"], wl["x"]
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    sess = sf.Session(sf.make_config(**wl), device=dev)
    h = sess.handle
    ring = [[sf_inputs.frame_tensors(wl, 0, b, i, device=dev) for b in range(nb)] for i in range(2)]
    fill = 100
    for t in range(fill):
        if t >= 1:
            sf.sf_evict(h, t, stream)
        for b in range(nb):
            _, k, v = ring[t % 2][b]
            sf.sf_write_record(h, b, t, k, v, stream)
    out = torch.empty((R, H, D), dtype=torch.float32, device=dev)
    ptrs = [[(q.data_ptr(), k.data_ptr(), v.data_ptr()) for (q, k, v) in fr] for fr in ring]
    lib, sptr, optr = sf._lib, stream.cuda_stream, out.data_ptr()
    t = fill

    def frames(n):
        nonlocal t
        for _ in range(n):
            fr = ptrs[t % 2]
            rc = 0
            for b in range(nb):
                rc |= lib.sf_step(h, b, t, fr[b][0], fr[b][1], fr[b][2], optr, ctypes.c_float(0.0), sptr)
            if rc != 0:
                raise RuntimeError("libsf call failed: " + sf.sf_last_error(h))
            t += 1

    frames(warmup)
    torch.cuda.synchronize()
    assert sess.view()["n_keys"] == 46688
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    frames(steps)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    sf.sf_profile_enable(h, True)
    frames(steps)
    kt = sf.sf_kernel_times_read(h)
    sf.sf_profile_enable(h, False)
    sess.close()
    avg = lambda kind: kt[kind][0] / max(kt[kind][1], 1)
    n_keys = 46688
    flop = 4.0 * R * n_keys * H * D
    call_ms = (kt["attend"][0] + kt["combine"][0]) / max(kt["attend"][1], 1)
    evict_bytes = nb * 2 * 2 * X * H * D * 2
    write_bytes = 2 * 2 * R * H * D * 2
    return {
        "workload": "long horizon, steady state: 28 blocks, 24 heads x 128, 45x80 raw + 256 summary tokens per "
                    "record, Y=4, W=96, 46688 keys per read; step = eviction + 28 x sf_step; no sink",
        "frames_per_s": round(steps / (ms * 1e-3), 3),
        "ms_per_step": round(ms / steps, 3),
        "attn_kernel": "attn_bf16_kernel<128, false> (split-key) + combine_kernel<128>",
        "attn_flop_per_launch": flop,
        "attn_avg_us": round(avg("attend") * 1e3, 2),
        "attn_tflops": round(flop / (avg("attend") * 1e-3) / 1e12, 2),
        "attn_frac_mfma": round(flop / (avg("attend") * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "combine_avg_us": round(avg("combine") * 1e3, 2),
        "attend_call_tflops": round(flop / (call_ms * 1e-3) / 1e12, 2),
        "attend_call_frac_mfma": round(flop / (call_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "evict_bytes": evict_bytes,
        "evict_avg_us": round(avg("evict") * 1e3, 3),
        "evict_gbps": round(evict_bytes / (avg("evict") * 1e-3) / 1e9, 1),
        "evict_frac_hbm": round(evict_bytes / (avg("evict") * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "write_bytes": write_bytes,
        "write_avg_us": round(avg("write") * 1e3, 3),
        "write_gbps": round(write_bytes / (avg("write") * 1e-3) / 1e9, 1),
        "attend_launches": kt["attend"][1], "evict_launches": kt["evict"][1],
    }


def batched_leg(sf, sf_inputs, torch, steps, warmup=2):
    """Eight sessions at the served shape (28 blocks, 16 heads of 64) at fill levels t = 0, 1,
    2, 3, 10, 23, 24, 31 (1,104 .. 6,528 keys, 35,424 in all per block); a step is one
    batched sf_attend per block over all eight (one stream-K launch, tail, combine)."""
    wl = sf_inputs.WORKLOADS["batched"]
    nb, R, H, D = wl["n_blocks"], wl["hw"] + wl["x"], wl["n_heads"], wl["head_dim"]
    levels = wl["frames"]
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    sessions = []
    for si, t_end in enumerate(levels):
        sess = sf.Session(sf.make_config(**wl), device=dev)
        for t in range(t_end + 1):
            if t >= 1:
                sf.sf_evict(sess.handle, t, stream)
            for b in range(nb):
                _, k, v = sf_inputs.frame_tensors(wl, si, b, t, device=dev)
                sf.sf_write_record(sess.handle, b, t, k, v, stream)
        sessions.append(sess)
    qs = [[sf_inputs.frame_tensors(wl, si, b, levels[si], device=dev)[0] for si in range(len(levels))]
          for b in range(nb)]
    outs = [torch.empty((R, H, D), dtype=torch.float32, device=dev) for _ in levels]
    n = len(sessions)
    hs = (ctypes.c_void_p * n)(*[s.handle for s in sessions])
    qarr = [(ctypes.c_void_p * n)(*[q.data_ptr() for q in qs[b]]) for b in range(nb)]
    oarr = (ctypes.c_void_p * n)(*[o.data_ptr() for o in outs])
    lib, sptr = sf._lib, stream.cuda_stream
    keys = [s.view()["n_keys"] for s in sessions]
    flop_block = sum(4.0 * R * kk * H * D for kk in keys)

    def step():
        rc = 0
        for b in range(nb):
            rc |= lib.sf_attend(hs, n, b, qarr[b], oarr, ctypes.c_float(0.0), sptr)
        if rc != 0:
            raise RuntimeError("libsf call failed: " + sf.sf_last_error(sessions[0].handle))

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    # the batch's launches are traced through the first session's handle
    sf.sf_profile_enable(sessions[0].handle, True)
    for _ in range(steps):
        step()
    kt = sf.sf_kernel_times_read(sessions[0].handle)
    sf.sf_profile_enable(sessions[0].handle, False)
    for s in sessions:
        s.close()
    avg = lambda kind: kt[kind][0] / max(kt[kind][1], 1)
    call_ms = (kt["attend"][0] + kt["tail"][0] + kt["combine"][0]) / max(kt["attend"][1], 1)
    return {
        "workload": "8 sessions at the served shape, fill levels t = 0,1,2,3,10,23,24,31 (keys " +
                    "/".join(str(k) for k in keys) + "); step = 28 x one batched sf_attend",
        "keys_per_block": sum(keys),
        "flop_per_block": flop_block,
        "ms_per_step": round(ms / steps, 4),
        "tflops": round(flop_block * nb / (ms / steps * 1e-3) / 1e12, 2),
        "attn_kernel": "attn_sk_kernel<false> (stream-K over all 8 sessions) + attn_tail_kernel + combine_sk_kernel",
        "attn_avg_us": round(avg("attend") * 1e3, 3),
        "attn_tflops": round(flop_block / (avg("attend") * 1e-3) / 1e12, 2),
        "attn_frac_mfma": round(flop_block / (avg("attend") * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "tail_avg_us": round(avg("tail") * 1e3, 3),
        "combine_avg_us": round(avg("combine") * 1e3, 3),
        "attend_call_us": round(call_ms * 1e3, 3),
        "attend_call_frac_mfma": round(flop_block / (call_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "attend_launches": kt["attend"][1],
    }


def lds_copy_calibration(sf, torch, nbytes=64 << 20, reps=10):
    """A copy of known size through LDS with the attention kernels' buffer-to-LDS transfer
    (sf_debug_lds_copy): the reference the counter runs scale FETCH_SIZE by on that path."""
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    sf.sf_debug_lds_copy(dst, src, nbytes)
    torch.cuda.synchronize()
    if not torch.equal(src, dst):
        raise RuntimeError("sf_debug_lds_copy: copy differs from its source")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        sf.sf_debug_lds_copy(dst, src, nbytes)
    e1.record()
    e1.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    return {"kernel": "lds_copy_kernel", "bytes_read": nbytes, "bytes_written": nbytes, "launches": reps + 1,
            "avg_us": round(us, 3), "gbps": round(2 * nbytes / (us * 1e-6) / 1e9, 1)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the memory of one session lives on one "
                                   "device and no multi-GPU path is built; run with --gpus 1"}), flush=True)
        sys.exit(2)

    import torch
    import compressed_memory_kv_amd as sf
    import sf_inputs

    wl = sf_inputs.WORKLOADS["rollout"]
    nb, R, H, D, X = wl["n_blocks"], wl["hw"] + wl["x"], wl["n_heads"], wl["head_dim"], wl["x"]
    sink_gap = 0 if args.no_sink else SINK_GAP
    cfg = sf.make_config(**wl, sink_gap=sink_gap)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sess = sf.Session(cfg, device=dev)
    h = sess.handle
    out = torch.empty((R, H, D), dtype=torch.float32, device=dev)

    # prefill: frames 0..PREFILL-1 through every block (untimed)
    for t in range(PREFILL):
        for b in range(nb):
            q, k, v = sf_inputs.frame_tensors(wl, 0, b, t, device=dev)
            sf.sf_step(h, b, t, q, k, v, out, 0.0, stream)
    ring = [[sf_inputs.frame_tensors(wl, 0, b, PREFILL + i, device=dev) for b in range(nb)] for i in range(RING)]
    torch.cuda.synchronize()

    # Pre-marshalled pointers and pre-created events keep the host ahead of the GPU.
    lib = sf._lib
    sptr = stream.cuda_stream
    ring_ptrs = [[(q.data_ptr(), k.data_ptr(), v.data_ptr()) for (q, k, v) in frame] for frame in ring]
    optr = out.data_ptr()

    def one_frame(t):
        # sf_step per block: the eviction (due at the frame's first block), the record
        # write and the attention read
        frame = ring_ptrs[(t - PREFILL) % RING]
        rc = 0
        for b in range(nb):
            qp, kp, vp = frame[b]
            rc |= lib.sf_step(h, b, t, qp, kp, vp, optr, ctypes.c_float(0.0), sptr)
        if rc != 0:
            raise RuntimeError("libsf call failed: " + sf.sf_last_error(h))

    t = PREFILL
    for _ in range(args.warmup):
        one_frame(t)
        t += 1
    torch.cuda.synchronize()
    assert sess.view()["n_keys"] == 6528

    def timed(steps):
        nonlocal t
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            one_frame(t)
            t += 1
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    # Timed region 1: the step as a caller runs it (the value).
    wall0 = time.perf_counter()
    total_ms = timed(args.steps)
    wall = time.perf_counter() - wall0
    # Timed region 2: the same steps with the library's kernel tracing on (every kernel it
    # launches stamps a start and an end HIP event on this stream).
    sf.sf_profile_enable(h, True)
    traced_ms = timed(args.steps)
    kt = sf.sf_kernel_times_read(h)
    sf.sf_profile_enable(h, False)

    avg = lambda kind: kt[kind][0] / max(kt[kind][1], 1)
    n_keys = 6528
    attn_flop = 4.0 * R * n_keys * H * D
    attn_avg_ms = avg("attend")
    # per attention call: the full-tile kernel plus the tail and combine launches, if any
    call_ms = (kt["attend"][0] + kt["tail"][0] + kt["combine"][0]) / max(kt["attend"][1], 1)
    attn_tflops = attn_flop / (attn_avg_ms * 1e-3) / 1e12
    call_tflops = attn_flop / (call_ms * 1e-3) / 1e12
    row_bytes = H * D * 2
    evict_bytes = nb * 2 * 2 * X * row_bytes   # K and V, read + write, every block
    evict_gbps = evict_bytes / (avg("evict") * 1e-3) / 1e9
    n_t = (D - 4 * (D // 6)) // 2                  # temporal RoPE planes per head
    sink_bytes = nb * R * H * (2 * n_t) * 2 * 2    # Z0 keys' temporal dims, read + write, every block
    frames_per_s = args.steps / (total_ms * 1e-3)

    result = {
        "metric": METRIC,
        "value": round(frames_per_s, 2),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, bf16, resident in HBM)",
        "config": {"workload": "served rollout, steady state: 28 blocks, 16 heads x 64, 24x42 raw + 96 summary "
                               "tokens per record, Y=2, W=24, 6528 keys per read; step = eviction + 28 x "
                               "sf_step (record write fused into the attention launch)" +
                               (f"; Z0 keys rotated forward when the gap reaches {sink_gap} (every "
                                f"{sink_gap - 1} frames)" if sink_gap else ""),
                   "blocks": nb, "heads": H, "head_dim": D, "record_rows": R, "keys": n_keys,
                   "sink_gap": sink_gap},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": profiled_traffic("profiles/attn_sk_kernel.served_rollout.txt",
                                                 "compressed_memory_kv_amd/csrc/sf_attn_sk.hip"),
                     "kernel": "attn_sk_kernel<true> (head_dim-64 attention of sf_step, stream-K)",
                     "flop_per_launch": attn_flop, "avg_launch_us": round(attn_avg_ms * 1e3, 3),
                     "launches": kt["attend"][1]},
        "attn_tflops": round(attn_tflops, 2),
        "attend_call_tflops": round(call_tflops, 2),
        "attend_call_us": round(call_ms * 1e3, 3),
        "evict_gbps": round(evict_gbps, 1),
        "evict_frac_hbm": round(evict_gbps / PEAK_HBM_GBPS, 4),
        "evict_avg_us": round(avg("evict") * 1e3, 3),
        "tail_avg_us": round(avg("tail") * 1e3, 3),
        "sink_launches": kt["sink"][1],
        "sink_avg_us": round(avg("sink") * 1e3, 3),
        "sink_gbps": round(sink_bytes / (avg("sink") * 1e-3) / 1e9, 1) if kt["sink"][1] else None,
        "separate_write_launches": kt["write"][1],   # 0: the attention launch writes the record
        "traced_ms_per_step": round(traced_ms / args.steps, 4),
        "wall_s": round(wall, 3),
    }
    if not args.no_rope_leg:
        result["rope_leg"] = rope_leg(sf, sf_inputs, torch, wl, sink_gap, args.steps, args.warmup)
    if not args.no_bias_leg:
        result["bias_leg"] = bias_leg(sf, sf_inputs, torch, wl, sink_gap, args.steps, args.warmup)
    if not args.no_batched_leg:
        result["batched_leg"] = batched_leg(sf, sf_inputs, torch, args.steps)
    if not args.no_evict_sweep:
        result["evict_sweep"] = evict_sweep(sf, sf_inputs, torch)
    if not args.no_heads_leg:
        result["heads_leg"] = heads_leg(sf, sf_inputs, torch, wl, sink_gap, args.steps, args.warmup)
    if not args.no_long_leg:
        result["long_leg"] = long_leg(sf, sf_inputs, torch, args.long_steps)
    result["lds_copy_calibration"] = lds_copy_calibration(sf, torch)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, sink_gap)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
