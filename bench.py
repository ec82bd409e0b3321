#!/usr/bin/env python3
"""Benchmark of the FP8 scaled-cast hot path on one MI355X.

One step = the per-128-group quantize/dequant round trip on the LLM
activation workload: bf16 x [16384, 7168] (N(0,1), 0.1 % of channels x50)
-> fp8q_cast_per_group128 -> e4m3fn q + float32 scale_inv [16384, 56]
-> fp8q_dequant_per_group128 -> bf16 [16384, 7168].  Inputs are resident in
HBM before the timed region; three buffer sets rotate so that a step does not
re-read what the previous one left in the 256 MB Infinity Cache.

`value` = algorithmic bytes of the step (every byte the method must read and
write, scales included) / wall time per step, in GB/s.  HIP events recorded on
the launch stream give the per-kernel average duration used for the roofline
of the dominant kernel (the group cast): one event before each cast and one
between cast and dequant (the next step's first event closes the dequant).
The events are created with hipEventDisableSystemFence: a timing-only event
then skips the system-scope cache write-back and invalidate that a default
event record performs, which otherwise adds about 3 us to every interval.  The other
hot-path operations (block dequant, per-tensor, per-channel, amax) are timed
on their own workloads after the main loop, with a cache flush between
iterations outside the events, and reported under "rows".

The CPU oracle is timed on the host over the same activation workload
(single-threaded, as written) as a reported baseline.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--no-rows] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E peak, 8 TB/s
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    """Timing events of the HIP runtime that torch (and libfp8q.so) already
    use in this process, created with hipEventDisableSystemFence."""

    def __init__(self):
        import ctypes
        path = [l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l][0]
        hip = ctypes.CDLL(path)
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip, self.ct, self.pool = hip, ctypes, []

    def new(self):
        e = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.pool.append(e)
        return e

    def record(self, e, stream):
        rc = self.hip.hipEventRecord(e, self.ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def us(self, a, b):
        self.hip.hipEventSynchronize(b)
        f = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(f), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value * 1e3

    def close(self):
        for e in self.pool:
            self.hip.hipEventDestroy(e)
        self.pool = []
METRIC = "quantize/dequant GB/s and % of HBM peak, per-128-group bf16→e4m3"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-rows", action="store_true", help="skip the per-row breakdown")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--rows-iters", type=int, default=50)
    return ap.parse_args()


def main():
    args = parse()
    if args.steps < 1 or args.warmup < 0 or args.rows_iters < 1:
        print("bench.py: --steps and --rows-iters must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py: fp8q measures one GPU only; --gpus {args.gpus} is not supported (the row, group and "
              "block kernels would shard by rows with no exchange, so a multi-GPU run is N independent copies)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dequantize_amax_reduce_amd as fq
    from dequantize_amax_reduce_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    st = torch.cuda.Stream(device=dev)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ------------------------------------------------------------------ inputs
    R, C = 16384, 7168
    G = C // 128
    log(f"generating activation workload bf16 [{R}, {C}]")
    xh, _ = W.activation_outlier_channels(rows=R, cols=C, seed=3)
    x0 = torch.from_numpy(xh).view(torch.int16).view(torch.bfloat16).to(dev)
    NSETS = 3
    sets = []
    for i in range(NSETS):
        sets.append(dict(
            x=x0 if i == 0 else x0.clone(),
            q=torch.empty((R, C), dtype=torch.uint8, device=dev),
            s=torch.empty((R, G), dtype=torch.float32, device=dev),
            y=torch.empty((R, C), dtype=torch.bfloat16, device=dev),
        ))
    torch.cuda.synchronize()
    cast_bytes = R * C * 2 + R * C + R * G * 4          # read bf16, write fp8 + scale_inv
    deq_bytes = R * C + R * G * 4 + R * C * 2           # read fp8 + scale_inv, write bf16
    step_bytes = cast_bytes + deq_bytes

    HE = HipEvents()

    def step(i, ev_start=None, ev_mid=None):
        b = sets[i % NSETS]
        if ev_start is not None:
            HE.record(ev_start, st)
        fq.fp8q_cast_per_group128(b["x"], b["q"], b["s"], "e4m3fn", stream=st)
        if ev_mid is not None:
            HE.record(ev_mid, st)
        fq.fp8q_dequant_per_group128(b["q"], b["s"], b["y"], "e4m3fn", stream=st)

    # ------------------------------------------------------------------ main loop
    log(f"warmup {args.warmup}, timed {args.steps} steps")
    ev_start = [HE.new() for _ in range(args.steps + 1)]
    ev_mid = [HE.new() for _ in range(args.steps)]
    with torch.cuda.stream(st):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, ev_start[i], ev_mid[i])
        HE.record(ev_start[args.steps], st)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    cast_us = [HE.us(ev_start[i], ev_mid[i]) for i in range(args.steps)]
    deq_us = [HE.us(ev_mid[i], ev_start[i + 1]) for i in range(args.steps)]
    cast_avg = float(np.mean(cast_us))
    deq_avg = float(np.mean(deq_us))
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    cast_gbps = cast_bytes / (cast_avg * 1e-6) / 1e9
    log(f"step {ms_per_step * 1e3:.1f} us  cast {cast_avg:.1f} us ({cast_gbps:.0f} GB/s)  "
        f"dequant {deq_avg:.1f} us ({deq_bytes / (deq_avg * 1e-6) / 1e9:.0f} GB/s)")

    rows = {
        "group128_cast_bf16_e4m3fn_16384x7168": _row(cast_bytes, cast_us, R * C),
        "group128_dequant_e4m3fn_bf16_16384x7168": _row(deq_bytes, deq_us, R * C),
    }
    # context for the roofline: the cast alone, back to back over the rotating
    # sets with one event pair per batch, i.e. its launch duration without a
    # pair of event records around every launch
    cast_b2b = _back_to_back(HE, st, NSETS, lambda i: fq.fp8q_cast_per_group128(
        sets[i % NSETS]["x"], sets[i % NSETS]["q"], sets[i % NSETS]["s"], "e4m3fn", stream=st))
    # round-trip error of the step's own output (outside the timed region)
    b0 = sets[(args.steps - 1) % NSETS]                 # written by the last timed step
    roundtrip = {"group128_e4m3fn_bf16_16384x7168": _roundtrip_err(
        torch, b0["x"], b0["y"], b0["s"].repeat_interleave(128, dim=1), "e4m3fn", out_rounding="bf16")}

    # ------------------------------------------------------------------ copy calibration
    # a plain device copy of known size: the reference for the HBM counters and a
    # practical ceiling (reported as context, not as the roofline peak)
    cp_n = 256 << 20
    a = torch.empty(cp_n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    with torch.cuda.stream(st):
        for _ in range(3):
            b.copy_(a)
        e0, e1 = HE.new(), HE.new()
        HE.record(e0, st)
        for _ in range(10):
            b.copy_(a)
        HE.record(e1, st)
    torch.cuda.synchronize()
    copy_us = HE.us(e0, e1) / 10
    copy_gbps = 2 * cp_n / (copy_us * 1e-6) / 1e9
    del a, b
    # the same byte volume as one group cast (cast_bytes, half read, half written)
    cv_n = (cast_bytes // 2) // 16 * 16
    a = torch.empty(cv_n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    with torch.cuda.stream(st):
        for _ in range(2):
            b.copy_(a)
        e0, e1 = HE.new(), HE.new()
        HE.record(e0, st)
        for _ in range(5):
            b.copy_(a)
        HE.record(e1, st)
    torch.cuda.synchronize()
    cv_us = HE.us(e0, e1) / 5
    del a, b
    del sets
    torch.cuda.empty_cache()

    # ------------------------------------------------------------------ other rows
    copy_ctx = {}
    if not args.no_rows:
        other, copy_ctx = _other_rows(fq, W, np, torch, dev, st, args.rows_iters, log, HE, x0, roundtrip)
        rows.update(other)
    del x0
    HE.close()

    # ------------------------------------------------------------------ CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        cpu = _cpu_baseline(xh, R, C, G, log)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "per-128-group quantize + dequant round trip: bf16 [16384, 7168] (N(0,1), 7 channels x50) "
                        "-> e4m3fn [16384, 7168] + float32 scale_inv [16384, 56] -> bf16 [16384, 7168]",
            "rows": R, "cols": C, "fp8_format": "e4m3fn", "input": "bf16", "output": "bf16",
            "bytes_per_step": step_bytes, "elements_per_s": round(2 * R * C / (ms_per_step * 1e-3), 1),
            "percent_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
            "buffer_sets_rotated": NSETS,
        },
        "roofline": {
            "kernel": "k_group128 (fp8q_cast_per_group128)",
            "bound": "hbm",
            "achieved": round(cast_gbps, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(cast_gbps / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(),
            "avg_launch_us": round(cast_avg, 3),
            "algorithmic_bytes_per_launch": cast_bytes,
            "back_to_back": _b2b_summary(cast_bytes, cast_b2b),
        },
        "roofline_block_dequant": _block_roofline(rows),
        "copy_reference": {"bytes": 2 * cp_n, "us": round(copy_us, 3), "gbps": round(copy_gbps, 1),
                           "same_volume_as_group_cast": {"bytes": 2 * cv_n, "us": round(cv_us, 3),
                                                          "gbps": round(2 * cv_n / (cv_us * 1e-6) / 1e9, 1)},
                           **{k: {"bytes": v["bytes"], "us": v["avg_us"], "gbps": v["gbps"]}
                              for k, v in copy_ctx.items()}},
        "cpu_baseline": cpu,
        "roundtrip_rel_err": roundtrip,
        "rows": rows,
    }
    print(json.dumps(out), flush=True)


# what the device code is made from: the kernel sources and the build script
# whose flags shape the code object (a change to any of them makes the committed
# counter summary stale)
KERNEL_SOURCES = ("dequantize_amax_reduce_amd/csrc/fp8q_device.h", "dequantize_amax_reduce_amd/csrc/fp8q_kernels.hip",
                  "dequantize_amax_reduce_amd/csrc/fp8q_shift.hip", "dequantize_amax_reduce_amd/csrc/fp8q_host.h",
                  "dequantize_amax_reduce_amd/build.py")
TRAFFIC_SUMMARY = "profiles/fp8q_kernels__bench_workloads__hbm_traffic.md"


def kernel_source_hash() -> str:
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _block_roofline(rows):
    """The metric's second headline kernel, the 128x128 block dequant on the
    weight workload, in the same form as `roofline` (events around each launch
    after a read flush, from the rows)."""
    r = rows.get("block128_dequant_e4m3fn_bf16_18432x7168")
    if r is None:
        return None
    return {"kernel": "k_block128_flat (fp8q_weight_dequant_block128)", "bound": "hbm", "achieved": r["gbps"],
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": r["frac_of_hbm_peak"],
            "traffic": measured_traffic(kernel="k_block128_flat"), "avg_launch_us": r["avg_us"],
            "algorithmic_bytes_per_launch": r["bytes"], "back_to_back": r.get("back_to_back")}


def measured_traffic(path=None, kernel=None):
    """HBM bytes per launch of the group-cast kernel (or of `kernel`, e.g.
    "k_block128_flat") from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, or None when that summary is missing or was taken on different
    kernel sources."""
    import re
    if path is None:
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), TRAFFIC_SUMMARY)
    try:
        text = open(path).read()
    except OSError:
        return None
    src = re.search(r"^kernel_sources_sha256:\s*([0-9a-f]{64})", text, re.M)
    key = "hbm_bytes_per_launch" if kernel is None else re.escape(f"hbm_bytes_per_launch[{kernel}]")
    val = re.search(r"^" + key + r":\s*([0-9.]+)", text, re.M)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


def _back_to_back(HE, st, nsets, fn, batches=5, per=12):
    """Per-launch time of fn(i) launched `per` times back to back (i cycling
    over the rotating buffer sets) between one pair of events; one value per
    batch, after one untimed round."""
    import torch
    us = []
    with torch.cuda.stream(st):
        for i in range(nsets):
            fn(i)
        for _ in range(batches):
            e0, e1 = HE.new(), HE.new()
            HE.record(e0, st)
            for i in range(per):
                fn(i)
            HE.record(e1, st)
            us.append(HE.us(e0, e1) / per)
    return us


def _b2b_summary(nbytes, us_list):
    import numpy as np
    med = float(np.median(us_list))
    return {"median_launch_us": round(med, 3), "min_launch_us": round(float(np.min(us_list)), 3),
            "frac": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "protocol": f"{len(us_list)} batches of back-to-back launches over rotating buffer sets, "
                        "one event pair per batch"}


def _row(nbytes, us_list, elems):
    import numpy as np
    avg = float(np.mean(us_list))
    gbps = nbytes / (avg * 1e-6) / 1e9
    return {"bytes": int(nbytes), "avg_us": round(avg, 3), "median_us": round(float(np.median(us_list)), 3),
            "min_us": round(float(np.min(us_list)), 3),
            "gbps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "elements_per_s": round(elems / (avg * 1e-6), 1)}


FP8_MIN_NORMAL = {"e4m3fn": 2.0 ** -6, "e5m2": 2.0 ** -14}
FP8_MANT_BITS = {"e4m3fn": 3, "e5m2": 2}


def _roundtrip_err(torch, x, y, sinv_elem, fmt, out_rounding="f32"):
    """Largest |y - x| / |x| over the elements whose scaled value |x| / scale_inv
    lies in the fp8 format's normal range (below it the format's spacing is
    absolute, not relative).  The stated tolerance is half an fp8 ulp,
    2^-(mantissa bits + 1): 2^-4 for e4m3fn, 2^-3 for e5m2; a bf16 output
    adds at most one bf16 rounding (2^-8 relative) on top."""
    xd = x.reshape(-1).double()
    yd = y.reshape(-1).double()
    sd = sinv_elem.reshape(-1).double()                  # one value per element, or one for all
    m = (xd.abs() / sd) >= FP8_MIN_NORMAL[fmt]
    rel = ((yd - xd).abs() / xd.abs())[m]
    tol = 2.0 ** -(FP8_MANT_BITS[fmt] + 1)
    out = {"max_rel_err": float(rel.max().item()) if rel.numel() else 0.0, "tolerance": tol,
           "elements_checked": int(m.sum().item()), "elements": int(xd.numel())}
    if out_rounding == "bf16":
        out["tolerance_with_output_rounding"] = (1 + tol) * (1 + 2.0 ** -8) - 1
    out["within"] = out["max_rel_err"] <= out.get("tolerance_with_output_rounding", tol)
    del xd, yd, sd, m, rel
    return out


def _other_rows(fq, W, np, torch, dev, st, iters, log, HE, act, roundtrip):
    """Each remaining hot-path operation on its own workload.  Between
    iterations, outside the events, a 1 GiB read (a max-reduction) replaces the
    256 MB Infinity Cache contents with clean lines, so inputs come from HBM
    and no dirty lines from an earlier write are written back inside the
    timed kernel."""
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    out = {}

    def timed(name, nbytes, elems, fn, into=out):
        with torch.cuda.stream(st):
            fn()
            fn()
            us = []
            e0, e1 = HE.new(), HE.new()
            for _ in range(iters):
                flush.max()
                HE.record(e0, st)
                fn()
                HE.record(e1, st)
                us.append(HE.us(e0, e1))
        into[name] = _row(nbytes, us, elems)
        log(f"{name}: {into[name]['avg_us']} us, {into[name]['gbps']} GB/s")

    # the per-128-group dequant of the step on its own, after a flush: the step
    # runs it right after the cast wrote q, so this row shows what the step's
    # dequant would take with q coming from HBM instead of the Infinity Cache
    Ra, Ca = act.shape
    qa8 = torch.empty((Ra, Ca), dtype=torch.uint8, device=dev)
    sa8 = torch.empty((Ra, Ca // 128), dtype=torch.float32, device=dev)
    ya8 = torch.empty((Ra, Ca), dtype=torch.bfloat16, device=dev)
    with torch.cuda.stream(st):
        fq.fp8q_cast_per_group128(act, qa8, sa8, "e4m3fn", stream=st)
    timed("group128_dequant_e4m3fn_bf16_16384x7168 (flushed, q from HBM)", Ra * Ca + Ra * (Ca // 128) * 4 + Ra * Ca * 2,
          Ra * Ca, lambda: fq.fp8q_dequant_per_group128(qa8, sa8, ya8, "e4m3fn", stream=st))
    del ya8
    # the same cast from views that start two elements into their buffers
    # (x 4-byte aligned, not 16; q 2-byte aligned): the shifted kernel, whose
    # aligned 16-byte loads are re-formed into each lane's elements by a
    # cross-lane shuffle and whose aligned stores straddle two lanes' codes
    xo = torch.empty(Ra * Ca + 2, dtype=torch.bfloat16, device=dev)
    xo[2:].copy_(act.reshape(-1))
    qo = torch.empty(Ra * Ca + 2, dtype=torch.uint8, device=dev)
    xv, qv = xo[2:].view(Ra, Ca), qo[2:].view(Ra, Ca)
    timed("group128_cast_bf16_e4m3fn_16384x7168 (x, q two elements into their buffers: k_group128_shift, "
          "aligned loads re-formed by a lane shuffle)", Ra * Ca * 3 + Ra * (Ca // 128) * 4, Ra * Ca,
          lambda: fq.fp8q_cast_per_group128(xv, qv, sa8, "e4m3fn", stream=st))
    del xo, qo, xv, qv
    # the same cast in the one-wavefront-per-group shape (64 lanes x 2 bf16,
    # 4-byte loads, 2-byte stores) on the aligned buffers, beside the
    # 16-lane / 16-byte k_group128 of the headline row
    timed("group128_cast_bf16_e4m3fn_16384x7168 (one wavefront per group, 64 lanes x 2 bf16: "
          "fp8q_cast_per_group128_wave64)", Ra * Ca * 3 + Ra * (Ca // 128) * 4, Ra * Ca,
          lambda: fq.fp8q_cast_per_group128_wave64(act, qa8, sa8, "e4m3fn", stream=st))

    # the flat paths on the activation's element count, from aligned buffers and
    # from views that start part-way into their buffers (the shifted stream):
    # x and y two elements in, q two bytes in (for fp32 y, one element in)
    na = act.numel()
    xs = torch.empty(na + 8, dtype=torch.bfloat16, device=dev)
    xs[2:2 + na].copy_(act.reshape(-1))
    qs = torch.empty(na + 8, dtype=torch.uint8, device=dev)
    ys = torch.empty(na + 8, dtype=torch.bfloat16, device=dev)
    yf = torch.empty(na + 4, dtype=torch.float32, device=dev)
    s1 = torch.empty(1, dtype=torch.float32, device=dev)
    sr = torch.empty(Ra, dtype=torch.float32, device=dev)
    wsv = torch.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device=dev)
    with torch.cuda.stream(st):
        fq.fp8q_cast_per_channel(act, qa8, sr, "e4m3fn", stream=st)
    views = {"aligned": (act.reshape(-1), qs[:na], ys[:na], yf[:na]),
             "views": (xs[2:2 + na], qs[2:2 + na], ys[2:2 + na], yf[1:1 + na])}
    for tag, (xv, qv, yv, yfv) in views.items():
        timed(f"per_tensor_cast_bf16_e4m3fn_16384x7168 ({tag}, amax pass + cast pass)", na * 5 + 4, na,
              lambda: fq.fp8q_cast_per_tensor(xv, qv, s1, wsv, "e4m3fn", stream=st))
        timed(f"per_tensor_dequant_e4m3fn_bf16_16384x7168 ({tag})", na * 3 + 4, na,
              lambda: fq.fp8q_dequant_per_tensor(qv, s1, yv, "e4m3fn", stream=st))
        timed(f"per_tensor_dequant_e4m3fn_f32_16384x7168 ({tag})", na * 5 + 4, na,
              lambda: fq.fp8q_dequant_per_tensor(qv, s1, yfv, "e4m3fn", stream=st))
        timed(f"group128_dequant_e4m3fn_bf16_16384x7168 ({tag})", na * 3 + Ra * (Ca // 128) * 4, na,
              lambda: fq.fp8q_dequant_per_group128(qv.view(Ra, Ca), sa8, yv.view(Ra, Ca), "e4m3fn", stream=st))
        timed(f"per_channel_cast_bf16_e4m3fn_16384x7168 ({tag})", na * 3 + Ra * 4, na,
              lambda: fq.fp8q_cast_per_channel(xv.view(Ra, Ca), qv.view(Ra, Ca), sr, "e4m3fn", stream=st))
        timed(f"per_channel_dequant_e4m3fn_bf16_16384x7168 ({tag})", na * 3 + Ra * 4, na,
              lambda: fq.fp8q_dequant_per_channel(qv.view(Ra, Ca), sr, yv.view(Ra, Ca), "e4m3fn", stream=st))
    del qa8, sa8, xs, qs, ys, yf, views

    # pipeline p2p cast of the activation (bf16 [16384, 7168]) with the format
    # chosen on the device, and back to bf16
    na = act.numel()
    qa = torch.empty(na, dtype=torch.uint8, device=dev)
    sa = torch.empty(1, dtype=torch.float32, device=dev)
    wa = torch.empty(1, dtype=torch.int32, device=dev)
    wsa = torch.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device=dev)
    ya = torch.empty(na, dtype=torch.bfloat16, device=dev)
    timed("pipeline_cast_bf16_16384x7168 (amax pass + cast pass, format chosen on the device)",
          2 * na * 2 + na + 4 + 4, na, lambda: fq.fp8q_cast_to_fp8_pipeline(act, qa, sa, wa, wsa, stream=st))
    timed("pipeline_dequant_bf16_16384x7168 (format read on the device)", na + 4 + 4 + na * 2, na,
          lambda: fq.fp8q_cast_from_fp8_pipeline(qa, wa, sa, ya, stream=st))
    del qa, sa, wa, wsa, ya

    # 128x128 block weight dequant: e4m3fn [18432, 7168] + float32 [144, 56] -> bf16
    log("block weight workload")
    ch, sh = W.block_weight()
    M, N = ch.shape
    qd = torch.from_numpy(ch).to(dev)
    sd = torch.from_numpy(sh).to(dev)
    yd = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    blk_bytes = M * N + sd.numel() * 4 + M * N * 2
    timed("block128_dequant_e4m3fn_bf16_18432x7168", blk_bytes, M * N,
          lambda: fq.fp8q_weight_dequant_block128(qd, sd, yd, "e4m3fn", stream=st))
    qs, ys = [qd, qd.clone(), qd.clone()], [yd, torch.empty_like(yd), torch.empty_like(yd)]
    out["block128_dequant_e4m3fn_bf16_18432x7168"]["back_to_back"] = _b2b_summary(blk_bytes, _back_to_back(
        HE, st, 3, lambda i: fq.fp8q_weight_dequant_block128(qs[i % 3], sd, ys[i % 3], "e4m3fn", stream=st)))
    del qd, sd, yd, ch, qs, ys

    # per-tensor e5m2 on the 1-D gradient payload bf16 [2^28]
    log("gradient payload workload")
    n = 1 << 28
    gh = W.gradient_payload(n=n)
    gd = torch.from_numpy(gh).view(torch.int16).view(torch.bfloat16).to(dev)
    del gh
    amax = torch.empty(4, dtype=torch.float32, device=dev)
    qg = torch.empty(n, dtype=torch.uint8, device=dev)
    sg = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device=dev)
    yg = torch.empty(n, dtype=torch.float32, device=dev)
    timed("amax_bf16_268435456", n * 2 + 4, n, lambda: fq.fp8q_amax(gd, amax, stream=st))
    timed("per_tensor_cast_bf16_e5m2_268435456 (amax pass + cast pass)", 2 * n * 2 + n + 4, n,
          lambda: fq.fp8q_cast_per_tensor(gd, qg, sg, ws, "e5m2", stream=st))
    timed("per_tensor_dequant_e5m2_f32_268435456", n + 4 + n * 4, n,
          lambda: fq.fp8q_dequant_per_tensor(qg, sg, yg, "e5m2", stream=st))
    torch.cuda.synchronize()
    roundtrip["per_tensor_e5m2_f32_268435456"] = _roundtrip_err(torch, gd, yg, sg, "e5m2")
    # FSDP parameter hook's parts on the same shard: cast with a given (all-reduced)
    # amax, dequant by division by the scale
    yb = torch.empty(n, dtype=torch.bfloat16, device=dev)
    fq.fp8q_amax_guarded(gd, amax, stream=st)
    timed("cast_with_amax_bf16_e5m2_268435456 (FSDP hook, one pass)", n * 2 + n + 8, n,
          lambda: fq.fp8q_cast_with_amax(gd, amax, qg, sg, "e5m2", stream=st))
    timed("dequant_div_scale_e5m2_bf16_268435456 (FSDP hook)", n + 4 + n * 2, n,
          lambda: fq.fp8q_dequant_div_scale(qg, sg, yb, "e5m2", stream=st))
    del yb
    # packed [scale_inv | payload] slots: the whole payload cast into one slot
    # (codes 4 bytes past the header), and 8 slots of 2^25 read back to bf16
    slot = torch.empty(4 + n, dtype=torch.uint8, device=dev)
    timed("packed_cast_bf16_e5m2_268435456 (amax pass + cast pass, codes at slot+4)", 2 * n * 2 + n + 4, n,
          lambda: fq.fp8q_cast_to_packed(gd, slot, ws, "e5m2", stream=st))
    del slot
    Wp, npk = 8, n // 8
    comb = torch.empty(Wp * (4 + npk), dtype=torch.uint8, device=dev)
    for r in range(Wp):
        fq.fp8q_cast_to_packed(gd[r * npk:(r + 1) * npk], comb[r * (4 + npk):(r + 1) * (4 + npk)], ws, "e5m2",
                               stream=st)
    yp = torch.empty((Wp, npk), dtype=torch.bfloat16, device=dev)
    timed("packed_dequant_e5m2_bf16_8x33554432 (all-gather receive side, one launch)",
          Wp * (4 + npk) + Wp * npk * 2, Wp * npk,
          lambda: fq.fp8q_dequant_packed(comb, Wp, npk, yp, "e5m2", stream=st))
    del comb, yp
    del gd, qg, yg

    # reduce step of the fp8-compressed collectives: one rank of 8 holding the
    # 8 received e5m2 chunks of a 2^28-element bf16 gradient bucket (2^25 each)
    log("received-chunks workload")
    Wn, nc = 8, 1 << 25
    ch, sc = W.received_chunks(Wn, nc, "e5m2", seed=6)
    qd = torch.from_numpy(ch).to(dev)
    sd = torch.from_numpy(sc).to(dev)
    del ch
    yd = torch.empty(nc, dtype=torch.bfloat16, device=dev)
    qo = torch.empty(nc, dtype=torch.uint8, device=dev)
    so = torch.empty(1, dtype=torch.float32, device=dev)
    timed("dequant_sum_e5m2_bf16_8x33554432 (reduce-scatter reduce)", Wn * nc + 4 * Wn + 2 * nc, nc,
          lambda: fq.fp8q_dequant_sum(qd, sd, yd, "e5m2", True, stream=st))
    timed("dequant_sum_requant_e5m2_bf16_8x33554432 (all-reduce reduce: sum pass + cast pass)",
          Wn * nc + 4 * Wn + 2 * nc + 2 * nc + nc + 4, nc,
          lambda: fq.fp8q_dequant_sum_requant(qd, sd, yd, qo, so, ws, "e5m2", True, stream=st))
    del qd, yd, qo

    # per-tensor and per-channel on [4096, 4096] fp32 / bf16 with row scales 10**U(-3,3)
    log("row-scaled [4096, 4096] workload")
    xf, xb, _ = W.tensor_rows_scaled()
    R, C = xf.shape
    for dt, xhost in (("f32", xf), ("bf16", xb)):
        if dt == "f32":
            xd = torch.from_numpy(xhost).to(dev)
            esz = 4
        else:
            xd = torch.from_numpy(xhost).view(torch.int16).view(torch.bfloat16).to(dev)
            esz = 2
        q = torch.empty((R, C), dtype=torch.uint8, device=dev)
        s1 = torch.empty(1, dtype=torch.float32, device=dev)
        sr = torch.empty(R, dtype=torch.float32, device=dev)
        y = torch.empty((R, C), dtype=xd.dtype, device=dev)
        for fmt in ("e4m3fn", "e5m2"):        # the configuration covers both formats
            timed(f"per_tensor_cast_{dt}_{fmt}_4096x4096 (2 passes)", 2 * R * C * esz + R * C + 4, R * C,
                  lambda: fq.fp8q_cast_per_tensor(xd, q, s1, ws, fmt, stream=st))
            timed(f"per_tensor_dequant_{fmt}_{dt}_4096x4096", R * C + 4 + R * C * esz, R * C,
                  lambda: fq.fp8q_dequant_per_tensor(q, s1, y, fmt, stream=st))
            timed(f"per_channel_cast_{dt}_{fmt}_4096x4096", R * C * esz + R * C + R * 4, R * C,
                  lambda: fq.fp8q_cast_per_channel(xd, q, sr, fmt, stream=st))
            timed(f"per_channel_dequant_{fmt}_{dt}_4096x4096", R * C + R * 4 + R * C * esz, R * C,
                  lambda: fq.fp8q_dequant_per_channel(q, sr, y, fmt, stream=st))
        del xd, q, y
    # context for the short rows above: torch's device copy of the same byte
    # volumes (half read, half written), timed the same way
    ctx = {}
    for label, nb in (("bf16_4096x4096_rows", 2 * R * C + R * C), ("f32_4096x4096_rows", 4 * R * C + R * C)):
        a = torch.empty(nb // 2, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        timed(f"same_volume_as_{label}", 2 * (nb // 2), 2 * (nb // 2), lambda: b.copy_(a), into=ctx)
        del a, b
    del flush
    torch.cuda.empty_cache()
    return out, ctx


def _cpu_baseline(xh, R, C, G, log):
    """The oracle, as written (single-threaded C, unchanged), on the same
    activation workload: per-group cast then per-group dequant back to bf16 over
    row blocks of 1024.  The value is the median of 3 runs on one thread.  The
    same calls are also spread over the process's CPUs (ctypes releases the
    GIL, and the row blocks are independent), as context."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    oracle.build(force=False)
    L = oracle.default()
    blk = 1024
    blocks = [xh[r:r + blk] for r in range(0, R, blk)]

    def one(xb):
        q, s = L.cast_per_group128(xb, "bf16", "e4m3fn")
        L.dequant_per_group128(q, "e4m3fn", s, "bf16")

    step_bytes = R * (C * 2 + C + G * 4 + C + G * 4 + C * 2)
    log("CPU oracle baseline (1 thread, 3 runs)")
    t1 = []
    for _ in range(3):
        t0 = time.perf_counter()
        for xb in blocks:
            one(xb)
        t1.append(time.perf_counter() - t0)
        if t1[-1] > 15.0:          # a slow host: keep the sample bounded
            break
    nthr = max(1, min(16, len(os.sched_getaffinity(0))))
    log(f"CPU oracle baseline ({nthr} threads, 3 runs)")
    tn = []
    with ThreadPoolExecutor(nthr) as pool:
        for _ in range(3):
            t0 = time.perf_counter()
            list(pool.map(one, blocks))
            tn.append(time.perf_counter() - t0)
    med1, medn = float(np.median(t1)), float(np.median(tn))
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    gbps = step_bytes / med1 / 1e9
    log(f"CPU oracle: {med1:.2f} s on 1 thread -> {gbps:.3f} GB/s; {medn:.2f} s on {nthr} threads")
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole activation workload (bf16 [{R}, {C}]) in row blocks of {blk}, per-group cast + "
                      f"dequant round trip, median of {len(t1)} runs of {med1:.1f} s single-threaded",
            "elements_per_s": round(2 * R * C / med1, 1),
            "parallel": {"value": round(step_bytes / medn / 1e9, 4), "cores": nthr,
                         "note": "the same unchanged oracle calls on independent row blocks, one per thread"},
            "cpu_model": cpu_model, "affinity_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
