#!/usr/bin/env python3
"""Benchmark of the NVFP4 / MXFP4 hot path on one MI355X.

One step = the W4A16 decode GEMV on the 17408 x 5120 NVFP4 weight for M = 1, 4
and 16 bf16 activation rows (the workload the metric is quoted on); `value` is
its algorithmic HBM bytes per second.  The weight sits in the decode layout
(segment-major, the same bytes as the row-major NVFP4 form, rewritten once when
the weight is loaded); the row-major GEMV is timed beside it.  The weight is
held in R rotating copies (R * 50.1 MB > 2 x the 256 MB Infinity Cache) so
every call reads it from HBM.

The same run also times the other kernels of the path on their own workloads
(weight quantize, dequantize, prefill W4A16 and W4A4 at M = 4096, MXFP4-weight
W4A16 decode and prefill, MXFP4 vs NVFP4 W4A4 at M = 8192) with HIP events on the stream they run on, and times the
CPU oracle on a bounded sample of the decode step as a reported baseline.

Prints one JSON line.  `--gpus N` with N > 1 exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NVFP4 GEMM TFLOP/s (prefill) + decode GEMV HBM GB/s, % of roofline"
HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
BF16_PEAK = 2.5e15         # dense bf16 MFMA, FLOP/s
FP4_PEAK = 10.1e15         # dense fp4 MFMA, FLOP/s
FP8_PEAK = 5.0e15          # dense fp8 MFMA (also an fp8 x fp4 product), FLOP/s
N, K = 17408, 5120
# component groups of --only-components / --only
COMPONENT_GROUPS = ["quant", "prefill_m4096", "mxfp4_w4a16", "m8192", "moe"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # a step takes about 38 us: 200 warm-up steps (8 ms) bring the clock to the rate
    # it sustains, and 500 timed steps (19 ms) average over it
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--rotate", type=int, default=12, help="weight copies cycled through")
    ap.add_argument("--trials", type=int, default=5, help="timed repetitions of the K steps (value: their median)")
    ap.add_argument("--comp-iters", type=int, default=20, help="timed launches per component")
    ap.add_argument("--skip-components", action="store_true")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--only-decode", action="store_true", help="decode step only (profiling runs)")
    ap.add_argument("--only-components", action="store_true",
                    help="quantize / dequantize / prefill GEMM components only (profiling runs)")
    ap.add_argument("--only-moe", action="store_true", help="grouped (MoE) GEMM components only (profiling runs)")
    ap.add_argument("--only", choices=COMPONENT_GROUPS, default=None,
                    help="with --only-components: one group of components (profiling runs)")
    ap.add_argument("--ceiling", action="store_true",
                    help="only the fixed-cost / streaming-rate split: a load-only read and the decode GEMV "
                         "at 1x, 2x and 4x the weight bytes")
    ap.add_argument("--ceiling-short", action="store_true",
                    help="with --ceiling: only the read at one workgroup per CU over 1x the bytes and the GEMV "
                         "at K = 5120 (counter runs: one configuration per kernel)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 512 MiB device copy (counter calibration)")
    return ap.parse_args()


def decode_bytes(M):
    return M * K * 2 + N * K // 2 + N * K // 16 + 4 + M * N * 2


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "decode_gemv_k5120_n17408_traffic.json")


def measured_traffic(Ms):
    """HBM bytes per launch (read + write, mean over M) from the committed counter
    summary, or None when the kernel sources changed since the counters were taken."""
    import hashlib

    try:
        d = json.load(open(TRAFFIC_JSON))
        h = hashlib.sha256()
        for f in d["kernel_sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest() != d["sha256"]:
            return None
        per = d["per_M_bytes"]
        return round(sum(per[str(M)]["fetch"] + per[str(M)]["write"] for M in Ms) / len(Ms))
    except (OSError, KeyError, ValueError):
        return None


class Timer:
    """HIP events on torch's current stream, which is the stream the library launches on.
    The timed loops replay library calls recorded by fp4.prepare(): the binding's
    argument checks run once, when a call is prepared, so a short kernel is not timed
    behind the Python that launches it."""

    def __init__(self, torch):
        self.torch = torch
        self.clock = ClockSampler()

    def per_launch(self, fn, iters, warmup=3, warm_s=0.05, sample_clock=False):
        """Seconds per launch over `iters` launches, after `warmup` launches and at
        least `warm_s` seconds of them (so heavy kernels are timed at the clock they
        sustain, not while it ramps up)."""
        torch = self.torch
        t0 = time.perf_counter()
        i = 0
        while i < warmup or (time.perf_counter() - t0 < warm_s and i < 1000):
            fn(i)
            if i >= warmup:
                torch.cuda.synchronize()
            i += 1
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        if sample_clock:
            self.clock.start()
        s.record()
        for i in range(iters):
            fn(i)
        e.record()
        e.synchronize()
        if sample_clock:
            self.clock.stop()
        return s.elapsed_time(e) * 1e-3 / iters   # seconds per launch


class ClockSampler:
    """The shader clock while a timed loop runs, read from the driver's sysfs
    (pp_dpm_sclk: the current level carries a '*') every few ms in a thread.  Empty
    where the file is not readable."""

    def __init__(self):
        import glob

        self.files = [f for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
                      if os.access(f, os.R_OK)]
        self.samples = []
        self._run = False
        self._thread = None

    def _read(self):
        for f in self.files:
            try:
                for line in open(f):
                    if "*" in line:
                        return float(line.split(":")[1].split("Mhz")[0].split("MHz")[0].strip())
            except (OSError, ValueError, IndexError):
                continue
        return None

    def _loop(self):
        while self._run:
            v = self._read()
            if v:
                self.samples.append(v)
            time.sleep(0.002)

    def start(self):
        import threading

        if not self.files:
            return
        self._run = True
        self._thread = threading.Thread(target=self._loop, daemon=True)
        self._thread.start()

    def stop(self):
        self._run = False
        if self._thread is not None:
            self._thread.join()
            self._thread = None

    def median_mhz(self):
        return float(np.median(self.samples)) if self.samples else None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; multi-GPU runs are not part of "
                                   "this build (the GEMM would shard by weight rows, see the design notes)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import block_scaled_fp4_04_amd as fp4
    from synthetic import WORKLOADS

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T = Timer(torch)

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel()}))
        return

    if args.ceiling:
        print(json.dumps(ceiling(args, torch, fp4, T, dev)))
        return

    if args.only_moe:
        print(json.dumps({"components": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                                                for kk, vv in v.items()}
                                         for k, v in moe_components(args, torch, fp4, T, dev).items()}}))
        return

    wl = WORKLOADS["decode_gemv_k5120_n17408"]
    log("generating decode weights 17408x5120 fp32 ...")
    w_np = wl.weights()
    w32 = torch.from_numpy(w_np).to(dev)
    wq = fp4.nvfp4_quantize(w32)
    torch.cuda.synchronize()
    if args.only_components:
        print(json.dumps({"components": components(args, torch, fp4, T, dev, w32, wq)}))
        return

    R = max(1, args.rotate)
    copies = [wq] + [fp4.PackedNVFP4(wq.codes.clone(), wq.scales.clone(), wq.tscale.clone(), N, K)
                     for _ in range(R - 1)]
    dcopies = [fp4.nvfp4_pack_decode(c) for c in copies]
    torch.cuda.synchronize()
    acts = {M: torch.from_numpy(wl.activations_bf16(M).view(np.int16)).view(torch.bfloat16).to(dev)
            for M in wl.M}
    outs = {M: torch.empty(M, N, dtype=torch.bfloat16, device=dev) for M in wl.M}
    # the library calls of every (weight copy, M), prepared once (checks made then)
    dec_calls = {(c, M): fp4.prepare(lambda c=c, M=M: fp4.gemm_w4a16_decode(acts[M], dcopies[c], out=outs[M]))
                 for c in range(R) for M in wl.M}

    # every GEMV call reads its own weight copy (12 x 50 MB > the 256 MB Infinity
    # Cache), as the distinct layers of a decode step would: no call finds its
    # weights in a cache
    def step(i):
        for j, M in enumerate(wl.M):
            dec_calls[((len(wl.M) * i + j) % R, M)]()

    # ------------------------------------------------------------ the step --
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    trials = []
    for _ in range(args.trials):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(args.steps):
            step(i)
        e.record()
        e.synchronize()
        trials.append(s.elapsed_time(e) / args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = float(np.median(trials))
    step_bytes = sum(decode_bytes(M) for M in wl.M)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    assert torch.isfinite(outs[16].float()).all()

    # per-launch durations of the decode kernel, each M on its own (launches back
    # to back on the library's stream; this agrees with a kernel trace's durations)
    dec, dec_rm = {}, {}
    it = max(args.steps, 30)
    for M in wl.M:
        t = T.per_launch(lambda i, M=M: dec_calls[(i % R, M)](), iters=it, warmup=5)
        dec[M] = {"us": t * 1e6, "GB/s": decode_bytes(M) / t / 1e9,
                  "frac_hbm": decode_bytes(M) / t / HBM_PEAK, "bytes": decode_bytes(M)}
        if not args.only_decode:
            rm = [fp4.prepare(lambda c=c, M=M: fp4.gemm_w4a16(acts[M], copies[c], out=outs[M])) for c in range(R)]
            t = T.per_launch(lambda i: rm[i % R](), iters=it, warmup=5)
            dec_rm[M] = {"us": t * 1e6, "GB/s": decode_bytes(M) / t / 1e9,
                         "frac_hbm": decode_bytes(M) / t / HBM_PEAK}
    mean_bytes = sum(decode_bytes(M) for M in wl.M) / len(wl.M)
    mean_t = sum(dec[M]["us"] for M in wl.M) / len(wl.M) * 1e-6
    achieved = mean_bytes / mean_t / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": round(achieved * 1e9 / HBM_PEAK, 4), "traffic": measured_traffic(wl.M),
                "kernel": "k_nv_gemv_dec (W4A16 decode GEMV on the decode layout, M in {1,4,16})",
                "bytes_per_launch_mean": mean_bytes, "us_per_launch_mean": round(mean_t * 1e6, 3),
                "timing": "HIP events around back-to-back launches on the library's stream, mean over M in {1,4,16}"}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_gemv_k5120_n17408", "M": list(wl.M), "K": K, "N": N,
                   "weights": "NVFP4 (E2M1, E4M3 per 16, fp32 per tensor) from N(0,0.02^2), 0.1% x20",
                   "weight_layout": "decode layout (segment-major [K/128][N][64] codes, [K/128][N][8] scales)",
                   "activations": "bf16 N(0,1)", "output": "bf16",
                   "weight_copies_rotated": R, "wall_s_timed_region": round(wall, 4)},
        "trials": {"n": args.trials, "ms_per_step": [round(t, 5) for t in trials],
                   "value_is": "median over the trials of the step time"},
        "roofline": roofline,
        "decode_per_M": {str(M): {k: round(v, 4) if isinstance(v, float) else v for k, v in d.items()}
                         for M, d in dec.items()},
        "decode_row_major_per_M": {str(M): {k: round(v, 4) for k, v in d.items()} for M, d in dec_rm.items()}
        if dec_rm else None,
    }

    if not args.only_decode and not args.skip_components:
        result["components"] = components(args, torch, fp4, T, dev, w32, wq)
        mhz = T.clock.median_mhz()
        result["sclk"] = {"median_mhz_during_gemm_loops": mhz, "samples": len(T.clock.samples),
                          "spec_mhz": 2400.0,
                          "note": "fractions of peak in the components are at 2.4 GHz; *_frac_at_sclk "
                                  "rescale the MFMA peaks to the sampled clock" if mhz else
                                  "the driver's clock file was not readable: no clock samples"}
        if mhz:
            for comp in result["components"].values():
                for k in list(comp):
                    if "frac" in k and "mfma" in k and isinstance(comp[k], float):
                        comp[k + "_at_sclk"] = round(comp[k] * 2400.0 / mhz, 4)

    if not args.only_decode and not args.skip_cpu:
        result["cpu_baseline"] = cpu_baseline(wl, wq, w_np)

    print(json.dumps(result))


def prepared(fp4, thunk):
    """A timing loop body that replays the library calls of `thunk` (see fp4.prepare)."""
    call = fp4.prepare(thunk)
    return lambda i: call()


def ceiling(args, torch, fp4, T, dev):
    """Per-launch time against bytes per launch, at 1x, 2x and 4x the decode weight's
    50.1 MB: for a load-only kernel that reads the bytes once and does nothing else
    (fp4.read_ceiling), and for the decode GEMV at K = 3072, 5120 and 8192.  A
    straight-line fit splits each into a fixed cost per launch (the intercept) and a
    streaming rate (the slope).  Every launch reads its own copy from a rotation
    whose total exceeds twice the 256 MB Infinity Cache."""
    R = max(4, args.rotate)
    wbytes = N * K // 2 + N * K // 16
    it = max(args.steps, 100)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    res = {"workload": "read: the decode weight's bytes (N = 17408, K = 5120: codes + scales) x {1, 2, 4}; "
                       "GEMV: N = 17408 at K = 3072, 5120, 8192",
           "rotated_copies": R, "launches_timed": it, "read": {}, "gemv": {}}

    def fit(xs, ys):
        b, a = np.polyfit(np.asarray(xs, float), np.asarray(ys, float), 1)
        return {"fixed_us": round(float(a), 3), "stream_TBps": round(1e-6 / float(b), 3)}  # b: us per byte

    short = args.ceiling_short
    for grid in ((256,) if short else (256, 512, 1024, 2048)):  # 1, 2, 4, 8 workgroups of 8 waves per CU
        xs, ys = [], []
        for mult in ((1,) if short else (1, 2, 4)):
            bufs = [torch.randint(0, 256, (wbytes * mult,), dtype=torch.uint8, device=dev) for _ in range(R)]
            calls = [fp4.prepare(lambda b=b: fp4.read_ceiling(b, grid, sink)) for b in bufs]
            t = T.per_launch(lambda i: calls[i % R](), iters=it, warmup=5)
            res["read"][f"grid{grid}_x{mult}"] = {"bytes": wbytes * mult, "us": round(t * 1e6, 3),
                                                  "TBps": round(wbytes * mult / t / 1e12, 3),
                                                  "frac_hbm": round(wbytes * mult / t / HBM_PEAK, 4)}
            xs.append(wbytes * mult)
            ys.append(t * 1e6)
            del bufs, calls
            torch.cuda.empty_cache()
        if not short:
            res["read"][f"grid{grid}_fit"] = fit(xs, ys)

    # the GEMV grows along K (K = 3072, 5120, 8192: 3, 5 and 8 of the 128-element
    # segments per wave, 8192 the largest K walked in one chunk), so its launch
    # geometry (218 workgroups of 80 weight rows) stays the same and only the bytes
    # per row grow
    g = torch.Generator(device="cpu").manual_seed(7)
    for M in (1, 16):
        xs, ys = [], []
        for k in ((5120,) if short else (3072, 5120, 8192)):
            a = (torch.randn(M, k, generator=g)).to(torch.bfloat16).to(dev)
            w = fp4.nvfp4_quantize((torch.randn(N, k, generator=g) * 0.02).to(dev))
            d0 = fp4.nvfp4_pack_decode(w)
            del w
            ds = [d0] + [fp4.DecodeNVFP4(d0.codes.clone(), d0.scales.clone(), d0.tscale, N, k) for _ in range(R - 1)]
            out = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            calls = [fp4.prepare(lambda d=d: fp4.gemm_w4a16_decode(a, d, out=out)) for d in ds]
            t = T.per_launch(lambda i: calls[i % R](), iters=it, warmup=5)
            b = M * k * 2 + N * k // 2 + N * k // 16 + 4 + M * N * 2
            res["gemv"][f"M{M}_K{k}"] = {"K": k, "bytes": b, "us": round(t * 1e6, 3),
                                            "TBps": round(b / t / 1e12, 3), "frac_hbm": round(b / t / HBM_PEAK, 4)}
            assert torch.isfinite(out.float()).all()
            xs.append(b)
            ys.append(t * 1e6)
            del ds, calls, d0, out
            torch.cuda.empty_cache()
        if not short:
            res["gemv"][f"M{M}_fit"] = fit(xs, ys)
    return res


def components(args, torch, fp4, T, dev, w32, wq):
    from synthetic import WORKLOADS

    it = args.comp_iters
    out = {}
    want = lambda grp: args.only in (None, grp)  # noqa: E731
    wl3 = WORKLOADS["prefill_w4a16_m4096"]

    if want("quant"):
        quant_components(fp4, T, dev, w32, wq, it, out)
    if want("prefill_m4096"):
        prefill_components(torch, fp4, T, dev, wq, wl3, it, out)
    if want("mxfp4_w4a16"):
        mx16_components(torch, fp4, T, dev, w32, wl3, it, out)
    if want("m8192"):
        m8192_components(torch, fp4, T, dev, w32, it, out)
    if want("moe"):
        out.update(moe_components(args, torch, fp4, T, dev))
    return {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
            for k, v in out.items()}


def quant_components(fp4, T, dev, w32, wq, it, out):
    import torch

    from synthetic import WORKLOADS

    # C1: the tiny round trip (256 x 256 fp32 weight quantized per tensor,
    # dequantized, W4A16 GEMM with 4 bf16 rows, fp32 out): latency of each call
    wl1 = WORKLOADS["tiny_roundtrip_256"]
    w1 = torch.from_numpy(wl1.weights()).to(dev)
    a1 = torch.from_numpy(wl1.activations_bf16(4).view(np.int16)).view(torch.bfloat16).to(dev)
    p1 = fp4.nvfp4_quantize(w1)
    y1 = torch.empty(256, 256, dtype=torch.float32, device=dev)
    c1 = torch.empty(4, 256, dtype=torch.float32, device=dev)
    ws1 = torch.empty(fp4.lib().nvfp4_quantize_workspace(256, 256, 0), dtype=torch.uint8, device=dev)
    t_q1 = T.per_launch(prepared(fp4, lambda: fp4.nvfp4_quantize(w1, out=p1, workspace=ws1)), it)
    t_d1 = T.per_launch(prepared(fp4, lambda: fp4.nvfp4_dequantize(p1, out=y1)), it)
    t_g1 = T.per_launch(prepared(fp4, lambda: fp4.gemm_w4a16(a1, p1, out=c1)), it)
    chain = fp4.prepare(lambda: (fp4.nvfp4_quantize(w1, out=p1, workspace=ws1), fp4.nvfp4_dequantize(p1, out=y1),
                                 fp4.gemm_w4a16(a1, p1, out=c1)))
    t_all1 = T.per_launch(lambda i: chain(), it)
    out["c1_tiny_roundtrip_256"] = {
        "quantize_us": t_q1 * 1e6, "dequantize_us": t_d1 * 1e6, "gemm_w4a16_us": t_g1 * 1e6,
        "all_three_us": t_all1 * 1e6,
        "note": "latency per call, back-to-back launches (the configuration is a correctness case)"}

    # weight quantize (fp32 -> NVFP4, per tensor: amax pass + quantize pass)
    w32b = w32.clone()   # two fp32 copies (712 MB) exceed the Infinity Cache
    ws = torch.empty(fp4.lib().nvfp4_quantize_workspace(N, K, 0), dtype=torch.uint8, device=dev)
    qo = fp4.PackedNVFP4(torch.empty_like(wq.codes), torch.empty_like(wq.scales),
                         torch.empty_like(wq.tscale), N, K)
    srcs = [w32, w32b]
    pq = [fp4.prepare(lambda x=x: fp4.nvfp4_quantize(x, out=qo, workspace=ws)) for x in srcs]
    t = T.per_launch(lambda i: pq[i % 2](), it)
    b = 2 * N * K * 4 + N * K // 2 + N * K // 16 + 4
    out["weight_quantize_fp32_17408x5120"] = {"us": t * 1e6, "GB/s": b / t / 1e9,
                                              "frac_hbm": b / t / HBM_PEAK, "bytes": b}
    del w32b

    # dequantize to bf16
    y = torch.empty(N, K, dtype=torch.bfloat16, device=dev)
    t = T.per_launch(prepared(fp4, lambda: fp4.nvfp4_dequantize(wq, out=y)), it)
    b = N * K // 2 + N * K // 16 + 4 + N * K * 2
    out["dequantize_bf16_17408x5120"] = {"us": t * 1e6, "GB/s": b / t / 1e9,
                                         "frac_hbm": b / t / HBM_PEAK, "bytes": b}
    del y

    # per-row activation quantize (bf16 -> NVFP4, one tensor scale per row), 4096 x
    # 5120, on 8 rotating copies (336 MB > the 256 MB Infinity Cache): the kernel
    # reads its input from HBM, as its counters show
    Ma = 4096
    acts = [torch.randn(Ma, K, dtype=torch.float32, device=dev).to(torch.bfloat16) for _ in range(8)]
    pa = fp4.PackedNVFP4(torch.empty(Ma, K // 2, dtype=torch.uint8, device=dev),
                         torch.empty(Ma, K // 16, dtype=torch.uint8, device=dev),
                         torch.empty(Ma, dtype=torch.float32, device=dev), Ma, K, True)
    pr = [fp4.prepare(lambda x=x: fp4.nvfp4_quantize(x, mode="row", out=pa)) for x in acts]
    t = T.per_launch(lambda i: pr[i % 8](), max(it, 40))
    b = Ma * K * 2 + Ma * K // 2 + Ma * K // 16 + 4 * Ma
    out["activation_quantize_rows_bf16_4096x5120_cold"] = {"us": t * 1e6, "GB/s": b / t / 1e9,
                                                           "frac_hbm": b / t / HBM_PEAK, "bytes": b}
    # MXFP4 quantize of the 8192 x 5120 bf16 activation (E8M0 per 32), cold as above
    acts = [torch.randn(2 * Ma, K, dtype=torch.float32, device=dev).to(torch.bfloat16) for _ in range(4)]
    pm = fp4.PackedMXFP4(torch.empty(2 * Ma, K // 2, dtype=torch.uint8, device=dev),
                         torch.empty(2 * Ma, K // 32, dtype=torch.uint8, device=dev), 2 * Ma, K)
    pr = [fp4.prepare(lambda x=x: fp4.mxfp4_quantize(x, out=pm)) for x in acts]
    t = T.per_launch(lambda i: pr[i % 4](), max(it, 40))
    b = 2 * Ma * K * 2 + 2 * Ma * K // 2 + 2 * Ma * K // 32
    out["mxfp4_quantize_bf16_8192x5120_cold"] = {"us": t * 1e6, "GB/s": b / t / 1e9,
                                                 "frac_hbm": b / t / HBM_PEAK, "bytes": b}
    # MXFP4 dequantize of that tensor to bf16
    y = torch.empty(2 * Ma, K, dtype=torch.bfloat16, device=dev)
    t = T.per_launch(prepared(fp4, lambda: fp4.mxfp4_dequantize(pm, out=y)), it)
    b = 2 * Ma * K // 2 + 2 * Ma * K // 32 + 2 * Ma * K * 2
    out["mxfp4_dequantize_bf16_8192x5120"] = {"us": t * 1e6, "GB/s": b / t / 1e9,
                                              "frac_hbm": b / t / HBM_PEAK, "bytes": b}
    del acts, pr, y


def prefill_components(torch, fp4, T, dev, wq, wl3, it, out):
    # prefill W4A16 and W4A4 at M = 4096
    M = 4096
    a = torch.from_numpy(wl3.activations_bf16(M).view(np.int16)).view(torch.bfloat16).to(dev)
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    fl = 2.0 * M * N * K
    t = T.per_launch(prepared(fp4, lambda: fp4.gemm_w4a16(a, wq, out=c)), it, sample_clock=True)
    # the same GEMMs on the weight in the decode layout (one packed weight for decode and prefill)
    wd = fp4.nvfp4_pack_decode(wq)
    t_d = T.per_launch(prepared(fp4, lambda: fp4.gemm_w4a16_decode(a, wd, out=c)), it)
    # yardstick: the same product as a dense bf16 GEMM in the vendor library
    # (torch.matmul -> hipBLASLt), the weight already widened to bf16 in HBM
    wb16 = fp4.nvfp4_dequantize(wq, torch.bfloat16)
    t_ref = T.per_launch(lambda i: torch.matmul(a, wb16.t(), out=c), it)
    del wb16
    out["prefill_w4a16_m4096"] = {"us": t * 1e6, "TFLOP/s": fl / t / 1e12, "frac_bf16_mfma": fl / t / BF16_PEAK,
                                  "decode_layout_us": t_d * 1e6, "decode_layout_TFLOP/s": fl / t_d / 1e12,
                                  "decode_layout_frac_bf16_mfma": fl / t_d / BF16_PEAK,
                                  "dense_bf16_library_us": t_ref * 1e6,
                                  "dense_bf16_library_frac_bf16_mfma": fl / t_ref / BF16_PEAK,
                                  "flop": fl, "mfma": "bf16 32x32x16 (NVFP4 widened exactly to bf16)"}
    # activation quantization alone (per row) and the fused W4A4 call
    wsa = fp4.gemm_w4a4_workspace(M, K, "row", dev)
    pa = fp4.w4a4_packed_a(wsa, M, K, "row")
    t_q = T.per_launch(prepared(fp4, lambda: fp4.nvfp4_quantize(a, mode="row", out=pa)), it)
    bq = M * K * 2 + M * K // 2 + M * K // 16 + 4 * M
    # the same on inputs that are not in any cache: 8 rotating copies (336 MB > the
    # 256 MB Infinity Cache); the figure above is the activation as a previous
    # kernel leaves it, resident in the Infinity Cache
    a_cold = [a.clone() for _ in range(8)]
    pq = [fp4.prepare(lambda x=x: fp4.nvfp4_quantize(x, mode="row", out=pa)) for x in a_cold]
    t_qc = T.per_launch(lambda i: pq[i % 8](), max(it, 40))
    del a_cold, pq
    t_g = T.per_launch(prepared(fp4, lambda: fp4.gemm_nvfp4_prequant(pa, wq, out=c)), it, sample_clock=True)
    t_all = T.per_launch(prepared(fp4, lambda: fp4.gemm_w4a4(a, wq, a_mode="row", out=c, workspace=wsa)), it)
    t_gd = T.per_launch(prepared(fp4, lambda: fp4.gemm_nvfp4_prequant_seg(pa, wd, out=c)), it)
    t_alld = T.per_launch(prepared(fp4, lambda: fp4.gemm_w4a4_seg(a, wd, a_mode="row", out=c, workspace=wsa)), it)
    out["prefill_w4a4_m4096"] = {
        "quant_us": t_q * 1e6, "quant_GB/s": bq / t_q / 1e9, "quant_frac_hbm": bq / t_q / HBM_PEAK,
        "quant_cold_us": t_qc * 1e6, "quant_cold_GB/s": bq / t_qc / 1e9, "quant_cold_frac_hbm": bq / t_qc / HBM_PEAK,
        "quant_bytes": bq,
        "gemm_us": t_g * 1e6, "gemm_TFLOP/s": fl / t_g / 1e12, "gemm_frac_bf16_mfma": fl / t_g / BF16_PEAK,
        "total_us": t_all * 1e6, "total_TFLOP/s": fl / t_all / 1e12,
        "decode_layout_gemm_us": t_gd * 1e6, "decode_layout_gemm_TFLOP/s": fl / t_gd / 1e12,
        "decode_layout_total_us": t_alld * 1e6}
    del a, c, wd


def mx16_components(torch, fp4, T, dev, w32, wl3, it, out):
    from synthetic import WORKLOADS

    # MXFP4 weights with bf16 activations (W4A16): decode GEMV at M = 1, 4, 16 on
    # the MXFP4 decode layout (12 rotating copies, as the NVFP4 step) and the
    # prefill GEMM at M = 4096
    wmx = fp4.mxfp4_quantize(w32)
    mcopies = [fp4.mxfp4_pack_decode(fp4.PackedMXFP4(wmx.codes.clone(), wmx.scales.clone(), N, K))
               for _ in range(12)]
    wl2 = WORKLOADS["decode_gemv_k5120_n17408"]
    mxd = {}
    for M in wl2.M:
        am = torch.from_numpy(wl2.activations_bf16(M).view(np.int16)).view(torch.bfloat16).to(dev)
        om = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        pm = [fp4.prepare(lambda c=c, am=am, om=om: fp4.mxfp4_gemm_w4a16_decode(am, c, out=om)) for c in mcopies]
        t = T.per_launch(lambda i, pm=pm: pm[i % 12](), max(it, 30), warmup=5)
        b = M * K * 2 + N * K // 2 + N * K // 32 + M * N * 2
        mxd[str(M)] = {"us": round(t * 1e6, 4), "GB/s": round(b / t / 1e9, 1), "frac_hbm": round(b / t / HBM_PEAK, 4),
                       "bytes": b}
    out["mxfp4_w4a16_decode_k5120_n17408"] = mxd
    md0 = mcopies[0]
    del mcopies
    a = torch.from_numpy(wl3.activations_bf16(4096).view(np.int16)).view(torch.bfloat16).to(dev)
    c = torch.empty(4096, N, dtype=torch.bfloat16, device=dev)
    fl = 2.0 * 4096 * N * K
    t = T.per_launch(prepared(fp4, lambda: fp4.mxfp4_gemm_w4a16(a, wmx, out=c)), it)
    t_d = T.per_launch(prepared(fp4, lambda: fp4.mxfp4_gemm_w4a16_decode(a, md0, out=c)), it)
    out["mxfp4_w4a16_prefill_m4096"] = {"us": t * 1e6, "TFLOP/s": fl / t / 1e12, "frac_bf16_mfma": fl / t / BF16_PEAK,
                                        "decode_layout_us": t_d * 1e6, "decode_layout_TFLOP/s": fl / t_d / 1e12,
                                        "flop": fl, "mfma": "bf16 32x32x16 (MXFP4 widened exactly to bf16)"}
    del a, c, wmx, md0


def m8192_components(torch, fp4, T, dev, w32, it, out):
    from synthetic import WORKLOADS

    # MXFP4 vs NVFP4 W4A4 at M = 8192 on identical bf16 inputs
    wl5 = WORKLOADS["mx_vs_nv_w4a4_m8192"]
    M = 8192
    a_np = wl5.activations_bf16(M)
    a = torch.from_numpy(a_np.view(np.int16)).view(torch.bfloat16).to(dev)
    wb = w32.to(torch.bfloat16)
    wmx = fp4.mxfp4_quantize(wb)
    wnv = fp4.nvfp4_quantize(wb)
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    fl = 2.0 * M * N * K
    wsm = torch.empty(fp4.lib().mxfp4_gemm_w4a4_workspace(M, K), dtype=torch.uint8, device=dev)
    pam = fp4.mxfp4_quantize(a)  # A row-major, for the GEMM half on its own
    t_mq = T.per_launch(prepared(fp4, lambda: fp4.mxfp4_quantize(a, out=pam)), it)
    t_mg = T.per_launch(prepared(fp4, lambda: fp4.mxfp4_gemm_prequant(pam, wmx, out=c)), it, sample_clock=True)
    torch.cuda.synchronize()
    c_2s = c.clone()  # the row-major two-stage kernel
    t_mall = T.per_launch(prepared(fp4, lambda: fp4.mxfp4_gemm_w4a4(a, wmx, out=c, workspace=wsm)), it)
    torch.cuda.synchronize()
    canon_equal = bool(torch.equal(c.view(torch.int16), c_2s.view(torch.int16)))
    c_mx = c.clone()
    # the same GEMM with W in the decode (segment-major) layout and A quantized into it
    wmd = fp4.mxfp4_pack_decode(wmx)
    wss = fp4.mxfp4_gemm_w4a4_seg_workspace(M, K, dev)
    pas = fp4.mxfp4_seg_packed_a(wss, M, K)
    fp4.mxfp4_gemm_w4a4_seg(a, wmd, out=c, workspace=wss)
    t_sg = T.per_launch(prepared(fp4, lambda: fp4.mxfp4_gemm_prequant_seg(pas, wmd, out=c)), it, sample_clock=True)
    t_sall = T.per_launch(prepared(fp4, lambda: fp4.mxfp4_gemm_w4a4_seg(a, wmd, out=c, workspace=wss)), it)
    torch.cuda.synchronize()
    seg_equal = bool(torch.equal(c.view(torch.int16), c_2s.view(torch.int16))) and canon_equal
    wsn = fp4.gemm_w4a4_workspace(M, K, "row", dev)
    t_nall = T.per_launch(prepared(fp4, lambda: fp4.gemm_w4a4(a, wnv, a_mode="row", out=c, workspace=wsn)), it)
    c_nv = c.clone()
    # the same with the NVFP4 weight in the decode layout (the layout the decode GEMV reads)
    wnd = fp4.nvfp4_pack_decode(wnv)
    t_nsall = T.per_launch(prepared(fp4, lambda: fp4.gemm_w4a4_seg(a, wnd, a_mode="row", out=c,
                                                                    workspace=wsn)), it)
    torch.cuda.synchronize()
    nv_seg_equal = bool(torch.equal(c.view(torch.int16), c_nv.view(torch.int16)))
    # W4A8: the same MXFP4 weights, activations as MXFP8
    ws8 = fp4.mxfp4_gemm_w4a8_workspace(M, K, dev)
    pa8 = fp4.mxfp8_packed_a(ws8, M, K)
    t_8q = T.per_launch(prepared(fp4, lambda: fp4.mxfp8_quantize(a, out=pa8)), it)
    t_8g = T.per_launch(prepared(fp4, lambda: fp4.mxfp4_gemm_w4a8_prequant(pa8, wmx, out=c)), it)
    t_8all = T.per_launch(prepared(fp4, lambda: fp4.mxfp4_gemm_w4a8(a, wmx, out=c, workspace=ws8)), it)
    c_a8 = c.clone()
    t_8sg = T.per_launch(prepared(fp4, lambda: fp4.mxfp4_gemm_w4a8_prequant_seg(pa8, wmd, out=c)), it)
    t_8sall = T.per_launch(prepared(fp4, lambda: fp4.mxfp4_gemm_w4a8_seg(a, wmd, out=c, workspace=ws8)), it)
    torch.cuda.synchronize()
    w4a8_seg_equal = bool(torch.equal(c.view(torch.int16), c_a8.view(torch.int16)))
    torch.cuda.synchronize()
    # quantization error against the unquantized bf16 product, on sampled rows
    rows = np.random.default_rng(0).choice(M, 64, replace=False)
    a64 = (a_np[rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    w64 = wb.float().cpu().numpy().astype(np.float64)
    ref = a64 @ w64.T
    rt = torch.from_numpy(rows).to(dev)
    err = {}
    for name, cc in (("mxfp4", c_mx), ("nvfp4", c_nv), ("w4a8_mxfp8_mxfp4", c_a8)):
        got = cc[rt].float().cpu().numpy().astype(np.float64)
        err[name] = {"rel_fro": float(np.linalg.norm(got - ref) / np.linalg.norm(ref)),
                     "max_abs_over_max_ref": float(np.abs(got - ref).max() / np.abs(ref).max())}
    out["mx_vs_nv_w4a4_m8192"] = {
        "mxfp4_quant_us": t_mq * 1e6, "mxfp4_gemm_us": t_mg * 1e6,
        "mxfp4_gemm_TFLOP/s": fl / t_mg / 1e12, "mxfp4_gemm_frac_fp4_mfma": fl / t_mg / FP4_PEAK,
        "mxfp4_total_us": t_mall * 1e6, "mxfp4_total_TFLOP/s": fl / t_mall / 1e12,
        "mxfp4_seg_gemm_us": t_sg * 1e6, "mxfp4_seg_gemm_TFLOP/s": fl / t_sg / 1e12,
        "mxfp4_seg_gemm_frac_fp4_mfma": fl / t_sg / FP4_PEAK, "mxfp4_seg_total_us": t_sall * 1e6,
        "mxfp4_seg_equals_row_major": seg_equal,
        "nvfp4_total_us": t_nall * 1e6, "nvfp4_total_TFLOP/s": fl / t_nall / 1e12,
        "nvfp4_frac_bf16_mfma": fl / t_nall / BF16_PEAK,
        "nvfp4_seg_total_us": t_nsall * 1e6, "nvfp4_seg_total_TFLOP/s": fl / t_nsall / 1e12,
        "nvfp4_seg_frac_bf16_mfma": fl / t_nsall / BF16_PEAK, "nvfp4_seg_equals_row_major": nv_seg_equal,
        "w4a8_quant_us": t_8q * 1e6, "w4a8_gemm_us": t_8g * 1e6,
        "w4a8_gemm_TFLOP/s": fl / t_8g / 1e12, "w4a8_gemm_frac_fp8_mfma": fl / t_8g / FP8_PEAK,
        "w4a8_total_us": t_8all * 1e6, "w4a8_total_TFLOP/s": fl / t_8all / 1e12,
        "w4a8_seg_gemm_us": t_8sg * 1e6, "w4a8_seg_gemm_TFLOP/s": fl / t_8sg / 1e12,
        "w4a8_seg_gemm_frac_fp8_mfma": fl / t_8sg / FP8_PEAK, "w4a8_seg_total_us": t_8sall * 1e6,
        "w4a8_seg_equals_row_major": w4a8_seg_equal,
        "error_vs_bf16_product_64_rows": err}
    del a, c, c_mx, c_2s, c_nv, c_a8, wmx, wnv, wnd, wsm, wsn, ws8, wmd, wss


def moe_components(args, torch, fp4, T, dev):
    """Grouped (MoE) GEMMs: 4096 tokens routed top-8 over 128 experts [1536, 2048];
    the router's permutation is applied inside the kernel (row_index)."""
    from synthetic import MOE_WORKLOADS

    it = args.comp_iters
    out = {}
    wlm = MOE_WORKLOADS["moe_e128_top8_t4096_k2048_n1536"]
    _, offs, ridx, _ = wlm.routing()
    rows = int(offs[-1])
    a = torch.from_numpy(wlm.activations_bf16().view(np.int16)).view(torch.bfloat16).to(dev)
    wexp = torch.from_numpy(wlm.expert_weights()).to(dev)
    env = fp4.nvfp4_quantize_experts(wexp)
    emx = fp4.mxfp4_quantize_experts(wexp)
    del wexp
    go = torch.from_numpy(offs).to(dev)
    ri = torch.from_numpy(ridx).to(dev)
    c = torch.empty(rows, wlm.N, dtype=torch.bfloat16, device=dev)
    wsg = fp4.nvfp4_grouped_gemm_w4a4_workspace(wlm.tokens, wlm.K, dev)
    fl = 2.0 * rows * wlm.N * wlm.K
    t_gnv = T.per_launch(prepared(fp4, lambda: fp4.nvfp4_grouped_gemm_w4a16(a, env, go, ri, out=c)), it)
    t_gmx = T.per_launch(prepared(fp4, lambda: fp4.mxfp4_grouped_gemm_w4a16(a, emx, go, ri, out=c)), it)
    t_g44 = T.per_launch(prepared(fp4, lambda: fp4.nvfp4_grouped_gemm_w4a4(a, env, go, ri, out=c, workspace=wsg)), it)
    loads = np.diff(offs)
    out["moe_grouped_" + wlm.name] = {
        "rows": rows, "experts": wlm.experts, "empty_experts": int((loads == 0).sum()),
        "max_rows_per_expert": int(loads.max()), "flop": fl,
        "nvfp4_w4a16_us": t_gnv * 1e6, "nvfp4_w4a16_TFLOP/s": fl / t_gnv / 1e12,
        "nvfp4_w4a16_frac_bf16_mfma": fl / t_gnv / BF16_PEAK,
        "mxfp4_w4a16_us": t_gmx * 1e6, "mxfp4_w4a16_TFLOP/s": fl / t_gmx / 1e12,
        "mxfp4_w4a16_frac_bf16_mfma": fl / t_gmx / BF16_PEAK,
        "nvfp4_w4a4_total_us": t_g44 * 1e6, "nvfp4_w4a4_total_TFLOP/s": fl / t_g44 / 1e12}
    return out


def cpu_baseline(wl, wq, w_np):
    """The oracle as it stands, timed on the host cores of this machine: the whole
    decode step (the `value` workload) plus one leg per other kernel of the path.

    * decode step: dequantize W to fp64 in C (OpenMP) and a numpy float64 product,
      for M = 1, 4 and 16, repeated for about 8 s; GB/s over the step's bytes;
    * quantizers and the dequantizer at full size, once each; GB/s over the same
      algorithmic bytes as the GPU figures;
    * the prefill GEMMs on a 128-row slice of A, scaled by M / 128 to the full M
      (labelled extrapolated); GFLOP/s over 2 M N K.  The oracle also forms the
      tolerance term sum |a w|, a second product, which these figures do not count."""
    import oracle
    from synthetic import WORKLOADS

    cores = len(os.sched_getaffinity(0))
    codes = wq.codes.cpu().numpy()
    scales = wq.scales.cpu().numpy()
    ts = wq.tscale.cpu().numpy()
    acts = {M: wl.activations_bf16(M) for M in wl.M}
    reps, t0 = 0, time.perf_counter()
    while True:
        for M in wl.M:
            oracle.gemm_w4a16_ref(acts[M], codes, scales, ts)
        reps += 1
        el = time.perf_counter() - t0
        if el > 8.0 or reps >= 40:
            break
    per_step = el / reps
    b = sum(decode_bytes(M) for M in wl.M)
    legs = {}

    def timed(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    bw = 2 * N * K * 4 + N * K // 2 + N * K // 16 + 4
    t = timed(lambda: oracle.nvfp4_quantize(w_np))
    legs["weight_quantize_fp32_17408x5120"] = {"s": round(t, 3), "GB/s": round(bw / t / 1e9, 3), "bytes": bw}
    bd = N * K // 2 + N * K // 16 + 4 + N * K * 4
    t = timed(lambda: oracle.nvfp4_dequantize(codes, scales, ts))
    legs["dequantize_fp32_17408x5120"] = {"s": round(t, 3), "GB/s": round(bd / t / 1e9, 3), "bytes": bd}
    a4 = WORKLOADS["prefill_w4a4_m4096"].activations_bf16(4096)
    bq = 4096 * K * 2 + 4096 * K // 2 + 4096 * K // 16 + 4 * 4096
    t = timed(lambda: oracle.nvfp4_quantize(a4, per_row=True))
    legs["activation_quantize_per_row_4096x5120"] = {"s": round(t, 3), "GB/s": round(bq / t / 1e9, 3), "bytes": bq}
    a8 = WORKLOADS["mx_vs_nv_w4a4_m8192"].activations_bf16(8192)
    bm = 8192 * K * 2 + 8192 * K // 2 + 8192 * K // 32
    t = timed(lambda: oracle.mxfp4_quantize(a8))
    legs["mxfp4_quantize_8192x5120"] = {"s": round(t, 3), "GB/s": round(bm / t / 1e9, 3), "bytes": bm}

    wb = oracle.f32_to_bf16_bits(w_np)                       # the C5 weights: fp32 -> bf16, then each format
    mc, ms = oracle.mxfp4_quantize(wb)
    nc, ns, nt = oracle.nvfp4_quantize(wb)
    sl = 128
    gemms = {
        "prefill_w4a16_m4096": (4096, lambda: oracle.gemm_w4a16_ref(a4[:sl], codes, scales, ts)),
        "prefill_w4a4_m4096": (4096, lambda: oracle.gemm_w4a4_ref(a4[:sl], codes, scales, ts, a_per_row=True)),
        "mxfp4_w4a4_m8192": (8192, lambda: oracle.mxfp4_gemm_w4a4_ref(a8[:sl], mc, ms)),
        "nvfp4_w4a4_m8192": (8192, lambda: oracle.gemm_w4a4_ref(a8[:sl], nc, ns, nt, a_per_row=True)),
    }
    for name, (M, fn) in gemms.items():
        t = timed(fn)
        legs[name] = {"slice_rows": sl, "slice_s": round(t, 3), "extrapolated_s": round(t * M / sl, 2),
                      "GFLOP/s": round(2.0 * sl * N * K / t / 1e9, 2), "extrapolated": True}
    return {"value": round(b / per_step / 1e9, 4), "unit": "GB/s", "cores": cores,
            "threads": oracle.num_threads(), "kind": "oracle",
            "sample": f"{reps} full decode step(s) (M=1,4,16 on the 17408x5120 NVFP4 weight): "
                      f"{per_step:.2f} s per step on the host; OpenMP threads for dequantization, "
                      "numpy BLAS for the fp64 product",
            "legs": legs}


if __name__ == "__main__":
    main()
