"""Throughput of the channels-last implicit-GEMM convolution forward on one MI355X.

A step is one pass over the fp16 3x3x3 NDHWC sweep
  (4,32^3,128->128, s1 p1), (1,64^3,64->128, s1 p1), (4,32^3,64->128, s2 p1)
with seeded synthetic inputs already resident in HBM; each convolution is one
launch of the library's auto path on the current stream.  The metric is
2*M*N*K FLOPs (M = output positions, N = C_out, K = C_in*27) per second over
the timed steps, in TFLOP/s.

The JSON line also carries
  roofline:     the dominant kernel (the path with the largest share of the
                step; the slab kernel runs both unit-stride 116-GFLOP
                convolutions) timed launch by launch with HIP events on the
                launch stream (one before each launch, each launch timed to
                the next event; timing-only events, recorded without a
                system-scope fence), against the MI355X dense fp16 MFMA peak.
                Those events go into a pass of max(steps, 50) steps run
                between the warm-up steps and the timed region, which holds
                no event between launches;
                The same object carries the kernel-trace figure of the committed
                rocprofv3 summary (trace_us, trace_frac) when that summary was
                taken on the current kernel sources;
  cpu_baseline: the float64 CPU oracle (OpenMP over this host's cores) on a
                share of one step's output rows (--cpu-fraction, default the
                whole step: every output row of the three convolutions).

``--sweep`` instead times every workload shape on its own (warm-up launches in
rounds of 10 until 50 ms have passed, then
``--launches`` launches each between two HIP events on the launch stream;
median and min), once with resident buffers and once "cold", rotating enough
(x, y) buffer sets (> 512 MB) that the 256 MB MALL cannot hold them; one JSON
line per workload.
"""
import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import implicit_gemm_conv_amd as igc  # noqa: E402
from conv_workloads import BWD_WORKLOADS, HEADLINE, VARIANT_WORKLOADS, WORKLOADS, make_inputs  # noqa: E402

PEAK_TFLOPS = {"fp16": 2516.6, "bf16": 2516.6, "fp32": 157.3}   # MI355X dense, published
METRIC = "conv fwd TFLOP/s (2·M·N·K) and % of MFMA peak, fp16 NDHWC 3×3×3 shapes"
# Per path: the kernel it launches on these shapes and the sources that kernel is built from
# (the stored counter figures are tied to their hash).
_COMMON = ["implicit_gemm_conv_amd/csrc/conv_device.h", "implicit_gemm_conv_amd/csrc/conv_params.h"]
KERNELS = {
    "slab": ("conv_slab_kernel<fp16, K_w=3, K_h=3>: 16x32-output x 128-channel tile, 32x32x16 MFMA",
             ["implicit_gemm_conv_amd/csrc/k_slab.hip", *_COMMON]),
    "phase": ("conv_phase_kernel<fp16, K_h=3, K_w=3>: 8x16-output x 64-channel tile, stride-phase "
              "staging, 32x32x16 MFMA",
              ["implicit_gemm_conv_amd/csrc/k_phase.hip", *_COMMON]),
    "strip": ("conv_strip_kernel<fp16, K_w=3>: 512x128 tile, 32x32x16 MFMA",
              ["implicit_gemm_conv_amd/csrc/k_strip.hip", *_COMMON]),
    "main": ("conv_main_kernel<fp16>: 128x128 tile, BK=64, 16x16x32 MFMA",
             ["implicit_gemm_conv_amd/csrc/k_main.hip", *_COMMON]),
}


class HipTimer:
    """HIP events used only to measure time, recorded on the launch stream.

    They are created with hipEventDisableSystemFence, the flag the HIP runtime
    documents for timing-only events: recording one skips the system-scope
    release (cache writeback and invalidation) that a default event performs,
    which cost the stream several microseconds per event (and now and then far
    more) and perturbed the kernel that followed.  The host reads them only
    after torch.cuda.synchronize().  They come from the HIP runtime torch
    loaded, so torch's stream handles are valid for them."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        lib = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        self.hip = ctypes.CDLL(lib if os.path.exists(lib) else "libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def event(self):
        e = ctypes.c_void_p()
        self._check(self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE),
                    "hipEventCreateWithFlags")
        self.events.append(e)
        return e

    def record(self, e, stream):
        self._check(self.hip.hipEventRecord(e, ctypes.c_void_p(stream.cuda_stream)), "hipEventRecord")

    def ms(self, a, b):
        out = ctypes.c_float()
        self._check(self.hip.hipEventElapsedTime(ctypes.byref(out), a, b), "hipEventElapsedTime")
        return out.value

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def traffic_file(path):
    return os.path.join(ROOT, "profiles", f"conv_{path}_fp16_c4ab_hbm_traffic.md")


def kernel_source_hash(path="slab"):
    """sha256 of the sources the path's kernel is built from, comments and blank lines left out
    (an edit to comments alone keeps the stored counter figures valid; any code change does not)."""
    h = hashlib.sha256()
    for rel in KERNELS[path][1]:
        with open(os.path.join(ROOT, rel)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def stored_traffic(path):
    """HBM bytes per launch of the path's kernel from the committed counter summary,
    or None when it is missing or was taken on other kernel sources."""
    if path not in KERNELS or not os.path.exists(traffic_file(path)):
        return None
    text = open(traffic_file(path)).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_hash and m_bytes) or m_hash.group(1) != kernel_source_hash(path):
        return None
    return float(m_bytes.group(1))


def trace_file(path):
    return os.path.join(ROOT, "profiles", "conv_fp16_c4_sweep_kernel_trace.md")


def stored_trace_ns(path):
    """Mean kernel-trace duration per launch of the path's kernel from the committed rocprofv3
    summary of this bench, or None when missing or taken on other kernel sources."""
    f = trace_file(path)
    if path not in KERNELS or not os.path.exists(f):
        return None
    text = open(f).read()
    m_path = re.search(r"dominant_path:\s*(\w+)", text)
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_ns = re.search(r"dominant_kernel_trace_mean_ns:\s*([0-9.]+)", text)
    if not (m_path and m_hash and m_ns) or m_path.group(1) != path or m_hash.group(1) != kernel_source_hash(path):
        return None
    return float(m_ns.group(1))


def copy_calibration(mib=512, reps=5):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = mib * 2**20 // 2
    a = torch.randn(n, device="cuda:0", dtype=torch.float32).to(torch.float16)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_copy": n * 2, "bytes_written_per_copy": n * 2,
                                           "copies": reps}}), flush=True)


def _var(wl):
    """dilation / groups of a workload (1 for the plain ones)."""
    return dict(dilation=wl.dilation or 1, groups=wl.groups)


def gemm_dims(wl):
    """M output positions, N = C_out, K = taps * C_in / groups: 2*M*N*K is the multiply-add
    count of the sum (grouped layers multiply each output by one group's channels only).
    Backward-data performs the forward pass's multiply-adds: M is dy's positions."""
    if wl.dx_shape is not None:
        return int(np.prod(wl.x_shape[:-1])), wl.w_shape[0], int(np.prod(wl.w_shape[1:]))
    out = igc.out_shape(wl.x_shape, wl.w_shape, wl.stride, wl.padding, **_var(wl))
    m = int(np.prod(out[:-1]))
    n = wl.w_shape[0]
    k = int(np.prod(wl.w_shape[1:]))
    return m, n, k


def kernel_key(wl):
    """The path AUTO takes; on these shapes a path launches one kernel instantiation."""
    return igc.select_path(wl.x_shape, wl.w_shape, wl.stride, wl.padding, wl.torch_dtype, **_var(wl))


def cpu_baseline(wls, inputs, fraction):
    """The oracle on `fraction` of the output rows of every convolution of one step
    (evenly spaced rows, all channels); 1.0 is one whole step."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    flops, dt, rows_done, rows_all = 0.0, 0.0, 0, 0
    for wl, (x, w) in zip(wls, inputs):
        xf = oracle.to_float64(x)
        wf = oracle.to_float64(w)
        m, n, k = gemm_dims(wl)
        count = max(1, int(round(m * fraction)))
        rows = np.linspace(0, m - 1, count).astype(np.int64)
        t0 = time.perf_counter()
        oracle.conv_fwd(xf, wf, wl.stride, wl.padding, rows=rows)
        dt += time.perf_counter() - t0
        flops += 2.0 * count * n * k
        rows_done += count
        rows_all += m
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows_done} of the {rows_all} output rows of one step (the three "
                      f"convolutions, evenly spaced rows, all channels), float64 direct loop, "
                      f"{flops / 1e9:.1f} GFLOP in {dt:.1f} s"}


def sweep(launches, names=None, tune=False):
    """Per-workload event timing, warm (resident buffers) and cold (rotated buffer sets).  With
    tune, each forward shape is first timed on every path (conv_tune) and AUTO then takes the
    fastest."""
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    timer = HipTimer()
    for name, wl in {**WORKLOADS, **VARIANT_WORKLOADS, **BWD_WORKLOADS}.items():
        if names and name not in names:
            continue
        bwd = wl.dx_shape is not None
        x, w = make_inputs(wl, dev)           # backward-data: x is dy, y is dx
        if bwd:
            shape = wl.dx_shape
            wt = igc.bwd_data_filter(w, wl.dx_shape, wl.stride, wl.padding)   # once per filter
        else:
            shape = igc.out_shape(wl.x_shape, wl.w_shape, wl.stride, wl.padding, **_var(wl))
        y = torch.empty(shape, dtype=wl.torch_dtype, device=dev)
        if tune and not bwd:
            igc.tune(x, w, wl.stride, wl.padding, reps=5, out=y, **_var(wl))
        m, n, k = gemm_dims(wl)
        flops = 2.0 * m * n * k
        esz = x.element_size()
        alg_bytes = esz * (x.numel() + w.numel() + y.numel())
        # cold: enough (x, y) sets that together they exceed 512 MB, at least 3
        sets = max(3, -(-(512 << 20) // (esz * (x.numel() + y.numel()))) + 1)
        xs = [x] + [x.clone() for _ in range(sets - 1)]
        ys = [y] + [torch.empty_like(y) for _ in range(sets - 1)]

        def timed(pairs):
            evs = [(timer.event(), timer.event()) for _ in pairs]
            for (xi, yi), (a, b) in zip(pairs, evs):
                timer.record(a, stream)
                if bwd:
                    igc.conv_bwd_data(xi, w, wl.dx_shape, wl.stride, wl.padding, out=yi, wt=wt)
                else:
                    igc.conv_fwd(xi, w, wl.stride, wl.padding, out=yi, **_var(wl))
                timer.record(b, stream)
            torch.cuda.synchronize()
            t = np.array([timer.ms(a, b) * 1e3 for a, b in evs])
            timer.close()
            return t

        # warm-up: at least 10 launches and 50 ms, so that every shape is timed at the clocks
        # the GPU settles to under load (a shape timed right after a light one otherwise
        # runs its first milliseconds slower)
        t0 = time.perf_counter()
        n_warm = 0
        while True:
            timed([(x, y)] * 10)
            n_warm += 10
            if time.perf_counter() - t0 >= 0.05:
                break
        warm = timed([(x, y)] * launches)
        cold = timed([(xs[i % sets], ys[i % sets]) for i in range(launches)])
        peak = PEAK_TFLOPS[wl.dtype]
        rec = {"workload": name, "path": "bwd_data" if bwd else kernel_key(wl), "dtype": wl.dtype,
               "gemm_mnk": [m, n, k],
               "gflop": round(flops / 1e9, 4), "alg_mb": round(alg_bytes / 1e6, 3), "launches": launches,
               "warmup_launches": n_warm}
        for tag, t in (("warm", warm), ("cold", cold)):
            med = float(np.median(t))
            rec[tag] = {"us_median": round(med, 2), "us_min": round(float(t.min()), 2),
                        "tflops": round(flops / (med * 1e-6) / 1e12, 2),
                        "pct_peak": round(100 * flops / (med * 1e-6) / 1e12 / peak, 2),
                        "alg_gbps": round(alg_bytes / (med * 1e-6) / 1e9, 1)}
        rec["cold"]["buffer_sets"] = sets
        print(json.dumps(rec), flush=True)
        del xs, ys, x, w, y
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-fraction", type=float, default=1.0,
                    help="share of one step's output rows the CPU oracle computes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy (counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="time every workload shape on its own (one JSON line each)")
    ap.add_argument("--launches", type=int, default=50, help="timed launches per shape in --sweep")
    ap.add_argument("--only", default="", help="comma-separated workload names for --sweep")
    ap.add_argument("--tune", action="store_true",
                    help="in --sweep, time every path per shape first and use the fastest (conv_tune)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the convolution would shard by batch or C_out with no exchange).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.sweep:
        sweep(args.launches, [n for n in args.only.split(",") if n], tune=args.tune)
        return
    wls = [WORKLOADS[n] for n in HEADLINE]
    inputs = [make_inputs(wl, dev) for wl in wls]
    outs = [torch.empty(igc.out_shape(wl.x_shape, wl.w_shape, wl.stride, wl.padding),
                        dtype=wl.torch_dtype, device=dev) for wl in wls]
    dims = [gemm_dims(wl) for wl in wls]
    flops = [2.0 * m * n * k for (m, n, k) in dims]
    step_flops = sum(flops)
    stream = torch.cuda.current_stream()

    def step(marks=None):
        for i, wl in enumerate(wls):
            x, w = inputs[i]
            if marks is not None:
                timer.record(marks[i], stream)
            igc.conv_fwd(x, w, wl.stride, wl.padding, out=outs[i])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Per-launch times, for the per-workload figures and the roofline: at
    # least 50 steps (more samples than a short timed region gives) with one
    # HIP event before every launch (and one after the last), each launch
    # timed from its own event to the next one.  This pass runs after the
    # warm-up steps and before the timed region.
    timer = HipTimer()
    n_ev = max(args.steps, 50)
    ev = [[timer.event() for _ in wls] for _ in range(n_ev)]
    ev_end = timer.event()
    torch.cuda.synchronize()
    for s in range(n_ev):
        step(ev[s])
    timer.record(ev_end, stream)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps between two synchronisations, with one
    # HIP event on the launch stream at each end and nothing else in between
    # (an event recorded between launches costs the stream a few us).
    t_start = timer.event()
    t_end = timer.event()
    torch.cuda.synchronize()
    timer.record(t_start, stream)
    for s in range(args.steps):
        step()
    timer.record(t_end, stream)
    torch.cuda.synchronize()
    total_ms = timer.ms(t_start, t_end)
    ms_per_step = total_ms / args.steps

    def launch_ms(s, i):
        nxt = ev[s][i + 1] if i + 1 < len(wls) else (ev[s + 1][0] if s + 1 < n_ev else ev_end)
        return timer.ms(ev[s][i], nxt)

    per = {}
    for i, wl in enumerate(wls):
        times = [launch_ms(s, i) for s in range(n_ev)]
        us = 1e3 * float(np.mean(times))
        per[wl.name] = {"path": kernel_key(wl), "us_mean": round(us, 3),
                        "us_min": round(1e3 * float(np.min(times)), 3),
                        "tflops": round(flops[i] / (us * 1e-6) / 1e12, 2),
                        "pct_peak": round(100 * flops[i] / (us * 1e-6) / 1e12 / PEAK_TFLOPS["fp16"], 2)}

    # Dominant kernel: the path with the largest summed launch time over the step.
    keys = [kernel_key(wl) for wl in wls]
    share = {k: sum(per[wl.name]["us_mean"] for wl, kk in zip(wls, keys) if kk == k) for k in set(keys)}
    dom_path = max(share, key=share.get)
    dom = [i for i, k in enumerate(keys) if k == dom_path]
    dom_us = float(np.mean([1e3 * launch_ms(s, i) for s in range(n_ev) for i in dom]))
    timer.close()
    dom_flops = float(np.mean([flops[i] for i in dom]))
    achieved = dom_flops / (dom_us * 1e-6) / 1e12
    alg_bytes = [2 * (int(np.prod(wl.x_shape)) + int(np.prod(wl.w_shape)) +
                      int(np.prod(igc.out_shape(wl.x_shape, wl.w_shape, wl.stride, wl.padding))))
                 for wl in wls]
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["fp16"],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["fp16"], 4),
                "timer": "HIP events on the launch stream, one per launch, each launch timed to the next event "
                         "(a pass of max(steps, 50) steps between the warm-up and the timed region)",
                "traffic": stored_traffic(dom_path),
                "kernel": KERNELS.get(dom_path, (dom_path,))[0] + " (" +
                          ", ".join(wls[i].name.split("_")[0] for i in dom) + ")",
                "kernel_source_sha256": kernel_source_hash(dom_path) if dom_path in KERNELS else None,
                "launch_us": round(dom_us, 3), "flops_per_launch": dom_flops,
                "algorithmic_bytes_per_launch": float(np.mean([alg_bytes[i] for i in dom]))}
    trace_ns = stored_trace_ns(dom_path)
    if trace_ns is not None:
        roofline["trace_us"] = round(trace_ns / 1e3, 3)
        roofline["trace_frac"] = round(dom_flops / (trace_ns * 1e-9) / 1e12 / PEAK_TFLOPS["fp16"], 4)
        roofline["trace_profile"] = os.path.relpath(trace_file(dom_path), ROOT)

    value = step_flops * args.steps / (total_ms * 1e-3) / 1e12
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded x ~ U[-1,1), w ~ N(0,1)/sqrt(fan_in), fp16)",
        "config": {"workload": "conv3d fwd fp16 NDHWC 3x3x3 pad 1 sweep: "
                               "(4,32^3,128->128,s1), (1,64^3,64->128,s1), (4,32^3,64->128,s2)",
                   "gemm_mnk": dims, "gflop_per_step": round(step_flops / 1e9, 3)},
        "per_workload": per,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wls, inputs, args.cpu_fraction)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
