"""Benchmark of the FP8 delayed-scaling hot path on one MI355X.

One step = one multi-tensor fused quantize+amax launch over every tensor of the
workload (bf16 -> FP8 with the previous step's scale) followed by one batched
amax_and_scale_update launch (history roll, amax selection, new scale/scale_inv, amax
reset), on inputs already resident in HBM; the same steps in one launch each
(fp8_quantize_amax_and_update) are timed beside.  Default workload: the full step of the
hidden-12288 / ffn-49152 MLP (activations (2048,12288) and (2048,49152), weights
12288x49152 and 49152x12288 to E4M3, the output gradient (2048,12288) to E5M2: 1.36 G
elements, 4.08 GB per step; history 1024).  Prints one JSON line.

Also measured in the same run: the same steps on the hidden-4096 MLP (0.5 GB) and on the
8192x16384 E5M2 gradient with saturation (0.4 GB); the achievable rate of the quantize
pass's traffic without its arithmetic (a 2:1 read:write stream with the same cache
policies, best of a sweep, at 0.5 GB and 4 GB; read-only and write-only beside); the
batched update of 1152 tensors with history 1024 (device time per call in a replayed
graph, per-call events warm and cold, host wall time per call) next to two floors on its
own grid (an empty kernel, one load->barrier->store round trip); dequantize; the
gelu-fused and LayerNorm-fused quantize against the unfused sequences; the FP8 GEMM
consumer on the hidden-4096 MLP's two dense shapes against torch._scaled_mm; a
device-to-device copy; and the CPU oracle on the same step (cpu_baseline), whose output
is compared byte for byte with the GPU's first step.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 matrix throughput, published
METRIC = "fused quantize+amax GB/s & % HBM peak; µs per batched scale update"
# The multi-tensor quantize with bf16 sources; launches of at least 256 MiB of codes take
# its instance with non-temporal stores.
STREAM_CODE_BYTES = 256 << 20


def roofline_kernel(w) -> str:
    big = sum(int(t.data.size) for t in w.tensors) >= STREAM_CODE_BYTES
    return "quantize_amax_kernel<1, false, %s>" % ("true" if big else "false")
PROBE_LIB = os.path.join(ROOT, "delayed_scaling_amax_amd", "libfp8q_probe.so")
OTHER_WORKLOADS = ("mlp_4096", "grad_8192x16384")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for name in ("quantize_amax.hip", "quant_math.h", "device_common.h", "host_common.h"):
        with open(os.path.join(ROOT, "delayed_scaling_amax_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", "quantize_amax_%s_traffic.txt" % workload)


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per quantize launch from the committed rocprofv3 counter summary, or
    None if absent, for another workload or kernel, or taken on a different kernel
    source."""
    try:
        kv = {}
        with open(traffic_file(workload)) as f:
            for line in f:
                if "=" in line and not line.startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if (kv.get("kernel_source_sha256_16") != kernel_hash() or kv.get("workload") != workload
                or kv.get("kernel") != kernel):
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def host_cpus() -> int:
    """CPUs this process may run on: its affinity set, bounded by a cgroup CPU quota
    when one is set."""
    n = len(os.sched_getaffinity(0))
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()
        if quota != "max":
            n = min(n, max(1, math.ceil(int(quota) / int(period))))
    except (OSError, ValueError):
        pass
    return max(1, n)


def alg_bytes_quantize(w) -> int:
    """Algorithmic bytes of one quantize launch: read every source element, write one
    FP8 byte per element, read each scale (4 B), read+write each amax (8 B)."""
    return sum(int(t.data.nbytes) + int(t.data.size) + 12 for t in w.tensors)


def alg_bytes_update(n: int, H: int) -> int:
    """History read + in-place write, amax read (and reset write), scale read + write,
    scale_inv write, format byte."""
    return 2 * H * n * 4 + n * 4 * 2 + n * 4 * 2 + n * 4 + n


def timed_launches(fn, reps=20):
    """Median time (us) of fn(i) between HIP events on the current stream, after 3
    untimed calls; fn(i) picks its buffers by i."""
    import torch
    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    return 1e3 * float(np.median([a.elapsed_time(b) for a, b in ev]))


def graph_us_per_call(fn, calls):
    """Device time per call of fn() from a HIP graph of `calls` calls replayed 5 times
    (no Python launch overhead and no per-call events in the timed region), or None if
    capture fails."""
    import torch
    try:
        g = torch.cuda.CUDAGraph()
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            with torch.cuda.graph(g, stream=s_cap):
                for _ in range(calls):
                    fn()
        torch.cuda.current_stream().wait_stream(s_cap)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        us = 1e3 * a.elapsed_time(b) / (5 * calls)
        del g
        return us
    except Exception as e:  # capture unsupported: report the other figures only
        log("graph capture failed: %r" % (e,))
        return None


def w_ln_input(workloads, threads, w=None):
    """The LayerNorm input: the mlp_4096 activation (2048,4,4096) as (8192, 4096) bf16
    (taken from w when that is the mlp_4096 workload already generated)."""
    if w is None or w.name != "mlp_4096":
        w = workloads.mlp_4096(threads=threads)
    act = w.tensors[0].data
    return act.reshape(-1, act.shape[-1]).view(np.int16)


class StepBench:
    """Device buffers of one workload's delayed-scaling step (R rotating copies of the
    inputs and outputs) and the timed regions over them."""

    def __init__(self, w, dev, rotate):
        import torch
        import delayed_scaling_amax_amd as d
        self.d, self.torch, self.w, self.dev, self.rotate = d, torch, w, dev, rotate
        self.fmts = [0 if t.fmt == "e4m3" else 1 for t in w.tensors]
        n = self.n = len(w.tensors)
        # R copies of the inputs and outputs, used in turn by successive steps: a step's
        # tensors were last touched R-1 steps earlier (>= 1 GB of traffic for the small
        # workloads), so they stream from HBM and not from the 256 MB MALL, as in a
        # training step where the GEMMs run between two quantizations of a tensor
        srcs0 = [torch.from_numpy(t.data.view(np.int16)).view(torch.bfloat16).to(dev)
                 for t in w.tensors]
        sets = [srcs0] + [[x.clone() for x in srcs0] for _ in range(rotate - 1)]
        self.outs = [[torch.empty(t.data.size, dtype=torch.uint8, device=dev)
                      for t in w.tensors] for _ in range(rotate)]
        self.scale = torch.tensor(w.first_scale, dtype=torch.float32, device=dev)
        self.scale_inv = torch.empty(n, dtype=torch.float32, device=dev)
        self.amax = torch.zeros(n, dtype=torch.float32, device=dev)
        self.hist = torch.zeros(w.history_len, n, dtype=torch.float32, device=dev)
        self.fdev = torch.tensor(self.fmts, dtype=torch.uint8, device=dev)
        self.ws = torch.zeros(1, dtype=torch.int32, device=dev)  # one-launch step counter
        self.entry_sets = [[(sets[r][i], self.outs[r][i], self.scale[i:i + 1],
                             self.amax[i:i + 1], self.fmts[i]) for i in range(n)]
                           for r in range(rotate)]
        self.step_no = 0
        self.qbytes = alg_bytes_quantize(w)
        self.ubytes = alg_bytes_update(n, w.history_len)

    def quantize(self, events=None):
        e = self.entry_sets[self.step_no % self.rotate]
        if events is None:
            self.d.fp8_multi_quantize_amax(e)
        else:  # the same launch, with events set to the kernel's own start and stop
            self.d.fp8_multi_quantize_amax_timed(e, *events)
        self.step_no += 1

    def update(self):
        self.d.fp8_amax_and_scale_update(self.amax, self.hist, self.scale, self.scale_inv,
                                         self.fdev, reset_amax=True)

    def step(self, events=None):
        """One step: the multi-tensor quantize + amax launch, then the batched update
        launch (reset amax)."""
        self.quantize(events)
        self.update()

    def one_launch_step(self, events=(None, None)):
        """The same step in one launch: the update runs in the block that finishes the
        quantize last."""
        self.d.fp8_quantize_amax_and_update(
            self.entry_sets[self.step_no % self.rotate], self.amax, self.hist, self.scale,
            self.scale_inv, self.fdev, self.ws, reset_amax=True, start_event=events[0],
            stop_event=events[1])
        self.step_no += 1

    def first_step(self):
        """The first step (prior scale), its codes, amax and FP8 meta kept on the host for
        the parity check against the oracle."""
        torch = self.torch
        self.quantize()
        torch.cuda.synchronize()
        codes = [x.cpu().numpy() for x in self.outs[0]]
        amax = self.amax.cpu().numpy().copy()
        self.update()
        torch.cuda.synchronize()
        meta = {"hist": self.hist.cpu().numpy().copy(), "scale": self.scale.cpu().numpy().copy(),
                "scale_inv": self.scale_inv.cpu().numpy().copy(),
                "amax": self.amax.cpu().numpy().copy()}
        return codes, amax, meta

    def run(self, K, warmup):
        """Two timed regions of K steps each, for the two-launch and the one-launch step.
        (1) The steps alone, bracketed by two stream events and the host clock, with a
        synchronize on both sides: ms per step and whole-step GB/s. (2) The same steps,
        each launch carrying two HIP events that take the kernel's own start and stop time
        (hipExtLaunchKernel): the kernel's live duration, without the dispatch latency that
        events recorded on the stream around the call would add.  Launches that carry
        events cost ~30 us more host time each, which would make small steps host-bound,
        so (1) carries none."""
        torch = self.torch
        for _ in range(warmup):
            self.step()
            self.one_launch_step()  # the first launches of each kernel load it
        torch.cuda.synchronize()

        def make_events():
            e = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
            for a, b in e:  # torch creates an event at its first record
                a.record()
                b.record()
            return e

        def region(fn):
            """(host wall ms per step, device ms per step, host enqueue us per step)."""
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            ev[0].record()
            for k in range(K):
                fn(k)
            ev[1].record()
            t_enq = time.perf_counter()  # all K steps enqueued (the host runs ahead)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            return ((t1 - t0) * 1e3 / K, ev[0].elapsed_time(ev[1]) / K, (t_enq - t0) * 1e6 / K)

        qb, ub = self.qbytes, self.ubytes
        ms, dev_ms, enq = region(lambda k: self.step())
        ev = make_events()
        region(lambda k: self.step(ev[k]))
        q_ms = [ev[k][0].elapsed_time(ev[k][1]) for k in range(K)]
        u_ms = [ev[k][1].elapsed_time(ev[k + 1][0]) for k in range(K - 1)] or [0.0]
        q_avg = 1e3 * float(np.mean(q_ms))
        r = {"ms_per_step": ms, "device_ms_per_step": dev_ms, "host_enqueue_us_per_step": enq,
             "value_gbps": (qb + ub) / (ms * 1e-3) / 1e9,
             "q_avg_us": q_avg, "q_median_us": 1e3 * float(np.median(q_ms)),
             "q_gbps": qb / (q_avg * 1e-6) / 1e9, "u_gap_avg_us": 1e3 * float(np.mean(u_ms))}
        # the two forms compared in alternating regions (one-launch first), so that a
        # drift of the clock over the run does not favour either; medians of 3 each
        pairs = []
        for _ in range(3):
            pairs.append((region(lambda k: self.one_launch_step()),
                          region(lambda k: self.step())))
        one_ms = float(np.median([p[0][0] for p in pairs]))
        one_dev = float(np.median([p[0][1] for p in pairs]))
        one_enq = float(np.median([p[0][2] for p in pairs]))
        two_ms = float(np.median([p[1][0] for p in pairs]))
        two_dev = float(np.median([p[1][1] for p in pairs]))
        ev1 = make_events()
        region(lambda k: self.one_launch_step(ev1[k]))
        s_ms = [ev1[k][0].elapsed_time(ev1[k][1]) for k in range(K)]
        s_avg = 1e3 * float(np.mean(s_ms))
        r["one_launch"] = {
            "entry": "fp8_quantize_amax_and_update (quantize + amax + update, one launch)",
            "ms_per_step": round(one_ms, 5), "device_ms_per_step": round(one_dev, 5),
            "host_enqueue_us_per_step": round(one_enq, 2),
            "two_launch_ms_per_step": round(two_ms, 5),
            "two_launch_device_ms_per_step": round(two_dev, 5),
            "timing": "medians of 3 regions of K steps per form, the forms alternating",
            "value_gbps": round((qb + ub) / (one_ms * 1e-3) / 1e9, 2),
            "kernel_avg_us": round(s_avg, 3),
            "kernel_median_us": round(1e3 * float(np.median(s_ms)), 3),
            "kernel_gbps": round((qb + ub) / (s_avg * 1e-6) / 1e9, 1)}
        log("%s: step %.4f ms (device %.4f ms, host enqueue %.1f us) = %.1f GB/s; quantize "
            "avg %.2f us (median %.2f) = %.1f GB/s; update + gaps avg %.2f us" % (
                self.w.name, ms, dev_ms, enq, r["value_gbps"], q_avg, r["q_median_us"],
                r["q_gbps"], r["u_gap_avg_us"]))
        log("%s: one-launch step %.4f ms (device %.4f ms) = %.1f GB/s vs two launches %.4f ms "
            "(device %.4f ms) in alternating regions; kernel avg %.2f us (median %.2f)" % (
                self.w.name, one_ms, one_dev, r["one_launch"]["value_gbps"], two_ms, two_dev,
                s_avg, r["one_launch"]["kernel_median_us"]))
        return r


def probe_lib():
    lib = ctypes.CDLL(PROBE_LIB)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.probe_stream.argtypes = [vp, vp, i64, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.probe_stream.restype = i32
    lib.probe_update_floor.argtypes = [vp, i64, i64, i32, vp]
    lib.probe_update_floor.restype = i32
    lib.probe_mfma.argtypes = [i32, i32, vp, vp, vp, vp]
    lib.probe_mfma.restype = i32
    return lib


def mfma_ceiling(plib, dev, cus, iters=2000, reps=12):
    """The FP8 matrix cores' sustained rate with register operands only (probe_mfma: one
    block of 4 wavefronts per CU, each wavefront iters x 16 independent 32x32x64 MFMAs),
    the best of `reps` launches (~0.9 ms each, back to back: the clock settles over the
    first few) timed with events taken by the kernel's own dispatch."""
    torch = __import__("torch")
    sink = torch.empty(cus * 256, dtype=torch.float32, device=dev)
    flops = float(cus) * 4 * iters * 16 * 2 * 32 * 32 * 64
    cs = torch.cuda.current_stream().cuda_stream
    best = None
    for _ in range(reps + 1):  # the first launch loads the kernel
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        b.record()
        torch.cuda.synchronize()
        st = plib.probe_mfma(cus, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(cs),
                             ctypes.c_void_p(a.cuda_event), ctypes.c_void_p(b.cuda_event))
        if st != 0:
            raise RuntimeError("probe_mfma failed: %d" % st)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3
        best = us if best is None or us < best else best
    return {"pflops": round(flops / best / 1e9, 3), "best_us": round(best, 2),
            "launch": "%d blocks x 4 wavefronts, %d x 16 MFMA 32x32x64 FP8 each" % (cus, iters)}


def stream_ceiling(plib, dev, units, sets, reps, cus):
    """The quantize pass's traffic without its arithmetic (16 B read + 8 B written per 8
    bf16 elements), timed like the quantize kernel (events attached to each launch, `sets`
    rotating buffers): the fastest of a sweep of loads in flight per thread and blocks per
    CU, with each of the quantize kernel's two cache-policy sets (non-temporal loads with
    device-scope stores, or with non-temporal device-scope stores: the kernel's choice
    for launches whose codes exceed the Infinity Cache), and with default ones; plus
    read-only and write-only rates of the same sizes (best of the same sweep).  rw_2to1
    is the faster of the kernel's two sets."""
    import torch
    srcs = [torch.empty(units * 16, dtype=torch.uint8, device=dev) for _ in range(sets)]
    for s in srcs:
        s.random_(0, 256)
    dsts = [torch.empty(units * 8, dtype=torch.uint8, device=dev) for _ in range(sets)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def best(mode, policy):
        by_bytes = {0: 24, 1: 16, 2: 8}[mode] * units
        out = None
        for u in (4, 8, 16):
            for bpc in (1, 2, 4, 8):
                blocks = cus * bpc
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(reps)]
                for a, b in ev:
                    a.record()
                    b.record()
                for i in range(reps + 2):
                    e = ev[i - 2] if i >= 2 else (None, None)
                    st = plib.probe_stream(srcs[i % sets].data_ptr(), dsts[i % sets].data_ptr(),
                                           units, mode, u, blocks, policy, sink.data_ptr(),
                                           stream, e[0].cuda_event if e[0] else None,
                                           e[1].cuda_event if e[1] else None)
                    if st != 0:
                        raise RuntimeError("probe_stream failed: %d" % st)
                torch.cuda.synchronize()
                us = 1e3 * float(np.mean([a.elapsed_time(b) for a, b in ev]))
                gbps = by_bytes / (us * 1e-6) / 1e9
                if out is None or gbps > out["gbps"]:
                    out = {"gbps": round(gbps, 1), "avg_us": round(us, 3), "loads_per_thread": u,
                           "blocks_per_cu": bpc}
        return out

    sc1, nt = best(0, 1), best(0, 2)
    sc1["stores"], nt["stores"] = "sc1", "nt sc1"
    res = {"bytes_2to1": 24 * units, "rotating_sets": sets,
           "rw_2to1": dict(nt if nt["gbps"] > sc1["gbps"] else sc1),
           "rw_2to1_sc1_stores": sc1, "rw_2to1_nt_stores": nt,
           "rw_2to1_default_policy": best(0, 0),
           "read_only": best(1, 1), "write_only": best(2, 1)}
    del srcs, dsts
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mlp_12288",
                    choices=["single_1024", "mlp_4096", "grad_8192x16384", "mlp_12288"])
    ap.add_argument("--no-others", action="store_true",
                    help="skip the steps of the other large workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-list", action="store_true",
                    help="skip the 1152-tensor list (32-entry launches against one planned "
                         "launch)")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the stream ceiling and update floor probes")
    ap.add_argument("--no-gelu", action="store_true",
                    help="skip the gelu-fused quantize measurement")
    ap.add_argument("--no-ln", action="store_true",
                    help="skip the layernorm-fused quantize measurement")
    ap.add_argument("--no-gemm", action="store_true",
                    help="skip the FP8 GEMM consumer comparison")
    ap.add_argument("--no-torch-ops", action="store_true",
                    help="skip the context run of the update as small torch ops (~15k tiny "
                         "launches; keep it out of profiler runs)")
    ap.add_argument("--update-calls", type=int, default=200)
    ap.add_argument("--rotate", type=int, default=3,
                    help="input/output sets used in turn by successive steps")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0 or args.rotate < 1 or args.update_calls < 1:
        ap.error("--steps, --rotate and --update-calls must be >= 1, --warmup >= 0")
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (the amax "
              "all-reduce across replicas is described in the design notes, not built); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import delayed_scaling_amax_amd as d
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    threads = workloads.default_threads()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    K = args.steps

    # ------------------------------------------------------------ the headline step
    t0 = time.time()
    w = workloads.make(args.workload, threads=threads)
    log("generated %s (%d tensors, %d elements) in %.1fs" % (w.name, len(w.tensors), w.numel,
                                                             time.time() - t0))
    sb = StepBench(w, dev, args.rotate)
    first_codes, first_amax, first_meta = sb.first_step()
    head = sb.run(K, args.warmup)
    n, fmts = sb.n, sb.fmts
    qbytes, ubytes = sb.qbytes, sb.ubytes
    del sb
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ the other large workloads
    others = {}
    w4096 = None
    codes4096 = None
    scale4096 = None
    if not args.no_others:
        for name in OTHER_WORKLOADS:
            if name == w.name:
                continue
            ow = workloads.make(name, threads=threads)
            osb = StepBench(ow, dev, args.rotate)
            r = osb.run(K, args.warmup)
            others[name] = {
                "description": ow.description, "elements": ow.numel,
                "alg_bytes_quantize": osb.qbytes, "ms_per_step": round(r["ms_per_step"], 5),
                "value_gbps": round(r["value_gbps"], 1),
                "quantize_avg_us": round(r["q_avg_us"], 3),
                "quantize_median_us": round(r["q_median_us"], 3),
                "quantize_gbps": round(r["q_gbps"], 1),
                "quantize_frac_hbm_peak": round(r["q_gbps"] / PEAK_HBM_GBPS, 4),
                "one_launch_step": r["one_launch"]}
            if name == "mlp_4096":  # the GEMM consumer runs on these codes and scales
                w4096, codes4096, scale4096 = ow, osb.outs[0], osb.scale
            del osb
            torch.cuda.empty_cache()
    if w.name == "mlp_4096":
        w4096 = w

    # ------------------------------------------------------------ 1152-tensor list
    # the 1152 FP8 tensors of the batched-update layout as one quantize list: through
    # fp8_multi_quantize_amax (one launch per 32 entries: 36) and through one planned
    # launch; host time per call (the C entry points called directly, the ctypes entry
    # array built once, so the binding's marshalling is not timed) and device time per
    # call (events around K back-to-back calls)
    list_out = None
    if not args.no_list:
        lw = workloads.make("list_1152", threads=threads)
        lfm = [0 if t.fmt == workloads.E4M3 else 1 for t in lw.tensors]
        lsrc = [torch.from_numpy(t.data.reshape(-1).view(np.int16)).view(torch.bfloat16).to(dev)
                for t in lw.tensors]
        ldst = [torch.empty(x.numel(), dtype=torch.uint8, device=dev) for x in lsrc]
        lscale = torch.ones(len(lsrc), dtype=torch.float32, device=dev)
        lamax = torch.zeros(len(lsrc), dtype=torch.float32, device=dev)
        lent = [(lsrc[i], ldst[i], lscale[i:i + 1], lamax[i:i + 1], lfm[i])
                for i in range(len(lsrc))]
        arr = d._entry_table(lent, dev)
        t0 = time.perf_counter()
        plan = d.fp8_multi_quantize_plan(lent)
        torch.cuda.synchronize()
        plan_us = (time.perf_counter() - t0) * 1e6
        cs = torch.cuda.current_stream(dev).cuda_stream
        pdesc = ctypes.byref(plan.desc)

        def chunked():
            d._check("fp8_multi_quantize_amax", d.lib.fp8_multi_quantize_amax(arr, len(lent), cs))

        def planned():
            d._check("fp8_multi_quantize_amax_planned",
                     d.lib.fp8_multi_quantize_amax_planned(pdesc, cs))

        def per_call(fn):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            a.record()
            for _ in range(K):
                fn()
            b.record()
            t_enq = time.perf_counter()
            torch.cuda.synchronize()
            return (t_enq - t0) * 1e6 / K, 1e3 * a.elapsed_time(b) / K

        c_host, c_dev = per_call(chunked)
        p_host, p_dev = per_call(planned)
        # the two forms' outputs are compared (codes of every tensor, amax bits)
        lamax.zero_()
        chunked()
        torch.cuda.synchronize()
        ref_codes = [x.clone() for x in ldst]
        ref_amax = lamax.clone()
        lamax.zero_()
        for x in ldst:
            x.zero_()
        planned()
        torch.cuda.synchronize()
        same = all(torch.equal(ref_codes[i], ldst[i]) for i in range(len(ldst))) and \
            torch.equal(ref_amax.view(torch.int32), lamax.view(torch.int32))
        lb = alg_bytes_quantize(lw)
        list_out = {"workload": lw.name, "description": lw.description,
                    "elements": lw.numel, "alg_bytes": lb, "tensors": len(lent),
                    "chunked_launches_per_call": -(-len(lent) // 32),
                    "chunked_host_us_per_call": round(c_host, 2),
                    "chunked_device_us_per_call": round(c_dev, 2),
                    "planned_host_us_per_call": round(p_host, 2),
                    "planned_device_us_per_call": round(p_dev, 2),
                    "planned_gbps": round(lb / (p_dev * 1e-6) / 1e9, 1),
                    "plan_build_us": round(plan_us, 1),
                    "planned_equals_chunked": bool(same)}
        log("list_1152: 36 launches %.1f us host / %.1f us device per call; one planned "
            "launch %.1f us host / %.1f us device (%.1f GB/s); plan built in %.0f us; %s" % (
                c_host, c_dev, p_host, p_dev, lb / (p_dev * 1e-6) / 1e9, plan_us,
                "identical" if same else "MISMATCH"))
        del lsrc, ldst, lent, plan, ref_codes
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ batched update, 1152 tensors
    uw = workloads.update_1152(threads=threads)
    un, uH = uw.amax.size, uw.history_len
    u_amax = torch.from_numpy(uw.amax).to(dev)
    u_hist = torch.from_numpy(uw.hist).to(dev)
    u_scale = torch.from_numpy(uw.scale).to(dev)
    u_sinv = torch.empty_like(u_scale)
    u_fmt = torch.tensor([0 if f == workloads.E4M3 else 1 for f in uw.formats],
                         dtype=torch.uint8, device=dev)

    def update_1152():
        d.fp8_amax_and_scale_update(u_amax, u_hist, u_scale, u_sinv, u_fmt, margin=0)

    for _ in range(10):
        update_1152()
    torch.cuda.synchronize()
    C = args.update_calls
    # (a) device time per call, back to back, in a replayed HIP graph
    graph_us = graph_us_per_call(update_1152, C)
    # floors on the update's own grid, the same way: an empty kernel, and one
    # load -> barrier -> store round trip over the rows the update loads
    floors = None
    if not args.no_probes:
        plib = probe_lib()
        f_hist = torch.from_numpy(uw.hist).to(dev)
        fstream = torch.cuda.current_stream(dev)

        def floor(mode):
            def f():
                st = plib.probe_update_floor(f_hist.data_ptr(), un, uH, mode,
                                             torch.cuda.current_stream(dev).cuda_stream)
                if st != 0:
                    raise RuntimeError("probe_update_floor failed: %d" % st)
            f()
            torch.cuda.synchronize()
            return graph_us_per_call(f, C)

        floors = {"empty_kernel_us": floor(0), "one_round_trip_us": floor(1)}
        floors = {k: (round(v, 3) if v else None) for k, v in floors.items()}
        del f_hist, fstream
    # (b) per-call events (include event-record overhead)
    uev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(C)]
    for a, b in uev:
        a.record()
        update_1152()
        b.record()
    torch.cuda.synchronize()
    warm_us = 1e3 * float(np.median([a.elapsed_time(b) for a, b in uev]))
    # (c) host wall time per call through the Python binding
    t0 = time.perf_counter()
    for _ in range(C):
        update_1152()
    torch.cuda.synchronize()
    wall_us = (time.perf_counter() - t0) * 1e6 / C
    # (d) cold: L2 and MALL flushed by a 1 GiB write before each call
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(20):
        flush.fill_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        update_1152()
        b.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    cold_us = 1e3 * float(np.median(cold))
    del flush
    ub1152 = alg_bytes_update(un, uH)
    log("update 1152x%d: graph-replay %s us/call (floors: empty %s, round trip %s), events "
        "warm %.2f us, cold %.2f us, host wall %.2f us/call" % (
            uH, "%.2f" % graph_us if graph_us else "n/a",
            floors and floors["empty_kernel_us"], floors and floors["one_round_trip_us"],
            warm_us, cold_us, wall_us))
    # (e) context only, never in the library: the same update as a sequence of small torch
    #     ops per module call (roll, insert, max, divide, guard, reciprocal, reset: ~10
    #     launches for the module's 3 tensors), the per-call pattern the fused kernel
    #     replaces; 384 module calls, host wall time for all of them
    torch_ops_us = None
    if not args.no_torch_ops:
        fmax = torch.where(u_fmt == 0, torch.tensor(448.0, device=dev),
                           torch.tensor(57344.0, device=dev))
        u_hist_t = u_hist.clone()
        u_amax_t = u_amax.clone()
        u_scale_t = u_scale.clone()
        u_sinv_t = torch.empty_like(u_sinv)

        def update_torch_ops():
            for m in range(un // 3):
                cs = slice(3 * m, 3 * m + 3)
                h = torch.roll(u_hist_t[:, cs], 1, 0)
                h[0] = u_amax_t[cs]
                u_hist_t[:, cs] = h
                sel = h.max(0).values
                sc = sel / fmax[cs]
                ok = torch.isfinite(sc) & (sc > 0)
                u_scale_t[cs] = torch.where(ok, sc, u_scale_t[cs])
                u_sinv_t[cs] = 1.0 / u_scale_t[cs]
                u_amax_t[cs] = 0.0

        update_torch_ops()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(3):
            update_torch_ops()
        torch.cuda.synchronize()
        torch_ops_us = (time.perf_counter() - t0) * 1e6 / 3
        del u_hist_t, u_amax_t, u_scale_t, u_sinv_t
        log("update 1152x%d as small torch ops per module call: %.0f us per update" % (
            uH, torch_ops_us))

    # ------------------------------------------------------------ achievable stream rates
    ceilings = None
    if not args.no_probes:
        plib = probe_lib()
        ceilings = {}
        # 0.5 GB (the hidden-4096 step's 167.8 M elements, three rotating sets, like the
        # step) and 4 GB (the hidden-12288 step's 1.36 G elements)
        for label, elems, sets in (("0.5GB", 167772160, 3), ("4GB", 1358954496, 1)):
            ceilings[label] = stream_ceiling(plib, dev, elems // 8, sets, 10, cus)
            torch.cuda.empty_cache()
            log("stream %s: 2:1 read:write %.1f GB/s (sc1 stores %.1f, nt stores %.1f, "
                "default policies %.1f), read-only %.1f, write-only %.1f" % (
                    label, ceilings[label]["rw_2to1"]["gbps"],
                    ceilings[label]["rw_2to1_sc1_stores"]["gbps"],
                    ceilings[label]["rw_2to1_nt_stores"]["gbps"],
                    ceilings[label]["rw_2to1_default_policy"]["gbps"],
                    ceilings[label]["read_only"]["gbps"], ceilings[label]["write_only"]["gbps"]))

    # ------------------------------------------------------------ dequantize (not in the step)
    # one 67,108,864-element tensor of codes (the hidden-4096 MLP's wi shape) back to bf16
    dq_n = 1 << 26
    dq_codes = torch.randint(0, 256, (dq_n,), dtype=torch.uint8, device=dev)
    dq_codes[(dq_codes & 0x7F) == 0x7F] = 0  # finite codes
    dq_scale = torch.tensor([1.0 / 448.0], dtype=torch.float32, device=dev)
    dq_out = torch.empty(dq_n, dtype=torch.bfloat16, device=dev)
    dq_us = timed_launches(lambda i: d.fp8_dequantize(dq_codes, dq_out, dq_scale, 0))
    dq_bytes = 3 * dq_n + 4
    del dq_out, dq_codes

    # ------------------------------------------------------------ gelu-fused quantize
    # (not in the step) the FFN activation of mlp_4096: bf16 pre-activation (2048,4,16384)
    # -> gelu -> E4M3 + amax in one kernel, against the unfused sequence (torch's tanh
    # gelu writing the bf16 activation, then the plain quantize reading it back)
    gelu_out = None
    if not args.no_gelu:
        gw = workloads.make("mlp_4096_preact", threads=threads)
        gsets = [torch.from_numpy(gw.tensors[0].data.reshape(-1).view(np.int16)).view(
            torch.bfloat16).to(dev)]
        gsets.append(gsets[0].clone())
        gn = gsets[0].numel()
        gdst = torch.empty(gn, dtype=torch.uint8, device=dev)
        gy = torch.empty(gn, dtype=torch.bfloat16, device=dev)
        gscale = torch.tensor([0.0078125], dtype=torch.float32, device=dev)
        gamax = torch.zeros(1, dtype=torch.float32, device=dev)

        def fused(i):
            d.fp8_gelu_quantize_amax(gsets[i % 2], gdst, gscale, gamax, 0)

        def unfused(i):
            torch.ops.aten.gelu.out(gsets[i % 2], approximate="tanh", out=gy)
            d.fp8_quantize_amax(gy, gdst, gscale, gamax, 0)

        f_us = timed_launches(fused)
        u_us = timed_launches(unfused)
        g_bytes = 3 * gn + 8
        gelu_out = {"workload": gw.name, "elements": gn, "format": "e4m3",
                    "fused_events_median_us": round(f_us, 3),
                    "fused_gbps": round(g_bytes / (f_us * 1e-6) / 1e9, 1),
                    "fused_alg_bytes": g_bytes,
                    "unfused_events_median_us": round(u_us, 3),
                    "unfused": "torch gelu(tanh) bf16 out + fp8_quantize_amax",
                    "speedup": round(u_us / f_us, 3)}
        log("gelu fused %.2f us (%.1f GB/s), unfused %.2f us" % (
            f_us, g_bytes / (f_us * 1e-6) / 1e9, u_us))
        del gsets, gdst, gy

    # ------------------------------------------------------------ layernorm-fused quantize
    # (not in the step) the transformer block's LayerNorm in front of the MLP: bf16 input
    # (2048,4,4096) (the mlp_4096 activation) -> LayerNorm (gamma, beta, eps 1e-6) ->
    # E4M3 + amax + per-row mean/rstd in one kernel, against torch's layer_norm writing
    # the bf16 output followed by the plain quantize.  Four input copies rotate so the
    # 67 MB input streams from HBM rather than the MALL.
    ln_out = None
    if not args.no_ln:
        lx0 = torch.from_numpy(w_ln_input(workloads, threads, w4096)).view(torch.bfloat16).to(dev)
        lsets = [lx0] + [lx0.clone() for _ in range(3)]
        lrows, lH = lx0.shape
        ln_ = lrows * lH
        gen = torch.Generator(device="cpu").manual_seed(12)
        lg = (1 + 0.1 * torch.randn(lH, generator=gen)).to(dev)
        lb = (0.1 * torch.randn(lH, generator=gen)).to(dev)
        lg16, lb16 = lg.to(torch.bfloat16), lb.to(torch.bfloat16)
        ldst = [torch.empty(ln_, dtype=torch.uint8, device=dev) for _ in range(2)]
        lmean = torch.empty(lrows, dtype=torch.float32, device=dev)
        lrstd = torch.empty(lrows, dtype=torch.float32, device=dev)
        lscale = torch.tensor([1 / 64], dtype=torch.float32, device=dev)
        lamax = torch.zeros(1, dtype=torch.float32, device=dev)

        def ln_fused(i):
            d.fp8_layernorm_quantize_amax(lsets[i % 4], ldst[i % 2], lscale, lamax, 0,
                                          gamma=lg, beta=lb, eps=1e-6, mean=lmean, rstd=lrstd)

        def ln_unfused(i):
            y = torch.nn.functional.layer_norm(lsets[i % 4], (lH,), lg16, lb16, 1e-6)
            d.fp8_quantize_amax(y, ldst[i % 2], lscale, lamax, 0)

        lf_us = timed_launches(ln_fused)
        lu_us = timed_launches(ln_unfused)
        l_bytes = 3 * ln_ + 8 * lrows + 8 * lH + 8
        ln_out = {"workload": "mlp_4096 activation (2048,4,4096) as the LayerNorm input",
                  "elements": ln_, "hidden": lH, "format": "e4m3",
                  "fused_events_median_us": round(lf_us, 3),
                  "fused_gbps": round(l_bytes / (lf_us * 1e-6) / 1e9, 1),
                  "fused_alg_bytes": l_bytes,
                  "unfused_events_median_us": round(lu_us, 3),
                  "unfused": "torch layer_norm bf16 out + fp8_quantize_amax",
                  "speedup": round(lu_us / lf_us, 3)}
        log("layernorm fused %.2f us (%.1f GB/s), unfused %.2f us" % (
            lf_us, l_bytes / (lf_us * 1e-6) / 1e9, lu_us))
        del lsets, ldst

    # ------------------------------------------------------------ FP8 GEMM consumer
    # (not in the step) the hidden-4096 MLP's two dense layers on the codes its step
    # produced: the activation (8192 x 4096 E4M3) times wi (its 16384 x 4096 codes read
    # K-contiguous), and an (8192 x 16384) E4M3 activation (seeded N(0,1) x 40) times wo
    # (its 4096 x 16384 codes); the step's per-tensor scales (the dequantization
    # multipliers) as the operand scales, bf16 out.  torch._scaled_mm (hipBLASLt) on the
    # same operands alongside.
    gemm_out = None
    if not args.no_gemm and codes4096 is not None:
        gen = torch.Generator(device=dev).manual_seed(12)
        h_codes = (torch.randn(8192, 16384, device=dev, generator=gen) * 40).to(
            torch.float8_e4m3fn).view(torch.uint8)
        cases = [("wi", codes4096[0].view(8192, 4096), codes4096[1].view(16384, 4096), 0, 1),
                 ("wo", h_codes, codes4096[2].view(4096, 16384), 0, 2)]
        gemm_out = {"peak_tflops": PEAK_FP8_TFLOPS, "out": "bf16", "shapes": []}
        for name, A, B, ia, ib in cases:
            gm, gk = A.shape
            gn = B.shape[0]
            gc = torch.empty(gm, gn, dtype=torch.bfloat16, device=dev)
            sa, sb_ = scale4096[ia:ia + 1], scale4096[ib:ib + 1]
            g_us = timed_launches(lambda i: d.fp8_gemm(A, 0, B, 0, sa, sb_, gc))
            flops = 2.0 * gm * gn * gk
            rec = {"layer": name, "M": gm, "N": gn, "K": gk, "events_median_us": round(g_us, 3),
                   "tflops": round(flops / g_us / 1e6, 1),
                   "frac_fp8_peak": round(flops / g_us / 1e6 / PEAK_FP8_TFLOPS, 4)}
            try:
                A8, B8 = A.view(torch.float8_e4m3fn), B.view(torch.float8_e4m3fn)
                t_us = timed_launches(lambda i: torch._scaled_mm(
                    A8, B8.t(), scale_a=sa, scale_b=sb_, out_dtype=torch.bfloat16))
                rec["torch_scaled_mm_us"] = round(t_us, 3)
                rec["torch_scaled_mm_tflops"] = round(flops / t_us / 1e6, 1)
            except (RuntimeError, TypeError) as e:
                rec["torch_scaled_mm"] = "unavailable: %s" % str(e)[:80]
            gemm_out["shapes"].append(rec)
            log("gemm %s %dx%dx%d: %.1f us (%.0f TFLOP/s)%s" % (
                name, gm, gn, gk, g_us, flops / g_us / 1e6,
                ", torch._scaled_mm %.1f us" % rec["torch_scaled_mm_us"]
                if "torch_scaled_mm_us" in rec else ""))
            del gc
        del h_codes
        if not args.no_probes:
            # the ceiling the GEMM is measured against: the same MFMA with register operands
            gemm_out["mfma_ceiling"] = mfma_ceiling(probe_lib(), dev, cus)
            log("mfma ceiling (register operands, 32x32x64 FP8): %.2f PFLOP/s" % (
                gemm_out["mfma_ceiling"]["pflops"]))
    del codes4096, scale4096

    # ------------------------------------------------------------ copy context
    cbuf = torch.empty(1 << 27, dtype=torch.float32, device=dev)  # 512 MiB
    cdst = torch.empty_like(cbuf)
    for _ in range(3):
        cdst.copy_(cbuf)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(10):
        cdst.copy_(cbuf)
    b.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * cbuf.numel() * 4 * 10 / (a.elapsed_time(b) * 1e-3) / 1e9
    del cbuf, cdst

    traffic = measured_traffic(w.name, roofline_kernel(w))
    q_gbps = head["q_gbps"]
    upd_roof = None
    if graph_us:
        upd_roof = {"bound": "hbm", "kernel": "amax_and_scale_update_kernel<4>",
                    "achieved": round(ub1152 / (graph_us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(ub1152 / (graph_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                    "alg_bytes": ub1152, "timing": "graph replay, us per call"}
    out = {
        "metric": METRIC, "value": round(head["value_gbps"], 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["ms_per_step"], 5),
        "device_ms_per_step": round(head["device_ms_per_step"], 5),
        "host_enqueue_us_per_step": round(head["host_enqueue_us_per_step"], 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded numpy PCG64, seed 12; shapes/distributions of the workload)",
        "config": {"workload": w.name, "description": w.description, "tensors": n,
                   "elements": w.numel, "history_len": w.history_len,
                   "formats": [t.fmt for t in w.tensors], "src_dtype": "bf16",
                   "alg_bytes_step": qbytes + ubytes, "rotating_input_sets": args.rotate},
        "one_launch_step": head["one_launch"],
        "quantize_amax": {"entry": "fp8_multi_quantize_amax",
                          "timing": "HIP events set to each launch's kernel start/stop "
                                    "(hipExtLaunchKernel), every step of the second region",
                          "avg_us": round(head["q_avg_us"], 3),
                          "median_us": round(head["q_median_us"], 3),
                          "gbps": round(q_gbps, 1),
                          "pct_hbm_peak": round(100 * q_gbps / PEAK_HBM_GBPS, 2),
                          "alg_bytes": qbytes},
        "other_workloads": others,
        "multi_tensor_list": list_out,
        "stream_ceiling": ceilings,
        "scale_update_us": {"workload": "update_1152 (96 layers x 4 linears x 3 tensors, "
                                        "history 1024, margin 0, in place, one launch)",
                            "graph_replay_us_per_call": (round(graph_us, 3) if graph_us
                                                         else None),
                            "floors_graph_replay_us": floors,
                            "events_warm_us": round(warm_us, 3),
                            "events_cold_us": round(cold_us, 3),
                            "host_wall_us_per_call": round(wall_us, 3),
                            "torch_ops_per_module_us_per_update": (
                                round(torch_ops_us, 1) if torch_ops_us else None),
                            "alg_bytes": ub1152,
                            "step_update_and_gaps_us": round(head["u_gap_avg_us"], 3)},
        "update_roofline": upd_roof,
        "dequantize": {"elements": dq_n, "out": "bf16", "events_median_us": round(dq_us, 3),
                       "gbps": round(dq_bytes / (dq_us * 1e-6) / 1e9, 1)},
        "gelu_quantize": gelu_out,
        "layernorm_quantize": ln_out,
        "fp8_gemm": gemm_out,
        "copy_d2d_gbps": round(copy_gbps, 1),
        "roofline": {"bound": "hbm", "kernel": roofline_kernel(w) + " (fp8_multi_quantize_amax)",
                     "achieved": round(q_gbps, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(q_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic},
    }

    # ------------------------------------------------------------ CPU oracle baseline
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.load()
        cpus = host_cpus()

        def oracle_step():
            amax_o = np.zeros(n, np.float32)
            codes_o = []
            for i, t in enumerate(w.tensors):
                c, amax_o[i] = orc.quantize_amax(t.data, fmts[i], float(w.first_scale[i]),
                                                 threads=cpus)
                codes_o.append(c)
            meta = orc.amax_and_scale_update(amax_o, np.zeros((w.history_len, n), np.float32),
                                             np.asarray(w.first_scale, np.float32),
                                             np.array(fmts, np.uint8), reset_amax=True)
            return codes_o, amax_o, meta

        # the first step is compared with the GPU's (codes, amax, and after the update
        # the history, scale, scale_inv and reset amax, all bit for bit); whole steps are
        # repeated until at least 10 s of oracle work have been timed (at most 100 steps)
        t0 = time.perf_counter()
        codes_o, o_amax, o_meta = oracle_step()
        reps = 1
        same = all(np.array_equal(c.reshape(-1), first_codes[i]) for i, c in enumerate(codes_o))
        same &= bool((o_amax.view(np.uint32) == first_amax.view(np.uint32)).all())
        same &= all(np.array_equal(o_meta[k].view(np.uint32), first_meta[k].view(np.uint32))
                    for k in ("hist", "scale", "scale_inv", "amax"))
        del codes_o
        while time.perf_counter() - t0 < 10.0 and reps < 100:
            oracle_step()
            reps += 1
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(reps * (qbytes + ubytes) / dt / 1e9, 3),
                               "unit": "GB/s", "cores": cpus, "kind": "oracle",
                               "sample": "%d full steps of %s (all %d elements each, the first "
                                         "step's inputs and prior scales), %d threads over "
                                         "contiguous chunks (every CPU the process may use), "
                                         "%.1f s" % (reps, w.name, w.numel, cpus, dt)}
        # the same oracle on one thread, on the first tensor alone
        t1 = time.perf_counter()
        orc.quantize_amax(w.tensors[0].data, fmts[0], float(w.first_scale[0]), threads=1)
        dt1 = time.perf_counter() - t1
        e1 = int(w.tensors[0].data.size)
        out["cpu_baseline_one_thread"] = {
            "value": round(3 * e1 / dt1 / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "ns_per_element": round(dt1 * 1e9 / e1, 3),
            "sample": "quantize+amax of %s (%d elements), one thread, %.2f s" % (
                w.tensors[0].name, e1, dt1)}
        out["parity_first_step"] = "bit-exact" if same else "MISMATCH"
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
