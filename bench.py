"""Benchmark of the FP8 delayed-scaling hot path on one MI355X.

One step = one multi-tensor fused quantize+amax launch over every tensor of the
workload (bf16 -> FP8 with the previous step's scale) followed by one batched
amax_and_scale_update launch (history roll, amax selection, new scale/scale_inv, amax
reset), on inputs already resident in HBM; the same steps in one launch each
(fp8_quantize_amax_and_update) are timed beside.  Default workload: the MLP at hidden
4096 / ffn 16384 (activation (2048,4,4096), weights 4096x16384 and 16384x4096, all
E4M3, history 16).  Prints one JSON line.

Also measured in the same run: the batched update of 1152 tensors with history 1024
(kernel time warm and cold, host wall time per call), dequantize, the gelu-fused
quantize of the MLP's FFN activation against the unfused gelu-then-quantize sequence,
the LayerNorm-fused quantize against LayerNorm-then-quantize, the FP8 GEMM consumer
on the MLP's two dense shapes against torch._scaled_mm, a device-to-device copy as the achievable-bandwidth context, and the CPU oracle on the same step (cpu_baseline), whose
output is compared byte for byte with the GPU's first step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 matrix throughput, published
METRIC = "fused quantize+amax GB/s & % HBM peak; µs per batched scale update"
KERNEL_SOURCE = os.path.join(ROOT, "delayed_scaling_amax_amd", "csrc", "quantize_amax.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "quantize_amax_mlp_4096_traffic.txt")
ROOFLINE_KERNEL = "quantize_amax_kernel<1, false>"  # the multi-tensor quantize, bf16 sources


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for name in ("quantize_amax.hip", "quant_math.h", "device_common.h", "host_common.h"):
        with open(os.path.join(ROOT, "delayed_scaling_amax_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per quantize launch from the committed rocprofv3 counter summary, or
    None if absent, for another workload or kernel, or taken on a different kernel
    source."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if "=" in line and not line.startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if (kv.get("kernel_source_sha256_16") != kernel_hash() or kv.get("workload") != workload
                or kv.get("kernel") != ROOFLINE_KERNEL):
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


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


def w_ln_input(workloads, threads, w=None):
    """The LayerNorm input: the mlp_4096 activation (2048,4,4096) as (8192, 4096) bf16
    (taken from w when that is the mlp_4096 workload already generated)."""
    if w is None or w.name != "mlp_4096":
        w = workloads.mlp_4096(threads=threads)
    act = w.tensors[0].data
    return act.reshape(-1, act.shape[-1]).view(np.int16)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mlp_4096",
                    choices=["single_1024", "mlp_4096", "grad_8192x16384", "mlp_12288"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
        print("bench.py measures one GPU: this build has no multi-GPU path (the amax "
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

    # ------------------------------------------------------------ inputs in HBM
    t0 = time.time()
    w = workloads.make(args.workload, threads=threads)
    log("generated %s (%d tensors, %d elements) in %.1fs" % (w.name, len(w.tensors), w.numel,
                                                             time.time() - t0))
    fmts = [0 if t.fmt == workloads.E4M3 else 1 for t in w.tensors]
    n = len(w.tensors)
    # R copies of the inputs and outputs, used in turn by successive steps: a step's
    # tensors were last touched R-1 steps (>= 1 GB of traffic) earlier, so they stream
    # from HBM and not from the 256 MB MALL, as in a training step where the GEMMs run
    # between two quantizations of the same tensor
    srcs0 = [torch.from_numpy(t.data.view(np.int16)).view(torch.bfloat16).to(dev)
             for t in w.tensors]
    sets = [srcs0] + [[x.clone() for x in srcs0] for _ in range(args.rotate - 1)]
    outs = [[torch.empty(t.data.size, dtype=torch.uint8, device=dev) for t in w.tensors]
            for _ in range(args.rotate)]
    scale = torch.tensor(w.first_scale, dtype=torch.float32, device=dev)
    scale_inv = torch.empty(n, dtype=torch.float32, device=dev)
    amax = torch.zeros(n, dtype=torch.float32, device=dev)
    hist = torch.zeros(w.history_len, n, dtype=torch.float32, device=dev)
    fdev = torch.tensor(fmts, dtype=torch.uint8, device=dev)
    entry_sets = [[(sets[r][i], outs[r][i], scale[i:i + 1], amax[i:i + 1], fmts[i])
                   for i in range(n)] for r in range(args.rotate)]
    dsts = outs[0]
    step_no = [0]

    def quantize(events=None):
        if events is None:
            d.fp8_multi_quantize_amax(entry_sets[step_no[0] % args.rotate])
        else:  # the same launch, with events set to the kernel's own start and stop
            d.fp8_multi_quantize_amax_timed(entry_sets[step_no[0] % args.rotate], *events)
        step_no[0] += 1

    def update():
        d.fp8_amax_and_scale_update(amax, hist, scale, scale_inv, fdev, reset_amax=True)

    def step(events=None):
        """One step: the multi-tensor quantize + amax launch, then the batched update
        launch (reset amax)."""
        quantize(events)
        update()

    ws = torch.zeros(1, dtype=torch.int32, device=dev)  # the one-launch step's counter

    def one_launch_step(events=(None, None)):
        """The same step in one launch: the update runs in the block that finishes the
        quantize last."""
        d.fp8_quantize_amax_and_update(entry_sets[step_no[0] % args.rotate], amax, hist,
                                       scale, scale_inv, fdev, ws, reset_amax=True,
                                       start_event=events[0], stop_event=events[1])
        step_no[0] += 1

    # first step (prior scale): kept on the host for the parity check against the oracle
    quantize()
    torch.cuda.synchronize()
    first_codes = [x.cpu().numpy() for x in dsts]
    first_amax = amax.cpu().numpy().copy()
    update()
    torch.cuda.synchronize()
    first_meta = {"hist": hist.cpu().numpy().copy(), "scale": scale.cpu().numpy().copy(),
                  "scale_inv": scale_inv.cpu().numpy().copy(), "amax": amax.cpu().numpy().copy()}

    for _ in range(args.warmup):
        step()
        one_launch_step()  # the first launches of each kernel load it
    torch.cuda.synchronize()

    # Two timed regions of K steps each. (1) The steps alone, bracketed by two stream
    # events and the host clock, with a synchronize on both sides: `value` and
    # ms_per_step. (2) The same steps, each quantize launch carrying two HIP events that
    # take the kernel's own start and stop time (hipExtLaunchKernel): its live duration
    # for the roofline, without the dispatch latency that events recorded on the stream
    # around the call would add. Launches that carry events cost ~30 us more host time
    # each, which would make small steps host-bound, so (1) carries none.
    K = args.steps

    def make_events():
        e = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for a, b in e:  # torch creates an event at its first record
            a.record()
            b.record()
        return e

    def steps_region(fn):
        """(host wall ms per step, device ms per step, host enqueue us per step) of K
        calls of fn(k)."""
        region = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        region[0].record()
        for k in range(K):
            fn(k)
        region[1].record()
        t_enq = time.perf_counter()  # all K steps enqueued (the host runs ahead)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return ((t1 - t0) * 1e3 / K, region[0].elapsed_time(region[1]) / K,
                (t_enq - t0) * 1e6 / K)

    qbytes = alg_bytes_quantize(w)
    ubytes = alg_bytes_update(n, w.history_len)
    ms_per_step, dev_ms_per_step, enq_us = steps_region(lambda k: step())
    value = (qbytes + ubytes) / (ms_per_step * 1e-3) / 1e9
    ev = make_events()
    steps_region(lambda k: step(ev[k]))
    q_ms = [ev[k][0].elapsed_time(ev[k][1]) for k in range(K)]
    u_ms = [ev[k][1].elapsed_time(ev[k + 1][0]) for k in range(K - 1)] or [0.0]
    q_avg_us = 1e3 * float(np.mean(q_ms))
    q_gbps = qbytes / (q_avg_us * 1e-6) / 1e9
    log("step %.4f ms (device %.4f ms, host enqueue %.1f us); quantize avg %.2f us (median "
        "%.2f) = %.1f GB/s; update + gaps avg %.2f us" % (
            ms_per_step, dev_ms_per_step, enq_us, q_avg_us, 1e3 * float(np.median(q_ms)),
            q_gbps, 1e3 * float(np.mean(u_ms))))

    # The same K steps in one launch each (fp8_quantize_amax_and_update), timed the same
    # two ways.
    one_ms, one_dev_ms, one_enq_us = steps_region(lambda k: one_launch_step())
    ev1 = make_events()
    steps_region(lambda k: one_launch_step(ev1[k]))
    s_ms = [ev1[k][0].elapsed_time(ev1[k][1]) for k in range(K)]
    s_avg_us = 1e3 * float(np.mean(s_ms))
    s_gbps = (qbytes + ubytes) / (s_avg_us * 1e-6) / 1e9
    log("one-launch step %.4f ms (device %.4f ms, host enqueue %.1f us); kernel avg %.2f us "
        "(median %.2f) = %.1f GB/s" % (one_ms, one_dev_ms, one_enq_us, s_avg_us,
                                       1e3 * float(np.median(s_ms)), s_gbps))
    one_launch = {"entry": "fp8_quantize_amax_and_update (quantize + amax + update, one "
                           "launch)",
                  "ms_per_step": round(one_ms, 5), "device_ms_per_step": round(one_dev_ms, 5),
                  "host_enqueue_us_per_step": round(one_enq_us, 2),
                  "value_gbps": round((qbytes + ubytes) / (one_ms * 1e-3) / 1e9, 2),
                  "kernel_avg_us": round(s_avg_us, 3),
                  "kernel_median_us": round(1e3 * float(np.median(s_ms)), 3),
                  "kernel_gbps": round(s_gbps, 1)}

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
    # (a) device time per call, back to back: C calls captured in one HIP graph and
    #     replayed, so neither Python launch overhead nor per-call events are timed
    graph_us = None
    try:
        g = torch.cuda.CUDAGraph()
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            with torch.cuda.graph(g, stream=s_cap):
                for _ in range(C):
                    update_1152()
        torch.cuda.current_stream().wait_stream(s_cap)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        graph_us = 1e3 * a.elapsed_time(b) / (5 * C)
        del g
    except Exception as e:  # capture unsupported: report the other figures only
        log("graph capture of the update failed: %r" % (e,))
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
    log("update 1152x%d: graph-replay %s us/call, events warm %.2f us, cold %.2f us, host "
        "wall %.2f us/call" % (uH, "%.2f" % graph_us if graph_us else "n/a", warm_us, cold_us,
                               wall_us))
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

    # ------------------------------------------------------------ dequantize (not in the step)
    # codes of the largest tensor of the step back to bf16 with its scale
    big = max(range(n), key=lambda i: w.tensors[i].data.size)
    dq_out = torch.empty(w.tensors[big].data.size, dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        d.fp8_dequantize(dsts[big], dq_out, scale[big:big + 1], fmts[big])
    torch.cuda.synchronize()
    dq_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(20)]
    for a, b in dq_ev:
        a.record()
        d.fp8_dequantize(dsts[big], dq_out, scale[big:big + 1], fmts[big])
        b.record()
    torch.cuda.synchronize()
    dq_us = 1e3 * float(np.median([a.elapsed_time(b) for a, b in dq_ev]))
    dq_bytes = 3 * w.tensors[big].data.size + 4
    del dq_out

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
        lx0 = torch.from_numpy(w_ln_input(workloads, threads, w)).view(torch.bfloat16).to(dev)
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
    # (not in the step) the MLP's two dense layers on the codes the step produced: the
    # activation (8192 x 4096 E4M3) times wi (its 16384 x 4096 codes read K-contiguous),
    # and an (8192 x 16384) E4M3 activation (seeded N(0,1) x 40) times wo (its 4096 x
    # 16384 codes); the step's per-tensor scales (the dequantization multipliers) as the
    # operand scales, bf16 out.
    # torch._scaled_mm (hipBLASLt) on the same operands alongside.
    gemm_out = None
    if not args.no_gemm and w.name == "mlp_4096":
        gen = torch.Generator(device=dev).manual_seed(12)
        h_codes = (torch.randn(8192, 16384, device=dev, generator=gen) * 40).to(
            torch.float8_e4m3fn).view(torch.uint8)
        cases = [("wi", dsts[0].view(8192, 4096), dsts[1].view(16384, 4096), 0, 1),
                 ("wo", h_codes, dsts[2].view(4096, 16384), 0, 2)]
        gemm_out = {"peak_tflops": PEAK_FP8_TFLOPS, "out": "bf16", "shapes": []}
        for name, A, B, ia, ib in cases:
            gm, gk = A.shape
            gn = B.shape[0]
            gc = torch.empty(gm, gn, dtype=torch.bfloat16, device=dev)
            sa, sb = scale[ia:ia + 1], scale[ib:ib + 1]
            g_us = timed_launches(lambda i: d.fp8_gemm(A, 0, B, 0, sa, sb, gc))
            flops = 2.0 * gm * gn * gk
            rec = {"layer": name, "M": gm, "N": gn, "K": gk, "events_median_us": round(g_us, 3),
                   "tflops": round(flops / g_us / 1e6, 1),
                   "frac_fp8_peak": round(flops / g_us / 1e6 / PEAK_FP8_TFLOPS, 4)}
            try:
                A8, B8 = A.view(torch.float8_e4m3fn), B.view(torch.float8_e4m3fn)
                t_us = timed_launches(lambda i: torch._scaled_mm(
                    A8, B8.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16))
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

    traffic = measured_traffic(w.name)
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "device_ms_per_step": round(dev_ms_per_step, 5),
        "host_enqueue_us_per_step": round(enq_us, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded numpy PCG64, seed 12; shapes/distributions of the workload)",
        "config": {"workload": w.name, "description": w.description, "tensors": n,
                   "elements": w.numel, "history_len": w.history_len,
                   "formats": [t.fmt for t in w.tensors], "src_dtype": "bf16",
                   "rotating_input_sets": args.rotate},
        "one_launch_step": one_launch,
        "quantize_amax": {"entry": "fp8_multi_quantize_amax",
                          "timing": "HIP events set to each launch's kernel start/stop "
                                    "(hipExtLaunchKernel), every step of the second region",
                          "avg_us": round(q_avg_us, 3),
                          "median_us": round(1e3 * float(np.median(q_ms)), 3),
                          "gbps": round(q_gbps, 1), "pct_hbm_peak": round(100 * q_gbps /
                                                                          PEAK_HBM_GBPS, 2),
                          "alg_bytes": qbytes},
        "scale_update_us": {"workload": "update_1152 (96 layers x 4 linears x 3 tensors, "
                                        "history 1024, margin 0, in place, one launch)",
                            "graph_replay_us_per_call": (round(graph_us, 3) if graph_us
                                                         else None),
                            "events_warm_us": round(warm_us, 3),
                            "events_cold_us": round(cold_us, 3),
                            "host_wall_us_per_call": round(wall_us, 3),
                            "torch_ops_per_module_us_per_update": (
                                round(torch_ops_us, 1) if torch_ops_us else None),
                            "alg_bytes": alg_bytes_update(un, uH),
                            "step_update_and_gaps_us": round(1e3 * float(np.mean(u_ms)), 3)},
        "dequantize": {"tensor": w.tensors[big].name, "elements": int(w.tensors[big].data.size),
                       "out": "bf16", "events_median_us": round(dq_us, 3),
                       "gbps": round(dq_bytes / (dq_us * 1e-6) / 1e9, 1)},
        "gelu_quantize": gelu_out,
        "layernorm_quantize": ln_out,
        "fp8_gemm": gemm_out,
        "copy_d2d_gbps": round(copy_gbps, 1),
        "roofline": {"bound": "hbm", "kernel": ROOFLINE_KERNEL + " (fp8_multi_quantize_amax)",
                     "achieved": round(q_gbps, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(q_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic},
    }

    # ------------------------------------------------------------ CPU oracle baseline
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.load()

        def oracle_step():
            amax_o = np.zeros(n, np.float32)
            codes_o = []
            for i, t in enumerate(w.tensors):
                c, amax_o[i] = orc.quantize_amax(t.data, fmts[i], float(w.first_scale[i]),
                                                 threads=threads)
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
                               "unit": "GB/s", "cores": threads, "kind": "oracle",
                               "sample": "%d full steps of %s (all %d elements each, the first "
                                         "step's inputs and prior scales), %d threads over "
                                         "contiguous chunks, %.1f s" % (
                                             reps, w.name, w.numel, threads, dt)}
        # the same oracle on one thread, on the activation tensor alone (33.5 M elements)
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
