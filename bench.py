"""Benchmark of the FP8 W8A8 scaled-GEMM path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--workload NAME ...] [--no-cpu]
                    [--pmc-calibrate]

Prints ONE JSON line.

Headline step: the large-layer workload, a 4096 x 28672 x 8192 linear layer.
X is bf16 [4096, 8192] drawn from Student-t(3); W is E4M3 [28672, 8192] with one
fp32 scale per output channel, quantized and packed into the matrix-core
fragment order offline.  One step runs both activation-scale arms of the
workload on the same X, each as one fp8_scaled_gemm call in exact accumulation
mode with bf16 output:
  * dynamic per-token scales, the quantization inside the call;
  * the static per-tensor scale RN32(120/448), the quantization inside the call.
Each call is a quantization kernel followed by the GEMM kernel.  `value` is the
step's 2 x 2MNK flops divided by its time, in TFLOP/s; inputs are resident in
HBM before the timed region starts.

`roofline` is for the step's dominant kernel, the large-tile exact GEMM at that
shape (gemm_big_exact, packed W, packed A as the call's workspace holds it),
timed per launch with HIP events on the library's stream over >= 100 back-to-back
launches on pre-quantized A.  It is priced against the dense FP8 matrix-core
peak (5.0 PFLOP/s); the bf16 matrix cores that exact accumulation runs on
(2.5 PFLOP/s) are stated beside it, with the graphics clock the chip sustained
under that loop (read in-process through the amdsmi library).

`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
`details` carries every other measured workload (the decode-shaped step,
prefill GEMMs in both accumulation modes, the quantizers, the KV-cache passes,
the block-wise, FP8-output, attention, RMSNorm and MXFP8 rows).  Each timed row
reports the median, minimum and 90th percentile of >= 100 timed calls (or
>= 200 ms): per-call HIP events for kernels of 50 us and more, HIP-graph replays
of 20 calls for shorter ones (so the host's launch rate stays out of them).

Inputs are seeded and synthetic (see workloads/).  One GPU only: --gpus > 1
exits with a message.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fp8_scaled_gemm TFLOPS + quant GB/s at 1 MI355X, as % of MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # dense FP8 matrix cores
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 matrix cores
PEAK_CLOCK_MHZ = 2400.0        # the clock of the published peaks
# HBM traffic of the roofline kernel from two rocprofv3 counter passes over
# `bench.py --quick --no-cpu --pmc-calibrate` (FETCH_SIZE, then WRITE_SIZE, KiB
# per dispatch, median over the dispatches), each scaled by what the counter
# reads for the 1 GiB calibration copy (FETCH_SIZE reads half the copy's bytes
# on this part, WRITE_SIZE all of them).  Valid only for the kernel source it
# was measured on: when the hash of these files differs, traffic is reported
# as null until the counters are taken again.
TRAFFIC = {"kernel": "gemm_big_exact<1, true, true> at 4096x28672x8192",
           "sources": ("scaled_gemm_amd/csrc/gemm_big.hip", "scaled_gemm_amd/csrc/gemm_common.h",
                       "scaled_gemm_amd/csrc/fp8_device.h"),
           "sha256": ("69e64a81484b0706b840324b91c6c3fc556f03a5db7c13400369fd4d407d6599",
                      "034379e5e5ce5c636a91aedd49d9e72f1bce8256d60c515dd9e88a0386a20847",
                      "3995d5f1aeacc4692dd13a666aa64d28c436a937ad879d464ad4a126345ca691"),
           "fetch_kib": 688645.0, "write_kib": 229376.0,
           "fetch_factor": 1048576.0 / 524299.5, "write_factor": 1048576.0 / 1048576.0}
LARGE_M, LARGE_N, LARGE_K = 4096, 28672, 8192
DEC_N, DEC_K = 14336, 4096
DEC_MS = (1, 8, 32)
W_COPIES = 8


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--quick", action="store_true", help="headline and roofline kernel only: skip the details")
    ap.add_argument("--workload", nargs="*", default=None,
                    help="detail workloads to run (default all): decode prefill large quant kv weights blockwise "
                         "fp8out attention mx rmsnorm")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the sustained-clock loops (for counter runs, which serialise dispatches)")
    ap.add_argument("--pmc-calibrate", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling HBM counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stats(d_ms: np.ndarray) -> dict:
    """Median, minimum, 90th percentile and mean of per-call durations (us)."""
    d = np.asarray(d_ms, dtype=np.float64) * 1e3
    return {"median_us": round(float(np.median(d)), 3), "min_us": round(float(d.min()), 3),
            "p90_us": round(float(np.percentile(d, 90)), 3), "mean_us": round(float(d.mean()), 3),
            "calls": int(d.size)}


class Timer:
    """HIP-event timing on the current stream (the stream the library launches on)."""

    def __init__(self, torch):
        self.torch = torch

    def _ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def per_call(self, fn, warmup=10, min_calls=100, min_ms=200.0, max_calls=3000):
        """Per-call durations (ms) of fn(i): an event is recorded between every two
        back-to-back calls, so each duration is the kernels' own time plus the
        dispatch gap to the next call -- the figure a kernel trace reports when
        the host keeps the queue ahead of the GPU."""
        torch = self.torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        a, b = self._ev(), self._ev()
        a.record()
        for i in range(3):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        est = max(a.elapsed_time(b) / 3, 1e-3)
        n = int(min(max_calls, max(min_calls, math.ceil(min_ms / est))))
        ev = [self._ev() for _ in range(n + 1)]
        ev[0].record()
        for i in range(n):
            fn(i)
            ev[i + 1].record()
        torch.cuda.synchronize()
        return np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])

    def graph(self, fn, inner=20, warmup=3, min_reps=100, min_ms=200.0, max_reps=2000):
        """Per-call durations (ms) of short calls: `inner` calls of fn are captured
        into one HIP graph, whose replays are timed with events between them;
        each value is a replay's duration / inner."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(warmup):
                fn(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(inner):
                fn(i)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        a, b = self._ev(), self._ev()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        est = max(a.elapsed_time(b), 1e-3)
        n = int(min(max_reps, max(min_reps, math.ceil(min_ms / est))))
        ev = [self._ev() for _ in range(n + 1)]
        ev[0].record()
        for i in range(n):
            g.replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        out = np.array([ev[i].elapsed_time(ev[i + 1]) / inner for i in range(n)])
        del g
        return out


def gbs_row(workload, d_ms, nbytes, **extra):
    s = stats(d_ms)
    g = nbytes / (s["median_us"] * 1e-6) / 1e9
    row = {"workload": workload, **extra, **s, "GB_s": round(g, 1), "frac_hbm": round(g / HBM_PEAK_GBS, 4)}
    return row


def tflops_row(workload, d_ms, flops, accum=None, **extra):
    s = stats(d_ms)
    tf = flops / (s["median_us"] * 1e-6) / 1e12
    row = {"workload": workload, **extra, **s, "TFLOPS": round(tf, 1), "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4)}
    if accum is not None:
        row["accum"] = accum
        if accum == "exact":
            row["frac_bf16_peak"] = round(tf / BF16_PEAK_TFLOPS, 4)
    return row


# ----------------------------------------------------------------------------- graphics clock
class ClockReader:
    """The graphics clock of the benchmark's GPU, read in-process through the
    amdsmi library (no child process).  value() returns the mean of the XCD
    clocks in MHz, or None when the library or the metric is unavailable."""

    def __init__(self, torch):
        self.handle = None
        self.api = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            pick = handles[0] if len(handles) == 1 else None
            if pick is None:
                bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
                for h in handles:
                    bdf = str(amdsmi.amdsmi_get_gpu_device_bdf(h))
                    if bus is not None and int(bdf.split(":")[1], 16) == int(bus):
                        pick = h
            self.handle, self.api = pick, amdsmi
        except Exception as e:  # the reading is optional
            self.error = str(e)[:120]

    def power_w(self):
        """Socket power (W) now, or None."""
        if self.handle is None:
            return None
        try:
            p = self.api.amdsmi_get_power_info(self.handle)
            for k in ("socket_power", "current_socket_power", "average_socket_power"):
                v = p.get(k)
                if isinstance(v, (int, float)) and 0 < v < 100000:
                    return int(v)
        except Exception:
            pass
        return None

    def power_cap_w(self):
        """The board's power cap (W), or None."""
        if self.handle is None:
            return None
        try:
            v = self.api.amdsmi_get_power_cap_info(self.handle).get("power_cap")
            if isinstance(v, (int, float)) and v > 0:
                return int(v / 1e6) if v > 1e5 else int(v)   # reported in microwatts
        except Exception:
            pass
        return None

    def value(self):
        if self.handle is None:
            return None
        try:
            m = self.api.amdsmi_get_gpu_metrics_info(self.handle)
            c = m.get("current_gfxclks")
            c = [int(v) for v in (c or []) if isinstance(v, (int, float)) and 0 < v < 10000]
            if c:
                return round(sum(c) / len(c))
            v = m.get("current_gfxclk") or m.get("average_gfxclk_frequency")
            if isinstance(v, (int, float)) and 0 < v < 10000:
                return int(v)
        except Exception:
            pass
        try:
            v = self.api.amdsmi_get_clock_info(self.handle, self.api.AmdSmiClkType.GFX).get("clk")
            return int(v) if isinstance(v, (int, float)) and 0 < v < 10000 else None
        except Exception:
            return None


def sustained_clock(torch, clock, launch, launch_ms, seconds=2.5, settle=0.8, samples=6, gap=0.2, power=None):
    """Graphics clock while the GPU runs back-to-back launches of one kernel:
    about `seconds` of launches are queued, then after `settle` s the clock is
    read `samples` times (and the socket power into the list `power`, if given).
    Returns (readings or None, ms per launch of the loop)."""
    torch.cuda.synchronize()
    n = max(1, int(seconds * 1e3 / launch_ms))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        launch(i)
    b.record()
    vals = []
    if clock is not None and clock.handle is not None:
        time.sleep(settle)
        for _ in range(samples):
            v = clock.value()
            if v:
                vals.append(v)
            if power is not None:
                w = clock.power_w()
                if w:
                    power.append(w)
            time.sleep(gap)
    torch.cuda.synchronize()
    return (vals or None), a.elapsed_time(b) / n


def measured_traffic():
    """HBM bytes per launch of the roofline kernel from the recorded counters,
    or None when its source has changed since they were taken."""
    if TRAFFIC is None:
        return None
    import hashlib
    for rel, want in zip(TRAFFIC["sources"], TRAFFIC["sha256"]):
        with open(os.path.join(ROOT, rel), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != want:
                return None
    return int(round(1024 * (TRAFFIC["fetch_kib"] * TRAFFIC["fetch_factor"] +
                             TRAFFIC["write_kib"] * TRAFFIC["write_factor"])))


# ----------------------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import scaled_gemm_amd as sg
    from workloads import STATIC_SCALE_DEN, STATIC_SCALE_NUM, large_layer_inputs

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no HIP device"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    T = Timer(torch)

    def to_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ------------------------------------------------------------ headline inputs
    log("generating the large-layer inputs")
    M, N, K = LARGE_M, LARGE_N, LARGE_K
    xb_host, w_host = large_layer_inputs()
    x = to_bf16(xb_host)
    w_t = torch.from_numpy(w_host).to(dev)
    # offline: per-channel quantization of W, then the fragment order
    wq_rm, sw = sg.fp8_quant_weight_per_channel(w_t)
    del w_t
    wp = sg.fp8_pack_weights(wq_rm)
    s_static = float(np.float32(STATIC_SCALE_NUM) / np.float32(STATIC_SCALE_DEN))
    s_static_t = torch.tensor([s_static], dtype=torch.float32, device=dev)
    sa_dyn = torch.empty(M, dtype=torch.float32, device=dev)
    y_dyn = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    y_sta = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws_dyn = torch.empty(sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_token", M, N, K), dtype=torch.uint8,
                         device=dev)
    ws_sta = torch.empty(sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_tensor", M, N, K),
                         dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(i):
        sg.fp8_scaled_gemm(x, sa_dyn, wp, sw, y=y_dyn, workspace=ws_dyn, w_layout="packed")
        sg.fp8_scaled_gemm(x, s_static_t, wp, sw, y=y_sta, workspace=ws_sta, a_scale_mode="per_tensor",
                           w_layout="packed")

    # ------------------------------------------------------------ headline timing
    log(f"headline: warmup {args.warmup}, steps {args.steps}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record()
    for i in range(args.steps):
        step(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[-1])
    per_step = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    ms_per_step = total_ms / args.steps
    step_flops = 2 * 2.0 * M * N * K
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    # ------------------------------------------------------------ dominant kernel
    log("roofline kernel")
    # the codes the dynamic arm's call writes to its workspace: the fragment order (packed A)
    aq_rm, sa = sg.fp8_quant_per_token(x)
    aq = sg.fp8_pack_weights(aq_rm)
    torch.cuda.synchronize()

    def gemm_kernel(i):
        sg.fp8_scaled_gemm(aq, sa, wp, sw, y=y_dyn, w_layout="packed", a_layout="packed", a_shape=(M, K))

    d = T.per_call(gemm_kernel, warmup=10, min_calls=100)
    ks = stats(d)
    flops = 2.0 * M * N * K
    achieved = flops / (ks["mean_us"] * 1e-6) / 1e12
    clock = None if args.no_clock else ClockReader(torch)
    watts = []
    mhz = None if clock is None else sustained_clock(torch, clock, gemm_kernel, ks["mean_us"] * 1e-3, power=watts)[0]
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP8_PEAK_TFLOPS, 4), "traffic": measured_traffic(),
                "kernel": "gemm_big_exact<bf16 out, packed W, packed A> (exact accumulation on the bf16 matrix "
                          "cores), 4096x28672x8192",
                "flops_per_launch": flops, "avg_launch_us": ks["mean_us"], "launch_stats": ks,
                "bf16_matrix_core_peak": BF16_PEAK_TFLOPS,
                "frac_of_bf16_peak": round(achieved / BF16_PEAK_TFLOPS, 4),
                "timing": "HIP events between back-to-back launches on the library's stream; achieved uses the mean"}
    if mhz:
        clk = float(np.median(mhz))
        roofline["sustained_gfx_clock_mhz"] = clk
        roofline["frac_of_bf16_peak_at_sustained_clock"] = round(
            achieved / (BF16_PEAK_TFLOPS * clk / PEAK_CLOCK_MHZ), 4)
    else:
        roofline["sustained_gfx_clock_mhz"] = None
    # the matrix cores run this loop under the board's power cap, which sets the clock
    roofline["socket_power_w_samples"] = watts or None
    roofline["power_cap_w"] = None if clock is None else clock.power_cap_w()

    details = [{"workload": "headline step: per-step durations", **stats(per_step)}]
    # the two arms' calls on their own, and the quantization kernels inside them
    d = T.per_call(lambda i: sg.fp8_scaled_gemm(x, sa_dyn, wp, sw, y=y_dyn, workspace=ws_dyn, w_layout="packed"))
    details.append(tflops_row("large-layer call, bf16 X, per-token quant inside the call", d, flops, "exact"))
    d = T.per_call(lambda i: sg.fp8_scaled_gemm(x, s_static_t, wp, sw, y=y_sta, workspace=ws_sta,
                                                a_scale_mode="per_tensor", w_layout="packed"))
    details.append(tflops_row("large-layer call, bf16 X, static per-tensor quant inside the call", d, flops,
                              "exact"))
    wanted = set(args.workload) if args.workload else {"decode", "prefill", "large", "quant", "kv", "weights",
                                                       "blockwise", "fp8out", "attention", "mx", "rmsnorm"}
    if args.quick:
        wanted = set()
    if "large" in wanted:
        details += large_rows(sg, torch, dev, T, x, xb_host, w_host, wq_rm, wp, sw, aq_rm, sa, s_static, clock)
    del aq, aq_rm, sa, ws_dyn, ws_sta, y_dyn, y_sta, wp, wq_rm, x
    torch.cuda.empty_cache()
    if wanted - {"large"}:
        details += run_details(sg, torch, dev, to_bf16, T, wanted, clock)

    # ------------------------------------------------------------ copy calibration
    if args.pmc_calibrate:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        details.append({"workload": "calibration copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30,
                        "launches": 3})
        del src, dst

    # ------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(xb_host, w_host, s_static, log)

    out = {"metric": METRIC, "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "e4m3", "data": "synthetic (seeded, workloads/)",
           "config": {"workload": "large-layer W8A8 linear 4096x28672x8192: X bf16 [4096,8192] Student-t(3); "
                                  "W E4M3 [28672,8192] per-channel fp32 scales, packed offline; one step = the "
                                  "dynamic per-token arm and the static per-tensor arm (s = RN32(120/448)), each "
                                  "one fp8_scaled_gemm call with the quantization inside; exact fp32 "
                                  "accumulation; bf16 out",
                      "M": M, "N": N, "K": K, "accum": "exact", "w_layout": "packed", "calls_per_step": 2,
                      "flops_per_step": step_flops},
           "roofline": roofline, "cpu_baseline": cpu, "details": details}
    print(json.dumps(out), flush=True)


# ----------------------------------------------------------------------------- detail rows
def large_rows(sg, torch, dev, T, x, xb_host, w_host, wq_rm, wp, sw, aq, sa, s_static, clock):
    """The large layer in both accumulation modes and operand layouts, the FP8
    matrix cores' clock, and the static-vs-dynamic comparison.  aq: the per-token
    codes [M, K], row-major."""
    out = []
    M, K = x.shape
    N = sw.shape[0]
    flops = 2.0 * M * N * K
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    st = torch.tensor([s_static], dtype=torch.float32, device=dev)
    aq_s = sg.fp8_quant_per_tensor_static(x, st)
    ap = sg.fp8_pack_weights(aq)
    for accum, wl, a_in, al in (("mfma_fp8", "packed", ap, "packed"), ("mfma_fp8", "packed", aq, "row_major"),
                                ("exact", "packed", ap, "packed"), ("exact", "row_major", aq, "row_major")):
        wbuf = wp if wl == "packed" else wq_rm
        d = T.per_call(lambda i: sg.fp8_scaled_gemm(a_in, sa, wbuf, sw, y=y, accum=accum, w_layout=wl, a_layout=al,
                                                    a_shape=(M, K)), min_calls=50)
        out.append(tflops_row(f"large-layer GEMM kernel {M}x{N}x{K} (pre-quantized A)", d, flops, accum,
                              w_layout=wl, a_layout=al))
    del ap
    d = T.per_call(lambda i: sg.fp8_scaled_gemm(aq_s, st, wp, sw, y=y, a_scale_mode="per_tensor",
                                                w_layout="packed"), min_calls=50)
    out.append(tflops_row(f"large-layer GEMM kernel {M}x{N}x{K}, per-tensor scale (pre-quantized A)", d, flops,
                          "exact", w_layout="packed", a_layout="row_major"))
    f = lambda i: sg.fp8_scaled_gemm(aq, sa, wp, sw, y=y, accum="mfma_fp8", w_layout="packed")
    ms = float(stats(T.per_call(f, warmup=3, min_calls=5, min_ms=1))["mean_us"]) * 1e-3
    watts = []
    mhz, ms = sustained_clock(torch, clock, f, ms, power=watts) if clock is not None else (None, ms)
    row = {"workload": f"sustained graphics clock, large-layer GEMM {M}x{N}x{K} loop (FP8 matrix cores)",
           "accum": "mfma_fp8", "mean_us": round(ms * 1e3, 1), "mhz_samples": mhz, "socket_power_w_samples": watts}
    if mhz:
        clk = float(np.median(mhz))
        row["mhz_median"] = clk
        row["frac_of_fp8_peak_at_this_clock"] = round(flops / (ms * 1e-3) / 1e12 /
                                                      (FP8_PEAK_TFLOPS * clk / PEAK_CLOCK_MHZ), 4)
    out.append(row)
    # static vs dynamic on the same seed: saturated codes, and relative Frobenius error of Y
    # against the float64 product of the unquantized X and W, on 256 rows
    sat_static = int(((aq_s & 0x7F) == 0x7E).sum())
    sat_dyn = int(((aq & 0x7F) == 0x7E).sum())
    rows = torch.arange(0, M, M // 256, device=dev)[:256]
    w_t = torch.from_numpy(w_host).to(dev)
    ref = x[rows].double() @ w_t.double().t()
    rel = {}
    for tag, a_c, s_c, mode in (("static", aq_s, st, "per_tensor"), ("dynamic", aq, sa, "per_token")):
        yy = sg.fp8_scaled_gemm(a_c, s_c, wq_rm, sw, a_scale_mode=mode)
        rel[tag] = float((yy[rows].double() - ref).norm() / ref.norm())
        del yy
    n_big = int((x.float().abs() * float(1.0 / s_static) >= 448.0).sum())
    out.append({"workload": "large-layer static vs dynamic (same seed)", "static_scale": s_static,
                "codes_at_max_static": sat_static, "codes_at_max_dynamic": sat_dyn,
                "inputs_beyond_448s_static": n_big, "rel_frobenius_static": round(rel["static"], 6),
                "rel_frobenius_dynamic": round(rel["dynamic"], 6), "rows_compared": 256})
    del w_t, ref, aq_s, y
    torch.cuda.empty_cache()
    return out


def run_details(sg, torch, dev, to_bf16, T, wanted, clock):
    """Every other configuration: the decode step, prefill GEMMs (both
    accumulation modes), per-token / static / per-channel quantizers, the KV
    passes and the next-row workloads."""
    from workloads import (STATIC_SCALE_DEN, STATIC_SCALE_NUM, decode_inputs, kv_append_inputs, kv_inputs,
                           large_layer_inputs, prefill_inputs)
    out = []

    def copies(t, n):
        return [t] + [t.clone() for _ in range(n - 1)]

    if "decode" in wanted:
        log("decode")
        w_host = None
        xs = {}
        for m in DEC_MS:
            xb, w, _ = decode_inputs(m, with_weight=(w_host is None))
            if w_host is None:
                w_host = w
            xs[m] = to_bf16(xb)
        wq_rm, sw = sg.fp8_quant_weight_per_channel(torch.from_numpy(w_host).to(dev))
        # W_COPIES copies of the weights defeat the 256 MB last-level cache
        wqs = copies(sg.fp8_pack_weights(wq_rm), W_COPIES)
        wrm = copies(wq_rm, W_COPIES)
        ys = {m: torch.empty((m, DEC_N), dtype=torch.bfloat16, device=dev) for m in DEC_MS}
        ws = {m: torch.empty(max(sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_token", m, DEC_N, DEC_K),
                                 256), dtype=torch.uint8, device=dev) for m in DEC_MS}
        sas = {m: torch.empty(m, dtype=torch.float32, device=dev) for m in DEC_MS}
        bytes_per_call = {m: DEC_N * DEC_K + 4 * DEC_N + 2 * m * DEC_K + 2 * m * DEC_N for m in DEC_MS}

        def dstep(i):
            # every call reads its own weight copy (three layers' weights per step)
            for j, m in enumerate(DEC_MS):
                sg.fp8_scaled_gemm(xs[m], sas[m], wqs[(i * len(DEC_MS) + j) % W_COPIES], sw, y=ys[m],
                                   workspace=ws[m], w_layout="packed")

        d = T.per_call(dstep)
        out.append(gbs_row("decode step: fp8_scaled_gemm on bf16 X [M,4096], M = 1, 8, 32, per-token quant in the "
                           "call, W [14336,4096] packed, exact", d, sum(bytes_per_call.values()), accum="exact"))
        d = T.graph(dstep, inner=8)
        out.append(gbs_row("decode step replayed from a HIP graph (8 steps per graph)", d,
                           sum(bytes_per_call.values()), accum="exact"))
        for m in DEC_MS:
            aq, sa = sg.fp8_quant_per_token(xs[m])
            ap = sg.fp8_pack_weights(aq)  # the order the fused call's workspace uses
            for layout, bufs, a_layout in (("packed", wqs, "packed"), ("packed", wqs, "row_major"),
                                           ("row_major", wrm, "row_major")):
                a_in = ap if a_layout == "packed" else aq
                for accum in ("exact", "mfma_fp8"):
                    d = T.graph(lambda i: sg.fp8_scaled_gemm(a_in, sa, bufs[i % W_COPIES], sw, y=ys[m], accum=accum,
                                                             w_layout=layout, a_layout=a_layout,
                                                             a_shape=(m, DEC_K)), inner=W_COPIES * 2)
                    kb = DEC_N * DEC_K + 4 * DEC_N + m * DEC_K + 4 * m + 2 * m * DEC_N
                    out.append(gbs_row(f"decode GEMM kernel M={m} N={DEC_N} K={DEC_K} (pre-quantized A)", d, kb,
                                       accum=accum, w_layout=layout, a_layout=a_layout))
            d = T.graph(lambda i: sg.fp8_scaled_gemm(xs[m], sas[m], wqs[i % W_COPIES], sw, y=ys[m], workspace=ws[m],
                                                     w_layout="packed"), inner=W_COPIES * 2)
            out.append(gbs_row(f"decode call M={m} (per-token quant in the call + GEMM)", d, bytes_per_call[m],
                               accum="exact", w_layout="packed"))
            d = T.graph(lambda i: sg.fp8_quant_per_token(xs[m], aq, sa))
            out.append(gbs_row(f"decode per-token quant X bf16 [{m},{DEC_K}]", d, 3 * m * DEC_K + 4 * m))
            del aq, sa, ap
        del wqs, wrm, xs
        torch.cuda.empty_cache()

    def gemm_rows(tag, x_list, wq_rm, sw, M, N, K):
        flops = 2.0 * M * N * K
        wq = sg.fp8_pack_weights(wq_rm)
        aq, sa = sg.fp8_quant_per_token(x_list[0])
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ap = sg.fp8_pack_weights(aq)
        for accum, layout, wbuf, a_layout in (("exact", "packed", wq, "packed"), ("exact", "packed", wq, "row_major"),
                                              ("mfma_fp8", "packed", wq, "packed"),
                                              ("exact", "row_major", wq_rm, "row_major")):
            a_in = ap if a_layout == "packed" else aq
            d = T.per_call(lambda i: sg.fp8_scaled_gemm(a_in, sa, wbuf, sw, y=y, accum=accum, w_layout=layout,
                                                        a_layout=a_layout, a_shape=(M, K)), min_calls=100)
            out.append(tflops_row(f"{tag} GEMM kernel {M}x{N}x{K} (pre-quantized A)", d, flops, accum,
                                  w_layout=layout, a_layout=a_layout))
        del ap
        ws = torch.empty(sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_token", M, N, K), dtype=torch.uint8,
                         device=dev)
        d = T.per_call(lambda i: sg.fp8_scaled_gemm(x_list[i % len(x_list)], None, wq, sw, y=y, workspace=ws,
                                                    w_layout="packed"))
        out.append(tflops_row(f"{tag} call {M}x{N}x{K} (bf16 X, per-token quant in the call)", d, flops, "exact"))
        return aq, sa

    def quant_rows(tag, x_list, M, K, static_scale=None):
        """The kernel's duration from HIP-graph replays (16 calls per graph, the
        inputs and outputs rotating over enough copies to miss the 256 MB
        last-level cache), and beside it the back-to-back per-call figure, which
        adds the ~2.5 us dispatch gap between two launches."""
        nbytes = 3 * M * K + (4 * M if static_scale is None else 4)
        q = [torch.empty((M, K), dtype=torch.uint8, device=dev) for _ in x_list]
        if static_scale is None:
            s = [torch.empty(M, dtype=torch.float32, device=dev) for _ in x_list]
            f = lambda i: sg.fp8_quant_per_token(x_list[i % len(x_list)], q[i % len(q)], s[i % len(s)])
            name = "per-token dynamic quant"
        else:
            sc = torch.tensor([static_scale], dtype=torch.float32, device=dev)
            f = lambda i: sg.fp8_quant_per_tensor_static(x_list[i % len(x_list)], sc, q=q[i % len(q)])
            name = "per-tensor static quant"
        b2b = stats(T.per_call(f))
        d = T.graph(f, inner=16)
        out.append(gbs_row(f"{tag} {name} X bf16 [{M},{K}]", d, nbytes, buffers=len(x_list),
                           timing="graph replays of 16 calls",
                           back_to_back_median_us=b2b["median_us"],
                           back_to_back_frac_hbm=round(nbytes / (b2b["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)))

    if "prefill" in wanted or "quant" in wanted or "rmsnorm" in wanted:
        for K in (4096, 14336):
            log(f"prefill K={K}")
            xb, w, _ = prefill_inputs(K)
            M, N = xb.shape[0], w.shape[0]
            x0 = to_bf16(xb)
            xl = copies(x0, 8 if K == 4096 else 2)
            if "quant" in wanted:
                quant_rows(f"prefill K={K}", xl, M, K)
            if "rmsnorm" in wanted and K == 4096:
                # RMSNorm of the rows with the per-token quantization fused in (gamma bf16 [K])
                g = torch.ones(K, dtype=torch.bfloat16, device=dev)
                qn, sn = sg.fp8_rmsnorm_quant_per_token(xl[0], g, 1e-6)
                d = T.graph(lambda i: sg.fp8_rmsnorm_quant_per_token(xl[i % len(xl)], g, 1e-6, q=qn, scales=sn),
                            inner=16)
                out.append(gbs_row(f"RMSNorm + per-token quant X bf16 [{M},{K}] (fused)", d,
                                   3 * M * K + 2 * K + 4 * M, buffers=len(xl), timing="graph replays of 16 calls"))
                del qn, sn
            if "prefill" in wanted:
                wq, sw = sg.fp8_quant_weight_per_channel(torch.from_numpy(w).to(dev))
                aq, sa = gemm_rows(f"prefill K={K}", xl, wq, sw, M, N, K)
                del wq, sw, aq, sa
            del xl, x0
            torch.cuda.empty_cache()

    if "quant" in wanted:
        log("large-layer quantizers")
        xb, _ = large_layer_inputs(with_weight=False)
        M, K = xb.shape
        s_static = float(np.float32(STATIC_SCALE_NUM) / np.float32(STATIC_SCALE_DEN))
        xl = copies(to_bf16(xb), 8)
        quant_rows("large-layer", xl, M, K, static_scale=s_static)
        quant_rows("large-layer", xl, M, K)
        del xl
        torch.cuda.empty_cache()

    if "weights" in wanted:
        log("weight quant")
        _, w, _ = decode_inputs(1)
        w_t = torch.from_numpy(w).to(dev)
        N, K = w.shape
        d = T.per_call(lambda i: sg.fp8_quant_weight_per_channel(w_t))
        out.append(gbs_row(f"per-channel weight quant W fp32 [{N},{K}] (offline)", d, 5 * N * K + 4 * N))
        del w_t

    if "blockwise" in wanted:
        log("block-wise")
        _, w, _ = decode_inputs(1)
        w_t = torch.from_numpy(w).to(dev)
        N, K = w.shape
        d = T.per_call(lambda i: sg.fp8_quant_weight_blockwise(w_t))
        out.append(gbs_row(f"block-wise weight quant W fp32 [{N},{K}] 128x128 blocks (offline)", d, 5 * N * K))
        wq, sw = sg.fp8_quant_weight_blockwise(w_t)
        wps = copies(sg.fp8_pack_weights(wq), 8)
        del w_t, wq
        for m in (1, 8, 32):
            xb, _, _ = decode_inputs(m, with_weight=False)
            x = to_bf16(xb)
            aq, sa = sg.fp8_quant_per_token_group(x, layout="packed")
            y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
            d = T.graph(lambda i: sg.fp8_quant_per_token_group(x, layout="packed", q=aq, scales=sa))
            out.append(gbs_row(f"block-wise act quant 1x128 X bf16 [{m},{K}]", d, 3 * m * K + 4 * m * (K // 128)))
            for accum in ("exact", "mfma_fp8"):
                d = T.graph(lambda i: sg.fp8_scaled_gemm_blockwise(aq, sa, wps[i % 8], sw, y=y, accum=accum,
                                                                   w_layout="packed", a_layout="packed",
                                                                   a_shape=(m, K), w_shape=(N, K)), inner=16)
                kb = N * K + 4 * sw.numel() + m * K + 4 * sa.numel() + 2 * m * N
                out.append(gbs_row(f"block-wise decode GEMM M={m} N={N} K={K}", d, kb, accum=accum))
        del wps
        torch.cuda.empty_cache()
        for K in (4096, 14336):
            xb, w, _ = prefill_inputs(K)
            M, N = xb.shape[0], w.shape[0]
            # enough activation copies that the 256 MB last-level cache cannot serve the quantizer's reads
            xl = copies(to_bf16(xb), 8 if K == 4096 else 3)
            # the codes in the fragment order and the activation scales k-block-major ([K/128, M]): the
            # large-tile kernels then copy whole 2 KB blocks of A and the scales of 64 rows of one k block
            # as one contiguous run
            aq, sa = sg.fp8_quant_per_token_group(xl[0], layout="packed", scale_layout="kmajor")
            d = T.per_call(lambda i: sg.fp8_quant_per_token_group(xl[i % len(xl)], layout="packed", q=aq, scales=sa,
                                                                  scale_layout="kmajor"))
            out.append(gbs_row(f"block-wise act quant 1x128 X bf16 [{M},{K}] (fragment order, k-block-major "
                               f"scales)", d, 3 * M * K + 4 * M * (K // 128)))
            wq, sw = sg.fp8_quant_weight_blockwise(torch.from_numpy(w).to(dev))
            wp = sg.fp8_pack_weights(wq)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            for accum, tag in (("mfma_fp8", ""), ("exact", " exact partials")):
                d = T.per_call(lambda i: sg.fp8_scaled_gemm_blockwise(aq, sa, wp, sw, y=y, accum=accum,
                                                                      w_layout="packed", w_shape=(N, K),
                                                                      a_layout="packed", a_shape=(M, K),
                                                                      a_scale_layout="kmajor"), min_calls=50)
                out.append(tflops_row(f"block-wise prefill GEMM {M}x{N}x{K}{tag} (packed A, k-block-major "
                                      f"activation scales)", d, 2.0 * M * N * K, accum))
            aq2, sa2 = sg.fp8_quant_per_token_group(xl[0])
            d = T.per_call(lambda i: sg.fp8_scaled_gemm_blockwise(aq2, sa2, wp, sw, y=y, accum="mfma_fp8",
                                                                  w_layout="packed", w_shape=(N, K)), min_calls=50)
            out.append(tflops_row(f"block-wise prefill GEMM {M}x{N}x{K} (row-major A, row-major activation "
                                  f"scales)", d, 2.0 * M * N * K, "mfma_fp8"))
            del xl, aq, sa, aq2, sa2, wq, wp, y
            torch.cuda.empty_cache()

    if "mx" in wanted:
        log("mxfp8")
        _, w, _ = decode_inputs(1)
        w_t = torch.from_numpy(w).to(dev)
        N, K = w.shape
        d = T.per_call(lambda i: sg.fp8_quant_mx(w_t, layout="packed", scale_layout="packed"))
        out.append(gbs_row(f"MX weight quant W fp32 [{N},{K}] 32-element blocks (offline)", d,
                           5 * N * K + N * K // 32))
        wp, wsc = sg.fp8_quant_mx(w_t, layout="packed", scale_layout="packed")
        wps = copies(wp, 8)
        del w_t
        for m in (1, 8, 32):
            xb, _, _ = decode_inputs(m, with_weight=False)
            x = to_bf16(xb)
            aq, sa = sg.fp8_quant_mx(x, layout="packed", scale_layout="packed")
            y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
            d = T.graph(lambda i: sg.fp8_quant_mx(x, layout="packed", scale_layout="packed", q=aq, scales=sa))
            out.append(gbs_row(f"MX act quant X bf16 [{m},{K}]", d, 3 * m * K + m * K // 32))
            d = T.graph(lambda i: sg.fp8_scaled_gemm_mx(aq, sa, wps[i % 8], wsc, y=y, w_layout="packed",
                                                        a_layout="packed", a_shape=(m, K), w_shape=(N, K)), inner=16)
            kb = N * K + wsc.numel() + m * K + sa.numel() + 2 * m * N
            out.append(gbs_row(f"MX decode GEMM M={m} N={N} K={K}", d, kb, accum="scaled mfma"))
            if m > 16:
                continue
            d = T.graph(lambda i: sg.fp8_scaled_gemm_mx_bf16(x, wps[i % 8], wsc, y=y, w_layout="packed",
                                                             w_shape=(N, K)), inner=16)
            kb = N * K + wsc.numel() + 2 * m * K + 2 * m * N
            out.append(gbs_row(f"MX decode call M={m} N={N} K={K} (bf16 X, MX quantization inside the GEMM)", d, kb,
                               accum="scaled mfma"))
        del wps, wp
        torch.cuda.empty_cache()
        for K in (4096, 14336):
            xb, w, _ = prefill_inputs(K)
            M, N = xb.shape[0], w.shape[0]
            # enough activation copies that the 256 MB last-level cache cannot serve the quantizer's reads
            xl = copies(to_bf16(xb), 8 if K == 4096 else 3)
            wp, wsc = sg.fp8_quant_mx(torch.from_numpy(w).to(dev), layout="packed", scale_layout="packed")
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            for fmt in ("e4m3", "e5m2"):
                aq, sa = sg.fp8_quant_mx(xl[0], fmt, layout="packed", scale_layout="packed")
                d = T.per_call(lambda i: sg.fp8_quant_mx(xl[i % len(xl)], fmt, layout="packed", scale_layout="packed",
                                                         q=aq, scales=sa))
                out.append(gbs_row(f"MX act quant X bf16 [{M},{K}] {fmt}", d, 3 * M * K + M * K // 32))
                d = T.per_call(lambda i: sg.fp8_scaled_gemm_mx(aq, sa, wp, wsc, a_fmt=fmt, y=y, w_layout="packed",
                                                               a_layout="packed", a_shape=(M, K), w_shape=(N, K)),
                               min_calls=50)
                out.append(tflops_row(f"MX prefill GEMM {M}x{N}x{K} A {fmt}", d, 2.0 * M * N * K, "scaled mfma"))
                del aq, sa
            del xl, wp, wsc, y
            torch.cuda.empty_cache()

    if "fp8out" in wanted:
        log("fp8 output epilogue")
        _, w, _ = decode_inputs(1)
        wq, sw = sg.fp8_quant_weight_per_channel(torch.from_numpy(w).to(dev))
        wps = copies(sg.fp8_pack_weights(wq), 8)
        N, K = w.shape
        xb, _, _ = decode_inputs(32, with_weight=False)
        aq, sa = sg.fp8_quant_per_token(to_bf16(xb))
        ap = sg.fp8_pack_weights(aq)
        so = torch.tensor([0.05], dtype=torch.float32, device=dev)
        yq = torch.empty((32, N), dtype=torch.uint8, device=dev)
        d = T.graph(lambda i: sg.fp8_scaled_gemm_fp8out(ap, sa, wps[i % 8], sw, so, y=yq, w_layout="packed",
                                                        a_layout="packed", a_shape=(32, K)), inner=16)
        kb = N * K + 4 * N + 32 * K + 4 * 32 + 32 * N
        out.append(gbs_row(f"decode GEMM kernel M=32 N={N} K={K}, E4M3 output (pre-quantized A)", d, kb,
                           accum="exact"))
        del wps, wq, aq, ap
        xb, w, _ = prefill_inputs(4096)
        M, N = xb.shape[0], w.shape[0]
        aq, sa = sg.fp8_quant_per_token(to_bf16(xb))
        ap = sg.fp8_pack_weights(aq)
        wq, sw = sg.fp8_quant_weight_per_channel(torch.from_numpy(w).to(dev))
        wp = sg.fp8_pack_weights(wq)
        yq = torch.empty((M, N), dtype=torch.uint8, device=dev)
        for accum in ("mfma_fp8", "exact"):
            d = T.per_call(lambda i: sg.fp8_scaled_gemm_fp8out(ap, sa, wp, sw, so, y=yq, accum=accum, w_layout="packed",
                                                               a_layout="packed", a_shape=(M, 4096)))
            out.append(tflops_row(f"prefill GEMM {M}x{N}x4096, E4M3 output (pre-quantized A)", d,
                                  2.0 * M * N * 4096, accum))
        del aq, ap, wq, wp, yq
        torch.cuda.empty_cache()

    if "kv" in wanted or "attention" in wanted:
        log("kv cache")
        k, v, kc, vc = kv_inputs(0)
        B, S, H, D = k.shape
        numel = B * S * H * D
        kt, vt = to_bf16(k), to_bf16(v)
        del k, v
        if "kv" in wanted:
            for fmt in ("e4m3", "e5m2"):
                sk = sg.fp8_kv_calibrate(kt, fmt)
                sv = sg.fp8_kv_calibrate(vt, fmt)
                qk = sg.fp8_kv_quant(kt, sk, fmt)
                qv = sg.fp8_kv_quant(vt, sv, fmt)
                dk = torch.empty_like(kt)
                dv = torch.empty_like(vt)
                d = T.per_call(lambda i: (sg.fp8_kv_calibrate(kt, fmt, sk), sg.fp8_kv_calibrate(vt, fmt, sv)))
                out.append(gbs_row(f"KV calibrate K+V [{B},{S},{H},{D}] {fmt}", d, 4 * numel))
                d = T.per_call(lambda i: (sg.fp8_kv_quant(kt, sk, fmt, out=qk), sg.fp8_kv_quant(vt, sv, fmt, out=qv)))
                out.append(gbs_row(f"KV quant K+V [{B},{S},{H},{D}] {fmt}", d, 6 * numel))
                d = T.per_call(lambda i: (sg.fp8_kv_dequant(qk, sk, fmt, out=dk),
                                          sg.fp8_kv_dequant(qv, sv, fmt, out=dv)))
                out.append(gbs_row(f"KV dequant K+V [{B},{S},{H},{D}] {fmt}", d, 6 * numel))
                del qk, qv, dk, dv
        if "attention" in wanted:
            # one decode step of attention over the quantized cache: 32 query heads over the 8 kv heads
            from workloads import attention_queries
            qt = to_bf16(attention_queries(0, b=B, hq=32, d=D))
            Lt = torch.full((B,), S, dtype=torch.int32, device=dev)
            ao = torch.empty((B, 32, D), dtype=torch.bfloat16, device=dev)
            aws = torch.empty(sg.fp8_kv_decode_attention_workspace_size(B, S, 32, H, D), dtype=torch.uint8,
                              device=dev)
            for fmt in ("e4m3", "e5m2"):
                sk = sg.fp8_kv_calibrate(kt, fmt)
                sv = sg.fp8_kv_calibrate(vt, fmt)
                qk = sg.fp8_kv_quant(kt, sk, fmt)
                qv = sg.fp8_kv_quant(vt, sv, fmt)
                d = T.per_call(lambda i: sg.fp8_kv_decode_attention(qt, qk, qv, sk, sv, Lt, fmt, out=ao,
                                                                    workspace=aws))
                out.append(gbs_row(f"KV decode attention q [{B},32,{D}] over K+V [{B},{S},{H},{D}] {fmt}", d,
                                   2 * numel + 2 * 2 * B * 32 * D + 8 * H))
                del qk, qv
            torch.cuda.empty_cache()
        sk = sg.fp8_kv_calibrate(kt, "e5m2")
        sv = sg.fp8_kv_calibrate(vt, "e5m2")
        kn, vn = kv_append_inputs(kc, vc)
        knt, vnt = to_bf16(kn), to_bf16(vn)
        del kt, vt
        torch.cuda.empty_cache()
        ck = torch.zeros((B, S + 1, H, D), dtype=torch.uint8, device=dev)
        cv = torch.zeros_like(ck)
        pos = torch.full((B,), S, dtype=torch.int32, device=dev)
        app = lambda i: (sg.fp8_kv_append(knt, pos, sk, ck, "e5m2"), sg.fp8_kv_append(vnt, pos, sv, cv, "e5m2"))
        d = T.graph(app, inner=20)
        row = {"workload": f"KV append 1 token/seq K+V into [{B},{S + 1},{H},{D}] (two kernels, HIP-graph replay)",
               **stats(d), "bytes": 2 * (B * H * D * 3)}
        # the binding's host cost per pair of calls, measured on its own
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(200):
            app(i)
        row["host_us_per_call_pair"] = round((time.perf_counter() - t0) / 200 * 1e6, 2)
        torch.cuda.synchronize()
        out.append(row)
        del ck, cv
        torch.cuda.empty_cache()
    return out


def cpu_baseline(xb_host, w_host, s_static, log):
    """The CPU oracle on a bounded sample of the headline workload: the per-token
    and the static per-tensor quantization of 64 of the 4096 rows of X, then for
    each arm the exact GEMM against 1024 of the 28672 output channels and the
    bf16 epilogue.  (The weights' per-channel quantization is the offline step
    and is not timed, as on the GPU.)  Reported in the headline's unit."""
    from oracle import w8a8
    from workloads import f32_from_bf16_bits
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    M, K = xb_host.shape
    N = w_host.shape[0]
    R, C = 64, 1024
    rows = np.arange(0, M, M // R)[:R]
    cols = np.arange(0, N, N // C)[:C]
    log("cpu baseline: oracle weight quantization of the sampled channels (untimed)")
    wq, sw = w8a8.quant_weight_per_channel(w_host[cols])
    x = f32_from_bf16_bits(xb_host[rows])
    s32 = np.float32(s_static)
    t = time.perf_counter()
    reps = 0
    while True:
        aq, sa = w8a8.quant_per_token(x)
        w8a8.scaled_gemm_bf16(aq, sa, wq, sw)
        aqs = w8a8.quant_static(x, s32)
        w8a8.scaled_gemm_bf16(aqs, s32, wq, sw)
        reps += 1
        if time.perf_counter() - t > 10.0 or reps >= 200:
            break
    dt = (time.perf_counter() - t) / reps
    flops = 2 * 2.0 * R * C * K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "blas_threads": int(blas_threads),
            "sample": f"both arms of the large layer on {R} of the {M} rows x {C} of the {N} output channels "
                      f"(K={K}): per-token and static quantization of the rows, exact float64 GEMM on decoded codes, "
                      f"bf16 epilogue; {reps} reps, {dt * 1e3:.1f} ms per rep; {cores} host cores in the affinity "
                      f"mask, numpy BLAS with {blas_threads} threads, the encoder single-threaded"}


if __name__ == "__main__":
    main()
