"""Benchmark of the FP8 W8A8 scaled-GEMM path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--workload NAME ...]

Prints ONE JSON line.  The headline step is the decode-shaped W8A8 GEMM:
for M in (1, 8, 32), one fp8_scaled_gemm call on bf16 activations X [M, 4096]
(per-token dynamic E4M3 quantization fused into the call) against E4M3 weights
[14336, 4096] with per-channel scales, exact fp32 accumulation, bf16 output.
`value` is that step's algorithmic HBM traffic divided by its time (GB/s):
weights + weight scales + X (bf16) + Y (bf16) per call, inputs resident in HBM.
The weights rotate through enough copies (8 x 58.7 MB) that the 256 MB
last-level cache cannot serve them.

`roofline` is for the step's dominant kernel, the skinny GEMM of the M = 32
call, timed per launch with HIP events on the library's stream (activations
pre-quantized and packed into the fragment order the fused call's workspace
uses, so the GEMM kernel is the only kernel between the events).
`cpu_baseline` times the CPU oracle on the same decode workload.
`details` carries every other measured workload (prefill and large-layer GEMMs
in both accumulation modes, the quantizers, the KV-cache passes).

Inputs are seeded and synthetic (see workloads/).  One GPU only: --gpus > 1
exits with a message.
"""

from __future__ import annotations

import argparse
import json
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
# HBM traffic of the roofline kernel from two rocprofv3 counter passes over
# `bench.py --quick --no-cpu --pmc-calibrate` (FETCH_SIZE, then WRITE_SIZE, KiB
# per dispatch, median over the dispatches), each scaled by what the counter
# reads for the 1 GiB calibration copy (FETCH_SIZE reads half the copy's bytes
# on this part, WRITE_SIZE all of them).  Valid only for the kernel source it
# was measured on: when the hash of these files differs, traffic is reported
# as null until the counters are taken again.
TRAFFIC = {"kernel": "gemm_skinny<false, 1, 2, 2, 4, 1, true, true, false>",
           "sources": ("scaled_gemm_amd/csrc/gemm_skinny.hip", "scaled_gemm_amd/csrc/gemm_common.h",
                       "scaled_gemm_amd/csrc/fp8_device.h"),
           "sha256": ("797e72980ff2a80d55ab2b6d8d479b1ac2618f76b2ac0332abc0c4afae61d362",
                      "89988b7a08724e97afd6856fd885427340a82060cced107b6d687ad8b1cc68d0",
                      "0d2b00789594dec510b6f2e4e0550571f66e7a453f59b99894367fce3213d427"),
           "fetch_kib": 29258.0, "write_kib": 896.0,
           "fetch_factor": 1048576.0 / 524299.5, "write_factor": 1048576.0 / 1048576.0}
DEC_N, DEC_K = 14336, 4096
DEC_MS = (1, 8, 32)
W_COPIES = 8


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--quick", action="store_true", help="headline only: skip the detail workloads")
    ap.add_argument("--workload", nargs="*", default=None,
                    help="detail workloads to run (default all): prefill large quant kv weights blockwise fp8out "
                         "attention mx rmsnorm")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--pmc-calibrate", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling HBM counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import scaled_gemm_amd as sg
    from workloads import decode_inputs

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no HIP device"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    def to_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def timed_events(fn, iters, warmup, reps=5):
        """Average duration (ms) of fn(i), from HIP events on the current stream
        (the stream the library launches on) around `iters` back-to-back calls;
        `reps` such measurements are returned.  Back-to-back launches keep the
        queue full, so the average is the kernels' own duration plus the small
        dispatch gap between them -- the figure a kernel trace reports."""
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        out = []
        for r in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(iters):
                fn(r * iters + i)
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) / iters)
        return np.array(out)

    # ------------------------------------------------------------ headline inputs
    log("generating decode inputs")
    w_host = None
    xs = {}
    for m in DEC_MS:
        xb, w, _ = decode_inputs(m, with_weight=(w_host is None))
        if w_host is None:
            w_host = w
        xs[m] = to_bf16(xb)
    w_t = torch.from_numpy(w_host).to(dev)
    wq_rm, sw = sg.fp8_quant_weight_per_channel(w_t)
    del w_t
    # weights are prepared offline: quantized per channel, then packed into the
    # matrix-core fragment order; W_COPIES copies defeat the last-level cache
    wp0 = sg.fp8_pack_weights(wq_rm)
    wqs = [wp0] + [wp0.clone() for _ in range(W_COPIES - 1)]
    wrm = [wq_rm] + [wq_rm.clone() for _ in range(W_COPIES - 1)]
    ys = {m: torch.empty((m, DEC_N), dtype=torch.bfloat16, device=dev) for m in DEC_MS}
    ws = {m: torch.empty(sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_token", m, DEC_N, DEC_K),
                         dtype=torch.uint8, device=dev) for m in DEC_MS}
    sas = {m: torch.empty(m, dtype=torch.float32, device=dev) for m in DEC_MS}
    torch.cuda.synchronize()

    def step(i):
        # every call reads its own weight copy (three layers' weights per step), so
        # no call finds the weight of the one before it in the last-level cache
        for j, m in enumerate(DEC_MS):
            sg.fp8_scaled_gemm(xs[m], sas[m], wqs[(i * len(DEC_MS) + j) % W_COPIES], sw, y=ys[m], workspace=ws[m],
                               w_layout="packed")

    # ------------------------------------------------------------ headline timing
    log(f"headline: warmup {args.warmup}, steps {args.steps}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps
    bytes_per_call = {m: DEC_N * DEC_K + 4 * DEC_N + 2 * m * DEC_K + 2 * m * DEC_N for m in DEC_MS}
    step_bytes = sum(bytes_per_call.values())
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # ------------------------------------------------------------ dominant kernel
    details = []
    kern = {}
    for m in DEC_MS:
        aq, sa = sg.fp8_quant_per_token(xs[m])
        # the fused call quantizes into its workspace in the fragment order; the
        # same codes packed here let the GEMM kernel be timed on its own
        ap = sg.fp8_pack_weights(aq)
        for layout, bufs, a_layout in (("packed", wqs, "packed"), ("packed", wqs, "row_major"),
                                       ("row_major", wrm, "row_major")):
            a_in = ap if a_layout == "packed" else aq
            for accum in ("exact", "mfma_fp8"):
                d = timed_events(lambda i: sg.fp8_scaled_gemm(a_in, sa, bufs[i % W_COPIES], sw, y=ys[m], accum=accum,
                                                              w_layout=layout, a_layout=a_layout,
                                                              a_shape=(m, DEC_K)), 100, 20)
                # algorithmic bytes of the GEMM kernel alone: W + s_w + A_q + s_a + Y
                kb = DEC_N * DEC_K + 4 * DEC_N + m * DEC_K + 4 * m + 2 * m * DEC_N
                kern[(m, accum, layout, a_layout)] = (kb, float(d.mean()))
                details.append({"workload": f"decode GEMM kernel M={m} N={DEC_N} K={DEC_K} (pre-quantized A)",
                                "accum": accum, "w_layout": layout, "a_layout": a_layout,
                                "avg_us": round(float(d.mean()) * 1e3, 2),
                                "min_us": round(float(np.min(d)) * 1e3, 2),
                                "GB_s": round(kb / (d.mean() * 1e-3) / 1e9, 1),
                                "frac_hbm": round(kb / (d.mean() * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        d = timed_events(lambda i: sg.fp8_scaled_gemm(xs[m], sas[m], wqs[i % W_COPIES], sw, y=ys[m],
                                                      workspace=ws[m], w_layout="packed"), 100, 20)
        details.append({"workload": f"decode call M={m} (fused per-token quant + GEMM)", "accum": "exact",
                        "w_layout": "packed", "avg_us": round(float(d.mean()) * 1e3, 2),
                        "GB_s": round(bytes_per_call[m] / (d.mean() * 1e-3) / 1e9, 1)})
        details += library_rows(torch, timed_events, "decode GEMM", aq, sa, wrm, sw, m, DEC_N, DEC_K, 100, 20)
    kb32, dur32 = kern[(32, "exact", "packed", "packed")]
    achieved = kb32 / (dur32 * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "kernel": "gemm_skinny<exact, bf16 out, 2 m-tiles, packed W, packed A> (decode M=32)",
                "avg_launch_us": round(dur32 * 1e3, 2), "bytes_per_launch": kb32,
                "timing": "HIP events around 100 back-to-back launches on the library's stream, mean of 5"}

    # the same step replayed from one HIP graph of 8 consecutive steps (every
    # weight copy once): the host's launch work leaves the timed region
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(8):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(8):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // 8)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        gms = a.elapsed_time(b) / (reps * 8)
        details.append({"workload": "headline decode step replayed from a HIP graph (8 steps per graph)",
                        "ms_per_step": round(gms, 5), "GB_s": round(step_bytes / (gms * 1e-3) / 1e9, 1),
                        "vs_eager_step": round(gms / ms_per_step, 4)})
        del g
    except Exception as e:  # recorded, not fatal: the eager figure above is the headline
        details.append({"workload": "headline decode step replayed from a HIP graph", "error": str(e)[:200]})

    # ------------------------------------------------------------ details
    wanted = set(args.workload) if args.workload else {"prefill", "large", "quant", "kv", "weights", "blockwise",
                                                       "fp8out", "attention", "mx", "rmsnorm"}
    if args.quick:
        wanted = set()
    del wqs[1:], wrm[1:]
    torch.cuda.empty_cache()
    if wanted:
        details += run_details(sg, torch, dev, to_bf16, timed_events, wanted, log)

    # ------------------------------------------------------------ copy calibration
    if args.pmc_calibrate:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        details.append({"workload": "calibration copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30,
                        "launches": 3})

    # ------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w_host, log)

    out = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "e4m3", "data": "synthetic (seeded, workloads/)",
           "config": {"workload": "decode-shaped W8A8 GEMM: X bf16 [M,4096] M in {1,8,32}, per-token dynamic E4M3 "
                                  "quant fused into the call; W E4M3 [14336,4096] per-channel fp32 scales, packed "
                                  "offline; exact fp32 accumulation; bf16 out",
                      "M": list(DEC_MS), "N": DEC_N, "K": DEC_K, "accum": "exact", "w_layout": "packed",
                      "weight_copies": W_COPIES,
                      "bytes_per_step": step_bytes},
           "roofline": roofline, "cpu_baseline": cpu, "details": details}
    print(json.dumps(out), flush=True)


def measured_traffic():
    """HBM bytes per launch of the roofline kernel from the recorded counters,
    or None when its source has changed since they were taken."""
    import hashlib
    for rel, want in zip(TRAFFIC["sources"], TRAFFIC["sha256"]):
        with open(os.path.join(ROOT, rel), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != want:
                return None
    return int(round(1024 * (TRAFFIC["fetch_kib"] * TRAFFIC["fetch_factor"] +
                             TRAFFIC["write_kib"] * TRAFFIC["write_factor"])))


def _gbs(nbytes, ms):
    return round(nbytes / (ms * 1e-3) / 1e9, 1)


def _tflops(flops, ms):
    return round(flops / (ms * 1e-3) / 1e12, 1)


def sustained_clock_mhz(torch, launch, launch_ms, seconds=2.5, settle=0.6, samples=4, gap=0.25):
    """Graphics clock while the GPU runs back-to-back launches of one kernel.

    Queues about `seconds` of launches, waits `settle` s (the tool's reading
    trails the load by up to half a second), then reads `amd-smi metric --clock`
    `samples` times from a child process and averages the 8 XCD clocks of each
    reading.  Returns (readings or None when the tool is missing, prints no
    clock or the run is under a profiler, average ms per launch of the loop from
    HIP events around it)."""
    import re
    import shutil
    import subprocess
    import time
    tool = shutil.which("amd-smi")
    if any(k.startswith("ROCPROF") for k in os.environ):
        # under rocprofv3 a child process starts with the profiler's library loaded, which
        # initialises the GPU before the tool's own interpreter starts: no child then
        tool = None
    torch.cuda.synchronize()
    n = max(1, int(seconds * 1e3 / launch_ms))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        launch(i)
    b.record()
    vals = []
    if tool is not None:
        time.sleep(settle)
        for _ in range(samples):
            r = subprocess.run([tool, "metric", "--clock"], capture_output=True, text=True, timeout=30)
            c = [int(v) for v in re.findall(r"GFX_\d+:\s+CLK: (\d+) MHz", r.stdout)]
            if c:
                vals.append(round(sum(c) / len(c)))
            time.sleep(gap)
    torch.cuda.synchronize()
    return (vals or None), a.elapsed_time(b) / n


def library_rows(torch, timed_events, tag, aq, sa, w_rm, sw, M, N, K, iters, warm):
    """The same product through the vendor library (torch._scaled_mm, i.e.
    hipBLASLt), timed beside this library's kernels as a yardstick: row-wise
    scales (the per-token x per-channel scaling computed here) and unit
    per-tensor scales (the library's plain FP8 GEMM).  Not part of any path of
    this library; an error is recorded in the row."""
    out = []
    w_rm = w_rm if isinstance(w_rm, list) else [w_rm]
    a8 = aq.view(torch.float8_e4m3fn)
    b8 = [w.view(torch.float8_e4m3fn).t() for w in w_rm]  # [K, N] column-major, the operand order it takes
    one = torch.ones((), dtype=torch.float32, device=aq.device)
    flops = 2.0 * M * N * K
    for scaling, s_a, s_b in (("row-wise", sa.view(M, 1), sw.view(1, N)), ("per-tensor (unit)", one, one)):
        row = {"workload": f"{tag} {M}x{N}x{K} through torch._scaled_mm (hipBLASLt), for comparison",
               "scaling": scaling}
        try:
            d = timed_events(lambda i: torch._scaled_mm(a8, b8[i % len(b8)], scale_a=s_a, scale_b=s_b,
                                                        out_dtype=torch.bfloat16), iters, warm, reps=3)
            row.update({"avg_us": round(float(d.mean()) * 1e3, 2), "TFLOPS": _tflops(flops, d.mean())})
        except Exception as e:  # the library may not offer the scaling on this build
            row["error"] = str(e).split("\n")[0][:160]
        out.append(row)
    return out


def run_details(sg, torch, dev, to_bf16, timed_events, wanted, log):
    """Every other configuration: prefill and large-layer GEMMs (both accumulation
    modes), per-token / static / per-channel quantizers and the KV-cache passes."""
    from workloads import (STATIC_SCALE_DEN, STATIC_SCALE_NUM, kv_append_inputs, kv_inputs, large_layer_inputs,
                           prefill_inputs)
    out = []

    def copies(t, n):
        return [t] + [t.clone() for _ in range(n - 1)]

    def gemm_rows(tag, x_list, wq_rm, sw, M, N, K, static_scale=None):
        flops = 2.0 * M * N * K
        wq = sg.fp8_pack_weights(wq_rm)
        if static_scale is None:
            aq, sa = sg.fp8_quant_per_token(x_list[0])
        else:
            sa = torch.tensor([static_scale], dtype=torch.float32, device=dev)
            aq = sg.fp8_quant_per_tensor_static(x_list[0], sa)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ap = sg.fp8_pack_weights(aq)  # the fragment order the fused call's workspace uses
        for accum, layout, wbuf, a_layout in (("exact", "packed", wq, "packed"), ("mfma_fp8", "packed", wq, "packed"),
                                              ("exact", "row_major", wq_rm, "row_major")):
            a_in = ap if a_layout == "packed" else aq
            d = timed_events(lambda i: sg.fp8_scaled_gemm(a_in, sa, wbuf, sw, y=y, accum=accum, w_layout=layout,
                                                          a_layout=a_layout, a_shape=(M, K),
                                                          a_scale_mode="per_token" if static_scale is None
                                                          else "per_tensor"), 10, 10, reps=3)
            tf = _tflops(flops, d.mean())
            row = {"workload": f"{tag} GEMM {M}x{N}x{K} (pre-quantized A)", "accum": accum, "w_layout": layout,
                   "a_layout": a_layout, "avg_us": round(float(d.mean()) * 1e3, 1), "TFLOPS": tf,
                   "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4)}
            if accum == "exact":
                row["frac_bf16_peak"] = round(tf / BF16_PEAK_TFLOPS, 4)
            out.append(row)
        del ap
        if static_scale is None:
            out.extend(library_rows(torch, timed_events, f"{tag} GEMM", aq, sa, wq_rm, sw, M, N, K, 10, 10))
        ws = torch.empty(sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_token", M, N, K), dtype=torch.uint8,
                         device=dev)
        mode = "per_token" if static_scale is None else "per_tensor"
        sa_in = None if static_scale is None else sa
        d = timed_events(lambda i: sg.fp8_scaled_gemm(x_list[i % len(x_list)], sa_in, wq, sw, y=y, workspace=ws,
                                                      a_scale_mode=mode, w_layout="packed"), 10, 10, reps=3)
        out.append({"workload": f"{tag} call {M}x{N}x{K} (bf16 X, {mode} quant fused)", "accum": "exact",
                    "avg_us": round(float(d.mean()) * 1e3, 1), "TFLOPS": _tflops(flops, d.mean())})
        return aq, sa

    def quant_rows(tag, x_list, M, K, static_scale=None):
        nbytes = 3 * M * K + (4 * M if static_scale is None else 4)
        q = [torch.empty((M, K), dtype=torch.uint8, device=dev) for _ in x_list]
        if static_scale is None:
            s = [torch.empty(M, dtype=torch.float32, device=dev) for _ in x_list]
            d = timed_events(lambda i: sg.fp8_quant_per_token(x_list[i % len(x_list)], q[i % len(q)],
                                                              s[i % len(s)]), 50, 5, reps=3)
            name = "per-token dynamic quant"
        else:
            sc = torch.tensor([static_scale], dtype=torch.float32, device=dev)
            d = timed_events(lambda i: sg.fp8_quant_per_tensor_static(x_list[i % len(x_list)], sc,
                                                                      q=q[i % len(q)]), 50, 5, reps=3)
            name = "per-tensor static quant"
        gbs = _gbs(nbytes, d.mean())
        out.append({"workload": f"{tag} {name} X bf16 [{M},{K}]", "avg_us": round(float(d.mean()) * 1e3, 2),
                    "GB_s": gbs, "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "buffers": len(x_list)})

    if "prefill" in wanted or "quant" in wanted or "rmsnorm" in wanted:
        for K in (4096, 14336):
            log(f"prefill K={K}")
            xb, w, _ = prefill_inputs(K)
            M, N = xb.shape[0], w.shape[0]
            x0 = to_bf16(xb)
            xl = copies(x0, 4 if K == 4096 else 2)
            if "quant" in wanted:
                quant_rows(f"prefill K={K}", xl, M, K)
            if "rmsnorm" in wanted and K == 4096:
                # RMSNorm of the rows with the per-token quantization fused in (gamma bf16 [K])
                g = torch.ones(K, dtype=torch.bfloat16, device=dev)
                qn, sn = sg.fp8_rmsnorm_quant_per_token(xl[0], g, 1e-6)
                d = timed_events(lambda i: sg.fp8_rmsnorm_quant_per_token(xl[i % len(xl)], g, 1e-6, q=qn, scales=sn),
                                 20, 3, reps=3)
                gbs = _gbs(3 * M * K + 2 * K + 4 * M, d.mean())
                out.append({"workload": f"RMSNorm + per-token quant X bf16 [{M},{K}] (fused)",
                            "avg_us": round(float(d.mean()) * 1e3, 2), "GB_s": gbs,
                            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "buffers": len(xl)})
                del qn, sn
            if "prefill" in wanted:
                wq, sw = sg.fp8_quant_weight_per_channel(torch.from_numpy(w).to(dev))
                aq, sa = gemm_rows(f"prefill K={K}", xl, wq, sw, M, N, K)
                if K == 14336:
                    # the clock the matrix cores actually ran at during a long loop of each mode
                    wp = sg.fp8_pack_weights(wq)
                    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                    for accum in ("mfma_fp8", "exact"):
                        f = lambda i: sg.fp8_scaled_gemm(aq, sa, wp, sw, y=y, accum=accum, w_layout="packed")
                        ms = float(timed_events(f, 3, 1, reps=1).mean())
                        mhz, ms = sustained_clock_mhz(torch, f, ms)
                        row = {"workload": f"sustained graphics clock, prefill GEMM {M}x{N}x{K} loop (row-major A, "
                                           "packed W)", "accum": accum, "avg_us": round(ms * 1e3, 1),
                               "mhz_samples": mhz}
                        if mhz:
                            clk = float(np.median(mhz))
                            peak = FP8_PEAK_TFLOPS if accum == "mfma_fp8" else BF16_PEAK_TFLOPS
                            row["mhz_median"] = clk
                            row["frac_of_peak_at_this_clock"] = round(
                                _tflops(2.0 * M * N * K, ms) / (peak * clk / 2400.0), 4)
                        out.append(row)
                    del wp, y
                del wq, sw, aq, sa
            del xl, x0
            torch.cuda.empty_cache()

    if "large" in wanted or "quant" in wanted:
        log("large layer")
        xb, w = large_layer_inputs()
        M, K = xb.shape
        N = w.shape[0]
        s_static = float(np.float32(STATIC_SCALE_NUM) / np.float32(STATIC_SCALE_DEN))
        x0 = to_bf16(xb)
        xl = copies(x0, 4)
        if "quant" in wanted:
            quant_rows("large-layer", xl, M, K, static_scale=s_static)
            quant_rows("large-layer", xl, M, K)
        if "large" in wanted:
            w_t = torch.from_numpy(w).to(dev)
            wq, sw = sg.fp8_quant_weight_per_channel(w_t)
            aq_s, sa_s = gemm_rows("large-layer static", xl, wq, sw, M, N, K, static_scale=s_static)
            aq_d, sa_d = gemm_rows("large-layer dynamic", xl, wq, sw, M, N, K)
            # static vs dynamic on the same seed: saturated codes, and relative Frobenius error of Y
            # against the float64 product of the unquantized X and W, on 256 rows
            sat_static = int(((aq_s & 0x7F) == 0x7E).sum())
            sat_dyn = int(((aq_d & 0x7F) == 0x7E).sum())
            rows = torch.arange(0, M, M // 256, device=dev)[:256]
            ref = x0[rows].double() @ w_t.double().t()
            rel = {}
            for tag, aq, sa, mode in (("static", aq_s, sa_s, "per_tensor"), ("dynamic", aq_d, sa_d, "per_token")):
                y = sg.fp8_scaled_gemm(aq, sa, wq, sw, a_scale_mode=mode)  # row-major W
                rel[tag] = float((y[rows].double() - ref).norm() / ref.norm())
            n_big = int((x0.float().abs() * float(1.0 / s_static) >= 448.0).sum())
            out.append({"workload": "large-layer static vs dynamic (same seed)", "static_scale": s_static,
                        "codes_at_max_static": sat_static, "codes_at_max_dynamic": sat_dyn,
                        "inputs_beyond_448s_static": n_big, "rel_frobenius_static": round(rel["static"], 6),
                        "rel_frobenius_dynamic": round(rel["dynamic"], 6), "rows_compared": 256})
            del w_t, wq, sw, ref
        del xl, x0
        torch.cuda.empty_cache()

    if "weights" in wanted:
        log("weight quant")
        from workloads import decode_inputs
        _, w, _ = decode_inputs(1)
        w_t = torch.from_numpy(w).to(dev)
        N, K = w.shape
        d = timed_events(lambda i: sg.fp8_quant_weight_per_channel(w_t), 20, 3, reps=3)
        out.append({"workload": f"per-channel weight quant W fp32 [{N},{K}] (offline)",
                    "avg_us": round(float(d.mean()) * 1e3, 1), "GB_s": _gbs(5 * N * K + 4 * N, d.mean()),
                    "frac_hbm": round(_gbs(5 * N * K + 4 * N, d.mean()) / HBM_PEAK_GBS, 4)})
        del w_t

    if "blockwise" in wanted:
        log("block-wise")
        from workloads import decode_inputs
        # decode shape: 1 x 128 activation groups, 128 x 128 weight blocks, packed operands
        _, w, _ = decode_inputs(1)
        w_t = torch.from_numpy(w).to(dev)
        N, K = w.shape
        d = timed_events(lambda i: sg.fp8_quant_weight_blockwise(w_t), 20, 3, reps=3)
        out.append({"workload": f"block-wise weight quant W fp32 [{N},{K}] 128x128 blocks (offline)",
                    "avg_us": round(float(d.mean()) * 1e3, 1), "GB_s": _gbs(5 * N * K, d.mean())})
        wq, sw = sg.fp8_quant_weight_blockwise(w_t)
        wp = sg.fp8_pack_weights(wq)
        wps = copies(wp, 8)
        del w_t, wq
        for m in (1, 8, 32):
            xb, _, _ = decode_inputs(m, with_weight=False)
            x = to_bf16(xb)
            aq, sa = sg.fp8_quant_per_token_group(x, layout="packed")
            y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
            d = timed_events(lambda i: sg.fp8_quant_per_token_group(x, layout="packed", q=aq, scales=sa), 100, 20)
            out.append({"workload": f"block-wise act quant 1x128 X bf16 [{m},{K}]",
                        "avg_us": round(float(d.mean()) * 1e3, 2)})
            for accum in ("exact", "mfma_fp8"):
                d = timed_events(lambda i: sg.fp8_scaled_gemm_blockwise(aq, sa, wps[i % 8], sw, y=y, accum=accum,
                                                                        w_layout="packed", a_layout="packed",
                                                                        a_shape=(m, K), w_shape=(N, K)), 100, 20)
                kb = N * K + 4 * sw.numel() + m * K + 4 * sa.numel() + 2 * m * N
                out.append({"workload": f"block-wise decode GEMM M={m} N={N} K={K}", "accum": accum,
                            "avg_us": round(float(d.mean()) * 1e3, 2), "GB_s": _gbs(kb, d.mean()),
                            "frac_hbm": round(_gbs(kb, d.mean()) / HBM_PEAK_GBS, 4)})
        del wps, wp
        torch.cuda.empty_cache()
        # prefill shapes
        for K in (4096, 14336):
            xb, w, _ = prefill_inputs(K)
            M, N = xb.shape[0], w.shape[0]
            xl = copies(to_bf16(xb), 2)
            aq, sa = sg.fp8_quant_per_token_group(xl[0])
            d = timed_events(lambda i: sg.fp8_quant_per_token_group(xl[i % 2], q=aq, scales=sa), 20, 3, reps=3)
            gbs = _gbs(3 * M * K + 4 * M * (K // 128), d.mean())
            out.append({"workload": f"block-wise act quant 1x128 X bf16 [{M},{K}]",
                        "avg_us": round(float(d.mean()) * 1e3, 2), "GB_s": gbs,
                        "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)})
            wq, sw = sg.fp8_quant_weight_blockwise(torch.from_numpy(w).to(dev))
            wp = sg.fp8_pack_weights(wq)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            d = timed_events(lambda i: sg.fp8_scaled_gemm_blockwise(aq, sa, wp, sw, y=y, accum="mfma_fp8",
                                                                    w_layout="packed", w_shape=(N, K)), 10, 3, reps=3)
            tf = _tflops(2.0 * M * N * K, d.mean())
            out.append({"workload": f"block-wise prefill GEMM {M}x{N}x{K}", "accum": "mfma_fp8",
                        "avg_us": round(float(d.mean()) * 1e3, 1), "TFLOPS": tf,
                        "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4)})
            del xl, aq, sa, wq, wp, y
            torch.cuda.empty_cache()

    if "mx" in wanted:
        log("mxfp8")
        from workloads import decode_inputs
        # decode shape: weights quantized offline straight into the packed MX order
        _, w, _ = decode_inputs(1)
        w_t = torch.from_numpy(w).to(dev)
        N, K = w.shape
        d = timed_events(lambda i: sg.fp8_quant_mx(w_t, layout="packed", scale_layout="packed"), 20, 3, reps=3)
        out.append({"workload": f"MX weight quant W fp32 [{N},{K}] 32-element blocks (offline)",
                    "avg_us": round(float(d.mean()) * 1e3, 1), "GB_s": _gbs(5 * N * K + N * K // 32, d.mean())})
        wp, ws = sg.fp8_quant_mx(w_t, layout="packed", scale_layout="packed")
        wps = copies(wp, 8)
        del w_t
        for m in (1, 8, 32):
            xb, _, _ = decode_inputs(m, with_weight=False)
            x = to_bf16(xb)
            aq, sa = sg.fp8_quant_mx(x, layout="packed", scale_layout="packed")
            y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
            d = timed_events(lambda i: sg.fp8_quant_mx(x, layout="packed", scale_layout="packed", q=aq, scales=sa),
                             100, 20)
            out.append({"workload": f"MX act quant X bf16 [{m},{K}]", "avg_us": round(float(d.mean()) * 1e3, 2)})
            d = timed_events(lambda i: sg.fp8_scaled_gemm_mx(aq, sa, wps[i % 8], ws, y=y, w_layout="packed",
                                                             a_layout="packed", a_shape=(m, K), w_shape=(N, K)),
                             100, 20)
            kb = N * K + ws.numel() + m * K + sa.numel() + 2 * m * N
            out.append({"workload": f"MX decode GEMM M={m} N={N} K={K}", "accum": "scaled mfma",
                        "avg_us": round(float(d.mean()) * 1e3, 2), "GB_s": _gbs(kb, d.mean()),
                        "frac_hbm": round(_gbs(kb, d.mean()) / HBM_PEAK_GBS, 4)})
            if m > 16:
                continue
            # the same call on bf16 X, quantized to MX blocks inside the GEMM kernel (one launch)
            d = timed_events(lambda i: sg.fp8_scaled_gemm_mx_bf16(x, wps[i % 8], ws, y=y, w_layout="packed",
                                                                  w_shape=(N, K)), 100, 20)
            kb = N * K + ws.numel() + 2 * m * K + 2 * m * N
            out.append({"workload": f"MX decode call M={m} N={N} K={K} (bf16 X, MX quantization inside the GEMM)",
                        "accum": "scaled mfma", "avg_us": round(float(d.mean()) * 1e3, 2), "GB_s": _gbs(kb, d.mean()),
                        "frac_hbm": round(_gbs(kb, d.mean()) / HBM_PEAK_GBS, 4)})
        del wps, wp
        torch.cuda.empty_cache()
        # prefill shapes, E4M3 and E5M2 activations
        for K in (4096, 14336):
            xb, w, _ = prefill_inputs(K)
            M, N = xb.shape[0], w.shape[0]
            xl = copies(to_bf16(xb), 2)
            wp, ws = sg.fp8_quant_mx(torch.from_numpy(w).to(dev), layout="packed", scale_layout="packed")
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            for fmt in ("e4m3", "e5m2"):
                aq, sa = sg.fp8_quant_mx(xl[0], fmt, layout="packed", scale_layout="packed")
                d = timed_events(lambda i: sg.fp8_quant_mx(xl[i % 2], fmt, layout="packed", scale_layout="packed",
                                                           q=aq, scales=sa), 20, 3, reps=3)
                gbs = _gbs(3 * M * K + M * K // 32, d.mean())
                out.append({"workload": f"MX act quant X bf16 [{M},{K}] {fmt}", "avg_us": round(float(d.mean()) * 1e3, 2),
                            "GB_s": gbs, "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)})
                d = timed_events(lambda i: sg.fp8_scaled_gemm_mx(aq, sa, wp, ws, a_fmt=fmt, y=y, w_layout="packed",
                                                                 a_layout="packed", a_shape=(M, K), w_shape=(N, K)),
                                 10, 3, reps=3)
                tf = _tflops(2.0 * M * N * K, d.mean())
                out.append({"workload": f"MX prefill GEMM {M}x{N}x{K} A {fmt}", "accum": "scaled mfma",
                            "avg_us": round(float(d.mean()) * 1e3, 1), "TFLOPS": tf,
                            "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4)})
                del aq, sa
            del xl, wp, ws, y
            torch.cuda.empty_cache()

    if "fp8out" in wanted:
        log("fp8 output epilogue")
        from workloads import decode_inputs
        # decode M = 32 and the K = 4096 prefill GEMM with E4M3 output codes
        # (per-tensor output scale), beside the same call with bf16 output
        _, w, _ = decode_inputs(1)
        wq, sw = sg.fp8_quant_weight_per_channel(torch.from_numpy(w).to(dev))
        wps = copies(sg.fp8_pack_weights(wq), 8)
        N, K = w.shape
        xb, _, _ = decode_inputs(32, with_weight=False)
        aq, sa = sg.fp8_quant_per_token(to_bf16(xb))
        ap = sg.fp8_pack_weights(aq)
        so = torch.tensor([0.05], dtype=torch.float32, device=dev)
        yq = torch.empty((32, N), dtype=torch.uint8, device=dev)
        d = timed_events(lambda i: sg.fp8_scaled_gemm_fp8out(ap, sa, wps[i % 8], sw, so, y=yq, w_layout="packed",
                                                             a_layout="packed", a_shape=(32, K)), 100, 20)
        kb = N * K + 4 * N + 32 * K + 4 * 32 + 32 * N
        out.append({"workload": f"decode GEMM kernel M=32 N={N} K={K}, E4M3 output (pre-quantized A)",
                    "accum": "exact", "avg_us": round(float(d.mean()) * 1e3, 2), "GB_s": _gbs(kb, d.mean()),
                    "frac_hbm": round(_gbs(kb, d.mean()) / HBM_PEAK_GBS, 4)})
        del wps, wq, aq, ap
        xb, w, _ = prefill_inputs(4096)
        M, N = xb.shape[0], w.shape[0]
        aq, sa = sg.fp8_quant_per_token(to_bf16(xb))
        ap = sg.fp8_pack_weights(aq)
        wq, sw = sg.fp8_quant_weight_per_channel(torch.from_numpy(w).to(dev))
        wp = sg.fp8_pack_weights(wq)
        yq = torch.empty((M, N), dtype=torch.uint8, device=dev)
        for accum in ("mfma_fp8", "exact"):
            d = timed_events(lambda i: sg.fp8_scaled_gemm_fp8out(ap, sa, wp, sw, so, y=yq, accum=accum,
                                                                 w_layout="packed", a_layout="packed",
                                                                 a_shape=(M, 4096)), 10, 3, reps=3)
            tf = _tflops(2.0 * M * N * 4096, d.mean())
            out.append({"workload": f"prefill GEMM {M}x{N}x4096, E4M3 output (pre-quantized A)", "accum": accum,
                        "avg_us": round(float(d.mean()) * 1e3, 1), "TFLOPS": tf,
                        "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4)})
        del aq, ap, wq, wp, yq
        torch.cuda.empty_cache()

    if "kv" in wanted or "attention" in wanted:
        log("kv cache")
        k, v, kc, vc = kv_inputs(0)
        B, S, H, D = k.shape
        numel = B * S * H * D
        kt, vt = to_bf16(k), to_bf16(v)
        del k, v
        for fmt in ("e4m3", "e5m2"):
            sk = sg.fp8_kv_calibrate(kt, fmt)
            sv = sg.fp8_kv_calibrate(vt, fmt)
            qk = sg.fp8_kv_quant(kt, sk, fmt)
            qv = sg.fp8_kv_quant(vt, sv, fmt)
            dk = torch.empty_like(kt)
            dv = torch.empty_like(vt)
            d = timed_events(lambda i: (sg.fp8_kv_calibrate(kt, fmt, sk), sg.fp8_kv_calibrate(vt, fmt, sv)), 10, 2, reps=3)
            out.append({"workload": f"KV calibrate K+V [{B},{S},{H},{D}] {fmt}", "avg_us": round(float(d.mean()) * 1e3, 1),
                        "GB_s": _gbs(4 * numel, d.mean()), "frac_hbm": round(_gbs(4 * numel, d.mean()) / HBM_PEAK_GBS, 4)})
            d = timed_events(lambda i: (sg.fp8_kv_quant(kt, sk, fmt, out=qk), sg.fp8_kv_quant(vt, sv, fmt, out=qv)),
                             10, 2, reps=3)
            out.append({"workload": f"KV quant K+V [{B},{S},{H},{D}] {fmt}", "avg_us": round(float(d.mean()) * 1e3, 1),
                        "GB_s": _gbs(6 * numel, d.mean()), "frac_hbm": round(_gbs(6 * numel, d.mean()) / HBM_PEAK_GBS, 4)})
            d = timed_events(lambda i: (sg.fp8_kv_dequant(qk, sk, fmt, out=dk), sg.fp8_kv_dequant(qv, sv, fmt, out=dv)),
                             10, 2, reps=3)
            out.append({"workload": f"KV dequant K+V [{B},{S},{H},{D}] {fmt}", "avg_us": round(float(d.mean()) * 1e3, 1),
                        "GB_s": _gbs(6 * numel, d.mean()), "frac_hbm": round(_gbs(6 * numel, d.mean()) / HBM_PEAK_GBS, 4)})
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
                d = timed_events(lambda i: sg.fp8_kv_decode_attention(qt, qk, qv, sk, sv, Lt, fmt, out=ao,
                                                                      workspace=aws), 20, 3, reps=3)
                nbytes = 2 * numel + 2 * 2 * B * 32 * D + 8 * H
                out.append({"workload": f"KV decode attention q [{B},32,{D}] over K+V [{B},{S},{H},{D}] {fmt}",
                            "avg_us": round(float(d.mean()) * 1e3, 1), "GB_s": _gbs(nbytes, d.mean()),
                            "frac_hbm": round(_gbs(nbytes, d.mean()) / HBM_PEAK_GBS, 4)})
                del qk, qv
            torch.cuda.empty_cache()
        kn, vn = kv_append_inputs(kc, vc)
        knt, vnt = to_bf16(kn), to_bf16(vn)
        del kt, vt
        torch.cuda.empty_cache()
        ck = torch.zeros((B, S + 1, H, D), dtype=torch.uint8, device=dev)
        cv = torch.zeros_like(ck)
        pos = torch.full((B,), S, dtype=torch.int32, device=dev)
        d = timed_events(lambda i: (sg.fp8_kv_append(knt, pos, sk, ck, "e5m2"), sg.fp8_kv_append(vnt, pos, sv, cv, "e5m2")),
                         200, 20, reps=3)
        out.append({"workload": f"KV append 1 token/seq K+V into [{B},{S + 1},{H},{D}]", "avg_us": round(float(d.mean()) * 1e3, 2),
                    "bytes": 2 * (B * H * D * 3)})
        del ck, cv
        torch.cuda.empty_cache()
    return out


def cpu_baseline(w_host, log):
    """The CPU oracle on the decode workload: per-token quantization of X plus the
    exact GEMM and bf16 epilogue, for M = 1, 8, 32 (the weight quantization is the
    offline step and is not timed).  Reported in the headline unit (GB/s of the
    same algorithmic bytes)."""
    from oracle import w8a8
    from workloads import decode_inputs, f32_from_bf16_bits
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    log("cpu baseline: oracle weight quantization (untimed)")
    # a bounded sample: the first 4096 of the 14336 output channels
    nsub = 4096
    wq, sw = w8a8.quant_weight_per_channel(w_host[:nsub])
    xs = {m: f32_from_bf16_bits(decode_inputs(m, with_weight=False)[0]) for m in DEC_MS}
    t = time.perf_counter()
    reps = 0
    while True:
        for m in DEC_MS:
            aq, sa = w8a8.quant_per_token(xs[m])
            w8a8.scaled_gemm_bf16(aq, sa, wq, sw)
        reps += 1
        if time.perf_counter() - t > 10.0 or reps >= 20:
            break
    dt = (time.perf_counter() - t) / reps
    sample_bytes = sum(nsub * DEC_K + 4 * nsub + 2 * m * DEC_K + 2 * m * nsub for m in DEC_MS)
    return {"value": round(sample_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"decode step (M=1,8,32, K=4096) on 4096 of the 14336 weight rows, {reps} reps, "
                      f"{dt * 1e3:.1f} ms per step; numpy/BLAS on {os.cpu_count()} host CPUs "
                      f"(BLAS threads {blas_threads}, the encoder single-threaded)"}


if __name__ == "__main__":
    main()
