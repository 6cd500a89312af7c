#!/usr/bin/env python3
"""Throughput of the block-scaled FP4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--tokens T]

The default run measures every workload of the metric -- FP4 GEMM TFLOP/s and GB/s
(with roofline fractions) at decode M = 1..32 and prefill M = 8192, and MoE tokens/s
-- and prints ONE JSON line.  Its headline is the decode GEMM at M = 32:

  decode   MXFP4 W4A4 GEMM, N=14336, K=4096, activations [M, 4096] bf16 N(0,1) with
           1% x20 outliers quantized on the fly, M = 1, 8, 32 (headline M = 32).  One
           step = the activation quantization plus the GEMM (the two launches of a
           fused fp4_gemm call, issued separately so the GEMM is timed by itself too).
           The weights rotate over copies that together exceed the 256 MB last-level
           cache, so every step streams them from HBM.  They are prepared once
           (fp4_prepare_weights: the layout the decode kernels stream); the GEMM on the
           row-major layout is timed beside it (gemm_us_row_major_weights).

and the other workloads ride along as records under "workloads":

  w4a16-small    NVFP4 W4A16 linear M=4 N=256 K=512 (launch-latency bound: us)
  prefill-nvfp4  NVFP4 W4A4 GEMM M=8192 N=4096 K=4096, fused activation quant, bf16 out
  prefill-mxfp4  the same GEMM in MXFP4
  moe-nvfp4      NVFP4 MoE, 128 experts top-8, hidden 2048, intermediate 768, T = 1, 64, 4096
  moe-mxfp4      MXFP4 MoE, 256 experts top-8 + shared, hidden 6144, intermediate 2048,
                 Zipf(1.1) routing, T = 64, 8192
  fp8-decode-mx, fp8-decode-rowwise
                 MXFP8 / FP8 rowwise (per-token x per-channel) GEMM, N=14336, K=4096,
                 M = 1, 8, 32: dynamic activation quantization + GEMM, rotated weights
  fp8-prefill-mx, fp8-prefill-block
                 MXFP8 / FP8 1x128-128x128 block-scaled GEMM, M=8192, N=4096, K=4096
  mx-w4a8-decode MX GEMM with FP4 (e2m1) weights and FP8 (e4m3) activations, N=14336,
                 K=4096, M = 1, 8, 32
  mxfp6-prefill  MXFP6 (e2m3) x MXFP6 (e2m3) GEMM, M=8192, N=4096, K=4096
  w4a16-prefill  NVFP4 W4A16 GEMM (bf16 activations), M=8192, N=4096, K=4096

--workload NAME measures one of them alone (its record becomes the line; used for
profiling runs).

Timing: every measured sequence is captured in a HIP graph (host launch overhead stays
out of the GPU timeline).  W untimed warmup steps, then the graph of exactly K steps is
replayed in 10 timed samples between two events on the launch stream, with
torch.cuda.synchronize() on both sides of each; the figure is the median sample.  The
dominant kernel's average launch time comes the same way from a graph of back-to-back
launches of that kernel alone (at least 50 per sample).  MoE records time the whole
fp4_moe_grouped_gemm call (all its launches, from bf16 hidden states and routing to
bf16 output); the router is timed on its own.  The CPU baseline times the oracle (test
infrastructure: the emulation definition in float64) on a bounded sample of each
workload, about 3 s each.
"""
import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp4": 10100.0, "fp8": 5000.0}
SAMPLES = 10
CPU_TARGET_S = 3.0
CSRC = os.path.join(ROOT, "block_scaled_fp4_quantize_amd", "csrc")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="all",
                   choices=["all", "decode", "w4a16-small", "prefill-nvfp4", "prefill-mxfp4",
                            "moe-nvfp4", "moe-mxfp4", "fp8-decode-mx", "fp8-decode-rowwise",
                            "fp8-prefill-mx", "fp8-prefill-block", "mx-w4a8-decode",
                            "mxfp6-prefill", "w4a16-prefill",
                            "prefill"])            # (old name of prefill-nvfp4)
    p.add_argument("--tokens", type=int, default=None, help="MoE token count (one)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run a plain elementwise kernel over 256 MiB (counter scaling)")
    return p.parse_args()


# ---------------------------------------------------------------------------------
# stored counter figures
# ---------------------------------------------------------------------------------


def source_hash(files):
    h = hashlib.sha256()
    for n in files:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(key):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current sources of that kernel; otherwise None."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(key)
    if not e or "sources" not in e or e.get("src_hash") != source_hash(e["sources"]):
        return None
    return e.get("bytes_per_launch")


# ---------------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------------


def capture(torch, fn, n):
    """A HIP graph of n calls fn(0) .. fn(n-1), captured on a side stream after one
    eager call (the library launches on torch's current stream, which during capture
    is the capturing stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def measure(torch, fn, steps, warmup, samples=SAMPLES):
    """W untimed warmup steps, then `samples` timed replays of a graph of exactly
    `steps` calls.  Returns (median ms per call, [ms per call of each sample], wall s
    of the timed replays)."""
    if warmup > 0:
        capture(torch, fn, warmup).replay()
    g = capture(torch, fn, steps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(samples)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for a, b in ev:
        torch.cuda.synchronize()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = [a.elapsed_time(b) / steps for a, b in ev]
    return statistics.median(per), per, wall


def kernel_avg_us(torch, fn, steps, warmup):
    """Average launch time (us) of one kernel from graphs of back-to-back launches."""
    ms, _, _ = measure(torch, fn, max(steps, 50), warmup)
    return ms * 1e3


def copy_bandwidth(torch):
    """Achievable HBM bandwidth: a plain device-to-device copy of 2 GiB (read + write
    counted), graph of back-to-back copies, median sample."""
    n = 1 << 29
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    ms, _, _ = measure(torch, lambda i: dst.copy_(src), 10, 2, samples=5)
    gbs = 2 * 4 * n / (ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"GBps": round(gbs, 1), "bytes_per_copy": 2 * 4 * n,
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "what": "torch copy_ of 2 GiB float32, read + write, graph of 10 copies, median of 5"}


def hbm_roof(achieved_gbs, copy, traffic=None, **extra):
    r = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    if copy:
        r["frac_of_copy"] = round(achieved_gbs / copy["GBps"], 4)
    r.update(extra)
    return r


def mfma_roof(achieved_tf, peak, traffic=None, **extra):
    r = {"bound": "mfma", "achieved": round(achieved_tf, 1), "peak": peak, "unit": "TFLOP/s",
         "frac": round(achieved_tf / peak, 4), "traffic": traffic}
    r.update(extra)
    return r


def bf16_tensor(torch, x, dev):
    import numpy as np
    import synth
    bits, vals = synth.bf16_bits(x)
    return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16), vals


# ---------------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------------


def bench_decode(args, torch, F, copy):
    import synth
    dev = torch.device("cuda:0")
    N, K, MMAX = 14336, 4096, 32
    w = torch.from_numpy(synth.normal((N, K), 0.02, seed=0, role=synth.WEIGHT)).to(dev)
    wc0 = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    ws0 = torch.empty((N, K // 32), dtype=torch.uint8, device=dev)
    F.fp4_quantize_weight(F.FP4_MXFP4, w, N, K, K, 1.0, wc0, ws0)
    del w
    wbytes = N * (K // 2 + K // 32)
    copies = max(2, -(-300 * 2 ** 20 // wbytes))          # > 256 MB last-level cache
    wc = torch.empty((copies, N, K // 2), dtype=torch.uint8, device=dev)
    ws = torch.empty((copies, N, K // 32), dtype=torch.uint8, device=dev)
    wc[:] = wc0
    ws[:] = ws0
    # the weights prepared once, as a serving engine would at load (fp4_prepare_weights);
    # the row-major layout is timed beside it
    wp = torch.empty_like(wc)
    chk = torch.zeros(1, dtype=torch.int32, device=dev)
    for c in range(copies):
        F.fp4_prepare_weights(F.FP4_MXFP4, wc[c], ws[c], N, K, wp[c], chk)
    a, _ = bf16_tensor(torch, synth.with_outliers(synth.normal((MMAX, K), seed=0, role=synth.ACT),
                                                  seed=0), dev)
    codes = torch.empty((MMAX, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((MMAX, K // 32), dtype=torch.uint8, device=dev)
    out = torch.empty((MMAX, N), dtype=torch.bfloat16, device=dev)
    names = {}

    def run(M):
        def quant(i):
            F.fp4_quantize_act(F.FP4_MXFP4, a, M, K, K, 1.0, codes, scales)
            names["quant"] = F.fp4_last_kernel()

        def gemm(i):
            c = i % copies
            F.fp4_gemm(F.FP4_MXFP4, F.FP4_W4A4, M, N, K, None, 0, codes, scales, wp[c], ws[c],
                       1.0, 1.0, out, N, F.FP4_OUT_BF16, F.FP4_FLAG_PREPARED_WEIGHTS, None, 0)
            names["gemm"] = F.fp4_last_kernel()

        def gemm_row_major(i):
            c = i % copies
            F.fp4_gemm(F.FP4_MXFP4, F.FP4_W4A4, M, N, K, None, 0, codes, scales, wc[c], ws[c],
                       1.0, 1.0, out, N, F.FP4_OUT_BF16, 0, None, 0)

        def step(i):
            quant(i)
            gemm(i)
        ms, per, wall = measure(torch, step, args.steps, args.warmup)
        quant(0)
        kus = kernel_avg_us(torch, gemm, args.steps, args.warmup)
        kus_rm = kernel_avg_us(torch, gemm_row_major, args.steps, args.warmup)
        qus = kernel_avg_us(torch, quant, args.steps, args.warmup)
        step_bytes = wbytes + M * K * 2 + M * N * 2                 # weights once, bf16 in, bf16 out
        kern_bytes = wbytes + M * (K // 2 + K // 32) + M * N * 2   # the GEMM's own operands
        flops = 2.0 * M * N * K
        kgbs = kern_bytes / (kus * 1e-6) / 1e9
        return {
            "M": M, "ms_per_step": ms, "samples_ms": [round(x, 6) for x in per], "wall_s": wall,
            "step_GBps": round(step_bytes / (ms * 1e-3) / 1e9, 2),
            "step_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 3),
            "gemm_us": round(kus, 3), "gemm_us_row_major_weights": round(kus_rm, 3),
            "quant_us": round(qus, 3),
            "gemm_TFLOPs": round(flops / (kus * 1e-6) / 1e12, 3),
            "roofline": hbm_roof(kgbs, copy, stored_traffic(f"decode_gemm_M{M}"),
                                 kernel=names.get("gemm"), algorithmic_bytes_per_launch=kern_bytes,
                                 avg_launch_us=round(kus, 3)),
        }

    per_m = {M: run(M) for M in (1, 8, MMAX)}
    main = per_m[MMAX]
    rec = {
        "metric": "FP4 decode GEMM GB/s (MXFP4 W4A4, M=32, N=14336, K=4096)",
        "value": main["step_GBps"], "unit": "GB/s", "ms_per_step": main["ms_per_step"],
        "dtype": "fp4",
        "config": {"workload": "MXFP4 W4A4 decode GEMV/GEMM, M=32 (also M=1, 8 under per_m), "
                               "N=14336, K=4096, activations quantized on the fly, weights "
                               "prepared once (fp4_prepare_weights)",
                   "M": MMAX, "N": N, "K": K, "weight_copies_rotated": copies},
        "roofline": main["roofline"],
        "per_m": {str(m): {k: v for k, v in r.items() if k not in ("wall_s",)}
                  for m, r in per_m.items()},
        "samples_ms": main["samples_ms"], "wall_s_timed": main["wall_s"],
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_decode()
    return rec


def bench_w4a16_small(args, torch, F, copy):
    import numpy as np
    import synth
    dev = torch.device("cuda:0")
    M, N, K = 4, 256, 512
    w = synth.normal((N, K), 0.02, seed=0, role=synth.WEIGHT)
    ws2 = float(np.float32(np.abs(w).max()) / np.float32(2688.0))
    wd = torch.from_numpy(w).to(dev)
    wc = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    wsc = torch.empty((N, K // 16), dtype=torch.uint8, device=dev)
    F.fp4_quantize_weight(F.FP4_NVFP4, wd, N, K, K, ws2, wc, wsc)
    a, _ = bf16_tensor(torch, synth.normal((M, K), seed=0, role=synth.ACT), dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    names = {}

    def gemm(i):
        F.fp4_gemm(F.FP4_NVFP4, F.FP4_W4A16, M, N, K, a, K, None, None, wc, wsc, ws2, 0.0,
                   out, N, F.FP4_OUT_BF16, 0, None, 0)
        names["gemm"] = F.fp4_last_kernel()

    ms, per, wall = measure(torch, gemm, max(args.steps, 50), args.warmup)
    nbytes = N * (K // 2 + K // 16) + M * K * 2 + M * N * 2
    flops = 2.0 * M * N * K
    rec = {
        "metric": "NVFP4 W4A16 linear us per call (M=4, N=256, K=512)",
        "value": round(ms * 1e3, 3), "unit": "us", "higher_is_better": False,
        "ms_per_step": ms, "dtype": "bf16",
        "config": {"workload": "NVFP4 W4A16 linear, weights [256, 512], activations [4, 512] bf16",
                   "M": M, "N": N, "K": K},
        "roofline": hbm_roof(nbytes / (ms * 1e-3) / 1e9, copy, None, kernel=names.get("gemm"),
                             algorithmic_bytes_per_launch=nbytes, avg_launch_us=round(ms * 1e3, 3),
                             note="launch-latency bound: 79,872 bytes take 10 ns at 8 TB/s"),
        "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 4),
        "samples_ms": [round(x, 6) for x in per], "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_w4a16_small()
    return rec


def bench_prefill(args, torch, F, copy, fmt):
    import numpy as np
    import synth
    dev = torch.device("cuda:0")
    M, N, K = 8192, 4096, 4096
    nv = fmt == "nvfp4"
    fm, G = (F.FP4_NVFP4, 16) if nv else (F.FP4_MXFP4, 32)
    w = synth.normal((N, K), 0.02, seed=0, role=synth.WEIGHT)
    ws2 = float(np.float32(np.abs(w).max()) / np.float32(2688.0)) if nv else 1.0
    wd = torch.from_numpy(w).to(dev)
    wc = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    wsc = torch.empty((N, K // G), dtype=torch.uint8, device=dev)
    F.fp4_quantize_weight(fm, wd, N, K, K, ws2, wc, wsc)
    del wd
    a, av = bf16_tensor(torch, synth.normal((M, K), seed=0, role=synth.ACT, index=3), dev)
    s = float(np.float32(np.abs(av).max()) / np.float32(2688.0)) if nv else 1.0
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // G), dtype=torch.uint8, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    # the workspace with room for the fused quantization and the stage-ordered scales
    wsn = F.fp4_gemm_workspace_size_mnk(fm, F.FP4_W4A4, M, N, K, 1)
    wsb = torch.empty(wsn, dtype=torch.uint8, device=dev)
    names = {}
    F.fp4_quantize_act(fm, a, M, K, K, s, codes, scales)

    def gemm(i):
        # pre-quantized activations: the scale re-layout pass and the GEMM kernel
        F.fp4_gemm(fm, F.FP4_W4A4, M, N, K, None, 0, codes, scales, wc, wsc, ws2, s,
                   out, N, F.FP4_OUT_BF16, 0, wsb, wsn)
        names["gemm"] = F.fp4_last_kernel()

    def step(i):
        # the whole fused W4A4 call: activation quantization, scale re-layout, GEMM
        F.fp4_gemm(fm, F.FP4_W4A4, M, N, K, a, K, None, None, wc, wsc, ws2, s,
                   out, N, F.FP4_OUT_BF16, 0, wsb, wsn)

    ms, per, wall = measure(torch, step, args.steps, args.warmup)
    kus = kernel_avg_us(torch, gemm, args.steps, 2)
    flops = 2.0 * M * N * K
    tf = flops / (kus * 1e-6) / 1e12
    # NVFP4 runs its products on fp16 MFMAs (exact decode), MXFP4 on the scaled FP4 MFMA
    pk = PEAK_TFLOPS["fp16"] if nv else PEAK_TFLOPS["fp4"]
    F_ = fmt.upper()
    rec = {
        "metric": f"FP4 prefill GEMM TFLOP/s ({F_} W4A4, M=8192, N=4096, K=4096)",
        "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": ms,
        "dtype": "fp16" if nv else "fp4",
        "config": {"workload": f"{F_} W4A4 prefill GEMM, fused activation quant, bf16 out",
                   "M": M, "N": N, "K": K},
        "roofline": mfma_roof(tf, pk, stored_traffic("prefill_gemm_" + fmt),
                              frac_of_fp4_peak=round(tf / PEAK_TFLOPS["fp4"], 4),
                              frac_of_fp8_peak=round(tf / PEAK_TFLOPS["fp8"], 4),
                              kernel=names.get("gemm"), algorithmic_flops_per_launch=flops,
                              avg_launch_us=round(kus, 2),
                              timed="scale_relayout + " + str(names.get("gemm")) +
                                    " back to back (one fp4_gemm call on quantized activations)"),
        "step_GBps": round((N * K * (0.5 + 1 / G) + M * K * 2 + M * N * 2) / (ms * 1e-3) / 1e9, 1),
        "samples_ms": [round(x, 6) for x in per], "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_prefill(fmt=fmt)
    return rec


# ---- FP8 family: MXFP8 and FP8 W8A8 -----------------------------------------------


def _fp8_scale_shape(mode, rows, K, weight):
    if mode == "mx":
        return (rows, K // 32), 1
    if mode == "rowwise":
        return (rows,), 4
    if mode == "block":
        return (((rows + 127) // 128) if weight else rows, K // 128), 4
    return None, 0


def _fp8_operands(torch, F, mode, N, K, dev, copies=1):
    import synth
    m = F.FP8_MODES[mode]
    w = torch.from_numpy(synth.normal((N, K), 0.02, seed=0, role=synth.WEIGHT)).to(dev)
    shp, esz = _fp8_scale_shape(mode, N, K, True)
    sdt = torch.uint8 if esz == 1 else torch.float32
    wc = torch.empty((copies, N, K), dtype=torch.uint8, device=dev)
    ws = torch.empty((copies,) + shp, dtype=sdt, device=dev)
    F.fp8_quantize_weight(m, w, N, K, K, 1.0, wc[0], ws[0])
    for c in range(1, copies):
        wc[c] = wc[0]
        ws[c] = ws[0]
    del w
    return wc, ws, N * K + ws[0].numel() * esz


def bench_fp8_decode(args, torch, F, copy, mode):
    import synth
    dev = torch.device("cuda:0")
    N, K, MMAX = 14336, 4096, 32
    m = F.FP8_MODES[mode]
    wbytes = N * K + (N * K // 32 if mode == "mx" else N * 4)
    copies = max(2, -(-300 * 2 ** 20 // wbytes))          # > 256 MB last-level cache
    wc, ws, wbytes = _fp8_operands(torch, F, mode, N, K, dev, copies)
    a, _ = bf16_tensor(torch, synth.with_outliers(synth.normal((MMAX, K), seed=0, role=synth.ACT),
                                                  seed=0), dev)
    codes = torch.empty((MMAX, K), dtype=torch.uint8, device=dev)
    shp, esz = _fp8_scale_shape(mode, MMAX, K, False)
    scales = torch.empty(shp, dtype=torch.uint8 if esz == 1 else torch.float32, device=dev)
    out = torch.empty((MMAX, N), dtype=torch.bfloat16, device=dev)
    names = {}

    def run(M):
        def quant(i):
            F.fp8_quantize_act(m, a, M, K, K, 1.0, codes, scales)
            names["quant"] = F.fp4_last_kernel()

        def gemm(i):
            c = i % copies
            F.fp8_gemm(m, M, N, K, codes, scales, 1.0, wc[c], ws[c], 1.0, out, N, F.FP4_OUT_BF16)
            names["gemm"] = F.fp4_last_kernel()

        def step(i):
            quant(i)
            gemm(i)
        ms, per, wall = measure(torch, step, args.steps, args.warmup)
        quant(0)
        kus = kernel_avg_us(torch, gemm, args.steps, args.warmup)
        qus = kernel_avg_us(torch, quant, args.steps, args.warmup)
        a_sc = M * K // 32 if mode == "mx" else M * 4
        step_bytes = wbytes + M * K * 2 + M * N * 2
        kern_bytes = wbytes + M * K + a_sc + M * N * 2
        flops = 2.0 * M * N * K
        return {
            "M": M, "ms_per_step": ms, "samples_ms": [round(x, 6) for x in per], "wall_s": wall,
            "step_GBps": round(step_bytes / (ms * 1e-3) / 1e9, 2),
            "gemm_us": round(kus, 3), "quant_us": round(qus, 3),
            "gemm_TFLOPs": round(flops / (kus * 1e-6) / 1e12, 3),
            "roofline": hbm_roof(kern_bytes / (kus * 1e-6) / 1e9, copy,
                                 stored_traffic(f"fp8_decode_{mode}_M{M}"),
                                 kernel=names.get("gemm"), algorithmic_bytes_per_launch=kern_bytes,
                                 avg_launch_us=round(kus, 3)),
        }

    per_m = {M: run(M) for M in (1, 8, MMAX)}
    main = per_m[MMAX]
    label = "MXFP8" if mode == "mx" else "FP8 rowwise"
    rec = {
        "metric": f"FP8 decode GEMM GB/s ({label}, M=32, N=14336, K=4096)",
        "value": main["step_GBps"], "unit": "GB/s", "ms_per_step": main["ms_per_step"],
        "dtype": "fp8",
        "config": {"workload": f"{label} decode GEMM, M=32 (also M=1, 8 under per_m), N=14336, "
                               "K=4096, dynamic activation quantization",
                   "M": MMAX, "N": N, "K": K, "weight_copies_rotated": copies},
        "roofline": main["roofline"],
        "per_m": {str(mm): {k: v for k, v in r.items() if k != "wall_s"} for mm, r in per_m.items()},
        "samples_ms": main["samples_ms"], "wall_s_timed": main["wall_s"],
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_fp8(mode, MMAX, N, K, w_rows=2048)
    return rec


def bench_fp8_prefill(args, torch, F, copy, mode):
    import synth
    dev = torch.device("cuda:0")
    M, N, K = 8192, 4096, 4096
    m = F.FP8_MODES[mode]
    wc, ws, wbytes = _fp8_operands(torch, F, mode, N, K, dev)
    wc, ws = wc[0], ws[0]
    a, _ = bf16_tensor(torch, synth.normal((M, K), seed=0, role=synth.ACT, index=3), dev)
    codes = torch.empty((M, K), dtype=torch.uint8, device=dev)
    shp, esz = _fp8_scale_shape(mode, M, K, False)
    scales = torch.empty(shp, dtype=torch.uint8 if esz == 1 else torch.float32, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    names = {}

    def quant(i):
        F.fp8_quantize_act(m, a, M, K, K, 1.0, codes, scales)
        names["quant"] = F.fp4_last_kernel()

    def gemm(i):
        F.fp8_gemm(m, M, N, K, codes, scales, 1.0, wc, ws, 1.0, out, N, F.FP4_OUT_BF16)
        names["gemm"] = F.fp4_last_kernel()

    def step(i):
        quant(i)
        gemm(i)

    ms, per, wall = measure(torch, step, args.steps, args.warmup)
    kus = kernel_avg_us(torch, gemm, args.steps, 2)
    qus = kernel_avg_us(torch, quant, args.steps, 2)
    flops = 2.0 * M * N * K
    tf = flops / (kus * 1e-6) / 1e12
    label = "MXFP8" if mode == "mx" else "FP8 block-scaled"
    rec = {
        "metric": f"FP8 prefill GEMM TFLOP/s ({label}, M=8192, N=4096, K=4096)",
        "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": ms,
        "dtype": "fp8",
        "config": {"workload": f"{label} prefill GEMM, dynamic activation quantization, bf16 out",
                   "M": M, "N": N, "K": K},
        "roofline": mfma_roof(tf, PEAK_TFLOPS["fp8"], stored_traffic(f"fp8_prefill_{mode}"),
                              kernel=names.get("gemm"), algorithmic_flops_per_launch=flops,
                              avg_launch_us=round(kus, 2)),
        "quant_us": round(qus, 2), "quant_kernel": names.get("quant"),
        "samples_ms": [round(x, 6) for x in per], "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_fp8(mode, 64, N, K, prefill=True)
    return rec


# ---- MX formats of any element type ---------------------------------------------------


def _mx_weights(torch, F, we, N, K, dev, copies=1):
    import synth
    e = F.MX_ELEMS[we]
    w = torch.from_numpy(synth.normal((N, K), 0.02, seed=0, role=synth.WEIGHT)).to(dev)
    wc = torch.empty((copies, N, K * F.MX_BITS[e] // 8), dtype=torch.uint8, device=dev)
    ws = torch.empty((copies, N, K // 32), dtype=torch.uint8, device=dev)
    F.mx_quantize_weight(e, w, N, K, K, wc[0], ws[0])
    for c in range(1, copies):
        wc[c] = wc[0]
        ws[c] = ws[0]
    del w
    return wc, ws, N * K * F.MX_BITS[e] // 8 + N * K // 32


def bench_mx_decode(args, torch, F, copy, ae="e4m3", we="e2m1"):
    import synth
    dev = torch.device("cuda:0")
    N, K, MMAX = 14336, 4096, 32
    ea, ew = F.MX_ELEMS[ae], F.MX_ELEMS[we]
    wbytes = N * K * F.MX_BITS[ew] // 8 + N * K // 32
    copies = max(2, -(-300 * 2 ** 20 // wbytes))          # > 256 MB last-level cache
    wc, ws, wbytes = _mx_weights(torch, F, we, N, K, dev, copies)
    a, _ = bf16_tensor(torch, synth.with_outliers(synth.normal((MMAX, K), seed=0, role=synth.ACT),
                                                  seed=0), dev)
    codes = torch.empty((MMAX, K * F.MX_BITS[ea] // 8), dtype=torch.uint8, device=dev)
    scales = torch.empty((MMAX, K // 32), dtype=torch.uint8, device=dev)
    out = torch.empty((MMAX, N), dtype=torch.bfloat16, device=dev)
    names = {}

    def run(M):
        def quant(i):
            F.mx_quantize_act(ea, a, M, K, K, codes, scales)

        def gemm(i):
            c = i % copies
            F.mx_gemm(ea, ew, M, N, K, codes, scales, wc[c], ws[c], out, N, F.FP4_OUT_BF16)
            names["gemm"] = F.fp4_last_kernel()

        def step(i):
            quant(i)
            gemm(i)
        ms, per, wall = measure(torch, step, args.steps, args.warmup)
        quant(0)
        kus = kernel_avg_us(torch, gemm, args.steps, args.warmup)
        step_bytes = wbytes + M * K * 2 + M * N * 2
        kern_bytes = wbytes + M * (K * F.MX_BITS[ea] // 8 + K // 32) + M * N * 2
        return {
            "M": M, "ms_per_step": ms, "samples_ms": [round(x, 6) for x in per], "wall_s": wall,
            "step_GBps": round(step_bytes / (ms * 1e-3) / 1e9, 2), "gemm_us": round(kus, 3),
            "roofline": hbm_roof(kern_bytes / (kus * 1e-6) / 1e9, copy,
                                 stored_traffic(f"mx_decode_{ae}_{we}_M{M}"),
                                 kernel=names.get("gemm"), algorithmic_bytes_per_launch=kern_bytes,
                                 avg_launch_us=round(kus, 3)),
        }

    per_m = {M: run(M) for M in (1, 8, MMAX)}
    main = per_m[MMAX]
    rec = {
        "metric": f"MX decode GEMM GB/s ({we} weights x {ae} activations, M=32, N=14336, K=4096)",
        "value": main["step_GBps"], "unit": "GB/s", "ms_per_step": main["ms_per_step"],
        "dtype": f"{we}x{ae}",
        "config": {"workload": f"MX GEMM, {we} weights x {ae} activations quantized on the fly, "
                               "M=32 (also M=1, 8 under per_m), N=14336, K=4096",
                   "M": MMAX, "N": N, "K": K, "weight_copies_rotated": copies},
        "roofline": main["roofline"],
        "per_m": {str(mm): {k: v for k, v in r.items() if k != "wall_s"} for mm, r in per_m.items()},
        "samples_ms": main["samples_ms"], "wall_s_timed": main["wall_s"],
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_mx(ae, we, MMAX, N, K, w_rows=2048)
    return rec


def bench_mx_prefill(args, torch, F, copy, ae="e2m3", we="e2m3"):
    import synth
    dev = torch.device("cuda:0")
    M, N, K = 8192, 4096, 4096
    ea, ew = F.MX_ELEMS[ae], F.MX_ELEMS[we]
    wc, ws, _ = _mx_weights(torch, F, we, N, K, dev)
    wc, ws = wc[0], ws[0]
    a, _ = bf16_tensor(torch, synth.normal((M, K), seed=0, role=synth.ACT, index=3), dev)
    codes = torch.empty((M, K * F.MX_BITS[ea] // 8), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    names = {}

    def quant(i):
        F.mx_quantize_act(ea, a, M, K, K, codes, scales)
        names["quant"] = F.fp4_last_kernel()

    def gemm(i):
        F.mx_gemm(ea, ew, M, N, K, codes, scales, wc, ws, out, N, F.FP4_OUT_BF16)
        names["gemm"] = F.fp4_last_kernel()

    def step(i):
        quant(i)
        gemm(i)

    ms, per, wall = measure(torch, step, args.steps, args.warmup)
    kus = kernel_avg_us(torch, gemm, args.steps, 2)
    qus = kernel_avg_us(torch, quant, args.steps, 2)
    flops = 2.0 * M * N * K
    tf = flops / (kus * 1e-6) / 1e12
    # the scaled MFMA runs 6- and 4-bit operands at the FP4/FP6 rate, anything with e4m3 at
    # the FP8 rate
    pk = PEAK_TFLOPS["fp8"] if "e4m3" in (ae, we) else PEAK_TFLOPS["fp4"]
    rec = {
        "metric": f"MX prefill GEMM TFLOP/s ({ae} x {we}, M=8192, N=4096, K=4096)",
        "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": ms,
        "dtype": f"{ae}x{we}",
        "config": {"workload": f"MX GEMM, {ae} activations quantized on the fly x {we} weights, "
                               "bf16 out", "M": M, "N": N, "K": K},
        "roofline": mfma_roof(tf, pk, stored_traffic(f"mx_prefill_{ae}_{we}"),
                              kernel=names.get("gemm"), algorithmic_flops_per_launch=flops,
                              avg_launch_us=round(kus, 2)),
        "quant_us": round(qus, 2), "quant_kernel": names.get("quant"),
        "samples_ms": [round(x, 6) for x in per], "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_mx(ae, we, 64, N, K, prefill=True)
    return rec


def bench_w4a16_prefill(args, torch, F, copy):
    import numpy as np
    import synth
    dev = torch.device("cuda:0")
    M, N, K = 8192, 4096, 4096
    w = synth.normal((N, K), 0.02, seed=0, role=synth.WEIGHT)
    ws2 = float(np.float32(np.abs(w).max()) / np.float32(2688.0))
    wd = torch.from_numpy(w).to(dev)
    wc = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    wsc = torch.empty((N, K // 16), dtype=torch.uint8, device=dev)
    F.fp4_quantize_weight(F.FP4_NVFP4, wd, N, K, K, ws2, wc, wsc)
    del wd
    a, _ = bf16_tensor(torch, synth.normal((M, K), seed=0, role=synth.ACT, index=3), dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    names = {}

    def gemm(i):
        F.fp4_gemm(F.FP4_NVFP4, F.FP4_W4A16, M, N, K, a, K, None, None, wc, wsc, ws2, 0.0,
                   out, N, F.FP4_OUT_BF16, 0, None, 0)
        names["gemm"] = F.fp4_last_kernel()

    ms, per, wall = measure(torch, gemm, args.steps, args.warmup)
    kus = kernel_avg_us(torch, gemm, args.steps, 2)
    flops = 2.0 * M * N * K
    tf = flops / (kus * 1e-6) / 1e12
    rec = {
        "metric": "FP4 W4A16 prefill GEMM TFLOP/s (NVFP4 weights, bf16 activations, M=8192, "
                  "N=4096, K=4096)",
        "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": ms,
        "dtype": "bf16",
        "config": {"workload": "NVFP4 W4A16 prefill GEMM, bf16 activations, bf16 out",
                   "M": M, "N": N, "K": K},
        "roofline": mfma_roof(tf, PEAK_TFLOPS["bf16"], stored_traffic("w4a16_prefill_nvfp4"),
                              kernel=names.get("gemm"), algorithmic_flops_per_launch=flops,
                              avg_launch_us=round(kus, 2)),
        "samples_ms": [round(x, 6) for x in per], "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_w4a16_prefill()
    return rec


class MoeLayer:
    """One of the two MoE layers on the device: a few experts quantized on the GPU, the
    others seeded row permutations of them (distinct memory, same distribution)."""

    def __init__(self, torch, F, fmt):
        import numpy as np
        import synth
        from block_scaled_fp4_quantize_amd import tensors as T
        self.torch, self.F, self.T_mod, self.fmt = torch, F, T, fmt
        dev = self.dev = torch.device("cuda:0")
        if fmt == "nvfp4":
            E, k, H, I, shared, zipf, copies = 128, 8, 2048, 768, False, None, 2
        else:
            E, k, H, I, shared, zipf, copies = 256, 8, 6144, 2048, True, 1.1, 1
        self.E, self.k, self.H, self.I, self.shared_on, self.zipf = E, k, H, I, shared, zipf
        G = self.G = 16 if fmt == "nvfp4" else 32
        fm = F.FP4_NVFP4 if fmt == "nvfp4" else F.FP4_MXFP4

        def qw(rows, cols, index, role):
            w = torch.from_numpy(synth.normal((rows, cols), 0.02, seed=0, role=role, index=index)).to(dev)
            ws2 = float(np.float32(float(w.abs().max().item()) / 2688.0)) if fmt == "nvfp4" else 1.0
            c = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
            s = torch.empty((rows, cols // G), dtype=torch.uint8, device=dev)
            F.fp4_quantize_weight(fm, w, rows, cols, cols, ws2, c, s)
            return c, s, ws2

        n_base = 4
        base = [(qw(2 * I, H, b, synth.W13), qw(H, I, b, synth.W2)) for b in range(n_base + 1)]
        # `copies` full sets of expert weights, used in turn by successive steps, so
        # that the set a decode step reads is not left in the 256 MB last-level cache
        self.sets = []
        s13, s2 = np.zeros(E, np.float32), np.zeros(E, np.float32)
        for c in range(copies):
            w13c = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev)
            w13s = torch.empty((E, 2 * I, H // G), dtype=torch.uint8, device=dev)
            w2c = torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev)
            w2s = torch.empty((E, H, I // G), dtype=torch.uint8, device=dev)
            for e in range(E):
                (c13, sc13, ws13), (c2, sc2, ws2) = base[e % n_base]
                p13 = torch.from_numpy(synth.rows_permutation(2 * I, seed=c, index=2 * e)).to(dev)
                p2 = torch.from_numpy(synth.rows_permutation(H, seed=c, index=2 * e + 1)).to(dev)
                w13c[e], w13s[e], w2c[e], w2s[e] = c13[p13], sc13[p13], c2[p2], sc2[p2]
                s13[e], s2[e] = ws13, ws2
            self.sets.append((w13c, w13s, w2c, w2s))
        self.s13, self.s2 = s13, s2
        self.sh = None
        if shared:
            (c13, sc13, _), (c2, sc2, _) = base[n_base]
            self.sh = dict(w13_codes=c13, w13_scales=sc13, w2_codes=c2, w2_scales=sc2)
        self.wbytes_expert = 3 * H * I // 2 + 3 * H * I // G

    def bench(self, args, T_, copy):
        import numpy as np
        import synth
        torch, F, T = self.torch, self.F, self.T_mod
        E, k, H, I, fmt = self.E, self.k, self.H, self.I, self.fmt
        dev = self.dev
        hidden, hv = bf16_tensor(torch, synth.normal((T_, H), seed=0, role=synth.HIDDEN), dev)
        # routing of successive steps varies (a decode step's tokens reach different
        # experts); the large batches already reach every expert
        n_var = 8 if T_ <= 64 else 1
        routes = []
        for v in range(n_var):
            if self.zipf:
                logits = synth.zipf_gumbel_logits(T_, E, self.zipf, seed=0, index=v)
            else:
                logits = synth.normal((T_, E), seed=0, role=synth.LOGITS, index=v)
            ld = torch.from_numpy(logits).to(dev)
            routes.append((ld,) + T.topk_softmax(ld, k))
        kw = {}
        if fmt == "nvfp4":
            a13 = np.full(E, np.float32(np.abs(hv).max() / 2688.0), np.float32)
            a2 = np.full(E, np.float32(4.0 / 2688.0), np.float32)   # fixed calibration for timing
            kw = dict(w13_scale_2=self.s13, w2_scale_2=self.s2, a13_scale=a13, a2_scale=a2)
        out = torch.empty((T_, H), dtype=torch.bfloat16, device=dev)
        variants, keep = [], []
        ws_need = 0
        for v in range(max(n_var, len(self.sets))):
            w13c, w13s, w2c, w2s = self.sets[v % len(self.sets)]
            moe = T.Moe(fmt, "w4a4", H, I, E, w13c, w13s, w2c, w2s, shared=self.sh, **kw)
            _, ids, w = routes[v % n_var]
            a, kp = moe.args(hidden, ids, w, out)
            keep.append((moe, kp))
            variants.append(a)
            ws_need = max(ws_need, F.fp4_moe_workspace_size(a))
        wsb = torch.empty(ws_need, dtype=torch.uint8, device=dev)

        def step(i):
            F.fp4_moe_grouped_gemm(variants[i % len(variants)], wsb, ws_need, device_tensor=hidden)

        ms, per, wall = measure(torch, step, args.steps, args.warmup)
        ld0 = routes[0][0]
        ids_r = torch.empty((T_, k), dtype=torch.int32, device=dev)
        w_r = torch.empty((T_, k), dtype=torch.float32, device=dev)
        router_us = kernel_avg_us(
            torch, lambda i: F.fp4_moe_topk_softmax(ld0, T_, E, k, 1, ids_r, w_r), args.steps, 2)
        touched = statistics.mean(int(torch.unique(r[1]).numel()) for r in routes)
        nbytes = (touched + (1 if self.sh else 0)) * self.wbytes_expert + T_ * H * 2 * 2
        flops = 2.0 * 3 * H * I * (T_ * k + (T_ if self.sh else 0))
        # roofline of the whole call: weight-streaming token counts against HBM, large
        # token counts against the MFMA peak of the format's instruction (NVFP4: fp16
        # MFMA on the exact decode; MXFP4: FP4 MFMA)
        if T_ * k >= 32 * E:
            peak = PEAK_TFLOPS["fp16"] if fmt == "nvfp4" else PEAK_TFLOPS["fp4"]
            roof = mfma_roof(flops / (ms * 1e-3) / 1e12, peak, None,
                             kernel="fp4_moe_grouped_gemm (whole call)",
                             algorithmic_flops_per_call=flops, avg_call_us=round(ms * 1e3, 2))
        else:
            roof = hbm_roof(nbytes / (ms * 1e-3) / 1e9, copy, None,
                            kernel="fp4_moe_grouped_gemm (whole call)",
                            algorithmic_bytes_per_call=int(nbytes), avg_call_us=round(ms * 1e3, 2))
        label = (f"{fmt.upper()} W4A4 MoE E={E} top-{k} H={H} I={I} T={T_}"
                 + (" + shared expert, Zipf(1.1) routing" if self.sh else ", N(0,1) logits"))
        rec = {
            "metric": f"{fmt.upper()} MoE tokens/s (T={T_})",
            "value": round(T_ / (ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": ms,
            "dtype": "fp16" if fmt == "nvfp4" else "fp4",
            "config": {"workload": label, "T": T_, "experts_touched_per_step": touched,
                       "routing_variants": n_var, "weight_sets": len(self.sets)},
            "roofline": roof,
            "achieved_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "achieved_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
            "router_us": round(router_us, 2),
            "samples_ms": [round(x, 6) for x in per], "wall_s_timed": wall,
        }
        if fmt == "nvfp4":
            rec["zero_input_scale_call"] = self.reject_case(hidden, routes[0], kw, out)
        if not args.no_cpu_baseline:
            rec["cpu_baseline"] = cpu_baseline_moe(self, hv, routes[0][1], routes[0][2], kw)
        return rec

    def reject_case(self, hidden, route, kw, out):
        """A weight-only checkpoint's zero activation scale: refused, nothing launched."""
        import numpy as np
        F, T = self.F, self.T_mod
        a13 = kw["a13_scale"].copy()
        a13[3] = 0.0
        kw2 = dict(kw, a13_scale=a13)
        moe = T.Moe(self.fmt, "w4a4", self.H, self.I, self.E, *self.sets[0], shared=self.sh, **kw2)
        st = moe(hidden, route[1], route[2], out, check=False)[1]
        return F.status_str(st)


# ---------------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample
# ---------------------------------------------------------------------------------


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def host_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = None
    return {"os_cpu_count": os.cpu_count(), "affinity_cpus": aff, "cpu_model": model,
            "blas_threads": blas_threads()}


def _repeat(fn, target_s):
    n, t0 = 0, time.perf_counter()
    while True:
        fn(n)
        n += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            return n, el


def cpu_baseline_decode(target_s=CPU_TARGET_S, rows=2048):
    import synth
    from oracle import gemm as OG
    from oracle import quant as OQ
    N, K, M = 14336, 4096, 32
    w = synth.normal((N, K), 0.02, seed=0, role=synth.WEIGHT)[:rows]
    wc, ws, _ = OQ.quantize_weight("mxfp4", w)          # checkpoint preparation, untimed
    a32 = synth.with_outliers(synth.normal((M, K), seed=0, role=synth.ACT), seed=0)
    _, av = synth.bf16_bits(a32)
    n, el = _repeat(lambda i: OG.gemm_fused("mxfp4", av, wc, ws), target_s)
    step_bytes = rows * (K // 2 + K // 32) + M * K * 2 + M * rows * 2
    return {"value": round(step_bytes * n / el / 1e9, 4), "unit": "GB/s",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"first {rows} of {N} weight rows (M=32, K=4096), {n} repetitions in "
                      f"{el:.1f} s: activation QDQ + float64 weight dequant + float64 matmul"}


def cpu_baseline_w4a16_small(target_s=1.0):
    import numpy as np
    import synth
    from oracle import gemm as OG
    from oracle import quant as OQ
    M, N, K = 4, 256, 512
    wc, ws, ws2 = OQ.quantize_weight("nvfp4", synth.normal((N, K), 0.02, seed=0, role=synth.WEIGHT))
    _, av = synth.bf16_bits(synth.normal((M, K), seed=0, role=synth.ACT))
    n, el = _repeat(lambda i: OG.gemm_w4a16("nvfp4", av, wc, ws, ws2), target_s)
    return {"value": round(el / n * 1e6, 2), "unit": "us", "cores": blas_threads(), "kind": "oracle",
            "sample": f"the whole workload, {n} repetitions in {el:.1f} s: float64 weight dequant "
                      "+ float64 matmul"}


def cpu_baseline_prefill(target_s=CPU_TARGET_S, rows=64, fmt="nvfp4"):
    import numpy as np
    import synth
    from oracle import gemm as OG
    from oracle import quant as OQ
    M, N, K = 8192, 4096, 4096
    w = synth.normal((N, K), 0.02, seed=0, role=synth.WEIGHT)
    wc, ws, ws2 = OQ.quantize_weight(fmt, w)
    _, av = synth.bf16_bits(synth.normal((M, K), seed=0, role=synth.ACT, index=3))
    s = float(np.float32(np.abs(av).max()) / np.float32(2688.0)) if fmt == "nvfp4" else 1.0
    n, el = _repeat(lambda i: OG.gemm_fused(fmt, av[i * rows % M:(i * rows % M) + rows], wc, ws,
                                            ws2, s), target_s)
    flops = 2.0 * rows * N * K * n
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{rows}-row slices of the 8192 activation rows against the full weight, "
                      f"{n} repetitions in {el:.1f} s"}


def cpu_baseline_moe(layer, hv, ids, w, kw, target_s=CPU_TARGET_S):
    """The oracle MoE layer over the first tokens of the same problem (same routing,
    the same expert codes and scales copied to the host), one token at a time, for
    about target_s seconds of oracle time (at least one token)."""
    import numpy as np
    from oracle import moe as OM
    fmt, E, k, H, I = layer.fmt, layer.E, layer.k, layer.H, layer.I
    w13c, w13s, w2c, w2s = layer.sets[0]
    ids_h = ids.cpu().numpy()
    w_h = w.cpu().numpy().astype(np.float64)
    cache = {}

    def expert(e):
        if e not in cache:
            kwe = {}
            if fmt == "nvfp4":
                kwe = dict(w13_scale_2=float(layer.s13[e]), w2_scale_2=float(layer.s2[e]),
                           a13_scale=float(kw["a13_scale"][e]), a2_scale=float(kw["a2_scale"][e]))
            cache[e] = OM.Expert(w13c[e].cpu().numpy(), w13s[e].cpu().numpy(),
                                 w2c[e].cpu().numpy(), w2s[e].cpu().numpy(), **kwe)
        return cache[e]

    # experts the sampled token does not reach carry no weights, only valid scales
    idle = OM.Expert(None, None, None, None, a13_scale=1.0, a2_scale=1.0)
    shared = None
    if layer.sh is not None:
        sh = layer.sh
        shared = OM.Expert(sh["w13_codes"].cpu().numpy(), sh["w13_scales"].cpu().numpy(),
                           sh["w2_codes"].cpu().numpy(), sh["w2_scales"].cpu().numpy())
    n, el = 0, 0.0
    while (el < target_s or n == 0) and n < hv.shape[0]:
        experts = {int(e): expert(int(e)) for e in ids_h[n]}      # host copies, untimed
        full = [experts.get(e, idle) for e in range(E)]
        t0 = time.perf_counter()
        OM.moe(fmt, "w4a4", hv[n:n + 1], ids_h[n:n + 1], w_h[n:n + 1], full, shared)
        el += time.perf_counter() - t0
        n += 1
    return {"value": round(n / el, 4), "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"the first {n} token(s) one at a time ({n} x {k} routed experts"
                      + (" + the shared expert" if layer.sh is not None else "")
                      + f", H={H}, I={I}) in {el:.1f} s of oracle time"}


def cpu_baseline_fp8(mode, M, N, K, w_rows=None, prefill=False, target_s=CPU_TARGET_S):
    """The oracle's FP8 chain (dynamic activation quantization, dequantization of both
    operands, float64 matmul) on a bounded sample."""
    import synth
    from oracle import fp8 as O8
    w = synth.normal((N, K), 0.02, seed=0, role=synth.WEIGHT)
    if w_rows:
        w = w[:w_rows]
    om = {"rowwise": O8.ROWWISE, "block": O8.BLOCK}
    if mode == "mx":
        wc, wsc = O8.quantize_mxfp8(w)
    else:
        wc, wsc = O8.quantize_weight(om[mode], w)
    idx = 3 if prefill else 0
    a = synth.normal((8192 if prefill else M, K), seed=0, role=synth.ACT, index=idx)
    if not prefill:
        a = synth.with_outliers(a, seed=0)
    _, av = synth.bf16_bits(a)

    def one(i):
        x = av[(i * M) % av.shape[0]:(i * M) % av.shape[0] + M]
        if mode == "mx":
            ac, asc = O8.quantize_mxfp8(x)
            return O8.gemm_mxfp8(ac, asc, wc, wsc)
        ac, asc = O8.quantize_act(om[mode], x)
        return O8.gemm(om[mode], ac, asc, wc, wsc)

    n, el = _repeat(one, target_s)
    rows = w.shape[0]
    if prefill:
        return {"value": round(2.0 * M * rows * K * n / el / 1e12, 6), "unit": "TFLOP/s",
                "cores": blas_threads(), "kind": "oracle",
                "sample": f"{M}-row slices of the 8192 activation rows against the full weight, "
                          f"{n} repetitions in {el:.1f} s"}
    wb = rows * K + (rows * K // 32 if mode == "mx" else rows * 4)
    step_bytes = wb + M * K * 2 + M * rows * 2
    return {"value": round(step_bytes * n / el / 1e9, 4), "unit": "GB/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"first {rows} of {N} weight rows (M={M}, K={K}), {n} repetitions in "
                      f"{el:.1f} s: activation quantization + float64 dequant + float64 matmul"}


def cpu_baseline_mx(ae, we, M, N, K, w_rows=None, prefill=False, target_s=CPU_TARGET_S):
    """The oracle's MX chain (activation quantization, dequantization of both operands,
    float64 matmul) on a bounded sample."""
    import synth
    from oracle import mx as OX
    w = synth.normal((N, K), 0.02, seed=0, role=synth.WEIGHT)
    if w_rows:
        w = w[:w_rows]
    wc, wsc = OX.quantize(we, w)
    a = synth.normal((8192 if prefill else M, K), seed=0, role=synth.ACT, index=3 if prefill else 0)
    if not prefill:
        a = synth.with_outliers(a, seed=0)
    _, av = synth.bf16_bits(a)

    def one(i):
        x = av[(i * M) % av.shape[0]:(i * M) % av.shape[0] + M]
        ac, asc = OX.quantize(ae, x)
        return OX.gemm(ae, ac, asc, we, wc, wsc)

    n, el = _repeat(one, target_s)
    rows = w.shape[0]
    if prefill:
        return {"value": round(2.0 * M * rows * K * n / el / 1e12, 6), "unit": "TFLOP/s",
                "cores": blas_threads(), "kind": "oracle",
                "sample": f"{M}-row slices of the 8192 activation rows against the full weight, "
                          f"{n} repetitions in {el:.1f} s"}
    bits = OX.BITS[we]
    step_bytes = rows * K * bits // 8 + rows * K // 32 + M * K * 2 + M * rows * 2
    return {"value": round(step_bytes * n / el / 1e9, 4), "unit": "GB/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"first {rows} of {N} weight rows (M={M}, K={K}), {n} repetitions in "
                      f"{el:.1f} s: activation quantization + float64 dequant + float64 matmul"}


def cpu_baseline_w4a16_prefill(target_s=CPU_TARGET_S, rows=64):
    import numpy as np
    import synth
    from oracle import gemm as OG
    from oracle import quant as OQ
    M, N, K = 8192, 4096, 4096
    wc, ws, ws2 = OQ.quantize_weight("nvfp4", synth.normal((N, K), 0.02, seed=0, role=synth.WEIGHT))
    _, av = synth.bf16_bits(synth.normal((M, K), seed=0, role=synth.ACT, index=3))
    n, el = _repeat(lambda i: OG.gemm_w4a16("nvfp4", av[i * rows % M:(i * rows % M) + rows], wc,
                                            ws, ws2), target_s)
    return {"value": round(2.0 * rows * N * K * n / el / 1e12, 6), "unit": "TFLOP/s",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"{rows}-row slices of the 8192 activation rows against the full weight, "
                      f"{n} repetitions in {el:.1f} s: float64 weight dequant + float64 matmul"}


# ---------------------------------------------------------------------------------


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the kernels run on a single MI355X; sharding is not implemented)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(1)
    import block_scaled_fp4_quantize_amd as F   # raises if libfp4.so is missing
    t_start = time.perf_counter()
    if args.copy_calibration:
        # a plain elementwise kernel that reads 256 MiB and writes 256 MiB: the
        # counter scale for FETCH_SIZE / WRITE_SIZE of the kernels measured after it
        src = torch.ones(64 * 2 ** 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    wl = "prefill-nvfp4" if args.workload == "prefill" else args.workload
    copy = copy_bandwidth(torch) if wl in ("all", "decode", "w4a16-small", "moe-nvfp4",
                                          "moe-mxfp4") else None

    def log(msg):
        print(f"[bench] {msg} ({time.perf_counter() - t_start:.1f} s)", file=sys.stderr, flush=True)

    records = {}
    if wl in ("all", "decode"):
        records["decode"] = bench_decode(args, torch, F, copy)
        log("decode done")
    if wl in ("all", "w4a16-small"):
        records["w4a16-small"] = bench_w4a16_small(args, torch, F, copy)
        log("w4a16-small done")
    for fmt in ("nvfp4", "mxfp4"):
        if wl in ("all", f"prefill-{fmt}"):
            records[f"prefill-{fmt}"] = bench_prefill(args, torch, F, copy, fmt)
            torch.cuda.empty_cache()
            log(f"prefill-{fmt} done")
    for fmt, toks in (("nvfp4", (1, 64, 4096)), ("mxfp4", (64, 8192))):
        if wl not in ("all", f"moe-{fmt}"):
            continue
        layer = MoeLayer(torch, F, fmt)
        for T_ in ((args.tokens,) if args.tokens else toks):
            records[f"moe-{fmt}-T{T_}"] = layer.bench(args, T_, copy)
            torch.cuda.empty_cache()
            log(f"moe-{fmt} T={T_} done")
        del layer
        torch.cuda.empty_cache()
    for mode in ("mx", "rowwise"):
        if wl in ("all", f"fp8-decode-{mode}"):
            if copy is None:
                copy = copy_bandwidth(torch)
            records[f"fp8-decode-{mode}"] = bench_fp8_decode(args, torch, F, copy, mode)
            torch.cuda.empty_cache()
            log(f"fp8-decode-{mode} done")
    for mode in ("mx", "block"):
        if wl in ("all", f"fp8-prefill-{mode}"):
            records[f"fp8-prefill-{mode}"] = bench_fp8_prefill(args, torch, F, copy, mode)
            torch.cuda.empty_cache()
            log(f"fp8-prefill-{mode} done")
    if wl in ("all", "mx-w4a8-decode"):
        if copy is None:
            copy = copy_bandwidth(torch)
        records["mx-w4a8-decode"] = bench_mx_decode(args, torch, F, copy)
        torch.cuda.empty_cache()
        log("mx-w4a8-decode done")
    if wl in ("all", "w4a16-prefill"):
        records["w4a16-prefill"] = bench_w4a16_prefill(args, torch, F, copy)
        torch.cuda.empty_cache()
        log("w4a16-prefill done")
    if wl in ("all", "mxfp6-prefill"):
        records["mxfp6-prefill"] = bench_mx_prefill(args, torch, F, copy)
        torch.cuda.empty_cache()
        log("mxfp6-prefill done")

    head_key = "decode" if wl == "all" else next(iter(records))
    head = dict(records[head_key])
    line = {"metric": head.pop("metric"), "value": head.pop("value"), "unit": head.pop("unit"),
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(head.pop("ms_per_step"), 6),
            "higher_is_better": head.pop("higher_is_better", True),
            "scaling": "weak", "vs_baseline": None, "dtype": head.pop("dtype", "fp4"),
            "data": "synthetic (seeded N(0,0.02) weights quantized on the GPU, N(0,1) activations)",
            "config": head.pop("config")}
    line.update(head)
    line["timing"] = (f"median of {SAMPLES} timed replays of a graph of {args.steps} steps "
                      f"after {args.warmup} warmup steps; kernel averages from graphs of "
                      f">= 50 back-to-back launches")
    line["host"] = host_info()
    if copy:
        line["hbm_copy"] = copy
    if wl == "all":
        line["workloads"] = {k: v for k, v in records.items() if k != head_key}
    line["bench_wall_s"] = round(time.perf_counter() - t_start, 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
