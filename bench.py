#!/usr/bin/env python3
"""Throughput of the block-scaled FP4 hot path on one MI355X.

    python bench.py [--steps K] [--warmup W]
                    [--workload decode|prefill|prefill-mxfp4|moe-nvfp4|moe-mxfp4]

Default workload (decode): MXFP4 W4A4 GEMM, N=14336, K=4096, activations
[32, 4096] bf16 N(0,1) with 1% x20 outliers quantized on the fly.  One step = the
activation quantization plus the GEMM at M=32 (the two launches the fused
fp4_gemm call makes, issued separately so the GEMM can be timed by itself).  The
weights rotate over enough copies that the set exceeds the 256 MB last-level
cache, so the GEMM streams them from HBM every step.  M=1 and M=8 are measured the
same way and reported under "per_m".

Other workloads (one JSON line each, not the default):
  prefill    NVFP4 W4A4 GEMM M=8192 N=4096 K=4096, fused quantization, bf16 out
  prefill-mxfp4  the same GEMM in MXFP4
  moe-nvfp4  NVFP4 MoE, 128 experts top-8, hidden 2048, intermediate 768, T=--tokens
  moe-mxfp4  MXFP4 MoE, 256 experts top-8 + shared, hidden 6144, intermediate 2048,
             Zipf(1.1) routing, T=--tokens

Timing: the launches are captured in HIP graphs so host launch overhead stays
out of the GPU timeline.  W untimed warmup steps, then exactly K steps replayed
between two events on the launch stream, with torch.cuda.synchronize() on both
sides.  The dominant kernel's average duration is measured the same way from a
graph of K back-to-back launches of that kernel alone (it includes the small gap
between graph nodes).  The CPU baseline times the oracle (test infrastructure, the emulation
definition in float64) on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp4": 10100.0, "fp8": 5000.0}
KERNEL_SOURCES = ["gemm.hip", "gemm_tile.hip", "gemm_resident.hip", "quant.hip", "moe.hip", "device.h",
                  "internal.h"]


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode",
                   choices=["decode", "prefill", "prefill-mxfp4", "moe-nvfp4", "moe-mxfp4"])
    p.add_argument("--tokens", type=int, default=None, help="MoE token count")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run a plain elementwise kernel over 256 MiB (counter scaling)")
    return p.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    for n in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_scaled_fp4_quantize_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(key):
    """HBM bytes per launch from the committed counter summary, if it was taken on
    the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(key)
    if not e or e.get("src_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


# ---------------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------------


def capture(torch, fn, n):
    """A HIP graph of n calls fn(0) .. fn(n-1), captured on a side stream after one
    eager call (the library launches on torch's current stream, which during
    capture is the capturing stream)."""
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


def timed_graph(torch, fn, steps, warmup):
    """W untimed warmup steps, then exactly K steps replayed from one graph between
    two events, with synchronizations on both sides.  Returns (ms per step, wall s)."""
    if warmup > 0:
        capture(torch, fn, warmup).replay()
    g = capture(torch, fn, steps)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, time.perf_counter() - wall0


def bench_decode(args, torch, F):
    import numpy as np
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
    a32 = synth.with_outliers(synth.normal((MMAX, K), seed=0, role=synth.ACT), seed=0)
    bits, _ = synth.bf16_bits(a32)
    a = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    codes = torch.empty((MMAX, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((MMAX, K // 32), dtype=torch.uint8, device=dev)
    out = torch.empty((MMAX, N), dtype=torch.bfloat16, device=dev)
    names = {}

    def run(M, steps, warmup):
        def quant(i):
            F.fp4_quantize_act(F.FP4_MXFP4, a, M, K, K, 1.0, codes, scales)
            names["quant"] = F.fp4_last_kernel()

        def gemm(i):
            c = i % copies
            F.fp4_gemm(F.FP4_MXFP4, F.FP4_W4A4, M, N, K, None, 0, codes, scales, wc[c], ws[c],
                       1.0, 1.0, out, N, F.FP4_OUT_BF16, 0, None, 0)
            names["gemm"] = F.fp4_last_kernel()

        def step(i):
            quant(i)
            gemm(i)
        # the step: activation quantization + GEMM, K times
        ms, wall = timed_graph(torch, step, steps, warmup)
        # the GEMM kernel alone: K back-to-back launches (same weight rotation)
        quant(0)
        kms, _ = timed_graph(torch, gemm, steps, warmup)
        step_bytes = wbytes + M * K * 2 + M * N * 2                  # weights once, bf16 in, bf16 out
        kern_bytes = wbytes + M * (K // 2 + K // 32) + M * N * 2    # the GEMM's own operands
        flops = 2.0 * M * N * K
        return dict(M=M, ms_per_step=ms, gemm_us=kms * 1e3, wall_s=wall,
                    step_GBps=step_bytes / (ms * 1e-3) / 1e9,
                    gemm_GBps=kern_bytes / (kms * 1e-3) / 1e9,
                    gemm_TFLOPs=flops / (kms * 1e-3) / 1e12,
                    gemm_frac_hbm=kern_bytes / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    step_bytes=step_bytes, kern_bytes=kern_bytes, kernel=names.get("gemm"))

    per_m = {}
    for M in (1, 8):
        per_m[M] = run(M, max(20, args.steps // 2), max(5, args.warmup // 2))
    main = run(MMAX, args.steps, args.warmup)
    per_m[MMAX] = main
    traffic = stored_traffic(f"decode_gemm_M{MMAX}")
    res = {
        "metric": "FP4 decode GEMM GB/s (MXFP4 W4A4, M=32, N=14336, K=4096)",
        "value": round(main["step_GBps"], 2),
        "unit": "GB/s",
        "ms_per_step": main["ms_per_step"],
        "dtype": "fp4",
        "config": {"workload": "MXFP4 W4A4 decode GEMV/GEMM, M=32 (also M=1, 8 under per_m), "
                               "N=14336, K=4096, activations quantized on the fly",
                   "M": MMAX, "N": N, "K": K, "weight_copies_rotated": copies},
        "roofline": {"bound": "hbm", "achieved": round(main["gemm_GBps"], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(main["gemm_frac_hbm"], 4), "traffic": traffic,
                     "kernel": main["kernel"], "algorithmic_bytes_per_launch": main["kern_bytes"],
                     "avg_launch_us": round(main["gemm_us"], 3)},
        "per_m": {str(m): {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()
                           if k in ("ms_per_step", "gemm_us", "step_GBps", "gemm_GBps",
                                    "gemm_TFLOPs", "gemm_frac_hbm", "kernel")}
                  for m, r in per_m.items()},
        "wall_s_timed": main["wall_s"],
    }
    return res


def bench_prefill(args, torch, F, fmt="nvfp4"):
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
    bits, av = synth.bf16_bits(synth.normal((M, K), seed=0, role=synth.ACT, index=3))
    s = float(np.float32(np.abs(av).max()) / np.float32(2688.0)) if nv else 1.0
    a = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // G), dtype=torch.uint8, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    names = {}

    def quant(i):
        F.fp4_quantize_act(fm, a, M, K, K, s, codes, scales)

    def gemm(i):
        F.fp4_gemm(fm, F.FP4_W4A4, M, N, K, None, 0, codes, scales, wc, wsc, ws2, s,
                   out, N, F.FP4_OUT_BF16, 0, None, 0)
        names["gemm"] = F.fp4_last_kernel()

    def step(i):
        quant(i)
        gemm(i)

    steps = max(5, args.steps // 20)
    ms, wall = timed_graph(torch, step, steps, max(2, args.warmup // 10))
    kms, _ = timed_graph(torch, gemm, steps, 2)
    flops = 2.0 * M * N * K
    tf = flops / (kms * 1e-3) / 1e12
    # NVFP4 runs its products on fp16 MFMAs (exact decode), MXFP4 on the scaled FP4 MFMA
    pk = PEAK_TFLOPS["fp16"] if nv else PEAK_TFLOPS["fp4"]
    F_ = fmt.upper()
    return {
        "metric": f"FP4 prefill GEMM TFLOP/s ({F_} W4A4, M=8192, N=4096, K=4096)",
        "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": ms,
        "steps_override": steps,
        "dtype": "fp16" if nv else "fp4",
        "config": {"workload": f"{F_} W4A4 prefill GEMM, fused activation quant, bf16 out",
                   "M": M, "N": N, "K": K},
        "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": pk,
                     "unit": "TFLOP/s", "frac": round(tf / pk, 4),
                     "frac_of_fp4_peak": round(tf / PEAK_TFLOPS["fp4"], 4),
                     "traffic": stored_traffic("prefill_gemm_" + fmt), "kernel": names.get("gemm"),
                     "avg_launch_us": round(kms * 1e3, 2)},
        "wall_s_timed": wall,
    }


def bench_moe(args, torch, F, fmt):
    import numpy as np
    from block_scaled_fp4_quantize_amd import tensors as T
    import synth
    dev = torch.device("cuda:0")
    if fmt == "nvfp4":
        E, k, H, I, T_ = 128, 8, 2048, 768, args.tokens or 64
        shared, zipf = False, None
    else:
        E, k, H, I, T_ = 256, 8, 6144, 2048, args.tokens or 64
        shared, zipf = True, 1.1
    G = 16 if fmt == "nvfp4" else 32
    fm = F.FP4_NVFP4 if fmt == "nvfp4" else F.FP4_MXFP4
    n_w = E + (1 if shared else 0)

    def qw(rows, cols, index, role):
        w = torch.from_numpy(synth.normal((rows, cols), 0.02, seed=0, role=role, index=index)).to(dev)
        ws2 = float(w.abs().max().item()) / 2688.0 if fmt == "nvfp4" else 1.0
        ws2 = float(np.float32(ws2))
        c = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((rows, cols // G), dtype=torch.uint8, device=dev)
        F.fp4_quantize_weight(fm, w, rows, cols, cols, ws2, c, s)
        return c, s, ws2

    # a few distinct experts quantized on the GPU, each further expert a row
    # permutation of one of them (distinct memory, same value distribution)
    n_base = 4
    base = [(qw(2 * I, H, b, synth.W13), qw(H, I, b, synth.W2)) for b in range(n_base + 1)]
    w13c = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev)
    w13s = torch.empty((E, 2 * I, H // G), dtype=torch.uint8, device=dev)
    w2c = torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev)
    w2s = torch.empty((E, H, I // G), dtype=torch.uint8, device=dev)
    s13, s2 = np.zeros(E, np.float32), np.zeros(E, np.float32)
    for e in range(E):
        (c13, sc13, ws13), (c2, sc2, ws2) = base[e % n_base]
        p13 = torch.from_numpy(synth.rows_permutation(2 * I, seed=0, index=2 * e)).to(dev)
        p2 = torch.from_numpy(synth.rows_permutation(H, seed=0, index=2 * e + 1)).to(dev)
        w13c[e], w13s[e], w2c[e], w2s[e] = c13[p13], sc13[p13], c2[p2], sc2[p2]
        s13[e], s2[e] = ws13, ws2
    sh = None
    if shared:
        (c13, sc13, ws13), (c2, sc2, ws2) = base[n_base]
        sh = dict(w13_codes=c13, w13_scales=sc13, w2_codes=c2, w2_scales=sc2)
    bits, hv = synth.bf16_bits(synth.normal((T_, H), seed=0, role=synth.HIDDEN))
    hidden = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    if zipf:
        logits = synth.zipf_gumbel_logits(T_, E, zipf, seed=0)
    else:
        logits = synth.normal((T_, E), seed=0, role=synth.LOGITS)
    ids, w = T.topk_softmax(torch.from_numpy(logits).to(dev), k)
    kw = {}
    if fmt == "nvfp4":
        a13 = np.full(E, np.float32(np.abs(hv).max() / 2688.0), np.float32)
        a2 = np.full(E, np.float32(4.0 / 2688.0), np.float32)   # fixed calibration for timing
        kw = dict(w13_scale_2=s13, w2_scale_2=s2, a13_scale=a13, a2_scale=a2)
    moe = T.Moe(fmt, "w4a4", H, I, E, w13c, w13s, w2c, w2s, shared=sh, **kw)
    out = torch.empty((T_, H), dtype=torch.bfloat16, device=dev)
    args_c, keep = moe.args(hidden, ids, w, out)
    wsb, need = moe.workspace_for(args_c)

    def step(i):
        F.fp4_moe_grouped_gemm(args_c, wsb, need, device_tensor=hidden)

    steps = max(5, args.steps // 10)
    ms, wall = timed_graph(torch, step, steps, max(2, args.warmup // 5))
    touched = int(torch.unique(ids).numel())
    wbytes_expert = 3 * H * I // 2 + 3 * H * I // G
    bytes_ = (touched + (1 if shared else 0)) * wbytes_expert + T_ * H * 2 * 2
    flops = 2.0 * 3 * H * I * (T_ * k + (T_ if shared else 0))
    # Roofline of the whole fp4_moe_grouped_gemm call (all of its launches on one
    # stream, timed by the step graph's events): weight-streaming decode token counts
    # against HBM, large token counts against the MFMA peak of the format's
    # instruction (NVFP4: fp16 MFMA on the exact decode; MXFP4: FP4 MFMA).
    if T_ * k >= 32 * E:
        peak = 2500.0 if fmt == "nvfp4" else 10100.0
        achieved = flops / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None,
                "kernel": "fp4_moe_grouped_gemm (whole call)",
                "algorithmic_flops_per_call": flops, "avg_call_us": round(ms * 1e3, 2)}
    else:
        achieved = bytes_ / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": 8000.0, "unit": "GB/s",
                "frac": round(achieved / 8000.0, 4), "traffic": None,
                "kernel": "fp4_moe_grouped_gemm (whole call)",
                "algorithmic_bytes_per_call": bytes_, "avg_call_us": round(ms * 1e3, 2)}
    res_cpu = None
    if not args.no_cpu_baseline:
        res_cpu = cpu_baseline_moe(fmt, hv, ids, w, w13c, w13s, w2c, w2s, s13, s2, sh, kw,
                                   E, k, H, I)
    out_line = {
        "metric": f"{fmt.upper()} MoE tokens/s (T={T_})", "value": round(T_ / (ms * 1e-3), 1),
        "unit": "tokens/s", "ms_per_step": ms, "steps_override": steps,
        "config": {"workload": f"{fmt.upper()} W4A4 MoE E={E} top-{k} H={H} I={I} T={T_}"
                               + (" + shared, Zipf(1.1)" if shared else ""),
                   "experts_touched": touched},
        "roofline": roof,
        "achieved_GBps": round(bytes_ / (ms * 1e-3) / 1e9, 1),
        "achieved_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
        "wall_s_timed": wall,
    }
    if res_cpu is not None:
        out_line["cpu_baseline"] = res_cpu
    return out_line


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


def cpu_baseline_decode(target_s=10.0, rows=2048):
    import numpy as np
    import synth
    from oracle import gemm as OG
    from oracle import quant as OQ
    N, K, M = 14336, 4096, 32
    w = synth.normal((N, K), 0.02, seed=0, role=synth.WEIGHT)[:rows]
    wc, ws, _ = OQ.quantize_weight("mxfp4", w)          # checkpoint preparation, untimed
    a32 = synth.with_outliers(synth.normal((M, K), seed=0, role=synth.ACT), seed=0)
    _, av = synth.bf16_bits(a32)
    n = 0
    t0 = time.perf_counter()
    while True:
        OG.gemm_fused("mxfp4", av, wc, ws)
        n += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    step_bytes = rows * (K // 2 + K // 32) + M * K * 2 + M * rows * 2
    return {"value": round(step_bytes * n / el / 1e9, 4), "unit": "GB/s",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"first {rows} of {N} weight rows (M=32, K=4096), {n} repetitions in "
                      f"{el:.1f} s: activation QDQ + float64 weight dequant + float64 matmul"}


def cpu_baseline_prefill(target_s=10.0, rows=64, fmt="nvfp4"):
    import numpy as np
    import synth
    from oracle import gemm as OG
    from oracle import quant as OQ
    M, N, K = 8192, 4096, 4096
    w = synth.normal((N, K), 0.02, seed=0, role=synth.WEIGHT)
    wc, ws, ws2 = OQ.quantize_weight(fmt, w)
    _, av = synth.bf16_bits(synth.normal((M, K), seed=0, role=synth.ACT, index=3))
    s = float(np.float32(np.abs(av).max()) / np.float32(2688.0)) if fmt == "nvfp4" else 1.0
    n = 0
    t0 = time.perf_counter()
    while True:
        OG.gemm_fused(fmt, av[n * rows % M:(n * rows % M) + rows], wc, ws, ws2, s)
        n += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    flops = 2.0 * rows * N * K * n
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{rows}-row slices of the 8192 activation rows against the full weight, "
                      f"{n} repetitions in {el:.1f} s"}


def cpu_baseline_moe(fmt, hv, ids, w, w13c, w13s, w2c, w2s, s13, s2, sh, kw, E, k, H, I,
                     target_s=10.0):
    """The oracle MoE layer over the first tokens of the same problem (same routing,
    the same expert codes and scales copied to the host), token by token, for about
    target_s seconds."""
    import numpy as np
    from oracle import moe as OM
    ids_h = ids.cpu().numpy()
    w_h = w.cpu().numpy().astype(np.float64)
    cache = {}

    def expert(e):
        if e not in cache:
            kwe = {}
            if fmt == "nvfp4":
                kwe = dict(w13_scale_2=float(s13[e]), w2_scale_2=float(s2[e]),
                           a13_scale=float(kw["a13_scale"][e]), a2_scale=float(kw["a2_scale"][e]))
            cache[e] = OM.Expert(w13c[e].cpu().numpy(), w13s[e].cpu().numpy(),
                                 w2c[e].cpu().numpy(), w2s[e].cpu().numpy(), **kwe)
        return cache[e]

    # experts the sampled token does not reach carry no weights, only valid scales
    idle = OM.Expert(None, None, None, None, a13_scale=1.0, a2_scale=1.0)
    shared = None
    if sh is not None:
        shared = OM.Expert(sh["w13_codes"].cpu().numpy(), sh["w13_scales"].cpu().numpy(),
                           sh["w2_codes"].cpu().numpy(), sh["w2_scales"].cpu().numpy())
    n = 0
    el = 0.0
    while el < target_s and n < hv.shape[0]:
        experts = {int(e): expert(int(e)) for e in ids_h[n]}      # host copies, untimed
        full = [experts.get(e, idle) for e in range(E)]
        t0 = time.perf_counter()
        OM.moe(fmt, "w4a4", hv[n:n + 1], ids_h[n:n + 1], w_h[n:n + 1], full, shared)
        el += time.perf_counter() - t0
        n += 1
    return {"value": round(n / el, 4), "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"the first {n} tokens one at a time ({n} x {k} routed experts"
                      + (" + the shared expert" if sh is not None else "")
                      + f", H={H}, I={I}) in {el:.1f} s of oracle time"}


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
    if args.copy_calibration:
        # a plain elementwise kernel that reads 256 MiB and writes 256 MiB: the
        # counter scale for FETCH_SIZE / WRITE_SIZE of the kernels measured after it
        src = torch.ones(64 * 2 ** 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if args.workload == "decode":
        res = bench_decode(args, torch, F)
        steps = args.steps
    elif args.workload in ("prefill", "prefill-mxfp4"):
        res = bench_prefill(args, torch, F, "nvfp4" if args.workload == "prefill" else "mxfp4")
        steps = res.pop("steps_override")
    else:
        res = bench_moe(args, torch, F, args.workload.split("-")[1])
        steps = res.pop("steps_override")
    line = {"metric": res.pop("metric"), "value": res.pop("value"), "unit": res.pop("unit"),
            "n_gpus": 1, "steps": steps, "warmup": args.warmup,
            "ms_per_step": round(res.pop("ms_per_step"), 6), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": res.pop("dtype", "fp4"),
            "data": "synthetic (seeded N(0,0.02) weights quantized on the GPU, N(0,1) activations)",
            "config": res.pop("config")}
    line.update(res)
    if not args.no_cpu_baseline:
        if args.workload == "decode":
            line["cpu_baseline"] = cpu_baseline_decode()
        elif args.workload in ("prefill", "prefill-mxfp4"):
            line["cpu_baseline"] = cpu_baseline_prefill(
                fmt="nvfp4" if args.workload == "prefill" else "mxfp4")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
