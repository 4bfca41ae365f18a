"""Benchmark of the NVFP4 decode hot path on one MI355X.

Workload (one "step"): the small-M decode sweep -- for every M in {1,2,4,8,16}
and every (K, N) in {(4096,14336), (14336,4096), (4096,6144)}, one nvfp4_gemm
call on bf16 activations X[M x K] (1% outlier channels x50, quantized to NVFP4
inside the call: amax, block scales, codes) against pre-quantized NVFP4
weights W[N x K] (from N(0, 0.02)), FP32 output. 15 calls per step.

Timing: each step is captured once in a HIP graph and replayed, so host launch
overhead is not measured. Every call reads a different copy of its weight
(ring of copies, > 512 MB between reuses) so the 256 MB last-level cache
cannot serve the weights; inputs are resident in HBM before timing starts.

value = algorithmic bytes of the step (weight codes + scales once, bf16 X once,
FP32 y once) / step time, in GB/s.

Also reported (same JSON line):
  roofline     the decode GEMM kernel alone (pre-quantized activations), HIP
               events over graph replays of that kernel, against 8 TB/s;
  cpu_baseline the CPU oracle (activation quantize + FP64 GEMM) on a bounded
               sample of the same sweep, on the host cores;
  detail       per (M, K, N) us/call and GB/s for the whole call and the kernel,
               the residue-compensated variant, the M=64 augmented-channel
               product and the prefill TFLOP/s.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from block_scaled_fp4_02_amd import inputs  # noqa: E402

METRIC = "NVFP4 GEMM µs & HBM GB/s at M=1–16; prefill TFLOP/s; % of roofline"
HBM_PEAK_GBS = 8000.0
F16_MFMA_PEAK_TFLOPS = 2500.0
FP4_MFMA_PEAK_TFLOPS = 10100.0
QUANT_BYTES_PER_ELEM = 2.5625      # bf16 read + codes + E4M3 scales
RING_BYTES = 640 << 20


def profiled_traffic():
    """HBM bytes per decode-kernel launch from the committed pmc summary, or None once the
    kernel source has changed since the counters were taken."""
    import hashlib
    import re
    try:
        md = open(os.path.join(ROOT, "profiles", "decode_kernel_decode_sweep.md")).read()
        src = open(os.path.join(ROOT, "block_scaled_fp4_02_amd", "csrc", "gemm_decode.hip"), "rb").read()
    except OSError:
        return None
    t = re.search(r"^traffic_bytes_per_launch: (\d+)$", md, re.M)
    h = re.search(r"^kernel_source_sha256: ([0-9a-f]{64})$", md, re.M)
    if not t or not h or h.group(1) != hashlib.sha256(src).hexdigest():
        return None
    return int(t.group(1))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def wbytes(N, K):
    return N * K // 2 + N * K // 16


def call_bytes(M, N, K):
    """Algorithmic bytes of one fused call: W once, bf16 X once, FP32 y once."""
    return wbytes(N, K) + 2 * M * K + 4 * M * N


def kernel_bytes(M, N, K):
    """Algorithmic bytes of the GEMM kernel on pre-quantized activations."""
    return wbytes(N, K) + M * K // 2 + M * K // 16 + 4 * M * N


class Ring:
    """Copies of one quantized weight, enough that reuse distance exceeds the MALL."""

    def __init__(self, wq, copies):
        from block_scaled_fp4_02_amd import nvfp4
        self.items = [wq]
        for _ in range(copies - 1):
            self.items.append(wq.clone())
        self.i = 0

    def next(self):
        t = self.items[self.i % len(self.items)]
        self.i += 1
        return t


def graph_time(fn, reps: int, inner: int = 1):
    """Capture fn() (inner calls) in a graph; replay `reps` times; return seconds per inner call."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                       # warm (first-call attributes, workspace growth)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.record()
    for _ in range(reps):
        g.replay()
    en.record()
    torch.cuda.synchronize()
    return st.elapsed_time(en) / 1e3 / reps / inner, g


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip residue/augmented/prefill detail")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--layout", choices=["tiled", "rowmajor"], default="tiled",
                    help="weight storage: tiled (packed once, before timing) or canonical row-major")
    ap.add_argument("--reps", type=int, default=20, help="graph replays per case in the per-case legs")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first copy this many MiB device-to-device (a plain copy of known size, for "
                         "scaling hardware byte counters)")
    ap.add_argument("--roofline-only", action="store_true",
                    help="run only the kernel-alone leg behind the roofline figure (for profiling: then every "
                         "decode-kernel launch of the process belongs to that figure, equally per case)")
    ap.add_argument("--headline-only", action="store_true",
                    help="run only the timed headline steps and print their line (for a kernel trace of the "
                         "fused calls as the headline replays them)")
    ap.add_argument("--prefill-case", default="",
                    help="M,K,N: run only the prefill product on pre-quantized activations, --reps launches "
                         "(for profiling the MFMA kernel; prints one line with its time)")
    ap.add_argument("--mx-prefill-case", default="",
                    help="M,K,N: run only the MXFP4 product on pre-quantized operands, --reps launches "
                         "(for profiling the scaled-FP4 tile kernel; prints one line with its time)")
    ap.add_argument("--quantize-case", default="",
                    help="M,K: run only the activation quantizer on bf16 X [M x K], --reps launches "
                         "(for profiling the quantizer passes; prints one line with its time)")
    ap.add_argument("--attention-case", type=int, default=-1,
                    help="0/1: run only decode attention (32 heads x 4096 tokens x 128) without/with "
                         "compensation on a ring of caches, --reps graph replays (for profiling)")
    ap.add_argument("--augmented-case", type=int, default=-1,
                    help="S: run only the M=64, K=4096, N=14336 augmented call (RMSNorm, channel reorder, "
                         "S residue columns, quantization in the call) on a weight ring, --reps graph replays "
                         "(for profiling the windowed decode kernel; prints one line with its time)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path shards along N with no collective, see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    from block_scaled_fp4_02_amd import nvfp4
    nvfp4.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration_mib > 0:
        src = torch.ones(args.copy_calibration_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.copy_calibration_mib} MiB done")
        del src, dst

    if args.prefill_case:
        prefill_case(nvfp4, dev, args.layout == "tiled", [int(v) for v in args.prefill_case.split(",")], args.reps)
        return
    if args.mx_prefill_case:
        mx_prefill_case(nvfp4, dev, [int(v) for v in args.mx_prefill_case.split(",")], args.reps)
        return
    if args.quantize_case:
        quantize_case(nvfp4, dev, [int(v) for v in args.quantize_case.split(",")], args.reps)
        return
    if args.attention_case >= 0:
        attention_case(nvfp4, dev, bool(args.attention_case), args.reps)
        return
    if args.augmented_case >= 0:
        augmented_case(nvfp4, dev, args.layout == "tiled", args.augmented_case, args.reps)
        return

    # ---------------- inputs, resident in HBM
    shapes = inputs.DECODE_SHAPES
    xs, rings, ys = {}, {}, {}
    # the same ring length for every shape (the smallest weight's count), so every case
    # launches the same number of kernels
    copies = max(max(2, -(-RING_BYTES // wbytes(N, K))) for (K, N) in shapes)
    for si, (K, N) in enumerate(shapes):
        x, w = inputs.decode_sweep(si)
        xs[si] = x.to(dev)
        wq = nvfp4.quantize(w.to(dev))
        if args.layout == "tiled":
            wq = nvfp4.pack_tiled(wq)       # one-time layout change of the static weight
        rings[si] = Ring(wq, copies)
        for M in inputs.DECODE_MS:
            ys[(si, M)] = torch.empty((M, N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step():
        for M in inputs.DECODE_MS:
            for si in range(len(shapes)):
                nvfp4.gemm(xs[si][:M], rings[si].next(), out=ys[(si, M)])

    step_bytes = sum(call_bytes(M, N, K) for M in inputs.DECODE_MS for (K, N) in shapes)

    value = sec_per_step = wall = None
    if not args.roofline_only:
        log("inputs ready; capturing step graphs")
        # One graph per ring phase, each holding exactly one step; step t replays graph t % phases,
        # so every call of consecutive steps reads a different weight copy.
        phases = copies
        graphs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
            torch.cuda.synchronize()
            for _ in range(phases):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    step()
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(s)
        for t in range(args.warmup):
            graphs[t % phases].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record()
        for t in range(args.steps):
            graphs[(args.warmup + t) % phases].replay()
        en.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        sec_per_step = st.elapsed_time(en) / 1e3 / args.steps
        value = step_bytes / sec_per_step / 1e9
        del graphs
        log(f"timed {args.steps} steps: {sec_per_step * 1e6:.1f} us/step, {value:.1f} GB/s")
        if args.headline_only:
            print(json.dumps({"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
                              "steps": args.steps, "warmup": args.warmup,
                              "ms_per_step": round(sec_per_step * 1e3, 5), "mode": "headline-only"}))
            return

    # ---------------- per-case detail: whole call and kernel alone. The kernel-alone leg
    # (pre-quantized activations) launches only the decode kernel, the same number of times
    # for every case, so a profiler's average over that kernel equals per_launch_us.
    detail = {"decode": []}
    kern_bytes_total, kern_time_total = 0.0, 0.0
    for si, (K, N) in enumerate(shapes):
        ring = rings[si]
        n = len(ring.items)
        for M in inputs.DECODE_MS:
            y = ys[(si, M)]
            x = xs[si][:M]
            aq = nvfp4.quantize(x)

            def fused():
                for _ in range(n):
                    nvfp4.gemm(x, ring.next(), out=y)

            def kern():
                for _ in range(n):
                    nvfp4.gemm(aq, ring.next(), out=y)

            tf = None if args.roofline_only else graph_time(fused, reps=args.reps, inner=n)[0]
            tk, _ = graph_time(kern, reps=args.reps, inner=n)
            log(f"case M={M} K={K} N={N}: call " + ("-" if tf is None else f"{tf * 1e6:.2f} us") +
                f", kernel {tk * 1e6:.2f} us")
            kern_bytes_total += kernel_bytes(M, N, K)
            kern_time_total += tk
            row = {"M": M, "K": K, "N": N,
                   "us_kernel": round(tk * 1e6, 3), "GBs_kernel": round(kernel_bytes(M, N, K) / tk / 1e9, 1),
                   "frac_hbm_kernel": round(kernel_bytes(M, N, K) / tk / 1e9 / HBM_PEAK_GBS, 4)}
            if tf is not None:
                row.update({"us_call": round(tf * 1e6, 3), "GBs_call": round(call_bytes(M, N, K) / tf / 1e9, 1)})
            detail["decode"].append(row)
    achieved = kern_bytes_total / kern_time_total / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": profiled_traffic(),
                "kernel": "decode_kernel<1,false,true,false> (M<=16 W4A4 decode product, pre-quantized "
                          "activations, tiled weights)" if args.layout == "tiled" else
                          "decode_kernel<1,false,false> (row-major weights)",
                "per_launch_bytes": round(kern_bytes_total / len(detail["decode"])),
                "per_launch_us": round(kern_time_total / len(detail["decode"]) * 1e6, 3)}

    if not args.no_extra and not args.roofline_only:
        detail.update(extra_detail(nvfp4, dev, args.layout == "tiled"))

    cpu = None if (args.no_cpu_baseline or args.roofline_only) else cpu_baseline(args.cpu_seconds)

    out = {
        "metric": METRIC, "value": None if value is None else round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": None if sec_per_step is None else round(sec_per_step * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded; Llama-like linear-layer shapes)",
        "config": {"workload": "small-M decode GEMM sweep M in {1,2,4,8,16} x (K,N) in "
                               "{(4096,14336),(14336,4096),(4096,6144)}, bf16 activations quantized in the call, "
                               f"{args.layout} NVFP4 weights",
                   "calls_per_step": 15, "bytes_per_step": step_bytes, "parallelism": "single GPU"},
        "roofline": roofline, "cpu_baseline": cpu, "detail": detail,
        "wall_s_timed": None if wall is None else round(wall, 3),
    }
    if args.roofline_only:
        out["mode"] = "roofline-only (kernel-alone leg; value is reported by the default run)"
    print(json.dumps(out))


def extra_detail(nvfp4, dev, tiled):
    """Residue K->2K overhead, M=64 augmented product, prefill TFLOP/s (one number each)."""
    res = {"gemv": [], "residue": [], "augmented": [], "quantizer": [], "prefill": [],
           "prefill_selective_residue": [], "mx_decode": [], "mx_prefill": []}
    prep = nvfp4.pack_tiled if tiled else (lambda t: t)
    # the single GEMV x[1 x 4096] W[4096 x 4096]^T: activation quantized in the call
    x, w = inputs.gemv_4096()
    xd = x.to(dev)
    wq = prep(nvfp4.quantize(w.to(dev)))
    ring = Ring(wq, max(2, -(-RING_BYTES // wbytes(4096, 4096))))
    n = len(ring.items)
    y = torch.empty((1, 4096), dtype=torch.float32, device=dev)
    aq = nvfp4.quantize(xd)

    def gemv_call():
        for _ in range(n):
            nvfp4.gemm(xd, ring.next(), out=y)

    def gemv_kern():
        for _ in range(n):
            nvfp4.gemm(aq, ring.next(), out=y)

    tf, _ = graph_time(gemv_call, 20, n)
    tk, _ = graph_time(gemv_kern, 20, n)
    res["gemv"].append({"M": 1, "K": 4096, "N": 4096, "us_call": round(tf * 1e6, 3),
                        "GBs_call": round(call_bytes(1, 4096, 4096) / tf / 1e9, 1),
                        "frac_hbm_call": round(call_bytes(1, 4096, 4096) / tf / 1e9 / HBM_PEAK_GBS, 4),
                        "us_kernel": round(tk * 1e6, 3),
                        "frac_hbm_kernel": round(kernel_bytes(1, 4096, 4096) / tk / 1e9 / HBM_PEAK_GBS, 4)})
    del ring
    # residue-compensated decode, K = N = 8192
    x, w = inputs.residue_8192(16)
    xd = x.to(dev)
    wq = prep(nvfp4.quantize(w.to(dev)))
    ring = Ring(wq, max(2, -(-RING_BYTES // wbytes(8192, 8192))))
    n = len(ring.items)
    for M in inputs.RESIDUE_MS:
        y = torch.empty((M, 8192), dtype=torch.float32, device=dev)
        xm = xd[:M]

        def base():
            for _ in range(n):
                nvfp4.gemm(xm, ring.next(), out=y)

        def comp():
            for _ in range(n):
                nvfp4.gemm_residue(xm, ring.next(), 8192, out=y)

        tb, _ = graph_time(base, 20, n)
        tc, _ = graph_time(comp, 20, n)
        res["residue"].append({"M": M, "K": 8192, "N": 8192, "us_plain": round(tb * 1e6, 3),
                               "us_residue": round(tc * 1e6, 3), "overhead": round(tc / tb - 1, 4),
                               "GBs_residue": round(call_bytes(M, 8192, 8192) / tc / 1e9, 1),
                               "frac_hbm_residue": round(call_bytes(M, 8192, 8192) / tc / 1e9 / HBM_PEAK_GBS, 4)})
    del ring
    # augmented channels, M = 64, K = 4096, N = 14336
    x, g, xcal, w = inputs.outlier_aug()
    xd, gd = x.to(dev), g.to(dev)
    perm = nvfp4.calibrate_perm(xcal.to(dev), gd)
    wq = prep(nvfp4.quantize(w.to(dev)[:, perm.long()].contiguous()))
    ring = Ring(wq, max(2, -(-RING_BYTES // wbytes(14336, 4096))))
    n = len(ring.items)
    y = torch.empty((64, 14336), dtype=torch.float32, device=dev)
    t0 = None
    for S in [0] + inputs.AUG_S:
        def aug():
            for _ in range(n):
                nvfp4.gemm_residue(xd, ring.next(), S, gamma=gd, eps=1e-6, perm=perm, out=y)
        t, _ = graph_time(aug, 20, n)
        t0 = t if S == 0 else t0
        flops = 2 * 64 * 14336 * (4096 + S)
        res["augmented"].append({"M": 64, "K": 4096, "S": S, "N": 14336, "us_call": round(t * 1e6, 3),
                                 "overhead_vs_S0": round(t / t0 - 1, 4),
                                 "GBs": round(call_bytes(64, 14336, 4096) / t / 1e9, 1),
                                 "frac_hbm": round(call_bytes(64, 14336, 4096) / t / 1e9 / HBM_PEAK_GBS, 4),
                                 "TFLOPs": round(flops / t / 1e12, 2)})
    del ring
    # prefill: bf16 out, activation quantize in the call
    torch.manual_seed(0)
    for si, (K, N) in enumerate(inputs.PREFILL_SHAPES):
        xall = torch.randn((8192, K), device=dev, dtype=torch.float32)
        cols = torch.from_numpy(inputs.outlier_columns(5, si, K, 0.01)).to(dev)
        xall[:, cols] *= 50.0
        xall = xall.to(torch.bfloat16)
        w = (torch.randn((N, K), device=dev, dtype=torch.float32) * 0.015).to(torch.bfloat16)
        wq = prep(nvfp4.quantize(w))          # the static weight in the bench's layout
        del w
        aq_cache = {}
        for M in inputs.PREFILL_MS:
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            xm = xall[:M]
            aq = nvfp4.quantize(xm)
            aq_cache[M] = aq

            def full():
                nvfp4.gemm(xm, wq, out=y)

            def kern():
                nvfp4.gemm(aq, wq, out=y)

            reps = 10 if M < 8192 else 4
            tf, _ = graph_time(full, reps, 1)
            tk, _ = graph_time(kern, reps, 1)
            flops = 2.0 * M * N * K
            res["prefill"].append({"M": M, "K": K, "N": N, "us_call": round(tf * 1e6, 1),
                                   "TFLOPs_call": round(flops / tf / 1e12, 1),
                                   "us_kernel": round(tk * 1e6, 1), "TFLOPs_kernel": round(flops / tk / 1e12, 1),
                                   "frac_f16_mfma_kernel": round(flops / tk / 1e12 / F16_MFMA_PEAK_TFLOPS, 4)})
            # the activation quantizer alone (amax pass + quantize pass): 2.5625 B per element,
            # on a ring of X copies larger than the last-level cache, every copy once per graph
            # replay (one call per replay would time the replay's own launch as well)
            nq = max(2, min(64, -(-RING_BYTES // (2 * M * K))))
            xr = [xm] + [xm.clone() for _ in range(nq - 1)]
            tq, _ = graph_time(lambda: [nvfp4.quantize(v) for v in xr], max(2, reps // 2), nq)
            del xr
            qb = QUANT_BYTES_PER_ELEM * M * K
            res["quantizer"].append({"M": M, "K": K, "us": round(tq * 1e6, 1), "GBs": round(qb / tq / 1e9, 1),
                                     "frac_hbm": round(qb / tq / 1e9 / HBM_PEAK_GBS, 4)})
            if M == 2048:
                # selective residue on the prefill product: top S = 512 columns (activation
                # quantized in the call, residue columns appended)
                S = 512
                ts, _ = graph_time(lambda: nvfp4.gemm_residue(xm, wq, S, out=y), reps, 1)
                fl = 2.0 * M * N * (K + S)
                res["prefill_selective_residue"].append({
                    "M": M, "K": K, "S": S, "N": N, "us_call": round(ts * 1e6, 1),
                    "overhead_vs_plain_call": round(ts / tf - 1, 4), "TFLOPs_call": round(fl / ts / 1e12, 1),
                    "frac_f16_mfma_call": round(fl / ts / 1e12 / F16_MFMA_PEAK_TFLOPS, 4)})
        del xall, wq, aq_cache
        torch.cuda.empty_cache()
    res.update(mx_detail(nvfp4, dev))
    res.update(attention_detail(nvfp4, dev))
    return res


def attention_bytes(H, T, D):
    """Algorithmic bytes of one decode-attention call: both caches once (codes and
    E4M3 scales), the bf16 query and the FP32 output."""
    return 2 * (H * T * D // 2 + H * T * D // 16) + 2 * H * D + 4 * H * D


def attention_ring(nvfp4, dev, H, T, D):
    q, k, vt = inputs.attention(H, T, D)
    kq, vq = nvfp4.quantize(k.to(dev)), nvfp4.quantize(vt.to(dev))
    copies = max(2, -(-RING_BYTES // attention_bytes(H, T, D)))
    return q.to(dev), [(kq, vq)] + [(kq.clone(), vq.clone()) for _ in range(copies - 1)]


def attention_detail(nvfp4, dev):
    """Decode attention over the NVFP4 KV cache (32 heads x 4096 tokens x 128), plain and
    with residue compensation, on a ring of cache copies (kernels alone, HIP graph)."""
    H, T, D = inputs.ATTN_SHAPE
    qd, ring = attention_ring(nvfp4, dev, H, T, D)
    out = torch.empty((H, D), dtype=torch.float32, device=dev)
    rows, t_plain = [], None
    for comp in (False, True):
        def run():
            for kq, vq in ring:
                nvfp4.decode_attention(qd, kq, vq, T, compensate=comp, out=out)

        t, _ = graph_time(run, 20, len(ring))
        t_plain = t if not comp else t_plain
        b = attention_bytes(H, T, D)
        rows.append({"H": H, "T": T, "D": D, "compensate": comp, "us_call": round(t * 1e6, 3),
                     "GBs": round(b / t / 1e9, 1), "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 4),
                     "overhead_vs_plain": round(t / t_plain - 1, 4)})
    del ring
    return {"decode_attention": rows}


def mx_detail(nvfp4, dev):
    """MXFP4 on the scaled FP4 matrix cores: decode sweep (kernel alone, weight ring) and
    prefill (kernel alone), against 8 TB/s and the 10.1 PFLOP/s dense FP4 peak."""
    out = {"mx_decode": [], "mx_prefill": []}
    for si, (K, N) in enumerate(inputs.DECODE_SHAPES):
        x, w = inputs.decode_sweep(si)
        wq = nvfp4.mx_pack_tiled(nvfp4.mx_quantize(w.to(dev)))   # the decode product's tiled weights
        wb = N * K // 2 + N * K // 32
        copies = max(2, -(-RING_BYTES // wb))
        ring = [wq] + [nvfp4.MXTensor(wq.codes.clone(), wq.scales.clone(), K, wq.layout, wq.rows)
                       for _ in range(copies - 1)]
        for M in inputs.DECODE_MS:
            aq = nvfp4.mx_quantize(x[:M].to(dev))
            y = torch.empty((M, N), dtype=torch.float32, device=dev)

            def kern():
                for r in ring:
                    nvfp4.mx_gemm(aq, r, out=y)

            t, _ = graph_time(kern, 20, len(ring))
            b = wb + M * K // 2 + M * K // 32 + 4 * M * N
            out["mx_decode"].append({"M": M, "K": K, "N": N, "us_kernel": round(t * 1e6, 3),
                                     "GBs_kernel": round(b / t / 1e9, 1),
                                     "frac_hbm_kernel": round(b / t / 1e9 / HBM_PEAK_GBS, 4)})
        del ring, wq
    torch.manual_seed(0)
    for (K, N) in inputs.PREFILL_SHAPES:
        w = (torch.randn((N, K), device=dev, dtype=torch.float32) * 0.015).to(torch.bfloat16)
        wq = nvfp4.mx_quantize(w)
        del w
        for M in inputs.PREFILL_MS:
            x = torch.randn((M, K), device=dev, dtype=torch.float32).to(torch.bfloat16)
            aq = nvfp4.mx_quantize(x)
            del x
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            t, _ = graph_time(lambda: nvfp4.mx_gemm(aq, wq, out=y), 10 if M < 8192 else 4, 1)
            fl = 2.0 * M * N * K
            out["mx_prefill"].append({"M": M, "K": K, "N": N, "us_kernel": round(t * 1e6, 1),
                                      "TFLOPs_kernel": round(fl / t / 1e12, 1),
                                      "frac_fp4_mfma_kernel": round(fl / t / 1e12 / FP4_MFMA_PEAK_TFLOPS, 4)})
            del aq, y
        del wq
        torch.cuda.empty_cache()
    return out


def prefill_case(nvfp4, dev, tiled, mkn, reps):
    """One prefill shape, kernel-alone (activations quantized before), `reps` launches."""
    M, K, N = mkn
    torch.manual_seed(0)
    x = torch.randn((M, K), device=dev, dtype=torch.float32).to(torch.bfloat16)
    w = (torch.randn((N, K), device=dev, dtype=torch.float32) * 0.015).to(torch.bfloat16)
    wq = nvfp4.quantize(w)
    if tiled:
        wq = nvfp4.pack_tiled(wq)
    del w
    aq = nvfp4.quantize(x)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    nvfp4.gemm(aq, wq, out=y)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        nvfp4.gemm(aq, wq, out=y)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / max(reps, 1)
    flops = 2.0 * M * N * K
    print(json.dumps({"prefill_case": [M, K, N], "reps": reps, "us_per_call": round(us, 1),
                      "TFLOPs": round(flops / us / 1e6, 1),
                      "frac_f16_mfma": round(flops / us / 1e6 / F16_MFMA_PEAK_TFLOPS, 4)}), flush=True)


def timed_launches(fn, reps):
    """fn() once untimed, then `reps` launches between HIP events; seconds per launch."""
    fn()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / 1e3 / max(reps, 1)


def mx_prefill_case(nvfp4, dev, mkn, reps):
    """One MXFP4 product shape, kernel alone (both operands quantized before), `reps` launches."""
    M, K, N = mkn
    torch.manual_seed(0)
    x = torch.randn((M, K), device=dev, dtype=torch.float32).to(torch.bfloat16)
    w = (torch.randn((N, K), device=dev, dtype=torch.float32) * 0.015).to(torch.bfloat16)
    aq, wq = nvfp4.mx_quantize(x), nvfp4.mx_quantize(w)
    del x, w
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    t = timed_launches(lambda: nvfp4.mx_gemm(aq, wq, out=y), reps)
    fl = 2.0 * M * N * K
    print(json.dumps({"mx_prefill_case": [M, K, N], "reps": reps, "us_per_call": round(t * 1e6, 1),
                      "TFLOPs": round(fl / t / 1e12, 1),
                      "frac_fp4_mfma": round(fl / t / 1e12 / FP4_MFMA_PEAK_TFLOPS, 4)}), flush=True)


def quantize_case(nvfp4, dev, mk, reps):
    """The activation quantizer alone on bf16 X [M x K] (amax pass + quantize pass), `reps` launches."""
    M, K = mk
    torch.manual_seed(0)
    x = torch.randn((M, K), device=dev, dtype=torch.float32).to(torch.bfloat16)
    t = timed_launches(lambda: nvfp4.quantize(x), reps)
    b = QUANT_BYTES_PER_ELEM * M * K
    print(json.dumps({"quantize_case": [M, K], "reps": reps, "us_per_call": round(t * 1e6, 1),
                      "GBs": round(b / t / 1e9, 1), "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 4)}),
          flush=True)


def attention_case(nvfp4, dev, comp, reps):
    """Decode attention alone on a ring of cache copies, `reps` graph replays."""
    H, T, D = inputs.ATTN_SHAPE
    qd, ring = attention_ring(nvfp4, dev, H, T, D)
    out = torch.empty((H, D), dtype=torch.float32, device=dev)

    def run():
        for kq, vq in ring:
            nvfp4.decode_attention(qd, kq, vq, T, compensate=comp, out=out)

    t, _ = graph_time(run, reps, len(ring))
    b = attention_bytes(H, T, D)
    print(json.dumps({"attention_case": [H, T, D], "compensate": comp, "reps": reps, "calls_per_replay": len(ring),
                      "us_per_call": round(t * 1e6, 2), "GBs": round(b / t / 1e9, 1),
                      "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 4)}), flush=True)


def augmented_case(nvfp4, dev, tiled, S, reps):
    """The M = 64 augmented-channel call alone (the extra-detail leg's inputs), `reps` graph replays."""
    prep = nvfp4.pack_tiled if tiled else (lambda t: t)
    x, g, xcal, w = inputs.outlier_aug()
    xd, gd = x.to(dev), g.to(dev)
    perm = nvfp4.calibrate_perm(xcal.to(dev), gd)
    wq = prep(nvfp4.quantize(w.to(dev)[:, perm.long()].contiguous()))
    ring = Ring(wq, max(2, -(-RING_BYTES // wbytes(14336, 4096))))
    n = len(ring.items)
    y = torch.empty((64, 14336), dtype=torch.float32, device=dev)

    def aug():
        for _ in range(n):
            nvfp4.gemm_residue(xd, ring.next(), S, gamma=gd, eps=1e-6, perm=perm, out=y)
    t, _ = graph_time(aug, reps, n)
    print(json.dumps({"augmented_case": [64, 4096, S, 14336], "reps": reps, "calls_per_replay": n,
                      "us_per_call": round(t * 1e6, 2)}), flush=True)


def cpu_baseline(budget_s: float):
    """The CPU oracle (unchanged) on a bounded sample of the decode sweep: for each case in
    sweep order, quantize X and run the FP64 GEMM against the oracle-quantized weight, until
    the time budget is spent. Value = algorithmic bytes of the cases done / their time."""
    import oracle
    oracle.lib()
    done, t_total, b_total = [], 0.0, 0
    for si, (K, N) in enumerate(inputs.DECODE_SHAPES):
        x, w = inputs.decode_sweep(si)
        ow = oracle.quantize(w)
        for M in inputs.DECODE_MS:
            t0 = time.perf_counter()
            oracle.gemm(oracle.quantize(x[:M]), ow)
            dt = time.perf_counter() - t0
            t_total += dt
            b_total += call_bytes(M, N, K)
            done.append(f"M={M},K={K},N={N}")
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    return {"value": round(b_total / t_total / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(done)} of 15 sweep calls ({', '.join(done)}), {t_total:.1f} s, single thread",
            "us_call_mean": round(t_total / len(done) * 1e6, 1)}


if __name__ == "__main__":
    main()
