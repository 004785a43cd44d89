"""Benchmark of the tiled dense GEMM on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Headline workload: f16 GEMM M=N=K=4096 with the fused epilogue
C = GELU_tanh(A.B + bias) (A, B = U[-1,1]/8, bias = U[-0.5,0.5], FP32
accumulation and epilogue, f16 output), one tg_gemm_bias_act launch per step,
inputs resident in HBM.  The timing protocol follows the pages (1000 warm-up
and 3000 timed launches, mean time per launch), bracketed by HIP events on
the launch stream.

Prints ONE JSON line with the metric, the roofline of the kernel (achieved
algorithmic TFLOP/s over the MI355X dense f16 MFMA peak), the CPU oracle
timed on a bounded sample of the same workload on the host cores, and the
secondary workloads (QKV, 8192^3 bf16, the M=16 bandwidth-bound product with
its GB/s against the HBM peak, and the small square shapes).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2516.6   # MI355X dense f16/bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_FP8_TFLOPS = 5033.2   # MI355X dense fp8 MFMA (twice the f16 rate)
METRIC = "GEMM TFLOP/s + % of MFMA peak (4096³ fp16); GB/s % HBM peak at M=16"
KERNEL_SOURCES = ["tiled_dense_gemm_09_amd/csrc/gemm_async.hip",
                  "tiled_dense_gemm_09_amd/csrc/tg_pipeline.h",
                  "tiled_dense_gemm_09_amd/csrc/tg_device.h",
                  "tiled_dense_gemm_09_amd/csrc/tg_launch.h",
                  "tiled_dense_gemm_09_amd/csrc/tg_api.cpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_tokens(text):
    """C++ source with comments removed and runs of whitespace collapsed
    (string and character literals kept whole), so that the hash below
    follows the code and not its comments."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash():
    """Hash of the kernel sources' code (comments and layout ignored): the
    HBM traffic record is reported only while it matches."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(code_tokens(fh.read()).encode())
    return h.hexdigest()[:16]


def time_launches(fn, steps, warmup, batches=1, per_batch=None):
    """Mean ms per launch over `steps` launches after `warmup` untimed ones.
    With batches > 1 the timed loop also carries events at `batches` evenly
    spaced boundaries, and the median of the per-batch means is returned
    beside the mean (the per-batch means, in launch order, are appended to
    the list per_batch when one is given)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    bounds = sorted(set(round(i * steps / batches) for i in range(batches + 1)))
    events = [torch.cuda.Event(enable_timing=True) for _ in bounds]
    events[0].record()
    done = 0
    for b, stop in zip(events[1:], bounds[1:]):
        while done < stop:
            fn()
            done += 1
        b.record()
    torch.cuda.synchronize()
    mean = events[0].elapsed_time(events[-1]) / steps
    if batches == 1:
        return mean
    in_order = [events[i].elapsed_time(events[i + 1]) / (bounds[i + 1] - bounds[i])
                for i in range(len(bounds) - 1)]
    if per_batch is not None:
        per_batch.extend(in_order)
    per = sorted(in_order)
    mid = len(per) // 2
    median = per[mid] if len(per) % 2 else 0.5 * (per[mid - 1] + per[mid])
    return mean, median


def dev(bits, dt):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dt == 1 else torch.bfloat16).cuda()


def traffic_record(workload):
    """HBM bytes per launch measured with rocprofv3 counters, if still valid."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload)
    except ValueError:
        return None
    if not rec or rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(p, target_s):
    """The oracle, as it stands, on a bounded row sample of the workload."""
    import oracle
    threads = oracle.max_threads()
    # grow the sample until one call takes >= 1 s, then size it for target_s
    rows, secs = 16, 0.0
    while True:
        t0 = time.perf_counter()
        oracle.gemm(p["dt"], p["A"], p["B"], p["bias"], p["act"], rows=(0, rows))
        secs = time.perf_counter() - t0
        if secs >= 1.0 or rows >= p["M"]:
            break
        rows = min(p["M"], rows * 4)
    if secs < target_s and rows < p["M"]:
        rows = int(min(p["M"], rows * target_s / secs))
        t0 = time.perf_counter()
        oracle.gemm(p["dt"], p["A"], p["B"], p["bias"], p["act"], rows=(0, rows))
        secs = time.perf_counter() - t0
    flops = 2.0 * rows * p["N"] * p["K"]
    rec = {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": "rows 0..%d of the %dx%dx%d workload, all %d columns (%.1f s, double "
                     "precision)" % (rows - 1, p["M"], p["N"], p["K"], p["N"], secs),
           "cpu_model": cpu_model()}
    # the two small square shapes in full, one thread (their GPU rates are
    # graph-replay launches of the same shapes)
    from tiled_dense_gemm_09_amd import inputs
    single = {}
    for name in ("f16_256", "f16_1024"):
        q = inputs.config_problem(name)
        t0 = time.perf_counter()
        oracle.gemm(q["dt"], q["A"], q["B"], threads=1)
        dt_s = time.perf_counter() - t0
        single[name] = {"s": round(dt_s, 4),
                        "GFLOP/s": round(2.0 * q["M"] * q["N"] * q["K"] / dt_s / 1e9, 3)}
    rec["single_thread_full"] = single
    return rec


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo (Linux)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--only", choices=["main", "plain", "ex", "mx", "attn", "qkv", "square8192",
                                       "skinny", "offgrid", "small", "vendor", "copy", "sweep",
                                       "streamk"],
                    help="run one workload only (for profiling); no JSON line")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-extra", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from tiled_dense_gemm_09_amd import inputs, tg
    assert torch.cuda.is_available(), "no GPU visible"

    if args.only == "sweep":
        run_sweep(torch, tg)
        return
    if args.only == "streamk":
        run_stream_k_sweep(torch, tg)
        return

    if args.only == "copy":
        # plain copy of a known size, for scaling the HBM byte counters
        n = 256 << 20
        x = torch.empty(n, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(args.steps):
            y.copy_(x)
        torch.cuda.synchronize()
        return

    # ---------------------------------------------------------------- main
    p = inputs.config_problem("f16_4096_gelu")
    M, N, K = p["M"], p["N"], p["K"]
    A, B, bias = dev(p["A"], 1), dev(p["B"], 1), dev(p["bias"], 1)
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")

    def step():
        tg.gemm(A, B, out=C, bias=bias, act="gelu_tanh")

    if args.only in (None, "main"):
        log("main: f16 %dx%dx%d bias+gelu, warmup %d, steps %d" % (M, N, K, args.warmup,
                                                                    args.steps))
        batch_ms = []
        ms, ms_median = time_launches(step, args.steps, args.warmup, batches=10,
                                      per_batch=batch_ms)
        kernel = tg.last_kernel()
        tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        log("  %s: %.4f ms/launch, %.1f TFLOP/s" % (kernel, ms, tflops))
        log("  batch means (ms, launch order): %s" % " ".join("%.4f" % b for b in batch_ms))
        if args.only == "main":
            return
        # The same launches under the pages' protocol (1000 warm-up, 3000
        # timed), after the measurement above: a short run starts at the idle
        # clock and then sees the board cut the clock within a few ms of full
        # load, a long one settles at the sustained clock.
        ms_sus = time_launches(step, 3000, 1000)
        sustained = {"warmup": 1000, "steps": 3000, "ms": round(ms_sus, 6),
                     "TFLOP/s": round(2.0 * M * N * K / (ms_sus * 1e-3) / 1e12, 1),
                     "frac_mfma_peak": round(2.0 * M * N * K / (ms_sus * 1e-3) / 1e12 /
                                             PEAK_F16_TFLOPS, 4)}
        log("  sustained (1000 + 3000 launches): %.4f ms/launch" % ms_sus)

    extra = {}
    if not args.no_extra or args.only:
        extra = run_secondary(args, torch, inputs, tg)
        if args.only:
            return

    # quick parity of the timed output on sampled elements
    import oracle
    cb = C.view(torch.int16).cpu().numpy().view(np.uint16)
    rng = np.random.default_rng(0)
    ii, jj = rng.integers(0, M, 512), rng.integers(0, N, 512)
    f64, _ = oracle.gemm_sample(1, p["A"], p["B"], ii, jj, p["bias"], oracle.ACT_GELU_TANH)
    got = cb[ii, jj].view(np.float16).astype(np.float64)
    err = np.abs(got - f64)
    parity = {"sampled": int(ii.size), "max_abs_err": float(err.max()),
              "pass": bool(np.all(err <= 1e-2 + 5e-3 * np.abs(f64)))}

    log("cpu baseline: oracle on a row sample (~%.0f s)" % args.cpu_seconds)
    cpu = cpu_baseline(p, args.cpu_seconds)

    traffic = traffic_record("f16_4096_gelu")
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "ms_per_step_median_of_10_batches": round(ms_median, 6),
        "ms_per_batch_in_order": [round(b, 5) for b in batch_ms],
        "sustained_pages_protocol": sustained,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "f16 GEMM M=N=K=4096, C = GELU_tanh(A.B + bias), FP32 accumulate",
                   "M": M, "N": N, "K": K, "kernel": kernel},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_F16_TFLOPS, 4),
                     "traffic": (traffic["fetch"] + traffic["write"]) if traffic else None,
                     "traffic_split": traffic},
        "cpu_baseline": cpu,
        "parity": parity,
        "secondary": extra,
    }
    print(json.dumps(line), flush=True)


def run_secondary(args, torch, inputs, tg):
    out = {}
    steps = max(10, min(args.steps, 300))
    warm = max(3, min(args.warmup, 50))

    if args.only in (None, "plain"):
        # the headline product without its epilogue, so the epilogue's cost shows
        p = inputs.config_problem("f16_4096_gelu")
        A, B = dev(p["A"], 1), dev(p["B"], 1)
        C = torch.empty((p["M"], p["N"]), dtype=torch.float16, device="cuda")
        ms = time_launches(lambda: tg.gemm(A, B, out=C), steps, warm)
        tf = 2.0 * p["M"] * p["N"] * p["K"] / (ms * 1e-3) / 1e12
        out["f16_4096x4096x4096_no_epilogue"] = {
            "ms": round(ms, 5), "TFLOP/s": round(tf, 1),
            "frac_mfma_peak": round(tf / PEAK_F16_TFLOPS, 4), "kernel": tg.last_kernel()}
        log("  ", out["f16_4096x4096x4096_no_epilogue"])
        del A, B, C

    if args.only in (None, "ex"):
        # the headline product with the weight stored [N,K] and a residual
        # added after the activation (tg_gemm_ex, one launch)
        p = inputs.config_problem("f16_4096_gelu")
        A, bias = dev(p["A"], 1), dev(p["bias"], 1)
        Wt = dev(np.ascontiguousarray(p["B"].T), 1)
        R = dev(inputs.draw(np.random.default_rng(99), (p["M"], p["N"]), "uniform", 1), 1)
        C = torch.empty((p["M"], p["N"]), dtype=torch.float16, device="cuda")
        for label, b, res in (("f16_4096_gelu_B_stored_NK", Wt.t(), None),
                              ("f16_4096_gelu_B_stored_NK_residual", Wt.t(), R),
                              ("f16_4096_gelu_residual", dev(p["B"], 1), R)):
            ms = time_launches(lambda: tg.gemm(A, b, out=C, bias=bias, act="gelu_tanh",
                                               residual=res), steps, warm)
            tf = 2.0 * p["M"] * p["N"] * p["K"] / (ms * 1e-3) / 1e12
            out[label] = {"ms": round(ms, 5), "TFLOP/s": round(tf, 1),
                          "frac_mfma_peak": round(tf / PEAK_F16_TFLOPS, 4),
                          "kernel": tg.last_kernel()}
            log("  ", label, out[label])
        del A, bias, Wt, R, C

    if args.only in (None, "mx"):
        # block-scaled 8-bit GEMM (e4m3 operands, e8m0 scales per 32 k, bf16 out)
        for n in (4096, 8192):
            p = inputs.mx_problem(inputs.FP8_E4M3, inputs.FP8_E4M3, n, n, n, seed=160 + n % 7)
            d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
            A, SA, B, SB = d(p["A"]), d(p["SA"]), d(p["B"]), d(p["SB"])
            C = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
            ms = time_launches(lambda: tg.gemm_mx(A, SA, B, SB, out=C), steps, warm)
            tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
            out["mx_e4m3_%dx%dx%d" % (n, n, n)] = {
                "ms": round(ms, 5), "TFLOP/s": round(tf, 1),
                "frac_fp8_mfma_peak": round(tf / PEAK_FP8_TFLOPS, 4), "kernel": tg.last_kernel()}
            log("  ", out["mx_e4m3_%dx%dx%d" % (n, n, n)])
            # context only: the ROCm library's 8-bit GEMMs (torch._scaled_mm) on
            # the same operands, with one scale per tensor (no block scaling)
            # and with the same e8m0 scales per 32 k
            ctx8 = out.setdefault("context_rocm_blas_fp8_scaled_mm", {})
            a8, b8 = A.view(torch.float8_e4m3fn), B.view(torch.float8_e4m3fn)
            one = torch.tensor(1.0, device="cuda")
            sa = SA.t().contiguous().view(torch.float8_e8m0fnu)
            sb = SB.t().contiguous().view(torch.float8_e8m0fnu)
            for key, (xa, xb) in (("e4m3_per_tensor_%d" % n, (one, one)),
                                  ("mx_e4m3_1x32_%d" % n, (sa, sb))):
                try:
                    ms = time_launches(lambda: torch._scaled_mm(
                        a8, b8.t(), scale_a=xa, scale_b=xb, out_dtype=torch.bfloat16), steps, warm)
                    ctx8[key] = {"ms": round(ms, 5),
                                 "TFLOP/s": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)}
                except Exception as e:  # not every build has both paths
                    ctx8[key] = {"error": str(e)[:120]}
            log("  ", ctx8)
            del A, SA, B, SB, C, a8, b8, sa, sb

    if args.only in (None, "attn"):
        # fused forward attention, head dim 128, 16384 tokens per launch;
        # flop = 4 B H S^2 D (non-causal), half of it causal
        for (b, hds, seq) in ((4, 16, 4096), (2, 16, 8192)):
            p = inputs.attention_problem(inputs.BF16, b, hds, seq, 128, seed=200 + seq % 9)
            q, k, v = (dev(p[n], 2) for n in ("Q", "K", "V"))
            o = torch.empty_like(q)
            for causal in (False, True):
                ms = time_launches(lambda: tg.attention(q, k, v, causal=causal, out=o), steps,
                                   warm)
                flop = 4.0 * b * hds * seq * seq * 128 * (0.5 if causal else 1.0)
                tf = flop / (ms * 1e-3) / 1e12
                key = "attn_bf16_%dx%dx%dx128%s" % (b, hds, seq, "_causal" if causal else "")
                out[key] = {"ms": round(ms, 5), "TFLOP/s": round(tf, 1),
                            "frac_mfma_peak": round(tf / PEAK_F16_TFLOPS, 4),
                            "kernel": tg.last_kernel()}
                log("  ", key, out[key])
            del q, k, v, o

    if args.only in (None, "qkv"):
        q = inputs.config_problem("bf16_qkv")
        X = dev(q["X"], 2)
        Ws = [dev(w, 2) for w in q["W"]]
        outs = [torch.empty((q["M"], q["N"]), dtype=torch.bfloat16, device="cuda")
                for _ in range(3)]
        log("qkv: bf16 X[%d,%d] x 3 W[%d,%d]" % (q["M"], q["K"], q["K"], q["N"]))
        ms = time_launches(lambda: tg.gemm_qkv(X, *Ws, outs=outs), steps, warm)
        tf = 3 * 2.0 * q["M"] * q["N"] * q["K"] / (ms * 1e-3) / 1e12
        out["bf16_qkv_8192x4096x4096x3"] = {"ms": round(ms, 5), "TFLOP/s": round(tf, 1),
                                            "frac_mfma_peak": round(tf / PEAK_F16_TFLOPS, 4),
                                            "kernel": tg.last_kernel()}
        log("  ", out["bf16_qkv_8192x4096x4096x3"])
        # context only: the library GEMM called three times on the same operands
        def three():
            for w, o in zip(Ws, outs):
                torch.matmul(X, w, out=o)
        ms = time_launches(three, steps, warm)
        out.setdefault("context_rocm_blas_torch_matmul", {})["bf16_qkv_three_matmuls"] = {
            "ms": round(ms, 5), "TFLOP/s": round(3 * 2.0 * q["M"] * q["N"] * q["K"] /
                                                 (ms * 1e-3) / 1e12, 1)}
        del X, Ws, outs

    if args.only in (None, "square8192"):
        p = inputs.config_problem("bf16_8192")
        A, B = dev(p["A"], 2), dev(p["B"], 2)
        C = torch.empty((p["M"], p["N"]), dtype=torch.bfloat16, device="cuda")
        log("square: bf16 8192^3")
        ms = time_launches(lambda: tg.gemm(A, B, out=C), steps, warm)
        tf = 2.0 * p["M"] * p["N"] * p["K"] / (ms * 1e-3) / 1e12
        out["bf16_8192x8192x8192"] = {"ms": round(ms, 5), "TFLOP/s": round(tf, 1),
                                      "frac_mfma_peak": round(tf / PEAK_F16_TFLOPS, 4),
                                      "kernel": tg.last_kernel()}
        log("  ", out["bf16_8192x8192x8192"])
        del A, B, C

    if args.only in (None, "skinny"):
        p = inputs.config_problem("bf16_skinny")
        X = dev(p["A"], 2)
        # four distinct copies of W (4 x 128 MiB > the 256 MB last-level cache),
        # used in rotation so every launch streams W from HBM
        Ws = [dev(p["B"], 2)]
        for _ in range(3):
            Ws.append(Ws[0].clone())
        Y = torch.empty((p["M"], p["N"]), dtype=torch.bfloat16, device="cuda")
        it = [0]

        def sk():
            tg.gemm(X, Ws[it[0] & 3], out=Y)
            it[0] += 1

        log("skinny: bf16 M=16 N=K=8192, W rotated over 4 buffers")
        ms = time_launches(sk, steps, warm)
        nbytes = 2 * (p["N"] * p["K"] + p["M"] * p["K"] + p["M"] * p["N"])
        gbs = nbytes / (ms * 1e-3) / 1e9
        ms_hot = time_launches(lambda: tg.gemm(X, Ws[0], out=Y), steps, warm)
        out["bf16_skinny_16x8192x8192"] = {
            "ms": round(ms, 5), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": nbytes,
            "cache_resident_ms": round(ms_hot, 5),
            "cache_resident_GB/s": round(nbytes / (ms_hot * 1e-3) / 1e9, 1),
            "kernel": tg.last_kernel()}
        log("  ", out["bf16_skinny_16x8192x8192"])
        # the same path at its upper row count (M = 32: two 16-row blocks per
        # W fragment), same rotated W, X ~ N(0, 1)
        X32 = dev(inputs.draw(np.random.default_rng(55), (32, p["K"]), "normal", 2), 2)
        Y32 = torch.empty((32, p["N"]), dtype=torch.bfloat16, device="cuda")

        def sk32():
            tg.gemm(X32, Ws[it[0] & 3], out=Y32)
            it[0] += 1

        ms = time_launches(sk32, steps, warm)
        nbytes = 2 * (p["N"] * p["K"] + 32 * p["K"] + 32 * p["N"])
        gbs = nbytes / (ms * 1e-3) / 1e9
        out["bf16_skinny_32x8192x8192"] = {
            "ms": round(ms, 5), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "TFLOP/s": round(2.0 * 32 * p["N"] * p["K"] / (ms * 1e-3) / 1e12, 1),
            "algorithmic_bytes": nbytes, "kernel": tg.last_kernel()}
        log("  ", out["bf16_skinny_32x8192x8192"])
        # the same product with W stored [N,K] (a linear layer's weight
        # layout), rotated over four copies, and the library beside it on the
        # same operands
        Wts = [w.t().contiguous().t() for w in Ws]

        def sknk():
            tg.gemm(X, Wts[it[0] & 3], out=Y)
            it[0] += 1

        def sknk_lib():
            torch.matmul(X, Wts[it[0] & 3], out=Y)
            it[0] += 1

        log("skinny: bf16 M=16 N=K=8192, W stored [N,K], rotated over 4 buffers")
        ms = time_launches(sknk, steps, warm)
        kern = tg.last_kernel()
        ml = time_launches(sknk_lib, steps, warm)
        nbytes = 2 * (p["N"] * p["K"] + p["M"] * p["K"] + p["M"] * p["N"])
        out["bf16_skinny_16x8192x8192_w_nk"] = {
            "ms": round(ms, 5), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": nbytes, "kernel": kern,
            "library_GB/s": round(nbytes / (ml * 1e-3) / 1e9, 1)}
        log("  ", out["bf16_skinny_16x8192x8192_w_nk"])
        del X, Ws, Wts, Y, X32, Y32
        # a decode step against an odd-sized vocabulary: W [4096, 50257]
        # (412 MB, larger than the last-level cache), row pitch off the
        # 16-byte grid, X ~ N(0,1), W ~ N(0,1/K)
        torch.manual_seed(4)
        M, N, K = 1, 50257, 4096
        X = torch.randn(M, K, dtype=torch.bfloat16, device="cuda")
        W = torch.randn(K, N, dtype=torch.bfloat16, device="cuda") * K ** -0.5
        Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        log("skinny: bf16 1x50257x4096, W pitch 50257")
        ms = time_launches(lambda: tg.gemm(X, W, out=Y), steps, warm)
        kern = tg.last_kernel()
        ml = time_launches(lambda: torch.matmul(X, W, out=Y), steps, warm)
        nbytes = 2 * (N * K + M * K + M * N)
        out["bf16_skinny_1x50257x4096_odd_pitch"] = {
            "ms": round(ms, 5), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": nbytes, "kernel": kern,
            "library_GB/s": round(nbytes / (ml * 1e-3) / 1e9, 1)}
        log("  ", out["bf16_skinny_1x50257x4096_odd_pitch"])
        del X, W, Y

    if args.only in (None, "offgrid"):
        # shapes off the configured tile grid, bf16, X ~ N(0,1), W ~ N(0,1/K):
        # a grid short of one wave of 256 x 256 tiles (192 x 192 tiles), a
        # ragged token count, and pitches off the 8-element grid (staged
        # copies); the ROCm library GEMM on the same operands beside each
        torch.manual_seed(3)
        for (M, N, K) in ((3072, 3072, 3072), (2049, 4096, 4096), (4095, 4095, 4095)):
            X = torch.randn(M, K, dtype=torch.bfloat16, device="cuda")
            W = torch.randn(K, N, dtype=torch.bfloat16, device="cuda") * K ** -0.5
            Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            f = 2.0 * M * N * K
            log("off-grid: bf16 %dx%dx%d" % (M, N, K))
            ms = time_launches(lambda: tg.gemm(X, W, out=Y), steps, warm)
            kern = tg.last_kernel()
            ml = time_launches(lambda: torch.matmul(X, W, out=Y), steps, warm)
            key = "bf16_%dx%dx%d" % (M, N, K)
            out[key] = {"ms": round(ms, 5), "TFLOP/s": round(f / (ms * 1e-3) / 1e12, 1),
                        "frac_mfma_peak": round(f / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
                        "kernel": kern, "library_TFLOP/s": round(f / (ml * 1e-3) / 1e12, 1)}
            log("  ", out[key])
            del X, W, Y

    if args.only in (None, "vendor"):
        # context only: the ROCm BLAS library GEMM (torch.matmul) on the same
        # operands, no epilogue; nothing of the measured path runs through it
        ctx = out.setdefault("context_rocm_blas_torch_matmul", {})
        for name, dtc in (("f16_4096_gelu", 1), ("bf16_8192", 2)):
            p = inputs.config_problem(name)
            A, B = dev(p["A"], dtc), dev(p["B"], dtc)
            C = torch.empty((p["M"], p["N"]), dtype=A.dtype, device="cuda")
            ms = time_launches(lambda: torch.matmul(A, B, out=C), steps, warm)
            tf = 2.0 * p["M"] * p["N"] * p["K"] / (ms * 1e-3) / 1e12
            ctx["%s_%dx%dx%d" % ("f16" if dtc == 1 else "bf16", p["M"], p["N"], p["K"])] = {
                "ms": round(ms, 5), "TFLOP/s": round(tf, 1)}
            del A, B, C
        # the same workload done the unfused way: the library GEMM with its
        # bias epilogue (torch.addmm), then GELU_tanh as a second pass
        p = inputs.config_problem("f16_4096_gelu")
        A, B, bias = dev(p["A"], 1), dev(p["B"], 1), dev(p["bias"], 1)
        C = torch.empty((p["M"], p["N"]), dtype=A.dtype, device="cuda")
        fn = torch.nn.functional.gelu
        ms = time_launches(lambda: fn(torch.addmm(bias, A, B, out=C), approximate="tanh"),
                           steps, warm)
        ctx["f16_4096_gelu_unfused_addmm_then_gelu"] = {
            "ms": round(ms, 5), "TFLOP/s": round(2.0 * 4096 ** 3 / (ms * 1e-3) / 1e12, 1)}
        del A, B, bias, C
        out["context_rocm_blas_torch_matmul"] = ctx
        log("  ", ctx)

    if args.only in (None, "small"):
        # A launch of these shapes takes less GPU time than the Python wrapper
        # takes to issue it, so back-to-back eager calls measure the host.  The
        # device rate comes from replaying a captured HIP graph of 100 launches
        # (checked bit for bit against the eager result); the eager rate is
        # kept beside it.
        for name in ("f16_256", "f16_1024"):
            p = inputs.config_problem(name)
            A, B = dev(p["A"], 1), dev(p["B"], 1)
            C = torch.empty((p["M"], p["N"]), dtype=torch.float16, device="cuda")
            flop = 2.0 * p["M"] * p["N"] * p["K"]
            ms_eager = time_launches(lambda: tg.gemm(A, B, out=C), steps, warm)
            kern = tg.last_kernel()
            ref = C.clone()
            ms_graph, same = graph_launch_ms(lambda: tg.gemm(A, B, out=C), C, ref,
                                             max(steps // 100, 5))
            tf = flop / (ms_graph * 1e-3) / 1e12
            key = "f16_%dx%dx%d" % (p["M"], p["N"], p["K"])
            out[key] = {"ms": round(ms_graph, 5), "TFLOP/s": round(tf, 2),
                        "frac_mfma_peak": round(tf / PEAK_F16_TFLOPS, 4), "kernel": kern,
                        "timing": "graph replay of 100 launches",
                        "graph_output_matches_eager": same,
                        "eager_ms": round(ms_eager, 5),
                        "eager_TFLOP/s": round(flop / (ms_eager * 1e-3) / 1e12, 2)}
            log("  ", name, out[key])
    return out


def run_sweep(torch, tg):
    """Rates across shapes beside the ROCm library (torch.matmul), one JSON
    object per shape on stdout: square f16/bf16 GEMMs from 512^3 to 8192^3
    (A, B = U[-1,1]/8, no epilogue; up to 2048^3 both sides replayed from
    captured graphs of 50 launches), bf16 products with M = 1..32
    (W ~ N(0, 1/K) rotated over enough copies to exceed 1 GiB; also W stored
    [N,K], and W on an odd pitch), token counts off the 64 grid, medium
    token counts and square shapes with B in either layout, and bf16 shapes
    off the tile grid (X ~
    N(0,1), W ~ N(0, 1/K)): token counts that
    leave a partial last tile, grids short of a wave of 256 x 256 tiles,
    pitches off the 8-element grid, and square sizes whose K is not a
    multiple of 128."""
    def graph_ms(fn, per=50, reps=10):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per):
                fn()
        torch.cuda.synchronize()
        return time_launches(lambda: g.replay(), reps, 2) / per

    torch.manual_seed(0)
    for dt in (torch.float16, torch.bfloat16):
        for n in (512, 1024, 2048, 3072, 4096, 6144, 8192):
            A = (torch.rand(n, n, device="cuda") * 2 - 1).to(dt) / 8
            B = (torch.rand(n, n, device="cuda") * 2 - 1).to(dt) / 8
            C = torch.empty(n, n, dtype=dt, device="cuda")
            steps = max(20, min(2000, int(2e13 / (2 * n ** 3))))

            def timed(fn):
                return graph_ms(fn) if n <= 2048 else time_launches(fn, steps, steps // 10 + 2)
            ms = timed(lambda: tg.gemm(A, B, out=C))
            kern = tg.last_kernel()
            ml = timed(lambda: torch.matmul(A, B, out=C))
            print(json.dumps({"shape": "%s %d^3" % (str(dt).split(".")[-1], n),
                              "ms": round(ms, 5), "TFLOP/s": round(2 * n ** 3 / ms / 1e9, 1),
                              "kernel": kern,
                              "library_TFLOP/s": round(2 * n ** 3 / ml / 1e9, 1)}), flush=True)
            del A, B, C
    for (N, K) in ((4096, 4096), (8192, 8192)):
        rot = max(1, (1 << 30) // (N * K * 2))
        Ws = [torch.randn(K, N, dtype=torch.bfloat16, device="cuda") * K ** -0.5
              for _ in range(rot)]
        for M in (1, 4, 8, 16, 24, 32):
            X = torch.randn(M, K, dtype=torch.bfloat16, device="cuda")
            Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            it = [0]

            def ours():
                tg.gemm(X, Ws[it[0] % rot], out=Y)
                it[0] += 1

            def lib():
                torch.matmul(X, Ws[it[0] % rot], out=Y)
                it[0] += 1
            ms = time_launches(ours, 500, 50)
            kern = tg.last_kernel()
            ml = time_launches(lib, 500, 50)
            nb = 2 * (K * N + M * K + M * N)
            print(json.dumps({"shape": "bf16 M=%d N=%d K=%d" % (M, N, K), "ms": round(ms, 5),
                              "GB/s": round(nb / ms / 1e6), "kernel": kern,
                              "library_GB/s": round(nb / ml / 1e6)}), flush=True)
        del Ws
    # small M with W stored [N,K] (rotated as above), and with W on an odd
    # pitch (one copy: 412 MB at N = 50257 already exceeds the last-level cache)
    for (N, K) in ((8192, 8192),):
        rot = max(1, (1 << 30) // (N * K * 2))
        Ws = [(torch.randn(N, K, dtype=torch.bfloat16, device="cuda") * K ** -0.5).t()
              for _ in range(rot)]
        for M in (1, 16, 32):
            X = torch.randn(M, K, dtype=torch.bfloat16, device="cuda")
            Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            it = [0]

            def ours():
                tg.gemm(X, Ws[it[0] % rot], out=Y)
                it[0] += 1

            def lib():
                torch.matmul(X, Ws[it[0] % rot], out=Y)
                it[0] += 1
            ms = time_launches(ours, 500, 50)
            kern = tg.last_kernel()
            ml = time_launches(lib, 500, 50)
            nb = 2 * (K * N + M * K + M * N)
            print(json.dumps({"shape": "bf16 M=%d N=%d K=%d, W stored [N,K]" % (M, N, K),
                              "ms": round(ms, 5), "GB/s": round(nb / ms / 1e6), "kernel": kern,
                              "library_GB/s": round(nb / ml / 1e6)}), flush=True)
        del Ws
    for (M, N, K) in ((1, 50257, 4096), (16, 50257, 4096), (32, 50257, 4096),
                      (16, 32000, 4096)):
        X = torch.randn(M, K, dtype=torch.bfloat16, device="cuda")
        W = (torch.randn(K, N + 1, dtype=torch.bfloat16, device="cuda") * K ** -0.5)[:, :N]
        Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        ms = time_launches(lambda: tg.gemm(X, W, out=Y), 200, 20)
        kern = tg.last_kernel()
        ml = time_launches(lambda: torch.matmul(X, W, out=Y), 200, 20)
        nb = 2 * (K * N + M * K + M * N)
        print(json.dumps({"shape": "bf16 M=%d N=%d K=%d, W pitch %d" % (M, N, K, N + 1),
                          "ms": round(ms, 5), "GB/s": round(nb / ms / 1e6), "kernel": kern,
                          "library_GB/s": round(nb / ml / 1e6)}), flush=True)
        del X, W, Y
    # token counts off the 64 grid, medium token counts (grids short of a
    # wave of 256 x 256 tiles: tile and split count from the launch-time
    # model) and square shapes, both B layouts
    for (M, N, K) in ((48, 4096, 4096), (100, 4096, 4096), (200, 4096, 4096),
                      (128, 4096, 14336), (384, 4096, 14336), (256, 14336, 4096),
                      (640, 14336, 4096), (1024, 4096, 4096), (1024, 8192, 8192),
                      (4096, 4096, 4096), (8192, 8192, 8192)):
        for trans in (False, True):
            X = torch.randn(M, K, dtype=torch.bfloat16, device="cuda")
            if trans:
                W = (torch.randn(N, K, dtype=torch.bfloat16, device="cuda") * K ** -0.5).t()
            else:
                W = torch.randn(K, N, dtype=torch.bfloat16, device="cuda") * K ** -0.5
            Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            f = 2.0 * M * N * K
            steps = max(20, min(500, int(2e13 / f)))
            ms = time_launches(lambda: tg.gemm(X, W, out=Y), steps, steps // 10 + 2)
            kern = tg.last_kernel()
            ml = time_launches(lambda: torch.matmul(X, W, out=Y), steps, steps // 10 + 2)
            print(json.dumps({"shape": "bf16 %dx%dx%d, B %s" % (M, N, K,
                                                                "stored [N,K]" if trans else "[K,N]"),
                              "ms": round(ms, 5), "TFLOP/s": round(f / ms / 1e9, 1),
                              "kernel": kern, "library_TFLOP/s": round(f / ml / 1e9, 1)}),
                  flush=True)
            del X, W, Y
    for (M, N, K) in ((2049, 4096, 4096), (3000, 11008, 4096), (5000, 4096, 4096),
                      (4096, 4000, 4096), (3584, 3584, 3584), (2304, 2304, 2304),
                      (4608, 4608, 4608), (4095, 4095, 4095), (4097, 4097, 4097),
                      (8191, 8191, 8191), (3000, 3000, 2999), (2000, 2000, 2000),
                      (4000, 4000, 4000), (8000, 8000, 8000)):
        X = torch.randn(M, K, dtype=torch.bfloat16, device="cuda")
        W = torch.randn(K, N, dtype=torch.bfloat16, device="cuda") * K ** -0.5
        Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        f = 2.0 * M * N * K
        steps = max(20, min(500, int(2e13 / f)))
        ms = time_launches(lambda: tg.gemm(X, W, out=Y), steps, steps // 10 + 2)
        kern = tg.last_kernel()
        ml = time_launches(lambda: torch.matmul(X, W, out=Y), steps, steps // 10 + 2)
        print(json.dumps({"shape": "bf16 %dx%dx%d" % (M, N, K), "ms": round(ms, 5),
                          "TFLOP/s": round(f / ms / 1e9, 1), "kernel": kern,
                          "library_TFLOP/s": round(f / ml / 1e9, 1)}), flush=True)
        del X, W, Y
        torch.cuda.empty_cache()


def run_stream_k_sweep(torch, tg):
    """Shapes whose 256 x 256 tiles leave a partial last wave, timed with
    stream-K as the library chooses it (TG_STREAMK=1), off (0) and on every
    such grid (2) in the same process, beside the ROCm library; bf16, X ~
    N(0,1), W ~ N(0, 1/K), one JSON object per shape."""
    torch.manual_seed(0)
    shapes = [(3072, 3072, 3072), (3584, 3584, 3584), (5120, 5120, 5120), (6144, 6144, 6144),
              (7168, 7168, 7168), (2049, 4096, 4096), (5000, 4096, 4096), (3000, 11008, 4096),
              (4608, 4096, 4096), (4096, 4096, 4096)]
    for (M, N, K) in shapes:
        X = torch.randn(M, K, dtype=torch.bfloat16, device="cuda")
        W = torch.randn(K, N, dtype=torch.bfloat16, device="cuda") * K ** -0.5
        Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        f = 2.0 * M * N * K
        steps = max(20, min(1000, int(4e13 / f)))
        rec = {"shape": "bf16 %dx%dx%d" % (M, N, K)}
        for flag, key in (("1", "default"), ("0", "off"), ("2", "any_size")):
            os.environ["TG_STREAMK"] = flag
            ms = time_launches(lambda: tg.gemm(X, W, out=Y), steps, steps // 5 + 2)
            rec[key] = {"TFLOP/s": round(f / ms / 1e9, 1), "kernel": tg.last_kernel()}
        os.environ.pop("TG_STREAMK")
        ml = time_launches(lambda: torch.matmul(X, W, out=Y), steps, steps // 5 + 2)
        rec["library_TFLOP/s"] = round(f / ml / 1e9, 1)
        print(json.dumps(rec), flush=True)
        del X, W, Y
        torch.cuda.empty_cache()


def graph_launch_ms(fn, out, ref, replays, per_graph=100):
    """Mean ms per launch of `fn` replayed from a captured graph of
    `per_graph` launches, and whether every replay left `out` equal to `ref`."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    torch.cuda.synchronize()
    same = True
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        same = same and bool(torch.equal(out, ref))
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / (replays * per_graph), same


if __name__ == "__main__":
    main()
