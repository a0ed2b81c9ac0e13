"""Benchmark of the 4-bit block quantizer on one MI355X.

Workload (one step): the 8192 x 8192 bf16 activation tensor with Student-t(3)
entries scaled by 0.02, transformed by the seeded 16-wide RHT and quantized
twice with the two-level scale (E4M3 block scale + FP32 tensor scale):
NVFP4-style E2M1 (alpha = amax / (6 x 448)) and E1M2 (alpha = amax / (3.5 x 448)).
A step is one tensor-amax pass (the amax after the RHT does not depend on
the element format, so both quantizations use it; each derives its own alpha)
followed by the fused RHT + quantize kernel per format, so a step reads the
input three times and writes two sets of codes and scales.  Inputs rotate over
8 resident copies (1 GiB, more than the 256 MB Infinity Cache) so that every
step reads HBM.

value = bf16 input bytes quantized per second (2 bytes x 2 quantizations x n
per step / step time), from K steps with events only at the ends of the
timed region.  The roofline object is for the dominant kernel, the fused RHT
+ quantize kernel: algorithmic bytes per launch (bf16 in + packed codes + E4M3
scales = 171,966,464 B) over its mean duration in a second timed region of K
back-to-back launches over the rotating copies (inputs cold in HBM), with HIP
events on the launch stream at the ends; a plain device copy of the input,
timed the same way, gives the rate a copy reaches.  The `qgemm` object times the
MXFP4 block-scaled GEMM at 8192^3 (A, B: N(0,1) bf16 -> RHT -> MXFP4).
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload,
and `qgemm.cpu_baseline` the oracle's binary64 GEMM on 1024 sampled rows of the
8192^3 product (extrapolated to the full product, and labelled so).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP4_PEAK_TFLOPS = 10100.0
ROWS = COLS = 8192
N_ELEM = ROWS * COLS
QUANT_BYTES = N_ELEM * 2 + N_ELEM // 2 + N_ELEM // 16  # bf16 in + codes + E4M3 scales
AMAX_BYTES = N_ELEM * 2
PMC_FILE = os.path.join(ROOT, "profiles", "quantize_row_e2m1_e4m3_rht_8192x8192_pmc.json")
KERNEL_SRC = os.path.join(ROOT, "block_scaled_bit_ufp4_amd", "csrc", "quantize.hip")
KV_PMC_FILE = os.path.join(ROOT, "profiles", "kv_decode_32x16384_pmc.json")
KV_KERNEL_SRC = os.path.join(ROOT, "block_scaled_bit_ufp4_amd", "csrc", "kvdecode.hip")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--copies", type=int, default=8)
    p.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    p.add_argument("--no-gemm", action="store_true", help="skip the qgemm leg")
    p.add_argument("--no-configs", action="store_true", help="skip the per-workload kernel timings")
    p.add_argument("--no-linear", action="store_true", help="skip the 4-bit linear-layer GEMMs")
    p.add_argument("--no-kv", action="store_true", help="skip the FP4 KV-cache decode attention")
    p.add_argument("--cpu-rows", type=int, default=ROWS)
    p.add_argument("--cpu-reps", type=int, default=2)
    p.add_argument("--cpu-gemm-rows", type=int, default=1024,
                   help="rows of the 8192^3 product the oracle GEMM computes for its cpu_baseline")
    p.add_argument("--cpu-config-rows", type=int, default=256,
                   help="view rows of each workload's quantizations the per-workload oracle timing covers")
    p.add_argument("--gemm-soak", type=float, default=0.0,
                   help="only run the 8192^3 MXFP4 GEMM back to back for this many seconds (for clock and power "
                        "sampling next to it), printing its time per call")
    p.add_argument("--cpu-threads", type=int, default=min(16, os.cpu_count() or 1),
                   help="host threads of the row-partitioned oracle timing (the box's CPU share is 16)")
    return p.parse_args()


# headers every kernel source includes: a change to them changes the kernels too
KERNEL_HEADERS = [os.path.join(ROOT, "block_scaled_bit_ufp4_amd", "csrc", h) for h in ("device.hpp", "kernels.hpp")]


def src_hash(path):
    """SHA-256 prefix of a kernel source together with the headers it includes."""
    h = hashlib.sha256()
    for p in [path] + KERNEL_HEADERS:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(pmc_file=None, kernel_src=None):
    """HBM bytes per launch of a kernel (by default the quantize kernel) from
    the committed rocprofv3 counter summary, if it was taken on the current
    kernel source."""
    try:
        d = json.load(open(pmc_file or PMC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != src_hash(kernel_src or KERNEL_SRC):
        return None
    return d.get("hbm_bytes_per_launch")


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(x_bits, rows, reps, threads):
    """The oracle, as it is, on the host: the bench step (amax + quantize for
    E2M1 and E1M2) over the first `rows` rows, `reps` times; first on one
    thread, then row-partitioned over `threads` host threads (the rows are
    independent once the tensor amax, the max of the slices' amaxes, is
    known; the C oracle runs outside the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle as O
    sample = np.ascontiguousarray(x_bits[:rows])
    cfgs = [O.Cfg(fmt, "e4m3", rht="random", rht_seed=0) for fmt in ("e2m1", "e1m2")]
    t0 = time.perf_counter()
    for _ in range(reps):
        for cfg in cfgs:
            a = O.amax(sample, cfg)
            O.quantize(sample, cfg, amax_value=a)
    dt1 = time.perf_counter() - t0
    parts = [np.ascontiguousarray(sample[i * rows // threads:(i + 1) * rows // threads]) for i in range(threads)]
    with ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        for _ in range(reps):
            for cfg in cfgs:
                a = max(ex.map(lambda p, c=cfg: O.amax(p, c), parts))
                list(ex.map(lambda p, c=cfg, am=a: O.quantize(p, c, amax_value=am), parts))
        dtn = time.perf_counter() - t0
    nbytes = reps * 2 * 2 * sample.size
    what = "the whole step" if rows == ROWS else f"the step on the first {rows} of {ROWS} rows"
    return {"value": round(nbytes / dtn / 1e9, 6), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} (two-level E2M1 and E1M2, amax + quantize, RHT) x {reps}, plain C, "
                      f"row-partitioned over {threads} host threads: {dtn:.2f} s",
            "seconds": round(dtn, 2),
            "single_thread": {"value": round(nbytes / dt1 / 1e9, 6), "seconds": round(dt1, 2), "cores": 1},
            "nproc": os.cpu_count(), "cpu_model": _cpu_model()}


def cpu_config_baselines(S, rows, threads):
    """The oracle's quantize call, as it is, on every workload's
    configurations: the first `rows` view rows of each (all of the 256x1024
    tensor), on one thread and row-partitioned over `threads` host threads;
    elements per second and bf16-input GB/s.  The sample is the same data the
    GPU legs quantize."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle as O

    def run(x, cfg, nrows):
        V = x.shape[0] if cfg.axis == "row" else x.shape[1]
        L = x.shape[1] if cfg.axis == "row" else x.shape[0]
        nrows = min(nrows, V)
        amax = O.amax_threads(x, cfg, threads) if cfg.scale == "e4m3" else None
        t0 = time.perf_counter()
        O.quantize(x, cfg, v0=0, v1=nrows, amax_value=amax)
        t1 = time.perf_counter() - t0
        parts = [(i * nrows // threads, (i + 1) * nrows // threads) for i in range(threads)]
        with ThreadPoolExecutor(threads) as ex:
            t0 = time.perf_counter()
            list(ex.map(lambda r: O.quantize(x, cfg, v0=r[0], v1=r[1], amax_value=amax), parts))
            tn = time.perf_counter() - t0
        n = nrows * L
        return {"elements": n, "single_thread": {"s": round(t1, 4), "Melem_per_s": round(n / t1 / 1e6, 3),
                                                 "GBps": round(2 * n / t1 / 1e9, 5)},
                "threads": {"cores": threads, "s": round(tn, 4), "Melem_per_s": round(n / tn / 1e6, 3),
                            "GBps": round(2 * n / tn / 1e9, 5)}}

    out = {"sample": f"the first {rows} view rows of each quantization (all of quantize_x); the oracle's quantize "
                     f"only (the tensor amax of two-level scales precomputed, not timed)", "cores": threads,
           "kind": "oracle"}
    x = S.quantize_x(256, 1024, seed=0)
    out["quantize_x_256x1024"] = {f: run(x, O.Cfg(f, "fp32"), 256) for f in ("e2m1", "e1m2")}
    x = S.activations_t3(ROWS, COLS, seed=0)
    out["activations_8192x8192"] = {f"{f}_{r}": run(x, O.Cfg(f, "e4m3", rht=r), rows)
                                    for f in ("e2m1", "e1m2", "int4") for r in ("random", "none")}
    c3 = {}
    for name, gen, shape in (("x", S.llama_x, (16384, 4096)), ("w", S.llama_w, (14336, 4096)),
                             ("dy", S.llama_dy, (16384, 14336))):
        x = gen(*shape, seed=0)
        for axis in ("row", "col"):
            sr = name == "dy"
            cfg = O.Cfg("e1m2", "fp32", rht="random", rounding="sr" if sr else "rtne", axis=axis,
                        sr_stream=1 if axis == "col" else 0)
            c3[f"{name}_{axis}"] = run(x, cfg, rows)
        del x
    out["llama_linear_e1m2"] = c3
    x, _ = S.mx_if4(16384, 8192, seed=0)
    out["mxfp4_if4_16384x8192"] = {"mxfp4_h16": run(x, O.Cfg("e2m1", "e8m0", 32, rht="det"), rows),
                                   "if4": run(x, O.Cfg("if4", "e4m3"), rows),
                                   "nvfp4": run(x, O.Cfg("e2m1", "e4m3"), rows)}
    x = S.gemm_a(ROWS, COLS, seed=0)
    out["gemm_operands_8192x8192"] = {"mxfp4_rht": run(x, O.Cfg("e2m1", "e8m0", 32, rht="random"), rows),
                                      "e1m2_rht": run(x, O.Cfg("e1m2", "fp32", rht="random"), rows)}
    return out


def gemm_soak(U, S, torch, dev, stream, seconds):
    """The 8192^3 MXFP4 GEMM back to back for `seconds`, printing the time per
    call every ~0.5 s (a clock and power sampler run beside it reads the
    chip in that state)."""
    M = N = K = 8192
    a = torch.from_numpy(S.gemm_a(M, K).view(np.int16)).view(torch.bfloat16).to(dev)
    b = torch.from_numpy(S.gemm_b(N, K).view(np.int16)).view(torch.bfloat16).to(dev)
    cfg = U.Cfg("e2m1", "e8m0", 32, rht="random", rht_seed=0)
    qa, qb = U.ufp4_quantize(a, cfg), U.ufp4_quantize(b, cfg)
    c = torch.empty((M, N), dtype=torch.float32, device=dev)
    t_end = time.time() + seconds
    res = []
    while time.time() < t_end:
        ms = _time(lambda: U.ufp4_qgemm(qa, qb, "mxfp4", c=c), torch, stream, 1500)
        res.append(ms)
        print(json.dumps({"t": round(time.time(), 3), "gemm_ms": round(ms, 5),
                          "tflops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)}), flush=True)
    return res


def cpu_gemm_baseline(S, rows, threads, M=8192, N=8192, K=8192):
    """The oracle's binary64 GEMM (the plain triple loop) on the first `rows`
    rows of Z = A B^T for the 8192^3 GEMM's bf16 inputs, row-partitioned over
    `threads` host threads, and on rows / 16 of them on one thread; both
    extrapolated to the full product and labelled so."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle as O

    def widen(bits):  # bf16 bits -> the float32 values they hold
        return (bits.astype(np.uint32) << 16).view(np.float32)

    a = widen(S.gemm_a(M, K)[:rows])
    b = np.ascontiguousarray(widen(S.gemm_b(N, K)))
    r1 = max(1, rows // 16)
    t0 = time.perf_counter()
    O.gemm_nt(a[:r1], b)
    dt1 = time.perf_counter() - t0
    parts = [np.ascontiguousarray(a[i * rows // threads:(i + 1) * rows // threads]) for i in range(threads)]
    with ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(O.gemm_nt, parts, [b] * threads))
        dtn = time.perf_counter() - t0
    gf = 2.0 * rows * N * K / 1e9
    return {"value": round(gf / dtn, 3), "unit": "GFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"binary64 Z = A B^T on {rows} of {M} rows ({gf:.1f} GFLOP), plain C, row-partitioned "
                      f"over {threads} host threads: {dtn:.2f} s",
            "extrapolated_full_product_s": round(dtn * M / rows, 1),
            "single_thread": {"value": round(2.0 * r1 * N * K / 1e9 / dt1, 3), "rows": r1,
                              "seconds": round(dt1, 2), "extrapolated_full_product_s": round(dt1 * M / r1, 1)}}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; --gpus must be 1 (the quantizer shards by rows "
                                   "with no exchange except a 4-byte amax MAX all-reduce, not run here)"}))
        sys.exit(2)
    import torch
    import block_scaled_bit_ufp4_amd as U
    import synthetic as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.gemm_soak > 0:
        gemm_soak(U, S, torch, dev, torch.cuda.current_stream(), args.gemm_soak)
        return
    t0 = time.time()
    x_bits = S.activations_t3(ROWS, COLS, seed=0)
    print(f"# generated input in {time.time() - t0:.1f} s, sha256 {S.digest(x_bits)[:16]}", file=sys.stderr,
          flush=True)
    x0 = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    xs = [x0] + [x0.clone() for _ in range(args.copies - 1)]
    cfgs = [U.Cfg("e2m1", "e4m3", rht="random", rht_seed=0), U.Cfg("e1m2", "e4m3", rht="random", rht_seed=0)]
    outs = [[U.alloc_qtensor(ROWS, COLS, c) for c in cfgs] for _ in range(args.copies)]
    amaxes = [torch.zeros(1, dtype=torch.float32, device=dev) for _ in range(args.copies)]
    amax_ws = torch.empty(U.ufp4_workspace_size(U.OP_AMAX, ROWS, COLS, cfgs[0]), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        j = i % args.copies
        # the tensor amax after the RHT depends on the rotation and axis only,
        # not on the element format: one pass serves both quantizations (each
        # derives its own alpha = amax / (gridmax x 448) from it)
        U.ufp4_amax(xs[j], cfgs[0], out=amaxes[j], ws=amax_ws)
        for f, cfg in enumerate(cfgs):
            U.ufp4_quantize(xs[j], cfg, amax=amaxes[j], out=outs[j][f])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # timed region 1: the K steps as a user runs them, events only at the ends
    # (this gives value and ms_per_step)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    # timed region 2: the roofline.  K back-to-back launches of each quantize
    # kernel over the rotating copies, events on the launch stream at the
    # ends only, with no amax pass before them: every launch reads its input
    # cold from HBM.  A plain device copy of the input over the same copies,
    # timed the same way, gives the rate a copy reaches.  (Inside the step the
    # kernel runs a few microseconds faster, just after the amax pass has read
    # the same input; events that a launch timestamps itself add a gap and
    # read several microseconds high, so neither serves as the kernel's HBM
    # rate.)
    def b2b(fn):
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(args.steps):
            fn(i % args.copies)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps
    q_ms = [b2b(lambda j, f=f, cfg=cfg: U.ufp4_quantize(xs[j], cfg, amax=amaxes[j], out=outs[j][f]))
            for f, cfg in enumerate(cfgs)]
    dst = [torch.empty_like(x0) for _ in range(args.copies)]
    copy_ms = b2b(lambda j: dst[j].copy_(xs[(3 * j + 1) % args.copies]))
    del dst
    copy_gbs = 2 * 2 * N_ELEM / (copy_ms * 1e-3) / 1e9
    value = 2 * N_ELEM * len(cfgs) / (ms_step * 1e-3) / 1e9
    achieved = QUANT_BYTES / (q_ms[0] * 1e-3) / 1e9
    traffic = traffic_from_profile()
    out = {
        "metric": "quantize GB/s (bf16 in) and % HBM peak; qGEMM TFLOP/s, 1 MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "8192x8192 bf16 Student-t(3)*0.02 activations; RHT-16 (seeded signs) + "
                               "two-level E4M3/FP32 scale; E2M1 (NVFP4-style) and E1M2; one tensor-amax pass "
                               "(shared: it does not depend on the format) + a fused quantize per format",
                   "rows": ROWS, "cols": COLS, "block": 16, "input_copies": args.copies},
        "pct_hbm_peak_step": round(100.0 * (AMAX_BYTES + 2 * QUANT_BYTES) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "row_kernel (fused RHT + E2M1 + E4M3 two-level quantize)",
                     "bytes_per_launch": QUANT_BYTES, "avg_launch_ms": round(q_ms[0], 5),
                     "e1m2_avg_launch_ms": round(q_ms[1], 5),
                     "timing": "second timed region: K back-to-back launches over the rotating copies (inputs "
                               "cold in HBM), HIP events on the launch stream at its ends",
                     "device_copy_GBps": round(copy_gbs, 1),
                     "frac_of_device_copy": round(achieved / copy_gbs, 4)},
    }
    if not args.no_gemm:
        out["qgemm"] = bench_gemm(U, S, torch, dev, stream)
    if not args.no_configs:
        out["configs"] = bench_configs(U, S, torch, dev, stream)
    if not args.no_linear:
        out["linear"] = bench_linear(U, S, torch, dev, stream)
    if not args.no_kv:
        out["kv_decode"] = bench_kv(U, S, torch, dev, stream)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(x_bits, args.cpu_rows, args.cpu_reps, args.cpu_threads)
        if not args.no_configs:
            out["cpu_baseline"]["per_config"] = cpu_config_baselines(S, args.cpu_config_rows, args.cpu_threads)
        if not args.no_gemm:
            out["qgemm"]["cpu_baseline"] = cpu_gemm_baseline(S, args.cpu_gemm_rows, args.cpu_threads)
    print(json.dumps(out), flush=True)


def _time(fn, torch, stream, reps, warm=2):
    """Milliseconds per call over reps back-to-back calls, HIP events on the
    stream at the ends only, after warm untimed calls."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def bench_gemm(U, S, torch, dev, stream, reps=10):
    """8192^3 block-scaled GEMMs: MXFP4 on the native scaled MFMA (the headline
    qGEMM), the E1M2 dequantize-to-bf16 path, and the plain bf16 GEMM."""
    M = N = K = 8192
    flop = 2.0 * M * N * K
    a = torch.from_numpy(S.gemm_a(M, K).view(np.int16)).view(torch.bfloat16).to(dev)
    b = torch.from_numpy(S.gemm_b(N, K).view(np.int16)).view(torch.bfloat16).to(dev)
    cfg = U.Cfg("e2m1", "e8m0", 32, rht="random", rht_seed=0)
    qa, qb = U.ufp4_quantize(a, cfg), U.ufp4_quantize(b, cfg)
    c = torch.empty((M, N), dtype=torch.float32, device=dev)
    # The clock ramps up over the first ~0.1 s of back-to-back GEMMs (an
    # alternating A/B read 0.36 ms per call in the first 20 and 0.30 ms by the
    # fifth 20): 300 untimed calls first, so the timed ones run at the rate
    # the chip sustains (at its power limit).
    ms_call = _time(lambda: U.ufp4_qgemm(qa, qb, "mxfp4", c=c), torch, stream, 5 * reps, warm=300)
    cfg2 = U.Cfg("e1m2", "fp32", rht="random", rht_seed=0)
    ea, eb = U.ufp4_quantize(a, cfg2), U.ufp4_quantize(b, cfg2)
    ws = torch.empty(U.ufp4_workspace_size(U.OP_QGEMM, M + N, K, cfg2), dtype=torch.uint8, device=dev)
    ms_e1m2 = _time(lambda: U.ufp4_qgemm(ea, eb, "bf16", c=c, ws=ws), torch, stream, 2 * reps, warm=100)
    ms_bf16 = _time(lambda: U.ufp4_gemm_bf16(a, b, c=c), torch, stream, 2 * reps, warm=100)
    tf = flop / (ms_call * 1e-3) / 1e12
    # attenuation and output SQNR of both paths against Z = A B^T of the bf16
    # inputs, and the whole path (quantize both operands, then the GEMM)
    zc5 = U.ufp4_gemm_bf16(a, b)
    quality = {}
    for name, fn in (("mxfp4", lambda: U.ufp4_qgemm(qa, qb, "mxfp4", c=c)),
                     ("e1m2", lambda: U.ufp4_qgemm(ea, eb, "bf16", c=c, ws=ws))):
        fn()
        sm = U.ufp4_eta(c, zc5).cpu().numpy()
        quality[name] = {"eta": round(float(sm[0] / sm[1]), 6), "sqnr_db": round(float(10 * np.log10(sm[1] / sm[2])), 3)}
    del zc5

    def e2e_mx():
        U.ufp4_quantize(a, cfg, out=qa)
        U.ufp4_quantize(b, cfg, out=qb)
        U.ufp4_qgemm(qa, qb, "mxfp4", c=c)

    def e2e_e1m2():
        U.ufp4_quantize(a, cfg2, out=ea)
        U.ufp4_quantize(b, cfg2, out=eb)
        U.ufp4_qgemm(ea, eb, "bf16", c=c, ws=ws)

    ms_e2e_mx = _time(e2e_mx, torch, stream, reps)
    ms_e2e_e1m2 = _time(e2e_e1m2, torch, stream, reps)
    # IF4 against NVFP4 and MXFP4 on the MXFP4/IF4 workload's data: A, B are
    # its two 8192-row halves (N(0,1) with uniform 1x32 blocks)
    xh, _ = S.mx_if4(2 * M, K, seed=0)
    xa = torch.from_numpy(xh[:M].view(np.int16)).view(torch.bfloat16).to(dev)
    xb = torch.from_numpy(xh[M:].view(np.int16)).view(torch.bfloat16).to(dev)
    zref = U.ufp4_gemm_bf16(xa, xb)
    c4 = {}
    for name, cfgf, mode in (("if4", U.Cfg("if4", "e4m3"), "bf16"), ("nvfp4", U.Cfg("e2m1", "e4m3"), "bf16"),
                             ("mxfp4_h16", U.Cfg("e2m1", "e8m0", 32, rht="det"), "mxfp4")):
        qa_, qb_ = U.ufp4_quantize(xa, cfgf), U.ufp4_quantize(xb, cfgf)
        ws_ = torch.empty(U.ufp4_workspace_size(U.OP_QGEMM, M + N, K, cfgf), dtype=torch.uint8, device=dev) \
            if mode == "bf16" else None
        ms_ = _time(lambda: U.ufp4_qgemm(qa_, qb_, mode, c=c, ws=ws_), torch, stream, 3)
        sm = U.ufp4_eta(c, zref).cpu().numpy()
        c4[name] = {"ms": round(ms_, 4), "eta": round(float(sm[0] / sm[1]), 6),
                    "sqnr_db": round(float(10 * np.log10(sm[1] / sm[2])), 3)}
    return {"workload": "8192^3 MXFP4 (E2M1 + E8M0/32, RHT-16) native scaled MFMA, fp32 out",
            "ms": round(ms_call, 4), "timing": "50 back-to-back calls (one kernel each) after 300 untimed ones (the clock settles), events at the ends",
            "tflops": round(tf, 1), "peak_tflops": FP4_PEAK_TFLOPS, "frac": round(tf / FP4_PEAK_TFLOPS, 4),
            "eta": quality["mxfp4"]["eta"], "sqnr_db": quality["mxfp4"]["sqnr_db"],
            "quantize_and_gemm_ms": round(ms_e2e_mx, 4),
            "quantize_and_gemm_tflops": round(flop / (ms_e2e_mx * 1e-3) / 1e12, 1),
            "e1m2_dequant_bf16": {"ms": round(ms_e1m2, 4), "tflops": round(flop / (ms_e1m2 * 1e-3) / 1e12, 1),
                                  "eta": quality["e1m2"]["eta"], "sqnr_db": quality["e1m2"]["sqnr_db"],
                                  "quantize_and_gemm_ms": round(ms_e2e_e1m2, 4),
                                  "note": "dequantize both operands to bf16 (workspace) + bf16 MFMA GEMM"},
            "bf16_reference": {"ms": round(ms_bf16, 4), "tflops": round(flop / (ms_bf16 * 1e-3) / 1e12, 1),
                               "peak_tflops": 2500.0},
            "mxfp4_if4_data_8192^3": c4}


def bench_linear(U, S, torch, dev, stream, reps=3):
    """The llama-shaped linear layer's three GEMMs (X 16384x4096, W
    14336x4096, dY 16384x14336) on 4-bit operands, for the UFP4 recipe (E1M2,
    RHT on all, SR on dY) and the E2M1 baseline (RHT on bwd_dw only): time of
    quantizing both operands, of the dequantize-to-bf16 GEMM, and the
    attenuation eta and output SQNR against the unquantized bf16 product."""
    import block_scaled_bit_ufp4_amd.linear as lin

    def dev_bf16(h):
        return torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(dev)

    def transposed(a):  # the column kernel without rotation: an exact transpose
        return U.ufp4_rht(a, axis="col", rht="none", out_dtype=torch.bfloat16)

    T, K, N = 16384, 4096, 14336
    x, w, dy = dev_bf16(S.llama_x(T, K)), dev_bf16(S.llama_w(N, K)), dev_bf16(S.llama_dy(T, N))
    z = {"fwd_y": U.ufp4_gemm_bf16(x, w), "bwd_dx": U.ufp4_gemm_bf16(dy, transposed(w)),
         "bwd_dw": U.ufp4_gemm_bf16(transposed(dy), transposed(x))}
    # 50 untimed GEMMs (~0.1 s) first, as in the 8192^3 leg: the clock settles
    ms_ref = _time(lambda: U.ufp4_gemm_bf16(x, w, c=z["fwd_y"]), torch, stream, reps, warm=50)
    out = {"workload": "linear layer X 16384x4096, W 14336x4096, dY 16384x14336; three GEMMs of 1.924 TFLOP each",
           "bf16_reference_gemm_ms": round(ms_ref, 4)}
    for name, r in (("ufp4", lin.UFP4), ("e2m1_baseline", lin.E2M1_BASELINE)):
        makers = {"fwd_y": lambda: lin.operands_fwd(x, w, r), "bwd_dx": lambda: lin.operands_dx(dy, w, r),
                  "bwd_dw": lambda: lin.operands_dw(dy, x, r)}
        res = {}
        for g, mk in makers.items():
            qa, qb = mk()
            M, Nn = z[g].shape
            Kk = qa.cfg.view_shape(qa.rows, qa.cols)[1]
            c = torch.empty_like(z[g])
            ws = torch.empty(U.ufp4_workspace_size(U.OP_QGEMM, M + Nn, Kk, qa.cfg), dtype=torch.uint8, device=dev)
            ms = _time(lambda: U.ufp4_qgemm(qa, qb, "bf16", c=c, ws=ws), torch, stream, reps, warm=50)
            ms_q = _time(mk, torch, stream, reps)
            sm = U.ufp4_eta(c, z[g]).cpu().numpy()
            res[g] = {"quantize_operands_ms": round(ms_q, 4), "gemm_ms": round(ms, 4),
                      "tflops": round(2.0 * M * Nn * Kk / (ms * 1e-3) / 1e12, 1),
                      "eta": round(float(sm[0] / sm[1]), 6),
                      "sqnr_db": round(float(10 * np.log10(sm[1] / sm[2])), 3)}
        out[name] = res
    return out


def bench_kv(U, S, torch, dev, stream, reps=20):
    """One decode step of attention against the FP4 KV cache at the Llama-3-8B
    attention shape (32 query heads, 8 KV heads, head dim 128) for 32
    sequences of 16384 tokens: MXFP8 query x MXFP4 keys (Walsh-Hadamard
    rotated, or not) and values on the scaled MFMA, and the FP8 (MXFP8) cache
    the UltraQuant section measures against.  Reports the step (decode kernel
    + split combine), the decode kernel alone, its HBM rate against the
    algorithmic bytes (cache + query + output), the cache quantization, the
    output error against exact attention (fp32 softmax over the unquantized
    bf16 keys and values) for random queries (near-uniform attention over the
    16k tokens) and for queries aimed at four tokens each (peaked attention),
    and the FP4 over FP8 decode speedup."""
    B, Hq, Hkv, L, D = 32, 32, 8, 16384, 128
    G = Hq // Hkv
    q, k, v = S.kv_decode(B, Hq, Hkv, L, D, seed=0)

    def dev_bf16(h):
        return torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(dev)

    qp = S.kv_peaked_q(k, Hq, seed=0)
    qd, kd, vd, qpd = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(qp)
    del k, v
    lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    sm = 1.0 / math.sqrt(D)

    def exact_attention(qx):
        ex = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        for b in range(B):  # fp32 reference, one sequence at a time
            qf = qx[b].float().view(Hkv, G, D)
            kt = kd[b].float().transpose(1, 2).contiguous()
            p = torch.softmax(torch.matmul(qf, kt) * sm, dim=-1)
            ex[b] = torch.matmul(p, vd[b].float()).view(Hq, D)
        return ex

    exact = exact_attention(qd)
    exact_peaked = exact_attention(qpd)
    cache_bytes = U.ufp4_kv_cache_bytes(B, Hkv, L, D)
    traffic = traffic_from_profile(KV_PMC_FILE, KV_KERNEL_SRC)
    alg_bytes = cache_bytes + B * Hq * D * 2 + B * Hq * D * 4
    out = {"workload": "decode step, 32 sequences x 16384 tokens, 32 query / 8 KV heads, head dim 128; FP4 cache "
                       "(E2M1 + UE8M0/32: keys per token over the head dim, values per channel over 32 tokens)",
           "cache_bytes": cache_bytes, "bytes_per_token_per_kv_head": 136, "bf16_bytes_per_token_per_kv_head": 512,
           "algorithmic_bytes_per_step": alg_bytes}
    for name, rot, fmt in (("rotated_keys", True, "fp4"), ("no_rotation", False, "fp4"),
                           ("fp8_baseline_rotated_keys", True, "fp8")):
        cache = U.ufp4_kv_cache_quantize(kd, vd, lens, rot, fmt=fmt)
        o = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        need = U.ufp4_kv_decode_workspace_size(B, Hq, Hkv, L)
        ws = torch.empty(max(16, need), dtype=torch.uint8, device=dev)
        ms_step = _time(lambda: U.ufp4_kv_decode(qd, cache, lens, Hkv, L, sm, rot, out=o, ws=ws, fmt=fmt),
                        torch, stream, reps)
        ms_quant = _time(lambda: U.ufp4_kv_cache_quantize(kd, vd, lens, rot, cache, fmt=fmt), torch, stream, 3)
        err = float(torch.linalg.norm(o - exact) / torch.linalg.norm(exact))
        op = U.ufp4_kv_decode(qpd, cache, lens, Hkv, L, sm, rot, ws=ws, fmt=fmt)
        err_peaked = float(torch.linalg.norm(op - exact_peaked) / torch.linalg.norm(exact_peaked))
        nbytes = U.ufp4_kv_cache_bytes(B, Hkv, L, D, fmt) + B * Hq * D * 6
        # one kernel per call here (B * Hkv >= 256 workgroups: no split, no
        # combine), so the back-to-back call time is the kernel's duration
        gbs = nbytes / (ms_step * 1e-3) / 1e9
        out[name] = {"cache_format": fmt, "step_us": round(ms_step * 1e3, 2),
                     "decode_kernel_GBps": round(gbs, 1),
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(gbs / HBM_PEAK_GBS, 4),
                                  "traffic": traffic if fmt == "fp4" else None,
                                  "kernel": f"kv_decode_kernel<{fmt == 'fp8'}>".lower(),
                                  "bytes_per_launch": nbytes},
                     "step_GBps": round(alg_bytes / (ms_step * 1e-3) / 1e9, 1),
                     "cache_quantize_us": round(ms_quant * 1e3, 2),
                     "rel_err_vs_exact_attention": round(err, 5),
                     "rel_err_vs_exact_attention_peaked_queries": round(err_peaked, 5)}
        del cache
    out["fp4_over_fp8_decode_speedup"] = round(out["fp8_baseline_rotated_keys"]["step_us"] /
                                               out["rotated_keys"]["step_us"], 3)
    return out


def _qbytes(n, cfg, elt=2):
    """Algorithmic bytes of one quantize pass over n input elements of elt
    bytes (bf16 by default)."""
    scale = 4 * n // cfg.block if cfg.scale == "fp32" else n // cfg.block
    return elt * n + n // 2 + scale


ROTATE_BYTES = 1 << 30   # inputs of a leg rotate over at least this many bytes (> 256 MB MALL + L2)


def _copies(x, min_bytes=ROTATE_BYTES):
    """x and clones of it, at least min_bytes in all (at least three)."""
    k = max(3, -(-min_bytes // (x.numel() * x.element_size())))
    return [x] + [x.clone() for _ in range(k - 1)]


def _time_rot(fn, n, torch, stream, reps=20):
    """Microseconds per call of fn(j) over reps back-to-back calls that
    rotate j over n copies, HIP events on the stream at the ends only: each
    call reads its input cold from HBM."""
    for j in range(n):
        fn(j)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        fn(i % n)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def _leg(U, torch, stream, xs, cfg, amax=None):
    """Kernel time and HBM rate of one quantize call on cold inputs: xs are
    copies of one tensor (over 1 GiB in all) and each has its own outputs;
    amax (one device float, the same for every copy) is given for E4M3 so the
    call is one kernel.  Returns the leg and the first copy's quantization."""
    x = xs[0]
    qs = [U.alloc_qtensor(x.shape[0], x.shape[1], cfg) for _ in xs]
    us = _time_rot(lambda j: U.ufp4_quantize(xs[j], cfg, amax=amax, out=qs[j]), len(xs), torch, stream)
    b = _qbytes(x.numel(), cfg, x.element_size())
    return {"us": round(us, 2), "bytes": b, "GBps": round(b / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}, qs[0]


def bench_configs(U, S, torch, dev, stream):
    """Kernel times of every workload: the quantizations of the five
    configurations, with each kernel's algorithmic bytes and HBM rate.  Every
    leg rotates its input over copies of more than 1 GiB (and its outputs
    over as many), so every launch reads HBM, not the 256 MB last-level
    cache."""
    def dev_bf16(h):
        return torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(dev)

    out = {"timing": "back-to-back calls rotating over input copies of more than 1 GiB in all (inputs cold in "
                     "HBM), HIP events at the ends; quantize_x excepted (0.5 MiB, launch-bound)"}
    # quantize_x: 256x1024, FP32 1x16, no RHT (launch-bound; correctness config)
    x = dev_bf16(S.quantize_x(256, 1024, seed=0))
    c1 = {}
    for fmt in ("e2m1", "e1m2"):
        cfg = U.Cfg(fmt, "fp32")
        leg, q = _leg(U, torch, stream, [x], cfg)
        leg["dequant_us"] = round(_time(lambda: U.ufp4_dequantize(q), torch, stream, 10) * 1e3, 2)
        leg["stats_us"] = round(_time(lambda: U.ufp4_stats(x, q), torch, stream, 10) * 1e3, 2)
        c1[fmt] = leg
    out["quantize_x_256x1024"] = c1
    # activations 8192^2: two-level E4M3 with and without RHT per format, and
    # the UFP4 recipe's FP32 single-level E1M2 with and without RHT
    xs = _copies(dev_bf16(S.activations_t3(ROWS, COLS, seed=0)))
    x = xs[0]
    c2 = {}
    for fmt in ("e2m1", "e1m2", "int4"):
        for rht in ("random", "none"):
            cfg = U.Cfg(fmt, "e4m3", rht=rht, rht_seed=0)
            c2[f"{fmt}_{rht}"] = _leg(U, torch, stream, xs, cfg, U.ufp4_amax(x, cfg))[0]
    for rht in ("random", "none"):
        c2[f"e1m2_fp32_{rht}"] = _leg(U, torch, stream, xs, U.Cfg("e1m2", "fp32", rht=rht, rht_seed=0))[0]
    cfg = U.Cfg("e2m1", "e4m3", rht="random", rht_seed=0)
    amax = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(U.ufp4_workspace_size(U.OP_AMAX, ROWS, COLS, cfg), dtype=torch.uint8, device=dev)
    us = _time_rot(lambda j: U.ufp4_amax(xs[j], cfg, out=amax, ws=ws), len(xs), torch, stream)
    c2["amax_pass"] = {"us": round(us, 2), "GBps": round(2 * x.numel() / (us * 1e-6) / 1e9, 1)}
    # the statistics and the dequantize (with the inverse RHT) of the E2M1 quantization
    q = U.ufp4_quantize(x, cfg, amax=U.ufp4_amax(x, cfg))
    sums = torch.empty(U.NSUMS, dtype=torch.float64, device=dev)
    sws = torch.empty(U.ufp4_workspace_size(U.OP_STATS, ROWS, COLS, cfg), dtype=torch.uint8, device=dev)
    qs = [q] + [U.ufp4_quantize(xs[j], cfg, amax=U.ufp4_amax(x, cfg)) for j in range(1, len(xs))]
    c2["stats_e2m1_us"] = round(_time_rot(lambda j: U.ufp4_stats(xs[j], qs[j], sums=sums, ws=sws), len(xs), torch,
                                          stream, 10), 2)
    ys = [torch.empty((ROWS, COLS), dtype=torch.float32, device=dev) for _ in range(3)]
    c2["dequant_inverse_rht_f32_us"] = round(_time_rot(lambda j: U.ufp4_dequantize(qs[j], inverse_rht=True,
                                                                                    y=ys[j % 3]),
                                                       len(xs), torch, stream, 10), 2)
    del ys, qs
    # The pages' one directly comparable figure: the fused RHT + quantize
    # against the quantize alone, and the unfused pair (the RHT as its own
    # pass writing y, then the quantize reading y) against the quantize alone,
    # for UFP4's E1M2 with the FP32 1x16 scale (1.06x / 1.07x fused, 1.62x /
    # 1.41x unfused on their two GPUs).  An fp32 intermediate reproduces the
    # fused codes exactly; a bf16 one is what a bf16 pipeline would store.
    ratios = {}
    for fmt, scale in (("e1m2", "fp32"), ("e2m1", "e4m3")):
        key = "e1m2_fp32" if fmt == "e1m2" else "e2m1"
        fused, alone = c2[f"{key}_random"]["us"], c2[f"{key}_none"]["us"]
        r = {"fused_us": fused, "quantize_only_us": alone, "fused_over_quantize_only": round(fused / alone, 4)}
        cfg_y = U.Cfg(fmt, scale, rht="none")
        for name, dt in (("fp32_intermediate", torch.float32), ("bf16_intermediate", torch.bfloat16)):
            ys = [torch.empty((ROWS, COLS), dtype=dt, device=dev) for _ in xs]
            for j in range(len(xs)):
                U.ufp4_rht(xs[j], rht="random", seed=0, y=ys[j])
            am = U.ufp4_amax(ys[0], cfg_y) if scale == "e4m3" else None
            qy = [U.alloc_qtensor(ROWS, COLS, cfg_y) for _ in xs]
            us_rht = _time_rot(lambda j: U.ufp4_rht(xs[j], rht="random", seed=0, y=ys[j]), len(xs), torch, stream)
            us_q = _time_rot(lambda j: U.ufp4_quantize(ys[j], cfg_y, amax=am, out=qy[j]), len(xs), torch, stream)
            us_pair = _time_rot(lambda j: (U.ufp4_rht(xs[j], rht="random", seed=0, y=ys[j]),
                                           U.ufp4_quantize(ys[j], cfg_y, amax=am, out=qy[j])), len(xs), torch, stream)
            r[f"unfused_{name}"] = {"rht_us": round(us_rht, 2), "quantize_us": round(us_q, 2),
                                    "pair_us": round(us_pair, 2),
                                    "pair_over_quantize_only": round(us_pair / alone, 4)}
            del ys, qy
        ratios[f"{fmt}_{scale}"] = r
    ratios["pages"] = {"fused_over_quantize_only": {"SM90": 1.06, "SM100": 1.07},
                       "unfused_over_quantize_only": {"SM90": 1.62, "SM100": 1.41},
                       "format": "E1M2, 1x16 blocks, FP32 scale, 16-wide Hadamard; other hardware: context"}
    c2["rht_cost"] = ratios
    out["activations_8192x8192"] = c2
    del xs, x
    # llama linear: E1M2, FP32 1x16, RHT-16 on all; SR (stream 0 row, 1 col) on dY
    c3 = {}
    for name, gen, shape in (("x", S.llama_x, (16384, 4096)), ("w", S.llama_w, (14336, 4096)),
                             ("dy", S.llama_dy, (16384, 14336))):
        xs = _copies(dev_bf16(gen(*shape, seed=0)))
        for axis in ("row", "col"):
            sr = name == "dy"
            cfg = U.Cfg("e1m2", "fp32", rht="random", rht_seed=0, rounding="sr" if sr else "rtne", axis=axis,
                        sr_seed=0, sr_stream=1 if axis == "col" else 0)
            c3[f"{name}_{axis}"] = _leg(U, torch, stream, xs, cfg)[0]
        del xs
    tot_b = sum(v["bytes"] for v in c3.values())
    tot_us = sum(v["us"] for v in c3.values())
    c3["all_six"] = {"us": round(tot_us, 2), "bytes": tot_b, "GBps": round(tot_b / (tot_us * 1e-6) / 1e9, 1)}
    out["llama_linear_e1m2"] = c3
    # mxfp4 + if4 on 16384x8192
    xh, _ = S.mx_if4(16384, 8192, seed=0)
    xs = _copies(dev_bf16(xh))
    c4 = {"mxfp4_h16": _leg(U, torch, stream, xs, U.Cfg("e2m1", "e8m0", 32, rht="det"))[0]}
    for fmt in ("if4", "e2m1"):
        cfg = U.Cfg(fmt, "e4m3")
        c4[fmt if fmt == "if4" else "nvfp4"] = _leg(U, torch, stream, xs, cfg, U.ufp4_amax(xs[0], cfg))[0]
    c4["if4_overhead_vs_nvfp4"] = round(c4["if4"]["us"] / c4["nvfp4"]["us"] - 1, 4)
    out["mxfp4_if4_16384x8192"] = c4
    del xs
    # gemm operands: 8192^2 to MXFP4 (RHT) and to E1M2 (RHT) with its bf16 dequantization
    xs = _copies(dev_bf16(S.gemm_a(ROWS, COLS, seed=0)))
    c5 = {"mxfp4_rht": _leg(U, torch, stream, xs, U.Cfg("e2m1", "e8m0", 32, rht="random", rht_seed=0))[0]}
    cfg = U.Cfg("e1m2", "fp32", rht="random", rht_seed=0)
    leg, _ = _leg(U, torch, stream, xs, cfg)
    qs = [U.ufp4_quantize(xj, cfg) for xj in xs]
    ys = [torch.empty((ROWS, COLS), dtype=torch.bfloat16, device=dev) for _ in xs]
    leg["dequant_bf16_us"] = round(_time_rot(lambda j: U.ufp4_dequantize(qs[j], y=ys[j]), len(xs), torch, stream), 2)
    c5["e1m2_rht"] = leg
    out["gemm_operands_8192x8192"] = c5
    del xs, qs, ys
    out["formats"] = bench_formats(U, S, torch, dev)
    return out


def bench_formats(U, S, torch, dev):
    """Quantization quality per format on the activation (8192x8192 t3*0.02)
    and MXFP4 (16384x8192 N(0,1) + uniform blocks) tensors, NVFP4-style
    two-level scale, with and without RHT: SQNR, signal factor alpha and mean
    shrinkage, from the statistics kernel.  The capped E2M1 grids are the
    pages' attempt to emulate a uniform grid on E2M1; int4 is NVINT4.  Then
    the llama-shaped linear layer's X, W and dY with the single-level FP32
    scale, E2M1 and E1M2, with the SQNR gain from the RHT."""
    def dev_bf16(h):
        return torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(dev)

    res = {}
    for name, xh in (("activations_8192x8192", S.activations_t3(ROWS, COLS, seed=0)),
                     ("mxfp4_data_16384x8192", S.mx_if4(16384, 8192, seed=0)[0])):
        x = dev_bf16(xh)
        d = {}
        for rht in ("none", "random"):
            for fmt in ("e2m1", "e2m1_max4", "e2m1_max3", "e2m1_max2", "e1m2", "int4"):
                cfg = U.Cfg(fmt, "e4m3", rht=rht, rht_seed=0)
                r = U.ufp4_stats_finalize(U.ufp4_stats(x, U.ufp4_quantize(x, cfg)))
                d[f"{fmt}_{rht}"] = {"sqnr_db": round(r["sqnr_db"], 3), "alpha": round(r["alpha"], 6),
                                     "mean_shrink": float(f"{r['mean_shrink']:.4e}")}
        res[name] = d
        del x
    # the linear layer's operands with the UFP4 recipe's single-level FP32
    # scale (row axis), E2M1 for contrast; dY also with stochastic rounding
    d = {}
    for name, xh in (("x_16384x4096", S.llama_x(16384, 4096)), ("w_14336x4096", S.llama_w(14336, 4096)),
                     ("dy_16384x14336", S.llama_dy(16384, 14336))):
        x = dev_bf16(xh)
        del xh
        e = {}
        for rht in ("none", "random"):
            for fmt, rnd in (("e2m1", "rtne"), ("e1m2", "rtne")) + ((("e1m2", "sr"),) if name.startswith("dy") else ()):
                cfg = U.Cfg(fmt, "fp32", rht=rht, rht_seed=0, rounding=rnd)
                r = U.ufp4_stats_finalize(U.ufp4_stats(x, U.ufp4_quantize(x, cfg)))
                e[f"{fmt}_{rht}" + ("_sr" if rnd == "sr" else "")] = {
                    "sqnr_db": round(r["sqnr_db"], 3), "alpha": round(r["alpha"], 6),
                    "mean_shrink": float(f"{r['mean_shrink']:.4e}")}
        for fmt in ("e2m1", "e1m2"):
            e[f"{fmt}_rht_gain_db"] = round(e[f"{fmt}_random"]["sqnr_db"] - e[f"{fmt}_none"]["sqnr_db"], 3)
        d[name] = e
        del x
    res["llama_linear_operands_fp32_scale"] = d
    res["gemm_eta"] = bench_formats_gemm(U, S, torch, dev)
    return res


def bench_formats_gemm(U, S, torch, dev):
    """Attenuation eta = <Zq,Z>/<Z,Z> and output SQNR of the product of two
    quantized operands per format (full and range-capped E2M1, NVINT4 and
    E1M2 through the dequantize-to-bf16 GEMM, MXFP4 through the native one),
    against Z = A B^T of the bf16 operands, on the data of three workloads:
    the activation tensor's two 4096-row halves (K = 8192; NVFP4-style
    two-level scale, with and without RHT), the linear layer's forward GEMM
    X W^T (K = 4096; FP32 1x16 scale, RHT as in the UFP4 recipe) and the
    MXFP4/IF4 tensor's two 8192-row halves (K = 8192; two-level scale, no
    RHT).  Both operands of a product share the sign diagonal."""
    def dev_bf16(h):
        return torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(dev)

    fmts = ("e2m1", "e2m1_max4", "e2m1_max3", "e2m1_max2", "int4", "e1m2")
    out = {"note": "eta < 1: the product is shrunk; int4 with the E4M3 two-level scale is NVINT4, e2m1 NVFP4"}

    def run(a, b, scale, rhts, extra=()):
        z = U.ufp4_gemm_bf16(a, b)
        c = torch.empty_like(z)
        r = {}
        for rht in rhts:
            for fmt in fmts:
                cfg = U.Cfg(fmt, scale, rht=rht, rht_seed=0)
                qa, qb = U.ufp4_quantize(a, cfg), U.ufp4_quantize(b, cfg)
                U.ufp4_qgemm(qa, qb, "bf16", c=c)
                rep = U.ufp4_eta(c, z).cpu().numpy()
                r[f"{fmt}_{rht}"] = {"eta": round(float(rep[0] / rep[1]), 6),
                                     "sqnr_db": round(float(10 * np.log10(rep[1] / rep[2])), 3)}
            for name, cfg, mode in extra:
                qa, qb = U.ufp4_quantize(a, cfg), U.ufp4_quantize(b, cfg)
                U.ufp4_qgemm(qa, qb, mode, c=c)
                rep = U.ufp4_eta(c, z).cpu().numpy()
                r[name] = {"eta": round(float(rep[0] / rep[1]), 6),
                           "sqnr_db": round(float(10 * np.log10(rep[1] / rep[2])), 3)}
        return r

    x = dev_bf16(S.activations_t3(ROWS, COLS, seed=0))
    out["activations_halves_4096x4096x8192"] = run(
        x[:ROWS // 2], x[ROWS // 2:], "e4m3", ("none", "random"),
        (("mxfp4_rht", U.Cfg("e2m1", "e8m0", 32, rht="random", rht_seed=0), "mxfp4"),))
    del x
    xl, wl = dev_bf16(S.llama_x(16384, 4096)), dev_bf16(S.llama_w(14336, 4096))
    out["llama_fwd_y_16384x14336x4096"] = run(xl, wl, "fp32", ("random",))
    del xl, wl
    xh, _ = S.mx_if4(16384, 8192, seed=0)
    x = dev_bf16(xh)
    out["mxfp4_if4_halves_8192x8192x8192"] = run(
        x[:8192], x[8192:], "e4m3", ("none",),
        (("if4", U.Cfg("if4", "e4m3"), "bf16"), ("mxfp4_h16", U.Cfg("e2m1", "e8m0", 32, rht="det"), "mxfp4")))
    return out


if __name__ == "__main__":
    main()
