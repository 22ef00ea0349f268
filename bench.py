"""Benchmark of the quantized-KV attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: qsdpa_decode over the 64K-context 4-bit GQA-4 cache (B=1,
Hq=32, Hk=8, D=128, L=65536, affine 4-bit group 64, fp16; the shape of the
MLX benchmark on the page "add fast::quantized_kv_update").  A step is one
decode call: the attention kernel (packed K/V streamed once, dequantized in
registers, online softmax per key split) and the split merge kernel.

Other workloads (``--workload``): tiny_decode, append_decode_b8_8bit (a step
appends a token per sequence and decodes over the grown cache: one
qsdpa_decode_append call, or qkv_update_append and qsdpa_decode with
``--separate-append``), q8_0_decode_gqa16 and q8_0_prefill_512 (one causal
prefill).

Inputs are resident in HBM before the timed region.  The quantized cache is
replicated R times (R * bytes >= twice the 256 MB Infinity Cache, at most 64
copies) and step i reads copy i mod R, so each step streams its bytes from
HBM rather than from the memory-side cache.

Prints one JSON line:
  value          algorithmic bytes of a step / time per step (GB/s)
  roofline       the dominant kernel (the attention kernel) alone: its
                 algorithmic bytes (decode) or flops (prefill) per launch over
                 its mean duration, timed with HIP events that the library
                 records on its stream around that kernel, in a second pass
                 of the same number of steps; traffic = HBM bytes per launch
                 from rocprofv3 counters (profiles/*.counters.txt) while the
                 kernel source is unchanged since they were taken, else null
  cpu_baseline   the CPU oracle timed on a bounded sample of the workload
  read_ceiling   a plain streaming read (include/qkv_measure.h) in the same job:
                 of the step's K/V pack bytes, rotating over as many buffers as
                 there are cache copies, and of one 1 GiB buffer (each the best
                 of 256 ... 8192 workgroups); step_frac is the attention
                 kernel's rate over the same-size read's
  latency_us     single calls, each after a 512 MB write that evicts the
                 Infinity Cache: p10 / median / p90 over 50 calls
                 (``--no-extras`` skips these two, for profiled runs)
``--graph`` times one replay of a HIP graph that captured the timed steps'
calls instead of the calls themselves (config.launch says which).
``--copy-mib N`` instead runs a plain N MiB device copy ``--steps`` times (the
known-size kernel the counter readings are scaled by).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, vendor figure
MFMA_F16_PEAK_TFLOPS = 2500.0    # dense fp16/bf16 matrix peak, vendor figure
MALL_BYTES = 256 * 2 ** 20
MAX_COPIES = 64
METRIC = "qsdpa_decode µs/step + achieved HBM GB/s (% peak), L=64K 4-bit GQA-4"


def pack_bytes(w, L) -> int:
    """Algorithmic bytes of the K and V packs over L tokens of every (b, kv head)."""
    rows = w.B * w.Hk * L
    if w.mode == "dense":
        return 2 * rows * w.D * 2
    if w.mode == "q8_0":
        per = w.D + 2 * (w.D // 32)
    elif w.mode == "qsym":
        per = w.D * w.bits // 8 + 2 * (w.D // 32)
    else:
        ss = 4 if w.dtype == "f32" else 2
        per = w.D * w.bits // 8 + 2 * (w.D // w.group_size) * ss
    return 2 * rows * per


def q_bytes(w, Lq=1) -> int:
    return w.B * w.Hq * Lq * w.D * (4 if w.dtype == "f32" else 2)


def append_bytes(w) -> int:
    """One token per (b, kv head): fp16 K and V read, their packed rows written."""
    return 2 * w.B * w.Hk * w.D * 2 + pack_bytes(w, 1)


def prefill_flops(w) -> int:
    """2 flops per multiply-add of QK^T and PV over the visible (query, key) pairs."""
    if w.causal:
        vis = sum(w.L - w.Lq + i + 1 for i in range(w.Lq))
    else:
        vis = w.Lq * w.L
    return 4 * w.B * w.Hq * vis * w.D


def counters_path(kernel: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}.{workload}.counters.txt")


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel's sources changed since it was taken."""
    path = counters_path(kernel, workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    from quantized_kv_cache_amd.profiling import kernel_hash
    if kv.get("kernel_source_hash") != kernel_hash(kernel):
        return None
    return int(float(kv["hbm_bytes_per_launch"]))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_64k_4bit_gqa4")
    ap.add_argument("--algo", default="auto",
                    choices=["auto", "generic", "matrix", "unfused", "dequant_f16"],
                    help="kernel choice; 'unfused' times the four-kernel composition and also "
                         "the fused decode of the same workload in the same job")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--copies", type=int, default=0, help="cache copies (0 = enough for 512 MB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip read_ceiling and latency_us (profiled runs: only the timed steps "
                         "and the kernel pass launch the attention kernel)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-mib", type=int, default=0)
    ap.add_argument("--op", default="attention", choices=["attention", "quantize"],
                    help="'quantize' times qkv_quantize of the workload's K and V caches "
                         "(alternating) instead of the attention step")
    ap.add_argument("--separate-append", action="store_true",
                    help="append workload: qkv_update_append and qsdpa_decode as two calls per step "
                         "instead of qsdpa_decode_append")
    ap.add_argument("--graph", action="store_true",
                    help="time one replay of a HIP graph that captured the timed steps' calls "
                         "(the same kernels without the per-call host path and launch gaps)")
    ap.add_argument("--read-sweep", action="store_true",
                    help="instead: the plain streaming read of the workload's K/V bytes over a "
                         "grid of load shapes (workgroups, threads, loads in flight, width)")
    return ap.parse_args()


def clone_pack(qkv, p):
    return qkv.Pack(p.mode, p.bits, p.group_size, p.D, p.codes.clone(),
                    None if p.scales is None else p.scales.clone(),
                    None if p.biases is None else p.biases.clone())


def make_caches(w, qkv, W, copies):
    inp = W.make_inputs(w)
    k = W.to_tensor(inp["k"], w.dtype)
    v = W.to_tensor(inp["v"], w.dtype)
    base_k = qkv.qkv_quantize(k, w.mode, w.bits, w.group_size, L_cap=w.cap)
    base_v = qkv.qkv_quantize(v, w.mode, w.bits, w.group_size, L_cap=w.cap)
    del k, v
    per = pack_bytes(w, w.cap)
    R = copies or min(MAX_COPIES, max(1, -(-2 * MALL_BYTES // per)))
    ks, vs = [base_k], [base_v]
    for _ in range(R - 1):
        ks.append(clone_pack(qkv, base_k))
        vs.append(clone_pack(qkv, base_v))
    return inp, ks, vs, R


def time_region(torch, run, first, steps, stream):
    """ms per step over `steps` calls of run(i), bracketed by events."""
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(first, first + steps):
        run(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def graph_region(torch, run, first, steps, stream):
    """ms per step over one replay of a graph that captured run(i) for the
    `steps` values of i, after one untimed replay."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        for i in range(first, first + steps):
            run(i)
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def kernel_pass(torch, run, attn_of, first, steps, stream):
    """Mean duration (ms) of the attention kernel over `steps` calls, from
    events the library records on its stream right around that kernel."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:            # create the HIP events before handing them over
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for n, i in enumerate(range(first, first + steps)):
        call = attn_of(i)
        call.set_timing(*evs[n])
        run(i)
        call.set_timing(None, None)
    torch.cuda.synchronize()
    d = [a.elapsed_time(b) for a, b in evs]
    return sum(d) / len(d)


def read_ceiling(torch, nbytes, copies, steps, stream):
    """Time a plain streaming read (include/qkv_measure.h) of nbytes per step,
    rotating over 'copies' buffers as the benchmark rotates over cache copies,
    and of one 1 GiB buffer, each with the best of a few workgroup counts.
    Returns (ms per same-size read, ms per 1 GiB read, their workgroups)."""
    import ctypes
    from quantized_kv_cache_amd import _lib
    lib = _lib.load()
    n16 = (nbytes + 15) // 16 * 16
    bufs = [torch.ones(n16, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    big = torch.ones(2 ** 30, dtype=torch.uint8, device="cuda")
    sink = torch.empty(4 * 8192, dtype=torch.int32, device="cuda")
    sp = ctypes.c_void_p(stream.cuda_stream)

    def rd(t, wgs):
        st = lib.qkv_measure_read(ctypes.c_void_p(t.data_ptr()), t.numel(), wgs,
                                  ctypes.c_void_p(sink.data_ptr()), sp)
        if st != _lib.QKV_OK:
            raise RuntimeError(lib.qkv_last_error().decode())

    def best(run_one, n, reps):
        res = []
        for wgs in (256, 512, 1024, 2048, 4096, 8192):
            for i in range(n):
                run_one(i, wgs)
            res.append((time_region(torch, lambda i: run_one(i, wgs), 0, reps, stream), wgs))
        return min(res)
    ms, wg = best(lambda i, g: rd(bufs[i % copies], g), 2 * copies, steps)
    ms_big, wg_big = best(lambda i, g: rd(big, g), 3, 20)
    del bufs, big
    return ms, ms_big, wg, wg_big


def read_sweep(torch, w, copies, steps):
    """The plain streaming read (qkv_measure_read_config) of the workload's
    per-step K/V pack bytes, rotating over 'copies' buffers, for every load
    shape of a grid; prints one line per shape, fastest first."""
    import ctypes
    from quantized_kv_cache_amd import _lib
    lib = _lib.load()
    stream = torch.cuda.current_stream()
    nbytes = (pack_bytes(w, w.L) + 15) // 16 * 16
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sink = torch.empty(8192 * 16, dtype=torch.int32, device="cuda")
    sp = ctypes.c_void_p(stream.cuda_stream)
    rows = []
    for width in (16, 8, 4):
        for threads in (256, 512, 1024):
            for u in (1, 2, 4, 8, 16):
                for wgs in (256, 512, 1024, 2048, 4096, 8192):
                    def rd(i, wgs=wgs, threads=threads, u=u, width=width):
                        t = bufs[i % copies]
                        st = lib.qkv_measure_read_config(ctypes.c_void_p(t.data_ptr()), nbytes, wgs,
                                                         threads, u, width,
                                                         ctypes.c_void_p(sink.data_ptr()), sp)
                        if st != _lib.QKV_OK:
                            raise RuntimeError(lib.qkv_last_error().decode())
                    for i in range(copies):
                        rd(i)
                    ms = time_region(torch, rd, 0, steps, stream)
                    rows.append((ms * 1e3, wgs, threads, u, width))
        print(f"# width {width} done", flush=True)
    rows.sort()
    print(f"# plain read of {nbytes} bytes per launch ({w.name} K/V packs), rotating over "
          f"{copies} buffers, {steps} launches per shape; us per launch and TB/s")
    print(f"{'us':>8} {'TB/s':>6} {'frac_8TB':>8} {'wgs':>5} {'threads':>7} {'in_flight':>9} {'width':>5}")
    for us, wgs, threads, u, width in rows:
        print(f"{us:8.2f} {nbytes / us / 1e6:6.3f} {nbytes / us / 1e6 / 8.0:8.3f} {wgs:5d} {threads:7d} "
              f"{u:9d} {width:5d}")


def call_latency(torch, run, first, n, stream):
    """n single steps, each after a 512 MB write (evicts the Infinity Cache),
    bracketed by their own events: p10, median and p90 in microseconds."""
    scrub = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for k in range(n):
        scrub.fill_(k & 255)
        a, b = evs[k]
        a.record(stream)
        run(first + k)
        b.record(stream)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return {"p10": round(us[n // 10], 2), "median": round(us[n // 2], 2),
            "p90": round(us[(9 * n) // 10], 2), "calls": n, "scrub_mib": 512}


def cpu_baseline(w, inp, budget_s):
    """The oracle as it stands on this host on a bounded sample of the
    workload: full steps (quantize-append the step's token, dequantize the
    packs, fp64 attention) repeated until about budget_s seconds have
    passed (a prefill step runs a bounded number of query positions)."""
    import numpy as np
    import oracle as orc
    from tests._cases import oracle_attention, oracle_pack
    from quantized_kv_cache_amd import workloads as W
    if w.mode == "dense":
        # the unquantized cache: fp64 attention over its fp16 values
        n, t0 = 0, time.perf_counter()
        while True:
            orc.attention(orc.to_f32(inp["q"], w.dtype), orc.to_f32(inp["k"], w.dtype),
                          orc.to_f32(inp["v"], w.dtype), w.scale)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s or n >= 50:
                break
        sec = el / n
        alg = pack_bytes(w, w.L) + 2 * q_bytes(w)
        return {"value": round(alg / sec / 1e9, 4), "unit": "GB/s", "cores": orc.num_threads(),
                "kind": "oracle",
                "sample": f"{n} x decode step of {w.name}, {sec * 1e3:.1f} ms each; the same "
                          f"algorithmic bytes per unit of work as the GPU figure"}
    kr = oracle_pack(inp["k"], w.dtype, w.mode, w.bits, w.group_size)
    vr = oracle_pack(inp["v"], w.dtype, w.mode, w.bits, w.group_size)
    q, L, mask, causal = inp["q"], w.L, None, w.causal
    what = "decode step"
    if w.Lq > 1:
        # the prefill on its last 16 query positions, with the causal rule as a mask
        idx = np.arange(w.Lq - 16, w.Lq)
        q = np.ascontiguousarray(q[:, :, idx])
        j = np.arange(L)[None, :]
        mask = np.where(j > (L - w.Lq + idx)[:, None], -np.inf, 0.0).astype(np.float32)[None, None]
        causal = False
        what = f"16 of the {w.Lq} query positions of the prefill"
    rng = np.random.default_rng(w.seed + 1)
    n, t0, work = 0, time.perf_counter(), 0.0
    while True:
        if w.steps:
            s = W.append_step_inputs(w, rng)
            kn = oracle_pack(s["k_new"], w.dtype, w.mode, w.bits, w.group_size)
            vn = oracle_pack(s["v_new"], w.dtype, w.mode, w.bits, w.group_size)
            kr2 = {k: None if a is None else np.concatenate([a, kn[k]], axis=2) for k, a in kr.items()}
            vr2 = {k: None if a is None else np.concatenate([a, vn[k]], axis=2) for k, a in vr.items()}
            oracle_attention(s["q"], w.dtype, kr2, vr2, L + 1, w.mode, w.bits, w.group_size,
                             w.scale)
            what = "append+decode step"
        else:
            oracle_attention(q, w.dtype, kr, vr, L, w.mode, w.bits, w.group_size, w.scale,
                             mask=mask, causal=causal)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 50:
            break
    sec = el / n
    if w.Lq > 1:
        frac = 16.0 / w.Lq   # bytes of the sampled part of the step
        alg = (pack_bytes(w, w.L) + 2 * q_bytes(w, w.Lq)) * frac
    else:
        alg = pack_bytes(w, w.L) + 2 * q_bytes(w) + (append_bytes(w) if w.steps else 0)
    return {"value": round(alg / sec / 1e9, 4), "unit": "GB/s", "cores": orc.num_threads(),
            "kind": "oracle",
            "sample": f"{n} x {what} of {w.name}, {sec * 1e3:.1f} ms each; the same "
                      f"algorithmic bytes per unit of work as the GPU figure"}


def quantize_mode(args, w, torch, qkv, W, stream):
    """qkv_quantize of the workload's K and V (fp16/fp32 [B,Hk,L,D] -> packs),
    alternating, back to back: the bytes read and written per call over its
    time, against the HBM peak.  The sources and packs are copied until a
    rotation holds at least 512 MB (twice the Infinity Cache), so each call
    reads and writes HBM."""
    inp = W.make_inputs(w)
    xs = [W.to_tensor(inp["k"], w.dtype), W.to_tensor(inp["v"], w.dtype)]
    src = xs[0].numel() * xs[0].element_size()
    dst = pack_bytes(w, w.L) // 2
    pairs = max(1, min(32, -(-512 * 2 ** 20 // (2 * (src + dst)))))
    calls = []
    for _ in range(pairs):
        for x in xs:
            xc = x.clone()
            calls.append(qkv.PreparedQuantize(xc, qkv.qkv_quantize(xc, w.mode, w.bits, w.group_size)))
    n = len(calls)
    for i in range(args.warmup):
        calls[i % n]()
    ms = time_region(torch, lambda i: calls[i % n](), 0, args.steps, stream)
    gbs = (src + dst) / (ms * 1e-3) / 1e9
    print(json.dumps({"metric": f"qkv_quantize {w.name} K/V GB/s (read + written)", "value": round(gbs, 1),
                      "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "us_per_call": round(ms * 1e3, 3), "bytes_read": src, "bytes_written": dst,
                      "rotation": n,
                      "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                   "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                   "kernel": "quantize_rows_kernel"},
                      "config": {"workload": w.name, "mode": w.mode, "bits": w.bits,
                                 "group_size": w.group_size, "dtype": w.dtype}}), flush=True)


def copy_mode(args):
    import torch
    n = args.copy_mib * 2 ** 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    stream = torch.cuda.current_stream()
    ms = time_region(torch, lambda i: dst.copy_(src), 0, args.steps, stream)
    print(json.dumps({"copy_bytes": n, "steps": args.steps, "ms_per_copy": round(ms, 5),
                      "GB/s": round(2 * n / ms / 1e6, 1)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; runs on several GPUs are "
                                   "not supported", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    if args.copy_mib:
        return copy_mode(args)
    import torch
    import quantized_kv_cache_amd as qkv
    from quantized_kv_cache_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    if args.graph:
        # a graph is captured on a stream other than the legacy default one: every
        # call below is marshalled on this one
        torch.cuda.set_stream(torch.cuda.Stream())
    stream = torch.cuda.current_stream()
    if args.read_sweep:
        per = pack_bytes(w, w.cap)
        R = args.copies or min(MAX_COPIES, max(1, -(-2 * MALL_BYTES // per)))
        return read_sweep(torch, w, R, args.steps)
    if args.op == "quantize":
        return quantize_mode(args, w, torch, qkv, W, stream)
    inp, ks, vs, R = make_caches(w, qkv, W, args.copies)
    ws = qkv.Workspace()

    if w.steps:
        # append + decode: step i appends one token per sequence at L + t and attends
        # L + t + 1 keys (t = i mod steps), on cache copy i mod R
        rng = inp["rng"]
        per_step = [W.append_step_inputs(w, rng) for _ in range(w.steps)]
        kn = [W.to_tensor(s["k_new"], w.dtype) for s in per_step]
        vn = [W.to_tensor(s["v_new"], w.dtype) for s in per_step]
        qs = [W.to_tensor(s["q"], w.dtype) for s in per_step]
        out = torch.empty_like(qs[0])
        if args.separate_append:
            # qkv_update_append, then qsdpa_decode: two launches per step
            appends = [[qkv.PreparedAppend(ks[c], vs[c], kn[t], vn[t]) for t in range(w.steps)]
                       for c in range(R)]
            calls = [[qkv.PreparedAttention(qs[t], ks[c], vs[c], w.L + t + 1, w.scale, out,
                                            num_splits=args.splits, algo=args.algo, workspace=ws)
                      for t in range(w.steps)] for c in range(R)]

            def run(i):
                t = i % w.steps
                appends[i % R][t](w.L + t)
                calls[i % R][t]()
        else:
            # qsdpa_decode_append: the append and the decode in one call
            calls = [[qkv.PreparedDecodeAppend(qs[t], ks[c], vs[c], kn[t], vn[t], w.L + t, w.scale, out,
                                               num_splits=args.splits, algo=args.algo, workspace=ws)
                      for t in range(w.steps)] for c in range(R)]

            def run(i):
                calls[i % R][i % w.steps]()

        def attn_of(i):
            return calls[i % R][i % w.steps]
        L_mean = w.L + (w.steps + 1) / 2.0
        step_bytes = pack_bytes(w, L_mean) + 2 * q_bytes(w) + append_bytes(w)
        plan_L = w.L + w.steps
        q0 = qs[0]
    else:
        q0 = W.to_tensor(inp["q"], w.dtype)
        out = torch.empty_like(q0)
        calls = [qkv.PreparedAttention(q0, ks[c], vs[c], w.L, w.scale, out, causal=w.causal,
                                       num_splits=args.splits, algo=args.algo, workspace=ws)
                 for c in range(R)]

        def attn_of(i):
            return calls[i % R]

        def run(i):
            calls[i % R]()
        step_bytes = pack_bytes(w, w.L) + 2 * q_bytes(w, w.Lq)
        plan_L = w.L

    for i in range(args.warmup):
        run(i)
    if args.graph:
        ms = graph_region(torch, run, args.warmup, args.steps, stream)
        last = args.warmup + args.steps - 1
        got = out.clone()
        run(last)                         # the graph's last call, eagerly
        torch.cuda.synchronize()
        if not torch.equal(got, out):
            sys.exit("bench: the graph replay's output differs from the eager call's")
    else:
        ms = time_region(torch, run, args.warmup, args.steps, stream)

    plan = qkv.qsdpa_plan(q0, ks[0], plan_L, args.splits, args.algo)
    kernel = plan["kernel"]
    if kernel == "attn_decode_narrow" or plan["num_splits"] == 1:
        # the attention call is one kernel launch: its mean duration is the time of a
        # back-to-back pass of the calls alone (for the append workload: the same
        # calls, on the caches the timed pass left; the one-call form rewrites the
        # step's row with the same bits)
        kms = time_region(torch, lambda i: attn_of(i)(), args.warmup + args.steps, args.steps, stream)
    else:
        kms = kernel_pass(torch, run, attn_of, args.warmup + args.steps, args.steps, stream)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    rec = {
        "metric": METRIC if w.name == "decode_64k_4bit_gqa4" else f"{w.name} achieved GB/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 3),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if plan["algo"] in ("matrix", "dequant_f16") else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hk": w.Hk, "D": w.D, "L": w.L,
                   "Lq": w.Lq, "mode": w.mode, "bits": w.bits, "group_size": w.group_size,
                   "cache_dtype": w.dtype, "cache_copies": R, "algo": args.algo,
                   "kernel": kernel, "num_splits": plan["num_splits"]},
    }
    rec["config"]["launch"] = "graph replay" if args.graph else "eager calls"
    if w.steps:
        rec["config"]["append"] = "separate launch" if args.separate_append else "in the decode call"
    traffic = stored_traffic(kernel, w.name)
    if w.Lq == 1:
        # per launch: the K/V pack bytes of the attended keys, q, and out when unsplit
        kb = pack_bytes(w, w.L if not w.steps else L_mean) + q_bytes(w) * (
            1 if plan["num_splits"] > 1 else 2)
        if w.steps and not args.separate_append:
            kb += append_bytes(w)          # the kernel also reads the new tokens and writes their rows
        ach = kb / (kms * 1e-3) / 1e9
        rec["roofline"] = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                           "traffic": traffic, "kernel": kernel,
                           "kernel_us": round(kms * 1e3, 3), "algorithmic_bytes": int(kb)}
    else:
        flops = prefill_flops(w)
        tf = flops / (kms * 1e-3) / 1e12
        rec["roofline"] = {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                           "traffic": traffic, "kernel": kernel,
                           "kernel_us": round(kms * 1e3, 3), "algorithmic_flops": flops}
    if args.algo == "unfused" and not w.steps:
        # the fused decode of the same inputs, timed the same way in this job
        fused = [qkv.PreparedAttention(q0, ks[c], vs[c], w.L, w.scale, torch.empty_like(q0),
                                       causal=w.causal, workspace=ws) for c in range(R)]
        for i in range(args.warmup):
            fused[i % R]()
        fms = time_region(torch, lambda i: fused[i % R](), 0, args.steps, stream)
        rec["vs_fused"] = {"fused_us_per_step": round(fms * 1e3, 3),
                           "fused_kernel": qkv.qsdpa_plan(q0, ks[0], w.L)["kernel"],
                           "unfused_over_fused": round(ms / fms, 3)}
    if not args.no_extras:
        rd_ms, big_ms, rd_wg, big_wg = read_ceiling(torch, pack_bytes(w, w.L), R, args.steps, stream)
        rd_gbs = pack_bytes(w, w.L) / (rd_ms * 1e-3) / 1e9
        rec["read_ceiling"] = {"step_bytes_GBps": round(rd_gbs, 1),
                               "GiB_GBps": round(2 ** 30 / (big_ms * 1e-3) / 1e9, 1),
                               "step_bytes": pack_bytes(w, w.L), "step_us": round(rd_ms * 1e3, 3),
                               "workgroups": [rd_wg, big_wg]}
        if w.Lq == 1:
            rec["read_ceiling"]["step_frac"] = round(rec["roofline"]["achieved"] / rd_gbs, 4)
        rec["latency_us"] = call_latency(torch, run, 2 * (args.warmup + args.steps), 50, stream)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
