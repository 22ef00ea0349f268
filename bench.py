"""Benchmark: qsdpa_decode on the 64K-context 4-bit GQA-4 decode workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one qsdpa_decode call over the whole cache (B=1, Hq=32, Hk=8,
D=128, L=65536, affine 4-bit group 64, fp16): the query prologue, the
packed K/V stream with in-register dequantization, the online softmax and the
fused split merge.  Inputs are resident in HBM before the timed region.  The
quantized cache is replicated R times (R * bytes >= 512 MB, twice the MI355X
Infinity Cache) and step i reads copy i mod R, so every step streams its
bytes from HBM rather than from the memory-side cache.

Prints one JSON line.  ``value`` is the achieved algorithmic HBM bandwidth
(GB/s) of the whole step; ``roofline`` prices the decode kernel against the
8 TB/s HBM peak; ``cpu_baseline`` times the CPU oracle on a bounded sample of
the same workload.  Other workloads (``--workload``) are for exploration and
print the same record shape.
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

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, vendor figure
MFMA_F16_PEAK_TFLOPS = 2500.0    # dense fp16/bf16 matrix peak
MALL_BYTES = 256 * 2 ** 20
METRIC = "qsdpa_decode µs/step + achieved HBM GB/s (% peak), L=64K 4-bit GQA-4"
PROFILE_FILE = os.path.join(ROOT, "profiles", "decode_64k_4bit_gqa4_traffic.json")


def pack_bytes(w, L) -> int:
    """Algorithmic bytes of K and V packs over L tokens of every (b, kv head)."""
    rows = w.B * w.Hk * L
    if w.mode == "q8_0":
        per = w.D + 2 * (w.D // 32)
    else:
        ss = 4 if w.dtype == "f32" else 2
        per = w.D * w.bits // 8 + 2 * (w.D // w.group_size) * ss
    return 2 * rows * per


def qo_bytes(w, Lq=1) -> int:
    es = 4 if w.dtype == "f32" else 2
    return 2 * w.B * w.Hq * Lq * w.D * es


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_64k_4bit_gqa4")
    ap.add_argument("--algo", default="auto", choices=["auto", "generic", "matrix"])
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--copies", type=int, default=0, help="cache copies (0 = enough for 512 MB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


def make_caches(w, qkv, to_dev, copies):
    from quantized_kv_cache_amd import workloads as W
    inp = W.make_inputs(w)
    k = to_dev(inp["k"], w.dtype)
    v = to_dev(inp["v"], w.dtype)
    base_k = qkv.qkv_quantize(k, w.mode, w.bits, w.group_size)
    base_v = qkv.qkv_quantize(v, w.mode, w.bits, w.group_size)
    del k, v
    per = pack_bytes(w, w.L)
    R = copies or max(1, -(-2 * MALL_BYTES // per))
    ks, vs = [base_k], [base_v]
    for _ in range(R - 1):
        ks.append(clone_pack(qkv, base_k))
        vs.append(clone_pack(qkv, base_v))
    return inp, ks, vs, R


def clone_pack(qkv, p):
    return qkv.Pack(p.mode, p.bits, p.group_size, p.D, p.codes.clone(), p.scales.clone(),
                    None if p.biases is None else p.biases.clone())


def time_steps(torch, step, steps, warmup, stream):
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        step(warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps       # ms per step (one launch per decode step)


def cpu_baseline(w, inp, budget_s):
    """The oracle as it stands on this host: dequantize the packs and run the
    fp64 attention, repeated until about budget_s seconds have passed."""
    import oracle as orc
    from tests._cases import oracle_attention, oracle_pack
    kr = oracle_pack(inp["k"], w.dtype, w.mode, w.bits, w.group_size)
    vr = oracle_pack(inp["v"], w.dtype, w.mode, w.bits, w.group_size)
    q = inp["q"]
    n, t0 = 0, time.perf_counter()
    while True:
        oracle_attention(q, w.dtype, kr, vr, w.L, w.mode, w.bits, w.group_size, w.scale,
                         causal=w.causal)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 50:
            break
    sec = el / n
    gbs = (pack_bytes(w, w.L) + qo_bytes(w, w.Lq)) / sec / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"{n} full step(s) of {w.name} (dequantize K/V packs + fp64 attention), "
                      f"{sec * 1e3:.1f} ms per step"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; multi-GPU runs are not part "
                                   "of this build", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import quantized_kv_cache_amd as qkv
    from quantized_kv_cache_amd import workloads as W
    from tests._cases import to_dev

    w = W.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    inp, ks, vs, R = make_caches(w, qkv, to_dev, args.copies)
    q = to_dev(inp["q"], w.dtype)
    out = torch.empty_like(q)
    ws = qkv.Workspace()

    if w.Lq == 1:
        calls = [qkv.PreparedDecode(q, ks[i], vs[i], w.L, w.scale, out, num_splits=args.splits,
                                    algo=args.algo, workspace=ws) for i in range(R)]

        def step(i):
            calls[i % R]()
    else:
        def step(i):
            qkv.qsdpa_prefill(q, ks[i % R], vs[i % R], w.L, w.scale, causal=w.causal,
                              num_splits=args.splits, algo=args.algo, out=out, workspace=ws)

    ms = time_steps(torch, step, args.steps, args.warmup, stream)
    alg_bytes = pack_bytes(w, w.L) + qo_bytes(w, w.Lq)
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    plan = qkv.qsdpa_plan(q, ks[0], w.L, args.splits, args.algo)
    matrix = plan["algo"] == "matrix"
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
        "dtype": "f16" if matrix else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hk": w.Hk, "D": w.D, "L": w.L,
                   "Lq": w.Lq, "mode": w.mode, "bits": w.bits, "group_size": w.group_size,
                   "cache_dtype": w.dtype, "cache_copies": R, "algo": args.algo,
                   "kernel": plan["algo"], "num_splits": plan["num_splits"]},
    }
    if w.Lq == 1:
        traffic = None
        if os.path.exists(PROFILE_FILE) and w.name == "decode_64k_4bit_gqa4":
            prof = json.load(open(PROFILE_FILE))
            if prof.get("kernel_source_hash") == kernel_hash():
                traffic = prof.get("hbm_bytes_per_launch")
        rec["roofline"] = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                           "traffic": traffic, "algorithmic_bytes": alg_bytes}
    else:
        flops = prefill_flops(w)
        tf = flops / (ms * 1e-3) / 1e12
        rec["roofline"] = {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                           "traffic": None, "algorithmic_flops": flops}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def prefill_flops(w) -> int:
    """2 flops per multiply-add of QK^T and PV over the visible (query, key) pairs."""
    if w.causal:
        vis = sum(w.L - w.Lq + i + 1 for i in range(w.Lq))
    else:
        vis = w.Lq * w.L
    return 4 * w.B * w.Hq * vis * w.D


def kernel_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "quantized_kv_cache_amd", "csrc"))):
        h.update(open(os.path.join(ROOT, "quantized_kv_cache_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
