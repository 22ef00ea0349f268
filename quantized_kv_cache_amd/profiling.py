"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python -m quantized_kv_cache_amd.profiling stats STATS_CSV --command CMD
    python -m quantized_kv_cache_amd.profiling counters --kernel NAME --workload W \\
        --fetch CSV --write CSV --copy-fetch CSV --copy-write CSV --copy-bytes N \\
        --command CMD [--command CMD ...]

``stats`` prints the per-kernel duration table of a ``--kernel-trace --stats``
run (``*_kernel_stats.csv``).  ``counters`` reads four ``--pmc`` runs (FETCH_SIZE
and WRITE_SIZE of the workload, then of a plain device copy of N bytes),
scales the kernel's per-dispatch counter means by bytes-per-count of the copy
(which reads and writes N bytes), and prints ``key = value`` lines, among them
``hbm_bytes_per_launch`` and ``kernel_source_hash`` (the hash of the kernel's
source files, so that a stale reading is recognised).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import statistics

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# sources whose change invalidates a kernel's counter readings
KERNEL_SOURCES = {
    "attn_matrix_decode": ["qkv_attn_matrix.hip", "qkv_merge.hpp", "qkv_mfma.hpp", "qkv_device.hpp",
                           "qkv_internal.hpp"],
    "attn_decode_narrow": ["qkv_attn_narrow.hip", "qkv_merge.hpp", "qkv_mfma.hpp", "qkv_device.hpp",
                           "qkv_internal.hpp", "qkv_quant_math.hpp"],
    "attn_matrix_prefill": ["qkv_prefill_matrix.hip", "qkv_mfma.hpp", "qkv_device.hpp", "qkv_internal.hpp"],
    "attn_generic_kernel": ["qkv_attn_generic.hip", "qkv_device.hpp", "qkv_internal.hpp"],
    "merge_splits_kernel": ["qkv_merge.hip", "qkv_merge.hpp", "qkv_device.hpp", "qkv_internal.hpp"],
    "merge_splits_small": ["qkv_merge.hip", "qkv_merge.hpp", "qkv_device.hpp", "qkv_internal.hpp"],
    "quantize_rows_kernel": ["qkv_quantize.hip", "qkv_device.hpp", "qkv_internal.hpp", "qkv_quant_math.hpp"],
    "unfused_scores_kernel": ["qkv_unfused.hip", "qkv_device.hpp", "qkv_internal.hpp"],
    "attn_decode_stream": ["qkv_attn_stream.hip", "qkv_mfma.hpp", "qkv_device.hpp", "qkv_internal.hpp"],
}


def _code_only(text: str) -> str:
    """Source text without // comments, trailing blanks and empty lines (the
    counters describe the code, so comment edits do not invalidate them)."""
    out = []
    for line in text.split("\n"):
        i = line.find("//")
        if i >= 0:
            line = line[:i]
        line = line.rstrip()
        if line:
            out.append(line)
    return "\n".join(out)


def kernel_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(_code_only(open(os.path.join(CSRC, f)).read()).encode())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    """Kernel name without namespaces, template arguments and parameters."""
    base = name.replace("(anonymous namespace)", "").split("(")[0]
    depth, out = 0, []
    for ch in base:
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif depth == 0:
            out.append(ch)
    s = "".join(out).strip()
    return s.split("::")[-1].split(" ")[-1]


def trace_table(path: str, skip: int) -> str:
    """Per-kernel durations from a --kernel-trace CSV, leaving out each
    kernel's first `skip` dispatches (warm-up launches)."""
    per = {}
    for r in csv.DictReader(open(path)):
        name = short_name(r["Kernel_Name"])
        per.setdefault(name, []).append((int(r["Dispatch_Id"]),
                                         (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    total = sum(d for v in per.values() for _, d in sorted(v)[skip:])
    lines = [f"{'kernel':<34} {'calls':>6} {'avg_us':>10} {'median_us':>10} {'min_us':>10} "
             f"{'max_us':>10} {'pct':>6}"]
    for name, v in sorted(per.items(), key=lambda kv: -sum(d for _, d in sorted(kv[1])[skip:])):
        ds = [d for _, d in sorted(v)[skip:]]
        if not ds:
            continue
        lines.append(f"{name[:34]:<34} {len(ds):>6} {statistics.fmean(ds):>10.3f} "
                     f"{statistics.median(ds):>10.3f} {min(ds):>10.3f} {max(ds):>10.3f} "
                     f"{100.0 * sum(ds) / total:>6.2f}")
    return "\n".join(lines)


def stats_table(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    lines = [f"{'kernel':<34} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}"]
    for r in rows:
        lines.append(f"{short_name(r['Name'])[:34]:<34} {int(r['Calls']):>6} "
                     f"{float(r['AverageNs']) / 1e3:>10.3f} {float(r['MinNs']) / 1e3:>10.3f} "
                     f"{float(r['MaxNs']) / 1e3:>10.3f} {float(r['Percentage']):>6.2f}")
    return "\n".join(lines)


def counter_means(path: str, counter: str) -> dict:
    """Mean per-dispatch value of `counter` for each kernel short name."""
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(short_name(r["Kernel_Name"]), {}).setdefault(r["Dispatch_Id"], 0.0)
        per[short_name(r["Kernel_Name"])][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: (statistics.fmean(v.values()), len(v)) for k, v in per.items()}


def copy_kernel_mean(path: str, counter: str) -> float:
    """Counter mean of the copy dispatches (the largest elementwise kernel)."""
    means = counter_means(path, counter)
    cands = {k: v for k, v in means.items() if "elementwise" in k or "copy" in k.lower()}
    name = max(cands, key=lambda k: cands[k][0])
    return cands[name][0]


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--command", action="append", default=[])
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("--skip", type=int, default=10)
    t.add_argument("--command", action="append", default=[])
    b = sub.add_parser("counters")
    for k in ("kernel", "workload", "fetch", "write", "copy_fetch", "copy_write"):
        b.add_argument("--" + k.replace("_", "-"), required=True)
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--command", action="append", default=[])
    b.add_argument("--dram", help="--pmc TCC_EA0_RDREQ_DRAM TCC_EA0_WRREQ_DRAM run of the workload")
    b.add_argument("--copy-dram", help="the same counters for the copy")
    b.add_argument("--sq", help="--pmc run of SQ/GRBM counters (MFMA, LDS, VALU activity)")
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        print("# rocprofv3 kernel durations")
        for c in args.command:
            print(f"# command: {c}")
        print(stats_table(args.csv))
        return
    if args.cmd == "trace":
        print(f"# rocprofv3 kernel durations, steady state (each kernel's first {args.skip} "
              f"dispatches left out)")
        for c in args.command:
            print(f"# command: {c}")
        print(trace_table(args.csv, args.skip))
        return
    fetch = counter_means(args.fetch, "FETCH_SIZE")
    write = counter_means(args.write, "WRITE_SIZE")
    k = args.kernel
    f_kib, nf = fetch[k]
    w_kib, nw = write[k]
    cf = copy_kernel_mean(args.copy_fetch, "FETCH_SIZE")
    cw = copy_kernel_mean(args.copy_write, "WRITE_SIZE")
    f_scale = args.copy_bytes / cf          # bytes per FETCH_SIZE count
    w_scale = args.copy_bytes / cw
    hbm = f_kib * f_scale + w_kib * w_scale
    print(f"# HBM traffic of {k} on the {args.workload} workload (rocprofv3 --pmc)")
    for c in args.command:
        print(f"# command: {c}")
    print(f"kernel = {k}")
    print(f"workload = {args.workload}")
    print(f"dispatches = {nf}")
    print(f"fetch_size_kib_per_dispatch = {f_kib:.1f}")
    print(f"write_size_kib_per_dispatch = {w_kib:.1f}")
    print(f"copy_bytes = {args.copy_bytes}")
    print(f"copy_fetch_size_kib = {cf:.1f}")
    print(f"copy_write_size_kib = {cw:.1f}")
    print(f"fetch_bytes_per_count = {f_scale:.4f}")
    print(f"write_bytes_per_count = {w_scale:.4f}")
    print(f"fetch_bytes_per_launch = {f_kib * f_scale:.0f}")
    print(f"write_bytes_per_launch = {w_kib * w_scale:.0f}")
    print(f"hbm_bytes_per_launch = {hbm:.0f}")
    if args.dram and args.copy_dram:
        # requests the L2 sends to the memory side (DRAM or its memory-side
        # cache), per dispatch, scaled by bytes per request of the copy
        rd = counter_means(args.dram, "TCC_EA0_RDREQ_DRAM")[k][0]
        wr = counter_means(args.dram, "TCC_EA0_WRREQ_DRAM")[k][0]
        crd = copy_kernel_mean(args.copy_dram, "TCC_EA0_RDREQ_DRAM")
        cwr = copy_kernel_mean(args.copy_dram, "TCC_EA0_WRREQ_DRAM")
        print(f"dram_read_requests_per_dispatch = {rd:.0f}")
        print(f"dram_write_requests_per_dispatch = {wr:.0f}")
        print(f"dram_read_bytes_per_request = {args.copy_bytes / crd:.2f}")
        print(f"dram_write_bytes_per_request = {args.copy_bytes / cwr:.2f}")
        print(f"dram_read_bytes_per_launch = {rd * args.copy_bytes / crd:.0f}")
        print(f"dram_write_bytes_per_launch = {wr * args.copy_bytes / cwr:.0f}")
    if args.sq:
        for cname in ("SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES",
                      "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU",
                      "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT"):
            m = counter_means(args.sq, cname).get(k)
            if m is not None:
                print(f"{cname.lower()}_per_dispatch = {m[0]:.0f}")
    print(f"kernel_source_hash = {kernel_hash(k)}")


if __name__ == "__main__":
    main()
