"""HBM traffic of the decode-attention kernel from rocprofv3 counters.

Two counter passes over the same program, one with FETCH_SIZE and one with WRITE_SIZE
(the counters cannot share a pass), give KiB per dispatch.  The program runs a plain device
copy of a known size (hipMemcpy device to device, 1 GiB) before every attention launch.  The
copy calibrates the counters: factor = bytes copied / counter bytes.  It also evicts the
L2 and infinity cache between attention launches.

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o run -- \\
        python3 -m kv_cache_bit_quantize_amd.traffic run --workload long-128k
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -o run -- \\
        python3 -m kv_cache_bit_quantize_amd.traffic run --workload long-128k
    python3 -m kv_cache_bit_quantize_amd.traffic summarize OUT/fetch/run_counter_collection.csv \\
        OUT/write/run_counter_collection.csv --out profiles/decode_attn_long-128k_counters

The summary gives the attention kernel's HBM bytes per launch next to its algorithmic
bytes, and records the hash of the kernel sources it was taken on.  `counters` summarizes other
counter runs of the attention kernels, `trace` a kernel-trace run of bench.py.
"""
import argparse
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 1 << 30
COPY_KERNEL = "copyBuffer"
# every file that shapes the decode-attention kernels' code
KERNEL_SOURCES = ["kv_cache_bit_quantize_amd/csrc/kivi_attn.hip", "kv_cache_bit_quantize_amd/csrc/kivi_attn_gqa.hip",
                  "kv_cache_bit_quantize_amd/csrc/kivi_attn_common.h", "kv_cache_bit_quantize_amd/csrc/kivi_device.h",
                  "kv_cache_bit_quantize_amd/csrc/kivi_internal.h", "kv_cache_bit_quantize_amd/build.py"]


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def run(args):
    import torch
    sys.path.insert(0, ROOT)
    from kv_cache_bit_quantize_amd import kivi, synth

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    k, v = synth.prefill_kv(w, device=dev)
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, device=dev)
    kivi.kivi_prefill(k, v, w.n_quant, cache)
    del k, v
    if cache.state[1] + args.launches > w.residual_cap:
        raise SystemExit("the launches would flush a group; use fewer")
    tokens = [synth.step_kv(w, s, device=dev) for s in range(args.launches)]
    queries = [synth.query(w, step=s + 1, device=dev) for s in range(args.launches)]
    out = torch.empty_like(queries[0])
    ws = cache.workspace(w.q_heads)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    rows = w.batch * w.kv_heads
    algo = 0
    for s in range(args.launches):
        dst.copy_(src)
        # one fused decode step (no flush): the new token is read, attended and stored
        kivi.kivi_decode_step(cache, *tokens[s], queries[s], synth.SM_SCALE_D128, out=out, workspace=ws)
        n_quant, n_res, _ = cache.state
        algo += rows * (n_quant * 96 + n_res * 512 + 2 * 512) + 2 * w.batch * w.q_heads * 128 * 2
    torch.cuda.synchronize()
    algo //= args.launches
    with open(args.meta, "w") as f:
        json.dump({"workload": w.name, "algorithmic_bytes_per_launch": algo, "launches": args.launches,
                   "kernel_source_hash": kernel_source_hash()}, f)
    print(f"ran {args.launches} copies of {COPY_BYTES} B and fused decode steps on {w.name}", flush=True)


def _per_dispatch(path, counter):
    """{kernel name: [counter value per dispatch]} from a rocprofv3 counter_collection csv."""
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            rows.setdefault((r["Dispatch_Id"], r["Kernel_Name"], r["Grid_Size"]), 0.0)
            rows[(r["Dispatch_Id"], r["Kernel_Name"], r["Grid_Size"])] += float(r["Counter_Value"])
    by_kernel = {}
    for (_, name, grid), val in rows.items():
        by_kernel.setdefault((name, int(grid)), []).append(val)
    return by_kernel


def summarize(args):
    meta = json.load(open(args.meta))
    result = {"workload": meta["workload"], "kernel_source_hash": meta["kernel_source_hash"],
              "algorithmic_bytes_per_launch": meta["algorithmic_bytes_per_launch"]}
    total = 0.0
    for counter, path in (("FETCH_SIZE", args.fetch_csv), ("WRITE_SIZE", args.write_csv)):
        k = _per_dispatch(path, counter)
        copies = [v for (name, grid), vals in k.items() if COPY_KERNEL in name for v in vals]
        # the calibration copies are the largest copy dispatches
        big = sorted(copies)[-meta["launches"]:]
        attn = [v for (name, grid), vals in k.items() if "attn_" in name and "kernel" in name for v in vals]
        if not big or not attn:
            raise SystemExit(f"{counter}: no copy or attention dispatches in {path}")
        copy_kib = sum(big) / len(big)
        attn_kib = sum(attn) / len(attn)
        # a copy reads and writes COPY_BYTES; the counter's reading of it fixes the scale
        factor = COPY_BYTES / (copy_kib * 1024.0)
        nbytes = attn_kib * 1024.0 * factor
        result[counter] = {"attn_kib_per_dispatch": attn_kib, "copy_kib_per_dispatch": copy_kib,
                           "copy_bytes": COPY_BYTES, "scale": factor, "attn_bytes_per_launch": nbytes,
                           "attn_dispatches": len(attn)}
        total += nbytes
    result["hbm_bytes_per_launch"] = total
    result["traffic_over_algorithmic"] = total / meta["algorithmic_bytes_per_launch"]
    with open(args.out + ".json", "w") as f:
        json.dump(result, f, indent=1)
    with open(args.out + ".md", "w") as f:
        f.write(f"# HBM traffic of decode attention, {meta['workload']}\n\n")
        f.write("Commands (from the repository root, on one MI355X):\n\n```\n")
        for c, path in (("FETCH_SIZE", args.fetch_csv), ("WRITE_SIZE", args.write_csv)):
            f.write(f"rocprofv3 --pmc {c} --output-format csv -d {os.path.dirname(path)} -o run -- "
                    f"python3 -m kv_cache_bit_quantize_amd.traffic run --workload {meta['workload']} "
                    f"--meta {args.meta}\n")
        f.write(f"python3 -m kv_cache_bit_quantize_amd.traffic summarize {args.fetch_csv} {args.write_csv} "
                f"--meta {args.meta} --out {args.out}\n```\n\n")
        f.write("| counter | attention KiB/dispatch | 1 GiB copy KiB/dispatch | scale | attention bytes/launch |\n")
        f.write("|---|---|---|---|---|\n")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            r = result[c]
            f.write(f"| {c} | {r['attn_kib_per_dispatch']:.1f} | {r['copy_kib_per_dispatch']:.1f} | "
                    f"{r['scale']:.4f} | {r['attn_bytes_per_launch']:.4e} |\n")
        f.write(f"\nHBM bytes per launch (read + write): {total:.4e}; algorithmic bytes per launch: "
                f"{meta['algorithmic_bytes_per_launch']:.4e}; ratio {result['traffic_over_algorithmic']:.4f}.\n")
        f.write(f"Kernel sources hash: `{meta['kernel_source_hash']}`.\n")
    print(json.dumps(result))


CU_NUM, SIMD_NUM, XCD_NUM = 256, 1024, 8     # MI355X


def _all_per_dispatch(paths):
    """{(kernel name, counter): [value per dispatch]} over several counter_collection csvs."""
    out = {}
    for path in paths:
        rows = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                key = (r["Dispatch_Id"], r["Kernel_Name"], r["Counter_Name"])
                rows[key] = rows.get(key, 0.0) + float(r["Counter_Value"])
        for (_, name, counter), val in rows.items():
            out.setdefault((name, counter), []).append(val)
    return out


def counters(args):
    """Per-dispatch averages of the counters in the given csvs for every attention kernel, and
    the figures derived from them (the expressions rocprofv3 lists for its derived metrics)."""
    data = _all_per_dispatch(args.csv)
    kernels = sorted({n for n, _ in data if "attn_" in n and "kernel" in n})
    lines = [f"# {args.title}\n", "Commands (from the repository root, on one MI355X; one rocprofv3 run per counter set):\n",
             "```"]
    lines += [c for c in args.command]
    lines += [f"python3 -m kv_cache_bit_quantize_amd.traffic counters {' '.join(args.csv)} --title '{args.title}' "
              f"--out {args.out} --command ...", "```\n"]
    summary = {}
    for k in kernels:
        avg = {c: sum(v) / len(v) for (n, c), v in data.items() if n == k}
        nd = min(len(v) for (n, c), v in data.items() if n == k)   # dispatches per counter set
        # the csv's GRBM_GUI_ACTIVE is summed over the XCDs; rocprofv3's derived metrics take
        # its largest per-XCD value, the kernel's busy cycles
        g = avg.get("GRBM_GUI_ACTIVE")
        g = g / XCD_NUM if g else g
        d = {}
        if g:
            if "SQ_ACTIVE_INST_VALU" in avg:
                d["VALU busy (SQ_ACTIVE_INST_VALU / CUs / GRBM_GUI_ACTIVE)"] = avg["SQ_ACTIVE_INST_VALU"] / CU_NUM / g
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                d["MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / SIMDs / GRBM_GUI_ACTIVE)"] = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMD_NUM / g
            if "SQ_WAVE_CYCLES" in avg:
                d["waves per CU (4 SQ_WAVE_CYCLES / CUs / GRBM_GUI_ACTIVE)"] = 4 * avg["SQ_WAVE_CYCLES"] / CU_NUM / g
            if "SQ_LDS_BANK_CONFLICT" in avg:
                d["LDS bank-conflict share of time (SQ_LDS_BANK_CONFLICT / CUs / GRBM_GUI_ACTIVE)"] = \
                    avg["SQ_LDS_BANK_CONFLICT"] / CU_NUM / g
            if "SQ_ACTIVE_INST_LDS" in avg:
                d["LDS instruction busy (SQ_ACTIVE_INST_LDS / CUs / GRBM_GUI_ACTIVE)"] = avg["SQ_ACTIVE_INST_LDS"] / CU_NUM / g
        if "SQ_WAIT_INST_ANY" in avg and "SQ_WAVE_CYCLES" in avg:
            d["wave time waiting on an instruction's operands (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES)"] = \
                avg["SQ_WAIT_INST_ANY"] / avg["SQ_WAVE_CYCLES"]
        if "SQ_LDS_BANK_CONFLICT" in avg and "SQ_LDS_IDX_ACTIVE" in avg:
            d["LDS conflict cycles per active LDS cycle"] = avg["SQ_LDS_BANK_CONFLICT"] / max(
                1.0, avg["SQ_LDS_IDX_ACTIVE"] - avg["SQ_LDS_BANK_CONFLICT"])
        if "TCC_HIT_sum" in avg and "TCC_MISS_sum" in avg:
            d["L2 hit rate (TCC_HIT / (TCC_HIT + TCC_MISS))"] = avg["TCC_HIT_sum"] / max(1.0, avg["TCC_HIT_sum"] + avg["TCC_MISS_sum"])
        if "SQC_ICACHE_MISSES" in avg and "SQC_ICACHE_REQ" in avg:
            d["instruction cache miss rate (SQC_ICACHE_MISSES / SQC_ICACHE_REQ)"] = avg["SQC_ICACHE_MISSES"] / max(1.0, avg["SQC_ICACHE_REQ"])
        if "SQ_INSTS_VALU" in avg and "SQ_WAVES" in avg:
            d["vector instructions per wave"] = avg["SQ_INSTS_VALU"] / avg["SQ_WAVES"]
        summary[k] = {"dispatches": nd, "counters": avg, "derived": d}
        lines.append(f"## `{k}` (averages over {nd} dispatches per counter run)\n")
        lines.append("| counter | average per dispatch |\n|---|---|")
        lines += [f"| {c} | {v:.6g} |" for c, v in sorted(avg.items())]
        if g:
            d["busy cycles per XCD (GRBM_GUI_ACTIVE / 8)"] = g
        if d:
            lines.append("\n| derived | value |\n|---|---|")
            lines += [f"| {c} | {v:.4g} |" for c, v in d.items()]
        lines.append("")
    with open(args.out + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(args.out + ".json", "w") as f:
        json.dump(summary, f, indent=1)
    print(json.dumps({k: v["derived"] for k, v in summary.items()}, indent=1))


def trace(args):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of bench.py: the library's
    kernels from the stats csv, and the dispatches of one kernel from the trace csv split into
    those right after a read_probe_kernel (the benchmark's flushed launches) and the others."""
    lines = [f"# {args.title}\n", "Command (from the repository root, on one MI355X):\n", "```", args.command, "```\n",
             "Library kernels (`run_kernel_stats.csv`; the prefill kernels run once per cache the benchmark "
             "builds, outside the timed steps):\n", "| kernel | calls | average us | min us | max us |",
             "|---|---|---|---|---|"]
    with open(args.stats_csv) as f:
        for r in csv.DictReader(f):
            if "kivi::" not in r["Name"]:
                continue
            name = r["Name"].split("(")[0].replace("void ", "")
            lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    rows = []
    with open(args.trace_csv) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    steps, flushed, name = [], [], None
    for i, (t0, t1, k) in enumerate(rows):
        if args.kernel not in k:
            continue
        name = k.split("(")[0].replace("void ", "")
        after_probe = i > 0 and "read_probe_kernel" in rows[i - 1][2]
        (flushed if after_probe else steps).append((t1 - t0) / 1e3)
    if name:
        st = sorted(steps)
        med = st[len(st) // 2] if len(st) % 2 else 0.5 * (st[len(st) // 2 - 1] + st[len(st) // 2])
        lines.append("")
        lines.append(f"`{name}` has two kinds of dispatch in this run (`run_kernel_trace.csv`): {len(steps)} "
                     f"dispatches not preceded by a read (the decode steps, warm-up included), average "
                     f"{sum(steps) / len(steps):.2f} us, median {med:.2f} us, min {st[0]:.2f} us; and {len(flushed)} "
                     f"attention-only launches each after a 1 GiB read by `read_probe_kernel` (the benchmark's "
                     f"flushed measurement), average {sum(flushed) / max(1, len(flushed)):.2f} us.")
        if args.bytes:
            lines.append("")
            lines.append(f"At {args.bytes} algorithmic bytes per launch, the decode steps' average is "
                         f"{args.bytes / (sum(steps) / len(steps)) / 1e3:.1f} GB/s "
                         f"({args.bytes / (sum(steps) / len(steps)) / 1e3 / 8000:.3f} of the 8 TB/s HBM peak).")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", default="long-128k")
    r.add_argument("--launches", type=int, default=5)
    r.add_argument("--meta", default="prof/traffic/meta.json")
    s = sub.add_parser("summarize")
    s.add_argument("fetch_csv")
    s.add_argument("write_csv")
    s.add_argument("--meta", default="prof/traffic/meta.json")
    s.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--title", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--command", nargs="*", default=[], help="the rocprofv3 commands that wrote the csvs")
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("trace_csv")
    t.add_argument("--kernel", required=True, help="substring of the kernel whose dispatches are split")
    t.add_argument("--bytes", type=int, default=0, help="algorithmic bytes per launch of that kernel")
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True, help="the rocprofv3 command that wrote the csvs")
    t.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.cmd == "trace":
        trace(a)
        return
    if a.cmd == "counters":
        counters(a)
        return
    if a.cmd == "run":
        os.makedirs(os.path.dirname(os.path.abspath(a.meta)), exist_ok=True)
        run(a)
    else:
        summarize(a)


if __name__ == "__main__":
    main()
