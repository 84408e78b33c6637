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
bytes, and records the hash of the kernel sources it was taken on.
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
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            d = "fetch" if c == "FETCH_SIZE" else "write"
            f.write(f"rocprofv3 --pmc {c} --output-format csv -d gpurun_out/traffic/{d} -o run -- "
                    f"python3 -m kv_cache_bit_quantize_amd.traffic run --workload {meta['workload']} "
                    f"--meta gpurun_out/traffic/meta.json\n")
        f.write("python3 -m kv_cache_bit_quantize_amd.traffic summarize gpurun_out/traffic/fetch/run_counter_collection.csv "
                f"gpurun_out/traffic/write/run_counter_collection.csv --meta gpurun_out/traffic/meta.json "
                f"--out {args.out}\n```\n\n")
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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", default="long-128k")
    r.add_argument("--launches", type=int, default=5)
    r.add_argument("--meta", default="gpurun_out/traffic/meta.json")
    s = sub.add_parser("summarize")
    s.add_argument("fetch_csv")
    s.add_argument("write_csv")
    s.add_argument("--meta", default="gpurun_out/traffic/meta.json")
    s.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.cmd == "run":
        os.makedirs(os.path.dirname(os.path.abspath(a.meta)), exist_ok=True)
        run(a)
    else:
        summarize(a)


if __name__ == "__main__":
    main()
