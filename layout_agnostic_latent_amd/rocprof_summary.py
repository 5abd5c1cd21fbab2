"""Summarise rocprofv3 output for the kernels of libsplash_attn.

Usage:
  python -m layout_agnostic_latent_amd.rocprof_summary --name NAME --command CMD \
      --trace DIR [--fetch DIR --write DIR --calib-kernel KERNEL --calib-read-bytes N \
      --calib-write-bytes N] [--bench-json FILE]

* --trace DIR: a `rocprofv3 --kernel-trace --stats --output-format csv` output
  directory; per-kernel call counts and average durations are taken from its
  kernel trace.
* --fetch / --write DIR: `rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE`
  output directories (KiB per dispatch).  The counters are scaled by what the
  same counter reads for a calibration kernel whose bytes are known (the page
  repack moves a known number of bytes each way).

Writes profiles/NAME.md (the figures, with the commands that produced them)
and profiles/NAME.json (machine-readable, including a hash of the decode
kernel's source so that a later build can tell whether the counters still
describe it).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")


def _code_tokens(src: str) -> str:
    """The source with comments removed and whitespace collapsed: edits to
    comments or layout leave the kernels, and so the hash, unchanged."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":  # string or character literal, kept verbatim
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code (not their comments), recorded with the
    counter runs: bench.py uses a record only while the hash still matches."""
    h = hashlib.sha256()
    for f in ("decode_attn.hip", "decode_attn16.hip", "decode_device.h", "lse_merge.hip", "kv_repack.hip", "common.h"):
        with open(os.path.join(PKG, "csrc", f), encoding="utf-8") as fh:
            h.update(_code_tokens(fh.read()).encode())
    return h.hexdigest()[:16]


def short(name: str) -> str:
    # the row-wave merge serves the split-KV partials (fp16, inside
    # splash_decode_attn) and splash_lse_merge (fp32): keep them apart
    if "split_merge_kernel" in name:
        if "<float" in name or "split_merge_kernelIf" in name:
            return "split_merge_kernel<fp32> (splash_lse_merge)"
        return "split_merge_kernel<fp16> (split-KV merge)"
    for key in ("decode_attn_kernel", "decode_attn16_kernel", "lse_merge_kernel", "kv_repack_kernel",
                "mfma_peak_kernel", "read_peak_kernel"):
        if key in name:
            i = name.find("<")
            j = name.find(">", i)
            return key + (name[i:j + 1] if key.startswith("decode_attn") and i >= 0 else "")
    return name.split("(")[0][:60]


def read_trace(d):
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    dur = defaultdict(list)
    for f in files:
        for row in csv.DictReader(open(f)):
            ns = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
            dur[short(row["Kernel_Name"])].append(ns / 1000.0)
    return dur


def read_pmc(d, counter):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    vals = defaultdict(list)
    for f in files:
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] == counter:
                vals[short(row["Kernel_Name"])].append(float(row["Counter_Value"]))
    return vals


def counters_main(argv) -> None:
    """--counters mode: a table of the decode kernel's per-dispatch counter
    averages for several runs (one rocprofv3 --pmc output directory each)."""
    ap = argparse.ArgumentParser()
    ap.add_argument("--counters", action="store_true")
    ap.add_argument("--name", required=True)
    ap.add_argument("--command", required=True, action="append")
    ap.add_argument("--run", required=True, action="append", nargs=3, metavar=("LABEL", "DIRS", "ALG_FLOPS"),
                    help="workload label, rocprofv3 output directories (comma-separated passes of one "
                         "workload), algorithmic FLOPs per decode call")
    ap.add_argument("--transpose", action="store_true",
                    help="one row per counter (with its value per wave), one column per workload")
    args = ap.parse_args(argv)
    rows = []
    for label, dirs, alg in args.run:
        vals = defaultdict(list)
        for d in dirs.split(","):
            for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
                for row in csv.DictReader(open(f)):
                    if "decode_attn" in row["Kernel_Name"]:
                        vals[row["Counter_Name"]].append(float(row["Counter_Value"]))
        rows.append((label, float(alg), {k: statistics.mean(v) for k, v in vals.items()}))
    names = sorted({k for _, _, v in rows for k in v})
    if args.transpose:
        return _transposed(args, rows, names)
    lines = [f"# {args.name}", "", "Produced by:", ""] + [f"    {c}" for c in args.command]
    lines += ["", f"Kernel source hash: `{kernel_source_hash()}`", "",
              "Per decode-kernel dispatch (average over the run's dispatches):", "",
              "| workload | " + " | ".join(names) + " | MFMA FLOPs / algorithmic | LDS conflict share |",
              "|---|" + "---|" * (len(names) + 2)]
    for label, alg, v in rows:
        fl = v.get("MfmaFlopsBF16")
        bank, active = v.get("SQ_LDS_BANK_CONFLICT"), v.get("SQ_LDS_IDX_ACTIVE")
        share = (bank / (active - bank)) if bank is not None and active and active > bank else None
        cells = [f"{v[n]:.6g}" if n in v else "" for n in names]
        lines.append(f"| {label} | " + " | ".join(cells) + f" | {'' if fl is None else f'{fl / alg:.3f}'} | "
                     f"{'' if share is None else f'{100 * share:.2f}%'} |")
    lines += ["", "MfmaUtil: MFMA busy cycles over (active cycles x SIMDs), percent. MfmaFlopsBF16: 512 x the "
              "bf16 MFMA op count. LDS conflict share: bank-conflict cycles over conflict-free LDS cycles."]
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, args.name + ".md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _transposed(args, rows, names) -> None:
    """Counter-per-row table: each workload's per-dispatch average and that
    divided by SQ_WAVES (a per-wave figure; the SQ cycle counters count
    4-cycle units)."""
    lines = [f"# {args.name}", "", "Produced by:", ""] + [f"    {c}" for c in args.command]
    lines += ["", f"Kernel source hash: `{kernel_source_hash()}`", "",
              "Per decode-kernel dispatch (average over the run's dispatches), and per wave:", "",
              "| counter | " + " | ".join(f"{label} | per wave" for label, _, _ in rows) + " |",
              "|---|" + "---|---|" * len(rows)]
    for n in names:
        cells = []
        for _, _, v in rows:
            w = v.get("SQ_WAVES")
            cells.append(f"{v[n]:.6g}" if n in v else "")
            cells.append(f"{v[n] / w:.6g}" if n in v and w else "")
        lines.append(f"| {n} | " + " | ".join(cells) + " |")
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, args.name + ".md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    if "--counters" in sys.argv[1:]:
        return counters_main(sys.argv[1:])
    ap = argparse.ArgumentParser()
    ap.add_argument("--name", required=True)
    ap.add_argument("--command", required=True, action="append", help="command(s) that produced the data")
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--calib-kernel", default="kv_repack_kernel")
    ap.add_argument("--calib-fetch", help="FETCH_SIZE run holding the calibration kernel (default: --fetch)")
    ap.add_argument("--calib-write", help="WRITE_SIZE run holding the calibration kernel (default: --write)")
    ap.add_argument("--calib-read-bytes", type=float)
    ap.add_argument("--calib-write-bytes", type=float)
    ap.add_argument("--bench-json", help="the bench.py JSON line of the traced run (for context)")
    args = ap.parse_args()

    dur = read_trace(args.trace)
    rec = {"name": args.name, "commands": args.command, "kernel_source_hash": kernel_source_hash(), "kernels": {}}
    for k, v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        rec["kernels"][k] = {"calls": len(v), "avg_us": round(statistics.mean(v), 3),
                             "min_us": round(min(v), 3), "max_us": round(max(v), 3)}
    if args.fetch and args.write:
        fetch = read_pmc(args.fetch, "FETCH_SIZE")
        write = read_pmc(args.write, "WRITE_SIZE")
        cfetch = read_pmc(args.calib_fetch or args.fetch, "FETCH_SIZE")
        cwrite = read_pmc(args.calib_write or args.write, "WRITE_SIZE")
        ck = args.calib_kernel
        f_scale = args.calib_read_bytes / 1024.0 / statistics.mean(cfetch[ck])
        w_scale = args.calib_write_bytes / 1024.0 / statistics.mean(cwrite[ck])
        rec["calibration"] = {"kernel": ck, "read_bytes": args.calib_read_bytes, "write_bytes": args.calib_write_bytes,
                              "fetch_kib_raw": statistics.mean(cfetch[ck]), "write_kib_raw": statistics.mean(cwrite[ck]),
                              "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)}
        for k in rec["kernels"]:
            if k in fetch and k in write:
                fb = statistics.mean(fetch[k]) * 1024.0 * f_scale
                wb = statistics.mean(write[k]) * 1024.0 * w_scale
                rec["kernels"][k].update({"fetch_kib_raw": statistics.mean(fetch[k]),
                                          "write_kib_raw": statistics.mean(write[k]),
                                          "hbm_read_bytes": int(fb), "hbm_write_bytes": int(wb),
                                          "traffic_bytes": int(fb + wb)})
    if args.bench_json:
        with open(args.bench_json) as f:
            rec["bench"] = json.loads(f.read().strip().splitlines()[-1])

    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, args.name + ".json"), "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"# {args.name}", "", "Produced by:", ""]
    lines += [f"    {c}" for c in args.command]
    lines += ["", f"Kernel source hash: `{rec['kernel_source_hash']}`", "",
              "| kernel | calls | avg us | min us | max us | HBM read MB | HBM write MB |",
              "|---|---|---|---|---|---|---|"]
    for k, r in rec["kernels"].items():
        rb = r.get("hbm_read_bytes")
        wb = r.get("hbm_write_bytes")
        lines.append(f"| `{k}` | {r['calls']} | {r['avg_us']} | {r['min_us']} | {r['max_us']} | "
                     f"{'' if rb is None else round(rb / 1e6, 2)} | {'' if wb is None else round(wb / 1e6, 2)} |")
    if "calibration" in rec:
        c = rec["calibration"]
        lines += ["", f"Counter calibration on `{c['kernel']}` (known bytes: {c['read_bytes']:.0f} read, "
                      f"{c['write_bytes']:.0f} written per dispatch): FETCH_SIZE x {c['fetch_scale']}, "
                      f"WRITE_SIZE x {c['write_scale']}."]
    if "bench" in rec:
        b = rec["bench"]
        lines += ["", "bench.py line of the traced run (timing perturbed by the tracer):", "",
                  f"    value {b['value']:.4g} {b['unit']}, ms/step {b['ms_per_step']}, "
                  f"roofline frac {b['roofline']['frac']}"]
    with open(os.path.join(PROFILES, args.name + ".md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
