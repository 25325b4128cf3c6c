"""Summaries of rocprofv3 output for profiles/.

  python -m fp8_transformer_step_amd.profiling stats <kernel_stats.csv> <out.md> --command "<cmd>"
      Markdown table of the library's kernels (calls, average/min/max us).
  python -m fp8_transformer_step_amd.profiling pmc <FETCH dir> <WRITE dir> <out.json> --command "<cmd>"
      HBM bytes per launch of every library kernel from one FETCH_SIZE run and
      one WRITE_SIZE run (KiB per dispatch), each scaled so that the same
      counter reads the known traffic of the calibration copy in the same run
      (an elementwise copy of 128 Mi fp32: 512 MiB read, 512 MiB written).
      Records the sha256 of each kernel's source so that stale numbers are
      ignored by bench.py.
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# rocprof kernel name (function name) -> (library kernel name, source file)
KERNELS = [
    (r"gu_small_kernel", "mlp_gu_small", "mlp.hip"),
    (r"down_small_kernel<[^>]*true", "mlp_down_small_fused", "mlp.hip"),
    (r"down_small_kernel", "mlp_down_small", "mlp.hip"),
    (r"\bgu_kernel", "mlp_gu", "mlp.hip"),
    (r"\bdown_kernel", "mlp_down", "mlp.hip"),
    (r"xq_kernel", "mlp_xq", "mlp.hip"),
    (r"hq_kernel", "mlp_hq", "mlp.hip"),
    (r"attn_split_kernel", "attn_split", "attention.hip"),
    (r"attn_merge_kernel", "attn_merge", "attention.hip"),
    (r"quant_block128_kernel", "quantize_block128", "quantize.hip"),
    (r"quant_rows_kernel<128>", "quantize_1x128", "quantize.hip"),
    (r"quant_rows_kernel<32>", "quantize_1x32", "quantize.hip"),
]
CALIB_BYTES = 512 << 20


def lib_kernel(name):
    for pat, lib, src in KERNELS:
        if "fp8s::" in name and re.search(pat, name):
            return lib, "fp8_transformer_step_amd/csrc/" + src
    return None, None


def _csv(path_or_dir, suffix):
    if os.path.isdir(path_or_dir):
        hits = glob.glob(os.path.join(path_or_dir, "**", "*" + suffix), recursive=True)
        if not hits:
            raise SystemExit(f"no *{suffix} under {path_or_dir}")
        return hits[0]
    return path_or_dir


def stats(csv_path, out_md, command):
    rows = list(csv.DictReader(open(_csv(csv_path, "kernel_stats.csv"))))
    lines = [f"# rocprofv3 kernel statistics\n", f"Command:\n\n```\n{command}\n```\n",
             "| library kernel | rocprof name | calls | avg us | min us | max us |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lib, _ = lib_kernel(r["Name"])
        if not lib:
            continue
        short = r["Name"].split("(")[0].replace("void ", "")
        lines.append(f"| {lib} | `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def _counter_means(run_dir):
    rows = list(csv.DictReader(open(_csv(run_dir, "counter_collection.csv"))))
    per, calib = {}, []
    for r in rows:
        v = float(r["Counter_Value"]) * 1024.0      # KiB -> bytes
        name = r["Kernel_Name"]
        lib, src = lib_kernel(name)
        if lib:
            per.setdefault((lib, src), []).append(v)
        elif "add" in name.lower() and int(r.get("Grid_Size", 0) or 0) >= (1 << 20):
            calib.append(v)
    if not calib:
        raise SystemExit(f"no calibration copy found in {run_dir}")
    return {k: statistics.mean(v) for k, v in per.items()}, statistics.median(calib)


def pmc(fetch_dir, write_dir, out_json, command):
    fetch, fcal = _counter_means(fetch_dir)
    write, wcal = _counter_means(write_dir)
    fs, ws = CALIB_BYTES / fcal, CALIB_BYTES / wcal
    out = {"command": command,
           "calibration": {"kernel": "elementwise fp32 copy of 128 Mi elements",
                           "known_read_bytes": CALIB_BYTES, "known_write_bytes": CALIB_BYTES,
                           "fetch_size_bytes": fcal, "write_size_bytes": wcal,
                           "fetch_scale": fs, "write_scale": ws},
           "kernels": {}}
    for (lib, src), fv in fetch.items():
        wv = write.get((lib, src), 0.0)
        sha = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
        out["kernels"][lib] = {"fetch_bytes": fv * fs, "write_bytes": wv * ws, "source": src,
                               "source_sha256": sha}
    json.dump(out, open(out_json, "w"), indent=1)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("out")
    a.add_argument("--command", required=True)
    b = sub.add_parser("pmc")
    b.add_argument("fetch_dir")
    b.add_argument("write_dir")
    b.add_argument("out")
    b.add_argument("--command", required=True)
    args = ap.parse_args()
    if args.cmd == "stats":
        stats(args.csv, args.out, args.command)
    else:
        pmc(args.fetch_dir, args.write_dir, args.out, args.command)


if __name__ == "__main__":
    main()
