"""Summaries of rocprofv3 output for profiles/.

  python -m fp8_transformer_step_amd.profiling stats <kernel_stats.csv> <out.md> --command "<cmd>"
      Markdown table of the library's kernels (calls, average/min/max us).
  python -m fp8_transformer_step_amd.profiling pmc <FETCH dir> <WRITE dir> <out.json> --command "<cmd>"
      HBM bytes per launch of every library kernel from one FETCH_SIZE run and
      one WRITE_SIZE run (KiB per dispatch), each scaled so that the same
      counter reads the known traffic of the calibration copy in the same run
      (an elementwise copy of 128 Mi fp32: 512 MiB read, 512 MiB written).
      Records the sha256 of the kernel sources (csrc/) so that bench.py
      ignores the numbers once any kernel has changed.
  python -m fp8_transformer_step_amd.profiling counters <kernel_stats.csv> <pass dir>... <out.md> --command "<cmd>"
      Per rocprof kernel (template arguments included): calls, average us,
      MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES, summed over the SIMDs, over the
      average duration x 2.4 GHz x 1024 SIMDs), FP8 MFMA rate
      (SQ_INSTS_VALU_MFMA_MOPS_F8 x 512 flop over the average duration) and
      LDS bank conflicts (SQ_LDS_BANK_CONFLICT over the conflict-free LDS
      cycles), from counter passes of the same command.
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

# rocprof kernel name (function name) -> library kernel name.  act_quant_kernel
# serves both the MLP's x quantisation (mlp_xq) and the other projections'
# (ql_act_quant); the profiler cannot tell the two apart.
KERNELS = [
    (r"gu_small_kernel", "mlp_gu_small"),
    (r"down_small_kernel", "mlp_down_small_fused"),
    (r"\bgu_kernel", "mlp_gu"),
    (r"\bdown_kernel", "mlp_down"),
    (r"act_quant_kernel", "act_quant"),
    (r"stream_read_kernel", "stream_read"),
    (r"pack_weight_kernel", "pack_weight"),
    (r"hq_kernel", "mlp_hq"),
    # split kernels: <D, G, SINGLE, PAGED>; balanced: <D, G, PAGED>
    (r"attn_split_kernel<\d+, \d+, true, true>", "attn_single_paged"),
    (r"attn_split_kernel<\d+, \d+, true, false>", "attn_single"),
    (r"attn_split_kernel<\d+, \d+, false, true>", "attn_split_paged"),
    (r"attn_split_kernel", "attn_split"),
    (r"attn_bal_kernel<\d+, \d+, true>", "attn_split_paged"),
    (r"attn_bal_kernel", "attn_split"),
    (r"attn_split_mx_kernel<\d+, \d+, true, true>", "attn_single_mx_paged"),
    (r"attn_split_mx_kernel<\d+, \d+, true, false>", "attn_single_mx"),
    (r"attn_split_mx_kernel<\d+, \d+, false, true>", "attn_split_mx_paged"),
    (r"attn_split_mx_kernel", "attn_split_mx"),
    (r"attn_bal_mx_kernel<\d+, \d+, true>", "attn_split_mx_paged"),
    (r"attn_bal_mx_kernel", "attn_split_mx"),
    # gemm_large_mx_kernel<PACKED, BS, SWI>; SWI = the large-M MLP's gate/up GEMM
    (r"gemm_large_mx_kernel<true, true, true>", "mlp_large_gu_bs"),
    (r"gemm_large_mx_kernel<true, false, true>", "mlp_large_gu_mx"),
    (r"gemm_large_mx_kernel<true, true", "gemm_large_bs_packed"),
    (r"gemm_large_mx_kernel<true", "gemm_large_mx_packed"),
    (r"gemm_large_mx_kernel", "gemm_large_mx"),
    (r"split_reduce_kernel", "mlp_large_down_reduce"),
    (r"quant_pack_kernel<\w+, true>", "mlp_large_hq"),
    (r"quant_pack_kernel", "mlp_large_xq"),
    (r"pack_mx_kernel", "pack_mx"),
    (r"extend_attn_kernel", "extend_attn"),
    (r"sample_kernel", "sample"),
    (r"window_shift_kernel", "window_shift"),
    (r"attn_merge_kernel", "attn_merge"),
    (r"qlinear_kernel", "qlinear"),
    (r"embed_kernel", "embed_sum"),
    (r"argmax_kernel", "argmax"),
    (r"embed_finish_kernel", "embed_finish"),
    (r"finish_kernel", "row_finish"),
    (r"quant_block128_kernel", "quantize_block128"),
    (r"quant_rows_kernel<128>", "quantize_1x128"),
    (r"quant_rows_kernel<32>", "quantize_1x32"),
]
CALIB_BYTES = 512 << 20


def lib_kernel(name):
    for pat, lib in KERNELS:
        if "fp8s::" in name and re.search(pat, name):
            return lib
    return None


def sources_sha256():
    """sha256 over every kernel source file of the library (sorted by name)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_transformer_step_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


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
        lib = lib_kernel(r["Name"])
        if not lib:
            continue
        short = r["Name"].split("(")[0].replace("void ", "")
        lines.append(f"| {lib} | `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def by_launch_shape(trace_csv, out_md, command, kernels, note=""):
    """Per (library kernel, grid) durations from a rocprofv3 kernel trace,
    for the kernels named in `kernels`: one row per launch shape (the grid
    identifies the problem size of a sweep), calls, average, min and max."""
    rows = list(csv.DictReader(open(_csv(trace_csv, "kernel_trace.csv"))))
    groups = {}
    for r in rows:
        lib = lib_kernel(r["Kernel_Name"])
        if lib not in kernels:
            continue
        wg = int(r["Workgroup_Size_X"])
        grid = (int(r["Grid_Size_X"]) // max(wg, 1), int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]))
        short = r["Kernel_Name"].split("(")[0].replace("void ", "")
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault((lib, short, grid, wg), []).append(us)
    lines = ["# rocprofv3 kernel durations by launch shape\n", f"Command:\n\n```\n{command}\n```\n",
             "One row per (kernel instance, grid); problem sizes that launch the same grid share a row "
             "(their average mixes them; min and max bound each).\n" + (f"\n{note}\n" if note else ""),
             "| library kernel | rocprof name | workgroups (x, y, z) | threads | calls | avg us | median us | "
             "min us | max us |",
             "|---|---|---|---|---|---|---|---|---|"]
    for (lib, short, grid, wg), v in sorted(groups.items()):
        lines.append(f"| {lib} | `{short}` | {grid[0]}, {grid[1]}, {grid[2]} | {wg} | {len(v)} | "
                     f"{statistics.mean(v):.1f} | {statistics.median(v):.1f} | {min(v):.1f} | {max(v):.1f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def _counter_means(run_dir):
    rows = list(csv.DictReader(open(_csv(run_dir, "counter_collection.csv"))))
    per, calib = {}, []
    for r in rows:
        v = float(r["Counter_Value"]) * 1024.0      # KiB -> bytes
        name = r["Kernel_Name"]
        lib = lib_kernel(name)
        if lib:
            per.setdefault(lib, []).append(v)
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
           "sources_sha256": sources_sha256(),
           "kernels": {}}
    for lib, fv in fetch.items():
        out["kernels"][lib] = {"fetch_bytes": fv * fs, "write_bytes": write.get(lib, 0.0) * ws}
    json.dump(out, open(out_json, "w"), indent=1)


SIMDS = 1024                      # 256 CUs x 4 SIMDs
CLOCK_HZ = 2.4e9                  # peak engine clock


def _per_kernel_counters(dirs):
    """{rocprof kernel name: {counter: mean value per dispatch}} over passes."""
    out = {}
    for d in dirs:
        acc = {}
        for r in csv.DictReader(open(_csv(d, "counter_collection.csv"))):
            name = r["Kernel_Name"]
            if not lib_kernel(name):
                continue
            key = (name.split("(")[0].replace("void ", ""), r["Counter_Name"])
            acc.setdefault(key, []).append(float(r["Counter_Value"]))
        for (name, ctr), v in acc.items():
            out.setdefault(name, {})[ctr] = statistics.mean(v)
    return out


def counters(stats_csv, dirs, out_md, command):
    dur = {}
    for r in csv.DictReader(open(_csv(stats_csv, "kernel_stats.csv"))):
        if lib_kernel(r["Name"]):
            dur[r["Name"].split("(")[0].replace("void ", "")] = (int(r["Calls"]), float(r["AverageNs"]) / 1e3)
    ctr = _per_kernel_counters(dirs)
    lines = ["# rocprofv3 counters: MFMA use and LDS bank conflicts\n", f"Command:\n\n```\n{command}\n```\n",
             "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) / (average duration x 2.4 GHz x 1024 "
             "SIMDs); FP8 rate = SQ_INSTS_VALU_MFMA_MOPS_F8 x 512 / average duration (dense FP8 peak "
             "5000 TFLOP/s); LDS conflicts = SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - "
             "SQ_LDS_BANK_CONFLICT).  (GRBM_GUI_ACTIVE, also collected, spans the counter window of all "
             "XCDs, not the kernel.)\n",
             "| rocprof kernel | calls | avg us | MFMA busy % | FP8 TFLOP/s | % of FP8 peak | LDS conflict % |",
             "|---|---|---|---|---|---|---|"]
    for name, c in sorted(ctr.items()):
        calls, us = dur.get(name, (0, 0.0))
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
        mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_F8")
        conf, idx = c.get("SQ_LDS_BANK_CONFLICT"), c.get("SQ_LDS_IDX_ACTIVE")
        f_busy = f"{100 * busy / (us * 1e-6 * CLOCK_HZ * SIMDS):.1f}" if busy is not None and us > 0 else "-"
        tf = mops * 512 / (us * 1e-6) / 1e12 if mops is not None and us > 0 else None
        f_tf = f"{tf:.0f}" if tf is not None else "-"
        f_pk = f"{100 * tf / 5000:.1f}" if tf is not None else "-"
        f_lds = f"{100 * conf / max(idx - conf, 1):.2f}" if conf is not None and idx else "-"
        lines.append(f"| `{name}` | {calls} | {us:.1f} | {f_busy} | {f_tf} | {f_pk} | {f_lds} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


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
    s = sub.add_parser("shapes")
    s.add_argument("trace")
    s.add_argument("out")
    s.add_argument("--kernels", required=True, help="comma-separated library kernel names")
    s.add_argument("--command", required=True)
    s.add_argument("--note", default="", help="a line of explanation printed above the table")
    c = sub.add_parser("counters")
    c.add_argument("stats")
    c.add_argument("dirs", nargs="+", help="counter pass directories, then the output .md")
    c.add_argument("--command", required=True)
    args = ap.parse_args()
    if args.cmd == "stats":
        stats(args.csv, args.out, args.command)
    elif args.cmd == "shapes":
        by_launch_shape(args.trace, args.out, args.command, set(args.kernels.split(",")), args.note)
    elif args.cmd == "pmc":
        pmc(args.fetch_dir, args.write_dir, args.out, args.command)
    else:
        counters(args.stats, args.dirs[:-1], args.dirs[-1], args.command)


if __name__ == "__main__":
    main()
