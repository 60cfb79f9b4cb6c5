"""Summaries of rocprofv3 output for the MoE kernels (text, a few KB).

    python -m mixture_experts_layer_46_amd.profsum stats  <kernel_stats.csv> <out.txt> --command CMD
    python -m mixture_experts_layer_46_amd.profsum traffic <fetch_counter_collection.csv>
        <write_counter_collection.csv> <out.txt> --workload NAME --command CMD
    python -m mixture_experts_layer_46_amd.profsum mfma <counter_collection.csv>
        <kernel_trace.csv> <agent_info.csv> <out.txt> --workload NAME --command CMD

`stats` tabulates calls and mean/min/max duration of each moe:: kernel from a
`--kernel-trace --stats` run.  `traffic` averages FETCH_SIZE and WRITE_SIZE (KiB per
dispatch) of each moe:: kernel and scales them to HBM bytes with the factor the same
counters give for the largest device copy in the run (a 1 GiB copy that the benchmark
makes with --copy-calibration: true bytes / counted bytes).  The traffic file also
records the sha256 of the grouped-GEMM source it was measured on, so a reader can tell
when the kernel has changed since.  `mfma` takes one pass of SQ_VALU_MFMA_BUSY_CYCLES and
GRBM_GUI_ACTIVE collected together with a kernel trace and reports, per kernel, the MFMA
pipes' busy fraction (busy cycles summed over all SIMDs / (SIMDs x GPU cycles)) and the
clock the kernel ran at (GUI-active cycles per XCC / duration).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os

HERE = os.path.dirname(os.path.abspath(__file__))
GEMM_SRC = os.path.join(HERE, "csrc", "grouped_gemm.hip")
COPY_BYTES = 1 << 30


def short_name(name: str) -> str:
    """Kernel name without the argument list ('void moe::k<..>(...)' -> 'k<..>')."""
    n = name.strip()
    if n.startswith("void "):
        n = n[5:]
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            n = n[:i]
            break
    return n.replace("moe::", "")


def _is_moe(name: str) -> bool:
    return "moe::" in name


def stats(csv_path: str, out_path: str, command: str) -> str:
    rows = list(csv.DictReader(open(csv_path)))
    lines = ["# rocprofv3 kernel-trace summary (MoE kernels)", f"# command: {command}",
             f"# summary: python3 -m mixture_experts_layer_46_amd.profsum stats {csv_path} {out_path}", "",
             f"{'calls':>6} {'mean_us':>10} {'min_us':>10} {'max_us':>10} {'total_ms':>10}  kernel"]
    for r in rows:
        if not _is_moe(r["Name"]):
            continue
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
                     f"{float(r['MinNs']) / 1e3:10.1f} {float(r['MaxNs']) / 1e3:10.1f} "
                     f"{float(r['TotalDurationNs']) / 1e6:10.3f}  {short_name(r['Name'])}")
    text = "\n".join(lines) + "\n"
    open(out_path, "w").write(text)
    return text


def _per_kernel(csv_path: str, counter: str):
    vals = collections.defaultdict(list)
    copies = []
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        v = float(r["Counter_Value"])
        if _is_moe(r["Kernel_Name"]):
            vals[short_name(r["Kernel_Name"])].append(v)
        elif "copyBuffer" in r["Kernel_Name"] or "copy" in r["Kernel_Name"].lower():
            copies.append(v)
    return vals, (max(copies) if copies else None)


def traffic(fetch_csv: str, write_csv: str, out_path: str, workload: str, command: str,
            up: str | None = None, down: str | None = None) -> str:
    fetch, copy_f = _per_kernel(fetch_csv, "FETCH_SIZE")
    write, copy_w = _per_kernel(write_csv, "WRITE_SIZE")
    kib = COPY_BYTES / 1024
    f_scale = kib / copy_f if copy_f and 0.5 * kib < copy_f < 2 * kib else None
    w_scale = kib / copy_w if copy_w and 0.5 * kib < copy_w < 2 * kib else None
    digest = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
    lines = ["# rocprofv3 PMC traffic summary (MoE kernels): FETCH_SIZE and WRITE_SIZE, KiB per",
             "# dispatch, averaged over dispatches, then scaled by the copy calibration",
             f"# command: {command}",
             f"# summary: python3 -m mixture_experts_layer_46_amd.profsum traffic {fetch_csv} {write_csv} {out_path}",
             f"workload: {workload}",
             f"grouped_gemm.hip sha256: {digest}",
             f"copy calibration fetch KiB counted for 1 GiB: {copy_f}",
             f"copy calibration write KiB counted for 1 GiB: {copy_w}",
             f"fetch scale: {f_scale}",
             f"write scale: {w_scale}", ""]
    lines.append(f"{'dispatches':>10} {'fetch_KiB':>14} {'write_KiB':>14} {'hbm_MB':>10}  kernel")
    per = {}
    for name in sorted(set(fetch) | set(write)):
        fv = sum(fetch[name]) / len(fetch[name]) if fetch.get(name) else 0.0
        wv = sum(write[name]) / len(write[name]) if write.get(name) else 0.0
        hbm = None
        if f_scale and w_scale:
            hbm = (fv * f_scale + wv * w_scale) * 1024
        per[name] = hbm
        hs = f"{hbm / 1e6:10.1f}" if hbm is not None else f"{'n/a':>10}"
        lines.append(f"{len(fetch.get(name, [])):10d} {fv:14.1f} {wv:14.1f} {hs}  {name}")
    lines.append("")
    for which, pat in (("up", up), ("down", down)):
        if not pat:
            continue
        hit = [n for n in per if n.startswith(pat)]
        if len(hit) == 1 and per[hit[0]] is not None:
            lines.append(f"{which} kernel: {pat}")
            lines.append(f"{which} hbm bytes per launch: {per[hit[0]]:.0f}")
    text = "\n".join(lines) + "\n"
    open(out_path, "w").write(text)
    return text


def _gpu_agent(agent_csv: str):
    for r in csv.DictReader(open(agent_csv)):
        if r.get("Agent_Type") == "GPU":
            return int(r["Simd_Count"]), int(r["Num_Xcc"]), int(r["Cu_Count"])
    raise ValueError(f"no GPU agent in {agent_csv}")


def mfma(counter_csv: str, trace_csv: str, agent_csv: str, out_path: str, workload: str, command: str) -> str:
    simds, xccs, cus = _gpu_agent(agent_csv)
    dur = {}
    for r in csv.DictReader(open(trace_csv)):
        dur[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    seen = collections.defaultdict(set)
    for r in csv.DictReader(open(counter_csv)):
        if not _is_moe(r["Kernel_Name"]):
            continue
        per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
        seen[short_name(r["Kernel_Name"])].add(r["Dispatch_Id"])
    digest = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
    lines = ["# rocprofv3 MFMA-busy summary (MoE kernels): SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs)",
             "# and GRBM_GUI_ACTIVE (summed over XCCs) per dispatch, with durations from the same run",
             f"# command: {command}",
             f"# summary: python3 -m mixture_experts_layer_46_amd.profsum mfma {counter_csv} {trace_csv} "
             f"{agent_csv} {out_path}",
             f"workload: {workload}",
             f"grouped_gemm.hip sha256: {digest}",
             f"gpu: {cus} CUs, {simds} SIMDs, {xccs} XCCs",
             "# clock and busy fraction only for kernels of at least 100 us", "",
             f"{'dispatches':>10} {'mean_us':>9} {'clock_GHz':>9} {'mfma_busy':>9}  kernel"]
    for name in sorted(seen):
        ids = [i for i in seen[name] if i in dur and "GRBM_GUI_ACTIVE" in per[i]
               and "SQ_VALU_MFMA_BUSY_CYCLES" in per[i]]
        if not ids:
            continue
        us = sum(dur[i] for i in ids) / len(ids) / 1e3
        gui = sum(per[i]["GRBM_GUI_ACTIVE"] for i in ids) / len(ids) / xccs
        busy = sum(per[i]["SQ_VALU_MFMA_BUSY_CYCLES"] for i in ids) / len(ids) / simds
        if us < 100:        # the counters' active window is not the kernel's: no rates
            lines.append(f"{len(ids):10d} {us:9.1f} {'-':>9} {'-':>9}  {name}")
            continue
        clock = gui / (us * 1e3)
        frac = busy / gui if gui > 0 else 0.0
        lines.append(f"{len(ids):10d} {us:9.1f} {clock:9.2f} {frac:9.3f}  {name}")
    text = "\n".join(lines) + "\n"
    open(out_path, "w").write(text)
    return text


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("out")
    a.add_argument("--command", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("out")
    b.add_argument("--workload", required=True)
    b.add_argument("--command", required=True)
    b.add_argument("--up", default=None, help="name prefix of the first-projection kernel")
    b.add_argument("--down", default=None, help="name prefix of the second-projection kernel")
    c = sub.add_parser("mfma")
    c.add_argument("counter_csv")
    c.add_argument("trace_csv")
    c.add_argument("agent_csv")
    c.add_argument("out")
    c.add_argument("--workload", required=True)
    c.add_argument("--command", required=True)
    args = ap.parse_args()
    if args.cmd == "stats":
        print(stats(args.csv, args.out, args.command), end="")
    elif args.cmd == "mfma":
        print(mfma(args.counter_csv, args.trace_csv, args.agent_csv, args.out, args.workload, args.command), end="")
    else:
        print(traffic(args.fetch_csv, args.write_csv, args.out, args.workload, args.command,
                      args.up, args.down), end="")


if __name__ == "__main__":
    main()
