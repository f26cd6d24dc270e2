"""Summaries of rocprofv3 output for the committed profile records.

  python -m flow_matching_diffusion_amd.profsum stats STATS_CSV --cmd "..."
      Per-kernel launch statistics from a `rocprofv3 --kernel-trace --stats` run (the
      *_kernel_stats.csv file) as a Markdown table on stdout.

  python -m flow_matching_diffusion_amd.profsum traffic --fetch CSV --write CSV --match TEXT
      --copy-match TEXT --copy-bytes N --key KEY [--cmd-fetch "..."] [--cmd-write "..."]
      HBM traffic per launch of the kernels whose name contains TEXT, from two
      `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs (*_counter_collection.csv).
      Both counters are in KiB per dispatch; each is scaled by the factor that makes a
      plain copy kernel of known size (COPY-MATCH, reading and writing N bytes) read N
      bytes (FETCH) and write N bytes (WRITE). Prints Markdown and merges
      {KEY: {fetch_bytes, write_bytes, ...}} into profiles/traffic.json, stamped with the
      hash of the sources that build KEY's kernel so that a stale record is never reported.

  python -m flow_matching_diffusion_amd.profsum trace TRACE_CSV --cmd "..." [--skip N]
      Per-launch-shape statistics from a `rocprofv3 --kernel-trace` run (the *_kernel_trace.csv
      file): dispatches grouped by kernel and grid, so that one kernel's launches on different
      workloads stay apart; the first N dispatches of each group (warm-up) are left out.

  python -m flow_matching_diffusion_amd.profsum counters CSV --cmd "..." [--xcds 8] [--cus 256]
      Matrix-core and LDS counters per kernel from a `rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES
      SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAVES GRBM_GUI_ACTIVE` run, dispatches
      grouped by kernel and by their matrix-core instruction count (so that launches of one kernel
      on different shapes stay apart). MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES over (GRBM_GUI_ACTIVE /
      xcds) x cus x 4 SIMDs; the pure matrix-core probe kernel, if present, shows what a fully busy
      unit reads.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _short(name: str, width: int = 110) -> str:
    name = name.replace("k2::", "")
    return name if len(name) <= width else name[:width - 3] + "..."


def stats(path: str, cmd: str) -> str:
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    out = [f"Command: `{cmd}`", "", "| kernel | calls | avg us | min us | max us | % of GPU time |",
           "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{100 * float(r['TotalDurationNs']) / total:.2f} |")
    return "\n".join(out)


def _per_kernel(path: str, counter: str) -> dict[str, list[float]]:
    """Counter value (summed over its instances) per dispatch, grouped by kernel name."""
    per_dispatch: dict[tuple[str, str], float] = collections.defaultdict(float)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"].startswith(counter):
            per_dispatch[(r["Dispatch_Id"], r["Kernel_Name"])] += float(r["Counter_Value"])
    grouped: dict[str, list[float]] = collections.defaultdict(list)
    for (_, name), v in per_dispatch.items():
        grouped[name].append(v)
    return grouped


def _pick(grouped: dict[str, list[float]], match: str) -> tuple[str, float]:
    names = [n for n in grouped if match in n]
    if not names:
        sys.exit(f"no kernel name contains {match!r}")
    vals = [v for n in names for v in grouped[n]]
    return names[0], sum(vals) / len(vals)


def traffic(a) -> str:
    fetch, write = _per_kernel(a.fetch, "FETCH_SIZE"), _per_kernel(a.write, "WRITE_SIZE")
    kname, f_kib = _pick(fetch, a.match)
    _, w_kib = _pick(write, a.match)
    cname, cf_kib = _pick(fetch, a.copy_match)
    _, cw_kib = _pick(write, a.copy_match)
    f_scale = a.copy_bytes / (cf_kib * 1024)
    w_scale = a.copy_bytes / (cw_kib * 1024)
    fetch_b, write_b = f_kib * 1024 * f_scale, w_kib * 1024 * w_scale
    sys.path.insert(0, ROOT)
    import bench  # the kernel-source hash that stamps the record

    rec = {"kernel": kname, "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
           "fetch_kib_raw": round(f_kib, 1), "write_kib_raw": round(w_kib, 1),
           "copy_kernel": cname, "copy_bytes": a.copy_bytes, "fetch_scale": round(f_scale, 4),
           "write_scale": round(w_scale, 4), "source_sha": bench.source_hash(a.key),
           "cmd_fetch": a.cmd_fetch, "cmd_write": a.cmd_write}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        allrec = json.load(open(path))
    except (OSError, ValueError):
        allrec = {}
    allrec[a.key] = rec
    with open(path, "w") as f:
        json.dump(allrec, f, indent=1, sort_keys=True)
        f.write("\n")
    return "\n".join([
        f"FETCH_SIZE command: `{a.cmd_fetch}`", f"WRITE_SIZE command: `{a.cmd_write}`", "",
        f"Calibration: `{_short(cname)}` moves {a.copy_bytes} bytes each way; the counters read "
        f"{cf_kib:.1f} KiB fetched and {cw_kib:.1f} KiB written, so FETCH is scaled by {f_scale:.4f} and "
        f"WRITE by {w_scale:.4f}.", "",
        f"`{_short(kname)}`: FETCH_SIZE {f_kib:.1f} KiB, WRITE_SIZE {w_kib:.1f} KiB per launch (raw); "
        f"scaled: {fetch_b / 1e9:.3f} GB read + {write_b / 1e9:.3f} GB written = "
        f"{(fetch_b + write_b) / 1e9:.3f} GB of HBM traffic per launch."])


def trace(path: str, cmd: str, skip: int = 0) -> str:
    groups: dict[tuple, list[dict]] = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        key = (r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]))
        groups[key].append(r)
    rows = []
    for (name, gx, gy, gz), rs in groups.items():
        rs.sort(key=lambda r: int(r["Start_Timestamp"]))
        used = rs[skip:] if len(rs) > skip else rs
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in used]
        r0 = used[0]
        rows.append((sum(d), name, gx, gy, gz, len(used), sum(d) / len(d), min(d), max(d), r0))
    rows.sort(key=lambda x: -x[0])
    out = [f"Command: `{cmd}`", "", f"First {skip} dispatches of each kernel and grid left out (warm-up).",
           "VGPR and AGPR are the trace's VGPR_Count and Accum_VGPR_Count columns; on this part VGPR_Count reads",
           "half of the register total the compiler reports for the kernel (for example 192 for a kernel built",
           "with 384, which runs one wave per SIMD).", "",
           "| kernel | grid (threads) | calls | avg us | min us | max us | VGPR | AGPR | LDS B | scratch B |",
           "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for tot, name, gx, gy, gz, n, avg, mn, mx, r0 in rows:
        out.append(f"| `{_short(name, 80)}` | {gx}x{gy}x{gz} | {n} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {r0['VGPR_Count']} | "
                   f"{r0['Accum_VGPR_Count']} | {r0['LDS_Block_Size']} | {r0['Scratch_Size']} |")
    return "\n".join(out)


def counters(path: str, cmd: str, xcds: int = 8, cus: int = 256) -> str:
    names = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAVES",
             "GRBM_GUI_ACTIVE")
    per: dict[tuple[str, str], dict[str, float]] = collections.defaultdict(lambda: collections.defaultdict(float))
    for r in csv.DictReader(open(path)):
        c = r["Counter_Name"]
        if c in names:
            per[(r["Dispatch_Id"], r["Kernel_Name"])][c] += float(r["Counter_Value"])
    groups: dict[tuple[str, int], list[dict[str, float]]] = collections.defaultdict(list)
    for (_, name), v in per.items():
        groups[(name, round(v.get("SQ_INSTS_MFMA", 0.0) / 1e5))].append(v)
    rows = []
    for (name, _), vs in groups.items():
        avg = {c: sum(v.get(c, 0.0) for v in vs) / len(vs) for c in names}
        cycles = avg["GRBM_GUI_ACTIVE"] / xcds
        busy = 100.0 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * cus * 4) if cycles else 0.0
        rows.append((avg["SQ_INSTS_MFMA"], name, len(vs), avg, cycles, busy))
    rows.sort(key=lambda r: -r[0])
    out = [f"Command: `{cmd}`", "",
           f"MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES / ((GRBM_GUI_ACTIVE / {xcds}) x {cus} CUs x 4 SIMDs); counters "
           "summed over their instances, averaged over the dispatches of each row.", "",
           "| kernel | dispatches | GUI cycles (per XCD) | MFMA insts (M) | LDS insts (M) | LDS insts per MFMA | "
           "LDS bank conflicts (M) | waves | MFMA busy % |", "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for minst, name, n, avg, cycles, busy in rows:
        if minst == 0 and avg["SQ_INSTS_LDS"] == 0:
            continue
        ratio = avg["SQ_INSTS_LDS"] / minst if minst else float("nan")
        out.append(f"| `{_short(name, 90)}` | {n} | {cycles:,.0f} | {minst / 1e6:.2f} | {avg['SQ_INSTS_LDS'] / 1e6:.2f} | "
                   f"{ratio:.2f} | {avg['SQ_LDS_BANK_CONFLICT'] / 1e6:.3f} | {avg['SQ_WAVES']:,.0f} | {busy:.1f} |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--match", required=True)
    t.add_argument("--copy-match", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--key", required=True)
    t.add_argument("--cmd-fetch", default="")
    t.add_argument("--cmd-write", default="")
    tr = sub.add_parser("trace")
    tr.add_argument("csv")
    tr.add_argument("--cmd", required=True)
    tr.add_argument("--skip", type=int, default=0)
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--cmd", required=True)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--cus", type=int, default=256)
    a = ap.parse_args()
    if a.what == "stats":
        print(stats(a.csv, a.cmd))
    elif a.what == "trace":
        print(trace(a.csv, a.cmd, a.skip))
    elif a.what == "counters":
        print(counters(a.csv, a.cmd, a.xcds, a.cus))
    else:
        print(traffic(a))


if __name__ == "__main__":
    main()
