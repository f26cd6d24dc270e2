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
      hash of the kernel sources so that a stale record is never reported.
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
           "write_scale": round(w_scale, 4), "source_sha": bench.source_hash(),
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
    a = ap.parse_args()
    print(stats(a.csv, a.cmd) if a.what == "stats" else traffic(a))


if __name__ == "__main__":
    main()
