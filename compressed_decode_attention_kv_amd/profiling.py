"""Summaries of rocprofv3 output for the library's kernels.

  python -m compressed_decode_attention_kv_amd.profiling stats <kernel_stats.csv>
  python -m compressed_decode_attention_kv_amd.profiling traffic <fetch counter_collection.csv> \
        <write counter_collection.csv> --calib-bytes N

`stats` prints the average duration per kernel.  `traffic` prints HBM bytes
per dispatch from the FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch),
the fetch side scaled by what the same counter reads for the library's
streaming-read kernel over a buffer of N bytes (non-temporal loads count at
half their size on this device), the write side by --write-factor (1.0: the
counter matches the known write volume of the quantize kernels).
"""
import argparse
import collections
import csv
import re
import sys


def short(name):
    name = re.sub(r"^void ", "", name)
    name = name.replace("tq::(anonymous namespace)::", "")
    name = name.replace("_ZN2tq12_GLOBAL__N_1", "")
    return name[:90]


def stats(path):
    rows = list(csv.DictReader(open(path)))
    out = ["%-90s %6s %14s" % ("kernel", "calls", "avg_us")]
    for r in rows:
        if "tq" not in r["Name"] and "stream_read" not in r["Name"]:
            continue
        out.append("%-90s %6s %14.2f" % (short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1000.0))
    return "\n".join(out)


def _per_kernel(path, counter):
    rows = list(csv.DictReader(open(path)))
    agg = collections.defaultdict(list)
    grid = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        grid.setdefault(r["Kernel_Name"], set()).add(int(r["Grid_Size"]))
    return agg, grid


def traffic(fetch_path, write_path, calib_bytes, write_factor=1.0):
    fetch, _ = _per_kernel(fetch_path, "FETCH_SIZE")
    write, _ = _per_kernel(write_path, "WRITE_SIZE")
    cal = [k for k in fetch if "stream_read" in k]
    if not cal:
        raise SystemExit("no streaming-read dispatch in %s" % fetch_path)
    fetch_factor = calib_bytes / (sum(fetch[cal[0]]) / len(fetch[cal[0]]) * 1024.0)
    out = ["fetch factor (bytes per counted byte; streaming read of %d B): %.4f" % (calib_bytes, fetch_factor),
           "write factor: %.4f" % write_factor,
           "%-90s %16s %16s" % ("kernel", "fetch_bytes", "write_bytes")]
    for k in sorted(fetch):
        if "tq" not in k and "stream_read" not in k:
            continue
        f = sum(fetch[k]) / len(fetch[k]) * 1024.0 * fetch_factor
        w = sum(write.get(k, [0])) / max(1, len(write.get(k, [0]))) * 1024.0 * write_factor
        out.append("%-90s %16.6g %16.6g" % (short(k), f, w))
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--write-factor", type=float, default=1.0)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats(a.csv))
    else:
        print(traffic(a.fetch_csv, a.write_csv, a.calib_bytes, a.write_factor))


if __name__ == "__main__":
    sys.exit(main())
