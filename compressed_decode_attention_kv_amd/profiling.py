"""Summaries of rocprofv3 output for the library's kernels.

  python -m compressed_decode_attention_kv_amd.profiling stats <kernel_stats.csv> [--last N]
  python -m compressed_decode_attention_kv_amd.profiling traffic <fetch counter_collection.csv> \
        <write counter_collection.csv> --calib-bytes N
  python -m compressed_decode_attention_kv_amd.profiling traffic-summary <fetch csv> <write csv> \
        --calib-bytes N --decode-bytes A --quantize-bytes Q --title "..." --command "..." [--command ...]
  python -m compressed_decode_attention_kv_amd.profiling counters <counter_collection.csv> [...]

Every summary lists every kernel of the run (the library's and any other,
e.g. the input generator's), keeping per kernel only the dispatches at its
largest grid size: the workload's full-size launch (a benchmark run also
makes small launches of the same kernels, e.g. one-token appends, which
would otherwise dominate the per-kernel averages and medians).  `stats`
prints, from the kernel trace beside the stats file, the average duration
per kernel over those dispatches and, with --last N, over the last N of
them as well: the timed steps of a benchmark run that makes no full-size
dispatch after them, i.e. the figure its HIP-event timing measures (the
first dispatches run while the clocks settle).  `traffic-summary` writes the
committed per-scheme summary: the traffic table, the decode chain's bytes
(query prep + split decode + combine), the quantize chain's bytes (the K and
V quantize launches of one step) and the hash of the sources of each chain
(a summary taken on other sources is not used).  `traffic` prints HBM bytes
per dispatch from the FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch),
the fetch side scaled by what the same counter reads for the library's
streaming-read kernel over a buffer of N bytes (non-temporal loads count at
half their size on this device), the write side by --write-factor (1.0: the
counter matches the known write volume of the quantize kernels).
`counters` prints, per kernel, the median over dispatches of rocprof's own
derived utilisations from SQ counters of one or more --pmc passes, each
computed within a dispatch against that dispatch's GRBM_GUI_ACTIVE:
  VALUBusy        = SQ_ACTIVE_INST_VALU / CUs / busy cycles
  LdsUtil         = SQ_LDS_IDX_ACTIVE / CUs / busy cycles
  LDSBankConflict = SQ_LDS_BANK_CONFLICT / CUs / busy cycles
  MfmaUtil        = SQ_VALU_MFMA_BUSY_CYCLES / SIMDs / busy cycles
The CSV sums GRBM_GUI_ACTIVE over the XCDs, so busy cycles are that sum over
the XCD count; CU, SIMD and XCD counts come from run_agent_info.csv beside it.
"""
import argparse
import collections
import csv
import hashlib
import os
import re
import sys

DECODE_SOURCES = ("decode_lut.hip", "decode.hip", "decode_mq.hip", "decode_mq_kernel.h", "decode_mq_wide.hip",
                  "device_common.h", "internal.h")
QUANTIZE_SOURCES = ("quant_mfma.hip", "quant.hip", "quant_sketch.hip", "device_common.h", "internal.h")
CHAIN = ("qprep_kernel", "decode_lut_kernel", "decode_mq_kernel", "decode_split_kernel", "sproj_kernel", "combine_kernel")
QCHAIN = ("quant_mfma_kernel", "quant_kernel", "quant_sketch_kernel")


def _sources_sha(files):
    h = hashlib.sha1()
    pkg = os.path.dirname(os.path.abspath(__file__))
    for f in files:
        h.update(open(os.path.join(pkg, "csrc", f), "rb").read())
    h.update(open(os.path.join(pkg, "build.py"), "rb").read())
    return h.hexdigest()


def decode_sources_sha():
    """sha1 over the sources of the decode chain's kernels and the build
    script (its per-source compiler flags shape the kernels too)."""
    return _sources_sha(DECODE_SOURCES)


def quantize_sources_sha():
    """sha1 over the sources of the quantize kernels and the build script."""
    return _sources_sha(QUANTIZE_SOURCES)


def short(name):
    # Names the profiler could not demangle (an fp16 template argument):
    # <len>quant_kernelILi<a>ELi<b>EDF16_EEvNS_11QuantParamsE.
    m = re.match(r"^(?:_ZN2tq12_GLOBAL__N_1)?\d*(\w+?)ILi(\d+)ELi(\d+)EDF16_EEvNS_\d+(\w+)E$", name)
    if m:
        name = "%s<%s, %s, _Float16>(tq::%s)" % m.groups()
    name = re.sub(r"^void ", "", name)
    name = name.replace("tq::(anonymous namespace)::", "")
    name = name.replace("_ZN2tq12_GLOBAL__N_1", "")
    return name[:90]


def _largest_grid(rows, grid_of):
    """The rows of each kernel's dispatches at that kernel's largest grid size."""
    top = {}
    for r in rows:
        k = r["Kernel_Name"]
        top[k] = max(top.get(k, 0), grid_of(r))
    return [r for r in rows if grid_of(r) == top[r["Kernel_Name"]]]


def _trace_grid(r):
    return int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])


def stats(path, last=None):
    """Calls and average duration per kernel (every kernel of the run), over
    the dispatches at its largest grid size, from run_kernel_trace.csv beside
    `path`; with `last`, also the average over the last `last` of them."""
    trace = os.path.join(os.path.dirname(path), "run_kernel_trace.csv")
    rows = sorted(csv.DictReader(open(trace)), key=lambda r: int(r["Start_Timestamp"]))
    calls = collections.Counter(r["Kernel_Name"] for r in rows)
    dur = collections.defaultdict(list)
    for r in _largest_grid(rows, _trace_grid):
        dur[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    head = "%-90s %6s %10s %14s" % ("kernel", "calls", "full-size", "avg_us")
    if last:
        head += " %18s" % ("avg_last%d_us" % last)
    out = [head]
    for k in sorted(dur, key=lambda k: -sum(dur[k])):
        line = "%-90s %6d %10d %14.2f" % (short(k), calls[k], len(dur[k]), sum(dur[k]) / len(dur[k]))
        if last:
            tail = dur[k][-last:]
            line += " %18.2f" % (sum(tail) / len(tail))
        out.append(line)
    return "\n".join(out)


def _per_kernel(path, counter):
    rows = _largest_grid([r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter],
                         lambda r: int(r["Grid_Size"]))
    agg = collections.defaultdict(list)
    for r in rows:
        agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return agg


def _traffic_table(fetch_path, write_path, calib_bytes, write_factor):
    fetch = _per_kernel(fetch_path, "FETCH_SIZE")
    write = _per_kernel(write_path, "WRITE_SIZE")
    cal = [k for k in fetch if "stream_read" in k]
    if not cal:
        raise SystemExit("no streaming-read dispatch in %s" % fetch_path)
    fetch_factor = calib_bytes / (sum(fetch[cal[0]]) / len(fetch[cal[0]]) * 1024.0)
    rows = []
    for k in sorted(fetch):
        f = sum(fetch[k]) / len(fetch[k]) * 1024.0 * fetch_factor
        w = sum(write.get(k, [0])) / max(1, len(write.get(k, [0]))) * 1024.0 * write_factor
        rows.append((short(k), f, w))
    return fetch_factor, rows


def traffic(fetch_path, write_path, calib_bytes, write_factor=1.0):
    fetch_factor, rows = _traffic_table(fetch_path, write_path, calib_bytes, write_factor)
    out = ["fetch factor (bytes per counted byte; streaming read of %d B): %.4f" % (calib_bytes, fetch_factor),
           "write factor: %.4f" % write_factor,
           "%-90s %16s %16s" % ("kernel", "fetch_bytes", "write_bytes")]
    out += ["%-90s %16.6g %16.6g" % r for r in rows]
    return "\n".join(out)


def traffic_summary(fetch_path, write_path, calib_bytes, algorithmic, qalgorithmic, title, commands,
                    write_factor=1.0):
    fetch_factor, rows = _traffic_table(fetch_path, write_path, calib_bytes, write_factor)
    chain = [r for r in rows if r[0].startswith(CHAIN)]
    cf = sum(r[1] for r in chain)
    cw = sum(r[2] for r in chain)
    qchain = [r for r in rows if r[0].startswith(QCHAIN)]
    qf = sum(r[1] for r in qchain)
    qw = sum(r[2] for r in qchain)
    out = ["# " + title]
    out += ["#   " + c for c in commands]
    out += ["# The fetch counter is scaled by the streaming-read kernel over %d bytes" % calib_bytes,
            "# (the packed planes' size; non-temporal loads count at half their size).",
            "#",
            "# fetch factor (bytes per counted byte): %.4f" % fetch_factor,
            "# write factor: %.4f" % write_factor,
            "# %-90s %16s %16s" % ("kernel", "fetch_bytes", "write_bytes")]
    out += ["# %-90s %16.6g %16.6g" % r for r in rows]
    out += ["#",
            "# decode chain = %s; algorithmic packed bytes = %d" % (" + ".join(r[0].split("(")[0] for r in chain),
                                                                   algorithmic),
            "decode_sources_sha1 = %s" % decode_sources_sha(),
            "decode_chain_fetch_bytes = %.6g" % cf,
            "decode_chain_write_bytes = %.6g" % cw,
            "decode_chain_bytes = %.6g" % (cf + cw),
            "ratio_to_algorithmic = %.4f" % ((cf + cw) / algorithmic),
            "#",
            "# quantize chain = %s (one K and one V launch); algorithmic bytes (inputs read + planes written) = %d"
            % (" + ".join(r[0].split("(")[0] for r in qchain), qalgorithmic),
            "quantize_sources_sha1 = %s" % quantize_sources_sha(),
            "quantize_chain_fetch_bytes = %.6g" % qf,
            "quantize_chain_write_bytes = %.6g" % qw,
            "quantize_chain_bytes = %.6g" % (qf + qw),
            "quantize_ratio_to_algorithmic = %.4f" % ((qf + qw) / qalgorithmic)]
    return "\n".join(out)


def _agent(path):
    info = os.path.join(os.path.dirname(path), "run_agent_info.csv")
    cu, simd, xcc = 256, 1024, 8
    if os.path.exists(info):
        for r in csv.DictReader(open(info)):
            if r.get("Agent_Type") == "GPU":
                cu, simd, xcc = int(r["Cu_Count"]), int(r["Simd_Count"]), int(r["Num_Xcc"])
    return cu, simd, xcc


_DERIVED = (  # name, numerator counter, divisor ("cu" or "simd")
    ("VALUBusy%", "SQ_ACTIVE_INST_VALU", "cu"),
    ("LdsUtil%", "SQ_LDS_IDX_ACTIVE", "cu"),
    ("LDSBankConflict%", "SQ_LDS_BANK_CONFLICT", "cu"),
    ("MfmaUtil%", "SQ_VALU_MFMA_BUSY_CYCLES", "simd"),
)


def counters(paths):
    """Per-kernel medians, over the dispatches at the kernel's largest grid
    size, of the VALU instruction count and of rocprof's derived utilisations
    (each computed within one dispatch)."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))   # kernel -> column -> values
    for path in paths:
        cu, simd, xcc = _agent(path)
        disp = collections.defaultdict(dict)
        names = {}
        rows = list(csv.DictReader(open(path)))
        for r in _largest_grid(rows, lambda r: int(r["Grid_Size"])):
            disp[r["Dispatch_Id"]][r["Counter_Name"]] = float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
        for did, c in disp.items():
            k = names[did]
            if "SQ_INSTS_VALU" in c:
                per[k]["VALU insts"].append(c["SQ_INSTS_VALU"])
            busy = c.get("GRBM_GUI_ACTIVE", 0.0) / xcc
            if busy <= 0:
                continue
            for name, num, unit in _DERIVED:
                if num in c:
                    per[k][name].append(100.0 * c[num] / (cu if unit == "cu" else simd) / busy)

    def median(v):
        v = sorted(v)
        return v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])

    cols = ["VALU insts"] + [d[0] for d in _DERIVED]
    out = ["# decode_sources_sha1 = %s" % decode_sources_sha(),
           "# quantize_sources_sha1 = %s" % quantize_sources_sha(),
           "%-90s %5s " % ("kernel", "disp") + " ".join("%16s" % c for c in cols)]
    for k in sorted(per):
        n = max(len(v) for v in per[k].values())
        out.append("%-90s %5d " % (short(k), n) +
                   " ".join(("%16.4g" % median(per[k][c])) if per[k].get(c) else "%16s" % "-" for c in cols))
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--last", type=int, default=None)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--write-factor", type=float, default=1.0)
    dt = sub.add_parser("traffic-summary")
    dt.add_argument("fetch_csv")
    dt.add_argument("write_csv")
    dt.add_argument("--calib-bytes", type=int, required=True)
    dt.add_argument("--decode-bytes", type=int, required=True)
    dt.add_argument("--quantize-bytes", type=int, required=True)
    dt.add_argument("--title", required=True)
    dt.add_argument("--command", action="append", default=[])
    dt.add_argument("--write-factor", type=float, default=1.0)
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats(a.csv, a.last))
    elif a.cmd == "counters":
        print(counters(a.csv))
    elif a.cmd == "traffic":
        print(traffic(a.fetch_csv, a.write_csv, a.calib_bytes, a.write_factor))
    else:
        print(traffic_summary(a.fetch_csv, a.write_csv, a.calib_bytes, a.decode_bytes, a.quantize_bytes, a.title,
                              a.command, a.write_factor))


if __name__ == "__main__":
    sys.exit(main())
