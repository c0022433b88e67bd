"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python -m expert_ffn_dispatch_amd.profiling stats  <kernel_stats.csv> <out.md> "<command>" [<kernel_trace.csv>]
    python -m expert_ffn_dispatch_amd.profiling traffic <fetch counter_collection.csv>
        <write counter_collection.csv> <kernel substring> <copy bytes> <out.txt> "<command>"
    python -m expert_ffn_dispatch_amd.profiling counters <out.md> "<command>" "<note>"
        <kernel substrings, separated by ;> <counter_collection.csv> [...]

Traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the named kernel,
each scaled by bytes / counter for a plain device copy of known size run in
the same process (the copy reads and writes `copy bytes`).  The summary
records a hash of the grouped expert kernels' sources so that a reader can
tell when the counters no longer describe the built kernels.
"""
import csv
import hashlib
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))


# sources of the grouped expert kernels, whose launch the traffic figures describe
FFN_SOURCES = ("ffn.hip", "ffn_stream.h", "ffn_common.h", "common.h", "kernels.h")


def source_hash() -> str:
    h = hashlib.sha256()
    for name in FFN_SOURCES:
        with open(os.path.join(PKG, "csrc", name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def _trace_durations(trace_csv: str):
    """kernel name -> list of dispatch durations (ns), in dispatch order."""
    out = {}
    if not trace_csv or not os.path.exists(trace_csv):
        return out
    for r in csv.DictReader(open(trace_csv)):
        out.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def summarize_stats(stats_csv: str, out_md: str, command: str, trace_csv: str = "") -> str:
    """Per-kernel table from the --stats summary; with the kernel trace also
    the median dispatch and the mean without the first dispatch (the first
    call of a kernel runs on cold caches and clocks)."""
    rows = list(csv.DictReader(open(stats_csv)))
    dur = _trace_durations(trace_csv)
    lines = [f"# rocprofv3 kernel statistics", "", f"command: `{command}`", "",
             "| kernel | calls | avg us | median us | avg w/o first us | min us | max us | share % |",
             "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        d = dur.get(r["Name"], [])
        med = f"{statistics.median(d) / 1e3:.1f}" if d else "-"
        rest = f"{statistics.mean(d[1:]) / 1e3:.1f}" if len(d) > 1 else "-"
        lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {med} | {rest} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    text = "\n".join(lines) + "\n"
    with open(out_md, "w") as f:
        f.write(text)
    return text


def _counter_values(path: str, counter: str):
    """kernel name -> list of per-dispatch values of `counter`."""
    out = {}
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _copy_kernel(vals):
    cands = [k for k in vals if "copy" in k.lower() or "elementwise" in k.lower()]
    return max(cands, key=lambda k: statistics.median(vals[k])) if cands else None


def summarize_traffic(fetch_csv: str, write_csv: str, kernel: str, copy_bytes: int, out_txt: str,
                      command: str) -> dict:
    f = _counter_values(fetch_csv, "FETCH_SIZE")
    w = _counter_values(write_csv, "WRITE_SIZE")
    kf = [k for k in f if kernel in k]
    kw = [k for k in w if kernel in k]
    if not kf or not kw:
        raise SystemExit(f"kernel {kernel!r} not found in counters")
    cf, cw = _copy_kernel(f), _copy_kernel(w)
    fetch_kib = statistics.median(f[kf[0]])
    write_kib = statistics.median(w[kw[0]])
    copy_fetch_kib = statistics.median(f[cf])
    copy_write_kib = statistics.median(w[cw])
    sf = copy_bytes / (copy_fetch_kib * 1024.0)
    sw = copy_bytes / (copy_write_kib * 1024.0)
    res = {
        "kernel": kf[0][:120],
        "fetch_kib_per_dispatch": fetch_kib, "write_kib_per_dispatch": write_kib,
        "copy_kernel": cf[:120], "copy_bytes": copy_bytes,
        "copy_fetch_kib": copy_fetch_kib, "copy_write_kib": copy_write_kib,
        "fetch_scale": sf, "write_scale": sw,
        "fetch_bytes": fetch_kib * 1024.0 * sf, "write_bytes": write_kib * 1024.0 * sw,
        "traffic_bytes": fetch_kib * 1024.0 * sf + write_kib * 1024.0 * sw,
        "kernel_source_hash": source_hash(),
        "command": command,
    }
    with open(out_txt, "w") as fh:
        fh.write("# HBM traffic of one dispatch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE\n")
        for k, v in res.items():
            fh.write(f"{k}: {v}\n")
    return res


def summarize_counters(counter_csvs, kernels, out_md: str, command: str, note: str = "") -> str:
    """Median per dispatch of every counter in the given counter_collection
    CSVs (one per --pmc pass) for each kernel whose name contains one of
    `kernels`; one markdown table, kernels as columns."""
    vals = {}
    for path in counter_csvs:
        for r in csv.DictReader(open(path)):
            for k in kernels:
                if k in r["Kernel_Name"]:
                    vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    names = sorted({c for v in vals.values() for c in v})
    lines = ["# rocprofv3 counters per dispatch (median)", "", f"command: `{command}`", ""]
    if note:
        lines += [note, ""]
    lines += ["| counter | " + " | ".join(kernels) + " |", "|---|" + "---|" * len(kernels)]
    for c in names:
        cells = [f"{statistics.median(vals[k][c]):.4g}" if c in vals.get(k, {}) else "-" for k in kernels]
        lines.append(f"| {c} | " + " | ".join(cells) + " |")
    text = "\n".join(lines) + "\n"
    with open(out_md, "w") as fh:
        fh.write(text)
    return text


def read_traffic(path: str):
    """Parse a traffic summary; None if missing or taken on other kernel sources."""
    if not os.path.exists(path):
        return None
    d = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            d[k.strip()] = v.strip()
    if d.get("kernel_source_hash") != source_hash():
        return None
    return d


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        # stats <kernel_stats.csv> <out.md> "<command>" [<kernel_trace.csv>]
        print(summarize_stats(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5] if len(sys.argv) > 5 else ""))
    elif sys.argv[1] == "traffic":
        print(summarize_traffic(sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5]), sys.argv[6], sys.argv[7]))
    elif sys.argv[1] == "counters":
        # counters <out.md> "<command>" "<note>" <kernel substrings separated by ;> <csv> [<csv> ...]
        print(summarize_counters(sys.argv[6:], sys.argv[5].split(";"), sys.argv[2], sys.argv[3], sys.argv[4]))
    else:
        raise SystemExit(__doc__)
