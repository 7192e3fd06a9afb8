"""Summaries of rocprofv3 output databases (SQLite) for the kernels of this library.

Two reports, both short Markdown text:

* ``stats``: the kernel-trace statistics (calls, total / mean duration) of one run.
* ``bytes``: HBM bytes per dispatch of one kernel from two counter runs, FETCH_SIZE
  and WRITE_SIZE (KiB per dispatch, as rocprofv3 reports them).  Each counter is
  scaled by what it reads for a plain device copy of known size in the same run
  (the largest ``copyBuffer`` dispatch), so the figure is in real bytes.  The report
  ends with a JSON block that ``bench.py`` reads, including a fingerprint of the
  kernel's sources: once the sources change, the figure no longer applies.

Usage::

    python -m selective_state_space_15_amd.profiling stats DB --cmd CMD --title TITLE
    python -m selective_state_space_15_amd.profiling bytes --fetch DB --write DB \\
        --kernel bwd_main_kernel --copy-bytes 268435456 --cmd-fetch CMD --cmd-write CMD \\
        --title TITLE
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sqlite3

_HERE = os.path.dirname(os.path.abspath(__file__))

# Sources whose text defines each profiled kernel (the fingerprint covers all of them).
KERNEL_SOURCES = {
    "bwd_main_kernel": ["csrc/bwd.hip", "csrc/common.hpp", "csrc/chunk_io.hpp", "csrc/launch.hpp"],
    "walk_kernel": ["csrc/fwd.hip", "csrc/common.hpp", "csrc/chunk_io.hpp", "csrc/launch.hpp"],
    "conv_bwd_kernel": ["csrc/conv.hip", "csrc/common.hpp", "csrc/launch.hpp"],
}


def source_fingerprint(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(_HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    if "at::native" in name:
        return "torch: " + name.replace("void ", "").split("<")[0].split("::")[-1]
    m = name.replace("void ", "").replace("ssd::(anonymous namespace)::", "").replace("ssd::", "")
    return m.split("(")[0]


def kernel_stats(db: str):
    con = sqlite3.connect(db)
    return list(con.execute(
        "select name, total_calls, total_duration, average, percentage from top_kernels"))


def pmc_per_dispatch(db: str, counter: str):
    """[(dispatch_id, kernel_name, value)] for one counter."""
    con = sqlite3.connect(db)
    return list(con.execute(
        "select dispatch_id, kernel_name, sum(value) from counters_collection "
        "where counter_name = ? group by dispatch_id, kernel_name order by dispatch_id", (counter,)))


def _kernel_mean(rows, kernel: str):
    vals = [v for _, n, v in rows if re.search(r"\b" + re.escape(kernel) + r"\b", n)]
    if not vals:
        raise SystemExit(f"no dispatch of {kernel}")
    return sum(vals) / len(vals), len(vals)


def _copy_value(rows):
    copies = [(v, n) for _, n, v in rows if "copyBuffer" in n]
    if not copies:
        raise SystemExit("no copyBuffer dispatch to calibrate against")
    return max(copies)[0]


def report_stats(db, cmd, title):
    out = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "", "```", cmd,
           "```", "",
           "rocprofv3 kernel statistics (durations in microseconds; torch's own input "
           "kernels included):", "", "| kernel | calls | total us | avg us | % |",
           "|---|---|---|---|---|"]
    for n, c, t, a, p in kernel_stats(db):
        out.append(f"| {short_name(n)} | {c} | {t:.1f} | {a:.1f} | {p:.1f} |")
    return "\n".join(out) + "\n"


def report_bytes(fetch_db, write_db, kernel, copy_bytes, cmd_fetch, cmd_write, title):
    fr, wr = pmc_per_dispatch(fetch_db, "FETCH_SIZE"), pmc_per_dispatch(write_db, "WRITE_SIZE")
    f_kib, nf = _kernel_mean(fr, kernel)
    w_kib, nw = _kernel_mean(wr, kernel)
    f_copy, w_copy = _copy_value(fr), _copy_value(wr)
    f_scale = copy_bytes / (f_copy * 1024.0)
    w_scale = copy_bytes / (w_copy * 1024.0)
    fetch_b = f_kib * 1024.0 * f_scale
    write_b = w_kib * 1024.0 * w_scale
    rec = {"kernel": kernel, "fetch_kib": f_kib, "write_kib": w_kib, "fetch_scale": f_scale,
           "write_scale": w_scale, "fetch_bytes": fetch_b, "write_bytes": write_b,
           "hbm_bytes_per_launch": fetch_b + write_b, "dispatches": [nf, nw],
           "source_fingerprint": source_fingerprint(kernel)}
    out = [f"# {title}", "",
           "Two counter runs (one counter each), from the repository root on one MI355X:", "",
           "```", cmd_fetch, cmd_write, "```", "",
           f"Calibration: a plain device copy of {copy_bytes} bytes in the same run reads "
           f"FETCH_SIZE = {f_copy:.1f} KiB and WRITE_SIZE = {w_copy:.1f} KiB, so the scale "
           f"factors are {f_scale:.3f} (fetch) and {w_scale:.3f} (write).", "",
           "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | fetch bytes | write bytes | "
           "HBM bytes per launch |", "|---|---|---|---|---|---|---|",
           f"| {kernel} | {nf} / {nw} | {f_kib:.1f} | {w_kib:.1f} | {fetch_b:.4g} | {write_b:.4g} | "
           f"{fetch_b + write_b:.4g} |", "",
           "Machine-readable (read by bench.py; valid while the source fingerprint matches):", "",
           "```json", json.dumps(rec), "```"]
    return "\n".join(out) + "\n"


def read_bytes_report(path: str):
    """The JSON record of a `bytes` report, or None."""
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, flags=re.S)
    return json.loads(m.group(1)) if m else None


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("db")
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", required=True)
    b = sub.add_parser("bytes")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernel", required=True)
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--cmd-fetch", required=True)
    b.add_argument("--cmd-write", required=True)
    b.add_argument("--title", required=True)
    a = ap.parse_args()
    if a.what == "stats":
        print(report_stats(a.db, a.cmd, a.title), end="")
    else:
        print(report_bytes(a.fetch, a.write, a.kernel, a.copy_bytes, a.cmd_fetch, a.cmd_write,
                           a.title), end="")


if __name__ == "__main__":
    main()
