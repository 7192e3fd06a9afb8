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


# ---------------------------------------------------------------------------- table
# Per-kernel counter table of `bench.py --pmc-probe` (one 16,384-token segment forward
# and backward at d_model 1024 shapes, then the two projections at L = 8192), from five
# runs: kernel trace, FETCH_SIZE, WRITE_SIZE, and two SQ counter sets.  Kernels that
# run twice per step under one name (the conv pre-pass of each pass, the scan of each
# pass) are told apart by their order inside the step.
PROBE_TOKENS = 16384
PROBE_LABELS = {  # (kernel, occurrence in the step) -> label
    ("conv_fwd_kernel<bf16_t, 4>", 0): "conv pre-pass (fwd: B, C)",
    ("conv_fwd_kernel<bf16_t, 4>", 1): "conv pre-pass (bwd: B, C)",
    ("dt_prepass_kernel<bf16_t>", 0): "dt table (fwd)",
    ("walk_kernel<bf16_t, 64, 128, 0>", 0): "walk_state (fwd)",
    ("walk_kernel<bf16_t, 64, 128, 1>", 0): "walk_out (fwd)",
    ("scan_kernel", 0): "scan (fwd, sub-segments)",
    ("scan_kernel", 1): "scan (bwd, chunk groups)",
    ("group_state_kernel<bf16_t, 64, 128, false, 2, true>", 0): "chunk_states (bwd)",
    ("group_state_kernel<bf16_t, 64, 128, true, 2, false>", 0): "dstate (bwd)",
    ("scan_rev_kernel", 0): "scan_rev (bwd)",
    ("bwd_main_kernel<bf16_t, 64, 128, 8>", 0): "bwd_main (bwd)",
    ("conv_bwd_kernel<bf16_t, true>", 0): "conv_bwd (bwd)",
    ("linear_kernel<LinShape<128, 128, 2, 2, 2, 2, true>, false, false, false, false, false, false>", 0):
        "in_proj 8192x4384x1024",
    ("linear_kernel<LinShape<128, 128, 2, 2, 2, 2, true>, false, false, false, false, false, false>", 1):
        "out_proj 8192x1024x2048",
}
# algorithmic bytes per token of each kernel's own inputs and outputs (bf16, d_model 1024
# shapes; fp16 in-group states of 64 x 128 per chunk of 64 and head, 32 heads)
_STATE = 32 * 64 * 128 * 2 // 64
PROBE_ALG_BYTES_PER_TOKEN = {
    "conv pre-pass (fwd: B, C)": 512 + 512,
    "conv pre-pass (bwd: B, C)": 512 + 512 + 512,
    "dt table (fwd)": 64 + 128,
    "walk_state (fwd)": 4096 + 256 + 128,
    "walk_out (fwd)": 4608 + 4096 + 128 + 4096,
    # raw x in, post-conv x out (the S walk convolves x for the main backward kernel)
    "chunk_states (bwd)": 4096 + 256 + 64 + _STATE + 4096,
    "dstate (bwd)": 512 + 4096 + 4096 + 64 + _STATE,
    "bwd_main (bwd)": 4096 + 768 + 4096 + 4096 + 64 + 2 * _STATE + 4096 + 4096 + 64 + 1024,
    "conv_bwd (bwd)": 4608 + 4096 + 1024 + 4608,
}
PROBE_ALG_BYTES = {  # the projections: operands and result once
    "in_proj 8192x4384x1024": 2 * (8192 * 1024 + 4384 * 1024 + 8192 * 4384),
    "out_proj 8192x1024x2048": 2 * (8192 * 2048 + 1024 * 2048 + 8192 * 1024),
}
CLOCK_HZ = 2.4e9
SIMDS = 256 * 4
HBM_PEAK = 8.0e12


def _dispatches(db: str):
    """[(dispatch_id, short kernel name)] in dispatch order, and {dispatch_id: {counter: value}}."""
    con = sqlite3.connect(db)
    vals = {}
    names = {}
    for d, k, c, v in con.execute("select dispatch_id, kernel_name, counter_name, sum(value) from "
                                  "counters_collection group by dispatch_id, kernel_name, counter_name"):
        vals.setdefault(d, {})[c] = v
        names[d] = short_name(k)
    return sorted(names.items()), vals


def _labelled(db: str):
    """{label: [counter dicts]} with labels from PROBE_LABELS (occurrence within each step)."""
    order, vals = _dispatches(db)
    out, seen, steps = {}, {}, 0
    for d, k in order:
        if k.startswith("bwd_main"):
            steps += 1
        key = (k, seen.get((k, steps), 0))
        seen[(k, steps)] = key[1] + 1
        lab = PROBE_LABELS.get(key) or PROBE_LABELS.get((k, key[1] % 2))
        if lab and "copyBuffer" not in k:
            out.setdefault(lab, []).append(vals[d])
        if "copyBuffer" in k:
            out.setdefault("copy", []).append(vals[d])
    return out


def _trace_durations(db: str):
    con = sqlite3.connect(db)
    out = {}
    order = list(con.execute("select name, duration from kernels order by start"))
    seen, steps = {}, 0
    for n, du in order:
        k = short_name(n)
        if k.startswith("bwd_main"):
            steps += 1
        occ = seen.get((k, steps), 0)
        seen[(k, steps)] = occ + 1
        lab = PROBE_LABELS.get((k, occ)) or PROBE_LABELS.get((k, occ % 2))
        if lab:
            out.setdefault(lab, []).append(du)
    return out


def report_table(trace, fetch, write, inst, util, copy_bytes, cmds, title):
    mean = lambda xs: sum(xs) / len(xs) if xs else float("nan")
    cval = lambda rows, c: mean([r.get(c, 0.0) for r in rows])
    dur = _trace_durations(trace)
    F, W, I, U = _labelled(fetch), _labelled(write), _labelled(inst), _labelled(util)
    f_scale = copy_bytes / (max(r["FETCH_SIZE"] for r in F["copy"]) * 1024.0)
    w_scale = copy_bytes / (max(r["WRITE_SIZE"] for r in W["copy"]) * 1024.0)
    out = [f"# {title}", "", "Commands (from the repository root on one MI355X; one counter set per run):", "",
           "```", *cmds, "```", "",
           f"Byte counters are scaled by what they read for a plain device copy of {copy_bytes} bytes in the "
           f"same run: FETCH_SIZE x {f_scale:.3f}, WRITE_SIZE x {w_scale:.3f}.  MFMA figures: flops = 512 x "
           "SQ_INSTS_VALU_MFMA_MOPS_BF16 (16,384 per 16x16x32 instruction); SQ_VALU_MFMA_BUSY_CYCLES counts "
           "SIMD cycles at 1,024 flops each, so MFMA busy = busy cycles / (duration x 2.4 GHz x 1,024 SIMDs).  "
           "VALU issue = SQ_INSTS_VALU x 4 cycles / (duration x 2.4 GHz x 1,024 SIMDs).  LDS conflict = "
           "SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS.  Algorithmic bytes: each kernel's own inputs and "
           "outputs, read or written once (the state kernels include their in-group state tiles).", "",
           "| kernel | avg us | HBM MB (counters) | alg MB | counter / alg | HBM TB/s | MFMA TFLOP/s | MFMA busy | "
           "VALU issue | LDS conflict | VALU insts / MFMA insts |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    labels = [l for l in list(PROBE_ALG_BYTES_PER_TOKEN) + list(PROBE_ALG_BYTES) if l in F]
    recs = {}
    for lab in labels:
        us = mean(dur.get(lab, [])) / 1e3
        hbm = cval(F[lab], "FETCH_SIZE") * 1024 * f_scale + cval(W[lab], "WRITE_SIZE") * 1024 * w_scale
        alg = PROBE_ALG_BYTES_PER_TOKEN.get(lab, 0) * PROBE_TOKENS or PROBE_ALG_BYTES.get(lab, 0)
        flops = 512 * cval(U[lab], "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        busy = cval(U[lab], "SQ_VALU_MFMA_BUSY_CYCLES")
        cyc = us * 1e-6 * CLOCK_HZ * SIMDS
        valu = cval(I[lab], "SQ_INSTS_VALU")
        mfma_i = cval(I[lab], "SQ_INSTS_MFMA")
        conf = cval(U[lab], "SQ_LDS_BANK_CONFLICT") / max(cval(U[lab], "SQ_ACTIVE_INST_LDS"), 1.0)
        rec = dict(us=us, hbm=hbm, alg=alg, tbs=hbm / (us * 1e-6) / 1e12, tflops=flops / (us * 1e-6) / 1e12,
                   mfma_busy=busy / cyc, valu_issue=valu * 4 / cyc, lds_conflict=conf,
                   valu_per_mfma=valu / max(mfma_i, 1.0))
        recs[lab] = rec
        out.append(f"| {lab} | {us:.1f} | {hbm / 1e6:.1f} | {alg / 1e6:.1f} | {hbm / alg:.2f} | {rec['tbs']:.2f} | "
                   f"{rec['tflops']:.0f} | {100 * rec['mfma_busy']:.1f}% | {100 * rec['valu_issue']:.1f}% | "
                   f"{conf:.2f} | {rec['valu_per_mfma']:.1f} |")
    out += ["", "Machine-readable:", "", "```json", json.dumps(recs), "```"]
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
    t = sub.add_parser("table")
    for k in ("trace", "fetch", "write", "inst", "util"):
        t.add_argument("--" + k, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--cmd", action="append", required=True)
    t.add_argument("--title", required=True)
    a = ap.parse_args()
    if a.what == "table":
        print(report_table(a.trace, a.fetch, a.write, a.inst, a.util, a.copy_bytes, a.cmd, a.title), end="")
        return
    if a.what == "stats":
        print(report_stats(a.db, a.cmd, a.title), end="")
    else:
        print(report_bytes(a.fetch, a.write, a.kernel, a.copy_bytes, a.cmd_fetch, a.cmd_write,
                           a.title), end="")


if __name__ == "__main__":
    main()
