"""Summaries of rocprofv3 CSV output for profiles/ (measurement tooling).

    python -m flashattention_backward_fa_amd.profile_summary traffic \
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \
        --kernels dkdv_kernel,dq_ds_kernel --workload gqa_causal --out FILE

    python -m flashattention_backward_fa_amd.profile_summary trace \
        --stats DIR --workload gqa_causal --out FILE [--bench-json FILE]

    python -m flashattention_backward_fa_amd.profile_summary mfma \
        --pmc DIR --kernels dkdv_kernel,dq_ds_kernel --workload gqa_causal --out FILE

    python -m flashattention_backward_fa_amd.profile_summary counters \
        --pmc DIR --kernels dkdv_kernel,dq_ds_kernel --workload gqa_causal --out FILE

trace: the per-kernel table of a --kernel-trace --stats run (calls, average,
min and max duration, share of GPU time), with the kernel source hash and,
when given, the bench.py JSON line of the same build.

--sources selects whose source hash is recorded: the default attention
kernels ("det") or Floyd attention ("floyd"); trace --match keeps only the
kernels whose names contain one of the given substrings.

mfma: MFMA-pipe utilisation per kernel from a --pmc GRBM_GUI_ACTIVE
SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA run.  SQ_VALU_MFMA_BUSY_CYCLES is the
sum over all 1024 SIMDs (it equals 32 cycles per v_mfma_f32_32x32x16_bf16
counted by SQ_INSTS_MFMA); GRBM_GUI_ACTIVE is the sum over the 8 XCDs, so a
kernel's elapsed shader cycles are GRBM_GUI_ACTIVE / 8 (divided by the
dispatch's duration this gives the shader clock, also reported).

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the named kernels are scaled
by what the same counters read for a plain device copy of known size (bench.py
--copy-calibration: 256 MiB read and written per launch) and written out with
the hash of the kernel source they were taken from; bench.py reports the
traffic only while that hash matches the current source.
"""

import argparse
import csv
import hashlib
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "flashattention_backward_fa_amd", "csrc")
# the sources the timed dK/dV and dQ kernels are compiled from
KERNEL_SRCS = tuple(os.path.join(CSRC, f) for f in ("fa_bwd_dkdv.h", "fa_bwd_dkdv_kernels.hip",
                                                    "fa_bwd_dkdv192_kernels.hip", "fa_bwd_det_kernels.hip",
                                                    "fa_bwd_tiles.h", "fa_bwd_schedule.h", "fa_bwd_internal.h"))
# the sources the Floyd attention kernels are compiled from
FLOYD_SRCS = tuple(os.path.join(CSRC, f) for f in ("fa_floyd_kernels.hip", "fa_floyd_internal.h", "fa_bwd_tiles.h",
                                                   "fa_bwd_schedule.h", "fa_bwd_internal.h"))
# the sources of the fused small-sequence kernel
FUSED_SRCS = tuple(os.path.join(CSRC, f) for f in ("fa_bwd_fused_kernels.hip", "fa_bwd_tiles.h",
                                                   "fa_bwd_schedule.h", "fa_bwd_internal.h", "fa_bwd_kernarg.h"))
SOURCES = {"det": KERNEL_SRCS, "floyd": FLOYD_SRCS, "fused": FUSED_SRCS}
COPY_BYTES = 256 << 20
XCDS = 8        # MI355X: 8 XCDs of 32 CUs
SIMDS = 1024    # 256 CUs x 4 SIMDs


def kernel_code_hash(paths=KERNEL_SRCS):
    """sha256 (16 hex digits) of the kernel sources with comments and blank
    lines removed: a summary stays valid across comment-only edits and goes
    stale on any change to the code."""
    parts = []
    for path in paths:
        text = open(path, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
        parts.append("\n".join(ln for ln in lines if ln.strip()))
    return hashlib.sha256("\n\f\n".join(parts).encode("utf-8")).hexdigest()[:16]


def _names(arg):
    """Kernel name substrings: separated by ';' when one is present (template
    arguments hold commas), else by ','."""
    return [n for n in arg.split(";" if ";" in arg else ",") if n]


def _rows(d):
    path = os.path.join(d, "run_counter_collection.csv")
    return list(csv.DictReader(open(path)))


def _per_dispatch(d, counter, match):
    vals = {}
    for r in _rows(d):
        if r["Counter_Name"] == counter and match(r["Kernel_Name"]):
            vals.setdefault(int(r["Dispatch_Id"]), 0.0)
            vals[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return list(vals.values())


def traffic(args):
    names = _names(args.kernels)
    cf = statistics.median(_per_dispatch(args.copy_fetch, "FETCH_SIZE", lambda n: "copyBuffer" in n))
    cw = statistics.median(_per_dispatch(args.copy_write, "WRITE_SIZE", lambda n: "copyBuffer" in n))
    f_scale = COPY_BYTES / (cf * 1024.0)
    w_scale = COPY_BYTES / (cw * 1024.0)
    lines = []
    per_kernel = []
    total = 0.0
    for n in names:
        f = statistics.median(_per_dispatch(args.fetch, "FETCH_SIZE", lambda k, n=n: n in k))
        w = statistics.median(_per_dispatch(args.write, "WRITE_SIZE", lambda k, n=n: n in k))
        fb, wb = f * 1024.0 * f_scale, w * 1024.0 * w_scale
        total += fb + wb
        lines.append(f"# {n}: FETCH_SIZE {f:.0f} KiB -> {fb / 2**20:.1f} MiB, WRITE_SIZE {w:.0f} KiB -> {wb / 2**20:.1f} MiB")
        per_kernel.append(f"hbm_bytes_per_launch.{n}: {fb + wb:.0f}")
    src_hash = kernel_code_hash(SOURCES[args.sources])
    out = [
        f"# HBM traffic per launch of {'+'.join(names)}, workload {args.workload}",
        f"# command: {args.command}",
        f"# calibration: copy of {COPY_BYTES >> 20} MiB reads FETCH_SIZE {cf:.0f} KiB (scale {f_scale:.3f}),",
        f"#   WRITE_SIZE {cw:.0f} KiB (scale {w_scale:.3f})",
        *lines,
        f"kernel_code_sha256_16: {src_hash}",
        f"hbm_bytes_per_launch: {total:.0f}",
        *per_kernel,
    ]
    text = "\n".join(out) + "\n"
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(text)
    sys.stdout.write(text)


def _short(name):
    for ns in ("fabwd", "ffloyd"):
        name = name.replace(ns + "::(anonymous namespace)::", "").replace(ns + "::", "")
    return name[:64]


def trace(args):
    rows = list(csv.DictReader(open(os.path.join(args.stats, "run_kernel_stats.csv"))))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    if args.match:
        rows = [r for r in rows if any(m in r["Name"] for m in _names(args.match))]
    src_hash = kernel_code_hash(SOURCES[args.sources])
    out = [
        f"# rocprofv3 kernel-trace summary, workload {args.workload}",
        f"# command: {args.command}",
        "# columns: kernel | calls | average us | min us | max us | share of GPU time",
    ]
    for r in rows:
        out.append(f"{_short(r['Name']):64s} | {int(r['Calls']):4d} | {float(r['AverageNs']) / 1e3:9.1f} | "
                   f"{float(r['MinNs']) / 1e3:9.1f} | {float(r['MaxNs']) / 1e3:9.1f} | {float(r['Percentage']):5.1f}%")
    out.append(f"kernel_code_sha256_16: {src_hash}")
    if args.bench_json:
        lines = [ln for ln in open(args.bench_json).read().splitlines() if ln.startswith("{")]
        out.append("bench.py line of this build: " + (lines[-1] if lines else "(none)"))
    text = "\n".join(out) + "\n"
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(text)
    sys.stdout.write(text)


def mfma(args):
    names = _names(args.kernels)
    rows = _rows(args.pmc)
    src_hash = kernel_code_hash(SOURCES[args.sources])
    out = [f"# MFMA-pipe utilisation per kernel, workload {args.workload}", f"# command: {args.command}",
           "# columns: kernel | MFMA instructions | MFMA busy cycles (all SIMDs) | elapsed cycles | "
           "utilisation | clock GHz"]
    tot_busy = tot_el = 0.0
    for n in names:
        match = lambda k, n=n: n in k  # noqa: E731
        busy = statistics.median(_per_dispatch(args.pmc, "SQ_VALU_MFMA_BUSY_CYCLES", match))
        gui = statistics.median(_per_dispatch(args.pmc, "GRBM_GUI_ACTIVE", match))
        insts = statistics.median(_per_dispatch(args.pmc, "SQ_INSTS_MFMA", match))
        durs = {}
        for r in rows:
            if match(r["Kernel_Name"]):
                durs[int(r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        dur_ns = statistics.median(durs.values())
        elapsed = gui / XCDS
        util = busy / (elapsed * SIMDS)
        tot_busy += busy
        tot_el += elapsed
        out.append(f"{n:40s} | {insts:12.0f} | {busy:14.0f} | {elapsed:11.0f} | {100 * util:5.1f} % | "
                   f"{elapsed / dur_ns:4.2f}")
        if dur_ns < 50_000:
            out.append(f"# {n}: a {dur_ns / 1000:.1f} us dispatch; the counters' window around it is longer than "
                       "the dispatch, so elapsed cycles and clock are overstated and utilisation understated")
    out.append(f"{'pair' if len(names) == 2 else 'combined'}_mfma_utilisation: {100 * tot_busy / (tot_el * SIMDS):.1f} %")
    out.append(f"kernel_code_sha256_16: {src_hash}")
    text = "\n".join(out) + "\n"
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(text)
    sys.stdout.write(text)


def counters(args):
    """Median per dispatch of every counter of a --pmc run, per named kernel."""
    names = _names(args.kernels)
    rows = _rows(args.pmc)
    src_hash = kernel_code_hash(SOURCES[args.sources])
    cnames = sorted({r["Counter_Name"] for r in rows})
    out = [f"# counters per dispatch (median over dispatches), workload {args.workload}", f"# command: {args.command}",
           "# columns: kernel | " + " | ".join(cnames)]
    for n in names:
        vals = [statistics.median(_per_dispatch(args.pmc, c, lambda k, n=n: n in k)) for c in cnames]
        out.append(f"{n:24s} | " + " | ".join(f"{v:.0f}" for v in vals))
    out.append(f"kernel_code_sha256_16: {src_hash}")
    text = "\n".join(out) + "\n"
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(text)
    sys.stdout.write(text)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    for k in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--kernels", "--workload"):
        t.add_argument(k, required=True)
    t.add_argument("--out")
    t.add_argument("--sources", choices=sorted(SOURCES), default="det")
    t.add_argument("--command", default="(see profiles/README.md)")
    tr = sub.add_parser("trace")
    tr.add_argument("--stats", required=True)
    tr.add_argument("--workload", required=True)
    tr.add_argument("--bench-json")
    tr.add_argument("--out")
    tr.add_argument("--sources", choices=sorted(SOURCES), default="det")
    tr.add_argument("--match", help="comma-separated substrings: keep only kernels whose name holds one")
    tr.add_argument("--command", default="(see profiles/README.md)")
    m = sub.add_parser("mfma")
    for k in ("--pmc", "--kernels", "--workload"):
        m.add_argument(k, required=True)
    m.add_argument("--out")
    m.add_argument("--sources", choices=sorted(SOURCES), default="det")
    m.add_argument("--command", default="(see profiles/README.md)")
    c = sub.add_parser("counters")
    for k in ("--pmc", "--kernels", "--workload"):
        c.add_argument(k, required=True)
    c.add_argument("--out")
    c.add_argument("--sources", choices=sorted(SOURCES), default="det")
    c.add_argument("--command", default="(see profiles/README.md)")
    args = ap.parse_args()
    if args.cmd == "counters":
        counters(args)
    elif args.cmd == "traffic":
        traffic(args)
    elif args.cmd == "trace":
        trace(args)
    else:
        mfma(args)


if __name__ == "__main__":
    main()
