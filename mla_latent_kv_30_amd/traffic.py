"""HBM traffic of a kernel from rocprofv3 counter runs, for the roofline report.

Two counter passes of the same command (one with FETCH_SIZE, one with
WRITE_SIZE; each needs its own pass on the hardware) give kilobytes per
dispatch as the memory controller saw them.  Both are scaled by what the same
counter reads for a plain device copy of known size run in the same command
(bench.py --calibrate-copy copies 256 MiB), so the figure is in true bytes.

    python -m mla_latent_kv_30_amd.traffic summarize --fetch DIR --write DIR \\
        --kernel decode_mfma_kernel --workload decode_h16 --out profiles/X.json

The same module summarises a matrix-core counter run (mfma subcommand:
SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE) and an
LDS counter run (lds subcommand: SQ_INSTS_LDS, SQ_INSTS_LDS_LOAD_BANDWIDTH,
SQ_LDS_BANK_CONFLICT, SQ_ACTIVE_INST_LDS, GRBM_GUI_ACTIVE).

The summary records a digest of the sources the kernel is built from;
bench.py reports the traffic only while those sources still have that digest.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 256 << 20        # bench.py --calibrate-copy
COPY_KERNEL = "copyBuffer"    # the runtime's device-to-device copy kernel


# The sources each measured kernel is compiled from (its file and the headers
# it includes); other kernels are digested over every source.
KERNEL_SOURCES = {
    "decode_mfma_kernel": ("decode.hip", "decode_common.h", "common.h", "kernels.h"),
    "decode_wide_kernel": ("decode_wide.hip", "decode_common.h", "common.h", "kernels.h"),
    "decode_f32_kernel": ("decode.hip", "decode_common.h", "common.h", "kernels.h"),
    "linear_kernel": ("linear.hip", "common.h", "kernels.h"),
}


_COMMENTS = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def code_text(source: str) -> str:
    """The code of a C++/HIP source without its comments and with whitespace
    runs collapsed, so that an edit to comments alone leaves a digest as it
    was."""
    return " ".join(_COMMENTS.sub(" ", source).split())


def source_digest(kernel: str = "") -> str:
    """Digest of the code of the sources `kernel` is built from (every kernel
    source if unknown) and of the compiler flags they are built with."""
    from mla_latent_kv_30_amd import build as _build

    names = KERNEL_SOURCES.get(kernel)
    h = hashlib.sha256()
    h.update(" ".join(f for f in _build.CFLAGS if not os.path.isabs(f)).encode())
    for src in sorted(names or _build.FILE_FLAGS):
        h.update(" ".join(_build.FILE_FLAGS.get(src, [])).encode())
    for path in sorted(glob.glob(os.path.join(HERE, "csrc", "*"))):
        base = os.path.basename(path)
        if path.endswith((".hip", ".h")) and (names is None or base in names):
            h.update(base.encode())
            with open(path, encoding="utf-8") as f:
                h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def _counter_csv(run_dir: str) -> str:
    found = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not found:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    return found[0]


def per_dispatch(run_dir: str, counter: str, kernel_substr: str) -> list:
    """Values of `counter` for every dispatch whose kernel name contains kernel_substr."""
    vals = {}
    with open(_counter_csv(run_dir)) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter and kernel_substr in row["Kernel_Name"]:
                vals[int(row["Dispatch_Id"])] = vals.get(int(row["Dispatch_Id"]), 0.0) + float(row["Counter_Value"])
    return [vals[k] for k in sorted(vals)]


def _largest(vals: list) -> list:
    """The dispatches within 1% of the largest (one kernel run in two forms:
    keep the form that moves more bytes)."""
    top = max(vals) if vals else 0.0
    return [v for v in vals if v >= 0.99 * top]


def summarize(fetch_dir: str, write_dir: str, kernel: str, workload: str, largest: bool = False) -> dict:
    fk = per_dispatch(fetch_dir, "FETCH_SIZE", kernel)
    wk = per_dispatch(write_dir, "WRITE_SIZE", kernel)
    if largest:
        fk, wk = _largest(fk), _largest(wk)
    fc = per_dispatch(fetch_dir, "FETCH_SIZE", COPY_KERNEL)
    wc = per_dispatch(write_dir, "WRITE_SIZE", COPY_KERNEL)
    if not fk or not wk:
        raise RuntimeError(f"no dispatches of {kernel} in the counter runs")
    if not fc or not wc:
        raise RuntimeError("no calibration copy in the counter runs (bench.py --calibrate-copy)")
    # the largest copy dispatch is the calibration copy
    f_scale = COPY_BYTES / (max(fc) * 1024.0)
    w_scale = COPY_BYTES / (max(wc) * 1024.0)
    fetch_kib = statistics.median(fk)
    write_kib = statistics.median(wk)
    fetch_b = fetch_kib * 1024.0 * f_scale
    write_b = write_kib * 1024.0 * w_scale
    return {
        "workload": workload, "kernel": kernel, "source_digest": source_digest(kernel),
        "dispatches": {"fetch": len(fk), "write": len(wk)},
        "fetch_kib_median": fetch_kib, "write_kib_median": write_kib,
        "copy_fetch_kib": max(fc), "copy_write_kib": max(wc),
        "fetch_scale": f_scale, "write_scale": w_scale,
        "fetch_bytes": fetch_b, "write_bytes": write_b, "traffic_bytes": fetch_b + write_b,
    }


PEAK_BF16_FLOPS = 2.5e15   # MI355X dense bf16 matrix cores
CLOCK_HZ = 2.4e9           # MI355X peak engine clock


def summarize_mfma(run_dir: str, kernel: str, workload: str, simds: int = 1024, largest: bool = False) -> dict:
    """Matrix-core counters of `kernel` (median over its dispatches):
    bf16 MFMA ops issued (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 = FLOPs), MFMA
    busy cycles summed over the SIMDs, and the dispatch duration.  Derived:
    the issued rate against the bf16 peak, and the busy fraction of the
    SIMDs' cycles at the peak clock over the dispatch."""
    path = _counter_csv(run_dir)
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel not in r["Kernel_Name"]:
                continue
            d = per.setdefault(r["Dispatch_Id"], {})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
            d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    rows = [d for d in per.values() if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in d and "SQ_VALU_MFMA_BUSY_CYCLES" in d]
    if not rows:
        raise RuntimeError(f"no dispatches of {kernel} with MFMA counters in {run_dir}")
    if largest:  # one kernel serving several products: keep the largest product's dispatches
        top = max(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for d in rows)
        rows = [d for d in rows if d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] == top]
    flops = statistics.median(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0 for d in rows)
    busy = statistics.median(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in rows)
    ns = statistics.median(d["ns"] for d in rows)
    return {
        "workload": workload, "kernel": kernel, "source_digest": source_digest(kernel), "dispatches": len(rows),
        "mfma_flops_issued": flops, "mfma_busy_cycles": busy, "duration_ns": ns,
        "issued_tflops": flops / (ns * 1e-9) / 1e12, "issued_frac": flops / (ns * 1e-9) / PEAK_BF16_FLOPS,
        "busy_frac": busy / (simds * ns * 1e-9 * CLOCK_HZ),
    }


LDS_COUNTERS = ("SQ_INSTS_LDS", "SQ_INSTS_LDS_LOAD_BANDWIDTH", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS",
                "GRBM_GUI_ACTIVE")


def summarize_lds(run_dir: str, kernel: str, workload: str) -> dict:
    """LDS counters of `kernel` (median over its dispatches): LDS
    instructions issued, bytes loaded from LDS (SQ_INSTS_LDS_LOAD_BANDWIDTH
    counts 64-byte units), cycles lost to bank conflicts and cycles with an
    LDS instruction in flight (both summed over the compute units), and the
    GPU's active cycles."""
    path = _counter_csv(run_dir)
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel not in r["Kernel_Name"]:
                continue
            d = per.setdefault(r["Dispatch_Id"], {})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
            d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    rows = [d for d in per.values() if all(c in d for c in LDS_COUNTERS)]
    if not rows:
        raise RuntimeError(f"no dispatches of {kernel} with LDS counters in {run_dir}")
    med = {c: statistics.median(d[c] for d in rows) for c in LDS_COUNTERS}
    return {
        "workload": workload, "kernel": kernel, "source_digest": source_digest(kernel), "dispatches": len(rows),
        "lds_instructions": med["SQ_INSTS_LDS"], "lds_load_bytes": med["SQ_INSTS_LDS_LOAD_BANDWIDTH"] * 64.0,
        "bank_conflict_cycles": med["SQ_LDS_BANK_CONFLICT"], "lds_active_cycles": med["SQ_ACTIVE_INST_LDS"],
        "gui_active_cycles": med["GRBM_GUI_ACTIVE"], "duration_ns": statistics.median(d["ns"] for d in rows),
    }


def load(kernel: str, workload: str, profiles_dir: str, what: str = "traffic"):
    """The stored summary (traffic or mfma) for (kernel, workload) if it
    matches the current sources, else None."""
    path = os.path.join(profiles_dir, f"{kernel}_{workload}_{what}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    return d if d.get("source_digest") == source_digest(kernel) else None


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--kernel", required=True)
    s.add_argument("--workload", required=True)
    s.add_argument("--command", default="", help="the profiled command, recorded in the summary")
    s.add_argument("--largest", action="store_true", help="only the dispatches that move the most bytes")
    s.add_argument("--out", required=True)
    mf = sub.add_parser("mfma")
    mf.add_argument("--dir", required=True)
    mf.add_argument("--kernel", required=True)
    mf.add_argument("--workload", required=True)
    mf.add_argument("--command", default="")
    mf.add_argument("--largest", action="store_true", help="only the dispatches of the largest product")
    mf.add_argument("--out", required=True)
    ld = sub.add_parser("lds")
    ld.add_argument("--dir", required=True)
    ld.add_argument("--kernel", required=True)
    ld.add_argument("--workload", required=True)
    ld.add_argument("--command", default="")
    ld.add_argument("--out", required=True)
    d = sub.add_parser("digest")
    d.add_argument("--kernel", default="")
    args = ap.parse_args()
    if args.cmd == "digest":
        print(source_digest(args.kernel))
        return
    if args.cmd == "lds":
        out = summarize_lds(args.dir, args.kernel, args.workload)
        out["command"] = args.command
        with open(args.out, "w") as f:
            json.dump(out, f, indent=1)
        print(json.dumps(out))
        return
    if args.cmd == "mfma":
        out = summarize_mfma(args.dir, args.kernel, args.workload, largest=args.largest)
        out["command"] = args.command
        with open(args.out, "w") as f:
            json.dump(out, f, indent=1)
        print(json.dumps(out))
        return
    out = summarize(args.fetch, args.write, args.kernel, args.workload, largest=args.largest)
    out["command"] = args.command
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
