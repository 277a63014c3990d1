"""Summaries of rocprofv3 output for the kernels of this library.

``python -m lut_sketched_matmul_amd.profiling`` turns the CSV files of one
``rocprofv3 --kernel-trace --stats`` run and of any number of
``rocprofv3 --pmc <counters>`` runs of the same program into a short
markdown summary: per-kernel durations, the start-to-start period of
back-to-back dispatches, per-dispatch counter means, and the HBM byte counts
scaled by what the same counters read for a plain copy kernel of known size.

The summary ends with a JSON block that ``bench.py`` reads to fill the
measured HBM traffic of its headline kernel. The block records a digest of
the kernel's source files; when the sources change, the digest no longer
matches and the stored counters are no longer used.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

# The files that define each profiled kernel family (host dispatch included).
KERNEL_SOURCES = {
    "decode": ["include/sketch_matmul.h", "lut_sketched_matmul_amd/csrc/skm_abi.hip",
               "lut_sketched_matmul_amd/csrc/skm_common.h", "lut_sketched_matmul_amd/csrc/skm_launch.h",
               "lut_sketched_matmul_amd/csrc/skm_decode.hip", "lut_sketched_matmul_amd/csrc/skm_decode_sets.hip",
               "lut_sketched_matmul_amd/csrc/skm_rowscale.hip"],
    "gemm": ["include/sketch_matmul.h", "lut_sketched_matmul_amd/csrc/skm_abi.hip",
             "lut_sketched_matmul_amd/csrc/skm_common.h", "lut_sketched_matmul_amd/csrc/skm_launch.h",
             "lut_sketched_matmul_amd/csrc/skm_gemm_common.h", "lut_sketched_matmul_amd/csrc/skm_gemm.hip",
             "lut_sketched_matmul_amd/csrc/skm_gemm_bwd.hip", "lut_sketched_matmul_amd/csrc/skm_rowscale.hip"],
    "optim": ["include/sketch_matmul.h", "lut_sketched_matmul_amd/csrc/skm_abi.hip",
              "lut_sketched_matmul_amd/csrc/skm_common.h", "lut_sketched_matmul_amd/csrc/skm_launch.h",
              "lut_sketched_matmul_amd/csrc/skm_optim.hip"],
    "sketch": ["include/sketch_matmul.h", "lut_sketched_matmul_amd/csrc/skm_abi.hip",
               "lut_sketched_matmul_amd/csrc/skm_common.h", "lut_sketched_matmul_amd/csrc/skm_launch.h",
               "lut_sketched_matmul_amd/csrc/skm_sketch.hip", "lut_sketched_matmul_amd/csrc/skm_factor.hip"],
}

# torch.add(src, 1.0, out=dst) on fp32: reads and writes this many bytes per launch
COPY_KERNEL = "vectorized_elementwise_kernel<4, at::native::CUDAFunctorOnSelf_add<float>"


def source_digest(family: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[family]:
        h.update(rel.encode())
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _one(path_glob: str) -> str:
    hits = sorted(glob.glob(path_glob, recursive=True))
    if not hits:
        raise FileNotFoundError(path_glob)
    return hits[0]


_TARG = [(r"Li(-?\d+)E", lambda m: m.group(1)), (r"Lb([01])E", lambda m: ("false", "true")[int(m.group(1))]),
         (r"DF16_", lambda m: "f16"), (r"DF16b", lambda m: "bf16"), (r"f", lambda m: "f32")]


def short_name(name: str) -> str:
    """Readable kernel name: the skm kernel and its template arguments."""
    m = re.search(r"\d+(k_[a-z0-9_]+)I", name)
    if m:
        rest, args = name[m.end():], []
        while rest and not rest.startswith("E"):
            for pat, fn in _TARG:
                t = re.match(pat, rest)
                if t:
                    args.append(fn(t))
                    rest = rest[t.end():]
                    break
            else:
                return m.group(1)
        return f"{m.group(1)}<{','.join(args)}>"
    m = re.search(r"::(k_[a-z0-9_]+)<([^,>]*)", name)  # already demangled by the profiler
    if m:
        return f"{m.group(1)}<{m.group(2)},...>"
    m = re.search(r"::(k_[a-z0-9_]+)\(", name)  # demangled, not a template
    if m:
        return m.group(1)
    if COPY_KERNEL in name:
        return "torch add (copy reference)"
    return name[:60]


# kernels whose launches are reported together whatever their grid size
MERGE_GRIDS = None


def _key(name: str, grid: int, wg: int):
    if MERGE_GRIDS and re.search(MERGE_GRIDS, short_name(name)):
        return (name, -1)
    return (name, grid // max(wg, 1))


def trace_stats(trace_csv: str):
    """Per (kernel, grid blocks): calls, mean / min / max duration (ns), and
    the mean start-to-start period over the longest run of consecutive
    dispatches."""
    rows = list(csv.DictReader(open(trace_csv)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    per = collections.defaultdict(list)
    runs = collections.defaultdict(list)  # key -> list of runs (lists of start times)
    prev = None
    for r in rows:
        k = _key(r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        s, e = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        per[k].append(e - s)
        if k != prev:
            runs[k].append([])
        runs[k][-1].append(s)
        prev = k
    out = {}
    for k, d in per.items():
        longest = max(runs[k], key=len)
        period = (longest[-1] - longest[0]) / (len(longest) - 1) if len(longest) > 1 else None
        out[k] = {"calls": len(d), "mean_ns": sum(d) / len(d), "min_ns": min(d), "max_ns": max(d),
                  "run": len(longest), "period_ns": period}
    return out


def counter_means(counter_csv: str):
    """Per ((kernel, grid blocks), counter): mean value per dispatch and the number of dispatches."""
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(counter_csv)):
        k = _key(r["Kernel_Name"], int(r["Grid_Size"]), int(r["Workgroup_Size"]))
        agg[(k, r["Counter_Name"])].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in agg.items()}


# MI355X: 8 accelerator dies (XCDs) of 32 CUs, 4 SIMDs per CU; MFMA peak for 16-bit inputs
XCDS, CUS_PER_XCD, SIMDS_PER_CU = 8, 32, 4
MFMA16_PEAK_TFLOPS = 2500.0


def summarize(stats_dir, pmc_dirs, kernel_regex, family, title, commands, copy_bytes, algorithmic_bytes=None,
              grid_bytes=None):
    st = trace_stats(_one(os.path.join(stats_dir, "**", "*kernel_trace.csv")))
    counters = {}
    for d in pmc_dirs:
        counters.update(counter_means(_one(os.path.join(d, "**", "*counter_collection.csv"))))
    pat = re.compile(kernel_regex)
    mine = sorted((k for k in st if pat.search(k[0])), key=lambda k: (short_name(k[0]), k[1]))
    copy = [k for k in st if COPY_KERNEL in k[0]]
    label = lambda k: f"{short_name(k[0])} [{k[1]} blocks]" if k[1] >= 0 else f"{short_name(k[0])} [all grids]"

    lines = [f"# {title}", "", "Commands (from the repository root; OUT is any output folder):", "", "```"]
    lines += commands
    lines += ["```", "", "## Kernel trace", "",
              "| kernel | calls | mean us | min us | max us | back-to-back run | start-to-start us |",
              "|---|---|---|---|---|---|---|"]
    for k in mine + copy:
        s = st[k]
        per = f"{s['period_ns'] / 1e3:.2f}" if s["period_ns"] else "-"
        lines.append(f"| `{label(k)}` | {s['calls']} | {s['mean_ns'] / 1e3:.2f} | {s['min_ns'] / 1e3:.2f} | "
                     f"{s['max_ns'] / 1e3:.2f} | {s['run']} | {per} |")

    names = sorted({c for (_, c) in counters})
    summary = {"family": family, "source_digest": source_digest(family), "kernels": {}}
    scale = {}
    if copy and copy_bytes:
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            v = counters.get((copy[0], c))
            if v:
                scale[c] = (copy_bytes / 1024.0) / v[0]
    if names:
        lines += ["", "## Counters (mean per dispatch)", "", "| kernel | " + " | ".join(names) + " |",
                  "|---|" + "---|" * len(names)]
        for k in mine + copy:
            vals = [counters.get((k, c)) for c in names]
            lines.append(f"| `{label(k)}` | " + " | ".join(f"{v[0]:.1f}" if v else "-" for v in vals) + " |")
    if scale:
        lines += ["", f"Copy reference: {copy_bytes} bytes read and written per launch. Scale factors "
                  "(known KiB / counter KiB): " + ", ".join(f"{c} x{v:.3f}" for c, v in scale.items()) + "."]
    derived = []
    for k in mine:
        s = st[k]
        e = {"calls": s["calls"], "mean_us": round(s["mean_ns"] / 1e3, 3),
             "period_us": round(s["period_ns"] / 1e3, 3) if s["period_ns"] else None}
        for c in names:
            v = counters.get((k, c))
            if v:
                e[c] = round(v[0], 3)
        if "FETCH_SIZE" in scale and "WRITE_SIZE" in scale and "FETCH_SIZE" in e and "WRITE_SIZE" in e:
            e["hbm_bytes"] = round(1024.0 * (e["FETCH_SIZE"] * scale["FETCH_SIZE"] +
                                             e["WRITE_SIZE"] * scale["WRITE_SIZE"]))
            e["hbm_GBps"] = round(e["hbm_bytes"] / (s["mean_ns"] * 1e-9) / 1e9, 1)
        mops = e.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) + e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        if mops:
            # one MOPS unit is 512 flops
            e["mfma_flops"] = mops * 512.0
            e["mfma_TFLOPs"] = round(e["mfma_flops"] / (s["mean_ns"] * 1e-9) / 1e12, 1)
            e["mfma_frac_of_peak"] = round(e["mfma_TFLOPs"] / MFMA16_PEAK_TFLOPS, 4)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in e and e.get("GRBM_GUI_ACTIVE"):
            # GRBM_GUI_ACTIVE is summed over the XCDs; the busy count is per SIMD
            simd_cycles = e["GRBM_GUI_ACTIVE"] / XCDS * XCDS * CUS_PER_XCD * SIMDS_PER_CU
            e["mfma_busy_frac"] = round(e["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles, 4)
        summary["kernels"][label(k)] = e
        parts = []
        algo = (grid_bytes or {}).get(k[1], algorithmic_bytes)
        if algo and grid_bytes and k[1] in grid_bytes:
            e["algorithmic_bytes"] = algo
        if "hbm_bytes" in e:
            parts.append(f"HBM bytes/launch {e['hbm_bytes']} ({e['hbm_GBps']} GB/s over the mean duration)")
            if algo:
                parts.append(f"algorithmic {algo} (ratio {e['hbm_bytes'] / algo:.3f})")
        if "mfma_TFLOPs" in e:
            parts.append(f"MFMA flops {e['mfma_flops']:.4g} -> {e['mfma_TFLOPs']} TFLOP/s "
                         f"({100 * e['mfma_frac_of_peak']:.1f}% of 2.5 PFLOP/s)")
        if "mfma_busy_frac" in e:
            parts.append(f"MFMA busy {100 * e['mfma_busy_frac']:.1f}% of SIMD cycles")
        if parts:
            derived.append(f"- `{label(k)}`: " + "; ".join(parts) + ".")
    if derived:
        lines += ["", "## Derived", ""] + derived
    if algorithmic_bytes:
        summary["algorithmic_bytes"] = algorithmic_bytes
    summary["scale"] = {c: round(v, 4) for c, v in scale.items()}
    lines += ["", "```json", json.dumps(summary, indent=1), "```", ""]
    return "\n".join(lines)


def load_summary(path: str):
    """The JSON block of a summary written by this module (None if absent)."""
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    return json.loads(m.group(1)) if m else None


def measured_bytes(path: str, kernel_prefix: str):
    """HBM bytes per launch of the first kernel whose short name starts with
    ``kernel_prefix``, if the summary's source digest matches the current
    sources; otherwise None."""
    s = load_summary(path)
    if not s or s.get("source_digest") != source_digest(s["family"]):
        return None
    for name, e in s["kernels"].items():
        if name.startswith(kernel_prefix) and "hbm_bytes" in e:
            return e["hbm_bytes"]
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--stats", required=True, help="output folder of the --kernel-trace --stats run")
    ap.add_argument("--pmc", nargs="*", default=[], help="output folders of --pmc runs")
    ap.add_argument("--kernels", required=True, help="regex selecting the kernels to report")
    ap.add_argument("--family", required=True, choices=sorted(KERNEL_SOURCES))
    ap.add_argument("--title", required=True)
    ap.add_argument("--command", action="append", default=[], help="command line to record (repeatable)")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--algorithmic-bytes", type=int, default=None)
    ap.add_argument("--grid-bytes", action="append", default=[],
                    help="BLOCKS=BYTES: algorithmic bytes of the launches with that grid (repeatable)")
    ap.add_argument("--merge-grids", default=None, help="regex: report these kernels' launches together")
    ap.add_argument("-o", "--out", required=True)
    a = ap.parse_args()
    global MERGE_GRIDS
    MERGE_GRIDS = a.merge_grids
    grid_bytes = {int(g.split("=")[0]): int(g.split("=")[1]) for g in a.grid_bytes}
    text = summarize(a.stats, a.pmc, a.kernels, a.family, a.title, a.command, a.copy_bytes, a.algorithmic_bytes,
                     grid_bytes)
    with open(a.out, "w") as f:
        f.write(text)


if __name__ == "__main__":
    main()
