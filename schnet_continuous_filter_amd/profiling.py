"""Summaries of rocprofv3 output for the kernels of this library.

  python -m schnet_continuous_filter_amd.profiling stats KT_STATS_CSV OUT_TXT --cmd "..."
  python -m schnet_continuous_filter_amd.profiling traffic FETCH_CSV WRITE_CSV \
      COPY_FETCH_CSV COPY_WRITE_CSV OUT_TXT --kernel k_cf_bwd --workload cg269x64 --cmd "..."

  python -m schnet_continuous_filter_amd.profiling util PMC_CSV OUT_TXT \
      --kernel k_cf_bwd --workload md1024 --cmd "..."

  python -m schnet_continuous_filter_amd.profiling insts OUT_TXT PMC_CSV [PMC_CSV ...] \
      --edges E --workload md1024 --cmd "..."

``traffic`` scales FETCH_SIZE and WRITE_SIZE (KiB per dispatch) by what the
same counters read for a device copy of known size (bench.py
--copy-calibration copies 256 MiB five times), and records the result with a
hash of the kernel source so that bench.py reports it only while the kernel
is unchanged.

``util`` averages the per-dispatch values of the derived counters MfmaUtil
(percent of the cycles the SIMDs' matrix units were busy: summed
SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE times the SIMD count) and
VALUBusy (percent of the cycles the vector ALUs issued: SQ_ACTIVE_INST_VALU
over the CU count times GRBM_GUI_ACTIVE), as rocprofv3 defines them, plus
any raw counters of the same run, and records them the same way.

``insts`` merges several counter passes over the same command and lists,
for every CFConv kernel, each counter's mean per dispatch, the instruction
counts (SQ_INSTS_*) per 16-edge tile of the E-edge list, and the share of
the waves' cycles spent waiting (SQ_WAIT_ANY over SQ_WAVE_CYCLES).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re

_CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
CFCONV_SRCS = [os.path.join(_CSRC, f) for f in ("cfconv.hip", "tile16.hpp", "common.hpp")]
COPY_BYTES = 256 * 1024 * 1024


def code_text(src: str) -> str:
    """C++ source without its comments and blank or trailing space, so that an
    edit of a comment does not change the hash of the code."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(line.rstrip() for line in src.splitlines() if line.strip())


def kernel_hash() -> str:
    """Hash of the code (comments removed) the CFConv kernels are compiled from."""
    h = hashlib.sha256()
    for f in CFCONV_SRCS:
        h.update(code_text(open(f, encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def stats(csv_path: str, out_txt: str, cmd: str, top: int = 25) -> None:
    rows = list(csv.DictReader(open(csv_path)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"# rocprofv3 --kernel-trace --stats summary", f"# command: {cmd}",
             f"# total kernel time {total / 1e6:.3f} ms over {sum(int(r['Calls']) for r in rows)} "
             "dispatches", "",
             f"{'kernel':72s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} "
             f"{'share%':>7s}"]
    for r in rows[:top]:
        lines.append(f"{r['Name'][:72]:72s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
                     f"{float(r['MinNs']) / 1e3:10.1f} {float(r['MaxNs']) / 1e3:10.1f} "
                     f"{float(r['Percentage']):7.2f}")
    open(out_txt, "w").write("\n".join(lines) + "\n")


def _per_kernel(csv_path):
    d = collections.defaultdict(list)
    for r in csv.DictReader(open(csv_path)):
        d[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return d


def _pick(d, substr):
    keys = [k for k in d if substr in k]
    if not keys:
        raise KeyError(f"no kernel matching {substr!r}")
    vals = sum((d[k] for k in keys), [])
    return sum(vals) / len(vals), len(vals), keys


def traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, out_txt, kernel, workload,
            cmd) -> dict:
    f_kib, nf, names = _pick(_per_kernel(fetch_csv), kernel)
    w_kib, nw, _ = _pick(_per_kernel(write_csv), kernel)
    cf_kib, _, _ = _pick(_per_kernel(copy_fetch_csv), "copyBuffer")
    cw_kib, _, _ = _pick(_per_kernel(copy_write_csv), "copyBuffer")
    f_scale = COPY_BYTES / (cf_kib * 1024.0)
    w_scale = COPY_BYTES / (cw_kib * 1024.0)
    rec = {
        "kernel": names[0], "workload": workload, "kernel_hash": kernel_hash(),
        "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib, "dispatches": nf,
        "copy_fetch_kib": cf_kib, "copy_write_kib": cw_kib, "fetch_scale": f_scale,
        "write_scale": w_scale,
        "bytes_per_launch": f_kib * 1024.0 * f_scale + w_kib * 1024.0 * w_scale,
        "command": cmd,
    }
    with open(out_txt, "w") as f:
        f.write(json.dumps(rec) + "\n")
    return rec


def _per_kernel_counter(csv_path):
    d = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(csv_path)):
        d[r["Counter_Name"]][r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return d


def util(pmc_csv, out_txt, kernel, workload, cmd) -> dict:
    d = _per_kernel_counter(pmc_csv)
    rec = {"workload": workload, "kernel_hash": kernel_hash(), "command": cmd, "counters": {}}
    for name, per in d.items():
        avg, n, keys = _pick(per, kernel)
        rec["kernel"] = keys[0]
        rec["dispatches"] = n
        rec["counters"][name] = avg
    if "MfmaUtil" in rec["counters"]:
        rec["mfma_busy"] = rec["counters"]["MfmaUtil"] / 100.0
    if "VALUBusy" in rec["counters"]:
        rec["valu_busy"] = rec["counters"]["VALUBusy"] / 100.0
    with open(out_txt, "w") as f:
        f.write(json.dumps(rec) + "\n")
    return rec


def insts(pmc_csvs, out_txt, edges, workload, cmd, kernel="k_cf_") -> dict:
    per = collections.defaultdict(dict)
    for c in pmc_csvs:
        for name, by_kernel in _per_kernel_counter(c).items():
            per[name].update(by_kernel)
    kernels = sorted({k for by_kernel in per.values() for k in by_kernel if kernel in k})
    tiles = -(-int(edges) // 16)
    rec = {"workload": workload, "kernel_hash": kernel_hash(), "edges": int(edges),
           "tiles": tiles, "command": cmd, "kernels": {}}
    lines = [f"# rocprofv3 --pmc counter passes over one command; {workload}, {edges} edges "
             f"= {tiles} tiles of 16 per dispatch", f"# command: {cmd}",
             f"# kernel_hash {rec['kernel_hash']}", ""]
    for k in kernels:
        means = {n: sum(v[k]) / len(v[k]) for n, v in per.items() if k in v}
        rec["kernels"][k] = means
        lines.append(k)
        for n in sorted(means):
            tail = f"  {means[n] / tiles:10.1f} per tile" if n.startswith("SQ_INSTS") else ""
            lines.append(f"  {n:28s} {means[n]:16.6g}{tail}")
        if "SQ_WAIT_ANY" in means and means.get("SQ_WAVE_CYCLES"):
            lines.append(f"  {'waiting share':28s} {means['SQ_WAIT_ANY'] / means['SQ_WAVE_CYCLES']:16.3f}"
                         "  (SQ_WAIT_ANY / SQ_WAVE_CYCLES)")
        lines.append("")
    with open(out_txt, "w") as f:
        f.write("\n".join(lines))
        f.write(json.dumps(rec) + "\n")
    return rec


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    for a in ("fetch", "write", "copy_fetch", "copy_write", "out"):
        t.add_argument(a)
    t.add_argument("--kernel", default="k_cf_bwd")
    t.add_argument("--workload", default="cg269x64")
    t.add_argument("--cmd", required=True)
    u = sub.add_parser("util")
    u.add_argument("csv")
    u.add_argument("out")
    u.add_argument("--kernel", default="k_cf_bwd")
    u.add_argument("--workload", default="md1024")
    u.add_argument("--cmd", required=True)
    n = sub.add_parser("insts")
    n.add_argument("out")
    n.add_argument("csvs", nargs="+")
    n.add_argument("--edges", type=int, required=True)
    n.add_argument("--workload", default="md1024")
    n.add_argument("--cmd", required=True)
    a = ap.parse_args()
    if a.what == "stats":
        stats(a.csv, a.out, a.cmd)
    elif a.what == "insts":
        insts(a.csvs, a.out, a.edges, a.workload, a.cmd)
    elif a.what == "util":
        print(json.dumps(util(a.csv, a.out, a.kernel, a.workload, a.cmd)))
    else:
        print(json.dumps(traffic(a.fetch, a.write, a.copy_fetch, a.copy_write, a.out, a.kernel,
                                 a.workload, a.cmd)))


if __name__ == "__main__":
    main()
