"""Summaries of rocprofv3 CSV output for the profiles kept with the library.

    python -m rank_recurrent_state_amd.prof_summary trace DIR
        per-kernel dispatch count, average and total duration from a
        `rocprofv3 --kernel-trace --stats --output-format csv -d DIR` run;
    python -m rank_recurrent_state_amd.prof_summary pmc FETCH_DIR WRITE_DIR [--copy-bytes B]
        per-kernel average FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two
        `rocprofv3 --pmc ... --output-format csv` runs, scaled to bytes by what the same counters
        read for the calibration copy of B bytes (the largest copy kernel in the run);
    python -m rank_recurrent_state_amd.prof_summary counters DIR
        per-kernel dispatch count and average value per dispatch of every counter in a
        `rocprofv3 --pmc ... --output-format csv -d DIR` run.

Only reads the CSV files rocprofv3 wrote; prints plain text.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import os
import sys


def _rows(d: str, suffix: str) -> list[dict]:
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    out = []
    for f in files:
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def _col(row: dict, *names: str) -> str:
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(f"none of {names} in {list(row)}")


def short(name: str, width: int = 96) -> str:
    return name if len(name) <= width else name[: width - 3] + "..."


def trace(d: str) -> None:
    rows = _rows(d, "kernel_trace.csv")
    agg = collections.defaultdict(list)
    for r in rows:
        start = int(_col(r, "Start_Timestamp", "start"))
        end = int(_col(r, "End_Timestamp", "end"))
        agg[_col(r, "Kernel_Name", "name")].append((end - start) / 1e3)
    print(f"{'calls':>7} {'avg_us':>11} {'min_us':>10} {'max_us':>10} {'total_ms':>10}  kernel")
    for name, ds in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        print(f"{len(ds):7d} {sum(ds) / len(ds):11.2f} {min(ds):10.2f} {max(ds):10.2f} "
              f"{sum(ds) / 1e3:10.2f}  {short(name)}")


def _pmc(d: str, counter: str) -> dict[str, list[float]]:
    rows = _rows(d, "counter_collection.csv")
    per = collections.defaultdict(float)
    names = {}
    for r in rows:
        if _col(r, "Counter_Name", "counter_name") != counter:
            continue
        disp = _col(r, "Dispatch_Id", "dispatch_id")
        per[disp] += float(_col(r, "Counter_Value", "value"))
        names[disp] = _col(r, "Kernel_Name", "kernel_name")
    agg = collections.defaultdict(list)
    for disp, v in per.items():
        agg[names[disp]].append(v)
    return agg


def pmc(fetch_dir: str, write_dir: str, copy_bytes: int) -> None:
    fetch = _pmc(fetch_dir, "FETCH_SIZE")
    write = _pmc(write_dir, "WRITE_SIZE")

    def copy_kernel(agg):
        cands = [(max(v), k) for k, v in agg.items() if "copy" in k.lower()]
        return max(cands)[1] if cands else None

    cf, cw = copy_kernel(fetch), copy_kernel(write)
    f_scale = copy_bytes / (max(fetch[cf]) * 1024.0) if cf else None
    w_scale = copy_bytes / (max(write[cw]) * 1024.0) if cw else None
    print(f"calibration copy of {copy_bytes} bytes: FETCH_SIZE {max(fetch[cf]) if cf else float('nan'):.1f} KiB "
          f"(scale {f_scale if f_scale else float('nan'):.4f}), WRITE_SIZE "
          f"{max(write[cw]) if cw else float('nan'):.1f} KiB (scale {w_scale if w_scale else float('nan'):.4f})")
    print(f"{'calls':>7} {'FETCH_KiB':>12} {'WRITE_KiB':>12} {'read_bytes':>14} {'write_bytes':>14}  kernel")
    for name in sorted(set(fetch) | set(write), key=lambda k: -sum(fetch.get(k, [0]))):
        fv, wv = fetch.get(name, []), write.get(name, [])
        fa = sum(fv) / len(fv) if fv else float("nan")
        wa = sum(wv) / len(wv) if wv else float("nan")
        rb = fa * 1024 * f_scale if f_scale else float("nan")
        wb = wa * 1024 * w_scale if w_scale else float("nan")
        print(f"{max(len(fv), len(wv)):7d} {fa:12.1f} {wa:12.1f} {rb:14.0f} {wb:14.0f}  {short(name)}")


def counters(d: str) -> None:
    rows = _rows(d, "counter_collection.csv")
    names = sorted({_col(r, "Counter_Name", "counter_name") for r in rows})
    agg = {n: _pmc(d, n) for n in names}
    kernels = sorted({k for a in agg.values() for k in a},
                     key=lambda k: -max(sum(a.get(k, [0])) for a in agg.values()))
    print(f"{'calls':>7} " + " ".join(f"{n:>20}" for n in names) + "  kernel")
    for k in kernels:
        calls = max(len(a.get(k, [])) for a in agg.values())
        vals = [(sum(a[k]) / len(a[k])) if a.get(k) else float("nan") for a in agg.values()]
        print(f"{calls:7d} " + " ".join(f"{v:20.1f}" for v in vals) + f"  {short(k)}")


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    p = sub.add_parser("pmc")
    p.add_argument("fetch_dir")
    p.add_argument("write_dir")
    p.add_argument("--copy-bytes", type=int, default=1 << 30)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        trace(a.dir)
    elif a.cmd == "counters":
        counters(a.dir)
    else:
        pmc(a.fetch_dir, a.write_dir, a.copy_bytes)


if __name__ == "__main__":
    main(sys.argv[1:])
