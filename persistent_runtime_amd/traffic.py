"""HBM traffic of the decode kernel from rocprofv3 counter runs.

rocprofv3 collects FETCH_SIZE and WRITE_SIZE (KiB per dispatch) in separate
runs; the same counters on a plain device copy of known size give the scale
that turns each counter into bytes on this machine.  The result is written as
JSON next to the profile summaries and read back by the benchmark, which uses
it only while the kernel sources are unchanged (the hash below).

    python -m persistent_runtime_amd.traffic --fetch DIR --write DIR \\
        --calib-fetch DIR --calib-write DIR --calib-bytes N --out FILE
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL = "mk_persistent_kernel"
COPY = "copyBuffer"


def kernel_source_hash() -> str:
    """Hash of the sources that decide the kernel's memory traffic."""
    h = hashlib.sha256()
    for f in ("kernels.h", "kernels_m1.hip", "mk_task.h", "planner.cpp"):
        with open(os.path.join(HERE, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _values(run_dir: str, counter: str, name: str) -> list[float]:
    path = os.path.join(run_dir, "run_counter_collection.csv")
    out = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter and name in r["Kernel_Name"]:
                out.append(float(r["Counter_Value"]))
    if not out:
        raise SystemExit(f"no {counter} samples for {name} in {path}")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--calib-fetch", required=True)
    ap.add_argument("--calib-write", required=True)
    ap.add_argument("--calib-bytes", type=float, required=True,
                    help="bytes one copy dispatch reads (= bytes it writes)")
    ap.add_argument("--out", required=True)
    ap.add_argument("--kernel", default=KERNEL + "<1>",
                    help="kernel name substring (the single-slot variant by default; "
                         "prompt chunks run another variant)")
    ap.add_argument("--command", action="append", default=[],
                    help="profiling command lines to record")
    a = ap.parse_args()
    fk = statistics.median(_values(a.fetch, "FETCH_SIZE", a.kernel))
    wk = statistics.median(_values(a.write, "WRITE_SIZE", a.kernel))
    cf = statistics.median(_values(a.calib_fetch, "FETCH_SIZE", COPY))
    cw = statistics.median(_values(a.calib_write, "WRITE_SIZE", COPY))
    sf = a.calib_bytes / (cf * 1024.0)   # bytes per counted KiB
    sw = a.calib_bytes / (cw * 1024.0)
    rec = {
        "kernel": a.kernel, "kernel_source_hash": kernel_source_hash(),
        "fetch_kib_per_launch": fk, "write_kib_per_launch": wk,
        "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes": a.calib_bytes,
        "fetch_scale": sf, "write_scale": sw,
        "read_bytes_per_launch": fk * 1024.0 * sf, "write_bytes_per_launch": wk * 1024.0 * sw,
        "bytes_per_launch": fk * 1024.0 * sf + wk * 1024.0 * sw,
        "commands": a.command,
    }
    with open(a.out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
