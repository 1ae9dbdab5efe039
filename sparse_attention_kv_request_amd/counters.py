"""Counter helpers for the rocprofv3 traffic figures.

``python -m sparse_attention_kv_request_amd.counters calib`` runs a plain
device-to-device copy of 256 MiB three times: the reference whose
``FETCH_SIZE`` / ``WRITE_SIZE`` readings (KiB per dispatch) calibrate what
those counters report for a known number of bytes.

``python -m sparse_attention_kv_request_amd.counters summarize FETCH.csv
WRITE.csv CALIB_FETCH.csv CALIB_WRITE.csv --kernel miss_copy --skip N``
reads rocprofv3 counter-collection CSVs and prints per-dispatch averages,
the calibration factors and the scaled traffic per launch as JSON.
"""
from __future__ import annotations

import argparse
import csv
import json
import statistics

CALIB_BYTES = 256 << 20


def calib():
    import torch

    a = torch.full((CALIB_BYTES,), 3, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {CALIB_BYTES} bytes x 3", flush=True)


def read_counter(path, kernel_substr, skip=0, limit=0):
    """Per-dispatch values of one counter for kernels whose name contains
    `kernel_substr`, in dispatch order, the first `skip` dropped and at most
    `limit` kept (0: all)."""
    vals = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name", "")
            if kernel_substr not in name:
                continue
            disp = int(row.get("Dispatch_Id", row.get("Correlation_Id", "0")))
            vals[disp] = vals.get(disp, 0.0) + float(row["Counter_Value"])
    seq = [vals[k] for k in sorted(vals)][skip:]
    return seq[:limit] if limit else seq


def summarize(args):
    fetch = read_counter(args.fetch, args.kernel, args.skip, args.limit)
    write = read_counter(args.write, args.kernel, args.skip, args.limit)
    cf = read_counter(args.calib_fetch, args.calib_kernel)
    cw = read_counter(args.calib_write, args.calib_kernel)
    kib = CALIB_BYTES / 1024
    f_factor = kib / statistics.median(cf)
    w_factor = kib / statistics.median(cw)
    out = {
        "kernel": args.kernel,
        "dispatches": len(fetch),
        "fetch_kib_per_dispatch": statistics.mean(fetch),
        "write_kib_per_dispatch": statistics.mean(write),
        "calib_fetch_kib": statistics.median(cf),
        "calib_write_kib": statistics.median(cw),
        "calib_expected_kib": kib,
        "fetch_factor": f_factor,
        "write_factor": w_factor,
        "traffic_bytes_per_launch": (statistics.mean(fetch) * f_factor
                                     + statistics.mean(write) * w_factor) * 1024,
    }
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("calib")
    s = sub.add_parser("summarize")
    s.add_argument("fetch")
    s.add_argument("write")
    s.add_argument("calib_fetch")
    s.add_argument("calib_write")
    s.add_argument("--kernel", default="miss_copy")
    s.add_argument("--calib-kernel", default="elementwise")
    s.add_argument("--skip", type=int, default=0)
    s.add_argument("--limit", type=int, default=0,
                   help="use at most this many dispatches after the skipped ones")
    a = ap.parse_args()
    if a.cmd == "calib":
        calib()
    else:
        summarize(a)


if __name__ == "__main__":
    main()
