"""Counter helpers for the rocprofv3 traffic and issue figures.

``python -m sparse_attention_kv_request_amd.counters calib`` runs a plain
device-to-device copy of 256 MiB three times: the reference whose
``FETCH_SIZE`` / ``WRITE_SIZE`` readings (KiB per dispatch) calibrate what
those counters report for a known number of bytes.

``python -m sparse_attention_kv_request_amd.counters record FETCH.csv WRITE.csv
CALIB_FETCH.csv CALIB_WRITE.csv --kernel K --skip N --limit M --workload W
--warmup X --steps Y --bench-line LINE.json`` averages one kernel's counters
over the selected dispatches, scales them by the calibration, and merges the
result, with the algorithmic bytes per launch from the bench line of the same
command and a hash of the kernel's sources, into
``profiles/traffic_counters.json`` (which bench.py reads).

``python -m sparse_attention_kv_request_amd.counters table`` prints the
committed entries as a markdown table.

``python -m sparse_attention_kv_request_amd.counters sq CSV --kernel K``
summarises SQ counters (issue, wait and matrix-core cycles) per wave.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import pathlib
import statistics

CALIB_BYTES = 256 << 20
ROOT = pathlib.Path(__file__).resolve().parents[1]
CSRC = pathlib.Path(__file__).resolve().parent / "csrc"
COUNTERS = ROOT / "profiles" / "traffic_counters.json"

# Sources each kernel is built from (kernel, arguments, launch shape and the
# helpers it uses): a counter figure applies only while these are unchanged.
KERNEL_SOURCES = {
    "miss_copy": ("copy.hip", "copy.h", "device_common.h"),
    # (copy.h: the rule that lets a swap call copy inside the lookup kernel)
    "lru_token_plan": ("plan_lru.hip", "device_common.h", "internal.h", "hisparse_api.cpp",
                       "copy.h"),
    "lru_page_plan": ("plan_lru.hip", "device_common.h", "internal.h", "hisparse_api.cpp",
                      "copy.h"),
    "clock_plan": ("plan_clock.hip", "device_common.h", "internal.h", "hisparse_api.cpp",
                   "copy.h"),
    # one call: topk_chunk_kernel (+ topk_merge_kernel when a row spans chunks)
    "topk": ("topk.hip", "device_common.h", "internal.h"),
    # one call: mla_decode (+ mla_combine when the locations are split)
    "mla_decode": ("mla_decode.hip", "device_common.h", "internal.h"),
}


def kernel_hash(kernel):
    m = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        m.update((CSRC / name).read_bytes())
    return m.hexdigest()[:16]


def traffic_key(kernel, workload, warmup, steps):
    return f"{kernel}|workload {workload}|warmup {warmup}|steps {steps}"


def traffic_from_profiles(kernel, workload, warmup, steps):
    """Counted bytes per launch from the committed summary, if it was taken on
    the kernel's current sources and on exactly these timed launches
    (workload, warm-up and step count); else None."""
    if not COUNTERS.exists():
        return None
    entry = json.loads(COUNTERS.read_text()).get("entries", {}).get(
        traffic_key(kernel, workload, warmup, steps))
    if entry is None or entry.get("sources_sha256_16") != kernel_hash(kernel):
        return None
    return entry.get("traffic_bytes_per_launch")


def calib():
    import torch

    a = torch.full((CALIB_BYTES,), 3, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {CALIB_BYTES} bytes x 3", flush=True)


def _rows(path):
    with open(path) as f:
        yield from csv.DictReader(f)


def read_counter(path, kernel_substr, skip=0, limit=0, counter=None):
    """Per-dispatch values of one counter for kernels whose name contains
    `kernel_substr`, in dispatch order, the first `skip` dropped and at most
    `limit` kept (0: all)."""
    vals = {}
    for row in _rows(path):
        if kernel_substr not in row.get("Kernel_Name", ""):
            continue
        if counter is not None and row["Counter_Name"] != counter:
            continue
        disp = int(row.get("Dispatch_Id", row.get("Correlation_Id", "0")))
        vals[disp] = vals.get(disp, 0.0) + float(row["Counter_Value"])
    seq = [vals[k] for k in sorted(vals)][skip:]
    return seq[:limit] if limit else seq


def summarize(fetch_csv, write_csv, calib_fetch, calib_write, kernels, skip, limit,
              calib_kernel="copyBuffer"):
    """Counted bytes per call of one or more kernels (a call that launches
    several kernels, e.g. selection + merge, sums their per-dispatch means);
    `skip` and `limit` apply to each kernel's own dispatch sequence."""
    cf = read_counter(calib_fetch, calib_kernel)
    cw = read_counter(calib_write, calib_kernel)
    kib = CALIB_BYTES / 1024
    f_factor = kib / statistics.median(cf)
    w_factor = kib / statistics.median(cw)
    fetch = write = 0.0
    counts = []
    for k in kernels:
        f = read_counter(fetch_csv, k, skip, limit)
        w = read_counter(write_csv, k, skip, limit)
        if not f:
            continue                      # a kernel this shape does not launch
        if len(f) != len(w):
            raise SystemExit(f"{k}: {len(f)} FETCH_SIZE but {len(w)} WRITE_SIZE dispatches")
        counts.append(f"{k}: {len(f)}")
        fetch += statistics.mean(f)
        write += statistics.mean(w)
    return {
        "dispatches": ", ".join(counts),
        "fetch_kib_per_dispatch": round(fetch, 2),
        "write_kib_per_dispatch": round(write, 2),
        "fetch_factor": round(f_factor, 4),
        "write_factor": round(w_factor, 4),
        "fetch_bytes_per_launch": int(fetch * f_factor * 1024),
        "write_bytes_per_launch": int(write * w_factor * 1024),
        "traffic_bytes_per_launch": int((fetch * f_factor + write * w_factor) * 1024),
    }


def record(args):
    out = summarize(args.fetch, args.write, args.calib_fetch, args.calib_write,
                    (args.match or args.kernel).split(","), args.skip, args.limit,
                    args.calib_kernel)
    line = {}
    if args.bench_line:
        line = json.loads(pathlib.Path(args.bench_line).read_text().strip().splitlines()[-1])
    if args.kernel == "miss_copy":
        # a copy reads each byte (host) and writes it (HBM)
        alg = 2 * line["roofline"]["bytes_per_launch"] if line else None
        model = None
    elif args.kernel in ("topk", "mla_decode"):
        alg, model = line.get("roofline", {}).get("bytes_per_call"), None
    else:
        sr = line.get("state_roofline") or line.get("roofline", {})   # swap / batched-state
        alg, model = sr.get("bytes_per_launch"), sr.get("kernel_model_bytes_per_launch")
        if args.fused:   # the lookup kernel that also copied: + each miss read and written
            copy = 2 * line["roofline"]["bytes_per_launch"]
            alg, model = alg + copy, (model + copy if model else None)
    entry = {"kernel": args.kernel, "workload": args.workload, "warmup": args.warmup,
             "steps": args.steps, **out,
             "algorithmic_bytes_per_launch": alg,
             "traffic_over_algorithmic": round(out["traffic_bytes_per_launch"] / alg, 3)
             if alg else None,
             "sources_sha256_16": kernel_hash(args.kernel), "command": args.cmd}
    if model:
        entry["kernel_model_bytes_per_launch"] = model
        entry["traffic_over_kernel_model"] = round(out["traffic_bytes_per_launch"] / model, 3)
    data = json.loads(COUNTERS.read_text()) if COUNTERS.exists() else {}
    data.setdefault("about", "Bytes per launch counted by rocprofv3 FETCH_SIZE and WRITE_SIZE "
                             "(one pass each), averaged over the timed launches of the named "
                             "bench command and scaled by what the counters read for a 256 MiB "
                             "device-to-device copy; beside them the algorithmic bytes per launch "
                             "from that command's bench line.  An entry applies while its "
                             "kernel's sources hash to sources_sha256_16.")
    data.setdefault("entries", {})[traffic_key(args.kernel, args.workload, args.warmup,
                                               args.steps)] = entry
    COUNTERS.write_text(json.dumps(data, indent=1, sort_keys=True) + "\n")
    print(json.dumps(entry, indent=1))


def table(_args):
    """The committed entries as a markdown table (one row per kernel and
    workload), in MB per launch."""
    data = json.loads(COUNTERS.read_text())
    print("| kernel | workload | fetch MB | write MB | counted MB | algorithmic MB | "
          "counted / algorithmic | kernel model MB | counted / model |")
    print("|---|---|---|---|---|---|---|---|---|")
    mb = lambda x: f"{x / 1e6:.3f}" if x else "-"
    for key in sorted(data["entries"]):
        e = data["entries"][key]
        print(f"| `{e['kernel']}` | {e['workload']} | {mb(e['fetch_bytes_per_launch'])} | "
              f"{mb(e['write_bytes_per_launch'])} | {mb(e['traffic_bytes_per_launch'])} | "
              f"{mb(e['algorithmic_bytes_per_launch'])} | {e['traffic_over_algorithmic']} | "
              f"{mb(e.get('kernel_model_bytes_per_launch'))} | "
              f"{e.get('traffic_over_kernel_model', '-')} |")


SQ_UNITS = 4   # the SQ cycle counters count in units of 4 cycles


def sq(args):
    """Per-wave SQ counter values of one kernel (mean over its dispatches):
    each counter's total per dispatch divided by the dispatch's waves."""
    per = {}
    waves = {}
    for row in _rows(args.csv):
        if args.kernel not in row.get("Kernel_Name", ""):
            continue
        disp = int(row.get("Dispatch_Id", row.get("Correlation_Id", "0")))
        waves[disp] = int(row["Grid_Size"]) // 64
        per.setdefault(row["Counter_Name"], {}).setdefault(disp, 0.0)
        per[row["Counter_Name"]][disp] += float(row["Counter_Value"])
    disps = sorted(waves)[args.skip:]
    out = {"kernel": args.kernel, "dispatches": len(disps),
           "waves_per_dispatch": statistics.mean(waves[d] for d in disps)}
    for name, vals in sorted(per.items()):
        out[name + "_per_wave"] = round(statistics.mean(vals[d] / waves[d] for d in disps), 1)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="action", required=True)
    sub.add_parser("calib")
    r = sub.add_parser("record")
    for name in ("fetch", "write", "calib_fetch", "calib_write"):
        r.add_argument(name)
    r.add_argument("--kernel", required=True)
    r.add_argument("--match", default="",
                   help="kernel name substrings, comma-separated, whose per-dispatch means "
                        "add up to one call (default: --kernel)")
    r.add_argument("--calib-kernel", default="copyBuffer")
    r.add_argument("--skip", type=int, default=0)
    r.add_argument("--limit", type=int, default=0,
                   help="use at most this many dispatches after the skipped ones")
    r.add_argument("--workload", required=True)
    r.add_argument("--warmup", type=int, required=True)
    r.add_argument("--steps", type=int, required=True)
    r.add_argument("--bench-line", default="")
    r.add_argument("--fused", action="store_true",
                   help="the launches copied their misses too (algorithmic bytes: state + "
                        "miss bytes read and written)")
    r.add_argument("--cmd", default="")
    sub.add_parser("table")
    q = sub.add_parser("sq")
    q.add_argument("csv")
    q.add_argument("--kernel", required=True)
    q.add_argument("--skip", type=int, default=0)
    a = ap.parse_args()
    if a.action == "calib":
        calib()
    elif a.action == "record":
        record(a)
    elif a.action == "table":
        table(a)
    else:
        sq(a)


if __name__ == "__main__":
    main()
