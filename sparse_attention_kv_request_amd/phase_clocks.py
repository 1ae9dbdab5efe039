"""Phase clocks of the token-mode plan kernel (with the copy it does for
calls of 16 or more rows) and the wait shares of the bf16 attention tile
loop, from the instrumented build of the library.

``python -m sparse_attention_kv_request_amd.phase_clocks build`` compiles the
sources with ``-DHISPARSE_PHASE_CLOCKS=1`` into
``_build/phase_clocks/libhisparse.so`` (the default library is untouched;
that build records nothing).  ``python -m
sparse_attention_kv_request_amd.phase_clocks run`` (on the GPU) drives that
library and prints a markdown summary:

* the 64-row, single-layer swap call of the headline workload (16 calls,
  the first 4 skipped): per workgroup the 100 MHz wall clock at each phase
  boundary of the plan, at the start and end of its row's copy, and the
  row's miss count; medians over workgroups and calls, the copy end per XCD
  (workgroup id mod 8), and the copy phase's rate;
* the same kernel with 512 instances in one launch (the batched-state
  bench): when its workgroups start and how long each runs;
* the top-k chunk kernel's phases (64 rows x 32768 scores), with the
  threshold step split into its first bin pick, the listing of that bin's
  keys and the two list passes, and the merge kernel's phases (128 rows x
  131072 scores);
* the attention bench's bf16 calls: the kernel's setup (locations, row
  table, queries and first tile), tile loop and epilogue, and the share of
  each wave's tile-loop clocks spent waiting for the next tile's gather and
  at the phase barrier.

The clock reads add a few instructions per phase, so the absolute times run
a little above the uninstrumented kernels'; the shares and the spread are
what the summary is for.
"""
from __future__ import annotations

import argparse
import ctypes
import pathlib
import sys

ROOT = pathlib.Path(__file__).resolve().parents[1]
VARIANT = ROOT / "_build" / "phase_clocks" / "libhisparse.so"
TICK_US = 0.01  # wall_clock64: 100 MHz
STAMPS = 10
PHASES = ["request/state/top-k loads, row checks", "entry validation",
          "join (row-key bitmap, ranks, resident-key matches, hit touch)",
          "representatives, miss bitmap, merged scan, miss lists",
          "victims, commit, order rewrite", "outputs"]


def build():
    from sparse_attention_kv_request_amd import build as b

    return b.build(verbose=True, defines=["-DHISPARSE_PHASE_CLOCKS=1"], lib=VARIANT)


def _plan_clocks(torch, binding, workloads, lib, calls=16, skip=4):
    import numpy as np

    fn = lib.hisparse_phase_clocks
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int]
    w = workloads.config(2, layers=1, steps=calls)
    host = [binding.HostKV(w.requests, w.seq_len, w.item_bytes)]
    workloads.fill_host_kv(w, [h.array for h in host], threads=16)
    trace = workloads.batch_trace(w, threads=16)
    dev = torch.device("cuda", 0)
    st = binding.HiSparseState(max_requests=w.requests, num_layers=1, hot_buffer_size=w.hot,
                               top_k=w.top_k, item_size_bytes=w.item_bytes,
                               max_seq_len=w.seq_len, host_kv=host)
    B = w.batch
    req = torch.arange(B, dtype=torch.int32, device=dev)
    seq = torch.full((B,), w.seq_len, dtype=torch.int32, device=dev)
    out = torch.empty((B, w.top_k), dtype=torch.int32, device=dev)
    mc = torch.empty(B, dtype=torch.int32, device=dev)
    phases, ends, xcd_end, rates, spans, plan_spans = [], [], [[] for _ in range(8)], [], [], []
    for s in range(calls):
        rows = torch.from_numpy(np.ascontiguousarray(trace[0, s, :, 0])).to(dev)
        st.swap_in_selected(0, req, seq, rows, out, mc)
        torch.cuda.synchronize()
        if s < skip:
            continue
        buf = np.zeros(B * STAMPS, np.int64)
        if fn(buf.ctypes.data, buf.size) != 0:
            raise SystemExit("hisparse_phase_clocks failed")
        t = buf.reshape(B, STAMPS)
        t0 = t[:, 0].min()
        phases.append(np.diff(t[:, :7], axis=1) * TICK_US)
        end = (t[:, 8] - t0) * TICK_US
        ends.append(end)
        for b in range(B):
            xcd_end[b % 8].append(end[b])
        spans.append(end.max())
        plan_spans.append((t[:, 6].max() - t0) * TICK_US)
        copy_us = (t[:, 8].max() - t[:, 7].min()) * TICK_US
        rates.append(t[:, 9].sum() * w.item_bytes / copy_us / 1e3)
    st.close()
    for h in host:
        h.free()
    ph = np.concatenate(phases)
    ends = np.concatenate(ends)
    return {"B": B, "calls": calls - skip, "phase_us": np.median(ph, axis=0),
            "phase_sum_us": float(np.median(ph.sum(axis=1))),
            "plan_span_us": float(np.median(plan_spans)), "span_us": float(np.median(spans)),
            "end_median_us": float(np.median(ends)), "end_p90_us": float(np.percentile(ends, 90)),
            "xcd_end_us": [float(np.median(x)) for x in xcd_end],
            "copy_GBps": float(np.median(rates))}


def _batched_dispatch(torch, binding, workloads, lib):
    """The 512-instance hit-only launch of the batched-state bench: when each
    workgroup starts and how long it runs (stamps of the last launch)."""
    import numpy as np

    import bench

    fn = lib.hisparse_phase_clocks
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int]
    args = argparse.Namespace(warmup=5, steps=20)
    res = bench.batched_state_bench(args, torch, binding, workloads)
    n = res["config"]["batch"]
    buf = np.zeros(n * STAMPS, np.int64)
    if fn(buf.ctypes.data, buf.size) != 0:
        raise SystemExit("hisparse_phase_clocks failed")
    t = buf.reshape(n, STAMPS)
    t0 = t[:, 0].min()
    start = (t[:, 0] - t0) * TICK_US
    run = (t[:, 8] - t[:, 0]) * TICK_US
    first_end = (t[:, 8] - t0).min() * TICK_US
    return {"n": n, "us_per_launch": res["roofline"]["avg_launch_us"],
            "start_span_us": float(start.max()), "start_median_us": float(np.median(start)),
            "run_median_us": float(np.median(run)), "first_end_us": float(first_end),
            "started_before_first_end": int((start < first_end).sum()),
            "wg_per_us": float(n / start.max()) if start.max() > 0 else float("inf")}


def _topk_phases(torch, binding, workloads, lib):
    import numpy as np

    import bench

    fn = lib.hisparse_topk_phase_clocks
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int]
    args = argparse.Namespace(warmup=5, steps=20, workload=2, no_cpu_baseline=True,
                              cpu_seconds=0)
    res = bench.topk_bench(args, torch, binding, workloads)
    n = res["config"]["batch"]
    buf = np.zeros(n * 9, np.int64)
    if fn(buf.ctypes.data, buf.size) != 0:
        raise SystemExit("hisparse_topk_phase_clocks failed")
    # stamps in time order: 0, 1, then 6, 7, 8 inside the threshold, 2 .. 5
    t = buf.reshape(n, 9)[:, [0, 1, 6, 7, 8, 2, 3, 4, 5]]
    return {"n": n, "us_per_call": res["roofline"]["us_per_call"],
            "phase_us": np.median(np.diff(t, axis=1), axis=0) * TICK_US,
            "span_us": float((t[:, -1].max() - t[:, 0].min()) * TICK_US)}


def _merge_phases(torch, binding, workloads, lib):
    import numpy as np

    import bench

    fn = lib.hisparse_topk_merge_phase_clocks
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int]
    args = argparse.Namespace(warmup=5, steps=20, workload=4, no_cpu_baseline=True,
                              cpu_seconds=0)
    res = bench.topk_bench(args, torch, binding, workloads)
    n = res["config"]["batch"]
    buf = np.zeros(n * 7, np.int64)
    if fn(buf.ctypes.data, buf.size) != 0:
        raise SystemExit("hisparse_topk_merge_phase_clocks failed")
    t = buf.reshape(n, 7)
    return {"n": n, "seq_len": res["config"]["seq_len"],
            "us_per_call": res["roofline"]["us_per_call"],
            "phase_us": np.median(np.diff(t, axis=1), axis=0) * TICK_US}


def _attention_waits(torch, binding, workloads, lib):
    import bench

    import numpy as np

    args = argparse.Namespace(warmup=5, steps=20, workload=2, item=1152, heads=128)
    res = bench.attention_bench(args, torch, binding, workloads)
    n = 256                                   # workgroups of a 64-row launch
    fn = lib.hisparse_attention_wait_clocks
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int]
    wv = np.zeros(n * 4 * 3, np.uint64)
    if fn(wv.ctypes.data, wv.size) != 0:
        raise SystemExit("hisparse_attention_wait_clocks failed")
    g, b, total = (float(x) for x in wv.reshape(n * 4, 3).sum(axis=0))
    waves = n * 4
    st = lib.hisparse_attention_phase_clocks
    st.restype = ctypes.c_int
    st.argtypes = [ctypes.c_void_p, ctypes.c_int]
    buf = np.zeros(n * 7, np.int64)
    if st(buf.ctypes.data, buf.size) != 0:
        raise SystemExit("hisparse_attention_phase_clocks failed")
    # stamps in time order: 0, then 6, 4, 5 in the setup, 1, 2, 3
    t = buf.reshape(n, 7)[:, [0, 6, 4, 5, 1, 2, 3]]
    return {"us_per_call": res["roofline"]["us_per_call"], "waves": waves,
            "gather_share": g / total, "barrier_share": b / total,
            "loop_clocks_per_wave": total / waves,
            "phase_us": np.median(np.diff(t, axis=1), axis=0) * TICK_US,
            "span_us": float((t[:, -1].max() - t[:, 0].min()) * TICK_US)}


def run():
    sys.path.insert(0, str(ROOT))
    import torch

    from sparse_attention_kv_request_amd import binding, workloads

    if not VARIANT.exists():
        raise SystemExit(f"{VARIANT} is missing: run this module's build step first")
    binding.LIB_PATH = VARIANT
    lib = binding.lib()
    torch.cuda.set_device(0)
    p = _plan_clocks(torch, binding, workloads, lib)
    d = _batched_dispatch(torch, binding, workloads, lib)
    k = _topk_phases(torch, binding, workloads, lib)
    mg = _merge_phases(torch, binding, workloads, lib)
    a = _attention_waits(torch, binding, workloads, lib)
    print(f"### Plan kernel with its copies: {p['B']} rows, one layer of the headline "
          f"workload, medians over {p['calls']} calls x {p['B']} workgroups\n")
    print("| phase | µs per workgroup |\n|---|---|")
    for name, v in zip(PHASES, p["phase_us"]):
        print(f"| {name} | {v:.2f} |")
    print(f"| sum | {p['phase_sum_us']:.2f} |\n")
    print(f"- last row's plan done {p['plan_span_us']:.1f} µs after the first workgroup started; "
          f"copies done: median row {p['end_median_us']:.1f} µs, 90th percentile "
          f"{p['end_p90_us']:.1f} µs, last {p['span_us']:.1f} µs")
    print("- copy end per XCD (workgroup id mod 8), median µs: " +
          ", ".join(f"XCD {x} {v:.0f}" for x, v in enumerate(p["xcd_end_us"])))
    print(f"- copy phase (first copy start to last copy end): {p['copy_GBps']:.2f} GB/s of miss "
          f"bytes\n")
    print(f"### The same kernel with {d['n']} instances in one launch (batched-state bench, "
          f"hit-only; stamps of the last launch)\n")
    print(f"- workgroup start times spread over {d['start_span_us']:.1f} µs (median "
          f"{d['start_median_us']:.1f} µs): {d['wg_per_us']:.1f} workgroups of 16 waves per µs")
    print(f"- each workgroup runs {d['run_median_us']:.1f} µs (median); the first finishes at "
          f"{d['first_end_us']:.1f} µs, by when {d['started_before_first_end']} have started")
    print(f"- {d['us_per_launch']} µs per launch (HIP events) in this instrumented build\n")
    print(f"### Top-k chunk kernel, {k['n']} rows x 32768 scores, k = 2048 (last launch)\n")
    print("| phase | µs per workgroup |\n|---|---|")
    for name, v in zip(["loads and first-digit histogram",
                        "threshold: first bin picked (4096-bin scan)",
                        "threshold: keys of that bin listed in LDS",
                        "threshold: first list pass (12-bit digit)",
                        "threshold: second list pass (8-bit digit)",
                        "bitmap selection", "output staging", "output"], k["phase_us"]):
        print(f"| {name} | {v:.2f} |")
    print(f"\n- span {k['span_us']:.1f} µs; {k['us_per_call']} µs per call in this instrumented "
          f"build\n")
    print(f"### Top-k merge kernel, {mg['n']} rows x {mg['seq_len']} scores (4 chunks of top-2048 "
          f"per row; last launch)\n")
    print("| phase | µs per workgroup |\n|---|---|")
    for name, v in zip(["chunk offsets published, LDS cleared", "candidate keys and histogram",
                        "exact threshold", "bitmap selection", "output staging", "output"],
                       mg["phase_us"]):
        print(f"| {name} | {v:.2f} |")
    print(f"\n- {mg['us_per_call']} µs per call (chunk + merge kernels) in this instrumented "
          f"build\n")
    print("### bf16 attention kernel (the attention bench's last launch: 64 rows x 128 heads x "
          "2048 locations, 256 workgroups)\n")
    print("| phase (workgroup, last launch) | µs |\n|---|---|")
    for name, v in zip(["setup: locations loaded, rows computed", "setup: row table barrier",
                        "setup: queries and first tile landed (first wave)",
                        "setup: first phase barrier (every wave's queries and tile)",
                        "tile loop", "split partials out"], a["phase_us"]):
        print(f"| {name} | {v:.2f} |")
    print(f"\n- kernel span {a['span_us']:.1f} µs")
    print(f"- share of a wave's loop clocks waiting for the next tile's gather: "
          f"{100 * a['gather_share']:.2f} %; at the phase barrier: {100 * a['barrier_share']:.2f} %")
    print(f"- {a['waves']} waves, {a['loop_clocks_per_wave']:.0f} loop clocks per wave; "
          f"{a['us_per_call']} µs per call in this instrumented build")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("action", choices=["build", "run"])
    if ap.parse_args().action == "build":
        build()
    else:
        run()


if __name__ == "__main__":
    main()
