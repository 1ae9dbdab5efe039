#!/usr/bin/env python3
"""Benchmark of the HiSparse swap-in hot path on one MI355X.

Default workload (single-step LRU, the bench line): 64 requests x 8 layers,
every (request, layer) an independent hot cache of 4096 slots over 32768 host
tokens of 656 bytes (fp8 MLA layout: 512 e4m3 latent + 4 fp32 scales + 64
bf16 rope), top-k 2048 per row and layer, 70 % step-to-step reuse with a
Zipf(1.1) recency bias.  One step is one decode step: the 8 per-layer swap
calls on one stream (one launch each: with 16 or more token rows the plan
kernel copies its rows' misses itself; fewer rows and page mode add the
miss-copy kernel).

``--workload 1|3|4|5`` measures the other workload shapes the same way
(1: B=1 bf16 rows; 3: multi-step CLOCK, also against S sequential LRU calls;
4: miss-heavy long context; 5: page mode).  Inputs (top-k traces) are resident
in HBM and the host KV tier in pinned host memory before the timed region;
reading the host tier over PCIe is the method's own miss copy.  Prints one
JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import pathlib
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "resolved top-k entries/s + miss copy GB/s per swap step, fraction of roofline"
PCIE5_X16_GBPS = 64.0     # published host interface of MI355X, per direction
HBM_PEAK_GBPS = 8000.0    # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--num-steps", type=int, default=4, help="MTP steps of workload 3")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle seconds per worker of the CPU baseline (one worker alone, "
                         "then one per core)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--repeats", type=int, default=5,
                    help="unprofiled timed runs on fresh states; the headline is their median")
    ap.add_argument("--no-link-probe", action="store_true")
    ap.add_argument("--attention", action="store_true",
                    help="time the sparse MLA decode attention over the swapped-in rows "
                         "instead of the swap step")
    ap.add_argument("--heads", type=int, default=128, help="attention heads (--attention)")
    ap.add_argument("--topk", action="store_true",
                    help="time the fused top-k selection + paged index table on the "
                         "batch/sequence shape of --workload (2: 64 x 32768, 4: 128 x 131072)")
    ap.add_argument("--hot", type=int, default=0,
                    help="hot buffer size override (slots, or pages in page mode)")
    ap.add_argument("--admission", default="recent", choices=["recent", "frequent", "first"],
                    help="CLOCK admission priority under multi-step overflow")
    ap.add_argument("--compare-admission", action="store_true",
                    help="workload 3: also run the other two admission priorities on the "
                         "same trace and report their misses per step")
    ap.add_argument("--extra-rows", type=int, default=0,
                    help="extra-row ring of the newest tokens (token mode)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the same steps replayed from HIP graphs (one captured "
                         "graph per step, reported beside the eager steps)")
    ap.add_argument("--batched-state", action="store_true",
                    help="state traffic of the plan kernel with config 2's 512 (request, layer) "
                         "instances in one launch, hit-only steady state")
    ap.add_argument("--item", type=int, default=0,
                    help="KV row bytes for --attention (1152 bf16 or 656 fp8; default: workload's)")
    return ap.parse_args()


def state_bytes_defined(w, m, distinct):
    """Algorithmic state bytes of one row of one call by the byte model the
    scope table fixes for the hit path and state: 16 B per resolved entry
    (4 B index read, 8 B one-bucket probe, 4 B output write), 4 B per
    distinct key (timestamp or reference write), 4 B per hot slot (the
    policy scan of victim selection) and 36 B per miss (8 B hash insert, 8 B
    hash delete, 4 + 4 B slot->key read and write, 12 B of plan)."""
    entries = w.num_steps * w.top_k
    return 16 * entries + 4 * distinct + 4 * w.hot + 36 * m


def state_bytes_kernel(w, m, distinct):
    """The same row by what the plan kernels here must move (no key->slot
    table: the lookup joins the row with the slot->key array): top-k read and
    output write (4 + 4 B per entry), the slot->key array read (4 B per
    slot), the policy state -- LRU: order read + write (2 + 2 B per slot) and
    a timestamp per distinct key (4 B); CLOCK: reference bits read + write
    (H/8 + H/8 B) -- page mode also the page table (4 B per hot page), and
    per miss the slot->key write (4 B), three plan words (12 B) and, in token
    mode, the two words of the host-row-ordered copy list (8 B), plus 16 B of
    request, length and control words."""
    entries = w.num_steps * w.top_k
    H = w.hot
    if w.policy == "clock":
        return 8 * entries + 4 * H + H // 4 + 24 * m + 16
    if w.page_size > 1:
        return 8 * entries + 4 * H + 4 * H + 4 * H + 4 * distinct + 16 * m + 16
    return 8 * entries + 4 * H + 4 * H + 4 * distinct + 24 * m + 16


def distinct_keys(w, trace):
    """Distinct keys per row of every call: tokens over all MTP steps, or
    pages in page mode.  trace: [L, steps, B, S, K] -> [L, steps, B]."""
    import numpy as np

    L, T, B = trace.shape[:3]
    out = np.empty((L, T, B), np.int64)
    for l in range(L):
        for t in range(T):
            for b in range(B):
                keys = trace[l, t, b].reshape(-1)
                keys = keys[keys >= 0] // w.page_size
                out[l, t, b] = np.unique(keys).size
    return out


def link_probes(torch, st, w, rows):
    """Host->HBM link: (i) hipMemcpyAsync of 1 GiB from pinned memory, (ii) the
    miss-copy kernel replaying a plan of consecutive host rows, (iii) the same
    kernel over a random row order (the gather pattern of real misses); and,
    for the HBM roofline's context, a 1 GiB device-to-device copy."""
    dev = torch.device("cuda", 0)
    res = {}
    src = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    src.fill_(1)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    best = 0.0
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src, non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    res["memcpy_h2d_GBps"] = round(best, 2)
    del src
    # HBM for reference: a 1 GiB device-to-device copy (bytes read + written)
    src = torch.empty_like(dst).fill_(2)
    best = 0.0
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, 2 * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    res["hbm_d2d_copy_GBps"] = round(best, 1)
    del src, dst
    B, N, H = w.batch, w.seq_len // w.page_size, w.hot
    unit = w.item_bytes * w.page_size
    per = min(N // 2, max(1, (1 << 30) // (B * unit)))
    mc = torch.full((B,), per, dtype=torch.int32, device=dev)
    j = torch.arange(per, dtype=torch.int32, device=dev)
    r = torch.arange(B, dtype=torch.int32, device=dev)[:, None]
    dst_rows = (r * rows + (j % H)[None, :]).contiguous()
    vic = torch.full((B, per), -1, dtype=torch.int32, device=dev)
    g = torch.Generator(device="cpu").manual_seed(5)
    orders = {"kernel_stream_GBps": j[None, :].expand(B, per),
              "kernel_gather_GBps": torch.stack([torch.randperm(N, generator=g)[:per]
                                                 for _ in range(B)]).to(dev, torch.int32)}
    for name, cols in orders.items():
        src_rows = (r * N + cols).contiguous()
        plan = (src_rows, dst_rows, vic)
        best = 0.0
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            st.copy_planned(0, mc, plan)
            e1.record()
            torch.cuda.synchronize()
            best = max(best, B * per * unit / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        res[name] = round(best, 2)
    # the probe overwrote device rows: empty the caches again
    st.request_reset(torch.arange(w.requests, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    return res


def cpu_baseline(w, overrides, budget_s):
    """The oracle as it stands on the host's cores: one worker process alone,
    then `cores` workers at once (up to 16, the CPU share of one GPU), each
    over its own instances (instances are independent).  Runs before this
    process touches the GPU; the workers are spawned interpreters."""
    import multiprocessing as mp

    from oracle.baseline_worker import run_instances

    cores = max(1, min(16, os.cpu_count() or 1))
    jobs = [(r, l) for l in range(w.layers) for r in range(w.batch)]
    ctx = mp.get_context("spawn")
    with ctx.Pool(1) as pool:
        e1, i1, s1 = pool.map(run_instances, [(w.cfg_id, overrides, jobs, budget_s)])[0]
    with ctx.Pool(cores) as pool:
        outs = pool.map(run_instances, [(w.cfg_id, overrides, jobs[c::cores], budget_s)
                                         for c in range(cores)])
    rate = sum(e / s for e, _, s in outs if s > 0)
    insts = sum(i for _, i, _ in outs)
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(line.split(":", 1)[1].strip() for line in f if line.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": round(rate, 1), "unit": "entries/s", "cores": cores, "kind": "oracle",
            "single_core_value": round(e1 / s1, 1) if s1 > 0 else None,
            "sample": (f"{cores} worker processes x about {budget_s:.0f} s of oracle time each, "
                       f"{insts} whole (request, layer) instances of {w.batch * w.layers} over "
                       f"all {w.steps} steps (byte copies into a shadow device buffer); "
                       f"alone, one worker did {i1} instances at the single-core rate; "
                       f"host: {model}")}


from sparse_attention_kv_request_amd.counters import traffic_from_profiles  # noqa: E402


WORKLOAD_TEXT = {
    1: "single-step LRU swap-in: 1 request, top_k 2048, hot {H}, 8192 host tokens x 1152 B (bf16)",
    2: ("single-step LRU swap-in: 64 requests x 8 layers, top_k 2048, hot buffer {H} slots, "
        "32768 host tokens x 656 B (fp8 MLA), 70% reuse + Zipf(1.1) recency"),
    3: ("multi-step CLOCK swap-in: 64 requests, {S} MTP steps x top_k 2048, hot {H}, "
        "32768 host tokens x 656 B, 80% intra-call share, 60% call-to-call reuse"),
    4: "single-step LRU swap-in: 128 requests, top_k 2048, hot {H}, 131072 host tokens x 656 B, 30% reuse",
    5: ("page-mode LRU swap-in: 32 requests, 256-token pages, 512 clustered tokens, "
        "64 hot pages, 65536 host tokens x 656 B"),
}


class Runner:
    """One workload on the GPU: host tier, traces, state, per-step calls."""

    def __init__(self, torch, binding, workloads, w, policy=None, admission="recent",
                 extra_rows=0, share=None, split=False):
        """split: every swap call defers its copy (HISPARSE_PLAN_DEFER_COPY)
        and the bench replays its plan at once on the same stream with the
        separate miss-copy kernel, timed with HIP events: the lookup kernel
        and the copy kernel of the same calls measured apart."""
        import numpy as np

        self.torch, self.w = torch, w
        self.np = np
        self.dev = torch.device("cuda", 0)
        self.policy = policy or w.policy
        self.owns_host = share is None
        if share is not None:       # same host tier and trace as another runner
            self.host, self.trace, self.topk = share.host, share.trace, share.topk
        else:
            t0 = time.perf_counter()
            self.host = [binding.HostKV(w.requests, w.seq_len, w.item_bytes)
                         for _ in range(w.layers)]
            workloads.fill_host_kv(w, [h.array for h in self.host], threads=16)
            log(f"host KV {w.layers} x {self.host[0].nbytes / 2**30:.2f} GiB in "
                f"{time.perf_counter() - t0:.1f} s")
            t0 = time.perf_counter()
            self.trace = workloads.batch_trace(w, threads=16)     # [L, steps, B, S, K]
            log(f"trace {self.trace.shape} in {time.perf_counter() - t0:.1f} s")
            self.topk = torch.from_numpy(np.ascontiguousarray(
                self.trace.transpose(1, 0, 2, 3, 4))).to(self.dev)  # [steps, L, B, S, K]
        # per-MTP-step rows for the sequential comparator: [steps, L, S, B, K]
        self.topk_seq = (self.topk.permute(0, 1, 3, 2, 4).contiguous()
                         if self.policy != "clock" and w.num_steps > 1 else None)
        B = w.batch
        self.req = torch.arange(B, dtype=torch.int32, device=self.dev)
        self.seq = torch.full((B,), w.seq_len, dtype=torch.int32, device=self.dev)
        multi = self.policy == "clock"
        self.st = binding.HiSparseState(
            max_requests=w.requests, num_layers=w.layers, hot_buffer_size=w.hot,
            top_k=w.top_k, item_size_bytes=w.item_bytes, max_seq_len=w.seq_len,
            max_steps=w.num_steps if multi else 1, page_size=w.page_size, policy=self.policy,
            host_kv=self.host, admission=admission, extra_rows=extra_rows)
        S = w.num_steps
        self.outs = [torch.empty((B, S, w.top_k) if multi else (B, w.top_k), dtype=torch.int32,
                                 device=self.dev) for _ in range(w.layers)]
        calls_per_step = 1 if (multi or S == 1) else S
        self.miss = torch.zeros((w.steps, w.layers, calls_per_step, B), dtype=torch.int32,
                                device=self.dev)
        self.split = split
        self.copy_ev = None
        if split:
            cap = self.st.capacity
            self.plans = [tuple(torch.empty((B, cap), dtype=torch.int32, device=self.dev)
                                for _ in range(3)) for _ in range(w.layers)]
        self.pt = self.npg = None
        if w.page_size > 1:
            self.pt = torch.empty((B, w.hot), dtype=torch.int32, device=self.dev)
            self.npg = torch.empty(B, dtype=torch.int32, device=self.dev)

    def step(self, s):
        st, w = self.st, self.w
        if self.split:
            for l in range(w.layers):
                mc = self.miss[s, l, 0]
                if self.policy == "clock":
                    st.swap_in_spec_multistep(l, self.req, self.seq, self.topk[s, l], self.outs[l],
                                              mc, plan=self.plans[l], defer_copy=True)
                else:
                    st.swap_in_selected(l, self.req, self.seq, self.topk[s, l, :, 0],
                                        self.outs[l], mc, page_table=self.pt,
                                        num_pages=self.npg, plan=self.plans[l], defer_copy=True)
                if self.copy_ev is not None:
                    ev = (self.torch.cuda.Event(enable_timing=True),
                          self.torch.cuda.Event(enable_timing=True))
                    ev[0].record()
                st.copy_planned(l, mc, self.plans[l])
                if self.copy_ev is not None:
                    ev[1].record()
                    self.copy_ev.append(ev)
            return
        for l in range(w.layers):
            if self.policy == "clock":
                st.swap_in_spec_multistep(l, self.req, self.seq, self.topk[s, l], self.outs[l],
                                          self.miss[s, l, 0])
            elif w.num_steps == 1:
                st.swap_in_selected(l, self.req, self.seq, self.topk[s, l, :, 0], self.outs[l],
                                    self.miss[s, l, 0], page_table=self.pt, num_pages=self.npg)
            else:  # sequential comparator: one single-step call per MTP step
                for k in range(w.num_steps):
                    st.swap_in_selected(l, self.req, self.seq, self.topk_seq[s, l, k],
                                        self.outs[l], self.miss[s, l, k])

    def timed(self, W, K, profile=True):
        """W warm-up steps, then K timed steps.  With `profile`, the library
        also records HIP events around each plan and copy launch (per-launch
        durations, at the cost of the event records between launches); the
        step time of such a run is not the headline's."""
        torch = self.torch
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        c0.record()
        for s in range(W):
            self.step(s)
            if s == 0:
                c1.record()
        torch.cuda.synchronize()
        # step 0 on the fresh state: every entry a miss (the cold step)
        self.cold_s = c0.elapsed_time(c1) * 1e-3 if W > 0 else None
        self.st.profile(profile)
        self.st.profile_read()
        self.copy_ev = [] if (profile and self.split) else None
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for s in range(W, W + K):
            self.step(s)
        e1.record()
        torch.cuda.synchronize()
        elapsed = e0.elapsed_time(e1) * 1e-3
        prof = self.st.profile_read()
        self.st.profile(False)
        if self.copy_ev is not None:   # the separate copy kernel of the split calls
            prof["copy_ms"] = sum(a.elapsed_time(b) for a, b in self.copy_ev)
            self.copy_ev = None
        flags = self.st.error_flags()
        if flags:
            raise SystemExit(f"device error flags {flags} during the benchmark")
        m = self.miss[W:W + K].cpu().numpy().astype(self.np.int64)
        return elapsed, prof, m

    def timed_pipelined(self, W, K):
        """The same steps with the copy deferred (HISPARSE_PLAN_DEFER_COPY):
        every swap call runs its plan kernel on one stream and its plan is
        replayed by hisparse_copy_planned on a second stream behind an event,
        so layer l's host reads overlap the plan kernels of the next layers.
        Plans are double-buffered per layer; a plan kernel waits for the copy
        that last read its buffer (two calls back).  Returns (elapsed seconds
        of the K timed steps, miss counts [K, L, 1, B])."""
        torch, w, st = self.torch, self.w, self.st
        B, L, cap = w.batch, w.layers, st.capacity
        plans = [[tuple(torch.empty((B, cap), dtype=torch.int32, device=self.dev)
                        for _ in range(3)) for _ in range(2)] for _ in range(L)]
        freed = [[None, None] for _ in range(L)]
        ps, cs = torch.cuda.Stream(), torch.cuda.Stream()
        torch.cuda.synchronize()

        def step(s):
            for l in range(L):
                buf = plans[l][s % 2]
                if freed[l][s % 2] is not None:
                    ps.wait_event(freed[l][s % 2])
                mc = self.miss[s, l, 0]
                if self.policy == "clock":
                    st.swap_in_spec_multistep(l, self.req, self.seq, self.topk[s, l], self.outs[l],
                                              mc, plan=buf, stream=ps, defer_copy=True)
                else:
                    st.swap_in_selected(l, self.req, self.seq, self.topk[s, l, :, 0],
                                        self.outs[l], mc, page_table=self.pt,
                                        num_pages=self.npg, plan=buf, stream=ps,
                                        defer_copy=True)
                planned = torch.cuda.Event()
                planned.record(ps)
                cs.wait_event(planned)
                st.copy_planned(l, mc, buf, stream=cs)
                done = torch.cuda.Event()
                done.record(cs)
                freed[l][s % 2] = done

        for s in range(W):
            step(s)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(ps)
        for s in range(W, W + K):
            step(s)
        cs.wait_stream(ps)
        e1.record(cs)
        torch.cuda.synchronize()
        if self.st.error_flags():
            raise SystemExit("device error flags during the pipelined steps")
        return e0.elapsed_time(e1) * 1e-3, self.miss[W:W + K].cpu().numpy().astype(self.np.int64)

    def replay_rate(self, s_rec, reps):
        """The plan/copy split: step s_rec's layer calls record their miss
        plans (this state has made steps 0 .. s_rec - 1), then the recorded
        plans are replayed `reps` times by the copy alone
        (hisparse_copy_planned), timed with HIP events.  Returns (miss bytes
        per replay of the 8 layers, seconds per replay)."""
        torch, w, st = self.torch, self.w, self.st
        for s in range(s_rec):
            self.step(s)
        cap = st.capacity
        B = w.batch
        plans, counts = [], []
        for l in range(w.layers):
            plan = tuple(torch.empty((B, cap), dtype=torch.int32, device=self.dev)
                         for _ in range(3))
            mc = torch.empty(B, dtype=torch.int32, device=self.dev)
            if self.policy == "clock":
                st.swap_in_spec_multistep(l, self.req, self.seq, self.topk[s_rec, l], self.outs[l],
                                          mc, plan=plan)
            else:
                st.swap_in_selected(l, self.req, self.seq, self.topk[s_rec, l, :, 0], self.outs[l],
                                    mc, page_table=self.pt, num_pages=self.npg, plan=plan)
            plans.append(plan)
            counts.append(mc)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for l in range(w.layers):
                st.copy_planned(l, counts[l], plans[l])
        e1.record()
        torch.cuda.synchronize()
        if st.error_flags():
            raise SystemExit("device error flags during the plan replays")
        misses = sum(int(c.sum().item()) for c in counts)
        return misses * w.item_bytes * w.page_size, e0.elapsed_time(e1) * 1e-3 / reps

    def timed_graphs(self, W, K):
        """The timed steps of timed() replayed from HIP graphs: each step's
        layer calls are captured once (on a side stream, outside the timed
        region) and replayed in order.  Runs on a fresh state after W eager
        warm-up steps, like timed()."""
        torch = self.torch
        for s in range(W):
            self.step(s)
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        graphs = []
        for s in range(W, W + K):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                self.step(s)
            graphs.append(g)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for g in graphs:
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        flags = self.st.error_flags()
        if flags:
            raise SystemExit(f"device error flags {flags} during the graph replays")
        return e0.elapsed_time(e1) * 1e-3

    def close(self):
        self.st.close()
        if self.owns_host:
            for h in self.host:
                h.free()


BF16_MFMA_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak


def batched_state_bench(args, torch, binding, workloads):
    """Plan-kernel state traffic with many instances per launch: config 2's
    64 requests x 8 layers as 512 requests of one layer, all resolved by one
    swap call.  After the first (cold) call every later call repeats the same
    top-k rows, so every entry hits: the step is the plan kernel alone
    (lookup, hit touch, LRU order rewrite, outputs; the copy it does for a
    call of this many rows has nothing to move).  Host KV bytes are left zero
    (no miss reads them after call 0)."""
    import numpy as np

    W, K = args.warmup, args.steps
    w = workloads.config(2, steps=2)
    R = w.batch * w.layers
    host = [binding.HostKV(R, w.seq_len, w.item_bytes)]
    st = binding.HiSparseState(max_requests=R, num_layers=1, hot_buffer_size=w.hot,
                               top_k=w.top_k, item_size_bytes=w.item_bytes,
                               max_seq_len=w.seq_len, host_kv=host)
    trace = workloads.batch_trace(w, threads=16)             # [L, steps, B, 1, K]
    rows = np.ascontiguousarray(trace[:, 0, :, 0].reshape(R, w.top_k))
    dev = torch.device("cuda", 0)
    topk = torch.from_numpy(rows).to(dev)
    req = torch.arange(R, dtype=torch.int32, device=dev)
    seq = torch.full((R,), w.seq_len, dtype=torch.int32, device=dev)
    out = torch.empty((R, w.top_k), dtype=torch.int32, device=dev)
    mc = torch.empty(R, dtype=torch.int32, device=dev)
    for _ in range(1 + W):
        st.swap_in_selected(0, req, seq, topk, out, mc)
    torch.cuda.synchronize()
    st.profile(True)
    st.profile_read()
    for _ in range(K):
        st.swap_in_selected(0, req, seq, topk, out, mc)
    torch.cuda.synchronize()
    prof = st.profile_read()
    st.profile(False)
    if int(mc.sum().item()) != 0 or st.error_flags():
        raise SystemExit("the batched-state steady state must be hit-only and error-free")
    distinct = np.array([np.unique(r[r >= 0]).size for r in rows])
    per_launch = sum(state_bytes_defined(w, 0, int(d)) for d in distinct)
    per_launch_kernel = sum(state_bytes_kernel(w, 0, int(d)) for d in distinct)
    plan_s = prof["plan_ms"] * 1e-3 / prof["calls"]
    st.close()
    host[0].free()
    gbps = per_launch / plan_s / 1e9
    return {"metric": "plan-kernel state GB/s, 512 instances per launch, hit-only",
            "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
            "ms_per_step": round(plan_s * 1e3, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "int32", "data": "synthetic",
            "config": {"workload": "config 2 instances (64 requests x 8 layers) as 512 rows of "
                                   "one launch, top_k 2048, hot 4096, step-0 rows repeated",
                       "batch": R, "top_k": w.top_k, "hot_buffer_size": w.hot},
            "roofline": {"bound": "hbm", "kernel": "lru_token_plan", "achieved": round(gbps, 2),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps / HBM_PEAK_GBPS, 4),
                         "avg_launch_us": round(plan_s * 1e6, 2), "bytes_per_launch": per_launch,
                         "kernel_model_bytes_per_launch": per_launch_kernel,
                         "kernel_model_GBps": round(per_launch_kernel / plan_s / 1e9, 2),
                         "traffic": traffic_from_profiles("lru_token_plan", "batched 512", W, K)}}


def attention_bench(args, torch, binding, workloads):
    """Sparse MLA decode attention over the rows the swap step left in the hot
    buffer: per row 2048 locations x `heads` heads; FLOPs 2 * (576 + 512)
    per (row, head, location); bytes = KV rows + q + out + lse + locations."""
    import numpy as np

    W, K = args.warmup, args.steps
    w = workloads.config(args.workload, steps=W + 1)
    if args.item:
        w = w.replace(item_bytes=args.item)
    item = w.item_bytes
    run = Runner(torch, binding, workloads, w)
    for s in range(W + 1):
        run.step(s)
    torch.cuda.synchronize()
    # valid MLA rows in the hot buffer: overwrite the random bytes with
    # well-formed latent/rope rows (the attention reads only what was copied)
    rng = np.random.default_rng(9)
    for l in range(w.layers):
        dev = run.st.dev_kv[l]
        flat = dev.reshape(-1, item)
        rows = torch.from_numpy(workloads.mla_kv_rows(rng, 4096, item)).to(dev.device)
        idx = torch.arange(flat.shape[0], device=dev.device) % 4096
        flat.copy_(rows[idx])
    B, H = w.batch, args.heads
    q = torch.from_numpy(workloads.mla_queries(rng, B, H).view(np.int16)).view(
        torch.bfloat16).to(run.dev)
    out = torch.empty((B, H, 512), dtype=torch.float32, device=run.dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=run.dev)
    need = binding.hisparse_sparse_mla_workspace_bytes(run.st.handle, B, H, w.top_k)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=run.dev)
    locs = [run.outs[l] for l in range(w.layers)]
    for l in range(w.layers):
        run.st.sparse_mla_decode(l, q, locs[l], out, lse, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        for l in range(w.layers):
            run.st.sparse_mla_decode(l, q, locs[l], out, lse, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    calls = K * w.layers
    per_call = e0.elapsed_time(e1) * 1e-3 / calls
    valid = int(sum(int((x >= 0).sum()) for x in locs)) // w.layers
    flops = 2.0 * (576 + 512) * H * valid
    byts = valid * item + B * H * (576 * 2 + 512 * 4 + 4) + B * w.top_k * 4
    splits = (need // (B * H * (512 * 2 + 8 * 4))) if need else 1  # fp16 partials + m, l, exponents
    run.close()
    tflops = flops / per_call / 1e12
    gbps = byts / per_call / 1e9
    return {
        "metric": "sparse MLA decode attention over swapped-in rows, TFLOP/s",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(per_call * 1e3 * w.layers, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"decode attention, {B} rows x {H} heads x {w.top_k} locations, "
                               f"{item}-B rows ({'fp8' if item == 656 else 'bf16'})",
                   "batch": B, "heads": H, "locations": w.top_k, "item_size_bytes": item,
                   "layers": w.layers, "splits": splits},
        "roofline": {"bound": "mfma" if flops / byts > BF16_MFMA_TFLOPS / 8.0 else "hbm",
                     "achieved_tflops": round(tflops, 2), "peak_tflops": BF16_MFMA_TFLOPS,
                     "frac_mfma": round(tflops / BF16_MFMA_TFLOPS, 4),
                     "achieved_GBps": round(gbps, 1), "peak_GBps": HBM_PEAK_GBPS,
                     "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4),
                     "us_per_call": round(per_call * 1e6, 2),
                     "flops_per_call": flops, "bytes_per_call": byts,
                     "traffic": traffic_from_profiles("mla_decode", f"{args.workload} attention "
                                                      f"{item} heads {H}", W, K)},
    }


def topk_bench(args, torch, binding, workloads):
    """Fused top-k selection + PAGED index table over synthetic indexer scores:
    one plan per step, one build per layer (8 layers, different scores each).
    Bytes per call = scores read + indices and locations written + the page
    table entries of the selected positions."""
    import time

    import numpy as np

    W, K = args.warmup, args.steps
    w = workloads.config(args.workload)
    B, N, k, P, L = w.batch, w.seq_len, w.top_k, 64, 8
    rng = np.random.default_rng(17)
    lens = np.full(B, N, np.int32)
    dev = torch.device("cuda", 0)
    logits = [torch.from_numpy(workloads.indexer_logits(rng, B, N)).to(dev) for _ in range(L)]
    pt = torch.from_numpy(rng.permutation(B * (N // P)).astype(np.int32).reshape(B, N // P)).to(dev)
    sl = torch.from_numpy(lens).to(dev)
    bld = binding.TopkIndexBuilder(B, N, k, device=dev)
    idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    locs = torch.empty((B, k), dtype=torch.int32, device=dev)
    bld.plan(sl)
    for _ in range(W):
        for l in range(L):
            bld.build(logits[l], sl, idx, locs, mode="paged", page_table=pt, page_size=P)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        bld.plan(sl)
        for l in range(L):
            bld.build(logits[l], sl, idx, locs, mode="paged", page_table=pt, page_size=P)
    e1.record()
    torch.cuda.synchronize()
    per_call = e0.elapsed_time(e1) * 1e-3 / (K * L)
    assert bld.error_flags() == 0
    byts = int(lens.sum()) * 4 + B * k * 12
    res = {
        "metric": "fused top-k selection + paged index table, rows/s",
        "value": round(B / per_call, 1), "unit": "rows/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(per_call * 1e3 * L, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"top-{k} of {B} rows x {N} indexer scores, paged table P={P}",
                   "batch": B, "seq_len": N, "top_k": k, "layers": L, "page_size": P},
        "roofline": {"bound": "hbm", "achieved": round(byts / per_call / 1e9, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(byts / per_call / 1e9 / HBM_PEAK_GBPS, 4),
                     "us_per_call": round(per_call * 1e6, 2), "bytes_per_call": byts,
                     "traffic": traffic_from_profiles("topk", f"{args.workload} topk", W, K)},
    }
    if not args.no_cpu_baseline:
        from oracle import topk_oracle
        host = logits[0].cpu().numpy()
        t0, rows = time.perf_counter(), 0
        while rows < B and time.perf_counter() - t0 < args.cpu_seconds:
            topk_oracle.topk_row(host[rows], N, k)
            rows += 1
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(rows / dt, 2), "unit": "rows/s", "cores": 1,
                               "kind": "oracle", "sample": f"{rows} rows of {N} scores, k={k}"}
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (every "
              "(request, layer) cache instance is independent, so requests would shard "
              "across GPUs with no exchange step). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from sparse_attention_kv_request_amd import workloads

    swap_mode = not (args.attention or args.topk or args.batched_state)
    over = {"steps": args.warmup + args.steps}
    if args.workload == 3:
        over["num_steps"] = args.num_steps
    if args.hot:
        over["hot"] = args.hot
    cpu_res = None
    if swap_mode and not args.no_cpu_baseline:
        # before this process touches the GPU: the workers are spawned
        log("timing the CPU oracle baseline")
        cpu_res = cpu_baseline(workloads.config(args.workload, **over), over, args.cpu_seconds)

    import torch

    from sparse_attention_kv_request_amd import binding

    torch.cuda.set_device(0)
    if args.attention:
        print(json.dumps(attention_bench(args, torch, binding, workloads)), flush=True)
        return
    if args.topk:
        print(json.dumps(topk_bench(args, torch, binding, workloads)), flush=True)
        return
    if args.batched_state:
        print(json.dumps(batched_state_bench(args, torch, binding, workloads)), flush=True)
        return
    W, K = args.warmup, args.steps
    w = workloads.config(args.workload, **over)
    run = Runner(torch, binding, workloads, w, admission=args.admission,
                 extra_rows=args.extra_rows)
    link = {} if args.no_link_probe else link_probes(torch, run.st, w, run.st.rows)
    if link:
        log(f"link probes {link}")
    # per-launch plan and copy durations (HIP events around each launch) ...
    elapsed_prof, prof, m = run.timed(W, K)
    fused = prof["calls"] > 0 and prof["fused_calls"] == prof["calls"]
    sprof = prof
    if fused:
        # the calls copied inside the lookup kernel: the same calls again with
        # the lookup kernel and the separate copy kernel timed apart
        s_run = Runner(torch, binding, workloads, w, admission=args.admission,
                       extra_rows=args.extra_rows, share=run, split=True)
        _, sprof, s_m = s_run.timed(W, K)
        s_run.close()
        if not (s_m == m).all():
            raise SystemExit("the split run missed different entries than the fused one")
    # ... and the step time of the same steps without those events, repeated
    # on fresh states (the median is the headline)
    runs, colds = [], []
    for _ in range(max(1, args.repeats)):
        u_run = Runner(torch, binding, workloads, w, admission=args.admission,
                       extra_rows=args.extra_rows, share=run)
        el, _, m_u = u_run.timed(W, K, profile=False)
        colds.append(u_run.cold_s)
        u_run.close()
        if not (m_u == m).all():
            raise SystemExit("an unprofiled run missed different entries than the profiled one")
        runs.append(el)
    elapsed = sorted(runs)[len(runs) // 2]

    unit = w.item_bytes * w.page_size
    miss_bytes = int(m.sum()) * unit
    entries = K * w.entries_per_step
    calls = prof["calls"]
    copy_s = sprof["copy_ms"] * 1e-3          # the separate copy kernel's summed time
    copy_gbps = miss_bytes / copy_s / 1e9
    plan_s = sprof["plan_ms"] * 1e-3          # the lookup kernel alone
    measured_link = max((v for k, v in link.items() if k != "hbm_d2d_copy_GBps"), default=None)
    dist = distinct_keys(w, run.trace[:, W:W + K])           # [L, K, B]
    pairs = list(zip(m[:, :, 0, :].transpose(1, 0, 2).reshape(-1), dist.reshape(-1)))
    state_bytes = sum(state_bytes_defined(w, int(x), int(d)) for x, d in pairs)
    state_bytes_k = sum(state_bytes_kernel(w, int(x), int(d)) for x, d in pairs)
    plan_kernel = {"lru": "lru_page_plan" if w.page_size > 1 else "lru_token_plan",
                   "clock": "clock_plan"}[w.policy]
    cfg = {"workload": WORKLOAD_TEXT[args.workload].format(S=w.num_steps, H=w.hot),
           "batch": w.batch, "layers": w.layers, "num_steps": w.num_steps, "top_k": w.top_k,
           "hot_buffer_size": w.hot, "seq_len": w.seq_len, "item_size_bytes": w.item_bytes,
           "page_size": w.page_size, "policy": w.policy}
    if w.policy == "clock":
        cfg["admission"] = args.admission
    if args.extra_rows:
        cfg["extra_rows"] = args.extra_rows
    res = {
        "metric": METRIC,
        "value": round(entries / elapsed, 1),
        "unit": "entries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(elapsed * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": cfg,
        "repeats": {"ms_per_step": [round(x * 1e3 / K, 4) for x in runs],
                    "statistic": "median", "state": "fresh per repeat, same trace"},
        "cold_step_ms": (round(sorted(colds)[len(colds) // 2] * 1e3, 4)
                         if colds and colds[0] is not None else None),
        "ms_per_step_profiled": round(elapsed_prof * 1e3 / K, 4),
        "step_over_copy_time": round(elapsed / copy_s, 4),
        "copy_in_lookup_kernel": fused,
        "miss_copy": {"GBps_per_step": round(miss_bytes / elapsed / 1e9, 2),
                      "bytes_per_step": miss_bytes // K,
                      "misses_per_step": int(m.sum()) // K},
        "link": link,
    }
    # the dominant kernel: the one that moves the misses over the host link
    # (the lookup kernel itself when it copies, else the miss-copy kernel)
    split = f"{args.workload} split" if fused else args.workload
    copy_kernel = {"bound": "pcie", "kernel": "miss_copy",
                   "achieved": round(copy_gbps, 2), "peak": PCIE5_X16_GBPS, "unit": "GB/s",
                   "frac": round(copy_gbps / PCIE5_X16_GBPS, 4),
                   "traffic": traffic_from_profiles("miss_copy", split, W, K),
                   "avg_launch_us": round(copy_s * 1e6 / max(calls, 1), 2),
                   "bytes_per_launch": miss_bytes // max(calls, 1),
                   "measured_link_GBps": measured_link,
                   "frac_of_measured_link": (round(copy_gbps / measured_link, 4)
                                             if measured_link else None)}
    if fused:
        fused_s = prof["plan_ms"] * 1e-3
        f_gbps = miss_bytes / fused_s / 1e9
        res["roofline"] = {"bound": "pcie", "kernel": f"{plan_kernel} (lookup and copy)",
                           "achieved": round(f_gbps, 2), "peak": PCIE5_X16_GBPS, "unit": "GB/s",
                           "frac": round(f_gbps / PCIE5_X16_GBPS, 4),
                           "traffic": traffic_from_profiles(plan_kernel, args.workload, W, K),
                           "avg_launch_us": round(fused_s * 1e6 / max(calls, 1), 2),
                           "bytes_per_launch": miss_bytes // max(calls, 1),
                           "measured_link_GBps": measured_link,
                           "frac_of_measured_link": (round(f_gbps / measured_link, 4)
                                                     if measured_link else None)}
        res["split_copy_kernel"] = copy_kernel
    else:
        res["roofline"] = copy_kernel
    res["state_roofline"] = {
        "bound": "hbm", "kernel": plan_kernel + (" (copy deferred)" if fused else ""),
        "achieved": round(state_bytes / plan_s / 1e9, 2),
        "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(state_bytes / plan_s / 1e9 / HBM_PEAK_GBPS, 5),
        "traffic": traffic_from_profiles(plan_kernel, split, W, K),
        "avg_launch_us": round(plan_s * 1e6 / max(calls, 1), 2),
        "bytes_per_launch": state_bytes // max(calls, 1),
        "kernel_model_bytes_per_launch": state_bytes_k // max(calls, 1),
        "kernel_model_GBps": round(state_bytes_k / plan_s / 1e9, 2)}
    # the copy deferred and replayed on a second stream: plans overlap copies
    if w.policy == "clock" or w.num_steps == 1:
        p_run = Runner(torch, binding, workloads, w, admission=args.admission,
                       extra_rows=args.extra_rows, share=run)
        p_elapsed, p_m = p_run.timed_pipelined(W, K)
        p_run.close()
        if not (p_m == m).all():
            raise SystemExit("the pipelined run missed different entries than the eager one")
        res["pipelined"] = {"ms_per_step": round(p_elapsed * 1e3 / K, 4),
                            "entries_per_s": round(entries / p_elapsed, 1),
                            "step_over_copy_time": round(p_elapsed / copy_s, 4)}
    if args.workload == 3:
        # the per-step path the multi-step call replaces: S single-step LRU calls
        seq_run = Runner(torch, binding, workloads, w, policy="lru", share=run)
        seq_elapsed, _, _ = seq_run.timed(W, K, profile=False)
        seq_run.close()
        res["sequential_lru"] = {
            "ms_per_call_multistep": round(elapsed * 1e3 / (K * w.layers), 4),
            "ms_per_call_sequential": round(seq_elapsed * 1e3 / (K * w.layers), 4),
            "latency_reduction": round(1 - elapsed / seq_elapsed, 4)}
    if args.compare_admission and w.policy == "clock":
        cmp = {args.admission: {"misses_per_step": int(m.sum()) // K,
                                "ms_per_step": round(elapsed * 1e3 / K, 4)}}
        for adm in ("recent", "frequent", "first"):
            if adm in cmp:
                continue
            other = Runner(torch, binding, workloads, w, admission=adm,
                           extra_rows=args.extra_rows, share=run)
            o_el, _, o_m = other.timed(W, K, profile=False)
            other.close()
            cmp[adm] = {"misses_per_step": int(o_m.sum()) // K,
                        "ms_per_step": round(o_el * 1e3 / K, 4)}
        res["admission_compare"] = cmp
    log("timing the replay of recorded miss plans (copy only)")
    r_run = Runner(torch, binding, workloads, w, admission=args.admission,
                   extra_rows=args.extra_rows, share=run)
    r_bytes, r_sec = r_run.replay_rate(W + K - 1, 10)
    r_run.close()
    res["plan_replay"] = {"kernel": "miss_copy", "bytes_per_replay": r_bytes,
                          "ms_per_replay": round(r_sec * 1e3, 4),
                          "GBps": round(r_bytes / r_sec / 1e9, 2),
                          "frac_of_measured_link": (round(r_bytes / r_sec / 1e9 / measured_link, 4)
                                                    if measured_link else None)}
    if not args.no_graph:
        log("timing the same steps replayed from HIP graphs")
        g_run = Runner(torch, binding, workloads, w, admission=args.admission,
                       extra_rows=args.extra_rows, share=run)
        g_elapsed = g_run.timed_graphs(W, K)
        g_run.close()
        res["graph"] = {"ms_per_step_eager": round(elapsed * 1e3 / K, 4),
                        "ms_per_step_graph": round(g_elapsed * 1e3 / K, 4),
                        "entries_per_s_graph": round(entries / g_elapsed, 1)}
    if cpu_res is not None:
        res["cpu_baseline"] = cpu_res
    run.close()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
