"""Oracle replay of whole cache instances of the five full-size workloads, for
the full-size parity tests.  TEST INFRASTRUCTURE: it runs in spawned worker
processes that never touch the GPU.

Each job regenerates one (request, layer) instance's top-k trace from its
seeds (the shared input generators) and runs it through the CPU oracle with
the instance's real request and layer numbers, so the rows, plans and state
it returns are directly comparable with what the library wrote for that row.
"""
from __future__ import annotations

import numpy as np

from oracle import hisparse_oracle as ora


def replay_instance(job):
    """job = (config id, workload overrides, request, layer).  Returns a dict
    with per-call ``out`` [calls, S*K] (or [calls, K]), ``miss_count``
    [calls], ``plan`` (list over calls of int32 [m, 3]), page mode
    ``page_table`` [calls, H] and ``num_pages`` [calls], and the final
    exported state."""
    from sparse_attention_kv_request_amd import workloads

    cfg_id, overrides, r, l = job
    w = workloads.config(cfg_id, **overrides)
    multi = w.policy == "clock"
    trace = workloads.instance_trace(w, r, l)            # [calls, S, K]
    st = ora.OracleState(max_requests=w.requests, num_layers=w.layers, hot=w.hot,
                         top_k=w.top_k, item_bytes=w.item_bytes, max_seq_len=w.seq_len,
                         max_steps=w.num_steps if multi else 1, page_size=w.page_size,
                         policy=w.policy)
    outs, mcs, plans, pts, nps = [], [], [], [], []
    for c in range(trace.shape[0]):
        if multi:
            res = st.swap_in_spec_multistep(l, [r], [w.seq_len], trace[c:c + 1])
        else:
            res = st.swap_in_selected(l, [r], [w.seq_len], trace[c:c + 1, 0])
        outs.append(np.asarray(res["out_locs"][0], np.int32).reshape(-1))
        mcs.append(int(res["miss_count"][0]))
        plans.append(np.asarray(res["plan"][0], np.int32).reshape(-1, 3))
        if w.page_size > 1:
            pts.append(np.asarray(res["page_table"][0], np.int32))
            nps.append(int(res["num_pages"][0]))
    inst = st.instance(r, l)
    out = {"r": r, "l": l, "out": np.stack(outs), "miss_count": np.asarray(mcs, np.int32),
           "plan": plans, "slot_key": np.asarray(inst.slot_key, np.int32),
           "ts": np.asarray(inst.ts, np.int32), "now": inst.now,
           "ref": np.asarray(inst.ref, np.int32), "hand": inst.hand,
           "map_keys": np.asarray(sorted(inst.key_slot), np.int32),
           "map_slots": np.asarray([inst.key_slot[k] for k in sorted(inst.key_slot)], np.int32),
           "flags": st.error_flags}
    if w.page_size > 1:
        out["page_table"] = np.stack(pts)
        out["num_pages"] = np.asarray(nps, np.int32)
    return out
