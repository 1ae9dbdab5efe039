"""GPU (HIP path through the C ABI) against the CPU oracle, element by element.

Sizes are small enough for the oracle to finish in seconds yet span several
thread tiles with ragged tails (K and H not multiples of the 1024-thread
workgroup or of 32-bit mask words), and every call is compared on outputs,
plan, error word, the whole device KV buffer and the touched instances' state.
"""
import numpy as np
import pytest
import torch

from tests.gpu_harness import Pair, log

pytestmark = pytest.mark.gpu


def make_rows(rng, B, K, N, prev=None, reuse=0.6, pad=0.02, dup=0.03, bad=0.0):
    """Top-k rows with step-to-step reuse, padding, in-row duplicates and
    (optionally) out-of-range entries."""
    rows = np.empty((B, K), np.int64)
    for b in range(B):
        if prev is not None and reuse > 0:
            keep = rng.choice(prev[b][prev[b] >= 0], size=min(int(reuse * K), int((prev[b] >= 0).sum())),
                              replace=False)
        else:
            keep = np.empty(0, np.int64)
        mask = np.zeros(N, bool)
        mask[keep] = True
        fresh = rng.choice(np.flatnonzero(~mask), size=K - keep.size, replace=False)
        rows[b] = rng.permutation(np.concatenate([keep, fresh]))
    u = rng.random((B, K))
    src = rng.integers(0, K, (B, K))
    rows = np.where(u < dup, np.take_along_axis(rows, src, 1), rows)
    rows = np.where((u >= dup) & (u < dup + pad), -1, rows)
    if bad:
        v = rng.random((B, K))
        rows = np.where(v < bad / 2, N + rng.integers(0, 5, (B, K)), rows)
        rows = np.where((v >= bad / 2) & (v < bad), -2 - rng.integers(0, 5, (B, K)), rows)
    return rows.astype(np.int32)


LRU_SHAPES = [
    # (H, K, N, I) -- ragged tiles, K == H, cfg-1-like bf16 rows, EPH = 8 variant
    (3000, 1500, 6000, 48),
    (100, 37, 300, 16),
    (300, 300, 1000, 32),
    (4096, 2048, 8192, 1152),
    (8000, 2048, 20000, 656),
    (5000, 3000, 9000, 32),      # K > 2048: 8 entries per thread
]


@pytest.mark.parametrize("H,K,N,I", LRU_SHAPES)
def test_lru_token_parity(H, K, N, I):
    log(f"lru token H={H} K={K} N={N} I={I}")
    rng = np.random.default_rng(H + K)
    R, L, B = 5, 2, 4
    p = Pair(R=R, L=L, H=H, K=K, N=N, I=I, seed=H)
    prev = {}
    try:
        for call in range(10):
            layer = call % L
            req = rng.permutation(R)[:B]
            rows = make_rows(rng, B, K, N, prev=prev.get(layer))
            prev[layer] = rows
            p.call(layer, req, np.full(B, N), rows, plan_extra=7 * (call % 2))
    finally:
        p.close()


def _random_lru_case(case):
    """Case `case` of a seeded sweep of the single-step LRU token path: top-k
    size (1 to 4096, ragged against the thread tiles), hot size, host length,
    item size, batch, layers, and the rows' reuse, in-row duplicate, padding
    and out-of-range rates."""
    rng = np.random.default_rng([20261204, case])
    K = int(rng.choice([1, 2, 31, 64, 257, 1000, 2048, 2049, 3000, 4096]))
    H = min(int(K + rng.integers(0, 3000)), 32768)
    N = int(max(K + 1, H // 2) + rng.integers(0, 6000))
    I = int(rng.choice([16, 32, 48, 656]))
    R = int(rng.integers(1, 7))
    B = int(rng.integers(1, R + 1))
    L = int(rng.integers(1, 3))
    return dict(K=K, H=H, N=N, I=I, R=R, B=B, L=L, reuse=float(rng.choice([0.0, 0.5, 0.9])),
                dup=float(rng.choice([0.0, 0.03, 0.3])), pad=float(rng.choice([0.0, 0.02, 0.2])),
                bad=float(rng.choice([0.0, 0.0, 0.01])))


@pytest.mark.parametrize("case", range(32))
def test_lru_token_random_shapes(case):
    c = _random_lru_case(case)
    log(f"lru token random case {case}: {c}")
    rng = np.random.default_rng([7, case])
    p = Pair(R=c["R"], L=c["L"], H=c["H"], K=c["K"], N=c["N"], I=c["I"], seed=case)
    prev = {}
    try:
        for call in range(6):
            layer = call % c["L"]
            req = rng.permutation(c["R"])[:c["B"]]
            rows = make_rows(rng, c["B"], c["K"], c["N"], prev=prev.get(layer), reuse=c["reuse"],
                             pad=c["pad"], dup=c["dup"], bad=c["bad"])
            prev[layer] = np.where(rows < c["N"], rows, -1)   # reuse only valid tokens
            p.call(layer, req, np.full(c["B"], c["N"]), rows)
    finally:
        p.close()


PAGE_SHAPES = [
    # (P, pages per request, H pages, K tokens, I)
    (16, 150, 64, 300, 32),
    (256, 64, 64, 512, 656),
    (4, 1000, 200, 700, 16),
]


@pytest.mark.parametrize("P,NP,H,K,I", PAGE_SHAPES)
def test_lru_page_parity(P, NP, H, K, I):
    log(f"lru page P={P} NP={NP} H={H} K={K} I={I}")
    rng = np.random.default_rng(P * 7 + K)
    R, L, B = 4, 1, 3
    N = P * NP
    p = Pair(R=R, L=L, H=H, K=K, N=N, I=I, P=P, seed=P)
    try:
        for call in range(10):
            req = rng.permutation(R)[:B]
            rows = np.empty((B, K), np.int64)
            for b in range(B):   # clustered tokens: a few page windows
                centres = rng.integers(0, N, 4)
                width = max(P * 3, 8)
                toks = np.clip(centres[rng.integers(0, 4, K)] + rng.integers(-width, width, K),
                               0, N - 1)
                rows[b] = toks
            if call == 4:        # one row naming more pages than the hot cache holds
                rows[0] = rng.choice(N, K, replace=False)
            rows[:, ::17] = -1
            p.call(0, req, np.full(B, N), rows.astype(np.int32))
    finally:
        p.close()


CLOCK_SHAPES = [
    # (H, K, N, I, S)
    (1000, 700, 5000, 32, 2),
    (1000, 700, 5000, 32, 4),
    (50, 100, 400, 16, 3),       # overflow every call
    (4096, 2048, 32768, 656, 4),  # S * K = 8192 entries per row
    (3000, 1024, 9000, 48, 3),
]


@pytest.mark.parametrize("H,K,N,I,S", CLOCK_SHAPES)
def test_clock_multistep_parity(H, K, N, I, S):
    log(f"clock H={H} K={K} N={N} I={I} S={S}")
    rng = np.random.default_rng(H + 3 * K + S)
    R, L, B = 4, 2, 3
    p = Pair(R=R, L=L, H=H, K=K, N=N, I=I, S=S, policy="clock", seed=K)
    prev = {}
    try:
        for call in range(8):
            layer = call % L
            req = rng.permutation(R)[:B]
            base = make_rows(rng, B, K, N, prev=prev.get(layer), reuse=0.5)
            prev[layer] = base
            steps = [base]
            for s in range(1, S):  # later steps share most of the first step's entries
                nxt = make_rows(rng, B, K, N, prev=base, reuse=0.8)
                steps.append(nxt)
            topk = np.stack(steps, axis=1)
            p.call(layer, req, np.full(B, N), topk, plan_extra=5 * (call % 2))
    finally:
        p.close()


def _random_clock_case(case):
    """Case `case` of a seeded sweep of the multi-step CLOCK path: steps,
    top-k size, hot size from half of K (overflow on every call) to 4K, host
    length, item size, requests, layers, reuse between calls and between
    steps, duplicate and padding rates, admission priority and the
    extra-row ring."""
    rng = np.random.default_rng([20261205, case])
    S = int(rng.integers(2, 5))
    K = int(rng.choice([1, 7, 64, 300, 1024, 2048]))
    H = max(1, min(int(rng.choice([max(1, K // 2), K, K + 500, 4 * K + 7])), 32768))
    N = int(K + 1 + rng.integers(0, 8000))
    return dict(S=S, K=K, H=H, N=N, I=int(rng.choice([16, 48, 656])), R=int(rng.integers(1, 5)),
                L=int(rng.integers(1, 3)), reuse=float(rng.choice([0.0, 0.5, 0.9])),
                share=float(rng.choice([0.5, 0.8, 1.0])), dup=float(rng.choice([0.0, 0.03])),
                pad=float(rng.choice([0.0, 0.05])),
                admission=str(rng.choice(["recent", "frequent", "first"])),
                extra=int(rng.choice([0, 0, 16])))


@pytest.mark.parametrize("case", range(24))
def test_clock_random_shapes(case):
    c = _random_clock_case(case)
    log(f"clock random case {case}: {c}")
    rng = np.random.default_rng([8, case])
    B = int(rng.integers(1, c["R"] + 1))
    p = Pair(R=c["R"], L=c["L"], H=c["H"], K=c["K"], N=c["N"], I=c["I"], S=c["S"], policy="clock",
             seed=case, admission=c["admission"], extra_rows=c["extra"])
    prev = {}
    try:
        for call in range(6):
            layer = call % c["L"]
            req = rng.permutation(c["R"])[:B]
            base = make_rows(rng, B, c["K"], c["N"], prev=prev.get(layer), reuse=c["reuse"],
                             dup=c["dup"], pad=c["pad"])
            prev[layer] = base
            steps = [base] + [make_rows(rng, B, c["K"], c["N"], prev=np.where(base >= 0, base, -1),
                                        reuse=c["share"], dup=c["dup"], pad=c["pad"])
                              for _ in range(1, c["S"])]
            p.call(layer, req, np.full(B, c["N"]), np.stack(steps, axis=1))
    finally:
        p.close()


def _random_page_case(case):
    """Case `case` of a seeded sweep of page mode: page size, pages per
    request, hot pages (some calls name more pages than fit: rejected rows),
    token count, item size, requests."""
    rng = np.random.default_rng([20261206, case])
    P = int(rng.choice([4, 16, 64, 256]))
    NP = int(rng.integers(8, 400))
    return dict(P=P, NP=NP, H=int(rng.integers(4, 200)), K=int(rng.integers(1, 1024)),
                I=int(rng.choice([16, 32])), R=int(rng.integers(1, 5)))


@pytest.mark.parametrize("case", range(24))
def test_lru_page_random_shapes(case):
    c = _random_page_case(case)
    log(f"page random case {case}: {c}")
    rng = np.random.default_rng([9, case])
    N = c["P"] * c["NP"]
    B = int(rng.integers(1, c["R"] + 1))
    p = Pair(R=c["R"], L=1, H=c["H"], K=c["K"], N=N, I=c["I"], P=c["P"], seed=case)
    try:
        for call in range(6):
            req = rng.permutation(c["R"])[:B]
            rows = np.empty((B, c["K"]), np.int64)
            for b in range(B):   # clustered tokens: four page windows
                centres = rng.integers(0, N, 4)
                width = max(c["P"] * 3, 8)
                rows[b] = np.clip(centres[rng.integers(0, 4, c["K"])]
                                  + rng.integers(-width, width, c["K"]), 0, N - 1)
            rows[:, ::13] = -1
            p.call(0, req, np.full(B, N), rows.astype(np.int32))
    finally:
        p.close()


def test_clock_with_fewer_steps_than_max():
    rng = np.random.default_rng(5)
    p = Pair(R=3, L=1, H=200, K=64, N=1000, I=16, S=4, policy="clock", seed=5)
    try:
        for call in range(8):
            S = 2 + call % 3
            topk = rng.integers(-1, 1000, (2, S, 64))
            p.call(0, rng.permutation(3)[:2], [1000, 1000], topk)
    finally:
        p.close()


def test_row_errors_and_padding():
    rng = np.random.default_rng(11)
    R, H, K, N = 6, 64, 40, 500
    p = Pair(R=R, L=1, H=H, K=K, N=N, I=16, seed=11)
    try:
        rows = make_rows(rng, 5, K, N, bad=0.1)
        rows[3] = -1                                            # all padding
        # rows 0 and 4 name the same request; row 2 has an out-of-range request
        p.call(0, [1, 2, 9, 3, 1], [N, 300, N, N, N], rows)
        rows = make_rows(rng, 4, K, N, bad=0.05)
        p.call(0, [0, 1, 2, 3], [N, 0, N + 1, -1], rows)         # seq_len 0, too long, negative
        rows = make_rows(rng, 3, K, N)
        p.call(0, [1, 2, 3], [N, N, N], rows)                    # clean call afterwards
    finally:
        p.close()


def test_request_reset_then_reuse():
    rng = np.random.default_rng(12)
    R, H, K, N = 4, 128, 100, 1000
    p = Pair(R=R, L=2, H=H, K=K, N=N, I=32, seed=12)
    try:
        for call in range(4):
            p.call(call % 2, [0, 1, 2], [N] * 3, make_rows(rng, 3, K, N))
        p.gpu.request_reset(torch.tensor([1, 7], dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        p.cpu.request_reset([1])
        assert p.gpu.error_flags() == 8                           # request 7 is out of range
        for r in range(R):
            for l in range(2):
                p.compare_state(r, l)
        for call in range(4):
            p.call(call % 2, [2, 1, 3], [N] * 3, make_rows(rng, 3, K, N))
    finally:
        p.close()


def test_import_export_roundtrip():
    rng = np.random.default_rng(13)
    R, H, K, N, I = 2, 300, 120, 2000, 32
    p = Pair(R=R, L=1, H=H, K=K, N=N, I=I, seed=13)
    try:
        keys = rng.choice(N, H - 40, replace=False)
        slot_key = np.full(H, -1, np.int32)
        where = rng.choice(H, keys.size, replace=False)
        slot_key[where] = keys
        ts = np.where(slot_key >= 0, rng.integers(0, 5, H), -1).astype(np.int32)
        ctrl = np.array([5, 0], np.int32)
        p.gpu.import_(1, 0, slot_key, ts, ctrl)
        p.cpu.import_(1, 0, slot_key, ts=ts, now=5)
        dev = p.gpu.dev_kv[0]
        for s in np.flatnonzero(slot_key >= 0):                   # resident rows hold their bytes
            dev[1, s] = torch.from_numpy(p.host[0].array[1, slot_key[s]])
        p.compare_state(1, 0)
        for _ in range(5):
            p.call(0, [1], [N], make_rows(rng, 1, K, N, prev=None), check_bytes=True)
        with pytest.raises(Exception):
            bad = slot_key.copy()
            bad[0] = bad[1] = 3
            p.gpu.import_(1, 0, bad, ts, ctrl)
    finally:
        p.close()


def test_hot_buffer_upper_bound():
    """hot_buffer_size at the pages' upper limit of 32768 slots."""
    rng = np.random.default_rng(14)
    H, K, N = 32768, 2048, 65536
    p = Pair(R=2, L=1, H=H, K=K, N=N, I=16, seed=14)
    try:
        prev = None
        for call in range(20):
            rows = make_rows(rng, 2, K, N, prev=prev, reuse=0.3)
            prev = rows
            p.call(0, [0, 1], [N, N], rows, check_state=(call % 5 == 4))
    finally:
        p.close()


SIXTEEN_SLOTS = [
    # (H, K, N): token caches of 8193..16384 slots run 16 slots per thread;
    # K <= 2048 two entries per thread, else eight
    (12000, 2048, 60000),
    (16384, 3000, 65536),
]


@pytest.mark.parametrize("H,K,N", SIXTEEN_SLOTS)
def test_lru_sixteen_slots_per_thread(H, K, N):
    log(f"LRU, 16 slots per thread: H={H} K={K} N={N}")
    rng = np.random.default_rng([H, K])
    p = Pair(R=2, L=1, H=H, K=K, N=N, I=16, seed=H)
    try:
        prev = None
        for call in range(16):   # about K/2 fresh keys per call: the cache fills, then evicts
            rows = make_rows(rng, 2, K, N, prev=prev, reuse=0.5)
            prev = rows
            p.call(0, [0, 1], [N, N], rows, check_state=(call % 4 == 3))
        assert len(p.cpu.instance(0, 0).key_slot) == H, "the cache was meant to fill"
    finally:
        p.close()


def test_host_side_argument_errors():
    p = Pair(R=2, L=1, H=64, K=16, N=100, I=16, seed=15)
    dev = torch.device("cuda", 0)
    i32 = dict(dtype=torch.int32, device=dev)
    req = torch.zeros(1, **i32)
    seq = torch.full((1,), 100, **i32)
    topk = torch.zeros((1, 16), **i32)
    out = torch.zeros((1, 16), **i32)
    mc = torch.zeros(1, **i32)
    from sparse_attention_kv_request_amd import binding as bd
    try:
        h = p.gpu.handle
        assert bd.hisparse_swap_in_selected(h, 1, 1, req.data_ptr(), seq.data_ptr(),
                                            topk.data_ptr(), out.data_ptr(), mc.data_ptr(),
                                            0, 0, None, 0) == bd.HISPARSE_E_INVAL   # layer
        assert bd.hisparse_swap_in_selected(h, 0, 3, req.data_ptr(), seq.data_ptr(),
                                            topk.data_ptr(), out.data_ptr(), mc.data_ptr(),
                                            0, 0, None, 0) == bd.HISPARSE_E_INVAL   # batch
        assert bd.hisparse_swap_in_selected(h, 0, 1, 0, seq.data_ptr(), topk.data_ptr(),
                                            out.data_ptr(), mc.data_ptr(), 0, 0, None,
                                            0) == bd.HISPARSE_E_INVAL               # NULL
        assert bd.hisparse_swap_in_spec_multistep(h, 0, 1, 2, req.data_ptr(), seq.data_ptr(),
                                                  topk.data_ptr(), out.data_ptr(),
                                                  mc.data_ptr(), None,
                                                  0) == bd.HISPARSE_E_INVAL         # policy
        assert bd.hisparse_swap_in_selected(h, 0, 0, 0, 0, 0, 0, 0, 0, 0, None,
                                            0) == bd.HISPARSE_OK                    # empty batch
        small = bd.HisparseMissPlan(out.data_ptr(), out.data_ptr(), out.data_ptr(), 15)
        import ctypes
        assert bd.hisparse_swap_in_selected(h, 0, 1, req.data_ptr(), seq.data_ptr(),
                                            topk.data_ptr(), out.data_ptr(), mc.data_ptr(),
                                            0, 0, ctypes.byref(small),
                                            0) == bd.HISPARSE_E_INVAL               # capacity
        cap = p.gpu.capacity
        plan_t = [torch.zeros((1, cap), **i32) for _ in range(3)]
        bad_flags = bd.HisparseMissPlan(*(x.data_ptr() for x in plan_t), cap, 2)
        assert bd.hisparse_swap_in_selected(h, 0, 1, req.data_ptr(), seq.data_ptr(),
                                            topk.data_ptr(), out.data_ptr(), mc.data_ptr(),
                                            0, 0, ctypes.byref(bad_flags),
                                            0) == bd.HISPARSE_E_INVAL               # flags
        with pytest.raises(ValueError):
            p.gpu.swap_in_selected(0, req, seq, topk, out, mc, defer_copy=True)
        # a pageable host buffer is not a valid host tier
        cfg = bd.HisparseConfig(max_requests=2, num_layers=1, hot_buffer_size=64, top_k=16,
                                max_steps=1, page_size=1, item_size_bytes=16, max_seq_len=100,
                                policy=0, max_batch=2)
        pageable = np.zeros(2 * 100 * 16, np.uint8)
        hp = (ctypes.c_void_p * 1)(pageable.ctypes.data)
        dp = (ctypes.c_void_p * 1)(p.gpu.dev_kv[0].data_ptr())
        cfg.host_kv = ctypes.cast(hp, ctypes.POINTER(ctypes.c_void_p))
        cfg.dev_kv = ctypes.cast(dp, ctypes.POINTER(ctypes.c_void_p))
        with pytest.raises(bd.HiSparseError):
            bd.hisparse_state_create(cfg, 0)
    finally:
        p.close()


@pytest.mark.parametrize("B", [2, 18])   # 18 rows: the call itself copies inside its plan kernel
def test_copy_planned_replays_the_plan(B):
    """Replaying the plan of a swap call reproduces its copies; an entry outside
    the buffers is skipped and flagged instead of being written."""
    rng = np.random.default_rng(16 + B)
    R, H, K, N, I = B + 1, 200, 150, 1000, 32
    reqs = [r for r in range(R) if r != 1]
    p = Pair(R=R, L=1, H=H, K=K, N=N, I=I, seed=16)
    dev = torch.device("cuda", 0)
    try:
        p.call(0, reqs, [N] * B, make_rows(rng, B, K, N))
        cap = p.gpu.capacity
        plan = tuple(torch.full((B, cap), -1, dtype=torch.int32, device=dev) for _ in range(3))
        mc = torch.empty(B, dtype=torch.int32, device=dev)
        out = torch.empty((B, K), dtype=torch.int32, device=dev)
        rows = torch.from_numpy(make_rows(rng, B, K, N)).to(dev)
        p.gpu.swap_in_selected(0, torch.tensor(reqs, dtype=torch.int32, device=dev),
                               torch.full((B,), N, dtype=torch.int32, device=dev), rows, out, mc,
                               plan=plan)
        torch.cuda.synchronize()
        p.gpu.dev_kv[0].zero_()
        p.gpu.copy_planned(0, mc, plan)
        torch.cuda.synchronize()
        host = torch.from_numpy(p.host[0].array).reshape(-1, I)
        flat = p.gpu.dev_kv[0].reshape(-1, I).cpu()
        src, dst = plan[0].cpu(), plan[1].cpu()
        n = mc.cpu()
        assert int(n.sum()) > 0
        for b in range(B):
            for j in range(int(n[b])):
                assert torch.equal(flat[dst[b, j]], host[src[b, j]])
        assert p.gpu.error_flags() == 0
        bad_src = plan[0].clone()
        bad_src[0, 0] = R * N + 5
        p.gpu.copy_planned(0, mc, (bad_src, plan[1], plan[2]))
        torch.cuda.synchronize()
        assert p.gpu.error_flags() == 16
    finally:
        p.close()


def _deferred_rows(rng, mode, B, S, K, N, P, prev):
    if mode == "page":   # three windows of 17 pages: at most 51 distinct pages per row
        rows = np.empty((B, K), np.int64)
        for b in range(B):
            centres = rng.integers(0, N, 3)
            rows[b] = np.clip(centres[rng.integers(0, 3, K)] + rng.integers(-8 * P, 8 * P, K),
                              0, N - 1)
        rows[:, ::13] = -1
        return rows.astype(np.int32)
    rows = np.stack([make_rows(rng, B, K, N, prev=prev, reuse=0.5) for _ in range(S)], 1)
    return rows if S > 1 else rows[:, 0]


@pytest.mark.parametrize("mode", ["lru", "page", "clock"])
def test_deferred_copy_pipelined_matches_eager(mode):
    """Swap calls with HISPARSE_PLAN_DEFER_COPY on one stream and their plans
    replayed by hisparse_copy_planned on another, the host never waiting in
    between: layer l's copy overlaps layer l+1's plan and later steps' plans.
    Outputs, miss counts and plans equal those of eager swap calls on a twin
    state (itself checked against the oracle after every call), and once the
    copies have landed the hot KV bytes are equal too."""
    rng = np.random.default_rng([31, len(mode)])
    R, L, K, I, B = 4, 3, 300, 32, 3
    S = 3 if mode == "clock" else 1
    P = 16 if mode == "page" else 1
    N, H = (4000, 500) if P == 1 else (16 * 400, 60)
    policy = "clock" if mode == "clock" else "lru"
    kw = dict(R=R, L=L, H=H, K=K, N=N, I=I, S=S, P=P, policy=policy, seed=31)
    eager, piped = Pair(**kw), Pair(**kw, shadow=False)
    dev = torch.device("cuda", 0)
    i32 = dict(dtype=torch.int32, device=dev)
    try:
        req_np = np.array([0, 1, 3], np.int32)
        req, seq = torch.from_numpy(req_np).to(dev), torch.full((B,), N, **i32)
        cap = piped.gpu.capacity
        calls, prev = [], None
        for step in range(4):                       # inputs and outputs, all allocated up front
            for l in range(L):
                rows = _deferred_rows(rng, mode, B, S, K, N, P, prev)
                prev = rows[:, 0] if S > 1 else (rows if P == 1 else None)
                c = dict(l=l, rows=rows, topk=torch.from_numpy(rows).to(dev),
                         out=torch.full(rows.shape, -7, **i32), mc=torch.full((B,), -7, **i32),
                         plan=tuple(torch.full((B, cap), -7, **i32) for _ in range(3)))
                if P > 1:
                    c["pt"], c["np"] = torch.full((B, H), -7, **i32), torch.full((B,), -7, **i32)
                calls.append(c)
        torch.cuda.synchronize()
        plan_s, copy_s = torch.cuda.Stream(), torch.cuda.Stream()
        for c in calls:
            if S > 1:
                piped.gpu.swap_in_spec_multistep(c["l"], req, seq, c["topk"], c["out"], c["mc"],
                                                 plan=c["plan"], stream=plan_s, defer_copy=True)
            else:
                piped.gpu.swap_in_selected(c["l"], req, seq, c["topk"], c["out"], c["mc"],
                                           page_table=c.get("pt"), num_pages=c.get("np"),
                                           plan=c["plan"], stream=plan_s, defer_copy=True)
            ev = torch.cuda.Event()
            ev.record(plan_s)
            copy_s.wait_event(ev)
            piped.gpu.copy_planned(c["l"], c["mc"], c["plan"], stream=copy_s)
        torch.cuda.synchronize()
        assert piped.gpu.error_flags() == 0
        misses = 0
        for c in calls:
            want_out, want_mc, want = eager.call(c["l"], req_np, [N] * B, c["rows"])
            assert np.array_equal(c["out"].cpu().numpy(), want_out)
            assert np.array_equal(c["mc"].cpu().numpy(), want_mc)
            if P > 1:
                assert np.array_equal(c["pt"].cpu().numpy(), want["page_table"])
            src, dst, vic = (x.cpu().numpy() for x in c["plan"])
            for b in range(B):
                m = int(want_mc[b])
                assert list(zip(src[b, :m].tolist(), dst[b, :m].tolist(), vic[b, :m].tolist())) \
                    == [tuple(x) for x in want["plan"][b]]
            misses += int(want_mc.sum())
        for l in range(L):
            assert torch.equal(piped.gpu.dev_kv[l], eager.gpu.dev_kv[l]), f"layer {l} KV differs"
        for r in req_np:
            for l in range(L):
                a, b = piped.gpu.export(int(r), l), eager.gpu.export(int(r), l)
                assert np.array_equal(a["slot_key"], b["slot_key"])
        log(f"deferred copy {mode}: {len(calls)} calls, {misses} misses, equal to eager")
    finally:
        piped.close()
        eager.close()


@pytest.mark.parametrize("B", [3, 20])   # 20 rows: the copy runs inside the plan kernel
@pytest.mark.parametrize("policy", ["lru", "clock"])
def test_graph_capture_replays_match_eager(policy, B):
    """Swap calls allocate nothing and never synchronise, so a call can be
    captured in a HIP graph; each replay (inputs refreshed by eager copies in
    between) must equal the same call made eagerly on a twin state."""
    rng = np.random.default_rng(21 + B)
    R, H, K, N, I = B + 1, 500, 300, 3000, 32
    S = 3 if policy == "clock" else 1
    eager = Pair(R=R, L=1, H=H, K=K, N=N, I=I, S=S, policy=policy, seed=21)
    graph = Pair(R=R, L=1, H=H, K=K, N=N, I=I, S=S, policy=policy, seed=21)
    dev = torch.device("cuda", 0)
    try:
        reqs = [r for r in range(R) if r != 1]     # B requests, one left out
        req = torch.tensor(reqs, dtype=torch.int32, device=dev)
        seq = torch.full((B,), N, dtype=torch.int32, device=dev)
        shape = (B, S, K) if S > 1 else (B, K)
        topk_buf = torch.zeros(shape, dtype=torch.int32, device=dev)
        out_g = torch.empty(shape, dtype=torch.int32, device=dev)
        mc_g = torch.empty(B, dtype=torch.int32, device=dev)
        side = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            if S > 1:
                graph.gpu.swap_in_spec_multistep(0, req, seq, topk_buf, out_g, mc_g)
            else:
                graph.gpu.swap_in_selected(0, req, seq, topk_buf, out_g, mc_g)
        torch.cuda.synchronize()
        prev = None
        for step in range(6):
            rows = np.stack([make_rows(rng, B, K, N, prev=prev, reuse=0.5) for _ in range(S)], 1)
            prev = rows[:, 0]
            rows = rows if S > 1 else rows[:, 0]
            topk_buf.copy_(torch.from_numpy(rows).to(dev))
            g.replay()
            torch.cuda.synchronize()
            got, got_mc = out_g.cpu().numpy(), mc_g.cpu().numpy()
            want_out, want_mc, _ = eager.call(0, reqs, [N] * B, rows)
            assert np.array_equal(got, want_out), f"replay {step} differs"
            assert np.array_equal(got_mc, want_mc)
            assert torch.equal(graph.gpu.dev_kv[0], eager.gpu.dev_kv[0])
        for r in reqs:
            a, b = graph.gpu.export(r, 0, with_map=True), eager.gpu.export(r, 0, with_map=True)
            for key in ("slot_key", "ctrl", "key_slot"):
                assert np.array_equal(a[key], b[key])
    finally:
        graph.close()
        eager.close()


PAGE_LARGE_TOPK = [
    # (P, pages per request, H pages, K tokens, I, windows): top-k above 2048
    # tokens takes the 8-entries-per-thread page kernel
    (16, 2000, 600, 2049, 32, 6),
    (8, 6000, 2000, 4096, 16, 16),
    (64, 1000, 300, 8192, 16, 3),
]


@pytest.mark.parametrize("P,NP,H,K,I,windows", PAGE_LARGE_TOPK)
def test_lru_page_large_topk(P, NP, H, K, I, windows):
    log(f"lru page large top-k P={P} NP={NP} H={H} K={K} I={I}")
    rng = np.random.default_rng([P, K])
    R, B = 3, 2
    N = P * NP
    p = Pair(R=R, L=1, H=H, K=K, N=N, I=I, P=P, seed=K)
    try:
        for call in range(8):
            req = rng.permutation(R)[:B]
            rows = np.empty((B, K), np.int64)
            for b in range(B):   # clustered tokens: `windows` windows of 80 pages
                centres = rng.integers(0, N, windows)
                w = 40 * P
                rows[b] = np.clip(centres[rng.integers(0, windows, K)] + rng.integers(-w, w, K),
                                  0, N - 1)
            rows[:, ::11] = -1
            p.call(0, req, np.full(B, N), rows.astype(np.int32))
    finally:
        p.close()


def test_batch_at_the_limit():
    """A call of HISPARSE_MAX_BATCH rows (16000): the miss copy's per-row
    prefix then fills its LDS to the limit, and every row is still copied."""
    B, H, K, N = 16000, 8, 4, 16
    rng = np.random.default_rng(17)
    p = Pair(R=B, L=1, H=H, K=K, N=N, I=16, seed=17)
    try:
        for call in range(3):
            rows = np.stack([rng.choice(N, K, replace=False) for _ in range(B)])
            _, mc, _ = p.call(0, np.arange(B), np.full(B, N), rows, check_state=False)
            assert int(mc.sum()) > 0
        for r in (0, 7777, B - 1):
            p.compare_state(r, 0)
    finally:
        p.close()


KEY_RANGE_SHAPES = [
    # (policy, N, H, K, S): the plan kernels index a row's keys by their rank
    # in an LDS bitmap of the request's keys when it fits (N <= 2^18 and the
    # LDS budget), and by an LDS hash otherwise
    ("lru", 200000, 4096, 2048, 1),     # a large bitmap (6250 words)
    ("lru", 300000, 4096, 2048, 1),     # beyond a bitmap: the hash path
    ("lru", 262144, 5000, 3000, 1),     # 2^18 keys with K = 3000: LDS too small for bitmaps
    ("clock", 300000, 3000, 1024, 4),   # hash path with overflow into scratch rows
    ("clock", 200000, 8192, 2048, 3),   # a large bitmap, 32 slots per thread
]


@pytest.mark.parametrize("policy,N,H,K,S", KEY_RANGE_SHAPES)
def test_key_range_paths(policy, N, H, K, S):
    log(f"key range policy={policy} N={N} H={H} K={K} S={S}")
    rng = np.random.default_rng([N, K, S])
    R, B = 2, 2
    p = Pair(R=R, L=1, H=H, K=K, N=N, I=16, S=S, policy=policy, seed=N % 1000)
    prev = None
    try:
        for call in range(6):
            base = make_rows(rng, B, K, N, prev=prev, reuse=0.5)
            prev = base
            if S == 1:
                topk = base
            else:
                topk = np.stack([base] + [make_rows(rng, B, K, N, prev=base, reuse=0.3)
                                          for _ in range(1, S)], axis=1)
            p.call(0, [0, 1], [N, N], topk)
    finally:
        p.close()
