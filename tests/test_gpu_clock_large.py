"""Multi-step CLOCK through the C ABI against the oracle where the hot buffer
is larger than 4096 slots, up to the pages' limit of 32768 (PR #32162
report, "Risks and impact": the hot_buffer_size boundary is the multi-step
kernel's named test gap), and the pages' own batch-1 four-step shape with 782
unique cross-step misses (same report, "Implementation breakdown" item 4 and
"Key files": a resident set is built up front, then one swap call) started
from an imported CLOCK state with mixed reference bits and a non-zero hand.

Every call is compared on outputs, miss counts, the ordered plan, the error
word, the whole device KV buffer and the exported state of the touched
instances (slot->key, reference bits, hand, key->slot).
"""
import numpy as np
import pytest
import torch

from tests.gpu_harness import Pair, log
from tests.test_gpu_parity import make_rows
from tests.test_oracle_pages_shapes import build_782_case

pytestmark = pytest.mark.gpu

CLOCK_LARGE = [
    # (H, K, N, I, S, calls, R, L, reuse, share): slots per thread 8 (H <= 8192),
    # 16 (H <= 16384) or 32 (H <= 32768); entries per thread 2 (S*K <= 2048) or 8.  `reuse` is
    # the fraction of a call's first step taken from the previous call,
    # `share` the fraction of the first step a later step repeats.
    (6000, 2048, 20000, 32, 4, 8, 3, 2, 0.3, 0.0),     # S*K = 8192 > H: overflow into scratch
    (6000, 1024, 20000, 32, 2, 10, 2, 1, 0.3, 0.5),    # S*K = 2048: two entries per thread
    (8192, 2048, 30000, 16, 4, 8, 3, 2, 0.3, 0.5),     # S*K = H: a call may fill the cache
    (12000, 2048, 40000, 16, 3, 10, 2, 1, 0.3, 0.5),   # 16 slots per thread
    (16384, 1024, 60000, 16, 2, 16, 2, 1, 0.0, 0.5),   # 16 slots, two entries per thread
    (32768, 2048, 65536, 16, 4, 14, 2, 1, 0.3, 0.5),   # the pages' upper bound
    (32768, 1024, 131072, 16, 2, 24, 1, 1, 0.0, 0.0),  # two entries, 32 slots per thread
]


@pytest.mark.parametrize("H,K,N,I,S,calls,R,L,reuse,share", CLOCK_LARGE)
def test_clock_large_hot_buffer(H, K, N, I, S, calls, R, L, reuse, share):
    log(f"clock large H={H} K={K} N={N} I={I} S={S} calls={calls}")
    rng = np.random.default_rng([H, K, S])
    B = min(R, 2)
    p = Pair(R=R, L=L, H=H, K=K, N=N, I=I, S=S, policy="clock", seed=H + S)
    prev = {}
    overflow_rows = evictions = 0
    try:
        for call in range(calls):
            layer = call % L
            req = rng.permutation(R)[:B]
            base = make_rows(rng, B, K, N, prev=prev.get(layer), reuse=reuse)
            prev[layer] = base
            steps = [base] + [make_rows(rng, B, K, N, prev=base, reuse=share)
                              for _ in range(1, S)]
            _, _, want = p.call(layer, req, np.full(B, N), np.stack(steps, axis=1),
                                plan_extra=3 * (call % 2))
            for b, r in enumerate(req):
                plan = want["plan"][b]
                overflow_rows += any(d - p.rows * int(r) >= H for _, d, _ in plan)
                evictions += sum(v != -1 for _, _, v in plan)
        log(f"  rows that overflowed {overflow_rows}, keys evicted {evictions}")
        if S * K > H:
            assert overflow_rows > 0, "the shape was meant to overflow"
        assert evictions > 0, "the cache was meant to fill and evict"
    finally:
        p.close()


def _import_clock(p, req, layer, slot_key, ref, hand):
    ctrl = np.array([0, hand], np.int32)
    p.gpu.import_(req, layer, slot_key, ref, ctrl)
    p.cpu.import_(req, layer, slot_key, ref=ref, hand=hand)
    dev = p.gpu.dev_kv[layer]
    host = p.host[layer].array
    occupied = np.flatnonzero(slot_key >= 0)
    dev[req, torch.from_numpy(occupied).to(dev.device)] = torch.from_numpy(
        host[req, slot_key[occupied]]).to(dev.device)


def test_pages_782_unique_misses_from_imported_clock_state():
    """The pages' correctness shape on the GPU: batch 1, four steps of top-k
    2048 over 32768 tokens, hot buffer 4096, a resident set of 3000 keys
    imported at scattered slots with random reference bits and the hand at
    slot 1234; the four rows name exactly 782 non-resident tokens, each in
    two steps.  miss_count must be 782 and all 782 rows byte-exact."""
    case, resident, topk, pool = build_782_case()
    H, K, N, S = case["H"], case["K"], case["N"], case["S"]
    rng = np.random.default_rng(7821)
    p = Pair(R=1, L=1, H=H, K=K, N=N, I=656, S=S, policy="clock", seed=782)
    try:
        slot_key = np.full(H, -1, np.int32)
        slot_key[rng.choice(H, resident.size, replace=False)] = resident
        ref = np.where(slot_key >= 0, rng.integers(0, 2, H), 0).astype(np.int32)
        _import_clock(p, 0, 0, slot_key, ref, hand=1234)
        p.compare_state(0, 0)                               # export == import
        out, mc, want = p.call(0, [0], [N], topk)
        assert int(mc[0]) == 782 == len(pool)
        assert sorted(s for s, _, _ in want["plan"][0]) == sorted(pool.tolist())
        flat = p.gpu.dev_kv[0].reshape(-1, 656).cpu().numpy()
        host = p.host[0].array.reshape(-1, 656)
        toks = topk.reshape(-1)
        rows = out.reshape(-1)
        assert np.array_equal(flat[rows], host[toks]), "a returned row does not hold its bytes"
        # the hand and reference bits keep evolving from the imported state
        nxt = np.stack([rng.permutation(np.concatenate(
            [rng.choice(resident, 1500, replace=False), rng.choice(pool, 300, replace=False),
             rng.choice(np.setdiff1d(np.arange(N), np.concatenate([resident, pool])), 248,
                        replace=False)])) for _ in range(S)])[None].astype(np.int32)
        p.call(0, [0], [N], nxt)
    finally:
        p.close()


@pytest.mark.parametrize("H,hand", [(4096, 4095), (9000, 17), (32768, 30000)])
def test_clock_import_export_roundtrip_then_calls(H, hand):
    """A CLOCK state imported with mixed reference bits and a hand anywhere in
    [0, H) exports unchanged and then evolves exactly as the oracle's."""
    rng = np.random.default_rng(H + hand)
    K, S, N = 1024, 3, 4 * H
    p = Pair(R=2, L=1, H=H, K=K, N=N, I=16, S=S, policy="clock", seed=H)
    try:
        for req in (0, 1):
            n_res = int(rng.integers(H // 4, H))
            slot_key = np.full(H, -1, np.int32)
            slot_key[rng.choice(H, n_res, replace=False)] = rng.choice(N, n_res, replace=False)
            ref = rng.integers(0, 2, H).astype(np.int32)
            _import_clock(p, req, 0, slot_key, ref, hand=hand if req == 0 else 0)
            p.compare_state(req, 0)
        with pytest.raises(Exception):
            p.gpu.import_(0, 0, np.full(H, -1, np.int32), np.full(H, 2, np.int32),
                          np.array([0, 0], np.int32))      # a reference bit of 2
        with pytest.raises(Exception):
            p.gpu.import_(0, 0, np.full(H, -1, np.int32), np.zeros(H, np.int32),
                          np.array([0, H], np.int32))      # hand outside [0, H)
        p.compare_state(0, 0)                               # rejected imports changed nothing
        prev = None
        for call in range(4):
            base = make_rows(rng, 2, K, N, prev=prev, reuse=0.4)
            prev = base
            steps = [base] + [make_rows(rng, 2, K, N, prev=base, reuse=0.7) for _ in range(1, S)]
            p.call(0, [0, 1], [N, N], np.stack(steps, axis=1))
    finally:
        p.close()
