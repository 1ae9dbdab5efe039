"""Seeded sequences of mixed API operations on one state, every step checked
against the oracle.

Each sequence interleaves, over two layers and five requests: swap calls,
swap calls whose copy is deferred (HISPARSE_PLAN_DEFER_COPY) and replayed by
hisparse_copy_planned on another stream, calls with rejected rows (a request
named twice, a length out of range) and out-of-range indices, request resets
(some naming a request outside the state), and imports of a random valid
instance state.  After every swap call the outputs, plan, error word and the
whole device KV buffer equal the oracle's; after every step the exported
state of every instance does.  Token LRU, page-mode LRU and multi-step CLOCK.
"""
import numpy as np
import pytest
import torch

from tests.gpu_harness import Pair, log

pytestmark = pytest.mark.gpu

R, L = 5, 2
MODES = {
    "lru": dict(P=1, S=1, policy="lru", H=300, K=120, N=2000, I=32),
    "page": dict(P=16, S=1, policy="lru", H=40, K=200, N=16 * 300, I=16),
    "clock": dict(P=1, S=3, policy="clock", H=400, K=150, N=3000, I=32),
}


def _token_row(rng, K, N, prev, bad):
    """K tokens: about half kept from `prev`, the rest fresh; 2 % padding,
    a few in-row duplicates, and (bad) a few indices past N."""
    keep = np.empty(0, np.int64)
    if prev is not None:
        live = np.unique(prev[(prev >= 0) & (prev < N)])
        keep = rng.choice(live, size=min(K // 2, live.size), replace=False)
    mask = np.zeros(N, bool)
    mask[keep] = True
    fresh = rng.choice(np.flatnonzero(~mask), size=K - keep.size, replace=False)
    row = rng.permutation(np.concatenate([keep, fresh]))
    row[rng.random(K) < 0.02] = -1
    dup = rng.random(K) < 0.03
    row[dup] = row[rng.integers(0, K, int(dup.sum()))]
    if bad:
        row[rng.random(K) < 0.02] = N + rng.integers(0, 50)
    return row


def _page_row(rng, K, N, P, H):
    """K tokens in three windows of about 20 pages (at most 60 pages: some
    rows overflow a 40-page cache and are rejected)."""
    centres = rng.integers(0, N, 3)
    row = np.clip(centres[rng.integers(0, 3, K)] + rng.integers(-10 * P, 10 * P, K), 0, N - 1)
    row[rng.random(K) < 0.02] = -1
    return row


def _rows(rng, cfg, B, prev, bad):
    K, N, P, S = cfg["K"], cfg["N"], cfg["P"], cfg["S"]
    if P > 1:
        return np.stack([_page_row(rng, K, N, P, cfg["H"]) for _ in range(B)]).astype(np.int32)
    if S > 1:
        rows = np.empty((B, S, K), np.int64)
        for b in range(B):
            base = _token_row(rng, K, N, prev, bad)
            for s in range(S):  # later steps repeat part of the first
                rows[b, s] = base if s == 0 else _token_row(rng, K, N, base, bad)
        return rows.astype(np.int32)
    return np.stack([_token_row(rng, K, N, prev, bad) for _ in range(B)]).astype(np.int32)


def _import_random(p, rng, cfg, r, l):
    """A random valid instance state on both sides; the GPU's resident rows
    get their bytes (an import moves state only)."""
    H, N, P = cfg["H"], cfg["N"], cfg["P"]
    nkeys = N // P
    n = int(rng.integers(0, H + 1))
    slot_key = np.full(H, -1, np.int32)
    slot_key[rng.choice(H, n, replace=False)] = rng.choice(nkeys, n, replace=False)
    occ = slot_key >= 0
    if cfg["policy"] == "lru":
        now = int(rng.integers(1, 30))
        ts = np.where(occ, rng.integers(0, now, H), -1).astype(np.int32)
        p.gpu.import_(r, l, slot_key, ts, np.array([now, 0], np.int32))
        p.cpu.import_(r, l, slot_key, ts=ts, now=now)
    else:
        ref = rng.integers(0, 2, H).astype(np.int32)
        hand = int(rng.integers(0, H))
        p.gpu.import_(r, l, slot_key, ref, np.array([0, hand], np.int32))
        p.cpu.import_(r, l, slot_key, ref=ref, hand=hand)
    dev = p.gpu.dev_kv[l]
    host = p.host[l].array
    for s in np.flatnonzero(occ):
        k = int(slot_key[s])
        dev[r, s] = torch.from_numpy(host[r, k * P:(k + 1) * P].reshape(-1)).to(dev.device)


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("mode", list(MODES))
def test_mixed_operation_sequence(mode, seed):
    cfg = MODES[mode]
    rng = np.random.default_rng([41, seed, len(mode)])
    p = Pair(R=R, L=L, H=cfg["H"], K=cfg["K"], N=cfg["N"], I=cfg["I"], S=cfg["S"], P=cfg["P"],
             policy=cfg["policy"], seed=100 + seed)
    N = cfg["N"]
    counts = {}
    prev = None
    try:
        for step in range(40):
            op = str(rng.choice(["swap", "deferred", "bad", "reset", "import"],
                                p=[0.4, 0.25, 0.15, 0.1, 0.1]))
            counts[op] = counts.get(op, 0) + 1
            if op in ("swap", "deferred", "bad"):
                B = int(rng.integers(1, R + 1))
                req = rng.permutation(R)[:B].astype(np.int32)
                seq = np.full(B, N, np.int32)
                if op == "bad":
                    if B > 1 and rng.random() < 0.5:
                        req[1] = req[0]                       # a request named twice
                    else:
                        seq[int(rng.integers(0, B))] = N + 1  # a length out of range
                    if rng.random() < 0.5:                    # a shorter valid length
                        seq[0] = min(seq[0], int(rng.integers(cfg["K"], N + 1)))
                rows = _rows(rng, cfg, B, prev, bad=op == "bad")
                if cfg["P"] == 1:
                    prev = rows[0] if rows.ndim == 2 else rows[0, 0]
                p.call(int(rng.integers(0, L)), req, seq, rows, check_state=False,
                       defer=op == "deferred")
            elif op == "reset":
                reqs = rng.permutation(R)[:int(rng.integers(1, R + 1))].tolist()
                outside = rng.random() < 0.3
                dev_reqs = reqs + ([R + 2] if outside else [])
                p.gpu.request_reset(torch.tensor(dev_reqs, dtype=torch.int32, device="cuda"))
                torch.cuda.synchronize()
                p.cpu.request_reset(reqs)
                assert p.gpu.error_flags() == (8 if outside else 0)
            else:
                _import_random(p, rng, cfg, int(rng.integers(0, R)), int(rng.integers(0, L)))
                torch.cuda.synchronize()
            for r in range(R):
                for l in range(L):
                    p.compare_state(r, l)
        log(f"api sequence {mode} seed {seed}: {counts}, every step equal to the oracle")
    finally:
        p.close()
