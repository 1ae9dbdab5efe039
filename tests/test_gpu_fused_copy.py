"""Swap calls whose copy runs inside the plan kernel, against the oracle.

Token-row swap calls of 16 rows or more copy their misses from the plan
kernel (each row's workgroup moves its own misses after its commit); fewer
rows, whole pages and deferred calls use the separate copy kernel.  These
cases put batches on both sides of that threshold through the C ABI and
compare every call with the oracle on outputs, miss counts, the ordered plan,
the error word, the whole device KV buffer and the exported state: single-step
LRU (key bitmaps and the LDS hash path, one and eight entries per thread),
multi-step CLOCK with and without overflow into scratch rows, rows rejected
inside a fused call, and fused calls interleaved with deferred ones.
"""
import numpy as np
import pytest

from tests.gpu_harness import Pair, log
from tests.test_gpu_parity import make_rows

pytestmark = pytest.mark.gpu

FUSE_MIN_ROWS = 16


def _lru_case(case):
    rng = np.random.default_rng([20261215, case])
    K = int(rng.choice([1, 64, 257, 1000, 2048, 3000]))
    H = int(K + rng.integers(0, 2500))
    # case 1 names keys past 2^18 (no key bitmaps: the LDS hash path)
    N = 300000 if case == 1 else int(max(K + 1, H // 2) + rng.integers(0, 5000))
    B = int(rng.integers(FUSE_MIN_ROWS, 41))
    return dict(K=K, H=H, N=N, I=16 if case == 1 else int(rng.choice([16, 48, 656])),
                R=B + int(rng.integers(0, 8)), B=B, L=int(rng.integers(1, 3)),
                reuse=float(rng.choice([0.0, 0.5, 0.9])), dup=float(rng.choice([0.0, 0.03])),
                pad=float(rng.choice([0.0, 0.02])), bad=float(rng.choice([0.0, 0.01])))


@pytest.mark.parametrize("case", range(16))
def test_fused_lru_random(case):
    c = _lru_case(case)
    log(f"fused lru case {case}: {c}")
    rng = np.random.default_rng([15, case])
    p = Pair(R=c["R"], L=c["L"], H=c["H"], K=c["K"], N=c["N"], I=c["I"], seed=case)
    prev = {}
    try:
        for call in range(5):
            layer = call % c["L"]
            req = rng.permutation(c["R"])[:c["B"]]
            rows = make_rows(rng, c["B"], c["K"], c["N"], prev=prev.get(layer), reuse=c["reuse"],
                             pad=c["pad"], dup=c["dup"], bad=c["bad"])
            prev[layer] = np.where(rows < c["N"], rows, -1)
            seq = np.full(c["B"], c["N"])
            if call == 3:
                seq[5] = c["N"] + 1          # one rejected row inside a fused call
            if call == 4:
                req[7] = req[2]              # a request named twice: both rows rejected
            p.call(layer, req, seq, rows, plan_extra=3 * (call % 2))
    finally:
        p.close()


CLOCK_CASES = [
    # (B, R, H, K, N, I, S, reuse, share): with S*K > H the steps' union
    # (share = 0: S*K keys) overflows into scratch rows
    (16, 20, 900, 300, 4000, 48, 4, 0.3, 0.0),
    (24, 24, 3000, 1024, 9000, 656, 2, 0.5, 0.8),
    (33, 40, 5000, 2048, 300000, 16, 3, 0.3, 0.0),   # no key bitmaps: the LDS hash path
    (20, 22, 6000, 2048, 20000, 16, 4, 0.0, 0.0),    # 8 entries per thread, 8 slots per thread
]


@pytest.mark.parametrize("B,R,H,K,N,I,S,reuse,share", CLOCK_CASES)
def test_fused_clock(B, R, H, K, N, I, S, reuse, share):
    log(f"fused clock B={B} R={R} H={H} K={K} N={N} I={I} S={S}")
    rng = np.random.default_rng([B, H, S])
    p = Pair(R=R, L=1, H=H, K=K, N=N, I=I, S=S, policy="clock", seed=H)
    prev = None
    overflow = 0
    try:
        for call in range(5):
            req = rng.permutation(R)[:B]
            base = make_rows(rng, B, K, N, prev=prev, reuse=reuse, pad=0.02)
            prev = base
            steps = [base] + [make_rows(rng, B, K, N, prev=np.where(base >= 0, base, -1),
                                        reuse=share, pad=0.02) for _ in range(1, S)]
            _, _, want = p.call(0, req, np.full(B, N), np.stack(steps, axis=1))
            for b, r in enumerate(req):
                overflow += any(d - p.rows * int(r) >= H for _, d, _ in want["plan"][b])
        log(f"  rows with scratch-row misses: {overflow}")
        if S * K > H:
            assert overflow > 0, "the shape was meant to overflow"
    finally:
        p.close()


@pytest.mark.parametrize("admission", ["frequent", "first"])
def test_fused_clock_admission_and_ring(admission):
    """Fused multi-step calls that overflow (S*K > H) under the other two
    admission priorities, with an extra-row ring of 16 rows: the newest
    tokens resolve to ring rows and never reach the copy list."""
    B, R, H, K, N, I, S = 16, 18, 700, 256, 3000, 32, 4
    rng = np.random.default_rng([16, len(admission)])
    p = Pair(R=R, L=1, H=H, K=K, N=N, I=I, S=S, policy="clock", seed=17,
             admission=admission, extra_rows=16)
    try:
        prev = None
        for call in range(5):
            req = rng.permutation(R)[:B]
            base = make_rows(rng, B, K, N, prev=prev, reuse=0.3)
            base[:, :4] = N - 1 - rng.integers(0, 16, (B, 4))   # ring tokens
            prev = base
            steps = [base] + [make_rows(rng, B, K, N, prev=np.where(base >= 0, base, -1),
                                        reuse=0.0) for _ in range(1, S)]
            p.call(0, req, np.full(B, N), np.stack(steps, axis=1))
    finally:
        p.close()


def test_threshold_and_deferred_interleave():
    """One state, batches of 15 (separate copy kernel) and 16 (fused) and
    deferred calls (separate copy replayed on another stream) in turn."""
    rng = np.random.default_rng(1516)
    R, L, H, K, N, I = 40, 2, 700, 256, 3000, 48
    p = Pair(R=R, L=L, H=H, K=K, N=N, I=I, seed=1516)
    last = np.full((L, R, K), -1, np.int64)   # each request's last row per layer
    try:
        for call, (B, defer) in enumerate([(15, False), (16, False), (40, False), (16, True),
                                           (15, False), (32, True), (17, False), (40, False)]):
            layer = call % L
            req = rng.permutation(R)[:B]
            rows = make_rows(rng, B, K, N, prev=last[layer, req], reuse=0.6, dup=0.03, pad=0.02)
            last[layer, req] = rows
            p.call(layer, req, np.full(B, N), rows, defer=defer)
        log("threshold / deferred interleave: every call equal to the oracle")
    finally:
        p.close()


def test_profile_counts_fused_calls():
    """The profile counts the calls that copied inside the lookup kernel:
    16-row token calls do, 4-row calls and deferred calls do not."""
    rng = np.random.default_rng(16)
    R, H, K, N, I = 20, 500, 128, 2000, 32
    p = Pair(R=R, L=1, H=H, K=K, N=N, I=I, seed=16)
    try:
        p.gpu.profile(True)
        p.gpu.profile_read()
        for B, defer in [(16, False), (4, False), (16, True), (20, False)]:
            req = rng.permutation(R)[:B]
            p.call(0, req, np.full(B, N), make_rows(rng, B, K, N), defer=defer)
        prof = p.gpu.profile_read()
        p.gpu.profile(False)
        log(f"profile {prof}")
        assert prof["calls"] == 4 and prof["fused_calls"] == 2
        assert prof["plan_ms"] > 0 and prof["copy_ms"] > 0
    finally:
        p.close()


FUSED_LARGE = [
    # (policy, H, K, N, S): 16 and 32 slots per thread, copies inside the plan kernel
    ("lru", 12000, 2048, 40000, 1),
    ("lru", 32768, 3000, 65536, 1),     # 8 entries per thread
    ("clock", 16384, 1024, 50000, 2),
    ("clock", 32768, 2048, 65536, 4),   # 8 entries per thread, overflow on the first call
]


@pytest.mark.parametrize("policy,H,K,N,S", FUSED_LARGE)
def test_fused_large_hot_buffers(policy, H, K, N, S):
    B = R = FUSE_MIN_ROWS
    log(f"fused large {policy} H={H} K={K} N={N} S={S} B={B}")
    rng = np.random.default_rng([H, K, S, 16])
    p = Pair(R=R, L=1, H=H, K=K, N=N, I=16, S=S, policy=policy, seed=H + 16)
    prev = None
    try:
        for call in range(4):
            req = rng.permutation(R)[:B]
            base = make_rows(rng, B, K, N, prev=prev, reuse=0.5)
            prev = base
            rows = base if S == 1 else np.stack(
                [base] + [make_rows(rng, B, K, N, prev=np.where(base >= 0, base, -1), reuse=0.3)
                          for _ in range(1, S)], axis=1)
            p.call(0, req, np.full(B, N), rows)
    finally:
        p.close()


def test_fused_lru_with_extra_row_ring():
    """Fused single-step LRU calls with a 32-row ring of the newest tokens:
    ring tokens resolve to ring rows, the rest are looked up and copied."""
    B, R, H, K, N, I = 20, 24, 600, 300, 4000, 48
    rng = np.random.default_rng(2032)
    p = Pair(R=R, L=2, H=H, K=K, N=N, I=I, seed=2032, extra_rows=32)
    try:
        prev = {}
        for call in range(6):
            layer = call % 2
            req = rng.permutation(R)[:B]
            rows = make_rows(rng, B, K, N, prev=prev.get(layer), reuse=0.5)
            rows[:, :6] = N - 1 - rng.integers(0, 40, (B, 6))   # in and just below the ring
            prev[layer] = rows
            p.call(layer, req, np.full(B, N), rows)
    finally:
        p.close()


def test_fused_clock_with_fewer_steps_than_max():
    """A state made for 4 steps called with 2, 3 and 4 steps by fused calls."""
    rng = np.random.default_rng(234)
    B, R, H, K, N = 18, 20, 900, 200, 3000
    p = Pair(R=R, L=1, H=H, K=K, N=N, I=16, S=4, policy="clock", seed=234)
    try:
        for call in range(6):
            S = 2 + call % 3
            req = rng.permutation(R)[:B]
            topk = rng.integers(-1, N, (B, S, K))
            p.call(0, req, np.full(B, N), topk)
    finally:
        p.close()
