"""Admission priority under multi-step overflow and the extra-row ring
(HIP path through the C ABI) against the CPU oracle, element by element:
outputs, miss plans, error word, the whole device KV buffer (the ring rows
must stay untouched) and the touched instances' state."""
import numpy as np
import pytest

from tests.gpu_harness import Pair, log
from tests.test_gpu_parity import make_rows

pytestmark = pytest.mark.gpu


def decode_rows(rng, K, seq, E, prev=None, reuse=0.5, pad=0.02, dup=0.03):
    """One top-k row per request over [0, seq_b): a share of the newest
    tokens (the ring window and just before it), some tokens of the previous
    call, the rest uniform; plus padding and in-row duplicates."""
    B = len(seq)
    rows = np.full((B, K), -1, np.int64)
    for b, sl in enumerate(int(x) for x in seq):
        pool = set()
        tail = np.arange(max(0, sl - E - 8), sl)
        pool.update(rng.choice(tail, min(tail.size, K // 4), replace=False).tolist())
        if prev is not None:
            old = prev[b][(prev[b] >= 0) & (prev[b] < sl)]
            take = min(old.size, int(reuse * K), K - len(pool))
            pool.update(rng.choice(old, take, replace=False).tolist())
        while len(pool) < min(K, sl):
            pool.update(rng.integers(0, sl, K - len(pool)).tolist())
        picked = rng.permutation(np.array(sorted(pool), np.int64))[:K]
        rows[b, :picked.size] = picked
    u = rng.random((B, K))
    src = rng.integers(0, K, (B, K))
    rows = np.where(u < dup, np.take_along_axis(rows, src, 1), rows)
    rows = np.where((u >= dup) & (u < dup + pad), -1, rows)
    return rows.astype(np.int32)


ADMISSION_SHAPES = [
    # (H, K, N, I, S): every call overflows the hot cache
    (50, 100, 400, 16, 3),
    (1000, 700, 5000, 32, 4),
    (2048, 2048, 32768, 656, 4),
]


@pytest.mark.parametrize("admission", ["frequent", "first"])
@pytest.mark.parametrize("H,K,N,I,S", ADMISSION_SHAPES)
def test_clock_admission_variants(admission, H, K, N, I, S):
    log(f"clock admission={admission} H={H} K={K} N={N} I={I} S={S}")
    rng = np.random.default_rng(H + K + S)
    R, L, B = 4, 2, 3
    p = Pair(R=R, L=L, H=H, K=K, N=N, I=I, S=S, policy="clock", seed=K, admission=admission)
    prev = {}
    try:
        for call in range(8):
            layer = call % L
            req = rng.permutation(R)[:B]
            base = make_rows(rng, B, K, N, prev=prev.get(layer), reuse=0.3)
            prev[layer] = base
            steps = [base] + [make_rows(rng, B, K, N, prev=base, reuse=0.5 + 0.1 * s)
                              for s in range(1, S)]
            p.call(layer, req, np.full(B, N), np.stack(steps, axis=1))
    finally:
        p.close()


LRU_EXTRA = [
    # (H, K, N, I, E)
    (300, 200, 2000, 32, 64),
    (3000, 1500, 6000, 48, 1),
    (4096, 2048, 8192, 656, 512),
    (100, 37, 300, 16, 300),          # E = N: every valid token lives in the ring
]


@pytest.mark.parametrize("H,K,N,I,E", LRU_EXTRA)
def test_lru_extra_ring(H, K, N, I, E):
    log(f"lru extra ring H={H} K={K} N={N} I={I} E={E}")
    rng = np.random.default_rng(H + E)
    R, L, B = 4, 2, 3
    p = Pair(R=R, L=L, H=H, K=K, N=N, I=I, seed=E, extra_rows=E)
    assert p.rows == H + E
    seq = rng.integers(max(K, N // 2), N - 20, R)
    prev = {}
    try:
        for call in range(10):
            layer = call % L
            req = rng.permutation(R)[:B]
            seq[req] += rng.integers(0, 3, B)          # decoding moves the window
            rows = decode_rows(rng, K, seq[req], E, prev=prev.get((layer, tuple(req))))
            prev[(layer, tuple(req))] = rows
            p.call(layer, req, seq[req], rows)
    finally:
        p.close()


@pytest.mark.parametrize("admission", ["recent", "frequent", "first"])
def test_clock_extra_ring_after_scratch(admission):
    """Multi-step CLOCK with scratch rows: the ring sits after them."""
    H, K, N, I, S, E = 200, 150, 3000, 32, 3, 40
    log(f"clock extra ring admission={admission}")
    rng = np.random.default_rng(7)
    R, B = 3, 2
    p = Pair(R=R, L=1, H=H, K=K, N=N, I=I, S=S, policy="clock", seed=3,
             admission=admission, extra_rows=E)
    assert p.rows == H + (S * K - H) + E
    seq = rng.integers(N // 2, N - 20, R)
    try:
        for call in range(8):
            req = rng.permutation(R)[:B]
            seq[req] += 1
            base = decode_rows(rng, K, seq[req], E)
            steps = [base] + [decode_rows(rng, K, seq[req], E, prev=base, reuse=0.6)
                              for _ in range(1, S)]
            p.call(0, req, seq[req], np.stack(steps, axis=1))
    finally:
        p.close()
