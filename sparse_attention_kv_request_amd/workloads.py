"""Seeded synthetic inputs for the HiSparse swap-in path.

This module only *draws inputs*: per-request top-k index traces and the host KV
bytes behind them.  It holds none of the swap-in arithmetic (no lookup, no
dedup, no eviction), so both the CPU oracle and the HIP path may consume what it
produces.

Every array is a pure function of ``(config id, request, layer)`` through
``numpy.random.SeedSequence([2026, cfg, r, l])`` for indices and
``[2026, cfg, r, l, 1]`` for KV bytes, so any single cache instance can be
regenerated on its own (the parity tests sample instances this way).

The five workloads exercise the shapes the pages describe: per-layer token
top-k chosen by a DSA indexer each decode step (sglang PR #20343 summary,
"Implementation breakdown"), multi-step MTP calls of 2-4 steps (PR #32162
report, "Implementation breakdown" item 2), and page-granular loads with
256-token pages and a top-k of 512 ("SGLang HiSparse" blog, sections 2.1 and
4.1).  The indexer needs trained weights, so its output is replaced by the
synthetic recipes below; the recipes (reuse fractions, recency bias, cluster
widths) are choices of this module, not numbers from the pages.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED_ROOT = 2026


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one synthetic workload.

    ``num_steps`` is the MTP step count S of a call (1 = single-step).
    ``steps`` is the number of calls made per (request, layer) instance.
    ``page_size`` is P (1 = token mode); ``hot`` counts slots, or pages when P > 1.
    """

    cfg_id: int
    name: str
    batch: int
    layers: int
    steps: int
    num_steps: int
    top_k: int
    seq_len: int
    hot: int
    item_bytes: int
    page_size: int = 1
    policy: str = "lru"           # "lru" (single-step) or "clock" (multi-step)
    kv_kind: str = "random"       # "random" bytes or "bf16_normal" latent+rope
    # recipe knobs (fractions of top_k unless stated)
    window: int = 0               # cfg 1: always-selected most recent tokens
    reuse: float = 0.0            # step-to-step (or call-to-call) reuse fraction
    zipf_s: float = 0.0           # cfg 2: recency bias exponent
    core_frac: float = 0.0        # cfg 3: share of a call's steps
    clusters: int = 0             # cfg 5
    sigma: float = 0.0            # cfg 5
    persist: float = 0.0          # cfg 5: fraction of cluster centres kept
    max_requests: int = 0         # request pool size; 0 means == batch

    @property
    def requests(self) -> int:
        return self.max_requests or self.batch

    @property
    def entries_per_step(self) -> int:
        """Resolved top-k entries per decode step over all rows and layers."""
        return self.batch * self.layers * self.num_steps * self.top_k

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads at full size.
CONFIGS = {
    1: Workload(1, "single-step LRU, B=1, bf16 1152-B items", batch=1, layers=1,
                steps=16, num_steps=1, top_k=2048, seq_len=8192, hot=4096,
                item_bytes=1152, kv_kind="bf16_normal", window=128, reuse=0.5),
    2: Workload(2, "single-step LRU, B=64 x 8 layers, fp8 656-B items", batch=64,
                layers=8, steps=32, num_steps=1, top_k=2048, seq_len=32768,
                hot=4096, item_bytes=656, reuse=0.7, zipf_s=1.1),
    3: Workload(3, "multi-step CLOCK, B=64, S=4", batch=64, layers=1, steps=32,
                num_steps=4, top_k=2048, seq_len=32768, hot=4096, item_bytes=656,
                policy="clock", reuse=0.6, core_frac=0.8),
    4: Workload(4, "miss-heavy long context, B=128", batch=128, layers=1,
                steps=16, num_steps=1, top_k=2048, seq_len=131072, hot=8192,
                item_bytes=656, reuse=0.3),
    5: Workload(5, "page mode, B=32, P=256, 64 hot pages", batch=32, layers=1,
                steps=32, num_steps=1, top_k=512, seq_len=65536, hot=64,
                item_bytes=656, page_size=256, clusters=8, sigma=300.0,
                persist=0.6),
}


def config(cfg_id: int, **overrides) -> Workload:
    """Return workload ``cfg_id``, optionally resized (``overrides``)."""
    w = CONFIGS[cfg_id]
    return w.replace(**overrides) if overrides else w


def _rng(cfg_id: int, r: int, l: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([SEED_ROOT, cfg_id, r, l, *extra])))


def _uniform_excluding(rng, n, count, excluded_mask):
    """``count`` distinct values uniform over ``[0, n)`` minus ``excluded_mask``."""
    pool = np.flatnonzero(~excluded_mask)
    if count > pool.size:
        raise ValueError("not enough candidates")
    return rng.choice(pool, size=count, replace=False)


def _weighted_excluding(rng, cdf, count, excluded_mask):
    """``count`` distinct draws by successive weighted sampling without replacement.

    Draws with replacement from the categorical distribution given by ``cdf``
    and keeps first-seen values not yet excluded, which is sequential sampling
    without replacement.
    """
    n = cdf.size
    taken = excluded_mask.copy()
    out = []
    need = count
    while need > 0:
        u = rng.random(2 * need + 16) * cdf[-1]
        cand = np.minimum(np.searchsorted(cdf, u, side="right"), n - 1)
        _, first = np.unique(cand, return_index=True)
        cand = cand[np.sort(first)]
        cand = cand[~taken[cand]][:need]
        taken[cand] = True
        out.append(cand)
        need -= cand.size
    return np.concatenate(out)


def _trace_window_reuse(w: Workload, rng) -> np.ndarray:
    """Config 1 recipe: the newest ``window`` tokens every step; of the rest,
    ``reuse`` carried over from the previous step, the others uniform."""
    n, k = w.seq_len, w.top_k
    win = np.arange(n - w.window, n)
    rest_n = k - w.window
    keep_n = int(round(w.reuse * rest_n))
    out = np.empty((w.steps, 1, k), np.int32)
    prev_rest = None
    for t in range(w.steps):
        mask = np.zeros(n, bool)
        mask[win] = True
        if prev_rest is None:
            rest = _uniform_excluding(rng, n, rest_n, mask)
        else:
            kept = rng.choice(prev_rest, size=keep_n, replace=False)
            mask[kept] = True
            fresh = _uniform_excluding(rng, n, rest_n - keep_n, mask)
            rest = np.concatenate([kept, fresh])
        prev_rest = rest
        out[t, 0] = rng.permutation(np.concatenate([win, rest]))
    return out


def _trace_zipf_reuse(w: Workload, rng) -> np.ndarray:
    """Config 2 recipe: weight (N - p)^-s favours recent positions; ``reuse`` of
    the previous step's set is kept, the rest drawn by weight."""
    n, k = w.seq_len, w.top_k
    weight = (n - np.arange(n, dtype=np.float64)) ** (-w.zipf_s)
    cdf = np.cumsum(weight)
    keep_n = int(round(w.reuse * k))
    out = np.empty((w.steps, 1, k), np.int32)
    prev = None
    for t in range(w.steps):
        mask = np.zeros(n, bool)
        if prev is None:
            sel = _weighted_excluding(rng, cdf, k, mask)
        else:
            kept = rng.choice(prev, size=keep_n, replace=False)
            mask[kept] = True
            sel = np.concatenate([kept, _weighted_excluding(rng, cdf, k - keep_n, mask)])
        prev = sel
        out[t, 0] = rng.permutation(sel)
    return out


def _trace_uniform_reuse(w: Workload, rng) -> np.ndarray:
    """Config 4 recipe: ``reuse`` of the previous set kept, the rest uniform."""
    n, k = w.seq_len, w.top_k
    keep_n = int(round(w.reuse * k))
    out = np.empty((w.steps, 1, k), np.int32)
    prev = None
    for t in range(w.steps):
        mask = np.zeros(n, bool)
        if prev is None:
            sel = _uniform_excluding(rng, n, k, mask)
        else:
            kept = rng.choice(prev, size=keep_n, replace=False)
            mask[kept] = True
            sel = np.concatenate([kept, _uniform_excluding(rng, n, k - keep_n, mask)])
        prev = sel
        out[t, 0] = rng.permutation(sel)
    return out


def _trace_mtp(w: Workload, rng) -> np.ndarray:
    """Config 3 recipe: per call a core shared by all S steps (``core_frac``
    of top_k) plus per-step extras; ``reuse`` of top_k comes from the previous
    call's union of rows."""
    n, k, s_n = w.seq_len, w.top_k, w.num_steps
    core_n = int(round(w.core_frac * k))
    extra_n = k - core_n
    keep_n = min(int(round(w.reuse * k)), core_n)
    out = np.empty((w.steps, s_n, k), np.int32)
    prev_union = None
    for c in range(w.steps):
        if prev_union is None:
            core = _uniform_excluding(rng, n, core_n, np.zeros(n, bool))
        else:
            kept = rng.choice(prev_union, size=keep_n, replace=False)
            mask = np.zeros(n, bool)
            mask[prev_union] = True
            core = np.concatenate([kept, _uniform_excluding(rng, n, core_n - keep_n, mask)])
        core_mask = np.zeros(n, bool)
        core_mask[core] = True
        union = [core]
        for s in range(s_n):
            extra = _uniform_excluding(rng, n, extra_n, core_mask)
            union.append(extra)
            out[c, s] = rng.permutation(np.concatenate([core, extra]))
        prev_union = np.unique(np.concatenate(union))
    return out


def _trace_clusters(w: Workload, rng) -> np.ndarray:
    """Config 5 recipe: ``clusters`` Gaussian clusters of top_k/clusters tokens
    (sigma tokens, truncated at 2.5 sigma); a fixed count of centres persists
    from step to step, the others are redrawn."""
    n, k = w.seq_len, w.top_k
    per = k // w.clusters
    keep_c = int(round(w.persist * w.clusters))
    trunc = 2.5 * w.sigma
    out = np.empty((w.steps, 1, k), np.int32)
    centres = None
    for t in range(w.steps):
        if centres is None:
            centres = rng.random(w.clusters) * n
        else:
            keep_idx = rng.choice(w.clusters, size=keep_c, replace=False)
            new = centres.copy()
            redraw = np.setdiff1d(np.arange(w.clusters), keep_idx)
            new[redraw] = rng.random(redraw.size) * n
            centres = new
        chosen = np.zeros(n, bool)
        toks = []
        for c in centres:
            got = 0
            while got < per:
                x = np.rint(rng.normal(c, w.sigma, size=4 * per)).astype(np.int64)
                ok = (x >= 0) & (x < n) & (np.abs(x - c) <= trunc)
                for v in x[ok]:
                    if not chosen[v]:
                        chosen[v] = True
                        toks.append(v)
                        got += 1
                        if got == per:
                            break
        out[t, 0] = rng.permutation(np.asarray(toks, np.int64))
    return out


_RECIPES = {1: _trace_window_reuse, 2: _trace_zipf_reuse, 3: _trace_mtp,
            4: _trace_uniform_reuse, 5: _trace_clusters}


def instance_trace(w: Workload, r: int, l: int) -> np.ndarray:
    """Top-k token indices of instance (request ``r``, layer ``l``):
    int32 ``[steps, num_steps, top_k]``."""
    return _RECIPES[w.cfg_id](w, _rng(w.cfg_id, r, l))


def batch_trace(w: Workload, threads: int = 8) -> np.ndarray:
    """All instances: int32 ``[layers, steps, batch, num_steps, top_k]``.

    Row b of every call is request b (``req_pool_indices = arange(batch)``).
    """
    out = np.empty((w.layers, w.steps, w.batch, w.num_steps, w.top_k), np.int32)
    jobs = [(r, l) for l in range(w.layers) for r in range(w.batch)]

    def run(job):
        r, l = job
        out[l, :, r] = instance_trace(w, r, l)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, jobs))
    return out


def _bf16_bytes(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (round to nearest even), as little-endian bytes."""
    b = x.astype(np.float32).view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return b.astype(np.uint16).view(np.uint8)


def instance_kv(w: Workload, r: int, l: int, out: np.ndarray | None = None) -> np.ndarray:
    """Host KV bytes of instance (r, l): uint8 ``[seq_len, item_bytes]``.

    ``random`` items are uniform bytes; ``bf16_normal`` items are 576 N(0,1)
    values in bfloat16 (the 512 latent + 64 rope dims of an MLA entry).
    """
    n, i_b = w.seq_len, w.item_bytes
    if out is None:
        out = np.empty((n, i_b), np.uint8)
    if w.kv_kind == "bf16_normal":
        rng = _rng(w.cfg_id, r, l, 1)
        vals = rng.standard_normal(n * (i_b // 2), dtype=np.float32)
        out.reshape(-1)[:] = _bf16_bytes(vals)
    else:
        bg = np.random.PCG64(np.random.SeedSequence([SEED_ROOT, w.cfg_id, r, l, 1]))
        words = bg.random_raw((n * i_b + 7) // 8).view(np.uint8)
        out.reshape(-1)[:] = words[: n * i_b]
    return out


def fill_host_kv(w: Workload, layer_arrays, threads: int = 16) -> None:
    """Fill per-layer host KV arrays (uint8 ``[requests, seq_len, item_bytes]``)
    for every request and layer of ``w``, in parallel threads."""
    jobs = [(r, l) for l in range(w.layers) for r in range(w.requests)]

    def run(job):
        r, l = job
        instance_kv(w, r, l, out=layer_arrays[l][r])

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, jobs))


# -- inputs of the decode-attention consumer -----------------------------------

MLA_LATENT, MLA_ROPE = 512, 64


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    b = x.astype(np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
            >> np.uint32(16)).astype(np.uint16)


def mla_kv_rows(rng: np.random.Generator, n: int, item_bytes: int) -> np.ndarray:
    """``n`` MLA KV rows with N(0,1) latent and rope values, as stored bytes.

    1152 B: 576 bfloat16.  656 B: 512 fp8 e4m3fn latent values quantised per
    128-dim tile with scale = max|x| / 448 (float32), the 4 scales, then 64
    bfloat16 rope values.
    """
    lat = rng.standard_normal((n, MLA_LATENT)).astype(np.float32)
    rope = rng.standard_normal((n, MLA_ROPE)).astype(np.float32)
    if item_bytes == 2 * (MLA_LATENT + MLA_ROPE):
        return _to_bf16_bits(np.concatenate([lat, rope], 1)).view(np.uint8).reshape(n, -1)
    if item_bytes == MLA_LATENT + 16 + 2 * MLA_ROPE:
        import torch

        tiles = lat.reshape(n, 4, 128)
        scale = (np.abs(tiles).max(axis=2) / np.float32(448.0)).astype(np.float32)
        scale = np.where(scale > 0, scale, np.float32(1.0))
        q = torch.from_numpy(tiles / scale[:, :, None]).to(torch.float8_e4m3fn)
        codes = q.view(torch.uint8).numpy().reshape(n, MLA_LATENT)
        out = np.empty((n, item_bytes), np.uint8)
        out[:, :MLA_LATENT] = codes
        out[:, MLA_LATENT:MLA_LATENT + 16] = scale.view(np.uint8).reshape(n, 16)
        out[:, MLA_LATENT + 16:] = _to_bf16_bits(rope).view(np.uint8).reshape(n, -1)
        return out
    raise ValueError(item_bytes)


def mla_queries(rng: np.random.Generator, batch: int, heads: int) -> np.ndarray:
    """bfloat16 bits [batch, heads, 576] of N(0,1) queries."""
    return _to_bf16_bits(rng.standard_normal((batch, heads, MLA_LATENT + MLA_ROPE)))


def indexer_logits(rng: np.random.Generator, batch: int, n: int) -> np.ndarray:
    """float32 [batch, n] stand-ins for indexer scores with the structure the
    index recipes above encode: N(0, 1) noise, the newest 128 positions
    raised by 4, and 8 Gaussian bumps (height 2.5, width 300 positions) at
    random centres, so that a top-2048 mixes recency, clusters and noise."""
    out = rng.standard_normal((batch, n)).astype(np.float32)
    pos = np.arange(n, dtype=np.float32)
    for b in range(batch):
        out[b, max(0, n - 128):] += np.float32(4.0)
        for c in rng.integers(0, n, size=8):
            lo, hi = max(0, c - 900), min(n, c + 900)
            out[b, lo:hi] += (2.5 * np.exp(-0.5 * ((pos[lo:hi] - c) / 300.0) ** 2)).astype(np.float32)
    return out
