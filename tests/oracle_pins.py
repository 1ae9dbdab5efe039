"""Pins that tie the CPU oracle to something other than itself.

Every check takes the oracle *module* as its first argument, so the same
battery runs against the real oracle (tests/test_oracle_pins.py) and against
copies with a planted mistake (tests/test_oracle_mutants.py), where at least
one check must fail.

What the checks compare against:

* textbook LRU (an ``OrderedDict``) and textbook second-chance CLOCK (a frame
  array with a hand) on one-key calls;
* closed forms: the first call from an empty cache, a repeated call, and a
  hot cache at least as large as the key universe (never evicts);
* independently written formulations on exhaustive / random tiny traces: a
  recency-ordered slot list for LRU and a two-lap (prefix) formulation of the
  CLOCK sweep, compared after every call on outputs, plan and full state;
* the invariants of every call (``check_call`` / ``check_instance``) with the
  shadow device buffer, i.e. every returned row holds the key's host bytes;
* page-mode translation closed forms (pages = distinct ``t div P`` ascending,
  token row = page row * P + ``t mod P``);
* the row-level error semantics (padding, bad index, duplicate request).
"""
from __future__ import annotations

import collections
import itertools

import numpy as np

EMPTY = -1


# --------------------------------------------------------------------------
# Independent formulations
# --------------------------------------------------------------------------

class TextbookLRU:
    """Plain LRU over keys with capacity H (no slots)."""

    def __init__(self, cap):
        self.cap = cap
        self.d = collections.OrderedDict()

    def access(self, key):
        """Returns (hit, evicted key or None)."""
        if key in self.d:
            self.d.move_to_end(key)
            return True, None
        ev = None
        if len(self.d) == self.cap:
            ev, _ = self.d.popitem(last=False)
        self.d[key] = True
        return False, ev


class TextbookClock:
    """Second-chance CLOCK over H frames; reference bit set on load and on hit."""

    def __init__(self, frames):
        self.key = [EMPTY] * frames
        self.ref = [0] * frames
        self.hand = 0

    def access(self, k):
        """Returns (hit, frame, evicted key)."""
        if k in self.key:
            f = self.key.index(k)
            self.ref[f] = 1
            return True, f, EMPTY
        while True:
            f = self.hand
            self.hand = (self.hand + 1) % len(self.key)
            if self.ref[f]:
                self.ref[f] = 0
                continue
            ev = self.key[f]
            self.key[f] = k
            self.ref[f] = 1
            return False, f, ev


class RecencyListLRU:
    """LRU kept as an explicit slot order (least recent first).

    Slots touched by a call move to the back in ascending slot order, which is
    the (timestamp, slot) order without storing timestamps.
    """

    def __init__(self, hot):
        self.order = list(range(hot))
        self.slot_key = [EMPTY] * hot
        self.where = {}

    def call(self, ws):
        hit_slots = {self.where[k] for k in ws if k in self.where}
        misses = [k for k in ws if k not in self.where]
        free = [s for s in self.order if s not in hit_slots]
        victims = free[: len(misses)]
        placed = []
        for k, s in zip(misses, victims):
            old = self.slot_key[s]
            if old != EMPTY:
                del self.where[old]
            self.slot_key[s] = k
            self.where[k] = s
            placed.append((k, s, old))
        touched = hit_slots | set(victims)
        self.order = [s for s in self.order if s not in touched] + sorted(touched)
        return placed


class TwoLapClock:
    """CLOCK sweep as two prefix selections over the circular slot order."""

    def __init__(self, hot):
        self.hot = hot
        self.slot_key = [EMPTY] * hot
        self.where = {}
        self.ref = [0] * hot
        self.hand = 0

    def call(self, ws, priority):
        """`priority[key]`: higher is admitted first under overflow (stable)."""
        hot = self.hot
        pinned = {self.where[k] for k in ws if k in self.where}
        for p in pinned:
            self.ref[p] = 1
        misses = [k for k in ws if k not in self.where]
        room = hot - len(pinned)
        by_priority = sorted(misses, key=lambda k: -priority[k])   # stable
        admit_set = set(by_priority[:room])
        admitted = [k for k in misses if k in admit_set]
        overflow = [k for k in misses if k not in admit_set]
        circ = [(self.hand + d) % hot for d in range(hot)]
        unpinned = [s for s in circ if s not in pinned]
        lap1 = [s for s in unpinned if self.ref[s] == 0]
        need = len(admitted)
        if need == 0:
            victims = []
        elif len(lap1) >= need:
            victims = lap1[:need]
            stop = (victims[-1] - self.hand) % hot
            for s in unpinned:
                if self.ref[s] and (s - self.hand) % hot < stop:
                    self.ref[s] = 0
        else:
            lap2 = [s for s in unpinned if self.ref[s] == 1]
            victims = lap1 + lap2[: need - len(lap1)]
            for s in unpinned:
                self.ref[s] = 0
        if victims:
            self.hand = (victims[-1] + 1) % hot
        placed = []
        for k, s in zip(admitted, victims):
            old = self.slot_key[s]
            if old != EMPTY:
                del self.where[old]
            self.slot_key[s] = k
            self.where[k] = s
            self.ref[s] = 1
            placed.append((k, s, old))
        return placed, overflow


# --------------------------------------------------------------------------
# Helpers
# --------------------------------------------------------------------------

def make_state(ora, *, R=1, L=1, H, K, N, S=1, P=1, I=16, policy="lru", seed=0,
               admission="recent", E=0):
    """Oracle state with a shadow device buffer and random host bytes."""
    rng = np.random.default_rng(seed)
    host = [rng.integers(0, 256, (R, N, I), dtype=np.uint8) for _ in range(L)]
    return ora.OracleState(max_requests=R, num_layers=L, hot=H, top_k=K, item_bytes=I,
                           max_seq_len=N, max_steps=S, page_size=P, policy=policy,
                           host_kv=host, admission=admission, extra_rows=E)


def resident(st, req, layer):
    return [set(st.instance(int(r), layer).key_slot) for r in req]


def checked_call(ora, st, layer, req, seq, topk, multi=False):
    before = resident(st, req, layer)
    if multi:
        res = st.swap_in_spec_multistep(layer, req, seq, topk)
    else:
        res = st.swap_in_selected(layer, req, seq, topk)
    ora.check_call(st, layer, req, seq, topk, res, before)
    for r in set(int(x) for x in req):
        ora.check_instance(st.instance(r, layer), st.policy)
    return res


# --------------------------------------------------------------------------
# Pins
# --------------------------------------------------------------------------

def pin_lru_textbook_k1(ora, seed=1, calls=400, N=12, H=5):
    """K = 1: hit/miss and eviction sequence equal a textbook LRU."""
    rng = np.random.default_rng(seed)
    st = make_state(ora, H=H, K=1, N=N)
    tb = TextbookLRU(H)
    key_of_row = {}
    for _ in range(calls):
        t = int(rng.integers(0, N))
        hit, ev = tb.access(t)
        res = checked_call(ora, st, 0, [0], [N], [[t]])
        assert res["miss_count"][0] == (0 if hit else 1)
        if not hit:
            (src, dst, victim), = res["plan"][0]
            assert src == t
            assert victim == (EMPTY if ev is None else ev)
            if ev is not None:
                assert key_of_row[dst] == ev
            key_of_row[dst] = t
        assert key_of_row[int(res["out_locs"][0, 0])] == t


def pin_clock_textbook_k1(ora, seed=2, calls=400, N=12, H=5):
    """K = 1 with the key repeated in both steps: slots, hits and evictions
    equal a textbook second-chance CLOCK."""
    rng = np.random.default_rng(seed)
    st = make_state(ora, H=H, K=1, N=N, S=2, policy="clock")
    tb = TextbookClock(H)
    for _ in range(calls):
        t = int(rng.integers(0, N))
        hit, frame, ev = tb.access(t)
        res = checked_call(ora, st, 0, [0], [N], [[[t], [t]]], multi=True)
        rows = st.rows
        assert res["miss_count"][0] == (0 if hit else 1)
        assert res["out_locs"][0, 0, 0] == frame and res["out_locs"][0, 1, 0] == frame
        if not hit:
            assert res["plan"][0] == [(t, frame, ev)]
        inst = st.instance(0, 0)
        assert inst.ref == tb.ref and inst.hand == tb.hand and inst.slot_key == tb.key
        assert rows == H


def pin_first_call_closed_form(ora, seed=3):
    """From empty: misses take slots 0..|W|-1 in first-occurrence order (LRU)
    or in hand order from 0 (CLOCK, hand ends at |W| mod H); no victims."""
    rng = np.random.default_rng(seed)
    N, H, K = 50, 40, 30
    keys = rng.integers(-1, N, K)
    ws = []
    for t in keys:
        if t >= 0 and t not in ws:
            ws.append(int(t))
    st = make_state(ora, H=H, K=K, N=N)
    res = checked_call(ora, st, 0, [0], [N], [keys])
    assert res["miss_count"][0] == len(ws)
    assert res["plan"][0] == [(t, j, EMPTY) for j, t in enumerate(ws)]
    for i, t in enumerate(keys):
        assert res["out_locs"][0, i] == (ws.index(t) if t >= 0 else -1)
    inst = st.instance(0, 0)
    assert inst.ts == [0] * len(ws) + [-1] * (H - len(ws)) and inst.now == 1

    S = 2
    st = make_state(ora, H=H, K=K, N=N, S=S, policy="clock")
    rows = np.stack([keys, rng.permutation(keys)])
    ws2 = []
    for t in rows.reshape(-1):
        if t >= 0 and t not in ws2:
            ws2.append(int(t))
    res = checked_call(ora, st, 0, [0], [N], rows[None], multi=True)
    sx = max(0, S * K - H)
    assert res["plan"][0] == [(t, j, EMPTY) for j, t in enumerate(ws2)]
    inst = st.instance(0, 0)
    assert inst.hand == len(ws2) % H
    assert inst.ref == [1] * len(ws2) + [0] * (H - len(ws2))
    assert st.rows == H + sx


def pin_repeat_and_large_cache(ora, seed=4):
    """A repeated call misses nothing and returns the same rows; with H >= N
    nothing is ever evicted and each key's slot is its global first-seen
    rank (LRU and CLOCK alike)."""
    rng = np.random.default_rng(seed)
    N, K = 30, 8
    for policy, S in (("lru", 1), ("clock", 3)):
        st = make_state(ora, H=N, K=K, N=N, S=S, policy=policy)
        first_seen = []
        for _ in range(25):
            if S == 1:
                topk = rng.integers(-1, N, (1, K))
                flat = topk.reshape(-1)
            else:
                topk = rng.integers(-1, N, (1, S, K))
                flat = topk.reshape(-1)
            new = []
            for t in flat:
                if t >= 0 and t not in first_seen and t not in new:
                    new.append(int(t))
            res = checked_call(ora, st, 0, [0], [N], topk, multi=S > 1)
            assert res["miss_count"][0] == len(new)
            first_seen += new
            for x, t in zip(res["out_locs"].reshape(-1), flat):
                assert x == (first_seen.index(t) if t >= 0 else -1)
            assert all(v == EMPTY for _, _, v in res["plan"][0])
            again = checked_call(ora, st, 0, [0], [N], topk, multi=S > 1)
            assert again["miss_count"][0] == 0
            assert np.array_equal(again["out_locs"], res["out_locs"])


def _lru_compare_trace(ora, H, N, trace):
    st = make_state(ora, H=H, K=len(trace[0]), N=N)
    ref = RecencyListLRU(H)
    for keys in trace:
        res = checked_call(ora, st, 0, [0], [N], [list(keys)])
        ws = []
        for t in keys:
            if t >= 0 and t not in ws:
                ws.append(t)
        exp = ref.call(ws)
        assert res["plan"][0] == exp
        for x, t in zip(res["out_locs"][0], keys):
            assert x == (ref.where[t] if t >= 0 else -1)
        inst = st.instance(0, 0)
        assert inst.slot_key == ref.slot_key
        assert sorted(range(H), key=lambda s: (inst.ts[s], s)) == ref.order


def pin_lru_bruteforce(ora):
    """Exhaustive tiny traces against the recency-list LRU (N <= 4, H <= 3,
    K <= 2, up to four calls), checking every invariant after every call."""
    for H, K, N, length in ((1, 1, 4, 4), (2, 1, 4, 4), (2, 2, 3, 3), (3, 2, 4, 2)):
        rows = list(itertools.product(range(-1, N), repeat=K))
        for trace in itertools.product(rows, repeat=length):
            _lru_compare_trace(ora, H, N, trace)


def pin_lru_random(ora, seed=5, trials=60):
    """Random longer traces against the recency-list LRU."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        H = int(rng.integers(1, 9))
        K = int(rng.integers(1, H + 1))
        N = int(rng.integers(K, 20))
        trace = [list(rng.integers(-1, N, K)) for _ in range(12)]
        _lru_compare_trace(ora, H, N, [[int(x) for x in row] for row in trace])


def _clock_compare_trace(ora, H, N, S, K, trace, import_state=None, admission="recent"):
    st = make_state(ora, H=H, K=K, N=N, S=S, policy="clock", admission=admission)
    ref = TwoLapClock(H)
    if import_state is not None:
        slot_key, refbits, hand = import_state
        st.import_(0, 0, slot_key, ref=refbits, hand=hand)
        ref.slot_key = list(slot_key)
        ref.where = {k: s for s, k in enumerate(slot_key) if k != EMPTY}
        ref.ref = list(refbits)
        ref.hand = hand
    for call in trace:
        topk = np.asarray(call).reshape(1, S, K)
        res = checked_call(ora, st, 0, [0], [N], topk, multi=True)
        ws, last, count = [], {}, {}
        for pos, t in enumerate(topk.reshape(-1)):
            t = int(t)
            if t < 0:
                continue
            if t not in ws:
                ws.append(t)
            if last.get(t) != pos // K:        # a step counts once however often it names t
                count[t] = count.get(t, 0) + 1
            last[t] = pos // K
        priority = {"recent": last, "frequent": count, "first": {t: 0 for t in ws}}[admission]
        placed, overflow = ref.call(ws, priority)
        rows = st.rows
        exp_plan = [(k, s, v) for k, s, v in placed] + \
                   [(k, H + j, EMPTY) for j, k in enumerate(overflow)]
        assert res["plan"][0] == exp_plan
        inst = st.instance(0, 0)
        assert inst.slot_key == ref.slot_key
        assert inst.ref == ref.ref and inst.hand == ref.hand
        scratch = {k: H + j for j, k in enumerate(overflow)}
        for x, t in zip(res["out_locs"].reshape(-1), topk.reshape(-1)):
            t = int(t)
            if t < 0:
                assert x == -1
            else:
                assert x == (ref.where[t] if t in ref.where else scratch[t])
        assert rows == H + max(0, S * K - H)


def pin_clock_bruteforce(ora):
    """Exhaustive tiny multi-step traces against the two-lap CLOCK."""
    N, S, K = 3, 2, 1
    rows = list(itertools.product(range(-1, N), repeat=S * K))
    for H in (1, 2):
        for trace in itertools.product(rows, repeat=3):
            _clock_compare_trace(ora, H, N, S, K, trace)


def pin_clock_random(ora, seed=6, trials=80):
    """Random traces (including overflow and imported states with arbitrary
    reference bits and hand) against the two-lap CLOCK."""
    rng = np.random.default_rng(seed)
    for trial in range(trials):
        H = int(rng.integers(1, 9))
        S = int(rng.integers(2, 5))
        K = int(rng.integers(1, 5))
        N = int(rng.integers(2, 16))
        trace = [rng.integers(-1, N, S * K).tolist() for _ in range(10)]
        imp = None
        if trial % 2:
            keys = rng.permutation(N)[:H]
            slot_key = [int(k) if rng.random() < 0.8 else EMPTY for k in keys]
            slot_key += [EMPTY] * (H - len(slot_key))
            refbits = [int(x) for x in rng.integers(0, 2, H)]
            imp = (slot_key, refbits, int(rng.integers(0, H)))
        _clock_compare_trace(ora, H, N, S, K, trace, imp)


def pin_overflow_closed_form(ora):
    """Reading R7 closed form: H = 4 empty slots, three steps with four
    distinct misses each and no key shared between steps; the four misses of
    the last step are admitted into slots 0..3 and the eight others go to
    scratch rows 4..11 in first-occurrence order."""
    H, S, K, N = 4, 3, 4, 40
    st = make_state(ora, H=H, K=K, N=N, S=S, policy="clock")
    topk = np.arange(12).reshape(1, S, K)
    res = checked_call(ora, st, 0, [0], [N], topk, multi=True)
    assert res["miss_count"][0] == 12
    assert res["plan"][0][:4] == [(8, 0, EMPTY), (9, 1, EMPTY), (10, 2, EMPTY), (11, 3, EMPTY)]
    assert res["plan"][0][4:] == [(t, 4 + t, EMPTY) for t in range(8)]
    assert res["out_locs"][0].reshape(-1).tolist() == [4, 5, 6, 7, 8, 9, 10, 11, 0, 1, 2, 3]


def pin_admission_variants(ora, seed=11, trials=40):
    """The admission priorities under overflow (R7 and two variants), by a
    closed form: H = 4 empty slots; steps {0,1,2,3}, {4,5,2,3}, {6,7,4,2};
    key 2 is named by three steps, 3 and 4 by two, 4 and 6, 7 last by step 2.
    Then random overflowing traces against the two-lap CLOCK with the same
    priority computed independently."""
    H, S, K, N = 4, 3, 4, 40
    topk = np.array([[0, 1, 2, 3], [4, 5, 2, 3], [6, 7, 4, 2]]).reshape(1, S, K)
    expected = {"recent": ([2, 4, 6, 7], [0, 1, 3, 5]),
                "frequent": ([0, 2, 3, 4], [1, 5, 6, 7]),
                "first": ([0, 1, 2, 3], [4, 5, 6, 7])}
    for admission, (admitted, overflow) in expected.items():
        st = make_state(ora, H=H, K=K, N=N, S=S, policy="clock", admission=admission)
        res = checked_call(ora, st, 0, [0], [N], topk, multi=True)
        assert res["plan"][0] == [(k, j, EMPTY) for j, k in enumerate(admitted)] + \
                                 [(k, H + j, EMPTY) for j, k in enumerate(overflow)]
    rng = np.random.default_rng(seed)
    for trial in range(trials):
        H = int(rng.integers(1, 6))
        S = int(rng.integers(2, 5))
        K = int(rng.integers(2, 5))
        N = int(rng.integers(H + 2, 20))
        trace = [rng.integers(-1, N, S * K).tolist() for _ in range(8)]
        for admission in ("frequent", "first"):
            _clock_compare_trace(ora, H, N, S, K, trace, admission=admission)


def pin_extra_ring(ora, seed=12, trials=30):
    """Reading R10 closed form: E = 4 newest tokens in the ring after the hot
    slots (rows 5..8 for H = 5).  With seq_len 20, tokens 16..19 are ring rows
    5 + t % 4; the others go through the LRU as if the ring tokens were not
    there.  Then random traces: a state with the ring and a state without,
    fed the same rows minus their ring entries, end every call in the same
    cache state with the same misses."""
    H, K, N, E = 5, 6, 40, 4
    st = make_state(ora, H=H, K=K, N=N, E=E)
    res = checked_call(ora, st, 0, [0], [20], np.array([[0, 16, 17, 19, 3, 16]]))
    assert res["out_locs"][0].tolist() == [0, 5, 6, 8, 1, 5]
    assert res["miss_count"][0] == 2 and [p[:2] for p in res["plan"][0]] == [(0, 0), (3, 1)]
    res = checked_call(ora, st, 0, [0], [24], np.array([[16, 17, 0, 21, -1, 23]]))
    assert res["out_locs"][0].tolist() == [2, 3, 0, 6, -1, 8]
    assert res["miss_count"][0] == 2
    rng = np.random.default_rng(seed)
    for trial in range(trials):
        clock = trial % 2 == 1
        H = int(rng.integers(2, 7))
        S = int(rng.integers(2, 4)) if clock else 1
        K = int(rng.integers(1, H + 1)) if not clock else int(rng.integers(1, 4))
        N = int(rng.integers(H + 4, 30))
        E = int(rng.integers(1, 5))
        pol = "clock" if clock else "lru"
        with_ring = make_state(ora, H=H, K=K, N=N, S=S, E=E, policy=pol)
        plain = make_state(ora, H=H, K=K, N=N, S=S, policy=pol)
        for call in range(8):
            seq = int(rng.integers(E + 1, N + 1))
            shape = (1, S, K) if clock else (1, K)
            topk = rng.integers(-1, seq, shape)
            res = checked_call(ora, with_ring, 0, [0], [seq], topk, multi=clock)
            stripped = np.where(topk >= seq - E, -1, topk)
            ref = checked_call(ora, plain, 0, [0], [seq], stripped, multi=clock)
            assert res["miss_count"].tolist() == ref["miss_count"].tolist()
            a, b = with_ring.instance(0, 0), plain.instance(0, 0)
            assert a.slot_key == b.slot_key and a.key_slot == b.key_slot
            ring = (topk >= seq - E) & (topk >= 0)
            base = H + (max(0, S * K - H) if clock else 0)     # after hot and scratch rows
            assert np.all(res["out_locs"][ring] == base + topk[ring] % E)
            assert np.all(res["out_locs"][~ring] == np.where(
                ref["out_locs"][~ring] >= 0,
                ref["out_locs"][~ring] // plain.rows * with_ring.rows + ref["out_locs"][~ring] % plain.rows,
                -1))


def pin_page_mode(ora, seed=7):
    """Page translation: pages are the distinct t div P in ascending order,
    ``page_table`` lists their rows, ``out_locs`` = page index * P + t mod P;
    the plan copies host pages ``r * N/P + p``.  With P = 1 the call equals a
    token-mode call whose row lists the distinct keys in ascending order."""
    rng = np.random.default_rng(seed)
    P, NP, H, K = 4, 10, 5, 6
    N = P * NP
    st = make_state(ora, R=2, H=H, K=K, N=N, P=P)
    for _ in range(40):
        topk = rng.integers(-1, N, (2, K))
        topk[1, : K // 2] = topk[1, 0]          # a repeated page / token
        pages = [sorted({int(t) // P for t in row if t >= 0}) for row in topk]
        if max(len(p) for p in pages) > H:
            continue
        before = [set(st.instance(r, 0).key_slot) for r in (0, 1)]
        res = checked_call(ora, st, 0, [0, 1], [N, N], topk)
        for b in range(2):
            assert res["num_pages"][b] == len(pages[b])
            assert res["miss_count"][b] == len(set(pages[b]) - before[b])
            for i, t in enumerate(topk[b]):
                if t < 0:
                    assert res["out_locs"][b, i] == -1
                else:
                    assert res["out_locs"][b, i] == pages[b].index(t // P) * P + t % P
            srcs = [s for s, _, _ in res["plan"][b]]
            assert srcs == [b * NP + p for p in pages[b] if p not in before[b]]
    # page mode equals token mode over page ids fed in ascending order
    stp = make_state(ora, H=5, K=6, N=12, P=2, seed=9)
    stt = make_state(ora, H=5, K=6, N=6, P=1, seed=9)
    for _ in range(30):
        row = rng.integers(-1, 12, 6)
        pages = sorted({int(t) // 2 for t in row if t >= 0})
        if len(pages) > 5:
            continue
        a = stp.swap_in_selected(0, [0], [12], [row])
        b = stt.swap_in_selected(0, [0], [6], [pages + [-1] * (6 - len(pages))])
        assert a["plan"][0] == b["plan"][0]
        assert a["page_table"][0, : len(pages)].tolist() == b["out_locs"][0, : len(pages)].tolist()


def pin_row_semantics(ora):
    """Padding (-1), out-of-range indices, rejected rows and duplicate
    requests (readings R9, R16)."""
    N, H, K = 20, 8, 4
    st = make_state(ora, R=3, H=H, K=K, N=N)
    res = st.swap_in_selected(0, [0, 1], [10, N], [[-1, 3, 10, -5], [19, 19, -1, 0]])
    assert res["out_locs"][0].tolist() == [-1, 0, -1, -1]
    assert res["out_locs"][1].tolist() == [H + 0, H + 0, -1, H + 1]
    assert res["miss_count"].tolist() == [1, 2]
    assert st.error_flags == ora.ERR_BAD_INDEX
    st.error_flags = 0
    res = st.swap_in_selected(0, [2, 2, 1], [N, N, N], [[1, 2, 3, 4]] * 3)
    assert res["out_locs"][:2].tolist() == [[-1] * 4] * 2
    assert res["miss_count"].tolist() == [0, 0, 4]
    assert st.error_flags == ora.ERR_DUP_REQUEST
    assert 2 not in {r for r, _ in st.inst}
    st.error_flags = 0
    res = st.swap_in_selected(0, [5, 0], [N, N + 1], [[1, 2, 3, 4]] * 2)
    assert res["out_locs"].tolist() == [[-1] * 4] * 2
    assert st.error_flags == ora.ERR_BAD_ROW
    # all-padding row is still a call: LRU clock advances, nothing resident,
    # and padding raises no error
    st2 = make_state(ora, H=4, K=2, N=6)
    st2.swap_in_selected(0, [0], [6], [[-1, -1]])
    assert st2.instance(0, 0).now == 1 and not st2.instance(0, 0).key_slot
    res = st2.swap_in_selected(0, [0], [6], [[5, -1]])
    assert res["out_locs"].tolist() == [[0, -1]] and st2.error_flags == 0
    # page overflow leaves the instance untouched
    st3 = make_state(ora, H=2, K=3, N=12, P=4)
    res = st3.swap_in_selected(0, [0], [12], [[0, 4, 8]])
    assert st3.error_flags == ora.ERR_PAGE_OVERFLOW
    assert res["out_locs"].tolist() == [[-1, -1, -1]] and res["num_pages"][0] == 0
    assert st3.instance(0, 0).now == 0


def pin_layers_independent(ora, seed=8):
    """Each (request, layer) is its own instance: interleaving another layer's
    and another request's calls changes nothing for a given instance."""
    rng = np.random.default_rng(seed)
    N, H, K = 30, 6, 4
    solo = make_state(ora, H=H, K=K, N=N)
    mixed = make_state(ora, R=3, L=2, H=H, K=K, N=N)
    for _ in range(20):
        row = rng.integers(-1, N, K)
        a = solo.swap_in_selected(0, [0], [N], [row])
        other = rng.integers(-1, N, (2, K))
        mixed.swap_in_selected(1, [1, 0], [N, N], other)
        b = mixed.swap_in_selected(0, [2, 0], [N, N], np.stack([other[0], row]))
        assert [(s % N, d % H, v) for s, d, v in a["plan"][0]] == \
               [(s % N, d % H, v) for s, d, v in b["plan"][1]]
        assert solo.instance(0, 0).slot_key == mixed.instance(0, 0).slot_key


def pin_multi_request_clock(ora, seed=10):
    """Several requests and layers in one multi-step batch with scratch rows
    (S * K > H): rows are ``r * (H + S*K - H) + slot`` and every returned row
    holds the key's host bytes (checked through the shadow device buffer)."""
    rng = np.random.default_rng(seed)
    R, L, H, S, K, N = 3, 2, 6, 3, 4, 25
    st = make_state(ora, R=R, L=L, H=H, K=K, N=N, S=S, policy="clock")
    assert st.rows == H + S * K - H
    for _ in range(15):
        req = rng.permutation(R)[:2]
        topk = rng.integers(-1, N, (2, S, K))
        layer = int(rng.integers(0, L))
        res = checked_call(ora, st, layer, req, [N, N], topk, multi=True)
        for b in range(2):
            for x, t in zip(res["out_locs"][b].reshape(-1), topk[b].reshape(-1)):
                if t >= 0:
                    assert x // st.rows == req[b]


def pin_sequential_comparator(ora, seed=13):
    """The per-step path the multi-step call replaces (PR #32162 report,
    "Features and motivation": one single-step call per speculative step).
    * K = 1: the S one-key calls of each multi-step row are S accesses of a
      textbook LRU, in step order;
    * steps with pairwise disjoint keys and H >= S*K, from empty: step s
      misses all of its K keys, which fill slots s*K .. s*K + K - 1 in the
      row's order, no victims, and the cache ends holding every key;
    * identical steps: step 0 misses its distinct keys, later steps miss
      nothing and return step 0's rows."""
    rng = np.random.default_rng(seed)
    N, H, S = 12, 4, 3
    st = make_state(ora, H=H, K=1, N=N)
    tb = TextbookLRU(H)
    for _ in range(60):
        keys = rng.integers(0, N, S)
        res = st.swap_sequential(0, [0], [N], keys.reshape(1, S, 1))
        assert len(res) == S
        for s, t in enumerate(keys):
            hit, ev = tb.access(int(t))
            assert res[s]["miss_count"][0] == (0 if hit else 1)
            if not hit:
                (src, _, victim), = res[s]["plan"][0]
                assert src == t and victim == (EMPTY if ev is None else ev)
    K = 5
    st = make_state(ora, H=S * K + 2, K=K, N=40)
    keys = rng.permutation(40)[:S * K].reshape(1, S, K)
    res = st.swap_sequential(0, [0], [40], keys)
    for s in range(S):
        assert res[s]["miss_count"][0] == K
        assert res[s]["plan"][0] == [(int(t), s * K + i, EMPTY) for i, t in enumerate(keys[0, s])]
        assert res[s]["out_locs"][0].tolist() == list(range(s * K, s * K + K))
    assert sorted(st.instance(0, 0).key_slot) == sorted(keys.reshape(-1).tolist())
    st = make_state(ora, H=8, K=K, N=40)
    row = rng.integers(-1, 40, K)
    res = st.swap_sequential(0, [0], [40], np.stack([row] * S)[None])
    distinct = len({int(t) for t in row if t >= 0})
    assert [r["miss_count"][0] for r in res] == [distinct] + [0] * (S - 1)
    for r in res[1:]:
        assert np.array_equal(r["out_locs"], res[0]["out_locs"])


def pin_request_reset(ora, seed=14):
    """A newly admitted request (request reset) empties that request's cache
    in every layer and leaves every other instance as it was; its next call
    is a first call from empty (closed form: misses fill slots 0, 1, ... in
    first-occurrence order, LRU counter back at 0; CLOCK hand back at 0)."""
    rng = np.random.default_rng(seed)
    R, L, N, K = 3, 2, 30, 5
    for policy, S, H in (("lru", 1, 8), ("clock", 2, 12)):
        st = make_state(ora, R=R, L=L, H=H, K=K, N=N, S=S, policy=policy)
        for _ in range(6):
            for layer in range(L):
                shape = (R, K) if S == 1 else (R, S, K)
                topk = rng.integers(0, N, shape)
                if S == 1:
                    st.swap_in_selected(layer, list(range(R)), [N] * R, topk)
                else:
                    st.swap_in_spec_multistep(layer, list(range(R)), [N] * R, topk)
        before = {(r, l): st.export(r, l) for r in range(R) for l in range(L)}
        st.request_reset([1])
        for r in range(R):
            for l in range(L):
                got = st.export(r, l)
                if r == 1:
                    assert got["slot_key"] == [EMPTY] * H and got["map"] == {}
                    assert got["ts"] == [-1] * H and got["now"] == 0
                    assert got["ref"] == [0] * H and got["hand"] == 0
                else:
                    assert got == before[(r, l)], f"instance ({r}, {l}) changed"
        keys = rng.permutation(N)[:K]
        ws = [int(t) for t in keys]
        if S == 1:
            res = st.swap_in_selected(1, [1], [N], keys[None])
        else:
            res = st.swap_in_spec_multistep(1, [1], [N], np.stack([keys] * S)[None])
        assert res["plan"][0] == [(N + t, st.rows + j, EMPTY) for j, t in enumerate(ws)]


ALL_PINS = [pin_first_call_closed_form, pin_overflow_closed_form, pin_admission_variants,
            pin_extra_ring,
            pin_row_semantics,
            pin_lru_textbook_k1, pin_clock_textbook_k1, pin_repeat_and_large_cache,
            pin_page_mode, pin_layers_independent, pin_multi_request_clock,
            pin_lru_random, pin_clock_random,
            pin_sequential_comparator, pin_request_reset,
            pin_clock_bruteforce, pin_lru_bruteforce]
