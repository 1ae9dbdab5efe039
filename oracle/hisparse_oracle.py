"""CPU oracle of the HiSparse swap-in path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product path (the HIP library and its
binding) never imports, links or runs it, and this module imports nothing from
the product package.

It is a plain, slow, per-request dictionary implementation written from the
pages:

* sglang PR #20343 summary, "Implementation breakdown" (实现拆解): the
  single-step swap-in looks each selected token up in a token->slot hash table,
  handles hits and misses, and keeps an LRU cache; host (CPU) memory holds the
  idle KV ("Executive summary" / "Features and motivation").
* PR #32162 report, "Implementation breakdown" item 1: the multi-step (MTP)
  variant treats the top-k of all speculative steps as one working set, dedups
  misses across steps, uses a CLOCK cache and updates the token->slot hash;
  item 2: steps 2..4 and an optional ``miss_src / miss_dst / miss_count``
  plan; "Risks and impact": data of the current call stays exact, admission
  becomes approximate (favouring recent steps) once the union of unique misses
  exceeds the hot-cache capacity, ``hot_buffer_size`` up to 32768.
* "SGLang HiSparse" blog, section 2.1 (``swap_in_selected_pages`` takes
  ``req_pool_indices, seq_lens, topk_indices, layer_id`` and returns a sparse
  page table), sections 1.2/1.3 and 2.3 (token indices translated to the set
  of pages holding them; a token is located by its page and in-page offset).

Where the pages leave a step open the plainest reading is taken; each reading
is listed at the function that applies it:

R1  caches start empty.
R2  the j-th miss (first-occurrence order; ascending page order in page mode)
    takes the j-th victim in policy order.
R3  LRU key is (ts, slot), ts = the instance's call counter; EMPTY has ts -1.
R4  every valid key of a call (hit or miss) is used at ``now``.
R5  keys of the current call are never victims (pinned for the call).
R6  CLOCK: ref <- 1 on hit and on insert; the hand starts at 0, walks slots in
    ascending order mod H, persists across calls, skips pinned slots without
    clearing them and stops just after the last victim.
R7  multi-step overflow (more misses than unpinned slots): admit the misses
    with the largest last step, ties by first occurrence; the rest go to
    per-request scratch rows H, H+1, ... and are not inserted in the map.
    Two variants of the priority, for comparing admission policies (the
    pages call admission under overflow approximate and name no rule):
    "frequent" = the number of steps naming the key, "first" = none (first
    occurrence alone).  R7 proper is "recent", the default.
R8  duplicates inside a call resolve to one row and count as one miss.
R9  -1 is padding (output -1, no error); any other index outside
    [0, seq_len) outputs -1 and raises the bad-index error bit.
R10 extra-page lookup (PR #32162 report, item 1: done before the hash
    lookup; its meaning is not given): each request keeps its newest E
    tokens on the device in a ring of E rows after its hot and scratch rows
    (row H + X + t mod E, written by the decode, not by these calls).  An
    entry t with seq_len - E <= t < seq_len resolves to its ring row: no
    probe, no miss, no copy, no change to the cache state.  Token mode only.
R11 each (request, layer) pair is an independent cache instance.
R14 page mode with more distinct pages than hot pages: error bit, the row
    outputs -1 and the instance is left untouched.
R15 page mode requires the host KV length to be a multiple of the page size.
R16 a request named twice in one batch is rejected (both rows output -1,
    error bit, state untouched); so is a row whose request index or
    sequence length is out of range.

Parity pins (tests/test_oracle_*.py): textbook LRU and second-chance CLOCK at
K = 1, closed forms (first call from empty, repeated calls, H >= N), an
independently written recency-list LRU and two-lap CLOCK on exhaustive tiny
traces, the invariants of every call, page translation closed forms, the
sequential comparator (a textbook LRU over its one-key steps, closed forms
for disjoint and identical steps), request reset (the named request empty in
every layer, every other instance unchanged, then a first call from empty),
and a planted-mistake (mutation) suite.  Multi-step overflow admission follows
reading R7 and is pinned by a closed-form case only; the pages call that
admission approximate, so beyond R7 it is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

EMPTY = -1

# Error bits raised by a call (sticky across calls until read).
ERR_BAD_INDEX = 1 << 0       # a top-k entry outside [0, seq_len) that is not -1
ERR_DUP_REQUEST = 1 << 1     # the same request twice in one batch
ERR_PAGE_OVERFLOW = 1 << 2   # more distinct pages than hot pages in one row
ERR_BAD_ROW = 1 << 3         # request index or sequence length out of range


class CacheInstance:
    """Hot cache of one (request, layer) pair (reading R11).

    ``key_slot`` is the token->slot (or page->slot) hash table of the pages;
    ``slot_key`` its inverse over the H hot slots.
    """

    def __init__(self, hot: int):
        self.hot = hot
        self.slot_key = [EMPTY] * hot
        self.key_slot: dict[int, int] = {}
        self.ts = [-1] * hot      # LRU timestamps (R3)
        self.now = 0              # LRU clock: calls made on this instance
        self.ref = [0] * hot      # CLOCK reference bits (R6)
        self.hand = 0             # CLOCK hand (R6)


def distinct_in_first_occurrence(keys):
    """Distinct keys of ``keys`` in order of first occurrence (R2, R8)."""
    seen = set()
    out = []
    for k in keys:
        if k not in seen:
            seen.add(k)
            out.append(k)
    return out


def lru_admit(inst: CacheInstance, working_set):
    """Resolve one call's working set under exact LRU.

    PR #20343 summary, "Implementation breakdown": hash lookup, hit/miss
    handling and an LRU update.  ``working_set`` lists distinct keys in the
    order their misses are to be placed (R2).  Returns the placements
    ``[(key, slot, evicted key or EMPTY)]`` in miss order.
    """
    hot = inst.hot
    in_call = set(working_set)
    hits = [k for k in working_set if k in inst.key_slot]
    misses = [k for k in working_set if k not in inst.key_slot]
    for k in hits:                                   # R4: hits are used now
        inst.ts[inst.key_slot[k]] = inst.now
    # R5: a slot holding a key of this call is never a victim.  R3: the
    # least recent (ts, slot) goes first; EMPTY slots have ts -1.
    candidates = [s for s in range(hot)
                  if inst.slot_key[s] == EMPTY or inst.slot_key[s] not in in_call]
    candidates.sort(key=lambda s: (inst.ts[s], s))
    assert len(candidates) >= len(misses), "working set larger than the hot cache"
    placed = []
    for j, key in enumerate(misses):                 # R2
        slot = candidates[j]
        evicted = inst.slot_key[slot]
        if evicted != EMPTY:
            del inst.key_slot[evicted]
        inst.slot_key[slot] = key
        inst.key_slot[key] = slot
        inst.ts[slot] = inst.now                     # R4: misses are used now
        placed.append((key, slot, evicted))
    inst.now += 1
    return placed


def clock_sweep(inst: CacheInstance, count: int, pinned: set):
    """Choose ``count`` victims with the CLOCK hand (reading R6).

    PR #32162 report, "Implementation breakdown" item 1 (CLOCK cache state);
    the walk is the textbook second-chance sweep with pinned slots skipped.
    """
    hot = inst.hot
    victims = []
    chosen = set()
    h = inst.hand
    while len(victims) < count:
        s = h
        h = (h + 1) % hot
        if s in pinned or s in chosen:
            continue
        if inst.ref[s]:
            inst.ref[s] = 0                           # second chance
            continue
        victims.append(s)
        chosen.add(s)
    if victims:
        inst.hand = h                                 # just after the last victim
    return victims


ADMISSION = ("recent", "frequent", "first")


def admission_priority(steps: set, admission: str) -> int:
    """R7 and its variants: the priority of a missing key under overflow
    (higher is admitted first; ties by first occurrence)."""
    if admission == "recent":
        return max(steps)
    if admission == "frequent":
        return len(steps)
    if admission == "first":
        return 0
    raise ValueError(admission)


def clock_admit(inst: CacheInstance, working_set, steps_of, admission="recent"):
    """Resolve one multi-step call's working set under CLOCK.

    PR #32162 report, "Implementation breakdown" item 1 and "Risks and impact".
    ``working_set``: distinct keys in first-occurrence order over the
    step-major flattened ``[steps, top_k]`` rows; ``steps_of[key]``: the set
    of steps the key appears in.  Returns ``(placed, overflow)`` where
    ``placed`` lists ``(key, slot, evicted)`` in admission order and
    ``overflow`` lists the keys sent to scratch rows (R7), in first-occurrence
    order.
    """
    hot = inst.hot
    hits = [k for k in working_set if k in inst.key_slot]
    misses = [k for k in working_set if k not in inst.key_slot]
    pinned = {inst.key_slot[k] for k in hits}        # R5
    for p in pinned:                                  # R6: ref set on hit
        inst.ref[p] = 1
    capacity = hot - len(pinned)
    if len(misses) <= capacity:
        admitted, overflow = misses, []
    else:                                             # R7
        rank = sorted(range(len(misses)),
                      key=lambda j: (-admission_priority(steps_of[misses[j]], admission), j))
        keep = set(rank[:capacity])
        admitted = [k for j, k in enumerate(misses) if j in keep]
        overflow = [k for j, k in enumerate(misses) if j not in keep]
    victims = clock_sweep(inst, len(admitted), pinned)
    placed = []
    for key, slot in zip(admitted, victims):         # R2
        evicted = inst.slot_key[slot]
        if evicted != EMPTY:
            del inst.key_slot[evicted]
        inst.slot_key[slot] = key
        inst.key_slot[key] = slot
        inst.ref[slot] = 1                            # R6: ref set on insert
        placed.append((key, slot, evicted))
    return placed, overflow


class OracleState:
    """All cache instances of one state, with the call semantics of the library.

    ``host_kv`` (optional) is a list over layers of uint8 arrays
    ``[max_requests, max_seq_len, item_bytes]``; when given, the oracle keeps a
    shadow of the device KV buffers (``dev_kv``) and performs every miss copy,
    so data exactness can be checked.
    """

    def __init__(self, *, max_requests, num_layers, hot, top_k, item_bytes,
                 max_seq_len, max_steps=1, page_size=1, policy="lru", host_kv=None,
                 admission="recent", extra_rows=0):
        if policy not in ("lru", "clock"):
            raise ValueError(policy)
        if admission not in ADMISSION:
            raise ValueError(admission)
        self.admission = admission
        if extra_rows and page_size > 1:
            raise ValueError("the extra-row ring is token mode only (R10)")
        self.E = extra_rows
        if page_size > 1 and max_seq_len % page_size:
            raise ValueError("page mode needs max_seq_len % page_size == 0 (R15)")
        self.R, self.L, self.H, self.K = max_requests, num_layers, hot, top_k
        self.I, self.N, self.S, self.P = item_bytes, max_seq_len, max_steps, page_size
        self.policy = policy
        self.scratch = max(0, max_steps * top_k - hot) if max_steps > 1 else 0
        self.ring = hot + self.scratch               # first extra-ring row (R10)
        self.rows = hot + self.scratch + extra_rows  # device rows per request
        self.inst: dict[tuple[int, int], CacheInstance] = {}
        self.error_flags = 0
        self.host_kv = host_kv
        self.dev_kv = None
        if host_kv is not None:
            unit = item_bytes * page_size
            self.dev_kv = [np.zeros((max_requests, self.rows, unit), np.uint8)
                           for _ in range(num_layers)]

    # -- helpers -----------------------------------------------------------
    def instance(self, r: int, l: int) -> CacheInstance:
        key = (r, l)
        if key not in self.inst:
            self.inst[key] = CacheInstance(self.H)   # R1
        return self.inst[key]

    def request_reset(self, reqs):
        """A newly admitted request starts from an empty cache in every layer."""
        for r in reqs:
            for l in range(self.L):
                self.inst.pop((int(r), l), None)

    def _row_error(self, b, req, seq_lens):
        r, sl = int(req[b]), int(seq_lens[b])
        if not (0 <= r < self.R and 0 <= sl <= self.N):
            return ERR_BAD_ROW
        if int(np.count_nonzero(np.asarray(req) == r)) > 1:
            return ERR_DUP_REQUEST
        return 0

    def _split_extra(self, entries, seq_len):
        """R10: (cached entries, extra entries) of a row's valid entries."""
        lo = seq_len - self.E
        if self.E == 0:
            return entries, []
        return [e for e in entries if e[1] < lo], [e for e in entries if e[1] >= lo]

    def _valid_entries(self, keys, seq_len):
        """(position, token) of the valid entries of a row (R9)."""
        out = []
        for i, t in enumerate(keys):
            t = int(t)
            if t == -1:
                continue
            if not (0 <= t < seq_len):
                self.error_flags |= ERR_BAD_INDEX
                continue
            out.append((i, t))
        return out

    def _copy(self, l, r, key, slot_row):
        if self.dev_kv is None:
            return
        if self.P == 1:
            self.dev_kv[l][r, slot_row] = self.host_kv[l][r, key]
        else:
            p0 = key * self.P
            self.dev_kv[l][r, slot_row] = self.host_kv[l][r, p0:p0 + self.P].reshape(-1)

    # -- single-step (LRU) ---------------------------------------------------
    def swap_in_selected(self, layer, req_pool_indices, seq_lens, topk):
        """One per-layer single-step call ("SGLang HiSparse" blog, §2.1).

        ``topk``: int ``[B, K]``.  Token mode returns ``out_locs[b, i]`` = the
        device row ``r * rows + slot`` of token ``topk[b, i]``.  Page mode
        (page_size P > 1) returns ``page_table[b, j]`` = ``r * H + slot`` of
        the j-th distinct page in ascending order (-1 beyond), ``num_pages[b]``
        and ``out_locs[b, i]`` = ``j * P + t % P`` (blog §2.3, PAGED mode).
        The plan lists ``(src, dst, evicted)`` per miss with ``src`` the host
        row (``r * N + t``, or host page ``r * N / P + p``), ``dst`` the device
        row and ``evicted`` the replaced key or -1 (PR #32162 report, item 2).
        """
        if self.policy != "lru":
            raise ValueError("single-step calls use an LRU state")
        topk = np.asarray(topk)
        B, K = topk.shape
        out = np.full((B, K), -1, np.int32)
        miss_count = np.zeros(B, np.int32)
        plan = [[] for _ in range(B)]
        page_table = np.full((B, self.H), -1, np.int32) if self.P > 1 else None
        num_pages = np.zeros(B, np.int32) if self.P > 1 else None
        for b in range(B):
            err = self._row_error(b, req_pool_indices, seq_lens)
            if err:
                self.error_flags |= err
                continue
            r = int(req_pool_indices[b])
            entries = self._valid_entries(topk[b], int(seq_lens[b]))
            entries, extra = self._split_extra(entries, int(seq_lens[b]))
            for i, t in extra:
                out[b, i] = r * self.rows + self.ring + t % self.E
            inst = self.instance(r, layer)
            if self.P == 1:
                ws = distinct_in_first_occurrence(t for _, t in entries)
                placed = lru_admit(inst, ws)
                for key, slot, ev in placed:
                    self._copy(layer, r, key, slot)
                    plan[b].append((r * self.N + key, r * self.rows + slot, ev))
                for i, t in entries:
                    out[b, i] = r * self.rows + inst.key_slot[t]
            else:
                pages = sorted({t // self.P for _, t in entries})
                if len(pages) > self.H:                 # R14
                    self.error_flags |= ERR_PAGE_OVERFLOW
                    continue
                placed = lru_admit(inst, pages)
                for key, slot, ev in placed:
                    self._copy(layer, r, key, slot)
                    plan[b].append((r * (self.N // self.P) + key, r * self.H + slot, ev))
                index_of = {p: j for j, p in enumerate(pages)}
                for j, p in enumerate(pages):
                    page_table[b, j] = r * self.H + inst.key_slot[p]
                num_pages[b] = len(pages)
                for i, t in entries:
                    out[b, i] = index_of[t // self.P] * self.P + t % self.P
            miss_count[b] = len(placed)
        res = {"out_locs": out, "miss_count": miss_count, "plan": plan}
        if self.P > 1:
            res["page_table"] = page_table
            res["num_pages"] = num_pages
        return res

    # -- multi-step (CLOCK) --------------------------------------------------
    def swap_in_spec_multistep(self, layer, req_pool_indices, seq_lens, topk):
        """One multi-step call over ``topk`` int ``[B, S, K]``, S in 2..4.

        PR #32162 report, "Implementation breakdown" items 1-2: all steps of
        a row form one working set, misses are deduplicated across steps and
        resolved by one CLOCK update.  ``out_locs[b, s, i]`` is the device row
        of token ``topk[b, s, i]``: its hot slot, or its scratch row
        ``H + j`` on overflow (R7).  The plan lists admitted misses first, in
        admission order, then the overflow misses.
        """
        if self.policy != "clock":
            raise ValueError("multi-step calls use a CLOCK state")
        topk = np.asarray(topk)
        B, S, K = topk.shape
        if not (2 <= S <= self.S):
            raise ValueError("num_steps must be in [2, max_steps]")
        out = np.full((B, S, K), -1, np.int32)
        miss_count = np.zeros(B, np.int32)
        plan = [[] for _ in range(B)]
        for b in range(B):
            err = self._row_error(b, req_pool_indices, seq_lens)
            if err:
                self.error_flags |= err
                continue
            r = int(req_pool_indices[b])
            flat = topk[b].reshape(-1)                # step-major (s, i)
            entries = self._valid_entries(flat, int(seq_lens[b]))
            entries, extra = self._split_extra(entries, int(seq_lens[b]))
            for pos, t in extra:
                out[b, pos // K, pos % K] = r * self.rows + self.ring + t % self.E
            ws = distinct_in_first_occurrence(t for _, t in entries)
            steps_of = {}
            for pos, t in entries:
                steps_of.setdefault(t, set()).add(pos // K)
            inst = self.instance(r, layer)
            placed, overflow = clock_admit(inst, ws, steps_of, self.admission)
            for key, slot, ev in placed:
                self._copy(layer, r, key, slot)
                plan[b].append((r * self.N + key, r * self.rows + slot, ev))
            scratch_row = {}
            for j, key in enumerate(overflow):
                scratch_row[key] = self.H + j
                self._copy(layer, r, key, self.H + j)
                plan[b].append((r * self.N + key, r * self.rows + self.H + j, EMPTY))
            for pos, t in entries:
                slot = inst.key_slot[t] if t in inst.key_slot else scratch_row[t]
                out[b, pos // K, pos % K] = r * self.rows + slot
            miss_count[b] = len(placed) + len(overflow)
        return {"out_locs": out, "miss_count": miss_count, "plan": plan}

    # -- sequential comparator -------------------------------------------------
    def swap_sequential(self, layer, req_pool_indices, seq_lens, topk):
        """The per-step path the multi-step kernel replaces: one single-step LRU
        call per speculative step (PR #32162 report, "Features and motivation")."""
        topk = np.asarray(topk)
        return [self.swap_in_selected(layer, req_pool_indices, seq_lens, topk[:, s])
                for s in range(topk.shape[1])]

    # -- state views -----------------------------------------------------------
    def export(self, r: int, l: int):
        inst = self.instance(r, l)
        return {"slot_key": list(inst.slot_key), "ts": list(inst.ts), "now": inst.now,
                "ref": list(inst.ref), "hand": inst.hand, "map": dict(inst.key_slot)}

    def import_(self, r: int, l: int, slot_key, ts=None, now=0, ref=None, hand=0):
        """Prepopulate an instance (the pages' tests build a resident set first,
        PR #32162 report, "Key files": ``_make_cache_index`` / ``_make_state``)."""
        inst = CacheInstance(self.H)
        inst.slot_key = [int(k) for k in slot_key]
        inst.key_slot = {k: s for s, k in enumerate(inst.slot_key) if k != EMPTY}
        if len(inst.key_slot) != sum(k != EMPTY for k in inst.slot_key):
            raise ValueError("a key is resident in two slots")
        inst.ts = [int(x) for x in ts] if ts is not None else [-1] * self.H
        inst.now = int(now)
        inst.ref = [int(x) for x in ref] if ref is not None else [0] * self.H
        inst.hand = int(hand)
        self.inst[(r, l)] = inst
        for s, k in enumerate(inst.slot_key):        # resident keys hold their bytes
            if k != EMPTY:
                self._copy(l, r, k, s)


# -- invariants (checked after every call in the tests) --------------------------

def check_instance(inst: CacheInstance, policy: str):
    """Structural invariants of one instance; raises AssertionError."""
    assert len(inst.key_slot) <= inst.hot, "occupancy above capacity"
    for s, k in enumerate(inst.slot_key):
        if k != EMPTY:
            assert inst.key_slot.get(k) == s, "slot_key and key_slot disagree"
    for k, s in inst.key_slot.items():
        assert inst.slot_key[s] == k, "key_slot and slot_key disagree"
    if policy == "lru":
        for s, k in enumerate(inst.slot_key):
            assert (k == EMPTY) == (inst.ts[s] == -1), "ts of EMPTY slots is -1"
            assert inst.ts[s] < inst.now
    else:
        assert 0 <= inst.hand < inst.hot
        assert all(x in (0, 1) for x in inst.ref)


def check_call(state: OracleState, layer, req_pool_indices, seq_lens, topk, res,
               resident_before):
    """Per-call invariants: no device row serves two keys, miss_count equals the
    distinct valid keys minus those resident at call start, every key of the
    call ends resident (or in scratch) and used, and -- with a shadow device
    buffer -- every returned row holds exactly that key's host bytes."""
    topk = np.asarray(topk)
    multi = topk.ndim == 3
    B = topk.shape[0]
    for b in range(B):
        r = int(req_pool_indices[b])
        if res["miss_count"][b] == 0 and np.all(res["out_locs"][b] == -1):
            continue
        keys = topk[b].reshape(-1)
        outs = np.asarray(res["out_locs"][b]).reshape(-1)
        sl = int(seq_lens[b])
        lo = sl - state.E if state.E else sl
        valid = [(i, int(t)) for i, t in enumerate(keys) if 0 <= t < lo]
        assert all(outs[i] == -1 for i, t in enumerate(keys) if not (0 <= t < sl))
        for i, t in enumerate(keys):                  # R10: the extra ring
            if lo <= t < sl:
                assert outs[i] == r * state.rows + state.ring + int(t) % state.E
        if state.P == 1:
            row_of = {}
            for i, t in valid:
                row_of.setdefault(t, outs[i])
                assert row_of[t] == outs[i], "duplicate key resolved twice"
            assert len(set(row_of.values())) == len(row_of), "row assigned twice"
            distinct = set(row_of)
            assert res["miss_count"][b] == len(distinct - resident_before[b])
            inst = state.instance(r, layer)
            if state.policy == "lru":
                for t in distinct:
                    assert inst.ts[inst.key_slot[t]] == inst.now - 1
            else:
                for t in distinct:
                    if t in inst.key_slot:
                        assert inst.ref[inst.key_slot[t]] == 1
            if state.dev_kv is not None:
                flat = state.dev_kv[layer].reshape(-1, state.I)
                for t, row in row_of.items():
                    assert np.array_equal(flat[row], state.host_kv[layer][r, t]), \
                        "returned row does not hold the key's bytes"
        else:
            pages = sorted({t // state.P for _, t in valid})
            assert res["num_pages"][b] == len(pages)
            assert res["miss_count"][b] == len(set(pages) - resident_before[b])
            pt = res["page_table"][b]
            assert len(set(pt[:len(pages)].tolist())) == len(pages)
            assert np.all(pt[len(pages):] == -1)
            if state.dev_kv is not None:
                dev_tok = state.dev_kv[layer].reshape(-1, state.I)
                for i, t in valid:
                    j, o = divmod(int(outs[i]), state.P)
                    row = int(pt[j]) * state.P + o
                    assert np.array_equal(dev_tok[row], state.host_kv[layer][r, t])
    if multi:
        assert topk.shape[1] >= 2
