"""Planted mistakes in the oracle must be caught by the pins (no GPU).

Each mutant is a one-line edit of ``oracle/hisparse_oracle.py`` of the kind a
reader could plausibly make (a wrong tie-break, a missed update, an off-by-one,
a transposed operand).  The mutated source is executed as a separate module and
the full pin battery runs against it; at least one pin must fail.
"""
import pathlib
import signal
import types

import pytest

from tests import oracle_pins as pins

SRC = (pathlib.Path(__file__).resolve().parents[1] / "oracle" / "hisparse_oracle.py").read_text()

MUTANTS = {
    "lru_tiebreak_slot_desc": (
        "candidates.sort(key=lambda s: (inst.ts[s], s))",
        "candidates.sort(key=lambda s: (inst.ts[s], -s))"),
    "lru_evicts_most_recent": (
        "candidates.sort(key=lambda s: (inst.ts[s], s))",
        "candidates.sort(key=lambda s: (-inst.ts[s], s))"),
    "lru_hits_not_touched": (
        "        inst.ts[inst.key_slot[k]] = inst.now\n",
        "        pass\n"),
    "lru_miss_ts_off_by_one": (
        "        inst.ts[slot] = inst.now                     # R4",
        "        inst.ts[slot] = inst.now - 1                 # R4"),
    "lru_clock_never_advances": (
        "    inst.now += 1\n",
        "    pass\n"),
    "lru_misses_reversed": (
        "    for j, key in enumerate(misses):                 # R2",
        "    for j, key in enumerate(misses[::-1]):           # R2"),
    "clock_ignores_pins": (
        "        if s in pinned or s in chosen:",
        "        if s in chosen:"),
    "clock_no_second_chance": (
        "            inst.ref[s] = 0                           # second chance\n            continue\n",
        "            inst.ref[s] = 0                           # second chance\n"),
    "clock_hand_at_last_victim": (
        "        inst.hand = h                                 # just after the last victim",
        "        inst.hand = victims[-1]"),
    "clock_hit_ref_not_set": (
        "        inst.ref[p] = 1\n",
        "        pass\n"),
    "clock_insert_ref_zero": (
        "        inst.ref[slot] = 1                            # R6: ref set on insert",
        "        inst.ref[slot] = 0"),
    "overflow_prefers_old_steps": (
        "key=lambda j: (-admission_priority(steps_of[misses[j]], admission), j)",
        "key=lambda j: (admission_priority(steps_of[misses[j]], admission), j)"),
    "last_step_from_offset": (
        "                steps_of.setdefault(t, set()).add(pos // K)",
        "                steps_of.setdefault(t, set()).add(pos % K)"),
    "extra_window_short": (
        "        lo = seq_len - self.E\n",
        "        lo = seq_len - self.E + 1\n"),
    "extra_ring_ignores_scratch": (
        "        self.ring = hot + self.scratch ",
        "        self.ring = hot "),
    "frequent_is_recent": (
        "    if admission == \"frequent\":\n        return len(steps)",
        "    if admission == \"frequent\":\n        return max(steps)"),
    "first_by_last_step": (
        "    if admission == \"first\":\n        return 0",
        "    if admission == \"first\":\n        return -max(steps)"),
    "scratch_rows_off_by_one": (
        "self.scratch = max(0, max_steps * top_k - hot) if max_steps > 1 else 0",
        "self.scratch = max(0, max_steps * top_k - hot + 1) if max_steps > 1 else 0"),
    "multistep_row_without_scratch": (
        "                out[b, pos // K, pos % K] = r * self.rows + slot",
        "                out[b, pos // K, pos % K] = r * self.H + slot"),
    "no_dedup": (
        "            seen.add(k)\n",
        "            pass\n"),
    "seq_len_bound_inclusive": (
        "            if not (0 <= t < seq_len):",
        "            if not (0 <= t <= seq_len):"),
    "padding_flagged": (
        "            if t == -1:\n                continue\n",
        "            if t == -2:\n                continue\n"),
    "duplicate_request_missed": (
        "if int(np.count_nonzero(np.asarray(req) == r)) > 1:",
        "if int(np.count_nonzero(np.asarray(req) == r)) > 2:"),
    "copy_from_slot_row": (
        "            self.dev_kv[l][r, slot_row] = self.host_kv[l][r, key]",
        "            self.dev_kv[l][r, slot_row] = self.host_kv[l][r, slot_row]"),
    "page_copy_offset": (
        "            p0 = key * self.P\n",
        "            p0 = key\n"),
    "pages_first_occurrence": (
        "                pages = sorted({t // self.P for _, t in entries})",
        "                pages = distinct_in_first_occurrence(t // self.P for _, t in entries)"),
    "page_offset_div": (
        "                    out[b, i] = index_of[t // self.P] * self.P + t % self.P",
        "                    out[b, i] = index_of[t // self.P] * self.P + t // self.P"),
    "page_table_without_request": (
        "                    page_table[b, j] = r * self.H + inst.key_slot[p]",
        "                    page_table[b, j] = inst.key_slot[p]"),
    "page_plan_src_token_units": (
        "plan[b].append((r * (self.N // self.P) + key, r * self.H + slot, ev))",
        "plan[b].append((r * self.N + key, r * self.H + slot, ev))"),
    "sequential_reuses_step_0": (
        "self.swap_in_selected(layer, req_pool_indices, seq_lens, topk[:, s])",
        "self.swap_in_selected(layer, req_pool_indices, seq_lens, topk[:, 0])"),
    "reset_only_layer_0": (
        "            for l in range(self.L):\n                self.inst.pop((int(r), l), None)",
        "            for l in range(1):\n                self.inst.pop((int(r), l), None)"),
    "reset_request_and_layer_transposed": (
        "                self.inst.pop((int(r), l), None)",
        "                self.inst.pop((l, int(r)), None)"),
}


def _load(name, src):
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def _alarm(signum, frame):
    raise TimeoutError("mutant did not finish")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation site for {name} not unique"
    mod = _load(name, SRC.replace(old, new))
    prev = signal.signal(signal.SIGALRM, _alarm)
    signal.alarm(60)
    caught = None
    try:
        for pin in pins.ALL_PINS:
            try:
                pin(mod)
            except Exception as e:  # any failing pin catches the mutant
                caught = (pin.__name__, type(e).__name__)
                break
    finally:
        signal.alarm(0)
        signal.signal(signal.SIGALRM, prev)
    assert caught is not None, f"mutant {name} survived every pin"


def test_unmutated_source_passes():
    mod = _load("identity", SRC)
    for pin in pins.ALL_PINS:
        pin(mod)
