"""Pins of the top-k / index-table oracle against things other than itself:
a characterisation of the selection rule checked by brute force over every
tiny input, torch.topk on distinct scores, closed forms, and planted mistakes
that these pins must catch."""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import topk_oracle as tk

NAN = float("nan")
INF = float("inf")


def is_valid_topk(values, n, k, chosen):
    """Reading T2 as a property, without sorting: `chosen` has min(k, n)
    distinct positions of [0, n), and every position outside it loses to every
    position inside (lower score, NaN lowest; on equal scores the higher
    position loses)."""
    if len(chosen) != min(k, n) or len(set(chosen)) != len(chosen):
        return False
    if any(not 0 <= p < n for p in chosen):
        return False

    def beats(p, q):  # p is preferred to q
        a, b = values[p], values[q]
        if math.isnan(a) or math.isnan(b):
            if math.isnan(a) and math.isnan(b):
                return p < q
            return math.isnan(b)
        return a > b or (a == b and p < q)

    outside = [q for q in range(n) if q not in chosen]
    return all(beats(p, q) for p in chosen for q in outside)


def test_brute_force_all_tiny_rows():
    """Every row over a 5-letter alphabet (NaN, -inf, -1, 0, 2) up to length
    5, every k up to 6 and every sequence length: the oracle's output is the
    unique subset the characterisation accepts, in ascending order."""
    alphabet = [NAN, -INF, -1.0, 0.0, 2.0]
    checked = 0
    for length in range(0, 6):
        for row in itertools.product(alphabet, repeat=length):
            vals = np.array(row, dtype=np.float32)
            for n in range(0, length + 1):
                for k in range(0, 7):
                    out = tk.topk_row(vals, n, k)
                    sel = [int(x) for x in out if x >= 0]
                    assert list(out[len(sel):]) == [-1] * (k - len(sel))
                    assert sel == sorted(sel)
                    assert is_valid_topk([float(v) for v in vals], n, k, sel), (row, n, k, sel)
                    # uniqueness: no other subset of the same size is valid
                    if length <= 4:
                        valid = [c for c in itertools.combinations(range(n), min(k, n))
                                 if is_valid_topk([float(v) for v in vals], n, k, list(c))]
                        assert valid == [tuple(sel)]
                    checked += 1
    assert checked > 10000


@pytest.mark.parametrize("seed", range(4))
def test_matches_torch_topk_on_distinct_scores(seed):
    rng = np.random.default_rng(seed)
    n = 5000
    vals = rng.permutation(n).astype(np.float32) * np.float32(0.37) - np.float32(900.0)
    for k in (1, 17, 2048, 4999, 5000, 6000):
        got = tk.topk_row(vals, n, k)
        ref = torch.topk(torch.from_numpy(vals), min(k, n)).indices.numpy()
        assert set(got[got >= 0].tolist()) == set(ref.tolist())
        assert np.all(np.diff(got[got >= 0]) > 0)


def test_closed_forms():
    n = 300
    inc = np.arange(n, dtype=np.float32)
    assert tk.topk_row(inc, n, 10).tolist() == list(range(290, 300))
    assert tk.topk_row(inc[::-1].copy(), n, 10).tolist() == list(range(10))
    const = np.full(n, 3.5, np.float32)
    assert tk.topk_row(const, n, 7).tolist() == list(range(7))
    # sequence length bounds the candidates
    assert tk.topk_row(inc, 50, 10).tolist() == list(range(40, 50))
    # k >= seq_len: everything, then padding
    assert tk.topk_row(inc, 5, 8).tolist() == [0, 1, 2, 3, 4, -1, -1, -1]
    assert tk.topk_row(inc, 0, 3).tolist() == [-1, -1, -1]
    # NaN below -inf
    v = np.array([NAN, -INF, NAN], np.float32)
    assert tk.topk_row(v, 3, 1).tolist() == [1]
    assert tk.topk_row(v, 3, 2).tolist() == [0, 1]


def test_index_tables():
    idx = np.array([0, 5, 17, 40, -1], np.int32)
    pt = np.array([9, 3, -1, 7, 2], np.int32)
    locs, err = tk.paged_locs(idx, pt, 16)
    assert locs.tolist() == [144, 149, 49, -1, -1] and err == tk.ERR_BAD_INDEX  # page 2 unmapped
    locs, err = tk.paged_locs(np.array([79, 80], np.int32), pt, 16)
    assert locs.tolist() == [2 * 16 + 15, -1] and err == tk.ERR_BAD_INDEX     # page 5 beyond table
    assert tk.ragged_locs(idx, 1000).tolist() == [1000, 1005, 1017, 1040, -1]


def test_row_rejection_and_batch():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((4, 64)).astype(np.float32)
    idx, locs, err = tk.topk_index_build(lg, np.array([64, 65, -1, 10]), 4, mode="ragged",
                                         row_offsets=np.array([0, 64, 128, 192]))
    assert err == tk.ERR_BAD_ROW
    assert np.all(idx[1] == -1) and np.all(idx[2] == -1) and np.all(locs[1] == -1)
    assert idx[3].tolist() == sorted(np.argsort(-lg[3, :10], kind="stable")[:4].tolist())
    assert locs[3].tolist() == (idx[3] + 192).tolist()


def test_plan_closed_forms_and_tiling():
    lens = np.array([0, 1, 1023, 1024, 32768, 32769, 65536, 100000, 131072, -3, 140000])
    info, items = tk.plan(lens, 131072)
    assert info[:, 1].tolist() == [1, 1, 1, 1, 1, 2, 2, 4, 4, 1, 1]
    assert items[info[5, 0]].tolist() == [5, 0, 0, 17408] and items[info[5, 0] + 1].tolist() == [5, 1, 17408, 15361]
    for b, s in enumerate(lens):
        s = s if 0 <= s <= 131072 else 0
        first, n = info[b]
        rows = items[first:first + n]
        assert np.all(rows[:, 0] == b) and rows[:, 1].tolist() == list(range(n))
        # chunks tile [0, s) in order, each at most the threshold, none empty when s > 0
        assert rows[0, 2] == 0 and int(rows[:, 3].sum()) == s
        assert np.all(rows[1:, 2] == rows[:-1, 2] + rows[:-1, 3])
        assert np.all(rows[:, 3] <= tk.SPLIT)
        if s > 0:
            assert np.all(rows[:, 3] > 0)
    assert len(items) == int(info[:, 1].sum())


def test_chunked_selection_equals_whole_row():
    """The property the chunked GPU selection relies on: the top-k of a row is
    the top-k of the union of its chunks' top-k."""
    rng = np.random.default_rng(11)
    s = 100000
    vals = np.round(rng.standard_normal(s) * 4).astype(np.float32)   # many ties
    info, items = tk.plan(np.array([s]), s)
    for k in (1, 100, 2048):
        cand = []
        for _, _, start, length in items:
            local = tk.topk_row(vals[start:start + length], length, k)
            cand.extend(int(p) + start for p in local if p >= 0)
        cand = np.array(sorted(cand))
        merged = cand[tk.topk_row(vals[cand], len(cand), k)]
        assert merged.tolist() == tk.topk_row(vals, s, k).tolist()


# ---- planted mistakes: each must be caught by the characterisation -------

def _mutant_tie_high(values, n, k):
    order = sorted(range(n), key=lambda p: (-(0 if math.isnan(values[p]) else 1),
                                           -(0 if math.isnan(values[p]) else values[p]), -p))
    return sorted(order[:k])


def _mutant_nan_high(values, n, k):
    order = sorted(range(n), key=lambda p: (-(1 if math.isnan(values[p]) else 0),
                                           -(0 if math.isnan(values[p]) else values[p]), p))
    return sorted(order[:k])


def _mutant_off_by_one(values, n, k):
    return [int(x) for x in tk.topk_row(np.array(values, np.float32), min(n + 1, len(values)), k)
            if x >= 0]


@pytest.mark.parametrize("mutant", [_mutant_tie_high, _mutant_nan_high, _mutant_off_by_one])
def test_planted_mistakes_are_caught(mutant):
    alphabet = [NAN, -INF, 0.0, 2.0]
    caught = False
    for row in itertools.product(alphabet, repeat=4):
        vals = [float(v) for v in row]
        for n in range(0, 4):
            for k in range(1, 4):
                if not is_valid_topk(vals, n, k, mutant(vals, n, k)):
                    caught = True
    assert caught
