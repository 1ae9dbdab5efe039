"""The pages' own test shapes, on the oracle (no GPU)."""
import json
import pathlib

import numpy as np

from oracle import hisparse_oracle as ora
from tests import oracle_pins as pins

FACTS = json.loads((pathlib.Path(__file__).parent / "golden" / "page_facts.json").read_text())


def build_782_case(seed=782):
    """Batch 1, four steps of top-k 2048 over 32768 tokens, hot buffer 4096.

    A resident set of 3000 keys is imported first; the four rows share hits
    and draw their misses from a pool of exactly 782 non-resident tokens, every
    pool token appearing in at least two steps (cross-step duplicates).
    Returns (state arguments, resident keys, topk [1, 4, 2048], miss pool).
    """
    want = FACTS["unique_cross_step_misses"]["value"]
    rng = np.random.default_rng(seed)
    N, H, K, S = 32768, 4096, 2048, 4
    perm = rng.permutation(N)
    resident = perm[:3000]
    pool = perm[3000:3000 + want]
    rows = []
    for s in range(S):
        # each pool token appears in two of the four steps
        miss_part = pool[(np.arange(want) % S == s) | (np.arange(want) % S == (s + 1) % S)]
        hit_part = rng.choice(resident, K - miss_part.size, replace=False)
        rows.append(rng.permutation(np.concatenate([miss_part, hit_part])))
    topk = np.stack(rows)[None].astype(np.int32)
    return dict(N=N, H=H, K=K, S=S), resident, topk, pool


def test_782_unique_cross_step_misses_exact_copy():
    p, resident, topk, pool = build_782_case()
    st = pins.make_state(ora, H=p["H"], K=p["K"], N=p["N"], S=p["S"], policy="clock", I=32)
    slot_key = list(resident) + [ora.EMPTY] * (p["H"] - resident.size)
    st.import_(0, 0, slot_key, ref=[0] * p["H"], hand=0)
    res = pins.checked_call(ora, st, 0, [0], [p["N"]], topk, multi=True)
    assert res["miss_count"][0] == FACTS["unique_cross_step_misses"]["value"]
    assert sorted(s for s, _, _ in res["plan"][0]) == sorted(pool.tolist())
    # every pool token appears in two steps yet is copied once
    assert len({d for _, d, _ in res["plan"][0]}) == len(pool)


def test_step_range_is_the_pages():
    lo, hi = FACTS["num_steps_range"]["value"]
    st = pins.make_state(ora, H=8, K=2, N=10, S=hi, policy="clock")
    for s in range(lo, hi + 1):
        st.swap_in_spec_multistep(0, [0], [10], np.zeros((1, s, 2), np.int32))
    for bad in (lo - 1, hi + 1):
        try:
            st.swap_in_spec_multistep(0, [0], [10], np.zeros((1, bad, 2), np.int32))
        except ValueError:
            continue
        raise AssertionError("step count outside the pages' range accepted")
