"""Top-k selection + index-table build (HIP, through the C ABI) against the
CPU oracle: indices, index tables, plan and error bits must match exactly."""
import numpy as np
import pytest
import torch

from oracle import topk_oracle as tk
from sparse_attention_kv_request_amd import binding
from tests.gpu_harness import DEV, log

pytestmark = pytest.mark.gpu


def logits_with_specials(rng, B, N, ties=False):
    x = rng.standard_normal((B, N)).astype(np.float32)
    if ties:
        x = np.round(x * 2).astype(np.float32)          # few distinct values
    flat = x.reshape(-1)
    for v in (np.nan, -np.inf, np.inf, -0.0, 0.0):
        flat[rng.choice(flat.size, max(1, flat.size // 500), replace=False)] = v
    return x


def run(logits, seq_lens, k, mode="none", page_table=None, page_size=1, row_offsets=None,
        layers=1, check_plan=True):
    B, N = logits.shape
    b = binding.TopkIndexBuilder(B, N, k, device=DEV)
    sl = torch.from_numpy(np.asarray(seq_lens, np.int32)).to(DEV)
    b.plan(sl)
    if check_plan:
        info, items = tk.plan(np.asarray(seq_lens), N)
        plan = b.plan_buf.cpu().numpy()
        n_items = len(items)
        assert plan[0] == n_items and plan[1] == N
        assert np.array_equal(plan[2:2 + 2 * B].reshape(B, 2), info)
        assert np.array_equal(plan[2 + 2 * B:2 + 2 * B + 4 * n_items].reshape(-1, 4), items)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)
    pt, ro = t(page_table), t(row_offsets)
    for layer in range(layers):
        lg = logits if layer == 0 else np.roll(logits, layer * 7, axis=1)
        idx = torch.full((B, k), 12345, dtype=torch.int32, device=DEV)
        locs = None if mode == "none" else torch.full((B, k), 12345, dtype=torch.int32, device=DEV)
        b.build(torch.from_numpy(lg).to(DEV), sl, idx, locs, mode=mode, page_table=pt,
                page_size=page_size, row_offsets=ro)
        torch.cuda.synchronize()
        ref_idx, ref_locs, ref_err = tk.topk_index_build(lg, np.asarray(seq_lens), k, mode=mode,
                                                          page_table=page_table,
                                                          page_size=page_size,
                                                          row_offsets=row_offsets)
        got = idx.cpu().numpy()
        bad = np.nonzero(np.any(got != ref_idx, axis=1))[0]
        assert bad.size == 0, f"layer {layer}: rows {bad[:5]} differ, e.g. {got[bad[0]][:8]} vs {ref_idx[bad[0]][:8]}"
        if mode != "none":
            assert np.array_equal(locs.cpu().numpy(), ref_locs)
        assert b.error_flags() == ref_err
    return b


def test_small_rows_edge_lengths():
    rng = np.random.default_rng(1)
    lg = logits_with_specials(rng, 6, 1000)
    run(lg, [0, 1, 63, 64, 1000, 999], 64)
    run(lg, [0, 1, 63, 64, 1000, 999], 1)
    run(lg, [1000, 5, 700, 64, 2, 999], 1000)


def test_ties_and_specials():
    rng = np.random.default_rng(2)
    lg = logits_with_specials(rng, 4, 5000, ties=True)
    run(lg, [5000, 4096, 1234, 4999], 777)
    const = np.full((2, 3000), 1.5, np.float32)
    run(const, [3000, 2000], 100)
    nan = np.full((1, 2048), np.nan, np.float32)
    nan[0, 100] = -np.inf
    run(nan, [2048], 10)


def test_split_rows_and_ragged_table():
    rng = np.random.default_rng(3)
    N = 32768 + 5000
    lg = logits_with_specials(rng, 5, N, ties=True)
    lens = [N, 32768, 32769, 40000 - 3000, 17]
    offs = np.cumsum([0] + lens[:-1]).astype(np.int32)
    run(lg, lens, 512, mode="ragged", row_offsets=offs, layers=3)


def test_long_rows_paged_table_with_holes():
    rng = np.random.default_rng(4)
    B, N, P = 3, 131072, 64
    lg = logits_with_specials(rng, B, N)
    pt = rng.permutation(B * (N // P)).astype(np.int32).reshape(B, N // P)
    pt[0, rng.choice(N // P, 50, replace=False)] = -1     # unmapped pages -> error bit
    run(lg, [131072, 100000, 70001], 2048, mode="paged", page_table=pt, page_size=P, layers=2)


def test_equal_scores_across_chunks():
    """All scores equal: the lowest positions win, across chunk boundaries."""
    lg = np.zeros((2, 4 * 32768), np.float32)
    run(lg, [4 * 32768, 3 * 32768 + 1], 2048)
    lg[1, -5:] = 1.0
    run(lg, [4 * 32768, 4 * 32768], 8)


def test_rejected_rows_and_unaligned_stride():
    rng = np.random.default_rng(5)
    lg = logits_with_specials(rng, 4, 4099)                 # row stride not a multiple of 4
    run(lg, [4099, -1, 4100, 300], 50, mode="ragged", row_offsets=[0, 1, 2, 3])


@pytest.mark.parametrize("B,N", [(64, 32768), (128, 131072)])
def test_full_size(B, N):
    """The two deployment shapes: 64 rows of 32768 and 128 rows of 131072
    scores, k = 2048, the recency-and-cluster score recipe of the bench."""
    from sparse_attention_kv_request_amd import workloads
    rng = np.random.default_rng(B)
    lg = workloads.indexer_logits(rng, B, N)
    lens = np.full(B, N, np.int32)
    lens[::3] = rng.integers(2048, N, size=len(lens[::3]))
    run(lg, lens, 2048)
    log(f"topk B={B} N={N}: exact")


def test_k_above_the_staging_limit():
    """k = 5000 (more outputs than the 4096 the kernels stage in LDS): the
    word-by-word output of single-chunk rows and of the merge of split rows."""
    rng = np.random.default_rng(6)
    lg = logits_with_specials(rng, 3, 32768, ties=True)
    run(lg, [32768, 20000, 4999], 5000, mode="paged",
        page_table=rng.permutation(3 * 512).astype(np.int32).reshape(3, 512), page_size=64)
    lg = logits_with_specials(rng, 2, 4 * 32768)
    run(lg, [4 * 32768, 3 * 32768 + 7], 5000, mode="ragged", row_offsets=[0, 4 * 32768])


def _random_topk_case(case):
    """Case `case` of a seeded sweep: rows, row length (1 to 131072, so
    single-chunk and split rows), k within the candidate limit, table mode,
    page size, ties, a rejected row, an unmapped page, one or two layers."""
    rng = np.random.default_rng([20261207, case])
    B = int(rng.integers(1, 41))
    N = int(rng.choice([1, 7, 100, 1000, 4096, 32767, 32768, 32769, 70000, 131072]))
    chunks = -(-N // 32768)
    k = int(rng.integers(1, min(4096, 32768 // chunks) + 1))
    mode = str(rng.choice(["none", "paged", "ragged"]))
    return dict(B=B, N=N, k=k, mode=mode, P=int(rng.choice([16, 64])), ties=bool(rng.random() < 0.3),
                reject=bool(rng.random() < 0.2), holes=bool(rng.random() < 0.3),
                layers=int(rng.integers(1, 3)))


@pytest.mark.parametrize("case", range(40))
def test_random_shapes(case):
    c = _random_topk_case(case)
    log(f"topk random case {case}: {c}")
    rng = np.random.default_rng([10, case])
    B, N, k = c["B"], c["N"], c["k"]
    lg = logits_with_specials(rng, B, N, ties=c["ties"])
    lens = rng.integers(0, N + 1, B)
    lens[rng.random(B) < 0.4] = N
    if c["reject"] and B > 1:
        lens[0] = -1 if rng.random() < 0.5 else N + 1
    kw = {}
    if c["mode"] == "paged":
        npg = -(-N // c["P"])
        pt = rng.permutation(B * npg).astype(np.int32).reshape(B, npg)
        if c["holes"]:
            pt[rng.integers(0, B), rng.integers(0, npg)] = -1
        kw = dict(mode="paged", page_table=pt, page_size=c["P"])
    elif c["mode"] == "ragged":
        kw = dict(mode="ragged",
                  row_offsets=np.cumsum(np.r_[0, np.maximum(lens[:-1], 0)]).astype(np.int32))
    run(lg, lens, k, layers=c["layers"], **kw)


def test_rejects_bad_arguments():
    with pytest.raises(binding.HiSparseError) as e:
        binding.TopkIndexBuilder(4, 17 * 32768, 2048, device=DEV)  # 17 chunks x 2048 > 32768
    assert e.value.code == binding.HISPARSE_E_UNSUPPORTED
    b = binding.TopkIndexBuilder(2, 70000, 4096, device=DEV)   # 3 chunks x 4096 <= 32768: ok
    idx = torch.empty((2, 4096), dtype=torch.int32, device=DEV)
    lg = torch.zeros((2, 70000), dtype=torch.float32, device=DEV)
    sl = torch.full((2,), 70000, dtype=torch.int32, device=DEV)
    b.plan(sl)
    with pytest.raises(binding.HiSparseError) as e:
        b.build(lg, sl, idx, None, mode="paged")               # paged without a table
    assert e.value.code == binding.HISPARSE_E_INVAL


def test_plan_made_for_other_sizes_is_rejected():
    """A plan built for other sizes: its entries outside this call's batch,
    row length or plan, and split rows without a candidate workspace, raise
    ERR_BAD_PLAN on the device and read nothing outside the buffers."""
    rng = np.random.default_rng(11)
    # (a) a plan of 4 rows x 100000 handed to 2 rows x 1000 (no workspace)
    log("topk plan for other sizes: 4x100000 plan, 2x1000 call")
    big = binding.TopkIndexBuilder(4, 100000, 16, device=DEV)
    big.plan(torch.full((4,), 100000, dtype=torch.int32, device=DEV))
    small = binding.TopkIndexBuilder(2, 1000, 16, device=DEV)
    small.plan_buf = big.plan_buf
    lg = torch.from_numpy(rng.standard_normal((2, 1000)).astype(np.float32)).to(DEV)
    idx = torch.empty((2, 16), dtype=torch.int32, device=DEV)
    small.build(lg, torch.full((2,), 1000, dtype=torch.int32, device=DEV), idx)
    torch.cuda.synchronize()
    assert small.error_flags() & binding.ERR_BAD_PLAN
    # (b) a plan of 2 rows x 100000 (4 chunks each) handed to 2 rows x 40000
    # (2 chunks each): chunks past the row length and the second row's merge
    # entry are rejected
    log("topk plan for other sizes: 2x100000 plan, 2x40000 call")
    big = binding.TopkIndexBuilder(2, 100000, 16, device=DEV)
    big.plan(torch.full((2,), 100000, dtype=torch.int32, device=DEV))
    mid = binding.TopkIndexBuilder(2, 40000, 16, device=DEV)
    mid.plan_buf = big.plan_buf
    lg = torch.from_numpy(rng.standard_normal((2, 40000)).astype(np.float32)).to(DEV)
    idx = torch.empty((2, 16), dtype=torch.int32, device=DEV)
    mid.build(lg, torch.full((2,), 40000, dtype=torch.int32, device=DEV), idx)
    torch.cuda.synchronize()
    assert mid.error_flags() & binding.ERR_BAD_PLAN
    # a plan made for the call's sizes: exact again, no error
    run(lg.cpu().numpy(), [40000, 40000], 16)


@pytest.mark.parametrize("N,k", [(70000, 2000), (3 * 32768 + 100, 3000), (8 * 32768, 4000)])
def test_merge_slot_counts(N, k):
    """Split rows whose most candidates per row (chunks x k: 6000, 12000,
    32000) take the merge's 8, 16 and 32 slots per thread; rows of every
    chunk count up to the longest, ties across chunks."""
    rng = np.random.default_rng(N + k)
    lg = logits_with_specials(rng, 3, N, ties=True)
    log(f"topk merge slots: N={N} k={k}")
    run(lg, [N, N // 2 + 1, 32769], k, mode="ragged", row_offsets=[0, N, 2 * N])
