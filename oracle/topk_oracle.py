"""CPU oracle of the top-k selection and index-table build that feed the
swap-in path.  TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke()
and the CPU-baseline leg of bench.py may import it.

What it computes ("SGLang HiSparse" blog, section 2.2: a planning step that
takes only the per-row sequence lengths and returns a plan reused by every
layer of a decode step, and a fused kernel that selects each row's top-k from
the indexer's scores and builds the index table in the same pass; section
2.3: in PAGED mode a selected token is located through the page table by its
page and in-page offset, in RAGGED mode by an offset into one contiguous
buffer; section 1.1: the indexer scores every position and keeps the top-k).

Readings (the pages give neither the selection rule's details nor the plan's
contents):

T1  The candidates of row b are the positions [0, seq_len_b); seq_len_b = 0
    selects nothing.  A row with seq_len_b < 0 or above the logits row length
    is rejected: its outputs are -1 and the bad-row error bit is set.
T2  The top-k is the min(k, seq_len_b) positions with the largest scores;
    among equal scores the lower position wins.  NaN counts as lower than
    every number, -inf included (so the selection is a total order).
T3  Output order: the selected positions in ascending order, then -1 up to k
    (an index table, not a ranking).
T4  Index table: PAGED  loc = page_table[b][p // P] * P + p % P, -1 stays -1;
    a position whose page entry is negative or beyond the table gives -1 and
    the bad-index error bit.  RAGGED  loc = row_offset[b] + p.
T5  The plan splits row b into n_b = max(1, ceil(seq_len_b / 32768))
    chunks (32768 positions is the threshold above which a row is shared by
    several workgroups) of length L_b = 1024 * ceil(ceil(seq_len_b / n_b) / 1024) (the
    last one shorter); a row outside [0, N] (N = the logits row length) gets
    one empty chunk.  It lists, per row, its first work item and n_b, and per
    work item (row, chunk, start, length).  The plan depends on the sequence
    lengths only, so one plan serves every layer of a step.

Every function is pinned by tests/test_topk_oracle.py (brute force over all
tiny inputs against a characterisation of T2, torch.topk on distinct scores,
closed forms, planted mistakes).
"""
from __future__ import annotations

import numpy as np

ERR_BAD_INDEX = 1
ERR_BAD_ROW = 8
SPLIT = 32768          # T5: positions above which a row is split
CHUNK_ALIGN = 1024


def selection_order(values: np.ndarray) -> np.ndarray:
    """Positions 0..n-1 in selection order (T2): score descending, NaN last,
    ties by ascending position."""
    v = np.asarray(values, dtype=np.float32)
    nan = np.isnan(v)
    score = np.where(nan, 0.0, v).astype(np.float64)
    pos = np.arange(v.size)
    # lexsort: last key is primary
    return np.lexsort((pos, -score, nan))


def topk_row(values: np.ndarray, seq_len: int, k: int) -> np.ndarray:
    """T1-T3 for one row: int32 [k] ascending selected positions, -1 padded."""
    out = np.full(k, -1, dtype=np.int32)
    n = max(0, int(seq_len))
    if n == 0 or k == 0:
        return out
    chosen = selection_order(values[:n])[:k]
    sel = np.sort(chosen)
    out[:sel.size] = sel
    return out


def paged_locs(indices: np.ndarray, page_table: np.ndarray, page_size: int):
    """T4 PAGED for one row: (locs int32 [k], error bits)."""
    locs = np.full(indices.shape, -1, dtype=np.int32)
    err = 0
    for i, p in enumerate(indices):
        if p < 0:
            continue
        j, off = divmod(int(p), page_size)
        if j >= page_table.size or page_table[j] < 0:
            err |= ERR_BAD_INDEX
            continue
        locs[i] = int(page_table[j]) * page_size + off
    return locs, err


def ragged_locs(indices: np.ndarray, row_offset: int) -> np.ndarray:
    """T4 RAGGED for one row."""
    return np.where(indices >= 0, indices + int(row_offset), -1).astype(np.int32)


def topk_index_build(logits: np.ndarray, seq_lens: np.ndarray, k: int, *, mode: str = "none",
                     page_table: np.ndarray | None = None, page_size: int = 1,
                     row_offsets: np.ndarray | None = None):
    """All rows: logits float32 [B, N].  Returns (indices [B, k], locs [B, k]
    or None, error bits)."""
    B, N = logits.shape
    idx = np.full((B, k), -1, dtype=np.int32)
    locs = None if mode == "none" else np.full((B, k), -1, dtype=np.int32)
    err = 0
    for b in range(B):
        s = int(seq_lens[b])
        if s < 0 or s > N:
            err |= ERR_BAD_ROW
            continue
        idx[b] = topk_row(logits[b], s, k)
        if mode == "paged":
            locs[b], e = paged_locs(idx[b], page_table[b], page_size)
            err |= e
        elif mode == "ragged":
            locs[b] = ragged_locs(idx[b], row_offsets[b])
    return idx, locs, err


def plan(seq_lens: np.ndarray, max_len: int):
    """T5: (row_info int32 [B, 2] = (first item, n_chunks), items int32
    [n_items, 4] = (row, chunk, start, length))."""
    row_info = np.zeros((len(seq_lens), 2), dtype=np.int32)
    items = []
    for b, s in enumerate(int(x) for x in seq_lens):
        s = s if 0 <= s <= max_len else 0
        n = max(1, -(-s // SPLIT))
        length = CHUNK_ALIGN * (-(-(-(-s // n)) // CHUNK_ALIGN))
        row_info[b] = (len(items), n)
        for c in range(n):
            start = c * length
            items.append((b, c, start, max(0, min(length, s - start))))
    return row_info, np.array(items, dtype=np.int32).reshape(-1, 4)
