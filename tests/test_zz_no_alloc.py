"""hisparse_topk_index_build_noalloc (the library's fixed scratch) against
hisparse_topk_index_build (the caller's workspace), through the C ABI: the
same indices, index table and error bits, on two calls in a row, the second
with a smaller input, and a size beyond the fixed scratch rejected before any
launch."""
import numpy as np
import pytest
import torch

from sparse_attention_kv_request_amd import binding
from tests.gpu_harness import DEV, log

pytestmark = pytest.mark.gpu


def _scores(rng, B, N):
    x = rng.standard_normal((B, N)).astype(np.float32)
    flat = x.reshape(-1)
    for v in (np.nan, -np.inf, np.inf, -0.0, 0.0):
        flat[rng.choice(flat.size, max(1, flat.size // 500), replace=False)] = v
    x[:, ::97] = np.round(x[:, ::97])                       # ties across chunks
    return x


def _both(rng, B, N, k, seq_lens, mode):
    """Runs the workspace and the fixed-scratch entry points on the same
    inputs; returns their (indices, locs, error bits)."""
    logits = torch.from_numpy(_scores(rng, B, N)).to(DEV)
    sl = torch.from_numpy(np.asarray(seq_lens, np.int32)).to(DEV)
    pages = (N + 63) // 64
    pt = torch.from_numpy(rng.permutation(B * pages).astype(np.int32).reshape(B, pages)).to(DEV)
    res = []
    for noalloc in (False, True):
        b = binding.TopkIndexBuilder(B, N, k, device=DEV)
        b.plan(sl)
        idx = torch.full((B, k), 12345, dtype=torch.int32, device=DEV)
        locs = torch.full((B, k), 12345, dtype=torch.int32, device=DEV)
        b.build(logits, sl, idx, locs, mode=mode, page_table=pt if mode == "paged" else None,
                page_size=64, row_offsets=sl if mode == "ragged" else None, noalloc=noalloc)
        torch.cuda.synchronize()
        res.append((idx.cpu().numpy(), locs.cpu().numpy(), b.error_flags()))
    return res


def test_noalloc_matches_workspace_entry_point():
    rng = np.random.default_rng(20261203)
    # call 1: 24 rows of up to 131072 scores (four chunks each), k = 2048:
    # 24 x 4 x (8 x 2048 + 4) bytes of candidates in the fixed scratch
    B, N, k = 24, 131072, 2048
    seq = rng.integers(1, N + 1, B)
    seq[:3] = [N, 32769, 40000]
    seq[3] = -1                                              # a rejected row
    need = binding.hisparse_topk_workspace_bytes(B, N, k)
    assert 0 < need <= 16 << 20
    log(f"no-alloc call 1: {B} x {N}, k {k}, {need} bytes of candidates")
    (i0, l0, e0), (i1, l1, e1) = _both(rng, B, N, k, seq, "paged")
    assert np.array_equal(i0, i1) and np.array_equal(l0, l1) and e0 == e1 == 8
    # call 2, smaller: 5 rows of up to 70000 scores, k = 1000; the array keeps
    # call 1's candidates, which call 2 overwrites before reading
    B, N, k = 5, 70000, 1000
    seq = rng.integers(32769, N + 1, B)
    log(f"no-alloc call 2: {B} x {N}, k {k}")
    (i0, l0, e0), (i1, l1, e1) = _both(rng, B, N, k, seq, "ragged")
    assert np.array_equal(i0, i1) and np.array_equal(l0, l1) and e0 == e1 == 0
    assert np.all(i1[:, :k] >= 0)


def test_noalloc_rejects_sizes_beyond_the_fixed_scratch():
    B, N, k = 300, 131072, 2048                              # 300 x 4 x 16388 bytes > 16 MiB
    assert binding.hisparse_topk_workspace_bytes(B, N, k) > 16 << 20
    c = binding.HisparseTopkCall(batch=B, max_len=N, k=k)
    assert binding.hisparse_topk_index_build_noalloc(c, None) == binding.HISPARSE_E_UNSUPPORTED
