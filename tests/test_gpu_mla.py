"""Sparse MLA decode attention (HIP, through the C ABI) against the float64
oracle, on rows that a swap call placed in the hot buffer.

The reference attends over the values the kernel computes
with (bf16 keys and values; fp8 rows dequantised in float32 and rounded to
bf16), and every output element and lse is held to the bound of
``tests/mla_check.py``: the kernel's float32 accumulation, bf16 softmax
weights, fp16 split outputs and log-sum-exp merge, per (row, head) and per
element (sum_i w_i |c_id| terms).  ``tests/test_mla_checker.py`` shows on
the CPU that the bound rejects a zeroed or doubled output, swapped heads and
a dropped location or tile.
"""
import numpy as np
import pytest
import torch

from oracle import sparse_mla_oracle as mla
from sparse_attention_kv_request_amd import binding, workloads
from tests import mla_check
from tests.gpu_harness import DEV, log

pytestmark = pytest.mark.gpu


def boost_rows(host, item, req_row, tokens, factor):
    """Multiplies the latent of the given host rows by `factor` (bf16 rows:
    re-rounded to bf16; fp8 rows: through their four scales, exactly)."""
    rows = host.array[req_row]
    for t in tokens:
        if item == mla.BF16_ROW:
            v = rows[t].view(np.uint16)[:mla.LATENT].astype(np.uint32) << 16
            f = v.view(np.float32) * np.float32(factor)
            rows[t].view(np.uint16)[:mla.LATENT] = (f.view(np.uint32) >> 16).astype(np.uint16)
        else:
            sc = rows[t, mla.LATENT:mla.LATENT + 16].view(np.float32)
            sc *= np.float32(factor)


def run_case(*, R, B, H, K, N, item, heads, P=1, seed=0, pad_row=None, calls=2, boost=None,
             check_rows=None):
    """One state, `calls` swap + decode calls; every batch row (or the
    `check_rows` sample) is compared with the oracle."""
    rng = np.random.default_rng(seed)
    host = binding.HostKV(R, N, item)
    for r in range(R):
        host.array[r] = workloads.mla_kv_rows(rng, N, item)
    st = binding.HiSparseState(max_requests=R, num_layers=1, hot_buffer_size=H, top_k=K,
                               item_size_bytes=item, max_seq_len=N, page_size=P,
                               host_kv=[host])
    scale = mla.default_scale()
    worst = 0.0
    try:
        for call in range(calls):
            req = rng.permutation(R)[:B].astype(np.int32)
            span = N if P == 1 else min(N, H * P)             # page mode: fits the hot pages
            topk = np.stack([rng.choice(span, K, replace=False) for _ in range(B)]).astype(np.int32)
            topk[:, ::7] = -1                                 # padding entries
            topk[:, 1] = topk[:, 2]                           # a duplicate entry
            if pad_row is not None:
                topk[pad_row] = -1
            for b, pos, factor in boost or ():
                boost_rows(host, item, req[b], [topk[b, pos]], factor)
            out_locs = torch.empty((B, K), dtype=torch.int32, device=DEV)
            mc = torch.empty(B, dtype=torch.int32, device=DEV)
            pt = nump = None
            if P > 1:
                pt = torch.empty((B, H), dtype=torch.int32, device=DEV)
                nump = torch.empty(B, dtype=torch.int32, device=DEV)
            t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
            st.swap_in_selected(0, t(req), t(np.full(B, N, np.int32)), t(topk), out_locs, mc,
                                page_table=pt, num_pages=nump)
            q_bits = workloads.mla_queries(rng, B, heads)
            q = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
            out = torch.full((B, heads, 512), float("nan"), dtype=torch.float32, device=DEV)
            lse = torch.full((B, heads), float("nan"), dtype=torch.float32, device=DEV)
            st.sparse_mla_decode(0, q, out_locs, out, lse, page_table=pt, softmax_scale=scale)
            torch.cuda.synchronize()
            assert st.error_flags() == 0
            # the oracle reads the host tier by token: row r*N + t
            locs_host = np.where(topk >= 0, req[:, None].astype(np.int64) * N + topk, -1)
            host_rows = host.array.reshape(R * N, item)
            got_out = out.cpu().numpy().astype(np.float64)
            got_lse = lse.cpu().numpy().astype(np.float64)
            if check_rows is not None:
                q_bits, locs_host = q_bits[check_rows], locs_host[check_rows]
                got_out, got_lse = got_out[check_rows], got_lse[check_rows]
            ref = mla_check.reference(q_bits, locs_host, host_rows, scale)
            ok, ratio, report = mla_check.check(got_out, got_lse, ref)
            assert ok, report
            if pad_row is not None:
                assert np.all(got_out[pad_row] == 0) and np.all(np.isneginf(got_lse[pad_row]))
            for b, pos, factor in boost or ():
                # the boosted row's score exceeds every unboosted score of its
                # batch row (so the first tile of its split) by far more than
                # the weights' 2^64 headroom, for some head
                keep = locs_host[b] >= 0
                lat, rope = mla.decode_rows(host_rows[locs_host[b][keep]])
                qd = mla.bf16_to_f64(q_bits[b])
                sc = scale * (qd[:, :512] @ lat.T + qd[:, 512:] @ rope.T) / np.log(2)
                boosted = {int(np.count_nonzero(keep[:pp])) for bb, pp, _ in boost if bb == b}
                plain = [i for i in range(sc.shape[1]) if i not in boosted]
                i_big = int(np.count_nonzero(keep[:pos]))
                assert (sc[:, i_big] - sc[:, plain].max(axis=1)).max() > 64
            worst = max(worst, ratio)
        log(f"mla item={item} P={P} heads={heads} B={B} K={K}: worst error / bound = {worst:.3g}")
    finally:
        st.close()
        host.free()


@pytest.mark.parametrize("item", [1152, 656])
def test_mla_token_rows_many_splits(item):
    """Small batch: the location list is split over many workgroups and merged."""
    run_case(R=3, B=2, H=2048, K=1000, N=4000, item=item, heads=128, seed=item, pad_row=1)


@pytest.mark.parametrize("item", [1152, 656])
def test_mla_token_rows_large_batch(item):
    run_case(R=40, B=40, H=600, K=300, N=1500, item=item, heads=64, seed=item + 1, calls=1)


@pytest.mark.parametrize("heads,B,K", [(200, 5, 300), (256, 2, 1000), (384, 3, 130)])
def test_mla_several_head_groups(heads, B, K):
    """More than 128 heads: several head groups per row (the last one partial
    for 200), split and unsplit rows."""
    run_case(R=B + 1, B=B, H=max(K, 256), K=K, N=K + 300, item=1152, heads=heads, seed=heads + B)


def test_mla_long_location_lists():
    """8000 locations per row over 128 rows: the split count comes from the
    2048-location cap per workgroup (4 splits of 2000, not the 2 that fill the
    CUs); sampled rows against the oracle."""
    run_case(R=128, B=128, H=8192, K=8000, N=8300, item=1152, heads=16, seed=8000, calls=1,
             check_rows=[0, 77, 127])


def test_mla_ragged_heads_and_locations():
    """Heads not a multiple of 16 and a location count not a multiple of 32."""
    run_case(R=4, B=3, H=128, K=77, N=500, item=1152, heads=24, seed=5)


@pytest.mark.parametrize("item", [1152, 656])
def test_mla_page_mode(item):
    run_case(R=3, B=3, H=40, K=200, N=16 * 64, item=item, heads=32, P=16, seed=item + 2)


def test_mla_page_mode_full_location_table():
    """2048 locations per row through the page table (64-token pages, 32 hot
    pages): every page-table lookup of a workgroup's location range."""
    run_case(R=4, B=4, H=32, K=2048, N=4096, item=1152, heads=64, P=64, seed=64)


@pytest.mark.parametrize("item", [1152, 656])
def test_mla_replay_after_large_score_jump(item):
    """Rows far above the first tile's scores (latent x2000, then x5000) in
    later tiles of a split: the split restarts with a raised reference."""
    run_case(R=64, B=64, H=400, K=300, N=1200, item=item, heads=128, seed=item + 3, calls=1,
             boost=[(0, 50, 2000.0), (0, 80, 5000.0), (7, 230, 3000.0)])


@pytest.mark.parametrize("item", [1152, 656])
def test_mla_replay_requested_by_the_last_tile(item):
    """The only large score of a split sits in its last tile (a full tile,
    and a partial one): the request is read after the range ends and the
    split still replays."""
    run_case(R=64, B=64, H=400, K=300, N=1200, item=item, heads=128, seed=item + 5, calls=1,
             boost=[(0, 80, 5000.0)])
    run_case(R=64, B=64, H=400, K=280, N=1200, item=item, heads=128, seed=item + 6, calls=1,
             boost=[(3, 270, 5000.0)])


@pytest.mark.parametrize("item", [1152, 656])
def test_mla_replay_in_two_tile_splits(item):
    """Splits of two tiles (64 rows x 256 locations: four splits of 64) with
    the large score in the second and last tile of three of them: the
    replay starts while the tiles past the range are still in flight."""
    run_case(R=64, B=64, H=400, K=256, N=1200, item=item, heads=128, seed=item + 13, calls=1,
             boost=[(0, 40, 5000.0), (0, 97, 3000.0), (0, 255, 4000.0)])


@pytest.mark.parametrize("item", [1152, 656])
def test_mla_split_outputs_beyond_fp16_range(item):
    """Split outputs far above fp16's largest finite value (65504): rows
    whose latent is multiplied by 5e4 to 2e5 dominate the heads of their
    batch rows, so those heads' outputs (and split partials) reach 1e5 and
    more.  The per-(split, head) power-of-two scaling of the fp16 partials
    keeps them finite and within the bound."""
    run_case(R=64, B=64, H=400, K=300, N=1200, item=item, heads=128, seed=item + 17, calls=1,
             boost=[(0, 50, 1e5), (3, 100, 2e5), (7, 250, 5e4)])


def _random_case(case):
    """Case `case` of a seeded sweep over batch, heads, location count, hot
    size and boosted rows (which force replays at varied tiles), alternating
    bf16 and fp8 rows."""
    rng = np.random.default_rng([20261203, case])
    item = [1152, 656][case % 2]
    B = int(rng.choice([1, 2, 3, 8, 17, 64]))
    heads = int(rng.choice([16, 48, 128]))
    K = int(rng.integers(3, 700))
    N = int(K + rng.integers(0, 800))
    H = int(K + rng.integers(0, 200))
    R = B + int(rng.integers(0, 3))
    boost = []
    if K > 40 and rng.random() < 0.6:
        for _ in range(int(rng.integers(1, 3))):
            pos = int(rng.integers(3, K))
            while pos % 7 == 0:                               # padding positions
                pos += 1
            if pos < K:
                boost.append((int(rng.integers(0, B)), pos, float(rng.choice([3000.0, 6000.0]))))
    return dict(R=R, B=B, H=H, K=K, N=N, item=item, heads=heads, seed=2000 + case, calls=1,
                boost=boost or None)


@pytest.mark.parametrize("case", range(24))
def test_mla_random_shapes(case):
    """Seeded random shapes, split counts and replays, against the oracle."""
    kw = _random_case(case)
    log(f"mla random case {case}: {kw}")
    run_case(**kw)


@pytest.mark.parametrize("item", [1152, 656])
def test_mla_unsplit_rows(item):
    """256 rows: one workgroup per row and head group already fills the
    chip, so the locations are not split (outputs written directly)."""
    run_case(R=256, B=256, H=300, K=200, N=600, item=item, heads=16, seed=item + 11, calls=1)


@pytest.mark.parametrize("item", [1152, 656])
def test_mla_bench_shape(item):
    """The bench's launch shape: 64 rows x 128 heads x 2048 locations (four
    splits of 512 per row), rows placed by a swap call; every row against the
    oracle."""
    run_case(R=64, B=64, H=4096, K=2048, N=8192, item=item, heads=128, seed=item + 9, calls=1)


def test_mla_rejects_bad_arguments():
    host = binding.HostKV(2, 64, 48)
    st = binding.HiSparseState(max_requests=2, num_layers=1, hot_buffer_size=64, top_k=8,
                               item_size_bytes=48, max_seq_len=64, host_kv=[host])
    try:
        q = torch.zeros((1, 16, 576), dtype=torch.bfloat16, device=DEV)
        locs = torch.zeros((1, 8), dtype=torch.int32, device=DEV)
        out = torch.zeros((1, 16, 512), dtype=torch.float32, device=DEV)
        with pytest.raises(binding.HiSparseError) as e:
            st.sparse_mla_decode(0, q, locs, out)              # 48-byte rows: no MLA layout
        assert e.value.code == binding.HISPARSE_E_UNSUPPORTED
        for bad_scale in (0.0, -0.5, float("inf"), float("nan")):
            rc = binding.hisparse_sparse_mla_decode(st.handle, 0, 1, 16, 8, q.data_ptr(),
                                                    locs.data_ptr(), None, bad_scale,
                                                    out.data_ptr(), None, None, 0, None)
            assert rc == binding.HISPARSE_E_INVAL
    finally:
        st.close()
        host.free()
