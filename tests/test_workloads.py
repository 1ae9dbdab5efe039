"""Seeded input generators: shapes, determinism and recipe properties (no GPU)."""
import numpy as np
import pytest

from sparse_attention_kv_request_amd import workloads as W


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_trace_shape_and_range(cfg):
    w = W.config(cfg)
    tr = W.instance_trace(w, 3, 0)
    assert tr.shape == (w.steps, w.num_steps, w.top_k) and tr.dtype == np.int32
    assert tr.min() >= 0 and tr.max() < w.seq_len
    for call in tr:
        for row in call:
            assert np.unique(row).size == row.size          # rows hold distinct tokens
    assert np.array_equal(tr, W.instance_trace(w, 3, 0))    # seeded
    assert not np.array_equal(tr, W.instance_trace(w, 4, 0))


def test_recipe_properties():
    w1 = W.config(1)
    tr = W.instance_trace(w1, 0, 0)[:, 0]
    for row in tr:
        assert set(range(w1.seq_len - w1.window, w1.seq_len)) <= set(row.tolist())
    w2 = W.config(2)
    tr = W.instance_trace(w2, 0, 0)[:, 0]
    for a, b in zip(tr[:-1], tr[1:]):
        assert len(set(a.tolist()) & set(b.tolist())) >= round(0.7 * w2.top_k)
    assert np.median(tr) > w2.seq_len * 0.5                   # recency bias
    w3 = W.config(3)
    tr = W.instance_trace(w3, 0, 0)
    core = round(0.8 * w3.top_k)
    for call in tr:
        common = set(call[0].tolist())
        for row in call[1:]:
            common &= set(row.tolist())
        assert len(common) >= core
    w5 = W.config(5)
    tr = W.instance_trace(w5, 0, 0)[:, 0]
    assert max(np.unique(row // w5.page_size).size for row in tr) <= 56 < w5.hot


def test_kv_bytes():
    w = W.config(2, seq_len=64)
    a = W.instance_kv(w, 1, 2)
    assert a.shape == (64, 656) and a.dtype == np.uint8
    assert np.array_equal(a, W.instance_kv(w, 1, 2))
    assert not np.array_equal(a, W.instance_kv(w, 1, 3))
    w1 = W.config(1, seq_len=32)
    b = W.instance_kv(w1, 0, 0).view(np.uint16).astype(np.uint32) << 16
    vals = b.view(np.float32)
    assert abs(float(vals.mean())) < 0.1 and 0.9 < float(vals.std()) < 1.1
