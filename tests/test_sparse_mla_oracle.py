"""Pins of the sparse MLA decode-attention oracle (no GPU).

The decoders are checked against torch's own bfloat16 and float8_e4m3fn
conversions over every code, the attention against torch's float64
scaled_dot_product_attention, and the whole call against closed forms.
"""
import math

import numpy as np
import pytest
import torch

from oracle import sparse_mla_oracle as mla
from sparse_attention_kv_request_amd import workloads as W


def test_e4m3fn_decoder_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = mla.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_bf16_decoder_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, 4096, dtype=np.uint64).astype(np.uint16)
    ours = mla.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_fp8_row_layout_closed_form():
    row = np.zeros((1, mla.FP8_ROW), np.uint8)
    row[0, :512] = 0x38                                # 1.0 in e4m3fn
    row[0, 512:528] = np.array([2.0, 0.5, -1.0, 4.0], np.float32).view(np.uint8)
    row[0, 528:] = np.full(64, 0x3F80, np.uint16).view(np.uint8)   # bf16 1.0
    lat, rope = mla.decode_rows(row)
    assert np.array_equal(lat[0], np.repeat([2.0, 0.5, -1.0, 4.0], 128))
    assert np.array_equal(rope[0], np.ones(64))


@pytest.mark.parametrize("item", [mla.BF16_ROW, mla.FP8_ROW])
def test_attention_matches_torch_sdpa_float64(item):
    rng = np.random.default_rng(item)
    H, n = 16, 37
    rows = W.mla_kv_rows(rng, n, item)
    q = mla.bf16_to_f64(W.mla_queries(rng, 1, H)[0])
    lat, rope = mla.decode_rows(rows)
    scale = 0.07
    out, lse = mla.attend(q, lat, rope, scale)
    k = torch.from_numpy(np.concatenate([lat, rope], 1))[None, None]      # [1,1,n,576]
    v = torch.from_numpy(lat)[None, None]
    qq = torch.from_numpy(q)[None, :, None]                                # [1,H,1,576]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qq, k.expand(1, H, n, 576), v.expand(1, H, n, 512), scale=scale)[0, :, 0]
    assert np.allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)
    s = scale * (q @ np.concatenate([lat, rope], 1).T)
    ref_lse = torch.logsumexp(torch.from_numpy(s), dim=1).numpy()
    assert np.allclose(lse, ref_lse, rtol=1e-13, atol=1e-13)


def test_closed_forms_and_masking():
    rng = np.random.default_rng(3)
    H, item = 4, mla.BF16_ROW
    rows = W.mla_kv_rows(rng, 10, item)
    q_bits = W.mla_queries(rng, 3, H)
    scale = mla.default_scale()
    lat, rope = mla.decode_rows(rows)
    # one valid entry: the output is that row's latent, lse its score
    locs = np.array([[-1, 4, -1], [2, 2, 2], [-1, -1, -1]])
    out, lse = mla.sparse_mla_decode(q_bits, locs, rows, scale)
    q0 = mla.bf16_to_f64(q_bits[0])
    assert np.allclose(out[0], np.tile(lat[4], (H, 1)), rtol=0, atol=1e-12)
    assert np.allclose(lse[0], scale * (q0 @ np.concatenate([lat[4], rope[4]])), atol=1e-12)
    # the same row three times: output is the row, lse gains log 3
    q1 = mla.bf16_to_f64(q_bits[1])
    assert np.allclose(out[1], np.tile(lat[2], (H, 1)), atol=1e-12)
    assert np.allclose(lse[1], scale * (q1 @ np.concatenate([lat[2], rope[2]])) + math.log(3),
                       atol=1e-12)
    # no valid entry
    assert np.all(out[2] == 0) and np.all(lse[2] == -np.inf)
    # permutation of the list and inserted padding change nothing
    base = np.array([[0, 5, 7, 9, 1]])
    perm = np.array([[9, -1, 1, 7, -1, 0, 5]])
    a = mla.sparse_mla_decode(q_bits[:1], base, rows, scale)
    b = mla.sparse_mla_decode(q_bits[:1], perm, rows, scale)
    assert np.allclose(a[0], b[0], atol=1e-12) and np.allclose(a[1], b[1], atol=1e-12)


def test_equal_scores_average_the_values():
    """A query orthogonal to every key gives equal scores: the mean latent."""
    rng = np.random.default_rng(4)
    rows = W.mla_kv_rows(rng, 6, mla.BF16_ROW)
    lat, rope = mla.decode_rows(rows)
    q = np.zeros((2, 576))
    out, lse = mla.attend(q, lat, rope, 0.5)
    assert np.allclose(out, np.tile(lat.mean(0), (2, 1)), atol=1e-12)
    assert np.allclose(lse, math.log(6), atol=1e-12)


def test_f32_to_bf16_rne_matches_torch():
    """The oracle's float32 -> bfloat16 rounding against torch's conversion
    (round to nearest, ties to even) over random values of every magnitude,
    exact ties (odd and even kept parts), subnormals, the largest finite
    values, infinities and NaN."""
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    hi = rng.integers(0, 2 ** 16, 4000, dtype=np.uint64) << np.uint64(16)
    ties = (hi | np.uint64(0x8000)).astype(np.uint32)
    low = rng.choice(np.array([0x7FFF, 0x8001, 0x0001, 0xFFFF], np.uint64), 4000)
    near = (hi | low).astype(np.uint32)
    special = np.array([0, 0x80000000, 0x00000001, 0x007FFFFF, 0x7F7FFFFF, 0xFF7FFFFF,
                        0x7F7F8000, 0x7F800000, 0xFF800000, 0x7FC00000], np.uint32)
    x = np.concatenate([bits, ties, near, special]).view(np.float32)
    got = mla.f32_to_bf16_rne(x)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    both_nan = np.isnan(got) & np.isnan(want)
    assert np.array_equal(got[~both_nan], want[~both_nan])
    assert np.array_equal(np.isnan(got), np.isnan(want))


def test_bf16_reading_of_fp8_rows_matches_torch():
    """The bf16 value of an fp8 row's latent: code value x float32 scale as one float32
    product, then bfloat16 -- against torch's float8_e4m3fn decoding and
    conversions, over every code and scales of many magnitudes."""
    rng = np.random.default_rng(4)
    n = 64
    rows = np.empty((n, mla.FP8_ROW), np.uint8)
    rows[:, :mla.LATENT] = np.tile(np.arange(256, dtype=np.uint8), 2)[None]
    rows[:, :mla.LATENT] = rng.permuted(rows[:, :mla.LATENT], axis=1)
    rows[:, :mla.LATENT][rows[:, :mla.LATENT] & 0x7F == 0x7F] = 0   # no NaN codes
    scales = (rng.random((n, 4)) * np.exp2(rng.integers(-20, 20, (n, 4)))).astype(np.float32)
    rows[:, mla.LATENT:mla.LATENT + 16] = scales.view(np.uint8).reshape(n, 16)
    rows[:, mla.LATENT + 16:] = rng.integers(0, 256, (n, 128), dtype=np.uint8)
    lat, rope = mla.decode_rows_bf16(rows)
    codes = torch.from_numpy(np.ascontiguousarray(rows[:, :mla.LATENT])).view(torch.float8_e4m3fn)
    prod = codes.to(torch.float32) * torch.from_numpy(np.repeat(scales, 128, axis=1))
    want = prod.to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(lat, want)
    _, rope_exact = mla.decode_rows(rows)
    assert np.array_equal(rope, rope_exact, equal_nan=True)
    # bf16 rows are read as stored
    b16 = rng.integers(0, 256, (8, mla.BF16_ROW), dtype=np.uint8)
    for u, v in zip(mla.decode_rows_bf16(b16), mla.decode_rows(b16)):
        assert np.array_equal(u, v, equal_nan=True)
