"""CPU oracle of sparse MLA decode attention over swapped-in rows.
TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py may import it.

What it computes ("SGLang HiSparse" blog, section 1 opening and sections
1.1-1.2: attention is exact over the top-k positions the indexer selected;
section 2.1: the sparse table a swap-in call returns goes straight to decode
attention).  For every batch row b and head h, with S(b) the valid entries of
the row's location list (a location of -1 is skipped):

    s_i   = scale * (q[b, h, :512] . c_i + q[b, h, 512:] . r_i)    i in S(b)
    out   = sum_i softmax(s)_i * c_i                                (512 dims)
    lse   = log sum_i exp(s_i)                                      (natural log)

c_i is the 512-dim latent of the KV row (it is both key and value) and r_i
its 64-dim rope key: the absorbed-MLA decode form.  Rows with no valid entry
give out = 0 and lse = -inf.  Everything is evaluated in float64 from the
exact values the stored bytes encode.

KV row layouts (the item bytes a swap call copies):

* 1152 B: 576 bfloat16 values (latent then rope);
* 656 B: 512 OCP fp8 e4m3fn latent values, 4 float32 scales (one per
  128-dim tile of the latent), 64 bfloat16 rope values.

These layouts and the 576/512/64 split are readings (the pages name neither).
The kernel computes with bf16 keys and values: fp8 rows are
dequantised by one float32 product per value and rounded to bf16;
``decode_rows_bf16`` gives those values, and the GPU parity tests attend over
them so that their tolerance covers only the kernel's accumulation and
softmax roundings.  "Parity unpinned" does not apply: every function below is
pinned by tests/test_sparse_mla_oracle.py against library decoders and
conversions, a library attention routine and closed forms.
"""
from __future__ import annotations

import math

import numpy as np

LATENT = 512
ROPE = 64
QK_DIM = LATENT + ROPE
BF16_ROW = 2 * QK_DIM          # 1152
FP8_ROW = LATENT + 16 + 2 * ROPE  # 656
FP8_TILE = 128


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64: the upper half of a float32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 (fn) codes -> float64, from the format definition:
    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, subnormals at
    exponent 0, no infinities, S.1111.111 is NaN."""
    c = codes.astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = sign * (1.0 + man / 8.0) * np.exp2(exp - 7.0)
    sub = sign * (man / 8.0) * 2.0 ** -6
    val = np.where(exp == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 values -> the nearest bfloat16 value (ties to the even
    significand), returned as float64.  From the format: bfloat16 is the upper
    16 bits of a float32, so rounding drops the low 16 bits, adding one unit
    of the kept part when they exceed half of it, or equal half of it and the
    kept part is odd.  Overflow rounds to infinity; NaN stays NaN."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    keep = u >> 16
    up = (low > 0x8000) | ((low == 0x8000) & ((keep & 1) == 1))
    r = ((keep + up.astype(np.uint64)) << 16).astype(np.uint32).view(np.float32)
    r = np.where(np.isnan(np.asarray(x, np.float32)), np.float32(np.nan), r)
    return r.astype(np.float64)


def decode_rows_bf16(rows: np.ndarray):
    """The values attention computes with: bf16 rows as stored;
    fp8 rows dequantised as one float32 product (code value x the tile's
    float32 scale, rounded to nearest even) and then rounded to bfloat16.
    Returns (latent [n, 512], rope [n, 64]) float64."""
    n, item = rows.shape
    if item == BF16_ROW:
        return decode_rows(rows)
    if item == FP8_ROW:
        codes = e4m3fn_to_f64(rows[:, :LATENT]).astype(np.float32)      # exact in float32
        scales = np.ascontiguousarray(rows[:, LATENT:LATENT + 16]).view(np.float32)
        prod = codes * np.repeat(scales, FP8_TILE, axis=1)               # float32 product
        rope = bf16_to_f64(np.ascontiguousarray(rows[:, LATENT + 16:]).view(np.uint16))
        return f32_to_bf16_rne(prod), rope
    raise ValueError(f"unsupported KV row of {item} bytes")


def decode_rows(rows: np.ndarray):
    """uint8 [n, item] KV rows -> (latent [n, 512], rope [n, 64]) float64."""
    n, item = rows.shape
    if item == BF16_ROW:
        vals = bf16_to_f64(np.ascontiguousarray(rows).view(np.uint16))
        return vals[:, :LATENT], vals[:, LATENT:]
    if item == FP8_ROW:
        lat = e4m3fn_to_f64(rows[:, :LATENT])
        scales = np.ascontiguousarray(rows[:, LATENT:LATENT + 16]).view(np.float32).astype(np.float64)
        lat = lat * np.repeat(scales, FP8_TILE, axis=1)
        rope = bf16_to_f64(np.ascontiguousarray(rows[:, LATENT + 16:]).view(np.uint16))
        return lat, rope
    raise ValueError(f"unsupported KV row of {item} bytes")


def attend(q: np.ndarray, latent: np.ndarray, rope: np.ndarray, scale: float):
    """Exact attention of heads q [H, 576] over n rows; returns (out [H, 512], lse [H])."""
    H = q.shape[0]
    if latent.shape[0] == 0:
        return np.zeros((H, LATENT)), np.full(H, -np.inf)
    s = scale * (q[:, :LATENT] @ latent.T + q[:, LATENT:] @ rope.T)   # [H, n]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    z = w.sum(axis=1, keepdims=True)
    out = (w / z) @ latent
    lse = (m + np.log(z))[:, 0]
    return out, lse


def sparse_mla_decode(q_bits: np.ndarray, locs: np.ndarray, kv_rows: np.ndarray, scale: float,
                      bf16_kv: bool = False):
    """q_bits: bfloat16 bits uint16 [B, H, 576]; locs: int [B, n] rows of
    kv_rows (uint8 [rows, item]), -1 skipped.  Returns (out [B, H, 512],
    lse [B, H]) in float64.  bf16_kv: attend over the rows' bf16 values
    (decode_rows_bf16: fp8 latents dequantised in float32, then rounded to
    bf16) instead of the exact values the bytes encode (identical for bf16
    rows)."""
    B, H, _ = q_bits.shape
    out = np.zeros((B, H, LATENT))
    lse = np.full((B, H), -np.inf)
    dec = decode_rows_bf16 if bf16_kv else decode_rows
    for b in range(B):
        rows = [int(x) for x in locs[b] if x >= 0]
        lat, rope = dec(kv_rows[rows]) if rows else (np.zeros((0, LATENT)),
                                                     np.zeros((0, ROPE)))
        out[b], lse[b] = attend(bf16_to_f64(q_bits[b]), lat, rope, scale)
    return out, lse


def default_scale() -> float:
    """1 / sqrt(576), the scale the tests use (the call takes any scale)."""
    return 1.0 / math.sqrt(QK_DIM)
