"""Reference and error bounds for the sparse MLA decode attention parity tests.

The reference is the float64 oracle (``oracle/sparse_mla_oracle.py``) over the
values the kernel computes with: bf16 queries and bf16 keys /
values (fp8 rows dequantised by one float32 product and rounded to bf16).
What is left between a correct kernel and that reference is the kernel's own
arithmetic, bounded here per (row, head) and per output element from first
principles (u = 2^-24, the float32 unit roundoff; gamma(n) = n u / (1 - n u)
bounds any float32 summation of n terms, in any order, relative to the sum
of their magnitudes):

* score of location i (natural-log units): the 576-term float32 dot product
  of exact bf16 products, then the scale and the shift by the weights'
  reference in float32, then exp2:
      delta_i = scale * gamma(576) * sum_d |q_d k_id|
                + 2^-23 (|s_i| + max_j |s_j| + 64) + 2^-21;
* exact softmax weights w_i move to w_i (1 + eps_i), with (for any score
  errors within delta) eps_i = max(1 - 1/D+_i, 1/D-_i - 1) and
  D+-_i = w_i + e^(+-delta_i) sum_{j != i} w_j e^(+-delta_j) -- exact, not
  first order, and small for a location that dominates its row;
* each weight is rounded to bf16 (relative 2^-8) for the P.V product; the
  normaliser sums the float32 weights (gamma(n), n = locations of the row);
  the P.V sums accumulate in float32 (gamma(n)); a split's normalised output
  is stored in fp16 (relative 2^-11, absolute 2^-24 below fp16's normal
  range) and the splits merge by weights exp2(m + log2 l - big) computed in
  float32 (relative 2 ln2 (3 u (2 (max|s| log2 e + 64) + 64) + 2^-22)).

Hence, with F_i the combined relative factor of location i,
    |out^_d - out_d| <= sum_i w_i |c_id| F_i + 2^-24,
    |lse^ - lse| <= max(log sum_i w_i e^delta_i, -log sum_i w_i e^-delta_i)
                    + gamma(n) + 2^-21 + 4 u (|lse| + max|s| + 64).
A row with no valid location must give out = 0 and lse = -inf exactly.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import sparse_mla_oracle as mla

U = 2.0 ** -24
LOG2E = 1.0 / math.log(2.0)


def gamma(n):
    return n * U / (1.0 - n * U)


def reference(q_bits, locs, kv_rows, scale):
    """Reference and bounds.  q_bits uint16 [B, H, 576]; locs int [B, n] rows
    of kv_rows (-1 skipped).  Returns dict with out [B, H, 512], lse [B, H],
    tol_out [B, H, 512], tol_lse [B, H], w (list over rows of [H, n_b]
    weights), empty [B] (rows without a valid location)."""
    B, H, _ = q_bits.shape
    out = np.zeros((B, H, mla.LATENT))
    lse = np.full((B, H), -np.inf)
    tol_out = np.zeros((B, H, mla.LATENT))
    tol_lse = np.zeros((B, H))
    weights = []
    empty = np.zeros(B, bool)
    for b in range(B):
        rows = [int(x) for x in locs[b] if x >= 0]
        if not rows:
            empty[b] = True
            weights.append(np.zeros((H, 0)))
            continue
        n = len(rows)
        lat, rope = mla.decode_rows_bf16(kv_rows[rows])
        k = np.concatenate([lat, rope], axis=1)                     # [n, 576]
        q = mla.bf16_to_f64(q_bits[b])                              # [H, 576]
        s = scale * (q @ k.T)                                       # [H, n]
        aqk = scale * (np.abs(q) @ np.abs(k).T)
        smax = np.abs(s).max(axis=1, keepdims=True)
        delta = gamma(mla.QK_DIM) * aqk + 2.0 ** -23 * (np.abs(s) + smax + 64.0) + 2.0 ** -21
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        w = e / z
        weights.append(w)
        out[b] = w @ lat
        lse[b] = (m + np.log(z))[:, 0]
        ep, em = np.exp(delta), np.exp(-delta)
        a_plus = (w * ep).sum(axis=1, keepdims=True)
        a_minus = (w * em).sum(axis=1, keepdims=True)
        d_plus = w + ep * np.maximum(a_plus - w * ep, 0.0)
        d_minus = w + em * np.maximum(a_minus - w * em, 0.0)
        eps = np.maximum(1.0 - 1.0 / d_plus, 1.0 / np.maximum(d_minus, 1e-300) - 1.0)
        g = gamma(n)
        merge = 2.0 * math.log(2.0) * (3.0 * U * (2.0 * (smax * LOG2E + 64.0) + 64.0) + 2.0 ** -22)
        grow = (1.0 + eps) * (1.0 + 2.0 ** -8)
        factor = grow * (1.0 + g + 2.0 ** -22) * (1.0 + 2.0 ** -23) - 1.0 \
            + grow * (g + 2.0 ** -11 + merge)
        tol_out[b] = (w * factor) @ np.abs(lat) + 2.0 ** -24
        tol_lse[b] = np.maximum(np.log(a_plus), -np.log(a_minus))[:, 0] + g + 2.0 ** -21 \
            + 4.0 * U * (np.abs(lse[b]) + smax[:, 0] + 64.0)
    return {"out": out, "lse": lse, "tol_out": tol_out, "tol_lse": tol_lse, "w": weights,
            "empty": empty}


def check(got_out, got_lse, ref):
    """Compares a result with the reference.  Returns (ok, worst error /
    bound over out and lse, a short report)."""
    got_out = np.asarray(got_out, np.float64)
    got_lse = np.asarray(got_lse, np.float64)
    empty = ref["empty"]
    if np.any(~np.isfinite(got_out)):
        return False, math.inf, "non-finite output"
    if empty.any():
        if not (np.all(got_out[empty] == 0) and np.all(np.isneginf(got_lse[empty]))):
            return False, math.inf, "a row without locations is not (0, -inf)"
    live = ~empty
    if not live.any():
        return True, 0.0, "no live rows"
    if np.any(~np.isfinite(got_lse[live])):
        return False, math.inf, "non-finite lse on a live row"
    eo = np.abs(got_out[live] - ref["out"][live]) / ref["tol_out"][live]
    el = np.abs(got_lse[live] - ref["lse"][live]) / ref["tol_lse"][live]
    worst = max(float(eo.max()), float(el.max()))
    report = f"out error/bound {eo.max():.3g}, lse error/bound {el.max():.3g}"
    return worst <= 1.0, worst, report
