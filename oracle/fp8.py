"""CPU float64 oracle for exact attention with FP8 operands (test infrastructure only).

TEST INFRASTRUCTURE ONLY: like the rest of ``oracle/``, only ``tests/``, ``__graft_entry__``
and ``bench.py``'s CPU baseline use it; it shares no code with the HIP library.

What it computes. "FlashAttention 与长上下文：先分清三张账" (section on FlashAttention-2/3) and
the aiknowledge.cn page on FlashAttention-3 name low-precision (FP8) execution as the FA-3
step, without a scaling scheme. The scheme read here (each choice listed in the design doc):

* Q, K and V arrive as OCP FP8 E4M3 codes with one fp32 descale per (batch, head):
  Q = decode(q) * q_descale, and likewise K, V. The dequantised values are what attention
  is computed on, exactly (they are exactly representable in float64).
* Scores in base 2: t_ij = scale * log2(e) * (Q K^T)_ij, masked entries -inf.
* Every row has an integer reference M_i = ceil(max_j t_ij). Its probabilities relative to
  M_i are 2^(t_ij - M_i) <= 1; they enter the P V product as FP8, scaled by 2^8 first:
      pq_ij = e4m3(256 * 2^(t_ij - M_i))      (round to nearest even)
  while the row sum stays exact:  l_i = sum_j 2^(t_ij - M_i).
* O_i = sum_j pq_ij V_j / (256 l_i),  LSE_i = ln(2) (M_i + log2 l_i).
  Because rounding to E4M3 commutes with scaling by a power of two (in its normal range), the
  result does not depend on which integer reference a blockwise (online) evaluation used on
  the way, so this whole-row form is what a tiled kernel computes too.

Pins are in ``tests/test_oracle_fp8.py``; no function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

from .attention import _visible

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Values of OCP E4M3 (fn) codes: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
    0 is subnormal (m/8 * 2^-6); code 0x7f / 0xff is NaN; there is no infinity."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e.astype(np.float64) - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def e4m3_round(x) -> np.ndarray:
    """Round float64 values to the nearest E4M3 value (ties to even), saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # spacing of E4M3 at |x|: 2^(e - 3) for |x| in [2^e, 2^(e+1)), e >= -6; 2^-9 below 2^-6
    _, E = np.frexp(np.where(a > 0, a, 1.0))  # a = f 2^E with f in [0.5, 1): e = E - 1 exactly
    e = np.maximum(E.astype(np.float64) - 1.0, -6.0)
    q = 2.0 ** (e - 3.0)
    r = np.round(a / q) * q  # numpy rounds halves to even
    r = np.minimum(r, E4M3_MAX)
    return np.where(a > 0, np.sign(x) * r, 0.0 * x)


def attention_fp8_head(q, k, v, *, scale, causal=False, n_valid=None, rows=None, window=None, p_scale=256.0):
    """Attention of one (batch, head) on dequantised FP8 operands with the FP8 P scheme above.

    q: [Lq, d]; k, v: [Lk, d] float64 (already dequantised). Returns (O [r, d], LSE [r]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Lq, Lk = q.shape[0], k.shape[0]
    row_idx = np.arange(Lq) if rows is None else np.asarray(rows)
    n = Lk if n_valid is None else int(n_valid)
    t = (scale * np.log2(np.e)) * (q[row_idx] @ k.T)
    vis = _visible(Lq, Lk, causal, n, row_idx, window)
    if n_valid is not None:
        vis[row_idx >= n, :] = False
    t = np.where(vis, t, -np.inf)
    tmax = t.max(axis=1) if Lk > 0 else np.full(len(row_idx), -np.inf)
    empty = ~np.isfinite(tmax)
    M = np.where(empty, 0.0, np.ceil(np.where(empty, 0.0, tmax)))
    w = np.exp2(t - M[:, None])  # 0 where masked
    l = w.sum(axis=1)
    pq = e4m3_round(p_scale * w)
    O = (pq @ v) / np.where(empty, 1.0, p_scale * l)[:, None]
    O[empty] = 0.0
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, np.log(2.0) * (M + np.log2(np.where(empty, 1.0, l))))
    return O, lse


def attention_fp8(q8, k8, v8, q_descale, k_descale, v_descale, *, scale, causal=False, seqlens=None, heads=None,
                  rows=None, window=None):
    """Batched FP8 attention: q8 [B, H, Lq, d], k8, v8 [B, Hkv, Lk, d] E4M3 codes (uint8),
    descales [B, H] for q and [B, Hkv] for k and v. Returns (O [B, H, r, d], LSE [B, H, r])."""
    B, H, Lq, d = q8.shape
    Hkv, Lk = k8.shape[1], k8.shape[2]
    group = H // Hkv
    r = Lq if rows is None else len(rows)
    O = np.full((B, H, r, d), np.nan)
    LSE = np.full((B, H, r), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        kvh = h // group
        n = None if seqlens is None else int(seqlens[b])
        Q = e4m3_decode(q8[b, h]) * float(q_descale[b, h])
        K = e4m3_decode(k8[b, kvh]) * float(k_descale[b, kvh])
        V = e4m3_decode(v8[b, kvh]) * float(v_descale[b, kvh])
        O[b, h], LSE[b, h] = attention_fp8_head(Q, K, V, scale=scale, causal=causal, n_valid=n, rows=rows,
                                                window=window)
    return O, LSE
