"""CPU float64 oracle for the gradients of exact attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
this module: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py`` use
it. It shares no code with the HIP library and never reads a value the HIP
library produced.

What it computes. "FlashAttention 与长上下文：先分清三张账", section
"FlashAttention 的关键是 online softmax", says the backward pass keeps the small
per-row statistics of the forward pass and recomputes the tile scores it needs,
instead of storing the score matrix. The pages give no gradient formulas: the
gradients here are the derivative of the forward definition (``attention.py``),
written out the naive, materialised way for one (batch, head) with the
upstream gradient dO of the output:

    P  = softmax(scale * Q K^T + M)            (rows of P sum to 1, or are 0)
    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij = sum_c dO_ic O_ic  (one number per query row)
    dS = P * (dP - D)                          (element-wise; D broadcast per row)
    dQ = scale * dS K
    dK = scale * dS^T Q

With grouped-query attention a KV head is shared by H / Hkv query heads, so its
dK and dV are the sums over those heads. Masked entries have P = 0 and so
contribute nothing; padding query rows (i >= n_b, which have O = 0) get dQ = 0
and contribute nothing to dK or dV; keys that no row sees get dK = dV = 0.

Pins (``tests/test_oracle_backward.py``): central finite differences of the
forward oracle on tiny heads, torch autograd on float64 scaled_dot_product_
attention, the zero-sum invariants sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i
(over rows that see a key), and planted mistakes that must fail.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_head


def attention_backward_head(q, k, v, do, *, scale, causal=False, n_valid=None, window=None):
    """Gradients (dQ [Lq, d], dK [Lk, d], dV [Lk, d]) of one head, given dO [Lq, d]."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    O, _, P = attention_head(q, k, v, scale=scale, causal=causal, n_valid=n_valid, return_p=True, window=window)
    dV = P.T @ do
    dP = do @ v.T
    D = (do * O).sum(axis=1)
    dS = P * (dP - D[:, None])
    dQ = scale * (dS @ k)
    dK = scale * (dS.T @ q)
    return dQ, dK, dV


def attention_backward(q, k, v, do, *, scale, causal=False, seqlens=None, window=None):
    """Gradients over [B, H, Lq, d] queries and [B, Hkv, Lk, d] keys/values.

    Returns (dQ [B, H, Lq, d], dK [B, Hkv, Lk, d], dV [B, Hkv, Lk, d]); dK and dV
    of a KV head are summed over its query heads.
    """
    B, H, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    assert H % Hkv == 0, "query heads must be a multiple of KV heads"
    group = H // Hkv
    if seqlens is not None:
        assert Lq == Lk, "per-sequence lengths need Lq == Lk"
    dQ = np.zeros((B, H, Lq, d))
    dK = np.zeros((B, Hkv, Lk, d))
    dV = np.zeros((B, Hkv, Lk, d))
    for b in range(B):
        n = None if seqlens is None else int(seqlens[b])
        for h in range(H):
            kvh = h // group
            gq, gk, gv = attention_backward_head(q[b, h], k[b, kvh], v[b, kvh], do[b, h], scale=scale,
                                                 causal=causal, n_valid=n, window=window)
            dQ[b, h] = gq
            dK[b, kvh] += gk
            dV[b, kvh] += gv
    return dQ, dK, dV
