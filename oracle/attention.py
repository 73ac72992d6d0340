"""CPU float64 oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library and never reads a value the HIP library produced.

What it computes (cited by page title and section):

* "FlashAttention 与长上下文：先分清三张账" (charles2530.github.io), section
  "标准 attention 的问题不只在 FLOPs", equation for O: one head computes
  O = softmax((Q K^T + M) / sqrt(d_h)) V, where M is a causal mask, a padding
  mask or another bias. Here M only takes the values 0 and -inf, so it does
  not matter whether M sits inside the 1/sqrt(d) factor; the scale is passed
  explicitly and multiplies Q K^T.
* "2.1 FlashAttention-2 的核心思想：把注意力算在 SRAM 里" (aiknowledge.cn),
  section 2.1.1: the three-step naive form (scores, softmax along the last
  axis, product with V) on ``[batch, heads, n, d]`` tensors. The oracle is
  exactly that form: it materialises S and P for every (batch, head).
* Same page 1, section "FlashAttention 的关键是 online softmax": the
  max-subtracted softmax, and the per-row log-sum-exp statistic kept for the
  backward pass (emitted here as LSE = m + ln(sum exp(S - m)), natural log).

Readings where the pages are silent (each is listed in the design doc):

* Causal alignment is bottom-right: key j is visible to query i when
  j <= i + (Lk - Lq). With Lq = Lk it is the usual lower triangle; for a
  single decode query it means "every cached key".
* GQA maps query head h to KV head floor(h / (H / Hkv)) (contiguous groups).
* With per-sequence lengths n_b (self-attention, Lq = Lk), keys j >= n_b are
  masked and query rows i >= n_b are padding: O = 0 and LSE = -inf there.
* A row that sees no key at all gets O = 0 and LSE = -inf (no NaN).
* Sliding window ("FlashAttention 与长上下文", section on prefill and decode,
  which lists the sliding window among the context-trimming methods without
  defining it): with window W >= 1 and the causal mask, query i sees only the
  W newest keys it is allowed to see, i + (Lk - Lq) - W < j <= i + (Lk - Lq);
  a decode query of context n sees keys max(0, n - W) .. n - 1.

Parity pins for every function here are in ``tests/test_oracle.py``; no
function in this module is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _visible(Lq: int, Lk: int, causal: bool, n_valid: int, rows=None, window=None) -> np.ndarray:
    """Boolean [len(rows), Lk]: key j visible to query row i.

    Padding: keys at or beyond ``n_valid`` are masked. Causal (bottom-right
    aligned): key j is masked when j > i + (Lk - Lq). Sliding window W (with
    causal): key j is also masked when j <= i + (Lk - Lq) - W.
    """
    i = np.arange(Lq) if rows is None else np.asarray(rows)
    j = np.arange(Lk)
    vis = np.broadcast_to(j[None, :] < n_valid, (len(i), Lk)).copy()
    if causal:
        vis &= j[None, :] <= (i[:, None] + (Lk - Lq))
    if window is not None:
        assert causal and window >= 1, "a sliding window needs the causal mask and W >= 1"
        vis &= j[None, :] > (i[:, None] + (Lk - Lq) - window)
    return vis


def attention_head(q, k, v, *, scale, causal=False, n_valid=None, rows=None, return_p=False, window=None):
    """Exact attention for one (batch, head) pair, the naive materialised way.

    q: [Lq, d]; k, v: [Lk, d] (float64). ``n_valid``: valid sequence length for
    both query rows and keys (None = no padding). ``rows``: optional subset of
    query rows to evaluate (the result is identical to slicing the full result).
    ``window``: sliding-window size W (needs ``causal``), None for none.
    Returns (O [r, d], LSE [r]) and optionally P [r, Lk].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Lq, Lk = q.shape[0], k.shape[0]
    row_idx = np.arange(Lq) if rows is None else np.asarray(rows)
    n = Lk if n_valid is None else int(n_valid)
    # Step 1: score matrix S = scale * Q K^T, with -inf where the mask hides a key.
    S = scale * (q[row_idx] @ k.T)
    vis = _visible(Lq, Lk, causal, n, row_idx, window)
    S = np.where(vis, S, NEG_INF)
    # Padding query rows (i >= n_valid) attend to nothing.
    if n_valid is not None:
        S[row_idx >= n, :] = NEG_INF
    # Step 2: row softmax with the row maximum subtracted.
    m = S.max(axis=1) if Lk > 0 else np.full(len(row_idx), NEG_INF)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    E = np.exp(S - m_safe[:, None])  # exp(-inf) = 0 for masked entries
    l = E.sum(axis=1)
    P = np.where(empty[:, None], 0.0, E / np.where(empty, 1.0, l)[:, None])
    # Step 3: O = P V, and the row log-sum-exp.
    O = P @ v
    with np.errstate(divide="ignore"):
        lse = np.where(empty, NEG_INF, m_safe + np.log(np.where(empty, 1.0, l)))
    if return_p:
        return O, lse, P
    return O, lse


def attention(q, k, v, *, scale, causal=False, seqlens=None, heads=None, rows=None, window=None):
    """Exact attention over [B, H, Lq, d] queries and [B, Hkv, Lk, d] keys/values.

    ``seqlens``: optional per-batch valid lengths (requires Lq == Lk).
    ``heads``: optional list of (b, h) pairs to evaluate; ``rows``: optional
    query-row subset applied to every evaluated head. ``window``: sliding window W.
    Returns (O, LSE) with shapes [B, H, r, d] and [B, H, r] (entries of heads not
    evaluated are NaN).
    """
    B, H, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    assert H % Hkv == 0, "query heads must be a multiple of KV heads"
    group = H // Hkv
    if seqlens is not None:
        assert Lq == Lk, "per-sequence lengths need Lq == Lk"
    r = Lq if rows is None else len(rows)
    O = np.full((B, H, r, d), np.nan)
    LSE = np.full((B, H, r), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        kvh = h // group
        n = None if seqlens is None else int(seqlens[b])
        O[b, h], LSE[b, h] = attention_head(q[b, h], k[b, kvh], v[b, kvh], scale=scale, causal=causal,
                                            n_valid=n, rows=rows, window=window)
    return O, LSE


def decode(q, k_cache, v_cache, ctx_lens, *, scale, heads=None, window=None):
    """Single-token decode: query [B, H, d] against cache [B, Hkv, Lmax, d].

    Request b sees cached keys 0 .. ctx_lens[b]-1 and nothing else (the new
    token is the newest position, so bottom-right causal alignment leaves every
    cached key visible). With a sliding window W it sees keys
    max(0, n - W) .. n - 1 of its context n. Returns (O [B, H, d], LSE [B, H]).
    """
    B, H, d = q.shape
    Hkv = k_cache.shape[1]
    group = H // Hkv
    O = np.full((B, H, d), np.nan)
    LSE = np.full((B, H), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        n = int(ctx_lens[b])
        kvh = h // group
        o, lse = attention_head(q[b, h][None, :], k_cache[b, kvh, :n], v_cache[b, kvh, :n], scale=scale,
                                causal=window is not None, window=window)
        O[b, h], LSE[b, h] = o[0], lse[0]
    return O, LSE


def decode_paged(q, k_pages, v_pages, block_table, ctx_lens, *, page_size, scale, heads=None, window=None):
    """Decode against a paged KV cache (PagedAttention's layout, "FlashAttention 与长上下文",
    prefill/decode section, which names paged KV allocation without fixing a layout).

    k_pages, v_pages: [num_pages, Hkv, P, d]; block_table: int [B, max_pages]. Cache
    position j of request b is row j % P of page block_table[b, j // P]. The pages of a
    request are gathered into one contiguous cache and decoded as ``decode`` does.
    Returns (O [B, H, d], LSE [B, H]).
    """
    B, H, d = q.shape
    Hkv = k_pages.shape[1]
    group = H // Hkv
    O = np.full((B, H, d), np.nan)
    LSE = np.full((B, H), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        n = int(ctx_lens[b])
        kvh = h // group
        pages = [int(p) for p in block_table[b, :(n + page_size - 1) // page_size]]
        K = np.concatenate([k_pages[p, kvh] for p in pages], axis=0)[:n] if pages else np.zeros((0, d))
        V = np.concatenate([v_pages[p, kvh] for p in pages], axis=0)[:n] if pages else np.zeros((0, d))
        o, lse = attention_head(q[b, h][None, :], K, V, scale=scale, causal=window is not None, window=window)
        O[b, h], LSE[b, h] = o[0], lse[0]
    return O, LSE


def online_softmax_rows(S, V, block):
    """Blockwise (online) softmax-times-V of one score row, in the pages' order.

    Follows "FlashAttention 与长上下文" section "FlashAttention 的关键是 online
    softmax": state (m, l, o) starts at (-inf, 0, 0); for each block S_j of the
    row and its V_j rows,
        m' = max(m, max S_j)
        l' = e^(m - m') l + sum_t e^(S_jt - m')
        o' = e^(m - m') o + sum_t e^(S_jt - m') V_jt
    and at the end O = o / l. Also returns LSE = m + ln l.

    S: [n] scores of one row (may contain -inf); V: [n, d]; block >= 1.
    """
    S = np.asarray(S, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    m, l, o = NEG_INF, 0.0, np.zeros(V.shape[1])
    for s0 in range(0, len(S), block):
        Sj, Vj = S[s0:s0 + block], V[s0:s0 + block]
        m_new = max(m, Sj.max())
        if m_new == NEG_INF:  # nothing visible yet: the state stays empty
            continue
        a = np.exp(m - m_new)  # e^(-inf) = 0 when m was -inf
        e = np.exp(Sj - m_new)
        l = a * l + e.sum()
        o = a * o + e @ Vj
        m = m_new
    if l == 0.0:
        return np.zeros(V.shape[1]), NEG_INF
    return o / l, m + np.log(l)


def merge(parts):
    """Merge per-part softmax results with the rule of "FlashAttention-2 的核心思想" §2.1.3.

    Each part is (m, l, O): the part's row max, its sum of e^(s - m), and its
    normalised output O = sum e^(s - m) v / l. Two states merge as
        m = max(m_a, m_b)
        l = e^(m_a - m) l_a + e^(m_b - m) l_b
        O = (e^(m_a - m) l_a / l) O_a + (e^(m_b - m) l_b / l) O_b
    applied left to right. Parts with l = 0 (nothing visible) are skipped.
    Returns (O, LSE) with LSE = m + ln l.
    """
    m, l, O = NEG_INF, 0.0, None
    for m_b, l_b, O_b in parts:
        if l_b == 0.0:
            continue
        if O is None:
            m, l, O = m_b, l_b, np.asarray(O_b, dtype=np.float64)
            continue
        m_new = max(m, m_b)
        wa = np.exp(m - m_new) * l
        wb = np.exp(m_b - m_new) * l_b
        l_new = wa + wb
        O = (wa / l_new) * O + (wb / l_new) * np.asarray(O_b, dtype=np.float64)
        m, l = m_new, l_new
    if O is None:
        return None, NEG_INF
    return O, m + np.log(l)


def part_state(S, V):
    """(m, l, O) of one part of a score row, for ``merge``: the plain softmax of the part."""
    S = np.asarray(S, dtype=np.float64)
    m = S.max() if len(S) else NEG_INF
    if m == NEG_INF:
        return NEG_INF, 0.0, np.zeros(V.shape[1])
    e = np.exp(S - m)
    l = e.sum()
    return m, l, (e @ np.asarray(V, dtype=np.float64)) / l
