"""Pins for the CPU oracle: values printed on the pages, closed forms, invariants,
special cases that reduce to a library routine, and brute force on tiny inputs.

Every pin is written against an implementation callable with the signature of
``oracle.attention_head`` so the same pins can be aimed at deliberately broken
copies of the oracle (``test_pins_catch_planted_mistakes``): each plausible
mistake must make at least one pin fail.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import attention_head

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_online_softmax.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Pins, each parameterised by the single-head implementation under test.
# ---------------------------------------------------------------------------

def pin_worked_example(head):
    """Scores [2,5,1,4] give the page's probabilities (§2.1.9) to 4 decimals.

    Embedding: d = 4, scale = 1, q = e0, k_j = s_j e0 (so S_j = s_j) and
    V = identity (so row 0 of O is the probability vector P).
    """
    g = _golden()
    s = np.array(g["scores"], dtype=np.float64)
    n = len(s)
    q = np.zeros((1, n)); q[0, 0] = 1.0
    k = np.zeros((n, n)); k[:, 0] = s
    v = np.eye(n)
    O, lse = head(q, k, v, scale=1.0)
    P = O[0]
    assert np.array_equal(np.round(P, 4), np.array(g["full_row"]["probs"]))
    # Intermediates printed on the page: the row max and e^(s - m) with their sum.
    exps = np.exp(s - s.max())
    assert s.max() == g["full_row"]["max"]
    assert np.array_equal(np.round(exps, 4), np.array(g["full_row"]["exps"], dtype=float))
    # The page's sums are 4-decimal approximations (1.4359 truncates 1.43598).
    assert abs(exps.sum() - g["full_row"]["exp_sum"]) <= 1e-4
    # LSE = m + ln(sum e^(s-m)); the page's 4-decimal sum bounds it to +-1e-4 / 1.4359.
    assert abs(lse[0] - (g["full_row"]["max"] + math.log(g["full_row"]["exp_sum"]))) < 1e-4
    # Closed form to full precision.
    assert abs(lse[0] - math.log(sum(math.exp(x) for x in s))) < 1e-12


def pin_bruteforce_tiny(head):
    """Pure-Python loops (math.exp, no numpy) on tiny random heads, masks included."""
    rng = np.random.default_rng(7)
    for trial in range(30):
        Lq = int(rng.integers(1, 6))
        Lk = Lq + int(rng.integers(0, 3))
        d = int(rng.integers(1, 5))
        q = rng.standard_normal((Lq, d)); k = rng.standard_normal((Lk, d)); v = rng.standard_normal((Lk, d))
        scale = float(rng.uniform(0.2, 2.0))
        causal = bool(trial % 2)
        n_valid = None
        if trial % 3 == 0 and Lq == Lk:
            n_valid = int(rng.integers(0, Lk + 1))
        O, lse = head(q, k, v, scale=scale, causal=causal, n_valid=n_valid)
        for i in range(Lq):
            n = Lk if n_valid is None else n_valid
            vis = [j for j in range(Lk) if j < n and (not causal or j <= i + (Lk - Lq))]
            if n_valid is not None and i >= n_valid:
                vis = []
            if not vis:
                assert all(O[i, c] == 0.0 for c in range(d)) and lse[i] == -math.inf
                continue
            sc = {j: scale * sum(q[i, c] * k[j, c] for c in range(d)) for j in vis}
            mx = max(sc.values())
            den = sum(math.exp(sc[j] - mx) for j in vis)
            for c in range(d):
                num = sum(math.exp(sc[j] - mx) * v[j, c] for j in vis)
                assert abs(O[i, c] - num / den) < 1e-12
            assert abs(lse[i] - (mx + math.log(den))) < 1e-12


def pin_torch_sdpa(head):
    """Agreement with torch's own scaled_dot_product_attention (CPU, float64) for Lq = Lk."""
    g = torch.Generator().manual_seed(11)
    for causal, L, d in [(False, 9, 4), (True, 9, 4), (True, 16, 8), (False, 3, 16)]:
        q = torch.randn(L, d, generator=g, dtype=torch.float64)
        k = torch.randn(L, d, generator=g, dtype=torch.float64)
        v = torch.randn(L, d, generator=g, dtype=torch.float64)
        scale = 1.0 / math.sqrt(d)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[None, None], k[None, None], v[None, None], is_causal=causal, scale=scale)[0, 0]
        O, _ = head(q.numpy(), k.numpy(), v.numpy(), scale=scale, causal=causal)
        assert np.allclose(O, ref.numpy(), atol=1e-12, rtol=0)


def pin_causal_row0_and_single_key(head):
    """Causal row 0 sees only key 0: O[0] = V[0], LSE[0] = scale q0.k0. Lk = 1 likewise."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((6, 5)); k = rng.standard_normal((6, 5)); v = rng.standard_normal((6, 5))
    O, lse = head(q, k, v, scale=0.7, causal=True)
    assert np.allclose(O[0], v[0], atol=1e-15, rtol=0)
    assert abs(lse[0] - 0.7 * q[0] @ k[0]) < 1e-12
    O1, lse1 = head(q[:1], k[:1], v[:1], scale=0.7)
    assert np.allclose(O1[0], v[0], atol=1e-15, rtol=0) and abs(lse1[0] - 0.7 * q[0] @ k[0]) < 1e-12


def pin_uniform(head):
    """Q = 0 makes every visible key equally likely: O_i is the mean of the visible
    V rows and LSE_i = ln(#visible). Causal: prefix means and ln(i + 1)."""
    rng = np.random.default_rng(5)
    L, d = 7, 3
    k = rng.standard_normal((L, d)); v = rng.standard_normal((L, d))
    q = np.zeros((L, d))
    O, lse = head(q, k, v, scale=1.0)
    assert np.allclose(O, np.tile(v.mean(0), (L, 1)), atol=1e-13, rtol=0)
    assert np.allclose(lse, math.log(L), atol=1e-13, rtol=0)
    Oc, lsec = head(q, k, v, scale=1.0, causal=True)
    for i in range(L):
        assert np.allclose(Oc[i], v[: i + 1].mean(0), atol=1e-13, rtol=0)
        assert abs(lsec[i] - math.log(i + 1)) < 1e-13


def pin_large_logits(head):
    """Scores in the thousands must not overflow (the row max is subtracted):
    two keys with scores 1000 and 999 give weights sigmoid(1) and sigmoid(-1)."""
    q = np.array([[1.0]])
    k = np.array([[1000.0], [999.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    O, lse = head(q, k, v, scale=1.0)
    p0 = 1.0 / (1.0 + math.exp(-1.0))
    assert np.allclose(O[0], [p0, 1 - p0], atol=1e-14, rtol=0)
    assert abs(lse[0] - (1000.0 + math.log1p(math.exp(-1.0)))) < 1e-12


def pin_permutation_and_convexity(head):
    """Non-causal: permuting K and V rows together changes nothing; every output
    element lies between the min and max of its V column."""
    rng = np.random.default_rng(9)
    q = rng.standard_normal((5, 4)); k = rng.standard_normal((8, 4)); v = rng.standard_normal((8, 4))
    O, lse = head(q, k, v, scale=0.5)
    perm = rng.permutation(8)
    Op, lsep = head(q, k[perm], v[perm], scale=0.5)
    assert np.allclose(O, Op, atol=1e-13, rtol=0) and np.allclose(lse, lsep, atol=1e-13, rtol=0)
    assert np.all(O >= v.min(0) - 1e-13) and np.all(O <= v.max(0) + 1e-13)


def pin_bottom_right_alignment(head):
    """Lq < Lk: the last query row sees every key, row i sees keys 0 .. i + Lk - Lq."""
    rng = np.random.default_rng(13)
    Lq, Lk, d = 3, 7, 2
    q = rng.standard_normal((Lq, d)); k = rng.standard_normal((Lk, d)); v = rng.standard_normal((Lk, d))
    O, lse = head(q, k, v, scale=1.0, causal=True)
    for i in range(Lq):
        n = i + Lk - Lq + 1
        Oi, lsei = head(q[i:i + 1], k[:n], v[:n], scale=1.0)
        assert np.allclose(O[i], Oi[0], atol=1e-13, rtol=0) and abs(lse[i] - lsei[0]) < 1e-13


PINS = [pin_worked_example, pin_bruteforce_tiny, pin_torch_sdpa, pin_causal_row0_and_single_key,
        pin_uniform, pin_large_logits, pin_permutation_and_convexity, pin_bottom_right_alignment]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(attention_head)


# ---------------------------------------------------------------------------
# Planted mistakes: each broken copy must fail at least one pin.
# ---------------------------------------------------------------------------

def _mutant(kind):
    def head(q, k, v, *, scale, causal=False, n_valid=None, rows=None, return_p=False):
        q = np.asarray(q, float); k = np.asarray(k, float); v = np.asarray(v, float)
        Lq, Lk = q.shape[0], k.shape[0]
        n = Lk if n_valid is None else n_valid
        sc = 1.0 if kind == "scale_dropped" else scale
        S = sc * (q @ k.T)
        i = np.arange(Lq)[:, None]; j = np.arange(Lk)[None, :]
        vis = j < n
        if causal:
            shift = 0 if kind == "top_left_causal" else (Lk - Lq)
            lim = i + shift + (1 if kind == "causal_off_by_one" else 0)
            vis = vis & (j <= lim)
        if n_valid is not None:
            vis = vis & (i < n)
        S = np.where(vis, S, -np.inf)
        m = S.max(1) if kind != "no_max_subtraction" else np.zeros(Lq)
        empty = ~np.isfinite(S.max(1))
        m = np.where(empty, 0.0, m)
        E = np.exp(S - m[:, None])
        if kind == "sign_flip":
            E = np.exp(-(S - m[:, None])) * vis
        l = E.sum(1)
        P = np.where(empty[:, None], 0.0, E / np.where(empty, 1.0, l)[:, None])
        if kind == "transposed_p":
            O = P.T[:Lq, :] @ v if P.shape[0] == P.shape[1] else P @ v[::-1]
        elif kind == "v_rows_reversed":
            O = P @ v[::-1]
        else:
            O = P @ v
        lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, l)))
        if kind == "lse_log2":
            lse = np.where(empty, -np.inf, m + np.log2(np.where(empty, 1.0, l)))
        return O, lse
    return head


MUTANTS = ["scale_dropped", "top_left_causal", "causal_off_by_one", "no_max_subtraction", "sign_flip",
           "transposed_p", "v_rows_reversed", "lse_log2"]


def test_mutant_harness_is_faithful():
    # The unmutated copy passes every pin, so a failure below is due to the mutation.
    for pin in PINS:
        pin(_mutant("none"))


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistakes(kind):
    head = _mutant(kind)
    failures = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(head)
        except AssertionError:
            failures += 1
    assert failures >= 1, f"no pin catches the planted mistake {kind!r}"


# ---------------------------------------------------------------------------
# Blockwise (online) form and the merge rule against the materialised form.
# ---------------------------------------------------------------------------

def test_worked_example_blockwise_and_merge():
    """Block A then block B through the online update and through the merge rule."""
    g = _golden()
    s = np.array(g["scores"], float)
    V = np.eye(4)
    O, lse = oracle.online_softmax_rows(s, V, block=2)
    assert np.array_equal(np.round(O, 4), np.array(g["full_row"]["probs"]))
    mA, lA, OA = oracle.part_state(s[:2], V[:2])
    assert mA == g["block_a"]["max"]
    assert abs(lA - g["block_a"]["weight_sum"]) <= 1e-4
    assert np.array_equal(np.round(OA[:2], 4), np.array(g["block_a"]["normalised"]))
    mB, lB, OB = oracle.part_state(s[2:], V[2:])
    assert np.array_equal(np.round(np.exp(s[2:] - 5.0), 4), np.array(g["block_b"]["weights"]))
    Om, lsem = oracle.merge([(mA, lA, OA), (mB, lB, OB)])
    assert np.allclose(Om, O, atol=1e-15) and abs(lsem - lse) < 1e-15
    # Merged weight sum with m unchanged (no rescale): 1.0498 + 0.3862 -> 1.4359.
    assert abs(lA + np.exp(s[2:] - 5.0).sum() - g["block_b"]["weight_sum_after_merge"]) <= 1e-4


def test_worked_example_block_c_rescale():
    """Appending block C = [10] rescales the history by e^(5 - 10) = e^-5."""
    g = _golden()
    s = np.array(g["scores"] + g["block_c"]["scores"], float)
    V = np.eye(5)
    mAB, lAB, OAB = oracle.part_state(s[:4], V[:4])
    mC, lC, OC = oracle.part_state(s[4:], V[4:])
    factor = math.exp(mAB - max(mAB, mC))
    assert abs(math.log(factor) - g["block_c"]["history_factor_exponent"]) < 1e-15
    Om, lse = oracle.merge([(mAB, lAB, OAB), (mC, lC, OC)])
    exact = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    assert np.allclose(Om, exact, atol=1e-15)
    # The history part carries weight e^-5 * l_AB / l_new, the new key 1 / l_new.
    l_new = factor * lAB + lC
    assert np.allclose(Om[:4], OAB[:4] * factor * lAB / l_new, atol=1e-15)
    assert abs(lse - math.log(np.exp(s).sum())) < 1e-12


def test_blockwise_equals_whole_row_bruteforce():
    """Online updates with block sizes 1, 2, 3, 5 and n equal the whole-row softmax
    (masked entries included) on 1000 random tiny rows."""
    rng = np.random.default_rng(2024)
    for trial in range(1000):
        n = int(rng.integers(1, 13)); d = int(rng.integers(1, 4))
        S = rng.standard_normal(n) * float(rng.uniform(0.1, 6.0))
        S[rng.random(n) < 0.3] = -np.inf
        V = rng.standard_normal((n, d))
        fin = np.isfinite(S)
        for beta in (1, 2, 3, 5, n):
            O, lse = oracle.online_softmax_rows(S, V, beta)
            if not fin.any():
                assert lse == -np.inf and np.all(O == 0.0)
                continue
            m = S[fin].max()
            e = np.where(fin, np.exp(S - m), 0.0)
            assert np.allclose(O, (e @ V) / e.sum(), atol=1e-12, rtol=0)
            assert abs(lse - (m + np.log(e.sum()))) < 1e-12


def test_merge_equals_whole_row_random_partitions():
    rng = np.random.default_rng(77)
    for trial in range(500):
        n = int(rng.integers(1, 20)); d = int(rng.integers(1, 4))
        S = rng.standard_normal(n) * 3.0
        S[rng.random(n) < 0.2] = -np.inf
        V = rng.standard_normal((n, d))
        cuts = sorted(set(rng.integers(0, n + 1, size=int(rng.integers(0, 5))).tolist()) | {0, n})
        parts = [oracle.part_state(S[a:b], V[a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
        Om, lse = oracle.merge(parts)
        Ob, lseb = oracle.online_softmax_rows(S, V, n)
        if not np.isfinite(S).any():
            assert Om is None and lse == -np.inf
            continue
        assert np.allclose(Om, Ob, atol=1e-12, rtol=0) and abs(lse - lseb) < 1e-12


def test_p_rows_sum_to_one_and_mask_zero():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((10, 4)); k = rng.standard_normal((10, 4)); v = rng.standard_normal((10, 4))
    _, _, P = attention_head(q, k, v, scale=0.5, causal=True, n_valid=8, return_p=True)
    assert np.allclose(P[:8].sum(1), 1.0, atol=1e-12)
    assert np.all(P[8:] == 0.0)
    assert np.all(np.triu(P, 1) == 0.0) and np.all(P[:, 8:] == 0.0)


# ---------------------------------------------------------------------------
# Batched wrappers: GQA, variable length, decode, row subsets.
# ---------------------------------------------------------------------------

def test_gqa_equals_repeated_kv():
    rng = np.random.default_rng(4)
    B, H, Hkv, L, d = 2, 8, 2, 6, 3
    q = rng.standard_normal((B, H, L, d)); k = rng.standard_normal((B, Hkv, L, d)); v = rng.standard_normal((B, Hkv, L, d))
    O, lse = oracle.attention(q, k, v, scale=0.6, causal=True)
    kr = np.repeat(k, H // Hkv, axis=1); vr = np.repeat(v, H // Hkv, axis=1)
    Or, lser = oracle.attention(q, kr, vr, scale=0.6, causal=True)
    assert np.array_equal(O, Or) and np.array_equal(lse, lser)
    # And torch's GQA semantics agree (enable_gqa pairs head h with KV head h // (H/Hkv)).
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True, scale=0.6, enable_gqa=True)
    assert np.allclose(O, ref.numpy(), atol=1e-12)


def test_varlen_equals_fresh_run_and_padding():
    rng = np.random.default_rng(8)
    B, H, L, d = 3, 2, 9, 4
    q = rng.standard_normal((B, H, L, d)); k = rng.standard_normal((B, H, L, d)); v = rng.standard_normal((B, H, L, d))
    seqlens = np.array([9, 4, 1])
    O, lse = oracle.attention(q, k, v, scale=0.5, causal=True, seqlens=seqlens)
    for b, n in enumerate(seqlens):
        Of, lsef = oracle.attention(q[b:b + 1, :, :n], k[b:b + 1, :, :n], v[b:b + 1, :, :n], scale=0.5, causal=True)
        assert np.allclose(O[b, :, :n], Of[0], atol=1e-14) and np.allclose(lse[b, :, :n], lsef[0], atol=1e-14)
        assert np.all(O[b, :, n:] == 0.0) and np.all(lse[b, :, n:] == -np.inf)


def test_decode_equals_last_causal_row():
    rng = np.random.default_rng(12)
    B, H, Hkv, Lmax, d = 2, 4, 2, 10, 3
    q = rng.standard_normal((B, H, d)); kc = rng.standard_normal((B, Hkv, Lmax, d)); vc = rng.standard_normal((B, Hkv, Lmax, d))
    ctx = np.array([10, 6])
    O, lse = oracle.decode(q, kc, vc, ctx, scale=0.4)
    for b, n in enumerate(ctx):
        # A prefill of n rows whose last query row is the decode query.
        qq = np.zeros((1, H, n, d)); qq[0, :, -1] = q[b]
        Op, lsep = oracle.attention(qq, kc[b:b + 1, :, :n], vc[b:b + 1, :, :n], scale=0.4, causal=True)
        assert np.allclose(O[b], Op[0, :, -1], atol=1e-14) and np.allclose(lse[b], lsep[0, :, -1], atol=1e-14)


def test_row_subset_equals_slice():
    rng = np.random.default_rng(21)
    q = rng.standard_normal((1, 2, 12, 4)); k = rng.standard_normal((1, 2, 12, 4)); v = rng.standard_normal((1, 2, 12, 4))
    rows = [0, 5, 11, 3]
    O, lse = oracle.attention(q, k, v, scale=0.5, causal=True, seqlens=[10], rows=rows)
    Of, lsef = oracle.attention(q, k, v, scale=0.5, causal=True, seqlens=[10])
    assert np.array_equal(O, Of[:, :, rows]) and np.array_equal(lse, lsef[:, :, rows])


def test_empty_and_degenerate():
    # No keys at all: O = 0, LSE = -inf.
    O, lse = attention_head(np.ones((2, 3)), np.zeros((0, 3)), np.zeros((0, 3)), scale=1.0)
    assert np.all(O == 0.0) and np.all(lse == -np.inf)
    # Constant V gives that constant regardless of scores.
    rng = np.random.default_rng(0)
    O, _ = attention_head(rng.standard_normal((4, 3)), rng.standard_normal((6, 3)), np.full((6, 3), 2.5), scale=3.0)
    assert np.allclose(O, 2.5, atol=1e-14)


def test_all_heads_pairs_enumerated():
    # Every (b, h) pair is evaluated exactly once when no subset is given.
    rng = np.random.default_rng(2)
    q = rng.standard_normal((2, 4, 3, 2)); k = rng.standard_normal((2, 2, 3, 2)); v = rng.standard_normal((2, 2, 3, 2))
    O, lse = oracle.attention(q, k, v, scale=1.0)
    assert np.isfinite(O).all() and np.isfinite(lse).all()
    for b, h in itertools.product(range(2), range(4)):
        Oh, lh = attention_head(q[b, h], k[b, h // 2], v[b, h // 2], scale=1.0)
        assert np.array_equal(O[b, h], Oh) and np.array_equal(lse[b, h], lh)
