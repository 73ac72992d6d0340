"""Pins for the paged-cache decode of the oracle (oracle.decode_paged).

* a contiguous cache cut into pages and scattered through a permuted block table decodes
  bit for bit like the contiguous cache through oracle.decode (itself pinned in
  tests/test_oracle.py), for several page sizes, contexts across page boundaries, GQA and
  a sliding window;
* one page per request with the identity table is the contiguous cache;
* planted mistakes (page index off by one, row within the page off by one, the page's
  head and row axes swapped) fail a pin.
"""
import numpy as np
import pytest

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _paginate(kc, P, seed):
    """Cut a contiguous cache [B, Hkv, Lmax, d] into pages [num_pages, Hkv, P, d] scattered by a
    random permutation; returns (pages, table)."""
    B, Hkv, Lmax, d = kc.shape
    mp = -(-Lmax // P)
    pad = np.zeros((B, Hkv, mp * P, d))
    pad[:, :, :Lmax] = kc
    perm = np.random.default_rng(seed).permutation(B * mp + 2)
    table = perm[:B * mp].reshape(B, mp)
    pages = _rand((B * mp + 2, Hkv, P, d), seed + 1)  # pages nobody names hold other data
    for b in range(B):
        for p in range(mp):
            pages[table[b, p]] = pad[b, :, p * P:(p + 1) * P]
    return pages, table


def pin_equals_contiguous(decode_paged):
    B, H, Hkv, Lmax, d = 3, 6, 2, 70, 5
    q, kc, vc = _rand((B, H, d), 1), _rand((B, Hkv, Lmax, d), 2), _rand((B, Hkv, Lmax, d), 3)
    ctx = np.array([70, 33, 1])
    for P in (4, 16, 32, 128):
        kp, table = _paginate(kc, P, 10 + P)
        vp, _ = _paginate(vc, P, 10 + P)
        for W in (None, 9):
            want = oracle.decode(q, kc, vc, ctx, scale=0.5, window=W)
            got = decode_paged(q, kp, vp, table, ctx, page_size=P, scale=0.5, window=W)
            np.testing.assert_array_equal(got[0], want[0], err_msg=f"P={P} W={W}")
            np.testing.assert_array_equal(got[1], want[1], err_msg=f"P={P} W={W}")


def pin_one_page_identity(decode_paged):
    B, H, Hkv, Lmax, d = 2, 2, 1, 40, 4
    q, kc, vc = _rand((B, H, d), 4), _rand((B, Hkv, Lmax, d), 5), _rand((B, Hkv, Lmax, d), 6)
    ctx = np.array([40, 17])
    table = np.arange(B).reshape(B, 1)
    got = decode_paged(q, kc, vc, table, ctx, page_size=Lmax, scale=0.3)
    want = oracle.decode(q, kc, vc, ctx, scale=0.3)
    np.testing.assert_array_equal(got[0], want[0])
    np.testing.assert_array_equal(got[1], want[1])


PINS = [pin_equals_contiguous, pin_one_page_identity]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_paged_pin(pin):
    pin(oracle.decode_paged)


def _mutant(kind):
    """A test-local paged decode with one planted indexing mistake."""
    def decode_paged(q, k_pages, v_pages, block_table, ctx_lens, *, page_size, scale, window=None):
        B, H, d = q.shape
        Hkv = k_pages.shape[1]
        O, L = np.zeros((B, H, d)), np.zeros((B, H))
        for b in range(B):
            n = int(ctx_lens[b])
            rows_k, rows_v = [], []
            for j in range(n):
                pi = j // page_size + (1 if kind == "page+1" and j >= page_size else 0)
                pi = min(pi, block_table.shape[1] - 1)
                r = (j % page_size + (1 if kind == "row+1" else 0)) % page_size
                pg = block_table[b, pi]
                rows_k.append(k_pages[pg, :, r] if kind != "swap" else k_pages[pg].reshape(page_size, Hkv, d)[r])
                rows_v.append(v_pages[pg, :, r] if kind != "swap" else v_pages[pg].reshape(page_size, Hkv, d)[r])
            K, V = np.stack(rows_k, axis=1), np.stack(rows_v, axis=1)  # [Hkv, n, d]
            for h in range(H):
                kvh = h // (H // Hkv)
                o, l = oracle.attention_head(q[b, h][None], K[kvh], V[kvh], scale=scale,
                                             causal=window is not None, window=window)
                O[b, h], L[b, h] = o[0], l[0]
        return O, L
    return decode_paged


def test_mutant_harness_is_faithful():
    for pin in PINS:
        pin(_mutant("none"))


@pytest.mark.parametrize("kind", ["page+1", "row+1", "swap"])
def test_planted_paging_mistake_fails_a_pin(kind):
    failed = 0
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin catches {kind}"
