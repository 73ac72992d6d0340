"""Pins for the sliding-window mask of the oracle, independent of its masking code.

The window is the causal mask cut to the W newest visible keys (reading of "FlashAttention
与长上下文", section on prefill and decode, where the sliding window is one of the
context-trimming methods): query i sees i + (Lk - Lq) - W < j <= i + (Lk - Lq).

* closed form: W = 1 leaves exactly one key per row, so O_i = V[i + Lk - Lq] and
  LSE_i = scale q_i . k_{i + Lk - Lq};
* brute force by slicing: each row's softmax over the keys k[lo:hi] taken out of the arrays
  (no mask), for ragged Lq != Lk and padding;
* special case: W >= the number of keys is plain causal attention;
* decode: the last W keys of the context, sliced;
* backward: central finite differences of the windowed forward;
* planted mistakes (off by one either way, the band on the wrong side) fail a pin.
"""
import importlib

import numpy as np
import pytest

import oracle
from oracle.attention import attention_head
from oracle.backward import attention_backward_head

A = importlib.import_module("oracle.attention")  # the module (the package exports a function of that name)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _slice_row(q_i, k, v, lo, hi, scale):
    """Softmax attention of one row over keys lo .. hi-1, written out directly."""
    if hi <= lo:
        return np.zeros(v.shape[1]), -np.inf
    s = scale * (k[lo:hi] @ q_i)
    m = s.max()
    e = np.exp(s - m)
    return e @ v[lo:hi] / e.sum(), m + np.log(e.sum())


CASES = [
    # (Lq, Lk, d, W, n_valid)
    (9, 9, 4, 1, None),
    (9, 9, 4, 3, None),
    (7, 12, 3, 4, None),   # Lq < Lk: the band starts at i + 5
    (12, 7, 3, 4, None),   # Lq > Lk: the first five rows see nothing
    (10, 10, 5, 6, 7),     # padding rows and keys
    (6, 6, 2, 100, None),  # window wider than the sequence
]


def pin_slices(head):
    for c, (Lq, Lk, d, W, n) in enumerate(CASES):
        q, k, v = _rand((Lq, d), 100 + c), _rand((Lk, d), 200 + c), _rand((Lk, d), 300 + c)
        O, L = head(q, k, v, scale=0.6, causal=True, n_valid=n, window=W)
        nk = Lk if n is None else n
        for i in range(Lq):
            if n is not None and i >= n:
                want_o, want_l = np.zeros(d), -np.inf
            else:
                hi = min(i + (Lk - Lq) + 1, nk)
                lo = max(i + (Lk - Lq) - W + 1, 0)
                want_o, want_l = _slice_row(q[i], k, v, lo, hi, 0.6)
            np.testing.assert_allclose(O[i], want_o, rtol=1e-12, atol=1e-12, err_msg=f"case {c} row {i}")
            assert (L[i] == want_l) or abs(L[i] - want_l) < 1e-12, (c, i, L[i], want_l)


def pin_window_one(head):
    q, k, v = _rand((8, 5), 1), _rand((11, 5), 2), _rand((11, 5), 3)
    O, L = head(q, k, v, scale=0.3, causal=True, window=1)
    for i in range(8):
        j = i + 3
        np.testing.assert_allclose(O[i], v[j], rtol=1e-13, atol=1e-13)
        assert abs(L[i] - 0.3 * float(q[i] @ k[j])) < 1e-12


def pin_wide_window_is_causal(head):
    q, k, v = _rand((10, 4), 4), _rand((13, 4), 5), _rand((13, 4), 6)
    O, L = head(q, k, v, scale=0.5, causal=True, window=13)
    O0, L0 = attention_head(q, k, v, scale=0.5, causal=True)
    np.testing.assert_array_equal(O, O0)
    np.testing.assert_array_equal(L, L0)


PINS = [pin_slices, pin_window_one, pin_wide_window_is_causal]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_window_pin(pin):
    pin(attention_head)


def _mutant(shift_lo=0, shift_hi=0, flip=False):
    """attention_head with a planted mistake in the window mask (test-local copy of the mask)."""
    def visible(Lq, Lk, causal, n_valid, rows=None, window=None):
        i = np.arange(Lq) if rows is None else np.asarray(rows)
        j = np.arange(Lk)
        vis = np.broadcast_to(j[None, :] < n_valid, (len(i), Lk)).copy()
        if causal:
            vis &= j[None, :] <= (i[:, None] + (Lk - Lq) + shift_hi)
        if window is not None:
            if flip:
                vis &= j[None, :] < (i[:, None] + (Lk - Lq) + window)
            else:
                vis &= j[None, :] > (i[:, None] + (Lk - Lq) - window + shift_lo)
        return vis

    def head(*args, **kw):
        saved = A._visible
        A._visible = visible
        try:
            return attention_head(*args, **kw)
        finally:
            A._visible = saved
    return head


def test_mutant_harness_is_faithful():
    for pin in PINS:
        pin(_mutant())


@pytest.mark.parametrize("kind", ["lo+1", "lo-1", "hi+1", "flip"])
def test_planted_window_mistake_fails_a_pin(kind):
    head = {"lo+1": _mutant(shift_lo=1), "lo-1": _mutant(shift_lo=-1), "hi+1": _mutant(shift_hi=1),
            "flip": _mutant(flip=True)}[kind]
    failed = 0
    for pin in PINS:
        try:
            pin(head)
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin catches {kind}"


def test_decode_window_is_last_keys_sliced():
    B, H, Hkv, Lmax, d = 3, 4, 2, 40, 8
    q, kc, vc = _rand((B, H, d), 7), _rand((B, Hkv, Lmax, d), 8), _rand((B, Hkv, Lmax, d), 9)
    ctx = np.array([40, 17, 3])
    for W in (1, 5, 16, 64):
        O, L = oracle.decode(q, kc, vc, ctx, scale=0.4, window=W)
        for b in range(B):
            for h in range(H):
                n = int(ctx[b])
                o, l = _slice_row(q[b, h], kc[b, h // 2], vc[b, h // 2], max(0, n - W), n, 0.4)
                np.testing.assert_allclose(O[b, h], o, rtol=1e-12, atol=1e-12)
                assert abs(L[b, h] - l) < 1e-12


def test_backward_window_matches_finite_differences():
    h = 1e-5
    for c, (Lq, Lk, d, W, n) in enumerate([(6, 6, 3, 2, None), (5, 8, 2, 3, None), (7, 7, 2, 3, 5)]):
        q, k, v, do = _rand((Lq, d), 50 + c), _rand((Lk, d), 60 + c), _rand((Lk, d), 70 + c), _rand((Lq, d), 80 + c)

        def loss(qq, kk, vv):
            O, _ = attention_head(qq, kk, vv, scale=0.7, causal=True, n_valid=n, window=W)
            return float((O * do).sum())
        got = attention_backward_head(q, k, v, do, scale=0.7, causal=True, n_valid=n, window=W)
        for which, g in enumerate(got):
            base = [q, k, v]
            want = np.zeros_like(base[which])
            for idx in np.ndindex(*want.shape):
                plus = [t.copy() for t in base]
                minus = [t.copy() for t in base]
                plus[which][idx] += h
                minus[which][idx] -= h
                want[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
            np.testing.assert_allclose(g, want, rtol=1e-6, atol=1e-7, err_msg=f"case {c} grad {'QKV'[which]}")


def test_window_needs_causal():
    q = _rand((3, 2), 1)
    with pytest.raises(AssertionError):
        attention_head(q, q, q, scale=1.0, causal=False, window=2)
