"""Pins for the FP8 attention oracle (oracle/fp8.py), independent of its own code.

* its E4M3 decoding and rounding against torch's float8_e4m3fn conversion (another
  implementation) over every code and over random values, ties and subnormals;
* closed forms: one visible key with an integer base-2 score gives O = V and LSE = ln2 * t;
  a zero query gives scores 0, an exact reference and O = mean(V);
* a hand-rounded case: probabilities (1, 0.3) become 256 and e4m3(76.8) = 80 before the
  product, so O = (256 v1 + 80 v2) / (256 * 1.3);
* the rounding error bound: each probability is off by at most 2^-4 of itself, so
  |O - O_exact| <= 2^-4 max_j |V_j - O_exact| row by row;
* power-of-two invariance: shifting every score by an integer in base 2 changes nothing;
* planted mistakes (no rounding, a P scale of 2^9, rounding toward zero) fail a pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as F
from oracle.attention import attention_head


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    np.testing.assert_array_equal(ours[~np.isnan(ours)], ref[~np.isnan(ref)])


def test_round_matches_torch_conversion():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0,
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000),               # subnormal range
        np.array([76.8, 0.0, -0.0, 448.0, 2.0 ** -9, 1.5 * 2.0 ** -10, 2.0 ** -10]),
        # midpoints between neighbouring values (ties to even)
        (F.e4m3_decode(np.arange(0, 126)) + F.e4m3_decode(np.arange(1, 127))) / 2,
    ])
    x = x[np.abs(x) <= 448]
    ours = F.e4m3_round(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def pin_single_key(fn):
    """One visible key whose base-2 score is an integer: its probability relative to the
    integer reference is exactly 1, 256 is an E4M3 value, so O = V and LSE = ln2 * t."""
    scale = 0.4
    n = np.array([3.0, -2.0, 5.0, 0.0, 1.0])
    q = np.zeros((3, 8)); q[:, 0] = 1.0
    k = np.zeros((5, 8)); k[:, 0] = n / (scale * np.log2(np.e))
    v = _rand((5, 8), 3)
    # causal with Lq = 3, Lk = 5 and a window of 1: row i sees key i + 2 only
    O, L = fn(q, k, v, scale=scale, causal=True, window=1)
    for i in range(3):
        np.testing.assert_allclose(O[i], v[i + 2], rtol=1e-12, atol=1e-12)
        assert abs(L[i] - math.log(2) * n[i + 2]) < 1e-12


def pin_zero_query_mean(fn):
    q = np.zeros((2, 6))
    k, v = _rand((7, 6), 4), _rand((7, 6), 5)
    O, L = fn(q, k, v, scale=0.9)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(axis=0), O.shape), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(L, math.log(7), rtol=1e-14)


def pin_hand_rounded(fn):
    scale = 0.5
    q = np.array([[1.0, 0.0]])
    k = np.array([[0.0, 0.0], [math.log(0.3) / scale, 0.0]])  # t = (0, log2 0.3)
    v = np.array([[1.0, 2.0], [-3.0, 5.0]])
    O, L = fn(q, k, v, scale=scale)
    want = (256 * v[0] + 80 * v[1]) / (256 * 1.3)
    np.testing.assert_allclose(O[0], want, rtol=1e-12)
    assert abs(L[0] - math.log(1.3)) < 1e-12


def pin_error_bound(fn):
    for seed in range(4):
        q, k, v = _rand((40, 16), 10 + seed), _rand((90, 16), 20 + seed), _rand((90, 16), 30 + seed)
        O, L = fn(q, k, v, scale=0.3, causal=True)
        Oe, Le = attention_head(q, k, v, scale=0.3, causal=True)
        for i in range(40):
            vis = np.arange(90) <= i + 50
            bound = 2.0 ** -4 * np.abs(v[vis] - Oe[i]).max(axis=0) + 1e-12
            assert np.all(np.abs(O[i] - Oe[i]) <= bound), (seed, i)
        np.testing.assert_allclose(L, Le, rtol=1e-12, atol=1e-12)


def pin_power_of_two_shift(fn):
    q, k, v = _rand((12, 8), 40), _rand((20, 8), 41), _rand((20, 8), 42)
    O, L = fn(q, k, v, scale=0.7)
    # add an integer (in base 2) to every score of a row through an extra dimension
    shift = 3.0 / (0.7 * np.log2(np.e))
    q2 = np.concatenate([q, np.ones((12, 1))], axis=1)
    k2 = np.concatenate([k, np.full((20, 1), shift)], axis=1)
    O2, L2 = fn(q2, k2, v, scale=0.7)
    np.testing.assert_allclose(O2, O, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L2, L + 3.0 * math.log(2), rtol=1e-12)


PINS = [pin_single_key, pin_zero_query_mean, pin_hand_rounded, pin_error_bound, pin_power_of_two_shift]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_fp8_oracle_pin(pin):
    pin(F.attention_fp8_head)


def _mutant(kind):
    def fn(q, k, v, **kw):
        saved = F.e4m3_round
        if kind == "no_round":
            F.e4m3_round = lambda x: np.asarray(x, dtype=np.float64)
        elif kind == "toward_zero":
            def rz(x):
                x = np.asarray(x, dtype=np.float64)
                a = np.abs(x)
                _, E = np.frexp(np.where(a > 0, a, 1.0))
                qq = 2.0 ** (np.maximum(E - 1.0, -6.0) - 3.0)
                return np.sign(x) * np.floor(a / qq) * qq
            F.e4m3_round = rz
        try:
            if kind == "p_scale_512":
                return F.attention_fp8_head(q, k, v, p_scale=512.0, **kw)
            return F.attention_fp8_head(q, k, v, **kw)
        finally:
            F.e4m3_round = saved
    return fn


def test_mutant_harness_is_faithful():
    for pin in PINS:
        pin(_mutant("none"))


@pytest.mark.parametrize("kind", ["no_round", "p_scale_512", "toward_zero"])
def test_planted_fp8_mistake_fails_a_pin(kind):
    failed = 0
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin catches {kind}"


def test_batched_wrapper_dequantises_per_head():
    rng = np.random.default_rng(50)
    B, H, Hkv, L, d = 2, 4, 2, 9, 16
    q8 = rng.integers(0, 0x7e, (B, H, L, d), dtype=np.uint8)
    k8 = rng.integers(0, 0x7e, (B, Hkv, L, d), dtype=np.uint8)
    v8 = rng.integers(0, 0x7e, (B, Hkv, L, d), dtype=np.uint8)
    qs, ks, vs = rng.uniform(0.01, 0.1, (B, H)), rng.uniform(0.01, 0.1, (B, Hkv)), rng.uniform(0.5, 2, (B, Hkv))
    O, L_ = oracle.attention_fp8(q8, k8, v8, qs, ks, vs, scale=0.25, causal=True)
    for b in range(B):
        for h in range(H):
            kvh = h // 2
            o, l = F.attention_fp8_head(F.e4m3_decode(q8[b, h]) * qs[b, h], F.e4m3_decode(k8[b, kvh]) * ks[b, kvh],
                                        F.e4m3_decode(v8[b, kvh]) * vs[b, kvh], scale=0.25, causal=True)
            np.testing.assert_array_equal(O[b, h], o)
            np.testing.assert_array_equal(L_[b, h], l)


def test_flip_allowance_marks_only_near_midpoint_probabilities():
    """parity.fp8_flip_slack: zero when every probability is far from an E4M3 midpoint, and one
    spacing's worth when a probability sits on one."""
    from parity import fp8_flip_slack
    scale = 0.5
    # t = (0, -1): x = 256 and 128, both E4M3 values, far from midpoints
    q = np.array([[1.0, 0.0]])
    k = np.array([[0.0, 0.0], [-1.0 / (scale * np.log2(np.e)), 0.0]])
    v = np.array([[1.0, 0.0], [3.0, 0.0]])
    assert fp8_flip_slack(q, k, v, scale=scale)[0] == 0.0
    # x2 = 256 * 2^t2 = 136, the midpoint between 128 and 144 (spacing 16)
    k2 = np.array([[0.0, 0.0], [np.log2(136 / 256) / (scale * np.log2(np.e)), 0.0]])
    got = fp8_flip_slack(q, k2, v, scale=scale)[0]
    assert abs(got - 16.0 * 3.0 / (256 + 136)) < 1e-9
