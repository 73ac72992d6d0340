"""Pins for the backward oracle (oracle/backward.py), independent of the oracle itself.

* central finite differences of the forward oracle (the definition of O), on tiny heads;
* torch autograd through float64 scaled_dot_product_attention (a library routine);
* invariants: sum_j dK_j = 0, sum_j dV_j = sum of dO over rows that see a key;
* GQA = the sum over query heads of the same computation with repeated K/V;
* planted mistakes (wrong sign, missing term or factor, transposes) must each fail a pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import attention_head
from oracle.backward import attention_backward, attention_backward_head


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _fd_grads(q, k, v, do, *, scale, causal, n_valid, h=1e-5):
    """Central differences of L = sum(O * dO) with respect to every entry of q, k and v."""
    def loss(qq, kk, vv):
        O, _ = attention_head(qq, kk, vv, scale=scale, causal=causal, n_valid=n_valid)
        return float((O * do).sum())
    grads = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(base[which])
        for idx in np.ndindex(*g.shape):
            plus = [t.copy() for t in base]
            minus = [t.copy() for t in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return grads


FD_CASES = [
    # (Lq, Lk, d, causal, n_valid)
    (4, 4, 3, False, None),
    (4, 4, 3, True, None),
    (3, 5, 4, True, None),    # bottom-right alignment, Lq < Lk
    (5, 3, 2, True, None),    # Lq > Lk: the first two rows see nothing
    (5, 5, 3, True, 3),       # padding rows and keys
    (6, 6, 2, False, 4),
]


def pin_finite_differences(bwd):
    for i, (Lq, Lk, d, causal, n) in enumerate(FD_CASES):
        q, k, v, do = _rand((Lq, d), 10 + i), _rand((Lk, d), 20 + i), _rand((Lk, d), 30 + i), _rand((Lq, d), 40 + i)
        scale = 0.7
        want = _fd_grads(q, k, v, do, scale=scale, causal=causal, n_valid=n)
        got = bwd(q, k, v, do, scale=scale, causal=causal, n_valid=n)
        for name, g, w in zip("QKV", got, want):
            np.testing.assert_allclose(g, w, rtol=1e-6, atol=1e-8, err_msg=f"d{name} case {i}")


def pin_torch_autograd(bwd):
    for causal in (False, True):
        L, d = 9, 5
        q, k, v, do = _rand((L, d), 51), _rand((L, d), 52), _rand((L, d), 53), _rand((L, d), 54)
        scale = 1.0 / math.sqrt(d)
        tq, tk, tv = (torch.tensor(t, requires_grad=True) for t in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None],
                                                             is_causal=causal, scale=scale)[0, 0]
        o.backward(torch.tensor(do))
        got = bwd(q, k, v, do, scale=scale, causal=causal, n_valid=None)
        for name, g, t in zip("QKV", got, (tq, tk, tv)):
            np.testing.assert_allclose(g, t.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=f"d{name} causal={causal}")


def pin_zero_sums(bwd):
    for causal, n in ((False, None), (True, None), (True, 13)):
        Lq = Lk = 17
        d = 6
        q, k, v, do = _rand((Lq, d), 61), _rand((Lk, d), 62), _rand((Lk, d), 63), _rand((Lq, d), 64)
        dQ, dK, dV = bwd(q, k, v, do, scale=0.4, causal=causal, n_valid=n)
        np.testing.assert_allclose(dK.sum(axis=0), 0.0, atol=1e-12)
        rows = np.arange(Lq) < (Lq if n is None else n)
        np.testing.assert_allclose(dV.sum(axis=0), do[rows].sum(axis=0), rtol=1e-12, atol=1e-12)


def _oracle_bwd(q, k, v, do, *, scale, causal, n_valid):
    return attention_backward_head(q, k, v, do, scale=scale, causal=causal, n_valid=n_valid)


PINS = [pin_finite_differences, pin_torch_autograd, pin_zero_sums]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_backward_oracle_meets_pin(pin):
    pin(_oracle_bwd)


def _mutant(kind):
    def bwd(q, k, v, do, *, scale, causal, n_valid):
        O, _, P = attention_head(q, k, v, scale=scale, causal=causal, n_valid=n_valid, return_p=True)
        dV = P.T @ do
        dP = do @ v.T
        D = (do * O).sum(axis=1)
        dS = P * (dP - D[:, None])
        dQ = scale * (dS @ k)
        dK = scale * (dS.T @ q)
        if kind == "no_D":
            dS = P * dP
            dQ, dK = scale * (dS @ k), scale * (dS.T @ q)
        elif kind == "dQ_no_scale":
            dQ = dS @ k
        elif kind == "dK_scale_squared":
            dK = scale * scale * (dS.T @ q)
        elif kind == "dV_untransposed_P":
            dV = P @ do  # shapes only agree when Lq == Lk; otherwise the pin fails by raising
        elif kind == "sign":
            dQ, dK = -dQ, -dK
        elif kind == "D_from_dP_unweighted":
            dS = P * (dP - dP.mean(axis=1, keepdims=True))
            dQ, dK = scale * (dS @ k), scale * (dS.T @ q)
        return dQ, dK, dV
    return bwd


MUTANTS = ["no_D", "dQ_no_scale", "dK_scale_squared", "dV_untransposed_P", "sign", "D_from_dP_unweighted"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_backward_mistake_fails_a_pin(kind):
    failed = False
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except (AssertionError, ValueError):
            failed = True
    assert failed, f"mutant {kind} passed every pin"


def test_gqa_equals_sum_over_repeated_heads():
    B, H, Hkv, L, d = 2, 6, 2, 11, 4
    q, do = _rand((B, H, L, d), 71), _rand((B, H, L, d), 72)
    k, v = _rand((B, Hkv, L, d), 73), _rand((B, Hkv, L, d), 74)
    dQ, dK, dV = attention_backward(q, k, v, do, scale=0.5, causal=True, seqlens=np.array([11, 7]))
    kr, vr = np.repeat(k, H // Hkv, axis=1), np.repeat(v, H // Hkv, axis=1)
    dQr, dKr, dVr = attention_backward(q, kr, vr, do, scale=0.5, causal=True, seqlens=np.array([11, 7]))
    np.testing.assert_allclose(dQ, dQr, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dK, dKr.reshape(B, Hkv, H // Hkv, L, d).sum(axis=2), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dV, dVr.reshape(B, Hkv, H // Hkv, L, d).sum(axis=2), rtol=1e-12, atol=1e-12)


def test_padding_rows_and_unseen_keys_get_zero_gradients():
    L, d, n = 9, 4, 6
    q, k, v, do = _rand((L, d), 81), _rand((L, d), 82), _rand((L, d), 83), _rand((L, d), 84)
    dQ, dK, dV = attention_backward_head(q, k, v, do, scale=0.5, causal=True, n_valid=n)
    assert np.all(dQ[n:] == 0) and np.all(dK[n:] == 0) and np.all(dV[n:] == 0)
    # Lq > Lk with bottom-right causal: the first Lq - Lk rows see nothing
    q2, do2 = _rand((7, d), 85), _rand((7, d), 86)
    dQ2, _, _ = attention_backward_head(q2, k[:4], v[:4], do2, scale=0.5, causal=True)
    assert np.all(dQ2[:3] == 0)


def test_package_exports_backward():
    assert oracle.attention_backward is attention_backward
