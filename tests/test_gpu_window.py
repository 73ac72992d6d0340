"""GPU parity of the sliding-window entry points (fa_fwd_sliding_window,
fa_decode_sliding_window, fa_bwd_sliding_window) against the fp64 oracle, through the C ABI.

The window keeps the causal band of the W newest visible keys per query; the oracle's
reading and pins are in tests/test_oracle_window.py. Tolerances as for the plain entry
points (parity.compare, parity.compare_grad).
"""
import math
import sys

import numpy as np
import pytest
import torch

import fa_inputs
import oracle
from parity import compare, compare_grad, grad_tolerances

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fa():
    import exact_attention_111_amd as fa
    return fa


def announce(**case):
    print("\n[case] " + " ".join(f"{k}={v}" for k, v in case.items()), flush=True)
    sys.stdout.flush()


def run_fwd(B, H, Hkv, Lq, Lk, d, W, *, seed, len_range=None):
    announce(entry="fa_fwd_sliding_window", B=B, H=H, Hkv=Hkv, Lq=Lq, Lk=Lk, d=d, W=W, seed=seed,
             len_range=len_range)
    x = fa_inputs.prefill_inputs(B, H, Hkv, Lq, Lk, d, seed=seed, device=DEV, len_range=len_range)
    scale = 1.0 / math.sqrt(d)
    o, lse = _fa().fwd(x["q"], x["k"], x["v"], causal=True, scale=scale, seqlens=x["seqlens"], window=W)
    torch.cuda.synchronize()
    sl = None if x["seqlens_cpu"] is None else x["seqlens_cpu"].numpy()
    q64, k64, v64 = (fa_inputs.as_oracle_f64(x[n]) for n in ("q", "k", "v"))
    O, LSE = oracle.attention(q64, k64, v64, scale=scale, causal=True, seqlens=sl, window=W)
    compare(o, lse, O, LSE, bf16_out=True, what=f"window B{B} H{H}/{Hkv} L{Lq}x{Lk} d{d} W{W}")
    return x, o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("W", [1, 37, 64, 200, 1000])
def test_window_prefill_ragged_gqa(d, W):
    # 300 rows: two 256-row query tiles (the second ragged), band edges inside and across
    # 64-key tiles; W = 1 leaves only the diagonal key, W = 1000 is wider than the sequence.
    x, o, _ = run_fwd(2, 4, 2, 300, 300, d, W, seed=400 + W + d)
    if W == 1:  # O_i = V[i] exactly
        assert torch.equal(o, x["v"].repeat_interleave(2, dim=1))


@pytest.mark.parametrize("Lq,Lk", [(100, 333), (333, 100), (1, 700)])
def test_window_unequal_lengths(Lq, Lk):
    run_fwd(1, 2, 1, Lq, Lk, 128, 50, seed=410 + Lq)


def test_window_varlen():
    run_fwd(3, 4, 2, 700, 700, 128, 130, seed=420, len_range=(1, 700))


def test_wide_window_equals_causal_bitwise():
    announce(entry="fa_fwd_sliding_window vs fa_fwd", B=1, H=4, L=600, d=128, W=600)
    x = fa_inputs.prefill_inputs(1, 4, 4, 600, 600, 128, seed=430, device=DEV)
    o1, l1 = _fa().fwd(x["q"], x["k"], x["v"], causal=True, window=600)
    o2, l2 = _fa().fwd(x["q"], x["k"], x["v"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_window_full_size_16k_sampled():
    """The 16,384-token causal workload with a 4096-key window, in the launch configuration
    bench.py times, on sampled rows of two heads."""
    w = fa_inputs.WORKLOADS["causal_prefill_B1_H32_L16384_d128"]
    W = 4096
    announce(entry="fa_fwd_sliding_window", workload=w.name, W=W, case="sampled rows")
    x = fa_inputs.workload_inputs(w, device=DEV)
    o, lse = _fa().fwd(x["q"], x["k"], x["v"], causal=True, scale=w.scale, window=W)
    torch.cuda.synchronize()
    rng = np.random.default_rng(431)
    rows = np.sort(np.concatenate([[0, 1, 255, 256, 4095, 4096, 4097, w.L - 1], rng.choice(w.L, 24, replace=False)]))
    for h in (0, 29):
        O, LSE = oracle.attention_head(*(fa_inputs.as_oracle_f64(x[n][0, h]) for n in ("q", "k", "v")),
                                       scale=w.scale, causal=True, rows=rows, window=W)
        compare(o[0, h, rows], lse[0, h, rows], O, LSE, bf16_out=True, what=f"16k W{W} head {h}")


@pytest.mark.parametrize("W", [1, 100, 2048, 3000, 10000])
def test_window_decode_chunks(W):
    """Contexts across 2048-key boundaries; windows of one key, inside 2048 keys, exactly 2048,
    across two 2048-key spans, and wider than every context. Windows of 1 and 100 keys take
    the chunk grid with shortened chunks (512 keys at this shape); windows of 2048 keys and
    more take the balanced partition, each unit's steps running from the one holding its
    window's first key and workgroups spanning several units."""
    B, H, Hkv, Lmax, d = 5, 8, 2, 5000, 128
    announce(entry="fa_decode_sliding_window", B=B, H=H, Hkv=Hkv, Lmax=Lmax, W=W)
    x = fa_inputs.decode_inputs(B, H, Hkv, Lmax, d, seed=440 + W, device=DEV)
    ctx = torch.tensor([1, 2047, 2048, 4500, 5000], dtype=torch.int32)
    scale = 1.0 / math.sqrt(d)
    o, lse = _fa().decode(x["q"], x["k_cache"], x["v_cache"], ctx.to(DEV), scale=scale, window=W)
    torch.cuda.synchronize()
    O, LSE = oracle.decode(*(fa_inputs.as_oracle_f64(x[n]) for n in ("q", "k_cache", "v_cache")), ctx.numpy(),
                           scale=scale, window=W)
    compare(o, lse, O, LSE, bf16_out=True, what=f"decode W{W}")


@pytest.mark.parametrize("W", [1, 700])
def test_window_decode_single_chunk(W):
    """A cache of at most 2048 keys takes the grid of 2048-key chunks (one per request and KV
    head), with the window's first key inside the chunk."""
    B, H, Hkv, Lmax, d = 3, 8, 2, 2000, 128
    announce(entry="fa_decode_sliding_window", B=B, H=H, Hkv=Hkv, Lmax=Lmax, W=W, case="chunk grid")
    x = fa_inputs.decode_inputs(B, H, Hkv, Lmax, d, seed=460 + W, device=DEV)
    ctx = torch.tensor([1, 1999, 2000], dtype=torch.int32)
    scale = 1.0 / math.sqrt(d)
    o, lse = _fa().decode(x["q"], x["k_cache"], x["v_cache"], ctx.to(DEV), scale=scale, window=W)
    torch.cuda.synchronize()
    O, LSE = oracle.decode(*(fa_inputs.as_oracle_f64(x[n]) for n in ("q", "k_cache", "v_cache")), ctx.numpy(),
                           scale=scale, window=W)
    compare(o, lse, O, LSE, bf16_out=True, what=f"decode chunk grid W{W}")


def test_window_decode_ignores_nan_before_window():
    """Cache positions before the window are never read: NaN there changes nothing."""
    B, H, Hkv, Lmax, d, W = 2, 4, 1, 4200, 64, 1500
    announce(entry="fa_decode_sliding_window", case="NaN before the window", W=W)
    x = fa_inputs.decode_inputs(B, H, Hkv, Lmax, d, seed=450, device=DEV)
    ctx = torch.tensor([4200, 2100], dtype=torch.int32, device=DEV)
    o1, l1 = _fa().decode(x["q"], x["k_cache"], x["v_cache"], ctx, window=W)
    kc, vc = x["k_cache"].clone(), x["v_cache"].clone()
    kc[0, :, :4200 - W] = float("nan"); vc[0, :, :4200 - W] = float("nan")
    kc[1, :, :2100 - W] = float("nan"); vc[1, :, :2100 - W] = float("nan")
    o2, l2 = _fa().decode(x["q"], kc, vc, ctx, window=W)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("W", [1, 40, 200])
def test_window_backward(d, W):
    B, H, Hkv, L = 2, 4, 2, 300
    announce(entry="fa_bwd_sliding_window", B=B, H=H, Hkv=Hkv, L=L, d=d, W=W)
    x = fa_inputs.prefill_inputs(B, H, Hkv, L, L, d, seed=460 + W + d, device=DEV)
    scale = 1.0 / math.sqrt(d)
    o, lse = _fa().fwd(x["q"], x["k"], x["v"], causal=True, scale=scale, window=W)
    g = torch.Generator(device=DEV).manual_seed(461 + W)
    do = torch.randn(o.shape, generator=g, device=DEV).to(torch.bfloat16)
    dq, dk, dv = _fa().bwd(x["q"], x["k"], x["v"], o, do, lse, causal=True, scale=scale, window=W)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = (fa_inputs.as_oracle_f64(t) for t in (x["q"], x["k"], x["v"], do))
    dQ, dK, dV = oracle.attention_backward(q64, k64, v64, do64, scale=scale, causal=True, window=W)
    # W = 1: one key per row, P = 1 whatever the score, so the exact dQ and dK are zero; the
    # allowance of those elements is the rounding of dP - D (its 2 P Delta term).
    tQ, tK, tV = grad_tolerances(q64, k64, v64, do64, scale=scale, causal=True, window=W)
    compare_grad(dq, dQ, f"dQ d{d} W{W}", tQ)
    compare_grad(dk, dK, f"dK d{d} W{W}", tK)
    compare_grad(dv, dV, f"dV d{d} W{W}", tV)


def test_window_backward_varlen_unequal():
    d, W = 128, 70
    for (Lq, Lk, lr, seed) in [(300, 300, (1, 300), 470), (120, 290, None, 471), (290, 120, None, 472)]:
        announce(entry="fa_bwd_sliding_window", Lq=Lq, Lk=Lk, W=W, len_range=lr)
        x = fa_inputs.prefill_inputs(3 if lr else 1, 2, 1, Lq, Lk, d, seed=seed, device=DEV, len_range=lr)
        o, lse = _fa().fwd(x["q"], x["k"], x["v"], causal=True, seqlens=x["seqlens"], window=W)
        do = torch.randn(o.shape, device=DEV, generator=torch.Generator(device=DEV).manual_seed(seed)).to(torch.bfloat16)
        dq, dk, dv = _fa().bwd(x["q"], x["k"], x["v"], o, do, lse, causal=True, seqlens=x["seqlens"], window=W)
        torch.cuda.synchronize()
        sl = None if x["seqlens_cpu"] is None else x["seqlens_cpu"].numpy()
        q64, k64, v64, do64 = (fa_inputs.as_oracle_f64(t) for t in (x["q"], x["k"], x["v"], do))
        dQ, dK, dV = oracle.attention_backward(q64, k64, v64, do64, scale=1.0 / math.sqrt(d), causal=True,
                                               seqlens=sl, window=W)
        tQ, tK, tV = grad_tolerances(q64, k64, v64, do64, scale=1.0 / math.sqrt(d), causal=True, seqlens=sl,
                                     window=W)
        compare_grad(dq, dQ, f"dQ {Lq}x{Lk}", tQ)
        compare_grad(dk, dK, f"dK {Lq}x{Lk}", tK)
        compare_grad(dv, dV, f"dV {Lq}x{Lk}", tV)


@pytest.mark.parametrize("W", [0, 16, 100])
def test_scores_far_below_zero(W):
    """Every score is about -100 (natural log units), so 2^(s * scale * log2 e) underflows to
    zero when taken against a shift of 0. With a narrow window most rows of a query tile meet
    their first visible key after the tile's first key tile; they must still take a reference
    from those keys rather than keep an all-zero sum (LSE would read -inf)."""
    fa = _fa()
    B, H, L, d = 1, 2, 400, 128
    announce(entry="fa_fwd_sliding_window" if W else "fa_fwd", case="scores far below zero", B=B, H=H, L=L, d=d, W=W)
    g = torch.Generator().manual_seed(470 + W)
    q = torch.randn(B, H, L, d, generator=g) * 0.5
    k = torch.randn(B, H, L, d, generator=g) * 0.5
    v = torch.randn(B, H, L, d, generator=g)
    scale = 1.0 / math.sqrt(d)
    q[..., 0] = 10.0 / scale
    k[..., 0] = -10.0
    q, k, v = (t.to(torch.bfloat16).to(DEV) for t in (q, k, v))
    o, lse = fa.fwd(q, k, v, causal=True, scale=scale, window=W or None)
    torch.cuda.synchronize()
    O, LSE = oracle.attention(*(fa_inputs.as_oracle_f64(t) for t in (q, k, v)), scale=scale, causal=True,
                              window=W or None)
    assert np.isfinite(LSE).all() and LSE.max() < -80
    compare(o, lse, O, LSE, bf16_out=True, what=f"scores far below zero W{W}")
