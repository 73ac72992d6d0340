"""GPU parity of fa_bwd against the fp64 backward oracle (through the C ABI).

Gradients have no tolerance of their own on the pages; the bound (``parity.compare_grad``)
comes from the arithmetic of the kernels and is applied element by element: P and dS enter
the products as bf16 (one rounding, at most 2^-8 relative) with fp32 accumulation, D comes
from the forward's bf16 O, and dQ, dK, dV are rounded to bf16. Each element may be off by
2^-7 of the sum of the absolute values of its terms, plus half a bf16 ulp of itself
(``parity.grad_tolerances``).
"""
import math
import sys

import numpy as np
import pytest
import torch

import fa_inputs
import oracle
from parity import GRAD_REL, compare_grad as _close, grad_keys_oracle, grad_rows_oracle, grad_tolerances, report

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fa():
    import exact_attention_111_amd as fa
    return fa


def announce(**case):
    print("\n[case] " + " ".join(f"{k}={v}" for k, v in case.items()), flush=True)
    sys.stdout.flush()


def _dout(shape, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)


def run_bwd(B, H, Hkv, Lq, Lk, d, *, causal, seed, len_range=None):
    fa = _fa()
    announce(entry="fa_bwd", B=B, H=H, Hkv=Hkv, Lq=Lq, Lk=Lk, d=d, causal=causal, seed=seed, len_range=len_range)
    x = fa_inputs.prefill_inputs(B, H, Hkv, Lq, Lk, d, seed=seed, device=DEV, len_range=len_range)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.fwd(x["q"], x["k"], x["v"], causal=causal, scale=scale, seqlens=x["seqlens"])
    do = _dout(o.shape, seed + 1000)
    dq, dk, dv = fa.bwd(x["q"], x["k"], x["v"], o, do, lse, causal=causal, scale=scale, seqlens=x["seqlens"])
    torch.cuda.synchronize()
    sl = None if x["seqlens_cpu"] is None else x["seqlens_cpu"].numpy()
    q64, k64, v64, do64 = (fa_inputs.as_oracle_f64(t) for t in (x["q"], x["k"], x["v"], do))
    dQ, dK, dV = oracle.attention_backward(q64, k64, v64, do64, scale=scale, causal=causal, seqlens=sl)
    tQ, tK, tV = grad_tolerances(q64, k64, v64, do64, scale=scale, causal=causal, seqlens=sl)
    tag = f"B{B} H{H}/{Hkv} L{Lq}x{Lk} d{d} c{int(causal)}"
    # With a single key every row that sees anything has P = 1 whatever its score, so the
    # exact dQ and dK are zero; what the kernel returns is the rounding of dP - D, which the
    # allowance of those elements covers (its 2 P Delta term).
    _close(dq, dQ, "dQ " + tag, tQ)
    _close(dk, dK, "dK " + tag, tK)
    _close(dv, dV, "dV " + tag, tV)
    return x, dq, dk, dv


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ragged_multi_tile_gqa(d, causal):
    # 300 rows = 2 x 128 + 44 (dQ blocks) and 2 x 128 + 44 keys (dK/dV blocks); 2 query heads per KV head
    run_bwd(2, 4, 2, 300, 300, d, causal=causal, seed=200 + d + int(causal))


@pytest.mark.parametrize("Lq,Lk", [(100, 333), (200, 70), (1, 257), (257, 1)])
def test_bwd_unequal_lengths(Lq, Lk):
    run_bwd(1, 2, 1, Lq, Lk, 128, causal=True, seed=210 + Lq)


def test_bwd_varlen_padding_is_zero():
    x, dq, dk, dv = run_bwd(3, 4, 2, 300, 300, 128, causal=True, seed=220, len_range=(1, 300))
    for b, n in enumerate(x["seqlens_cpu"].tolist()):
        assert torch.all(dq[b, :, n:] == 0) and torch.all(dk[b, :, n:] == 0) and torch.all(dv[b, :, n:] == 0)


def test_bwd_gqa_matches_repeated_kv():
    fa = _fa()
    announce(entry="fa_bwd", case="GQA vs repeated KV", B=1, H=8, Hkv=2, L=260, d=128)
    x = fa_inputs.prefill_inputs(1, 8, 2, 260, 260, 128, seed=230, device=DEV)
    o, lse = fa.fwd(x["q"], x["k"], x["v"], causal=True)
    do = _dout(o.shape, 231)
    dq, dk, dv = fa.bwd(x["q"], x["k"], x["v"], o, do, lse, causal=True)
    kr = x["k"].repeat_interleave(4, dim=1).contiguous()
    vr = x["v"].repeat_interleave(4, dim=1).contiguous()
    dq2, dk2, dv2 = fa.bwd(x["q"], kr, vr, o, do, lse, causal=True)
    assert torch.equal(dq, dq2)  # dQ does not depend on how K/V are shared
    for g, g2 in ((dk, dk2), (dv, dv2)):
        summed = g2.float().view(1, 2, 4, 260, 128).sum(dim=2)
        err = (g.float() - summed).abs().max() / summed.abs().max()
        assert err < 2.0 ** -7, float(err)


def test_bwd_empty_calls():
    fa = _fa()
    announce(entry="fa_bwd", case="empty and degenerate")
    # no query rows: dK = dV = 0
    q = torch.zeros(1, 2, 0, 64, device=DEV, dtype=torch.bfloat16)
    k = torch.randn(1, 2, 70, 64, device=DEV).to(torch.bfloat16)
    lse = torch.zeros(1, 2, 0, device=DEV)
    dq, dk, dv = fa.bwd(q, k, k, q, q, lse, causal=False)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)
    # no keys: dQ = 0
    q = torch.randn(1, 2, 50, 64, device=DEV).to(torch.bfloat16)
    k = torch.zeros(1, 2, 0, 64, device=DEV, dtype=torch.bfloat16)
    o, lse = fa.fwd(q, k, k)
    dq, dk, dv = fa.bwd(q, k, k, o, q, lse)
    torch.cuda.synchronize()
    assert torch.all(dq == 0)


def test_bwd_full_size_causal_L16384_d128_sampled():
    """The 16,384-token causal workload at full size: sampled dQ rows of two heads and
    sampled dK/dV keys of one head against the oracle."""
    fa = _fa()
    w = fa_inputs.WORKLOADS["causal_prefill_B1_H32_L16384_d128"]
    announce(entry="fa_bwd", workload=w.name, case="sampled rows and keys")
    x = fa_inputs.workload_inputs(w, device=DEV)
    o, lse = fa.fwd(x["q"], x["k"], x["v"], causal=True, scale=w.scale)
    do = _dout(o.shape, 240)
    dq, dk, dv = fa.bwd(x["q"], x["k"], x["v"], o, do, lse, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(241)
    rows = np.sort(np.concatenate([[0, 1, 127, 128, w.L - 1], rng.choice(w.L, 27, replace=False)]))
    keys = np.sort(np.concatenate([[0, 1, 63, 64, w.L - 1], rng.choice(w.L, 11, replace=False)]))
    for h in (0, 21):
        q64, k64, v64, do64 = (fa_inputs.as_oracle_f64(t[0, h]) for t in (x["q"], x["k"], x["v"], do))
        dQ, tQ = grad_rows_oracle(q64, k64, v64, do64, rows, scale=w.scale, causal=True)
        r = _close(dq[0, h, rows], dQ, f"dQ rows head {h}", tQ)
        report(f"fa_bwd {w.name}: dQ, {len(rows)} rows of head {h}: max err/allowance {r:.3f}")
        if h == 0:
            dK, dV, tK, tV = grad_keys_oracle(q64, k64, v64, do64, keys, scale=w.scale, causal=True)
            rk = _close(dk[0, h, keys], dK, "dK keys head 0", tK)
            rv = _close(dv[0, h, keys], dV, "dV keys head 0", tV)
            report(f"fa_bwd {w.name}: dK, dV, {len(keys)} keys of head 0: max err/allowance {rk:.3f}, {rv:.3f}")


def test_bwd_full_size_gqa_varlen_sampled():
    """The GQA variable-length workload (B=8, 32 query / 8 KV heads, lengths up to 8192) at full
    size, in the order its dK/dV and dQ launches deal (batch, KV head) pairs to the XCDs.
    Gradients start NaN: every row of a sequence must come back finite and every padding row
    exactly zero. Then sampled dQ rows of one query head per sequence (its first and last rows
    and rows of 128-row blocks across it) and sampled dK/dV keys of one KV head, summed over its
    four query heads, against the oracle ("FlashAttention 与长上下文", the online-softmax
    section: the backward recomputes P from the saved row statistics)."""
    fa = _fa()
    w = fa_inputs.WORKLOADS["gqa_varlen_prefill_B8_H32_Hkv8_L8192_d128"]
    announce(entry="fa_bwd", workload=w.name, case="every row written, sampled rows and keys")
    x = fa_inputs.workload_inputs(w, device=DEV)
    sl = x["seqlens"]
    o, lse = fa.fwd(x["q"], x["k"], x["v"], causal=True, scale=w.scale, seqlens=sl)
    do = _dout(o.shape, 250)
    nan = float("nan")
    dq = torch.full_like(x["q"], nan)
    dk, dv = torch.full_like(x["k"], nan), torch.full_like(x["v"], nan)
    fa.bwd(x["q"], x["k"], x["v"], o, do, lse, causal=True, scale=w.scale, seqlens=sl, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    lens = x["seqlens_cpu"].tolist()
    for b, n in enumerate(lens):
        for name, g in (("dQ", dq), ("dK", dk), ("dV", dv)):
            assert bool(torch.isfinite(g[b, :, :n]).all()), f"{name} of sequence {b}: a valid row was not written"
            assert bool((g[b, :, n:] == 0).all()), f"{name} of sequence {b}: a padding row is not zero"
    rng = np.random.default_rng(251)
    group = w.H // w.Hkv
    for b, n in enumerate(lens):
        h = (5 * b + 3) % w.H
        rows = np.unique(np.concatenate([[0, n - 1], np.minimum(128 * np.arange(0, n // 128 + 1, 9)
                                                                + rng.integers(0, 128), n - 1)]))
        q64, k64, v64, do64 = (fa_inputs.as_oracle_f64(t[b, hh, :n]) for t, hh in
                               ((x["q"], h), (x["k"], h // group), (x["v"], h // group), (do, h)))
        dQ, tQ = grad_rows_oracle(q64, k64, v64, do64, rows, scale=w.scale, causal=True)
        r = _close(dq[b, h, rows], dQ, f"dQ rows of sequence {b} head {h}", tQ)
        report(f"fa_bwd {w.name}: dQ, {len(rows)} rows of sequence {b} (length {n}), head {h}: "
               f"max err/allowance {r:.3f}")
    b = int(np.argmin(lens))  # the shortest sequence keeps the key oracle quick
    n, kvh = lens[b], 3
    keys = np.unique(np.concatenate([[0, 1, n - 1], rng.choice(n, 9, replace=False)]))
    k64, v64 = (fa_inputs.as_oracle_f64(t[b, kvh, :n]) for t in (x["k"], x["v"]))
    dK = dV = tK = tV = 0.0
    for h in range(kvh * group, (kvh + 1) * group):
        q64, do64 = (fa_inputs.as_oracle_f64(t[b, h, :n]) for t in (x["q"], do))
        gk, gv, ak, av = grad_keys_oracle(q64, k64, v64, do64, keys, scale=w.scale, causal=True)
        dK, dV, tK, tV = dK + gk, dV + gv, tK + ak, tV + av
    rk = _close(dk[b, kvh, keys], dK, f"dK keys of sequence {b} KV head {kvh}", tK)
    rv = _close(dv[b, kvh, keys], dV, f"dV keys of sequence {b} KV head {kvh}", tV)
    report(f"fa_bwd {w.name}: dK, dV, {len(keys)} keys of sequence {b} (length {n}), KV head {kvh} "
           f"(four query heads): max err/allowance {rk:.3f}, {rv:.3f}")


@pytest.mark.parametrize("d", [64, 128])
def test_empty_and_single_token_sequences(d):
    """Per-sequence lengths 0, 300 and 1 in one call. The empty sequence has no visible key:
    O = 0, LSE = -inf and zero gradients, with no NaN anywhere; the others match the oracle."""
    fa = _fa()
    B, H, Hkv, L = 3, 4, 2, 300
    announce(entry="fa_fwd + fa_bwd", case="lengths 0, 300, 1", B=B, H=H, Hkv=Hkv, L=L, d=d)
    x = fa_inputs.prefill_inputs(B, H, Hkv, L, L, d, seed=240 + d, device=DEV)
    sl_cpu = torch.tensor([0, 300, 1], dtype=torch.int32)
    sl = sl_cpu.to(DEV)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.fwd(x["q"], x["k"], x["v"], causal=True, scale=scale, seqlens=sl)
    do = _dout(o.shape, 241 + d)
    dq, dk, dv = fa.bwd(x["q"], x["k"], x["v"], o, do, lse, causal=True, scale=scale, seqlens=sl)
    ow, lsew = fa.fwd(x["q"], x["k"], x["v"], causal=True, scale=scale, seqlens=sl, window=37)
    torch.cuda.synchronize()
    for t in (o, dq, dk, dv, ow):
        assert torch.isfinite(t.float()).all()
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.all(ow[0] == 0) and torch.all(torch.isneginf(lsew[0]))
    assert torch.all(dq[0] == 0) and torch.all(dk[0] == 0) and torch.all(dv[0] == 0)
    q64, k64, v64, do64 = (fa_inputs.as_oracle_f64(t) for t in (x["q"], x["k"], x["v"], do))
    O, LSE = oracle.attention(q64, k64, v64, scale=scale, causal=True, seqlens=sl_cpu.numpy())
    from parity import compare
    compare(o[1:], lse[1:], O[1:], LSE[1:], bf16_out=True, what=f"lengths 0/300/1 d{d}")
    OW, LSEW = oracle.attention(q64, k64, v64, scale=scale, causal=True, seqlens=sl_cpu.numpy(), window=37)
    compare(ow[1:], lsew[1:], OW[1:], LSEW[1:], bf16_out=True, what=f"lengths 0/300/1 window 37 d{d}")
    dQ, dK, dV = oracle.attention_backward(q64, k64, v64, do64, scale=scale, causal=True, seqlens=sl_cpu.numpy())
    tQ, tK, tV = grad_tolerances(q64, k64, v64, do64, scale=scale, causal=True, seqlens=sl_cpu.numpy())
    _close(dq, dQ, f"dQ lengths 0/300/1 d{d}", tQ)
    _close(dk, dK, f"dK lengths 0/300/1 d{d}", tK)
    _close(dv, dV, f"dV lengths 0/300/1 d{d}", tV)


@pytest.mark.parametrize("d", [64, 128])
def test_gqa_grouped_order_varlen(d):
    """8 (batch, KV head) pairs, so the GQA workgroup orders (prefill, dQ and dK/dV) deal whole
    pairs to the XCDs; variable lengths, causal; forward and gradients against the oracle."""
    from parity import compare
    for causal, seed, lr in ((True, 250 + d, (1, 300)), (False, 260 + d, None)):
        x, _, _, _ = run_bwd(2, 16, 4, 300, 300, d, causal=causal, seed=seed, len_range=lr)
        scale = 1.0 / math.sqrt(d)
        o, lse = _fa().fwd(x["q"], x["k"], x["v"], causal=causal, scale=scale, seqlens=x["seqlens"])
        torch.cuda.synchronize()
        sl = None if x["seqlens_cpu"] is None else x["seqlens_cpu"].numpy()
        O, LSE = oracle.attention(*(fa_inputs.as_oracle_f64(x[n]) for n in ("q", "k", "v")), scale=scale,
                                  causal=causal, seqlens=sl)
        compare(o, lse, O, LSE, bf16_out=True, what=f"GQA 8 pairs fwd d{d} c{int(causal)}")
