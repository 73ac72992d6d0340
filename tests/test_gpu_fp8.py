"""GPU parity of fa_fwd_fp8 (FP8 prefill), through the C ABI, against two references:

* the fp64 FP8 oracle (oracle/fp8.py), at the tolerance of the bf16 prefill. The oracle writes
  out the same P rounding, so only fp32 sums differ, plus probabilities that lie within fp32
  error of an E4M3 rounding midpoint and may round the other way; each such element adds its
  one-spacing effect on O to that row's allowance (parity.fp8_flip_slack);
* exact fp64 attention of the dequantised inputs (oracle.attention_head), at the E4M3 bound
  the FP8 oracle is pinned to: 2^-4 of sum_j P_ij |V_jc| per element (parity.compare_fp8_exact),
  which does not depend on the P scheme being the kernel's own."""
import math
import sys

import numpy as np
import pytest
import torch

import fa_inputs
import oracle
from parity import check_written, compare, compare_fp8_exact, fp8_flip_slack, nan_filled_outputs, report

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fa():
    import exact_attention_111_amd as fa
    return fa


def announce(**case):
    print("\n[case] " + " ".join(f"{k}={v}" for k, v in case.items()), flush=True)
    sys.stdout.flush()


def run_fp8(B, H, Hkv, Lq, Lk, *, causal, seed, window=None, len_range=None):
    d = 128
    announce(entry="fa_fwd_fp8", B=B, H=H, Hkv=Hkv, Lq=Lq, Lk=Lk, causal=causal, window=window, seed=seed,
             len_range=len_range)
    x = fa_inputs.fp8_prefill_inputs(B, H, Hkv, Lq, Lk, d, seed=seed, device=DEV, len_range=len_range)
    scale = 1.0 / math.sqrt(d)
    o, lse = _fa().fwd_fp8(x["q"], x["k"], x["v"], x["q_descale"], x["k_descale"], x["v_descale"], causal=causal,
                           scale=scale, seqlens=x["seqlens"], window=window)
    torch.cuda.synchronize()
    sl = None if x["seqlens_cpu"] is None else x["seqlens_cpu"].numpy()
    arrs = [x[n].cpu().numpy() for n in ("q", "k", "v", "q_descale", "k_descale", "v_descale")]
    O, LSE = oracle.attention_fp8(*arrs, scale=scale, causal=causal, seqlens=sl, window=window)
    slack = np.zeros(LSE.shape)
    for b in range(B):
        for h in range(H):
            kvh = h // (H // Hkv)
            Q = oracle.e4m3_decode(arrs[0][b, h]) * float(arrs[3][b, h])
            K = oracle.e4m3_decode(arrs[1][b, kvh]) * float(arrs[4][b, kvh])
            V = oracle.e4m3_decode(arrs[2][b, kvh]) * float(arrs[5][b, kvh])
            n_b = None if sl is None else int(sl[b])
            slack[b, h] = fp8_flip_slack(Q, K, V, scale=scale, causal=causal, n_valid=n_b, window=window)
            compare_fp8_exact(o[b, h], lse[b, h], Q, K, V, scale=scale, causal=causal, n_valid=n_b, window=window,
                              what=f"fp8 b{b} h{h}")
    st = compare(o, lse, O, LSE, bf16_out=True, what=f"fp8 B{B} H{H}/{Hkv} L{Lq}x{Lk} c{int(causal)} W{window}",
                 o_slack=slack)
    print(f"  rows with flip allowance: {int((slack > 0).sum())} of {slack.size}; {st}", flush=True)
    return x, o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_ragged_gqa(causal):
    run_fp8(2, 4, 2, 300, 300, causal=causal, seed=600 + int(causal))


@pytest.mark.parametrize("Lq,Lk", [(100, 333), (333, 100), (1, 700)])
def test_fp8_unequal_lengths(Lq, Lk):
    run_fp8(1, 2, 1, Lq, Lk, causal=True, seed=610 + Lq)


def test_fp8_more_tiles_than_compute_units():
    # 261 query tiles (more than the GPU's compute units): several tiles per workgroup, the
    # last round nearly empty; 29 heads, not a multiple of the 8 XCDs.
    run_fp8(3, 29, 29, 768, 768, causal=True, seed=630)


def test_fp8_varlen():
    run_fp8(3, 4, 2, 700, 700, causal=True, seed=620, len_range=(1, 700))


@pytest.mark.parametrize("W", [1, 100])
def test_fp8_window(W):
    run_fp8(2, 2, 1, 400, 400, causal=True, seed=630 + W, window=W)


def test_fp8_empty_and_no_keys():
    announce(entry="fa_fwd_fp8", case="empty / no keys")
    fa = _fa()
    q = torch.zeros(1, 2, 0, 128, dtype=torch.uint8, device=DEV)
    ds = torch.ones(1, 2, device=DEV)
    o, lse = fa.fwd_fp8(q, q, q, ds, ds, ds)
    assert o.shape == (1, 2, 0, 128)
    x = fa_inputs.fp8_prefill_inputs(1, 2, 2, 50, 0, 128, seed=640, device=DEV)
    o, lse = fa.fwd_fp8(x["q"], x["k"], x["v"], x["q_descale"], x["k_descale"], x["v_descale"])
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_fp8_full_size_16k_sampled():
    """The 16,384-token causal workload with FP8 inputs in bench.py's launch configuration:
    sampled rows of two heads against the oracle."""
    w = fa_inputs.WORKLOADS["causal_prefill_B1_H32_L16384_d128"]
    announce(entry="fa_fwd_fp8", workload=w.name, case="sampled rows")
    x = fa_inputs.fp8_prefill_inputs(w.B, w.H, w.Hkv, w.L, w.L, w.d, seed=w.seed, device=DEV)
    o, lse = _fa().fwd_fp8(x["q"], x["k"], x["v"], x["q_descale"], x["k_descale"], x["v_descale"], causal=True,
                           scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(650)
    rows = np.sort(np.concatenate([[0, 1, 255, 256, w.L - 1], rng.choice(w.L, 27, replace=False)]))
    for h in (0, 19):
        Q = oracle.e4m3_decode(x["q"][0, h].cpu().numpy()) * float(x["q_descale"][0, h])
        K = oracle.e4m3_decode(x["k"][0, h].cpu().numpy()) * float(x["k_descale"][0, h])
        V = oracle.e4m3_decode(x["v"][0, h].cpu().numpy()) * float(x["v_descale"][0, h])
        O, LSE = oracle.attention_fp8_head(Q, K, V, scale=w.scale, causal=True, rows=rows)
        slack = fp8_flip_slack(Q, K, V, scale=w.scale, causal=True, rows=rows)
        st = compare(o[0, h, rows], lse[0, h, rows], O, LSE, bf16_out=True, what=f"fp8 16k head {h}", o_slack=slack)
        r = compare_fp8_exact(o[0, h, rows], lse[0, h, rows], Q, K, V, scale=w.scale, causal=True, rows=rows,
                              what=f"fp8 16k head {h}")
        report(f"fa_fwd_fp8 {w.name}, head {h}, {len(rows)} rows: vs FP8 oracle O {st['o_max']:.3g} "
               f"LSE {st['lse_max']:.3g}; vs exact attention max err/allowance {r:.3f}")


def test_fp8_gqa_varlen_full_size():
    """The GQA variable-length workload with FP8 inputs (one workgroup per 256-row query tile,
    8,192 of them): outputs start NaN, every valid row must be written and every padding row
    come back O = 0, LSE = -inf; then the first and last row of every query tile and 8 random
    rows of one query head per sequence against both references."""
    w = fa_inputs.WORKLOADS["gqa_varlen_prefill_B8_H32_Hkv8_L8192_d128"]
    announce(entry="fa_fwd_fp8", workload=w.name, case="every tile written, sampled rows")
    x = fa_inputs.fp8_prefill_inputs(w.B, w.H, w.Hkv, w.L, w.L, w.d, seed=w.seed, device=DEV,
                                     len_range=w.len_range)
    o, lse = nan_filled_outputs((w.B, w.H, w.L, w.d), (w.B, w.H, w.L), torch.bfloat16, device=DEV)
    _fa().fwd_fp8(x["q"], x["k"], x["v"], x["q_descale"], x["k_descale"], x["v_descale"], causal=True,
                  scale=w.scale, seqlens=x["seqlens"], out=o, lse=lse)
    torch.cuda.synchronize()
    lens = x["seqlens_cpu"].tolist()
    check_written(o, lse, lens)
    rng = np.random.default_rng(660)
    group = w.H // w.Hkv
    for b, n in enumerate(lens):
        h = (7 * b + 2) % w.H
        kvh = h // group
        rows = np.unique(np.concatenate([np.arange(0, n, 256), np.minimum(np.arange(255, n + 255, 256), n - 1),
                                         rng.choice(n, 8, replace=False)]))
        Q = oracle.e4m3_decode(x["q"][b, h, :n].cpu().numpy()) * float(x["q_descale"][b, h])
        K = oracle.e4m3_decode(x["k"][b, kvh, :n].cpu().numpy()) * float(x["k_descale"][b, kvh])
        V = oracle.e4m3_decode(x["v"][b, kvh, :n].cpu().numpy()) * float(x["v_descale"][b, kvh])
        O, LSE = oracle.attention_fp8_head(Q, K, V, scale=w.scale, causal=True, rows=rows)
        slack = fp8_flip_slack(Q, K, V, scale=w.scale, causal=True, rows=rows)
        st = compare(o[b, h, rows], lse[b, h, rows], O, LSE, bf16_out=True, what=f"fp8 varlen b{b} h{h}",
                     o_slack=slack)
        r = compare_fp8_exact(o[b, h, rows], lse[b, h, rows], Q, K, V, scale=w.scale, causal=True, rows=rows,
                              what=f"fp8 varlen b{b} h{h}")
        report(f"fa_fwd_fp8 {w.name}: sequence {b} (length {n}), head {h}, {len(rows)} rows: vs FP8 oracle "
               f"O {st['o_max']:.3g} LSE {st['lse_max']:.3g}; vs exact attention max err/allowance {r:.3f}")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_scores_rising_across_tiles(causal):
    """Scores that rise by hundreds of base-2 units along the keys: each row's reference passes
    its output frame by more than 64 several times, so the kernel's rare frame move (o and l
    rescaled by an exact power of two) runs on many tiles. Q is all ones and key j's row is the
    E4M3 value nearest 1 + 15 j / L in every dim, so row i's scores grow with its keys; V is
    random. Against both references."""
    B, H, Hkv, L, d = 1, 2, 1, 1000, 128
    announce(entry="fa_fwd_fp8", case="rising scores", causal=causal, L=L)
    g = torch.Generator().manual_seed(670)
    qf = torch.ones((B, H, L, d))
    kf = (1.0 + 15.0 * torch.arange(L, dtype=torch.float32) / L)[None, None, :, None].expand(B, Hkv, L, d)
    vf = torch.randn((B, Hkv, L, d), generator=g)
    codes = [t.contiguous().to(torch.float8_e4m3fn).view(torch.uint8).to(DEV) for t in (qf, kf, vf)]
    ones_q = torch.ones((B, H), dtype=torch.float32, device=DEV)
    ones_kv = torch.ones((B, Hkv), dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(d)
    o, lse = _fa().fwd_fp8(codes[0], codes[1], codes[2], ones_q, ones_kv, ones_kv, causal=causal, scale=scale)
    torch.cuda.synchronize()
    arrs = [t.cpu().numpy() for t in codes] + [ones_q.cpu().numpy(), ones_kv.cpu().numpy(), ones_kv.cpu().numpy()]
    O, LSE = oracle.attention_fp8(*arrs, scale=scale, causal=causal)
    K = oracle.e4m3_decode(arrs[1][0, 0])
    Q = oracle.e4m3_decode(arrs[0][0, 0])
    t_range = (Q[0] @ K[-1] - Q[0] @ K[0]) * scale / math.log(2.0)
    assert t_range > 3 * 64, t_range  # the reference must pass the frame by more than 64 several times
    for h in range(H):
        V = oracle.e4m3_decode(arrs[2][0, 0])
        slack = fp8_flip_slack(Q, K, V, scale=scale, causal=causal)
        compare(o[0, h], lse[0, h], O[0, h], LSE[0, h], bf16_out=True, what=f"fp8 rising scores h{h}", o_slack=slack)
        compare_fp8_exact(o[0, h], lse[0, h], Q, K, V, scale=scale, causal=causal, what=f"fp8 rising scores h{h}")
