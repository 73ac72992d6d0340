"""Full-size parity of the five workloads, in the launch configuration bench.py times.

Every workgroup's output is compared with the fp64 oracle:

* the single-head fp32 workload and the B=4, L=2048, d=64 causal prefill: every row of every head;
* the L=16384 causal prefill and the GQA variable-length prefill: every (batch, head), one
  random row of every 32-row block (the rows one wave owns), plus the first and last row of
  every 256-row query tile (the rows one workgroup owns);
* the decode workload: every (request, head) pair, one request at a time (its K/V slices are
  widened to fp64 once and serve the 4 query heads of their group).

Outputs start out NaN-filled (``out=``/``lse=``) and the whole tensor is checked on the GPU:
finite on valid rows, exactly O = 0 and LSE = -inf on padding rows, so a tile that is never
written fails even where the oracle does not look.

Tolerance (the stated bound; reading of the bf16 output rounding as in tests/parity.py): O
max-abs <= 1e-2 beyond the output's own rounding, O mean-abs <= 1e-3, LSE <= 1e-3 abs, with
the oracle fed the bf16-rounded inputs ("2.1 FlashAttention-2 的核心思想" §2.1.5: the tiled
computation gives the same result as the plain one; §2.1.7: shapes and lengths are checked).
"""
import math
import sys
import time

import numpy as np
import pytest
import torch

import fa_inputs
import oracle
from parity import check_written, compare, nan_filled_outputs, report, rows_per_workgroup

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fa():
    import exact_attention_111_amd as fa
    return fa


def announce(**case):
    print("\n[case] " + " ".join(f"{k}={v}" for k, v in case.items()), flush=True)
    sys.stdout.flush()


def run_prefill_workload(name, every_row):
    fa = _fa()
    w = fa_inputs.WORKLOADS[name]
    announce(entry="fa_fwd" if w.io == "bf16" else "fa_fwd_f32", workload=name, every_row=every_row)
    x = fa_inputs.workload_inputs(w, device=DEV)
    dtype = torch.bfloat16 if w.io == "bf16" else torch.float32
    o, lse = nan_filled_outputs((w.B, w.H, w.L, w.d), (w.B, w.H, w.L), dtype)
    fa.fwd(x["q"], x["k"], x["v"], causal=w.causal, scale=w.scale, seqlens=x["seqlens"], out=o, lse=lse)
    torch.cuda.synchronize()
    sl = None if x["seqlens_cpu"] is None else x["seqlens_cpu"].numpy()
    check_written(o, lse, sl)

    t0 = time.perf_counter()
    # The oracle sees bf16-rounded inputs, widened exactly to fp64 (per head, to bound memory).
    q_h, k_h, v_h = (x[n].detach().cpu().to(torch.bfloat16) for n in ("q", "k", "v"))
    o_h, lse_h = o.detach().cpu(), lse.detach().cpu()
    rng = np.random.default_rng(w.seed + 1000)
    group = w.H // w.Hkv
    worst = {"o_max": 0.0, "o_mean_max": 0.0, "lse_max": 0.0}
    n_rows = 0
    last = time.perf_counter()
    for b in range(w.B):
        n = w.L if sl is None else int(sl[b])
        for kvh in range(w.Hkv):
            K = k_h[b, kvh].double().numpy()
            V = v_h[b, kvh].double().numpy()
            for h in range(kvh * group, (kvh + 1) * group):
                rows = np.arange(n) if every_row else rows_per_workgroup(n, rng)
                if len(rows) == 0:
                    continue
                O, LSE = oracle.attention_head(q_h[b, h].double().numpy(), K, V, scale=w.scale, causal=w.causal,
                                               n_valid=None if sl is None else n, rows=rows)
                ri = torch.from_numpy(rows)
                st = compare(o_h[b, h, ri], lse_h[b, h, ri], O, LSE, bf16_out=(w.io == "bf16"),
                             what=f"{name} b{b} h{h}")
                worst["o_max"] = max(worst["o_max"], st["o_max"])
                worst["o_mean_max"] = max(worst["o_mean_max"], st["o_mean"])
                worst["lse_max"] = max(worst["lse_max"], st["lse_max"])
                n_rows += len(rows)
            if time.perf_counter() - last > 20:
                last = time.perf_counter()
                print(f"  ... batch {b}, KV head {kvh}: {n_rows} rows compared", flush=True)
    secs = time.perf_counter() - t0
    report(f"{name}: {n_rows} rows of all {w.B * w.H} (batch, head) pairs; worst O error beyond rounding "
           f"{worst['o_max']:.3g} (bound 1e-2), worst per-head O mean {worst['o_mean_max']:.3g} (1e-3), "
           f"worst LSE {worst['lse_max']:.3g} (1e-3); oracle {secs:.1f} s")
    return worst


def test_single_head_fp32_every_row():
    run_prefill_workload("single_head_fp32_L128_d64", every_row=True)


def test_causal_prefill_L2048_d64_every_row():
    run_prefill_workload("causal_prefill_B4_H16_L2048_d64", every_row=True)


def test_causal_prefill_L16384_d128_every_workgroup():
    run_prefill_workload("causal_prefill_B1_H32_L16384_d128", every_row=False)


def test_gqa_varlen_prefill_every_workgroup():
    run_prefill_workload("gqa_varlen_prefill_B8_H32_Hkv8_L8192_d128", every_row=False)


def test_decode_every_request_and_head():
    fa = _fa()
    w = fa_inputs.WORKLOADS["decode_B64_H32_Hkv8_ctx32768_d128"]
    announce(entry="fa_decode", workload=w.name, case="every (request, head)")
    x = fa_inputs.workload_inputs(w, device=DEV)
    o = torch.full((w.B, w.H, w.d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((w.B, w.H), float("nan"), dtype=torch.float32, device=DEV)
    fa.decode(x["q"], x["k_cache"], x["v_cache"], x["ctx_lens"], scale=w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all(), "an output of the decode is not finite"

    t0 = time.perf_counter()
    ctx = x["ctx_lens_cpu"].numpy()
    q_h, o_h, lse_h = x["q"].cpu(), o.cpu(), lse.cpu()
    group = w.H // w.Hkv
    Os, Ls = np.empty((w.B, w.H, w.d)), np.empty((w.B, w.H))
    for b in range(w.B):
        n = int(ctx[b])
        kb = x["k_cache"][b, :, :n].cpu()  # one request's valid cache at a time
        vb = x["v_cache"][b, :, :n].cpu()
        for kvh in range(w.Hkv):
            K = kb[kvh].double().numpy()
            V = vb[kvh].double().numpy()
            for h in range(kvh * group, (kvh + 1) * group):
                Oh, Lh = oracle.attention_head(q_h[b, h][None].double().numpy(), K, V, scale=w.scale)
                Os[b, h], Ls[b, h] = Oh[0], Lh[0]
        if b % 16 == 15:
            print(f"  ... requests 0..{b} done", flush=True)
    st = compare(o_h, lse_h, Os, Ls, bf16_out=True, what=w.name)
    report(f"{w.name}: all {w.B * w.H} (request, head) pairs; O error beyond rounding {st['o_max']:.3g} "
           f"(bound 1e-2), O mean {st['o_mean']:.3g} (1e-3), LSE {st['lse_max']:.3g} (1e-3); "
           f"oracle {time.perf_counter() - t0:.1f} s")
