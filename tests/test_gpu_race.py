"""Race check of the direct-to-LDS load pipelines (prefill, FP8 prefill, both backward kernels).

The loads into LDS are issued as instructions the compiler does not track, so their ordering
rests on hand-placed waits and barriers. libfa_serial.so is built from the same sources with
every load stage fenced on both sides (all loads waited for, then a workgroup barrier): no load
is in flight while anything computes and no slot is refilled before every wave is past its
earlier reads. The arithmetic is identical, so every output must be bit for bit equal to the
pipelined library's. A read before a load landed, or a slot refilled too early, would differ
("2.1 FlashAttention-2 的核心思想" §2.1.5: the tiled computation must give the plain result).
Shapes: ragged tails, Lq != Lk, variable lengths, sliding windows, GQA, and the full-size
16,384-token and GQA variable-length workloads in bench.py's launch configuration.
"""
import math
import sys

import pytest
import torch

import fa_inputs
from parity import report

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fa():
    import exact_attention_111_amd as fa
    return fa


def announce(**case):
    print("\n[case] " + " ".join(f"{k}={v}" for k, v in case.items()), flush=True)
    sys.stdout.flush()


def both(fn):
    """fn() run through libfa.so, then through libfa_serial.so; results as a pair of tuples."""
    fa = _fa()
    a = fn()
    torch.cuda.synchronize()
    with fa.binding.library_variant(fa.binding.SERIAL_LIB_PATH):
        b = fn()
        torch.cuda.synchronize()
    return a, b


def assert_bitwise(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        assert x.shape == y.shape, (what, i)
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.float32 else x.view(torch.int32),
                           y.view(torch.uint8) if y.dtype != torch.float32 else y.view(torch.int32)), \
            f"{what}: output {i} differs between the pipelined and the fenced build"


def _ms(fn, n=5):
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


FWD_CASES = [
    # (B, H, Hkv, Lq, Lk, d, causal, window, len_range, seed)
    (2, 3, 3, 300, 300, 64, True, None, None, 900),
    (2, 3, 3, 300, 300, 128, False, None, None, 901),
    (1, 4, 2, 100, 333, 128, True, None, None, 902),
    (1, 4, 2, 333, 100, 64, True, None, None, 903),
    (3, 8, 2, 700, 700, 128, True, None, (1, 700), 904),
    (2, 4, 2, 500, 500, 128, True, 37, None, 905),
    (2, 4, 2, 500, 500, 64, True, 200, (1, 500), 906),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}L{c[3]}x{c[4]}d{c[5]}c{int(c[6])}W{c[7]}")
def test_prefill_and_backward_fenced_equal(case):
    B, H, Hkv, Lq, Lk, d, causal, W, lr, seed = case
    announce(entry="fa_fwd + fa_bwd (pipelined vs fenced)", B=B, H=H, Hkv=Hkv, Lq=Lq, Lk=Lk, d=d, causal=causal,
             window=W, len_range=lr)
    fa = _fa()
    x = fa_inputs.prefill_inputs(B, H, Hkv, Lq, Lk, d, seed=seed, device=DEV, len_range=lr)
    g = torch.Generator(device=DEV).manual_seed(seed + 7)
    do = torch.randn((B, H, Lq, d), generator=g, device=DEV).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)

    def run():
        o, lse = fa.fwd(x["q"], x["k"], x["v"], causal=causal, scale=scale, seqlens=x["seqlens"], window=W)
        dq, dk, dv = fa.bwd(x["q"], x["k"], x["v"], o, do, lse, causal=causal, scale=scale, seqlens=x["seqlens"],
                            window=W)
        return o, lse, dq, dk, dv
    a, b = both(run)
    assert_bitwise(a, b, "prefill + backward")


def test_fp32_prefill_fenced_equal():
    announce(entry="fa_fwd_f32 (pipelined vs fenced)", B=1, H=2, L=300, d=64)
    fa = _fa()
    x = fa_inputs.prefill_inputs(1, 2, 1, 300, 300, 64, seed=910, device=DEV, io="f32")
    a, b = both(lambda: fa.fwd(x["q"], x["k"], x["v"], causal=True))
    assert_bitwise(a, b, "fp32 prefill")


@pytest.mark.parametrize("causal,W,lr", [(False, None, None), (True, None, (1, 600)), (True, 50, None)])
def test_fp8_prefill_fenced_equal(causal, W, lr):
    announce(entry="fa_fwd_fp8 (pipelined vs fenced)", causal=causal, window=W, len_range=lr)
    fa = _fa()
    x = fa_inputs.fp8_prefill_inputs(2, 4, 2, 600, 600, 128, seed=920, device=DEV, len_range=lr)
    a, b = both(lambda: fa.fwd_fp8(x["q"], x["k"], x["v"], x["q_descale"], x["k_descale"], x["v_descale"],
                                   causal=causal, seqlens=x["seqlens"], window=W))
    assert_bitwise(a, b, "fp8 prefill")


@pytest.mark.parametrize("name", ["causal_prefill_B1_H32_L16384_d128", "gqa_varlen_prefill_B8_H32_Hkv8_L8192_d128",
                                  "causal_prefill_B4_H16_L2048_d64"])
def test_full_size_workloads_fenced_equal(name):
    w = fa_inputs.WORKLOADS[name]
    announce(entry="fa_fwd (+ fa_fwd_fp8, fa_bwd at 16k) pipelined vs fenced", workload=name)
    fa = _fa()
    x = fa_inputs.workload_inputs(w, device=DEV)
    call = lambda: fa.fwd(x["q"], x["k"], x["v"], causal=w.causal, scale=w.scale, seqlens=x["seqlens"])  # noqa: E731
    a, b = both(call)
    assert_bitwise(a, b, f"{name} prefill")
    # The fenced build is really the one called: its launches take longer (no load overlaps compute).
    t_pipe = _ms(call)
    with fa.binding.library_variant(fa.binding.SERIAL_LIB_PATH):
        t_fenced = _ms(call)
    report(f"race check {name}: prefill bitwise equal to the fenced build; {t_pipe:.3f} ms pipelined, "
           f"{t_fenced:.3f} ms fenced")
    if name == "causal_prefill_B1_H32_L16384_d128":
        g = torch.Generator(device=DEV).manual_seed(930)
        do = torch.randn(a[0].shape, generator=g, device=DEV).to(torch.bfloat16)
        o, lse = a
        ga, gb = both(lambda: fa.bwd(x["q"], x["k"], x["v"], o, do, lse, causal=True, scale=w.scale))
        assert_bitwise(ga, gb, f"{name} backward")
        del x
        y = fa_inputs.fp8_prefill_inputs(w.B, w.H, w.Hkv, w.L, w.L, w.d, seed=w.seed, device=DEV)
        fa8, fb8 = both(lambda: fa.fwd_fp8(y["q"], y["k"], y["v"], y["q_descale"], y["k_descale"], y["v_descale"],
                                           causal=True, scale=w.scale))
        assert_bitwise(fa8, fb8, f"{name} fp8 prefill")
