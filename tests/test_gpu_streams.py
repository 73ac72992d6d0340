"""Calls on different streams at the same time: the library keeps no state between calls
(the persistent grid's tile assignment is computed from the workgroup id alone, with no
shared counters), so concurrent prefills, decodes and backward passes on two streams each
give the bits the same call gives alone."""
import math
import sys

import pytest
import torch

import fa_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fa():
    import exact_attention_111_amd as fa
    return fa


def announce(**case):
    print("\n[case] " + " ".join(f"{k}={v}" for k, v in case.items()), flush=True)
    sys.stdout.flush()


def test_concurrent_calls_on_two_streams_equal_calls_alone():
    announce(entry="fa_fwd x2 + fa_decode + fa_bwd on two streams", seed=960)
    fa = _fa()
    # two dense prefills with more query tiles than compute units (persistent grids), a decode
    # and a backward
    xa = fa_inputs.prefill_inputs(1, 40, 40, 1792, 1792, 128, seed=960, device=DEV)
    xb = fa_inputs.prefill_inputs(2, 32, 8, 1100, 1100, 64, seed=961, device=DEV)
    xd = fa_inputs.decode_inputs(8, 32, 8, 9000, 128, seed=962, device=DEV)
    sa, sb = 1.0 / math.sqrt(128), 1.0 / math.sqrt(64)

    def run_a():
        o, l = fa.fwd(xa["q"], xa["k"], xa["v"], causal=True, scale=sa)
        return [o, l]

    def run_b():
        o, l = fa.fwd(xb["q"], xb["k"], xb["v"], causal=False, scale=sb)
        dout = torch.ones_like(xb["q"])
        dq, dk, dv = fa.bwd(xb["q"], xb["k"], xb["v"], o, dout, l, causal=False, scale=sb)
        od, ld = fa.decode(xd["q"], xd["k_cache"], xd["v_cache"], xd["ctx_lens"], scale=sa)
        return [o, l, dq, dk, dv, od, ld]

    alone_a = run_a()
    torch.cuda.synchronize()
    alone_b = run_b()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        with torch.cuda.stream(s1):
            got_a = run_a()
        with torch.cuda.stream(s2):
            got_b = run_b()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(got_a, alone_a)):
            assert torch.equal(x, y), f"rep {rep}: stream 1 output {i} differs from the call alone"
        for i, (x, y) in enumerate(zip(got_b, alone_b)):
            assert torch.equal(x, y), f"rep {rep}: stream 2 output {i} differs from the call alone"
