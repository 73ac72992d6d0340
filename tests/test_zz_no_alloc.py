"""fa_decode_noalloc (the decode entry point that allocates nothing; its split partials live
in the library's fixed per-GPU array) against fa_decode with a caller workspace, through the
C ABI: two calls in a row, the second smaller, each bit for bit equal to fa_decode (same
kernels, same split) and within the stated tolerance of the oracle on sampled heads."""
import math
import sys

import numpy as np
import pytest
import torch

import fa_inputs
import oracle
from parity import compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fa():
    import exact_attention_111_amd as fa
    return fa


def _one(B, H, Hkv, Lmax, d, seed, len_range):
    fa = _fa()
    print(f"\\n[case] entry=fa_decode_noalloc B={B} H={H} Hkv={Hkv} Lmax={Lmax} d={d} seed={seed}", flush=True)
    sys.stdout.flush()
    x = fa_inputs.decode_inputs(B, H, Hkv, Lmax, d, seed=seed, device=DEV, len_range=len_range)
    scale = 1.0 / math.sqrt(d)
    o = torch.full((B, H, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=DEV)
    fa.decode_noalloc(x["q"], x["k_cache"], x["v_cache"], x["ctx_lens"], scale=scale, out=o, lse=lse)
    o_ref, lse_ref = fa.decode(x["q"], x["k_cache"], x["v_cache"], x["ctx_lens"], scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "O differs from fa_decode"
    assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), "LSE differs from fa_decode"
    rng = np.random.default_rng(seed)
    G = H // Hkv
    ctx = x["ctx_lens_cpu"].numpy()
    pairs = sorted({(int(rng.integers(B)), int(rng.integers(H))) for _ in range(12)} | {(0, 0), (B - 1, H - 1)})
    Os, Ls, og, lg = [], [], [], []
    for b, h in pairs:
        n = int(ctx[b])
        Oh, Lh = oracle.attention_head(fa_inputs.as_oracle_f64(x["q"][b, h][None]),
                                       fa_inputs.as_oracle_f64(x["k_cache"][b, h // G, :n]),
                                       fa_inputs.as_oracle_f64(x["v_cache"][b, h // G, :n]), scale=scale)
        Os.append(Oh[0]); Ls.append(Lh[0]); og.append(o[b, h]); lg.append(lse[b, h])
    compare(torch.stack(og), torch.stack(lg), np.stack(Os), np.array(Ls), bf16_out=True,
            what=f"fa_decode_noalloc B{B} Lmax{Lmax}")


def test_noalloc_two_calls_second_smaller():
    # the decode workload's shape (16.25 MiB of partials), then a smaller ragged call
    _one(64, 32, 8, 32768, 128, seed=5, len_range=(8192, 32768))
    _one(3, 8, 2, 4500, 64, seed=77, len_range=(1, 4500))

