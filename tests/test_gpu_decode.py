"""GPU parity of fa_decode (split-K + LSE combine) against the fp64 oracle."""
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


def announce(**case):
    print("\n[case] " + " ".join(f"{k}={v}" for k, v in case.items()), flush=True)
    sys.stdout.flush()


def run_decode(B, H, Hkv, Lmax, d, *, seed, ctx=None, len_range=(1, None), heads=None):
    announce(entry="fa_decode", B=B, H=H, Hkv=Hkv, Lmax=Lmax, d=d, seed=seed, ctx=ctx)
    x = fa_inputs.decode_inputs(B, H, Hkv, Lmax, d, seed=seed, device=DEV, len_range=len_range)
    if ctx is not None:
        x["ctx_lens_cpu"] = torch.tensor(ctx, dtype=torch.int32)
        x["ctx_lens"] = x["ctx_lens_cpu"].to(DEV)
    scale = 1.0 / math.sqrt(d)
    o, lse = _fa().decode(x["q"], x["k_cache"], x["v_cache"], x["ctx_lens"], scale=scale)
    torch.cuda.synchronize()
    ctx_np = x["ctx_lens_cpu"].numpy()
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    Os, Ls, og, lg = [], [], [], []
    G = H // Hkv
    for b, h in pairs:
        n = int(ctx_np[b])
        Oh, Lh = oracle.attention_head(fa_inputs.as_oracle_f64(x["q"][b, h][None]),
                                       fa_inputs.as_oracle_f64(x["k_cache"][b, h // G, :n]),
                                       fa_inputs.as_oracle_f64(x["v_cache"][b, h // G, :n]), scale=scale)
        Os.append(Oh[0]); Ls.append(Lh[0]); og.append(o[b, h]); lg.append(lse[b, h])
    st = compare(torch.stack(og), torch.stack(lg), np.stack(Os), np.array(Ls), bf16_out=True,
                 what=f"decode B{B} H{H}/{Hkv} Lmax{Lmax} d{d}")
    return st, x, o, lse


@pytest.mark.parametrize("d", [64, 128])
def test_decode_multi_chunk_ragged(d):
    # 4500 keys = 2 full 2048-key chunks + 404; 1 key; one key short of a chunk; a chunk exactly.
    run_decode(4, 8, 2, 4500, d, seed=100 + d, ctx=[4500, 1, 2047, 2048])


@pytest.mark.parametrize("H,Hkv", [(4, 4), (16, 2), (12, 2), (3, 1)])
def test_decode_group_sizes(H, Hkv):
    # group 1, 8 (two passes of 4 heads), 6 (a partial pass) and 3
    run_decode(2, H, Hkv, 700, 128, seed=110 + H, ctx=[700, 300])


@pytest.mark.parametrize("H,Hkv,d", [(16, 2, 128), (12, 2, 64), (3, 1, 128)])
def test_decode_balanced_partition(H, Hkv, d):
    """A contiguous cache longer than one 2048-key chunk, without a window, is split into equal
    step ranges per workgroup, cut where a (request, KV head, head slot) unit ends. Mixed
    lengths (empty, 1, 31, 32, 33 keys, full) make workgroups span several units and requests;
    group 8 takes two head passes, group 6 a partial one."""
    ctx = [0, 1, 31, 32, 33, 5000, 2049, 0, 4096, 777, 5000, 2]
    st, x, o, lse = run_decode(len(ctx), H, Hkv, 5000, d, seed=130 + H + d, ctx=ctx)
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.all(o[7] == 0) and torch.all(torch.isneginf(lse[7]))
    st, x, o, lse = run_decode(2, H, Hkv, 3000, d, seed=140 + H + d, ctx=[0, 0])  # no keys at all
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_decode_empty_context_and_empty_call():
    fa = _fa()
    announce(entry="fa_decode", case="ctx = 0 and B = 0")
    st, x, o, lse = run_decode(2, 4, 2, 64, 128, seed=120, ctx=[0, 64])
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    q = torch.zeros(0, 4, 128, device=DEV, dtype=torch.bfloat16)
    kc = torch.zeros(0, 2, 64, 128, device=DEV, dtype=torch.bfloat16)
    o, lse = fa.decode(q, kc, kc, torch.zeros(0, dtype=torch.int32, device=DEV))
    assert o.shape == (0, 4, 128)


def test_decode_equals_last_prefill_row():
    """Decode over a cache of n keys equals the last row of a causal prefill of n rows."""
    fa = _fa()
    announce(entry="fa_decode vs fa_fwd", B=1, H=8, Hkv=2, n=1000, d=128)
    n = 1000
    x = fa_inputs.prefill_inputs(1, 8, 2, n, n, 128, seed=130, device=DEV)
    o_p, lse_p = fa.fwd(x["q"], x["k"], x["v"], causal=True)
    q_last = x["q"][:, :, -1].contiguous()
    o_d, lse_d = fa.decode(q_last, x["k"], x["v"], torch.tensor([n], dtype=torch.int32, device=DEV))
    assert (o_d.float() - o_p[:, :, -1].float()).abs().max() < 2e-2
    assert (lse_d - lse_p[:, :, -1]).abs().max() < 1e-3


def test_decode_nan_beyond_context_ignored():
    fa = _fa()
    announce(entry="fa_decode", case="NaN past ctx", B=2, H=4, Hkv=1, Lmax=900, d=128)
    x = fa_inputs.decode_inputs(2, 4, 1, 900, 128, seed=140, device=DEV, len_range=(1, 900))
    ctx = torch.tensor([600, 37], dtype=torch.int32, device=DEV)
    o1, l1 = fa.decode(x["q"], x["k_cache"], x["v_cache"], ctx)
    kc, vc = x["k_cache"].clone(), x["v_cache"].clone()
    kc[0, :, 600:] = float("nan"); vc[0, :, 600:] = float("nan")
    kc[1, :, 37:] = float("nan"); vc[1, :, 37:] = float("nan")
    o2, l2 = fa.decode(x["q"], kc, vc, ctx)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_deterministic():
    fa = _fa()
    announce(entry="fa_decode", case="determinism", B=8, H=32, Hkv=8, Lmax=4096, d=128)
    x = fa_inputs.decode_inputs(8, 32, 8, 4096, 128, seed=150, device=DEV, len_range=(1000, 4096))
    o1, l1 = fa.decode(x["q"], x["k_cache"], x["v_cache"], x["ctx_lens"])
    o2, l2 = fa.decode(x["q"], x["k_cache"], x["v_cache"], x["ctx_lens"])
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
