"""GPU parity of fa_decode_paged (paged KV cache) against the fp64 oracle and against the
contiguous fa_decode, through the C ABI."""
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


def _paginate(cache, P, seed):
    """Scatter a contiguous cache [B, Hkv, Lmax, d] into a pool [pages, Hkv, P, d] through a
    random permutation; pages no table row names hold other values."""
    B, Hkv, Lmax, d = cache.shape
    mp = -(-Lmax // P)
    g = torch.Generator(device="cpu").manual_seed(seed)
    perm = torch.randperm(B * mp + 3, generator=g)
    table = perm[:B * mp].reshape(B, mp).to(torch.int32)
    pool = torch.randn((B * mp + 3, Hkv, P, d), device=cache.device).to(cache.dtype)
    padded = torch.zeros((B, Hkv, mp * P, d), device=cache.device, dtype=cache.dtype)
    padded[:, :, :Lmax] = cache
    pool[table.reshape(-1).long().to(cache.device)] = padded.reshape(B, Hkv, mp, P, d).permute(0, 2, 1, 3, 4).reshape(
        B * mp, Hkv, P, d)
    return pool, table.to(cache.device)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("P", [16, 64, 256, 2048, 4096])
def test_paged_equals_contiguous_bitwise(d, P):
    """Same arithmetic and the same split of the keys (pages up to 4096 positions, so balanced
    runs cross many 128-page windows at P = 16), rows from other addresses: the outputs are
    identical."""
    B, H, Hkv, Lmax = 4, 8, 2, 5000
    announce(entry="fa_decode_paged vs fa_decode", d=d, P=P, B=B, H=H, Hkv=Hkv, Lmax=Lmax)
    x = fa_inputs.decode_inputs(B, H, Hkv, Lmax, d, seed=500 + P + d, device=DEV)
    ctx = torch.tensor([1, 2047, 2049, 5000], dtype=torch.int32, device=DEV)
    kp, table = _paginate(x["k_cache"], P, 501)
    vp, _ = _paginate(x["v_cache"], P, 501)
    # the contiguous cache gets the paged one's capacity (max_pages * P), which sets the split
    cap = table.shape[1] * P
    kc = torch.zeros((B, Hkv, cap, d), device=DEV, dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    kc[:, :, :Lmax], vc[:, :, :Lmax] = x["k_cache"], x["v_cache"]
    for W in (None, 700):
        o1, l1 = _fa().decode(x["q"], kc, vc, ctx, window=W)
        o2, l2 = _fa().decode_paged(x["q"], kp, vp, table, ctx, window=W)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), (P, W)


@pytest.mark.parametrize("P,W", [(16, None), (64, None), (16, 300), (32, 5000)])
def test_paged_against_oracle(P, W):
    B, H, Hkv, Lmax, d = 6, 12, 2, 4600, 128
    announce(entry="fa_decode_paged", B=B, H=H, Hkv=Hkv, Lmax=Lmax, d=d, P=P, W=W)
    x = fa_inputs.paged_decode_inputs(B, H, Hkv, Lmax, d, P, seed=510 + P, device=DEV)
    ctx = torch.tensor([1, 15, 17, 2048, 4097, 4600], dtype=torch.int32)
    o, lse = _fa().decode_paged(x["q"], x["k_pages"], x["v_pages"], x["block_table"], ctx.to(DEV), window=W)
    torch.cuda.synchronize()
    O, LSE = oracle.decode_paged(*(fa_inputs.as_oracle_f64(x[n]) for n in ("q", "k_pages", "v_pages")),
                                 x["block_table_cpu"].numpy(), ctx.numpy(), page_size=P, scale=1.0 / math.sqrt(d),
                                 window=W)
    compare(o, lse, O, LSE, bf16_out=True, what=f"paged P{P} W{W}")


def test_paged_table_entries_past_context_not_read_and_bad_entries_clamped():
    B, H, Hkv, Lmax, d, P = 2, 4, 1, 600, 64, 16
    announce(entry="fa_decode_paged", case="table entries past the context / out of range")
    x = fa_inputs.paged_decode_inputs(B, H, Hkv, Lmax, d, P, seed=520, device=DEV)
    ctx = torch.tensor([100, 37], dtype=torch.int32, device=DEV)
    o1, l1 = _fa().decode_paged(x["q"], x["k_pages"], x["v_pages"], x["block_table"], ctx)
    t = x["block_table"].clone()
    t[0, 7:] = -12345        # positions >= 112 of request 0: never read
    t[1, 3:] = 1 << 30       # positions >= 48 of request 1: never read
    o2, l2 = _fa().decode_paged(x["q"], x["k_pages"], x["v_pages"], t, ctx)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # an entry inside the context that is out of range reads the clamped page
    n = x["num_pages"]
    t_bad, t_clamped = x["block_table"].clone(), x["block_table"].clone()
    t_bad[0, 2], t_clamped[0, 2] = n + 50, n - 1
    t_bad[1, 0], t_clamped[1, 0] = -7, 0
    o3, l3 = _fa().decode_paged(x["q"], x["k_pages"], x["v_pages"], t_bad, ctx)
    o4, l4 = _fa().decode_paged(x["q"], x["k_pages"], x["v_pages"], t_clamped, ctx)
    torch.cuda.synchronize()
    assert torch.equal(o3, o4) and torch.equal(l3, l4)


def test_paged_decode_full_size_sampled():
    """The decode workload (64 requests, 32 query / 8 KV heads, contexts 8192..32768) with its
    cache in 16-key pages scattered through the pool, in bench.py's configuration; sampled
    (request, head) pairs against the oracle on those requests' gathered pages, and every pair
    against the contiguous decode."""
    w = fa_inputs.WORKLOADS["decode_B64_H32_Hkv8_ctx32768_d128"]
    P = 16
    announce(entry="fa_decode_paged", workload=w.name, P=P, case="sampled heads")
    x = fa_inputs.paged_decode_inputs(w.B, w.H, w.Hkv, w.L, w.d, P, seed=w.seed, device=DEV,
                                      len_range=w.len_range)
    o, lse = _fa().decode_paged(x["q"], x["k_pages"], x["v_pages"], x["block_table"], x["ctx_lens"], scale=w.scale)
    torch.cuda.synchronize()
    ctx = x["ctx_lens_cpu"].numpy()
    rng = np.random.default_rng(530)
    for b, h in [(0, 0), (63, 31)] + [(int(rng.integers(64)), int(rng.integers(32))) for _ in range(4)]:
        kvh = h // (w.H // w.Hkv)
        npg = -(-int(ctx[b]) // P)
        pages = x["block_table"][b, :npg].long()
        kp = fa_inputs.as_oracle_f64(x["k_pages"][pages][:, kvh:kvh + 1])  # [npg, 1, P, d]
        vp = fa_inputs.as_oracle_f64(x["v_pages"][pages][:, kvh:kvh + 1])
        O, LSE = oracle.decode_paged(fa_inputs.as_oracle_f64(x["q"][b:b + 1, h:h + 1]), kp, vp,
                                     np.arange(npg)[None], ctx[b:b + 1], page_size=P, scale=w.scale)
        compare(o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], O, LSE, bf16_out=True, what=f"paged 32k b{b} h{h}")
    # Every (request, head): bitwise equal to the contiguous decode of the same cache gathered
    # from its pages, with the paged call's capacity (that decode's every pair is checked
    # against the oracle at full size). Table entries past a context are never read by either;
    # they are clamped into the pool only so that the gather stays in bounds.
    tbl = x["block_table"].long().clamp(0, x["k_pages"].shape[0] - 1)
    cap = tbl.shape[1] * P
    kc = x["k_pages"][tbl].permute(0, 2, 1, 3, 4).reshape(w.B, w.Hkv, cap, w.d).contiguous()
    vc = x["v_pages"][tbl].permute(0, 2, 1, 3, 4).reshape(w.B, w.Hkv, cap, w.d).contiguous()
    o2, l2 = _fa().decode(x["q"], kc, vc, x["ctx_lens"], scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2), "paged decode differs from the contiguous decode"
