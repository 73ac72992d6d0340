"""The Python binding rejects malformed tensors before anything reaches the C ABI.

libfa only receives raw pointers and sizes, so a k/v whose shape does not match q, a short
or host-resident length tensor, or a block table with too few rows would be read out of
bounds by the kernels. Every such call must raise ValueError on the host (no GPU needed:
CPU tensors stop at the shape checks, or at the device check when every shape is right).
"""
import pytest
import torch

fa = pytest.importorskip("exact_attention_111_amd")

bf = torch.bfloat16


def _pf(B=2, H=4, Hkv=2, L=8, d=64):
    return (torch.zeros(B, H, L, d, dtype=bf), torch.zeros(B, Hkv, L, d, dtype=bf),
            torch.zeros(B, Hkv, L, d, dtype=bf))


def test_fwd_shape_checks():
    q, k, v = _pf()
    with pytest.raises(ValueError, match="v must have shape"):
        fa.fwd(q, k, v[:, :, :5].contiguous())
    with pytest.raises(ValueError, match="k must have shape"):
        fa.fwd(q, torch.zeros(3, 2, 8, 64, dtype=bf), v)           # batch differs from q
    with pytest.raises(ValueError, match="k must have shape"):
        fa.fwd(q, torch.zeros(2, 2, 8, 128, dtype=bf), v)          # head dim differs from q
    with pytest.raises(ValueError, match="4-D"):
        fa.fwd(q[0], k, v)
    with pytest.raises(ValueError, match="out must have shape"):
        fa.fwd(q, k, v, out=torch.zeros(2, 4, 7, 64, dtype=bf))
    with pytest.raises(ValueError, match="lse must have shape"):
        fa.fwd(q, k, v, lse=torch.zeros(2, 4, 9))
    with pytest.raises(ValueError, match="lse must be float32"):
        fa.fwd(q, k, v, lse=torch.zeros(2, 4, 8, dtype=torch.float64))
    with pytest.raises(ValueError, match="seqlens must have shape"):
        fa.fwd(q, k, v, seqlens=torch.zeros(1, dtype=torch.int32))  # fewer than B lengths
    with pytest.raises(ValueError, match="seqlens must be int32"):
        fa.fwd(q, k, v, seqlens=torch.zeros(2, dtype=torch.int64))
    with pytest.raises(ValueError, match="contiguous"):
        fa.fwd(q.transpose(2, 3).contiguous().transpose(2, 3), k, v)
    with pytest.raises(ValueError, match="runs on a GPU"):
        fa.fwd(q, k, v)  # every shape right: host tensors stop at the device check


def test_fwd_fp8_shape_checks():
    u8 = torch.uint8
    q, k, v = torch.zeros(1, 4, 8, 128, dtype=u8), torch.zeros(1, 2, 8, 128, dtype=u8), torch.zeros(1, 2, 8, 128,
                                                                                                     dtype=u8)
    qs, ks, vs = torch.ones(1, 4), torch.ones(1, 2), torch.ones(1, 2)
    with pytest.raises(ValueError, match="q_descale must have shape"):
        fa.fwd_fp8(q, k, v, torch.ones(1, 2), ks, vs)
    with pytest.raises(ValueError, match="v_descale must have shape"):
        fa.fwd_fp8(q, k, v, qs, ks, torch.ones(2))
    with pytest.raises(ValueError, match="v must have shape"):
        fa.fwd_fp8(q, k, torch.zeros(1, 2, 9, 128, dtype=u8), qs, ks, vs)
    with pytest.raises(ValueError, match="runs on a GPU"):
        fa.fwd_fp8(q, k, v, qs, ks, vs)


def test_decode_shape_checks():
    q = torch.zeros(2, 4, 64, dtype=bf)
    kc = torch.zeros(2, 2, 100, 64, dtype=bf)
    ctx = torch.tensor([5, 9], dtype=torch.int32)
    with pytest.raises(ValueError, match="v_cache must have shape"):
        fa.decode(q, kc, torch.zeros(2, 2, 99, 64, dtype=bf), ctx)
    with pytest.raises(ValueError, match="k_cache must have shape"):
        fa.decode(q, torch.zeros(1, 2, 100, 64, dtype=bf), kc, ctx)
    with pytest.raises(ValueError, match="ctx_lens must have shape"):
        fa.decode(q, kc, kc, torch.tensor([5], dtype=torch.int32))  # a length short
    with pytest.raises(ValueError, match="ctx_lens must be int32"):
        fa.decode(q, kc, kc, ctx.long())
    with pytest.raises(ValueError, match="out must have shape"):
        fa.decode(q, kc, kc, ctx, out=torch.zeros(2, 4, 32, dtype=bf))
    with pytest.raises(ValueError, match="runs on a GPU"):
        fa.decode(q, kc, kc, ctx)


def test_decode_paged_shape_checks():
    q = torch.zeros(2, 4, 128, dtype=bf)
    kp = torch.zeros(10, 2, 16, 128, dtype=bf)
    table = torch.zeros(2, 4, dtype=torch.int32)
    ctx = torch.tensor([5, 9], dtype=torch.int32)
    with pytest.raises(ValueError, match="block_table must have B = 2 rows"):
        fa.decode_paged(q, kp, kp, table[:1].contiguous(), ctx)
    with pytest.raises(ValueError, match="v_pages must have shape"):
        fa.decode_paged(q, kp, torch.zeros(10, 2, 32, 128, dtype=bf), table, ctx)
    with pytest.raises(ValueError, match="ctx_lens must have shape"):
        fa.decode_paged(q, kp, kp, table, torch.tensor([1, 2, 3], dtype=torch.int32))
    with pytest.raises(ValueError, match="block_table must be int32"):
        fa.decode_paged(q, kp, kp, table.long(), ctx)
    with pytest.raises(ValueError, match="runs on a GPU"):
        fa.decode_paged(q, kp, kp, table, ctx)


def test_bwd_shape_checks():
    q, k, v = _pf(d=128)
    lse = torch.zeros(2, 4, 8)
    with pytest.raises(ValueError, match="dout must have shape"):
        fa.bwd(q, k, v, q, q[:, :, :4].contiguous(), lse)
    with pytest.raises(ValueError, match="o must have shape"):
        fa.bwd(q, k, v, q[:1].contiguous(), q, lse)
    with pytest.raises(ValueError, match="lse must have shape"):
        fa.bwd(q, k, v, q, q, lse[:, :2].contiguous())
    with pytest.raises(ValueError, match="dk must have shape"):
        fa.bwd(q, k, v, q, q, lse, dk=torch.zeros_like(q))
    with pytest.raises(ValueError, match="seqlens must have shape"):
        fa.bwd(q, k, v, q, q, lse, seqlens=torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="runs on a GPU"):
        fa.bwd(q, k, v, q, q, lse)
