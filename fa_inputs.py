"""Seeded synthetic inputs for the attention workloads.

This module is shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``.
It only draws random numbers and lays them out; it holds none of the attention
arithmetic, so neither the CPU oracle nor the HIP path depends on the other
through it.

Recipe (the same for every workload):

* A CPU ``torch.Generator`` seeded with ``seed`` draws the integer lengths first
  (per-sequence valid lengths, or per-request KV-cache lengths), uniform over an
  inclusive range, so lengths never depend on the device.
* A second generator on the target device, seeded with ``seed + 1``, draws Q,
  then K, then V as i.i.d. standard normal float32 in full row-major buffers.
  Padding rows and cache positions past a request's length are drawn too, so a
  mask that leaks changes the result.
* bf16 workloads round the float32 draws to bf16 (round-to-nearest-even). The
  fp32 workload keeps float32 for the kernel and gives the oracle the
  bf16-rounded copy (the kernel rounds on load in the same way).

Layouts: Q and O are ``[B, H, Lq, d]``; K and V are ``[B, Hkv, Lk, d]``; the
decode query is ``[B, H, d]`` and the KV cache ``[B, Hkv, Lmax, d]``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    """One named attention workload (shapes, dtype, mask and seed)."""

    name: str
    kind: str  # "prefill" or "decode"
    B: int
    H: int
    Hkv: int
    L: int  # Lq = Lk for prefill, Lmax (cache capacity) for decode
    d: int
    io: str  # "bf16" or "f32"
    causal: bool
    seed: int
    len_range: tuple | None = None  # inclusive (lo, hi) for varlen / ctx lengths
    notes: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The five workloads: a single-head fp32 check, causal prefill at 2k and 16k,
# GQA variable-length prefill, and decode over a long KV cache.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_head_fp32_L128_d64", "prefill", 1, 1, 1, 128, 64, "f32", False, 1,
                 notes="non-causal, fp32 Q/K/V/O"),
        Workload("causal_prefill_B4_H16_L2048_d64", "prefill", 4, 16, 16, 2048, 64, "bf16", True, 2),
        Workload("causal_prefill_B1_H32_L16384_d128", "prefill", 1, 32, 32, 16384, 128, "bf16", True, 3),
        Workload("gqa_varlen_prefill_B8_H32_Hkv8_L8192_d128", "prefill", 8, 32, 8, 8192, 128, "bf16", True, 4,
                 len_range=(2048, 8192), notes="causal + padding mask"),
        Workload("decode_B64_H32_Hkv8_ctx32768_d128", "decode", 64, 32, 8, 32768, 128, "bf16", False, 5,
                 len_range=(8192, 32768), notes="Lq=1, split-K + LSE combine"),
    ]
}


def draw_lengths(n: int, lo: int, hi: int, seed: int) -> torch.Tensor:
    """n integers uniform over the inclusive range [lo, hi], as int32 on the CPU."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randint(lo, hi + 1, (n,), generator=g, dtype=torch.int64).to(torch.int32)


def _normal(shape, gen, device, chunk_elems=1 << 28):
    """float32 N(0,1) draws of `shape`, generated in slices to bound peak memory."""
    out = torch.empty(shape, dtype=torch.float32, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk_elems):
        e = min(flat.numel(), s + chunk_elems)
        flat[s:e] = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
    return out


def _normal_bf16(shape, gen, device, chunk_elems=1 << 28):
    """bf16 (RNE) of float32 N(0,1) draws, produced slice by slice."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk_elems):
        e = min(flat.numel(), s + chunk_elems)
        flat[s:e] = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    return out


def prefill_inputs(B, H, Hkv, Lq, Lk, d, *, seed, device="cpu", io="bf16", len_range=None):
    """Q, K, V (and optional per-sequence lengths) for a prefill call.

    Returns a dict with ``q, k, v`` in the kernel's I/O dtype, ``seqlens``
    (int32 [B] on ``device`` or None) and ``seqlens_cpu``.
    """
    seqlens = None
    if len_range is not None:
        seqlens = draw_lengths(B, len_range[0], len_range[1], seed)
    gen = torch.Generator(device=device).manual_seed(seed + 1)
    make = _normal if io == "f32" else _normal_bf16
    q = make((B, H, Lq, d), gen, device)
    k = make((B, Hkv, Lk, d), gen, device)
    v = make((B, Hkv, Lk, d), gen, device)
    return {
        "q": q, "k": k, "v": v,
        "seqlens": None if seqlens is None else seqlens.to(device),
        "seqlens_cpu": seqlens,
    }


def decode_inputs(B, H, Hkv, Lmax, d, *, seed, device="cpu", len_range=(1, None)):
    """Decode query, KV cache and per-request context lengths (all bf16 / int32)."""
    lo, hi = len_range
    hi = Lmax if hi is None else hi
    ctx = draw_lengths(B, lo, hi, seed)
    gen = torch.Generator(device=device).manual_seed(seed + 1)
    q = _normal_bf16((B, H, d), gen, device)
    kc = _normal_bf16((B, Hkv, Lmax, d), gen, device)
    vc = _normal_bf16((B, Hkv, Lmax, d), gen, device)
    return {"q": q, "k_cache": kc, "v_cache": vc, "ctx_lens": ctx.to(device), "ctx_lens_cpu": ctx}


def paged_decode_inputs(B, H, Hkv, Lmax, d, page_size, *, seed, device="cpu", len_range=(1, None), spare_pages=3):
    """Decode inputs with the KV cache in pages: pools k_pages, v_pages [num_pages, Hkv, P, d]
    (bf16) and an int32 block table [B, ceil(Lmax / P)] whose entries are a random
    permutation of the pool's pages (scattered, as an allocator leaves them after churn),
    plus ``spare_pages`` pages that no table row names. Context lengths as decode_inputs."""
    lo, hi = len_range
    hi = Lmax if hi is None else hi
    ctx = draw_lengths(B, lo, hi, seed)
    max_pages = (Lmax + page_size - 1) // page_size
    num_pages = B * max_pages + spare_pages
    g = torch.Generator(device="cpu").manual_seed(seed + 2)
    table = torch.randperm(num_pages, generator=g)[:B * max_pages].reshape(B, max_pages).to(torch.int32)
    gen = torch.Generator(device=device).manual_seed(seed + 1)
    q = _normal_bf16((B, H, d), gen, device)
    kp = _normal_bf16((num_pages, Hkv, page_size, d), gen, device)
    vp = _normal_bf16((num_pages, Hkv, page_size, d), gen, device)
    return {"q": q, "k_pages": kp, "v_pages": vp, "block_table": table.to(device), "block_table_cpu": table,
            "ctx_lens": ctx.to(device), "ctx_lens_cpu": ctx, "page_size": page_size, "num_pages": num_pages}


def fp8_prefill_inputs(B, H, Hkv, Lq, Lk, d, *, seed, device="cpu", len_range=None):
    """FP8 prefill inputs: q, k, v as OCP E4M3 codes (uint8) of seeded normal values, each
    (batch, head) scaled into the format's range by its own descale (amax / 240), and the
    descales (fp32 [B, H] for q, [B, Hkv] for k and v). Dequantised: x = decode(code) * descale."""
    seqlens = None
    if len_range is not None:
        seqlens = draw_lengths(B, len_range[0], len_range[1], seed)
    gen = torch.Generator(device=device).manual_seed(seed + 1)
    out = {}
    for name, heads, L in (("q", H, Lq), ("k", Hkv, Lk), ("v", Hkv, Lk)):
        x = _normal((B, heads, L, d), gen, device)
        amax = x.abs().amax(dim=(2, 3)).clamp(min=1e-6) if x.numel() else torch.ones(x.shape[:2], device=device)
        ds = (amax / 240.0).to(torch.float32)
        codes = (x / ds[:, :, None, None]).to(torch.float8_e4m3fn).view(torch.uint8)
        out[name], out[name + "_descale"] = codes.contiguous(), ds.contiguous()
    out["seqlens"] = None if seqlens is None else seqlens.to(device)
    out["seqlens_cpu"] = seqlens
    return out


def workload_inputs(w: Workload, device="cpu"):
    """Inputs for a named workload at its full size."""
    if w.kind == "prefill":
        return prefill_inputs(w.B, w.H, w.Hkv, w.L, w.L, w.d, seed=w.seed, device=device, io=w.io,
                              len_range=w.len_range)
    return decode_inputs(w.B, w.H, w.Hkv, w.L, w.d, seed=w.seed, device=device, len_range=w.len_range)


def as_oracle_f64(t: torch.Tensor):
    """The float64 numpy array the oracle sees: bf16 rounding (RNE) first, then exact widening."""
    return t.detach().to("cpu").to(torch.bfloat16).to(torch.float64).numpy()
