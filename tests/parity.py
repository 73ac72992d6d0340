"""Comparison of HIP-path outputs with the fp64 oracle, at the stated tolerance.

Tolerance: O within max-abs 1e-2 and mean-abs 1e-3, LSE within 1e-3 abs, with the
oracle fed the bf16-rounded inputs. For a bf16 output the rounding of the output
itself is not counted as error: an element passes when it is within 1e-2 of the exact
value plus half a bf16 ulp of that value (|O| >= 4 alone has a half ulp of 0.0156), and
the mean is taken against the oracle rounded to bf16. fp32 outputs are compared with
the exact value directly. Rows the oracle marks empty (LSE = -inf) must be exactly
O = 0 and LSE = -inf.
"""
import numpy as np
import torch

O_MAX = 1e-2
O_MEAN = 1e-3
LSE_MAX = 1e-3


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |x| (8 significand bits): 2^(e - 9) for |x| in [2^(e-1), 2^e)."""
    _, e = np.frexp(np.abs(x))
    return np.where(x == 0, 0.0, np.ldexp(1.0, e - 9))


def compare(o_gpu, lse_gpu, O_ref, LSE_ref, *, bf16_out: bool, what: str = "", o_slack=None):
    """Assert parity; returns a dict of error statistics. Arrays are broadcast-compatible.
    ``o_slack``: optional per-row allowance (shape of LSE_ref) added to the max-abs bound of O,
    for results with several correct values (fp8_flip_slack)."""
    o = o_gpu.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(o_gpu) else np.asarray(o_gpu)
    lse = lse_gpu.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(lse_gpu) else np.asarray(lse_gpu)
    O_ref = np.asarray(O_ref, dtype=np.float64)
    LSE_ref = np.asarray(LSE_ref, dtype=np.float64)
    assert o.shape == O_ref.shape, (what, o.shape, O_ref.shape)
    assert lse.shape == LSE_ref.shape, (what, lse.shape, LSE_ref.shape)
    assert not np.isnan(o).any(), f"{what}: NaN in O"
    empty = ~np.isfinite(LSE_ref)  # rows that see no key
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: LSE = -inf rows differ"
    empty_o = np.broadcast_to(empty[..., None], O_ref.shape)
    assert np.all(o[empty_o] == 0.0), f"{what}: empty rows must have O = 0"
    full_o = ~empty_o
    stats = {"rows": int((~empty).sum())}
    if not full_o.any():
        return stats
    slack = 0.0 if o_slack is None else np.broadcast_to(np.asarray(o_slack, dtype=np.float64)[..., None], O_ref.shape)
    err = np.abs(o - O_ref)[full_o]
    if bf16_out:
        excess = (np.abs(o - O_ref) - half_ulp_bf16(O_ref) - slack)[full_o]
        ref_r = torch.from_numpy(np.ascontiguousarray(O_ref)).to(torch.bfloat16).double().numpy()
        mean = float(np.abs(o - ref_r)[full_o].mean())
        worst = float(excess.max())
        assert worst <= O_MAX, f"{what}: O error beyond output rounding {worst:.3g} > {O_MAX}"
    else:
        mean = float(err.mean())
        worst = float(err.max())
        assert worst <= O_MAX, f"{what}: O max-abs error {worst:.3g} > {O_MAX}"
    assert mean <= O_MEAN, f"{what}: O mean-abs error {mean:.3g} > {O_MEAN}"
    lerr = float(np.abs(lse[~empty] - LSE_ref[~empty]).max())
    assert lerr <= LSE_MAX, f"{what}: LSE error {lerr:.3g} > {LSE_MAX}"
    stats.update(o_max=worst, o_mean=mean, lse_max=lerr, o_raw_max=float(err.max()))
    return stats


# Gradients (fa_bwd): P and dS enter the products as bf16 (2^-9 relative rounding) with fp32
# accumulation, and dQ, dK, dV are rounded to bf16, so each gradient is held relative to its
# own size: max |err| <= 2^-5 max |ref| and mean |err| <= 2^-7 mean |ref|.
G_MAX_REL = 2.0 ** -5
G_MEAN_REL = 2.0 ** -7


def compare_grad(got, ref, what, floor=1e-30):
    """Assert gradient parity. ``floor``: the size below which a gradient counts as zero
    (then the bound is absolute). Returns (max-rel, mean-rel)."""
    got = got.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(got) else np.asarray(got)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref)
    mx = err.max() / max(np.abs(ref).max(), floor) if err.size else 0.0
    mn = err.mean() / max(np.abs(ref).mean(), floor) if err.size else 0.0
    print(f"  {what}: max|err|/max|ref| = {mx:.2e}, mean|err|/mean|ref| = {mn:.2e}", flush=True)
    assert mx <= G_MAX_REL and mn <= G_MEAN_REL, f"{what}: {mx:.3e} / {mn:.3e}"
    return mx, mn


# FP8 prefill: a probability x = 2^8 2^(t - m) is rounded to E4M3. The GPU forms t from the FP8
# matrix cores' sums and v_exp_f32; measured against float64 its x deviate by up to 3e-5
# relative (the worst outliers of a 300 x 300 case, each explained by one single flipped
# rounding), so an x that lies that close to a rounding midpoint of E4M3 may round the other
# way on the GPU: both values are correct roundings of the same quantity within the kernel's
# precision. Each such element can move O_i by one E4M3 spacing of x_j times |v_j| over
# sum_j x_j. fp8_flip_slack returns that allowance per row for elements within a relative
# band of 2^-12 of a midpoint (eight times the measured deviation; about 1 in 250 elements).
FLIP_BAND = 2.0 ** -12


def fp8_flip_slack(Q, K, V, *, scale, causal=False, n_valid=None, rows=None, window=None):
    """Per-row O allowance for E4M3 rounding decisions that fp32 can take either way (fp64
    inputs already dequantised; the same masks as the oracle)."""
    import importlib
    OA = importlib.import_module("oracle.attention")  # the module (the package exports a function of that name)
    Lq, Lk = Q.shape[0], K.shape[0]
    row_idx = np.arange(Lq) if rows is None else np.asarray(rows)
    n = Lk if n_valid is None else int(n_valid)
    t = (scale * np.log2(np.e)) * (Q[row_idx] @ K.T)
    vis = OA._visible(Lq, Lk, causal, n, row_idx, window)
    t = np.where(vis, t, -np.inf)
    tmax = t.max(axis=1) if Lk > 0 else np.full(len(row_idx), -np.inf)
    M = np.ceil(np.where(np.isfinite(tmax), tmax, 0.0))
    x = 256.0 * np.exp2(t - M[:, None])
    _, E = np.frexp(np.where(x > 0, x, 1.0))
    spacing = 2.0 ** (np.maximum(E - 1.0, -6.0) - 3.0)
    frac = x / spacing - np.floor(x / spacing)
    near = (np.abs(frac - 0.5) * spacing <= FLIP_BAND * x) & (x > 0)
    vmax = np.abs(V).max(axis=1)
    num = (np.where(near, spacing, 0.0) * vmax[None, :]).sum(axis=1)
    den = np.maximum(x.sum(axis=1), 1e-300)
    return num / den
