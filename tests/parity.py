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

# Lines of per-workload error statistics, printed at the end of the test session
# (tests/conftest.py), so that a quiet pytest run still shows them.
SUMMARY = []


def report(line: str):
    SUMMARY.append(line)
    print(line, flush=True)


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


# Gradients (fa_bwd). The pages give no tolerance for the backward pass; this bound follows
# the kernels' arithmetic, element by element. bf16 keeps 8 significant bits, so one rounding
# moves a value by at most u = 2^-8 of itself. Every product term of a gradient carries
# bf16-rounded factors: P and dS = P (dP - D) are rounded to bf16 before their products, and
# D_i = sum_c dO_ic O_ic is formed from the forward's bf16 O, whose own error is within a
# rounding of sum_j P_ij |V_j|. Accumulation is fp32. So the error of an element is at most two
# roundings (2u = 2^-7) of the SUM OF ABSOLUTE VALUES of its terms, plus the rounding of the
# bf16 output itself:
#     dV_jc:  2^-7 sum_i P_ij |dO_ic|
#     dK_jc:  2^-7 scale sum_i W_ij |Q_ic|     W_ij = |dS_ij| + 2 P_ij Delta_i
#     dQ_ic:  2^-7 scale sum_j W_ij |K_jc|     Delta_i = sum_c |dO_ic| (P |V|)_ic
# (summed over the query heads of a KV head for dK and dV). The bound is per element: a row of
# small gradients is held to its own terms, not to the largest gradient of the tensor, and
# exact zeros (a single key gives dQ = dK = 0) are held to the rounding of dP - D.
GRAD_REL = 2.0 ** -7
G_MEAN_REL = 2.0 ** -7


def grad_terms_head(q, k, v, do, *, scale, causal=False, n_valid=None, window=None):
    """(P, |dS|, Delta) of one head from the oracle's P (float64): the magnitudes that set the
    gradient error allowances above. Rows of P are 0 where a row sees nothing."""
    from oracle.attention import attention_head
    O, _, P = attention_head(q, k, v, scale=scale, causal=causal, n_valid=n_valid, return_p=True, window=window)
    D = (do * O).sum(axis=1)
    absdS = np.abs(P * (do @ v.T - D[:, None]))
    delta = (np.abs(do) * (P @ np.abs(v))).sum(axis=1)
    return P, absdS, delta


def grad_tolerances(q, k, v, do, *, scale, causal=False, seqlens=None, window=None):
    """Per-element allowances (tQ [B,H,Lq,d], tK, tV [B,Hkv,Lk,d]) for fa_bwd against the
    oracle, on float64 inputs of the same layout as the oracle's."""
    B, H, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    group = H // Hkv
    tQ = np.zeros((B, H, Lq, d))
    tK = np.zeros((B, Hkv, Lk, d))
    tV = np.zeros((B, Hkv, Lk, d))
    for b in range(B):
        n = None if seqlens is None else int(seqlens[b])
        for h in range(H):
            kvh = h // group
            P, absdS, delta = grad_terms_head(q[b, h], k[b, kvh], v[b, kvh], do[b, h], scale=scale, causal=causal,
                                              n_valid=n, window=window)
            W = absdS + 2.0 * P * delta[:, None]
            tQ[b, h] = GRAD_REL * scale * (W @ np.abs(k[b, kvh]))
            tK[b, kvh] += GRAD_REL * scale * (W.T @ np.abs(q[b, h]))
            tV[b, kvh] += GRAD_REL * (P.T @ np.abs(do[b, h]))
    return tQ, tK, tV


def compare_grad(got, ref, what, tol):
    """Assert gradient parity element by element: |got - ref| <= tol + half a bf16 ulp of ref,
    and mean |err| <= 2^-7 of the mean |ref| (or of the mean allowance, if larger). Returns the largest err / allowance."""
    got = got.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(got) else np.asarray(got)
    ref = np.asarray(ref, dtype=np.float64)
    tol = np.broadcast_to(np.asarray(tol, dtype=np.float64), ref.shape)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    if not got.size:
        return 0.0
    err = np.abs(got - ref)
    allow = tol + half_ulp_bf16(ref)
    ratio = np.where(allow > 0, err / np.where(allow > 0, allow, 1.0), np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max())
    # mean error against the mean size of the gradient (or of its terms, where the exact
    # gradient is zero, as with a single key)
    mn = err.mean() / max(np.abs(ref).mean(), allow.mean(), 1e-30)
    at = np.unravel_index(int(ratio.argmax()), ratio.shape)
    print(f"  {what}: max err/allowance = {worst:.3f} (at {tuple(int(i) for i in at)}: err {err[at]:.3g}, "
          f"allowance {allow[at]:.3g}), mean|err|/mean|ref| = {mn:.2e}", flush=True)
    assert worst <= 1.0, f"{what}: error {err[at]:.3g} beyond its allowance {allow[at]:.3g} at {at}"
    assert mn <= G_MEAN_REL, f"{what}: mean error {mn:.3e}"
    return worst


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


# FP8 prefill against the EXACT attention of the dequantised inputs (not the scheme oracle).
# E4M3 keeps 4 significant bits, so rounding 2^8 p to it moves each probability by at most 2^-4
# of itself (both neighbours of a midpoint qualify, so a flipped rounding stays inside this),
# while the row sum l is exact. O_i - O_exact_i = sum_j (pq_j - p_j) V_j / l, so
#     |O_ic - O_exact_ic| <= 2^-4 sum_j P_ij |V_jc| + half a bf16 ulp of O_exact_ic
#                            + 2^-12 max_j |V_jc|   (fp32 sums; probabilities below E4M3's normal range)
# with P the exact probabilities; LSE is held to the bf16 bar (1e-3), since l adds unrounded p.
# On random data this is the 2^-4 x (spread of V) bound the FP8 oracle is pinned to.
FP8_REL = 2.0 ** -4


def compare_fp8_exact(o_gpu, lse_gpu, Q, K, V, *, scale, causal=False, n_valid=None, rows=None, window=None,
                      what=""):
    """Assert the FP8 prefill output of one head against exact fp64 attention of the dequantised
    Q, K, V (float64 arrays), element by element at the bound above. Returns the largest
    error / allowance ratio."""
    from oracle.attention import attention_head
    o = o_gpu.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(o_gpu) else np.asarray(o_gpu)
    lse = lse_gpu.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(lse_gpu) else np.asarray(lse_gpu)
    O, LSE, P = attention_head(Q, K, V, scale=scale, causal=causal, n_valid=n_valid, rows=rows, window=window,
                               return_p=True)
    empty = ~np.isfinite(LSE)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: LSE = -inf rows differ"
    assert np.all(o[empty] == 0.0), f"{what}: empty rows must have O = 0"
    if empty.all():
        return 0.0
    allow = FP8_REL * (P @ np.abs(V)) + half_ulp_bf16(O) + 2.0 ** -12 * np.abs(V).max(axis=0)[None, :]
    ratio = (np.abs(o - O) / allow)[~empty]
    worst = float(ratio.max())
    lerr = float(np.abs(lse[~empty] - LSE[~empty]).max())
    print(f"  {what}: vs exact attention: max err/allowance = {worst:.3f}, LSE {lerr:.3g}", flush=True)
    assert worst <= 1.0, f"{what}: O beyond the E4M3 bound against exact attention ({worst:.3f})"
    assert lerr <= LSE_MAX, f"{what}: LSE error {lerr:.3g} > {LSE_MAX}"
    return worst


# Coverage of every workgroup: rows sampled per query tile and per wave, and outputs that
# start out NaN so that a tile never written is caught over the whole tensor.
QTILE = 256  # query rows per prefill workgroup
WBLK = 32    # query rows per wave


def rows_per_workgroup(n_valid, rng):
    """One random row of every 32-row block below n_valid, plus the first and last row of every
    256-row query tile (clipped to n_valid)."""
    rows = set()
    for t0 in range(0, n_valid, QTILE):
        rows.add(t0)
        rows.add(min(t0 + QTILE, n_valid) - 1)
    for b0 in range(0, n_valid, WBLK):
        rows.add(int(rng.integers(b0, min(b0 + WBLK, n_valid))))
    return np.array(sorted(rows), dtype=np.int64)


def nan_filled_outputs(shape_o, shape_lse, dtype, device="cuda:0"):
    o = torch.full(shape_o, float("nan"), dtype=dtype, device=device)
    lse = torch.full(shape_lse, float("nan"), dtype=torch.float32, device=device)
    return o, lse


def check_written(o, lse, n_valid):
    """Whole-tensor check on the GPU: rows below n_valid[b] finite, rows at or past it O = 0
    and LSE = -inf (n_valid None: every row valid)."""
    B = o.shape[0]
    L = o.shape[2]
    for b in range(B):
        n = L if n_valid is None else int(n_valid[b])
        assert torch.isfinite(o[b, :, :n]).all(), f"batch {b}: a valid O row is not finite (unwritten?)"
        assert torch.isfinite(lse[b, :, :n]).all(), f"batch {b}: a valid LSE is not finite (unwritten?)"
        if n < L:
            assert torch.all(o[b, :, n:] == 0), f"batch {b}: padding rows of O are not 0"
            assert torch.all(torch.isneginf(lse[b, :, n:])), f"batch {b}: padding LSE is not -inf"


# Exact gradients of selected rows (dQ) or keys (dK, dV) of one head, for long sequences where
# the whole-tensor oracle is too slow; each returns the elements' allowances beside them.
def _attention_head(*args, **kw):
    import importlib
    return importlib.import_module("oracle.attention").attention_head(*args, **kw)


def grad_rows_oracle(q, k, v, do, rows, *, scale, causal):
    """dQ rows exactly: each row needs only its own P and dP rows. Also returns each element's
    allowance (``parity.grad_tolerances``, restricted to these rows)."""
    dQ, tQ = [], []
    for i in rows:
        O, _, P = _attention_head(q, k, v, scale=scale, causal=causal, rows=[i], return_p=True)
        dP = do[i] @ v.T
        D = float(do[i] @ O[0])
        dQ.append(scale * ((P[0] * (dP - D)) @ k))
        delta = float(np.abs(do[i]) @ (P[0] @ np.abs(v)))
        W = np.abs(P[0] * (dP - D)) + 2.0 * P[0] * delta
        tQ.append(GRAD_REL * scale * (W @ np.abs(k)))
    return np.stack(dQ), np.stack(tQ)


def grad_keys_oracle(q, k, v, do, keys, *, scale, causal, block=1024, row_from=0):
    """dK, dV rows of the given keys exactly: O and LSE of every row first (in row blocks),
    then the columns of P and dS for those keys. With a causal mask and every key at or after
    row_from, rows before row_from see none of them and are left out."""
    L = q.shape[0]
    assert row_from == 0 or (causal and min(keys) >= row_from)
    R = np.arange(row_from, L)
    O = np.empty((len(R), q.shape[1]))
    OA = np.empty_like(O)  # P |V|, for the allowances
    LSE = np.empty(len(R))
    for r0 in range(0, len(R), block):
        sel = np.arange(r0, min(len(R), r0 + block))
        O[sel], LSE[sel] = _attention_head(q, k, v, scale=scale, causal=causal, rows=R[sel])
        OA[sel], _ = _attention_head(q, k, np.abs(v), scale=scale, causal=causal, rows=R[sel])
    qR, doR = q[R], do[R]
    D = (doR * O).sum(axis=1)
    delta = (np.abs(doR) * OA).sum(axis=1)
    dK, dV, tK, tV = [], [], [], []
    for j in keys:
        s = scale * (qR @ k[j])
        vis = (R >= j) if causal else np.ones(len(R), bool)
        p = np.where(vis, np.exp(np.where(vis, s, 0.0) - LSE), 0.0)
        dp = doR @ v[j]
        ds = p * (dp - D)
        dK.append(scale * (ds @ qR))
        dV.append(p @ doR)
        tK.append(GRAD_REL * scale * ((np.abs(ds) + 2.0 * p * delta) @ np.abs(qR)))
        tV.append(GRAD_REL * (p @ np.abs(doR)))
    return np.stack(dK), np.stack(dV), np.stack(tK), np.stack(tV)
