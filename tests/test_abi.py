"""The C ABI without a GPU: libfa.so loads, exports every function include/fa.h declares,
and rejects malformed calls on the host before anything is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

fa = pytest.importorskip("exact_attention_111_amd")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = fa.lib()
    names = _declared_functions()
    assert set(names) == {"fa_fwd", "fa_fwd_sliding_window", "fa_fwd_fp8", "fa_fwd_f32", "fa_decode", "fa_decode_sliding_window",
                          "fa_decode_noalloc", "fa_decode_paged",
                          "fa_decode_workspace_bytes", "fa_bwd", "fa_bwd_sliding_window", "fa_bwd_workspace_bytes",
                          "fa_status_string"}
    assert set(names) == set(fa.binding.SYMBOLS)
    for name in names:
        assert hasattr(L, name), name


def test_status_strings():
    assert fa.status_string(0) == "FA_OK"
    assert fa.status_string(1) == "FA_ERR_INVALID"
    assert fa.status_string(2) == "FA_ERR_UNSUPPORTED"
    assert fa.status_string(3) == "FA_ERR_HIP"
    assert fa.status_string(4) == "FA_ERR_TOO_LARGE"


# Fake, never-dereferenced device addresses: validation only looks at their values.
A = 0x10000
A2 = 0x20000
MIS = 0x10008  # 8-byte aligned only


def _fwd(q=A, k=A, v=A, o=A2, lse=A2, B=1, H=2, Hkv=1, Lq=4, Lk=4, d=64, scale=0.125, causal=0, seqlens=None,
         fn="fa_fwd"):
    L = fa.lib()
    return getattr(L, fn)(q, k, v, o, lse, B, H, Hkv, Lq, Lk, d, scale, causal, seqlens, None)


@pytest.mark.parametrize("fn", ["fa_fwd", "fa_fwd_f32"])
def test_fwd_validation(fn):
    INV, UNS = fa.binding.FA_ERR_INVALID, fa.binding.FA_ERR_UNSUPPORTED
    assert _fwd(q=None, fn=fn) == INV
    assert _fwd(o=None, fn=fn) == INV
    assert _fwd(lse=None, fn=fn) == INV
    assert _fwd(k=MIS, fn=fn) == INV
    assert _fwd(B=-1, fn=fn) == INV
    assert _fwd(Hkv=0, fn=fn) == INV
    assert _fwd(H=3, Hkv=2, fn=fn) == INV
    assert _fwd(scale=0.0, fn=fn) == INV
    assert _fwd(scale=float("nan"), fn=fn) == INV
    assert _fwd(scale=float("inf"), fn=fn) == INV
    assert _fwd(causal=2, fn=fn) == INV
    assert _fwd(Lq=4, Lk=5, seqlens=A, fn=fn) == INV  # lengths need Lq == Lk
    assert _fwd(d=96, fn=fn) == UNS
    assert _fwd(d=256, fn=fn) == UNS
    assert _fwd(d=0, fn=fn) == INV
    # Empty calls are valid and enqueue nothing (so they are safe without a GPU).
    assert _fwd(B=0, fn=fn) == 0
    assert _fwd(H=0, fn=fn) == 0
    assert _fwd(Lq=0, Lk=0, fn=fn) == 0
    assert _fwd(q=None, o=None, lse=None, B=0, fn=fn) == 0


def test_decode_workspace_bytes():
    L = fa.lib()
    assert L.fa_decode_workspace_bytes(64, 32, 32768, 128) == 64 * 32 * (32768 // 2048) * 130 * 4
    assert L.fa_decode_workspace_bytes(2, 4, 2049, 64) == 2 * 4 * 2 * 66 * 4
    assert L.fa_decode_workspace_bytes(2, 4, 2048, 64) == 2 * 4 * 1 * 66 * 4
    assert L.fa_decode_workspace_bytes(2, 4, 0, 64) == 0
    assert L.fa_decode_workspace_bytes(-1, 4, 10, 64) == 0


def test_decode_validation():
    L = fa.lib()
    INV, UNS = fa.binding.FA_ERR_INVALID, fa.binding.FA_ERR_UNSUPPORTED
    need = L.fa_decode_workspace_bytes(2, 4, 100, 64)

    def call(q=A, k=A, v=A, o=A2, lse=A2, B=2, H=4, Hkv=2, Lmax=100, d=64, scale=0.125, ctx=A, ws=A2, wsb=need):
        return L.fa_decode(q, k, v, o, lse, B, H, Hkv, Lmax, d, scale, ctx, ws, wsb, None)

    assert call(q=None) == INV
    assert call(ctx=None) == INV
    assert call(ws=None) == INV
    assert call(wsb=need - 1) == INV
    assert call(ws=MIS) == INV
    assert call(H=4, Hkv=3) == INV
    assert call(scale=-1.0) == INV
    assert call(d=80) == UNS
    assert call(B=0) == 0
    assert call(H=0, q=None, o=None, lse=None) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from exact_attention_111_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "_LIB_PATH", str(tmp_path / "missing" / "libfa.so"))
    with pytest.raises(ImportError):
        binding.lib()


def test_bwd_workspace_bytes():
    L = fa.lib()
    assert L.fa_bwd_workspace_bytes(1, 32, 16384) == 32 * 16384 * 8
    assert L.fa_bwd_workspace_bytes(2, 3, 0) == 0
    assert L.fa_bwd_workspace_bytes(-1, 3, 5) == 0


def test_bwd_validation():
    L = fa.lib()
    INV, UNS = fa.binding.FA_ERR_INVALID, fa.binding.FA_ERR_UNSUPPORTED
    need = L.fa_bwd_workspace_bytes(2, 4, 100)

    def call(q=A, k=A, v=A, o=A, do=A, lse=A, dq=A, dk=A, dv=A, B=2, H=4, Hkv=2, Lq=100, Lk=100, d=128,
             scale=0.125, causal=1, seqlens=None, ws=A2, ws_bytes=need):
        return L.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, B, H, Hkv, Lq, Lk, d, scale, causal, seqlens, ws, ws_bytes,
                        None)
    assert call(dk=None) == INV
    assert call(do=MIS) == INV
    assert call(H=5) == INV
    assert call(scale=-1.0) == INV
    assert call(causal=3) == INV
    assert call(Lq=4, Lk=5, seqlens=A) == INV
    assert call(ws=None) == INV
    assert call(ws_bytes=need - 4) == INV
    assert call(d=96) == UNS
    assert call(B=0) == 0  # empty: nothing to write, nothing enqueued


def test_sliding_window_validation():
    """window < 1 is rejected by all three sliding-window entry points; everything else is
    validated as for the plain entry points."""
    L = fa.lib()
    INV = fa.binding.FA_ERR_INVALID
    for w in (0, -3):
        assert _fwd(causal=w, fn="fa_fwd_sliding_window") == INV
    assert _fwd(causal=4, fn="fa_fwd_sliding_window", H=3, Hkv=2) == INV  # H % Hkv
    assert _fwd(causal=4, fn="fa_fwd_sliding_window", d=96) == fa.binding.FA_ERR_UNSUPPORTED
    assert _fwd(causal=4, fn="fa_fwd_sliding_window", B=0) == fa.binding.FA_OK  # empty call, nothing enqueued
    need = L.fa_decode_workspace_bytes(2, 4, 100, 128)
    for w in (0, -1):
        assert L.fa_decode_sliding_window(A, A, A, A2, A2, 2, 4, 2, 100, 128, 0.1, A, w, A2, need, None) == INV
    assert L.fa_decode_sliding_window(A, A, A, A2, A2, 2, 4, 2, 100, 128, 0.1, A, 8, A2, need - 1, None) == INV
    bneed = L.fa_bwd_workspace_bytes(2, 4, 100)
    for w in (0, -2):
        assert L.fa_bwd_sliding_window(A, A, A, A, A, A, A2, A2, A2, 2, 4, 2, 100, 100, 128, 0.1, w, None, A2, bneed,
                                       None) == INV
    assert L.fa_bwd_sliding_window(A, A, A, A, A, A, A2, A2, A2, 2, 4, 2, 100, 100, 128, 0.1, 5, None, A2,
                                   bneed - 1, None) == INV


def test_decode_paged_validation():
    L = fa.lib()
    INV, UNS, OK = fa.binding.FA_ERR_INVALID, fa.binding.FA_ERR_UNSUPPORTED, fa.binding.FA_OK
    need = L.fa_decode_workspace_bytes(2, 4, 8 * 16, 128)

    def call(q=A, kp=A, vp=A, o=A2, lse=A2, B=2, H=4, Hkv=2, d=128, scale=0.1, P=16, npg=20, table=A, mp=8,
             ctx=A, window=0, ws=A2, wsb=need):
        return L.fa_decode_paged(q, kp, vp, o, lse, B, H, Hkv, d, scale, P, npg, table, mp, ctx, window, ws, wsb, None)
    assert call(P=24) == INV               # not a power of two
    assert call(P=0) == INV
    assert call(P=8) == UNS                # power of two below 16
    assert call(window=-1) == INV
    assert call(table=None) == INV
    assert call(table=A + 2) == INV        # misaligned table
    assert call(npg=0) == INV              # no pages for B > 0
    assert call(kp=None) == INV
    assert call(ctx=None) == INV
    assert call(wsb=need - 1) == INV
    assert call(H=5) == INV
    assert call(d=96) == UNS
    assert call(mp=1 << 27, P=32) == INV   # capacity past 2^31 positions
    assert call(B=0, table=None, npg=0) == OK  # empty call


def test_fwd_fp8_validation():
    L = fa.lib()
    INV, UNS, OK = fa.binding.FA_ERR_INVALID, fa.binding.FA_ERR_UNSUPPORTED, fa.binding.FA_OK

    def call(q=A, k=A, v=A, qs=A2, ks=A2, vs=A2, o=A2, lse=A2, B=1, H=2, Hkv=1, Lq=4, Lk=4, d=128, scale=0.1,
             causal=1, window=0, seqlens=None):
        return L.fa_fwd_fp8(q, k, v, qs, ks, vs, o, lse, B, H, Hkv, Lq, Lk, d, scale, causal, window, seqlens, None)
    assert call(d=64) == UNS
    assert call(window=-1) == INV
    assert call(window=3, causal=0) == INV
    assert call(qs=None) == INV
    assert call(vs=A2 + 2) == INV   # misaligned descale
    assert call(q=MIS) == INV
    assert call(H=3, Hkv=2) == INV
    assert call(scale=0.0) == INV
    assert call(B=0) == OK


def test_race_check_library_exports_the_same_abi():
    """libfa_serial.so (the fenced race-check build) exports the same entry points."""
    import ctypes
    L = ctypes.CDLL(fa.binding.SERIAL_LIB_PATH)
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_decode_noalloc_validation():
    """The allocation-free decode checks its arguments as fa_decode does, and rejects a call
    whose workspace would exceed the fixed 32 MiB array, all on the host (nothing enqueued)."""
    L = fa.lib()
    INV, UNS, BIG, OK = (fa.binding.FA_ERR_INVALID, fa.binding.FA_ERR_UNSUPPORTED, fa.binding.FA_ERR_TOO_LARGE,
                         fa.binding.FA_OK)

    def call(q=A, k=A, v=A, o=A2, lse=A2, B=2, H=4, Hkv=2, Lmax=100, d=128, scale=0.1, ctx=A):
        return L.fa_decode_noalloc(q, k, v, o, lse, B, H, Hkv, Lmax, d, scale, ctx, None)
    assert call(q=None) == INV
    assert call(ctx=None) == INV
    assert call(H=5) == INV
    assert call(scale=0.0) == INV
    assert call(d=96) == UNS
    # the decode workload (64 requests, 32 heads, 32k keys) fits: 16.25 MiB of partials
    assert L.fa_decode_workspace_bytes(64, 32, 32768, 128) <= 32 << 20
    # 256 requests of 64 heads at 64k keys would need 260 MiB
    assert call(B=256, H=64, Hkv=8, Lmax=65536) == BIG
    assert call(B=0) == OK  # empty: nothing to do, no device touched
