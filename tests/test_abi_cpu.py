"""The C-ABI library loads, exports what include/w4.h declares, and rejects bad arguments
on the host before touching a device (CPU only: no kernel is launched here)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4.h")

W4_OK, W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN, W4_ERR_WORKSPACE, W4_ERR_DEVICE = 0, -1, -2, -3, -4, -5

P = 4096  # a fake, 16-byte aligned "device" address: never dereferenced by these calls


def _lib():
    from int4_weight_only_group_amd._lib import lib
    return lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def test_header_declares_the_five_entry_points():
    names = _declared()
    for n in ("w4_pack", "w4_gemv", "w4_dequant_f16_t", "gemm_f16", "logits_argmax_topk", "w4_strerror"):
        assert n in names, names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for n in _declared():
        assert hasattr(lib, n), n
    out = os.popen(f"nm -D --defined-only {lib._name}").read()
    for n in _declared():
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def test_strerror():
    lib = _lib()
    for s in range(-8, 1):
        assert lib.w4_strerror(s)
    assert lib.w4_strerror(0) == b"ok"


def test_pack_argument_errors():
    lib = _lib()
    assert lib.w4_pack(None, P, 4, 64, None) == W4_ERR_NULL
    assert lib.w4_pack(P, None, 4, 64, None) == W4_ERR_NULL
    assert lib.w4_pack(P, P, 0, 64, None) == W4_ERR_SHAPE
    assert lib.w4_pack(P, P, 4, 96, None) == W4_ERR_SHAPE
    assert lib.w4_pack(P, P, 4, 0, None) == W4_ERR_SHAPE
    assert lib.w4_pack(P + 8, P, 4, 64, None) == W4_ERR_ALIGN


def test_gemv_argument_errors():
    lib = _lib()
    g = lambda **kw: lib.w4_gemv(kw.get("qw", P), P, P, kw.get("x", P), kw.get("ldx", 128), P,
                                 kw.get("ldy", 8), kw.get("M", 1), kw.get("N", 8), kw.get("K", 128),
                                 None, None, None)
    assert g(qw=None) == W4_ERR_NULL
    assert g(M=0) == W4_ERR_SHAPE
    assert g(M=17) == W4_ERR_SHAPE
    assert g(K=100, ldx=104) == W4_ERR_SHAPE
    assert g(ldx=64) == W4_ERR_SHAPE
    assert g(ldy=4) == W4_ERR_SHAPE
    assert g(x=P + 2) == W4_ERR_ALIGN
    assert g(ldx=132) == W4_ERR_ALIGN
    n = ctypes.c_size_t(123)
    assert lib.w4_gemv(P, P, P, P, 128, P, 8, 1, 8, 128, None, ctypes.byref(n), None) == W4_OK
    assert n.value == 0


def test_quantize_argument_errors():
    lib = _lib()
    q = lambda **kw: lib.w4_quantize(kw.get("w", P), kw.get("ldw", 128), kw.get("qw", P), kw.get("s", P),
                                     kw.get("b", P), kw.get("N", 4), kw.get("K", 128), None)
    assert q(w=None) == W4_ERR_NULL
    assert q(b=None) == W4_ERR_NULL
    assert q(N=0) == W4_ERR_SHAPE
    assert q(K=96, ldw=96) == W4_ERR_SHAPE
    assert q(ldw=64) == W4_ERR_SHAPE
    assert q(w=P + 8) == W4_ERR_ALIGN
    assert q(ldw=132) == W4_ERR_ALIGN
    assert q(qw=P + 4) == W4_ERR_ALIGN
    assert q(s=P + 1) == W4_ERR_ALIGN


def test_sym128_argument_errors():
    lib = _lib()
    g = lambda **kw: lib.w4_gemv_sym128(kw.get("qw", P), kw.get("s", P), P, kw.get("ldx", 256), P, 8,
                                        kw.get("M", 1), 8, kw.get("K", 256), None, None, None)
    assert g(qw=None) == W4_ERR_NULL
    assert g(K=192, ldx=192) == W4_ERR_SHAPE     # K % 128 != 0
    assert g(M=17) == W4_ERR_SHAPE
    assert g(s=P + 2) == W4_ERR_ALIGN
    d = lambda **kw: lib.w4_dequant_f16_t_sym128(P, P, kw.get("wt", P), kw.get("ldwt", 8), 8,
                                                 kw.get("K", 128), None)
    assert d(wt=None) == W4_ERR_NULL
    assert d(K=64) == W4_ERR_SHAPE
    assert d(ldwt=4) == W4_ERR_SHAPE
    assert d(wt=P + 1) == W4_ERR_ALIGN


def test_dequant_and_gemm_argument_errors():
    lib = _lib()
    assert lib.w4_dequant_f16_t(P, P, P, None, 8, 8, 64, None) == W4_ERR_NULL
    assert lib.w4_dequant_f16_t(P, P, P, P, 4, 8, 64, None) == W4_ERR_SHAPE
    assert lib.w4_dequant_f16_t(P, P, P, P + 1, 8, 8, 64, None) == W4_ERR_ALIGN
    assert lib.gemm_f16(None, 8, P, 8, P, 8, 2, 8, 8, None, None, None) == W4_ERR_NULL
    assert lib.gemm_f16(P, 4, P, 8, P, 8, 2, 8, 8, None, None, None) == W4_ERR_SHAPE
    assert lib.gemm_f16(P, 8, P, 8, P, 8, 0, 8, 8, None, None, None) == W4_ERR_SHAPE
    assert lib.gemm_f16(P + 1, 8, P, 8, P, 8, 2, 8, 8, None, None, None) == W4_ERR_ALIGN
    assert lib.gemm_f16(P, 8, P, 8, P + 2, 8, 2, 8, 8, None, None, None) == W4_ERR_ALIGN


def test_topk_argument_errors_and_workspace_query():
    lib = _lib()
    t = lambda **kw: lib.logits_argmax_topk(kw.get("lg", P), kw.get("ldl", kw.get("V", 100)), kw.get("M", 1),
                                            kw.get("V", 100), kw.get("k", 5), P, P, kw.get("ws", None),
                                            kw.get("wsb", None), None)
    assert t(lg=None) == W4_ERR_NULL
    assert t(k=0) == W4_ERR_SHAPE
    assert t(k=257, V=1000) == W4_ERR_SHAPE
    assert t(k=6, V=5) == W4_ERR_SHAPE
    assert t(ldl=50) == W4_ERR_SHAPE
    assert t(lg=P + 2) == W4_ERR_ALIGN
    n = ctypes.c_size_t(0)
    assert t(V=151936, k=40, M=1, wsb=ctypes.byref(n)) == W4_OK
    assert n.value == 2374 * 8  # one row: one 8-byte key per group of 64 logits
    small = ctypes.c_size_t(n.value - 8)
    assert t(V=151936, k=40, ws=P, wsb=ctypes.byref(small)) == W4_ERR_WORKSPACE
    assert t(V=151936, k=40, ws=None, wsb=None) == W4_ERR_WORKSPACE
    n2 = ctypes.c_size_t(7)
    assert t(V=2, k=1, M=16, wsb=ctypes.byref(n2)) == W4_OK and n2.value == 0


def test_gemv_topk_argument_errors_and_workspace_query():
    lib = _lib()
    g = lambda **kw: lib.w4_gemv_topk(kw.get("qw", P), P, P, kw.get("x", P), kw.get("V", 151936), kw.get("K", 2048),
                                      kw.get("k", 40), kw.get("lg", P), P, P, kw.get("ws", None), kw.get("wsb", None),
                                      None)
    assert g(qw=None) == W4_ERR_NULL
    assert g(lg=None) == W4_ERR_NULL
    assert g(k=0) == W4_ERR_SHAPE
    assert g(k=65) == W4_ERR_SHAPE
    assert g(V=30, k=40) == W4_ERR_SHAPE
    assert g(K=96) == W4_ERR_SHAPE
    assert g(K=4160) == W4_ERR_SHAPE
    assert g(V=524289, k=64) == W4_ERR_SHAPE     # beyond the documented 524288 rows
    assert g(V=524288, k=64, wsb=ctypes.byref(ctypes.c_size_t(0))) == W4_OK
    assert g(x=P + 8) == W4_ERR_ALIGN
    assert g(lg=P + 2) == W4_ERR_ALIGN
    n = ctypes.c_size_t(0)
    assert g(wsb=ctypes.byref(n)) == W4_OK
    assert n.value == 2374 * 8  # one key per 64 logits
    small = ctypes.c_size_t(n.value - 8)
    assert g(ws=P, wsb=ctypes.byref(small)) == W4_ERR_WORKSPACE
    n2 = ctypes.c_size_t(0)
    assert g(V=100, K=64, k=3, wsb=ctypes.byref(n2)) == W4_OK and n2.value == 0  # one selection pass
    n3 = ctypes.c_size_t(0)
    assert g(V=262144, K=3840, k=64, wsb=ctypes.byref(n3)) == W4_OK and n3.value == 4096 * 8


@pytest.mark.skipif(_has_gpu(), reason="checks the no-device error path")
def test_valid_call_without_device_reports_device_error():
    lib = _lib()
    assert lib.w4_pack(P, P, 4, 64, None) == W4_ERR_DEVICE
    assert lib.gemm_f16(P, 8, P, 8, P, 8, 2, 8, 8, None, None, None) == W4_ERR_DEVICE


def test_binding_names_match_abi():
    import int4_weight_only_group_amd as w4
    for n in ("w4_pack", "w4_gemv", "w4_dequant_f16_t", "gemm_f16", "logits_argmax_topk"):
        assert callable(getattr(w4, n))
    assert w4.topk_workspace_bytes(8, 262144, 64) == 8 * 64 * 64 * 8


def test_gemm_workspace_query():
    # The workspace each GEMM plan asks for: none when the output tiles fill the CUs at least
    # half way; ksplit * M * N * 4 bytes when K is split
    lib = _lib()
    A = 1 << 20

    def need(m, n, k):
        nb = ctypes.c_size_t(0)
        assert lib.gemm_f16(A, k, A, n, A, n, m, n, k, None, ctypes.byref(nb), None) == W4_OK
        return nb.value
    assert need(4096, 4096, 4096) == 0                      # 256 tiles: one full round
    assert need(1570, 22016, 2048) == 0                     # 430 tiles of 320 x 256
    assert need(1570, 2048, 11008) == 6 * 1570 * 2048 * 4   # 40 tiles, K split 6 ways
    assert need(600, 2048, 4096) == 8 * 600 * 2048 * 4      # 24 tiles, 8 slices of 8 K-tiles of 64
    assert need(600, 25608, 64) == 0                        # 202 tiles
    assert need(8, 4096, 256) == 0                          # small-M path


def test_gemv_workspace_query_and_errors():
    # the matrix-core GEMV splits K two ways across workgroups for rows of K >= 6144 on at most
    # 128 workgroups; the partial sums need 2 * M * N * 4 bytes, every other shape none
    lib = _lib()
    A = 1 << 20

    def need(m, n, k):
        nb = ctypes.c_size_t(7)
        assert lib.w4_gemv(A, A, A, A, k, A, n, m, n, k, None, ctypes.byref(nb), None) == W4_OK
        return nb.value
    assert need(16, 2048, 6144) == 2 * 16 * 2048 * 4      # 128 row blocks
    assert need(8, 2048, 11008) == 2 * 8 * 2048 * 4
    assert need(3, 2048, 20480) == 2 * 3 * 2048 * 4      # M = 3 past 16384 elements
    assert need(5, 2064, 8192) == 0                      # 129 row blocks
    assert need(8, 3840, 15360) == 4 * 8 * 3840 * 4      # 28 MB of codes at M = 8: 4 staged K-ranges
    assert need(8, 30720, 3840) == 0                     # 56 MB, 960 workgroups: one K-range
    assert need(7, 1000, 51200) == 13 * 7 * 1000 * 4     # 13 staged K-ranges
    assert need(16, 3840, 15360) == 0                    # M = 16: 240 row blocks, no split
    assert need(16, 2048, 4096) == 0                     # K below 6144
    assert need(16, 12288, 6144) == 0                    # 768 row blocks, four per wave: 192
    assert need(1, 2048, 11008) == 0                     # M = 1: row slices
    assert need(4, 2048, 11008) == 0                     # M = 4 within 16384: row slices
    n = ctypes.c_size_t(need(16, 2048, 6144) - 16)
    assert lib.w4_gemv(A, A, A, A, 6144, A, 2048, 16, 2048, 6144, A, ctypes.byref(n), None) == W4_ERR_WORKSPACE
    assert lib.w4_gemv(A, A, A, A, 6144, A, 2048, 16, 2048, 6144, None, None, None) == W4_ERR_WORKSPACE
    big = ctypes.c_size_t(1 << 20)
    assert lib.w4_gemv(A, A, A, A, 6144, A, 2048, 16, 2048, 6144, A + 8, ctypes.byref(big), None) == W4_ERR_ALIGN
    s = ctypes.c_size_t(0)
    assert lib.w4_gemv_sym128(A, A, A, 6144, A, 2048, 16, 2048, 6144, None, ctypes.byref(s), None) == W4_OK
    assert s.value == need(16, 2048, 6144)                # the symmetric GEMV splits the same way


def test_gemm_dequant_next_argument_errors_and_overlap():
    # gemm_f16_dequant_next: gemm_f16's and w4_dequant_f16_t's checks, the GEMM's workspace
    # query, and overlaps between one operation's outputs and the other's data (host-side)
    lib = _lib()
    W4_ERR_OVERLAP = -8
    GB = 1 << 30
    base = dict(A=1 * GB, lda=64, B=2 * GB, ldb=64, C=3 * GB, ldc=64, M=16, N=64, K=64, ws=None, wsb=None,
                qw=4 * GB, s=5 * GB, b=6 * GB, wt=7 * GB, ldwt=128, Nq=128, Kq=256)

    def call(**kw):
        a = dict(base, **kw)
        return lib.gemm_f16_dequant_next(a["A"], a["lda"], a["B"], a["ldb"], a["C"], a["ldc"], a["M"], a["N"],
                                         a["K"], a["ws"], a["wsb"], a["qw"], a["s"], a["b"], a["wt"], a["ldwt"],
                                         a["Nq"], a["Kq"], None)
    assert call(A=None) == W4_ERR_NULL
    assert call(wt=None) == W4_ERR_NULL
    assert call(b=None) == W4_ERR_NULL
    assert call(M=0) == W4_ERR_SHAPE
    assert call(lda=32) == W4_ERR_SHAPE
    assert call(Kq=96) == W4_ERR_SHAPE
    assert call(ldwt=100) == W4_ERR_SHAPE
    assert call(C=3 * GB + 2) == W4_ERR_ALIGN
    assert call(qw=4 * GB + 4) == W4_ERR_ALIGN
    assert call(wt=7 * GB + 1) == W4_ERR_ALIGN
    # the workspace query answers with gemm_f16's size, before any overlap or device check
    for m, n, k in ((1570, 2048, 11008), (600, 2048, 4096), (1570, 22016, 2048)):
        got, ref = ctypes.c_size_t(0), ctypes.c_size_t(0)
        assert call(M=m, N=n, K=k, lda=k, ldb=n, ldc=n, wsb=ctypes.byref(got)) == W4_OK
        assert lib.gemm_f16(GB, k, GB, n, GB, n, m, n, k, None, ctypes.byref(ref), None) == W4_OK
        assert got.value == ref.value
    small = ctypes.c_size_t(16)
    assert call(M=600, N=2048, K=4096, lda=4096, ldb=2048, ldc=2048, ws=8 * GB,
                wsb=ctypes.byref(small)) == W4_ERR_WORKSPACE
    # wt [256][128] f16 = 64 KiB; C [16][64] f32 = 4 KiB; qw 16 KiB; scales/biases 1 KiB each
    assert call(wt=1 * GB + 16) == W4_ERR_OVERLAP         # wt inside A
    assert call(wt=2 * GB - 65536 + 16) == W4_ERR_OVERLAP  # wt's last row reaches into B
    assert call(wt=3 * GB) == W4_ERR_OVERLAP               # wt on C
    assert call(wt=4 * GB + 16 * 1024 - 16) == W4_ERR_OVERLAP  # wt's first bytes on qw's last
    assert call(C=5 * GB + 1024 - 16) == W4_ERR_OVERLAP    # C's first bytes on the scales' last
    assert call(C=6 * GB - 4096 + 16) == W4_ERR_OVERLAP    # C's last row reaches into the biases
    need = 8 * 600 * 2048 * 4
    big = ctypes.c_size_t(need)
    split = dict(M=600, N=2048, K=4096, lda=4096, ldb=2048, ldc=2048, wsb=ctypes.byref(big))
    assert call(ws=7 * GB - need + 16, **split) == W4_ERR_OVERLAP  # workspace end on wt
    assert call(ws=4 * GB + 4096, **split) == W4_ERR_OVERLAP       # workspace over qw
    # touching ranges do not overlap: wt right after qw's 16 KiB, C right before the scales
    assert call(wt=4 * GB + 16 * 1024) in (W4_ERR_DEVICE, W4_OK)
    assert call(C=5 * GB - 4096) in (W4_ERR_DEVICE, W4_OK)
    if not _has_gpu():
        assert call() == W4_ERR_DEVICE


def test_gemm_dequant_next_sym128_argument_errors_and_overlap():
    # the symmetric group-128 twin: Kq % 128 == 0, scales [Nq][Kq/128], no biases; the same
    # workspace query and overlap rule
    lib = _lib()
    W4_ERR_OVERLAP = -8
    GB = 1 << 30
    base = dict(A=1 * GB, lda=64, B=2 * GB, ldb=64, C=3 * GB, ldc=64, M=16, N=64, K=64, ws=None, wsb=None,
                qw=4 * GB, s=5 * GB, wt=7 * GB, ldwt=128, Nq=128, Kq=256)

    def call(**kw):
        a = dict(base, **kw)
        return lib.gemm_f16_dequant_next_sym128(a["A"], a["lda"], a["B"], a["ldb"], a["C"], a["ldc"], a["M"],
                                                a["N"], a["K"], a["ws"], a["wsb"], a["qw"], a["s"], a["wt"],
                                                a["ldwt"], a["Nq"], a["Kq"], None)
    assert call(s=None) == W4_ERR_NULL
    assert call(qw=None) == W4_ERR_NULL
    assert call(Kq=192) == W4_ERR_SHAPE   # a multiple of 64 but not of 128
    assert call(s=5 * GB + 2) == W4_ERR_ALIGN
    got, ref = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert call(M=1570, N=2048, K=11008, lda=11008, ldb=2048, ldc=2048, wsb=ctypes.byref(got)) == W4_OK
    assert lib.gemm_f16(GB, 11008, GB, 2048, GB, 2048, 1570, 2048, 11008, None, ctypes.byref(ref), None) == W4_OK
    assert got.value == ref.value
    # scales [128][2] f16 = 512 bytes: C's first bytes on their last is an overlap, right after is not
    assert call(C=5 * GB + 512 - 16) == W4_ERR_OVERLAP
    assert call(C=5 * GB + 512) in (W4_ERR_DEVICE, W4_OK)
    assert call(wt=5 * GB - 65536 + 16) == W4_ERR_OVERLAP  # wt's last row on the scales
    if not _has_gpu():
        assert call() == W4_ERR_DEVICE
