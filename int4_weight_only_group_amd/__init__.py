"""Group-wise affine int4 weight-only linear layer for MI355X (gfx950).

Thin Python binding over the C ABI in include/w4.h (libw4.so).  Every function here only
checks and marshals torch tensors (dtype, device, strides) and calls the library on the
current HIP stream; all computation happens in the HIP kernels.  There is no CPU fallback.

Weight format: packed codes ``qw`` int32 [N][K/8] (uint32 bit patterns, eight 4-bit codes
per word, low nibble first), ``scales`` and ``biases`` float16 [N][K/64]; the weight is
w[n][k] = scales[n][k//64] * q[n][k] + biases[n][k//64].
"""

from __future__ import annotations

import ctypes
import functools

import torch

from ._lib import lib, LIB_PATH  # noqa: F401

__all__ = [
    "W4Error", "w4_pack", "w4_quantize", "w4_gemv", "w4_gemv_sym128", "w4_dequant_f16_t_sym128", "w4_dequant_f16_t", "gemm_f16", "gemm_f16_dequant_next", "gemm_f16_dequant_next_sym128", "logits_argmax_topk",
    "logits_argmax_topk_noalloc", "w4_gemv_topk", "gemv_topk_workspace_bytes",
    "topk_workspace_bytes", "gemm_workspace_bytes", "status_string",
]

W4_OK = 0


class W4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


def status_string(status: int) -> str:
    return lib().w4_strerror(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != W4_OK:
        raise W4Error(fn, status)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.device.index != torch.cuda.current_device():
        # the library launches on the current device; a pointer of another one would fault
        raise ValueError(f"{name} is on {t.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}")


def _rowmajor(t: torch.Tensor, name: str) -> int:
    """Leading dimension of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with contiguous rows (stride(1) == 1)")
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def _contig(t: torch.Tensor, name: str) -> None:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def w4_pack(q: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """uint8 codes [N][K] -> packed int32 words [N][K/8] (eight codes per word)."""
    _dev(q, "q", torch.uint8)
    _contig(q, "q")
    n, k = q.shape
    if out is None:
        out = torch.empty((n, k // 8), dtype=torch.int32, device=q.device)
    _dev(out, "out", torch.int32)
    _contig(out, "out")
    if tuple(out.shape) != (n, k // 8):
        raise ValueError("out must be [N][K/8]")
    _check("w4_pack", lib().w4_pack(q.data_ptr(), out.data_ptr(), n, k, _stream()))
    return out


def w4_quantize(w: torch.Tensor, out: tuple | None = None):
    """float16 weights [N][K] (rows contiguous) -> (qw int32 [N][K/8], scales float16 [N][K/64],
    biases float16 [N][K/64]): the min/max affine fit per group of 64 (see include/w4.h)."""
    _dev(w, "w", torch.float16)
    if w.dim() != 2:
        raise ValueError("w must be [N][K]")
    ldw = _rowmajor(w, "w")
    n, k = w.shape
    if out is None:
        out = (torch.empty((n, k // 8), dtype=torch.int32, device=w.device),
               torch.empty((n, k // 64), dtype=torch.float16, device=w.device),
               torch.empty((n, k // 64), dtype=torch.float16, device=w.device))
    qw, s, b = out
    _dev(qw, "qw", torch.int32)
    _dev(s, "scales", torch.float16)
    _dev(b, "biases", torch.float16)
    for t, nm in ((qw, "qw"), (s, "scales"), (b, "biases")):
        _contig(t, nm)
    if tuple(qw.shape) != (n, k // 8) or tuple(s.shape) != (n, k // 64) or tuple(b.shape) != (n, k // 64):
        raise ValueError("outputs must be [N][K/8], [N][K/64], [N][K/64]")
    _check("w4_quantize", lib().w4_quantize(w.data_ptr(), ldw, qw.data_ptr(), s.data_ptr(), b.data_ptr(),
                                            n, k, _stream()))
    return qw, s, b


def _w4_args(qw, scales, biases):
    _dev(qw, "qw", torch.int32)
    _dev(scales, "scales", torch.float16)
    _dev(biases, "biases", torch.float16)
    for t, nm in ((qw, "qw"), (scales, "scales"), (biases, "biases")):
        _contig(t, nm)
    n, kw = qw.shape
    k = kw * 8
    if tuple(scales.shape) != (n, k // 64) or tuple(biases.shape) != (n, k // 64):
        raise ValueError("scales and biases must be [N][K/64]")
    return n, k


def w4_gemv(qw: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, x: torch.Tensor,
            out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y[m][n] = sum_k w[n][k] x[m][k] for x float16 [M][K] (M <= 16) -> float32 [M][N].

    Shapes that split K across workgroups need a workspace (see gemv_workspace_bytes); one is
    allocated when none (or too small a one) is given.
    """
    n, k = _w4_args(qw, scales, biases)
    _dev(x, "x", torch.float16)
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be [M][K]")
    ldx = _rowmajor(x, "x")
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    if tuple(out.shape) != (m, n):
        raise ValueError("out must be [M][N]")
    ldy = _rowmajor(out, "out")
    need = gemv_workspace_bytes(m, n, k)
    ws_ptr, cap = None, None
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        ws_ptr = workspace.data_ptr()
        cap = ctypes.byref(ctypes.c_size_t(workspace.numel() * workspace.element_size()))
    _check("w4_gemv", lib().w4_gemv(qw.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                                    x.data_ptr(), ldx, out.data_ptr(), ldy, m, n, k, ws_ptr, cap,
                                    _stream()))
    return out


@functools.lru_cache(maxsize=256)
def gemv_workspace_bytes(m: int, n: int, k: int) -> int:
    """Workspace bytes w4_gemv needs for M rows of x and an [N][K] int4 matrix (0 for most shapes)."""
    need = ctypes.c_size_t(0)
    p = ctypes.c_void_p(16)
    _check("w4_gemv", lib().w4_gemv(p, p, p, p, k, p, n, m, n, k, None, ctypes.byref(need), None))
    return int(need.value)


def w4_dequant_f16_t(qw: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """Transposed f16 scratch: float16 [K][N], out[k][n] = RN16(s*q + b)."""
    n, k = _w4_args(qw, scales, biases)
    if out is None:
        out = torch.empty((k, n), dtype=torch.float16, device=qw.device)
    _dev(out, "out", torch.float16)
    if tuple(out.shape) != (k, n):
        raise ValueError("out must be [K][N]")
    ldwt = _rowmajor(out, "out")
    _check("w4_dequant_f16_t", lib().w4_dequant_f16_t(qw.data_ptr(), scales.data_ptr(),
                                                      biases.data_ptr(), out.data_ptr(), ldwt, n,
                                                      k, _stream()))
    return out


def _sym_args(qw, scales):
    _dev(qw, "qw", torch.int32)
    _dev(scales, "scales", torch.float16)
    _contig(qw, "qw")
    _contig(scales, "scales")
    n, kw = qw.shape
    k = kw * 8
    if k % 128 != 0 or tuple(scales.shape) != (n, k // 128):
        raise ValueError("the symmetric group-128 format needs K % 128 == 0 and scales [N][K/128]")
    return n, k


def w4_gemv_sym128(qw: torch.Tensor, scales: torch.Tensor, x: torch.Tensor,
                   out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Symmetric group-128 GEMV: y[m][n] = sum_k scales[n][k//128] (q[n][k] - 8) x[m][k].

    Takes w4_gemv's workspace (gemv_workspace_bytes; allocated when none or too small a one
    is given)."""
    n, k = _sym_args(qw, scales)
    _dev(x, "x", torch.float16)
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be [M][K]")
    ldx = _rowmajor(x, "x")
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    if tuple(out.shape) != (m, n):
        raise ValueError("out must be [M][N]")
    ldy = _rowmajor(out, "out")
    need = gemv_workspace_bytes(m, n, k)
    ws_ptr, cap = None, None
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        ws_ptr = workspace.data_ptr()
        cap = ctypes.byref(ctypes.c_size_t(workspace.numel() * workspace.element_size()))
    _check("w4_gemv_sym128", lib().w4_gemv_sym128(qw.data_ptr(), scales.data_ptr(), x.data_ptr(), ldx,
                                                  out.data_ptr(), ldy, m, n, k, ws_ptr, cap, _stream()))
    return out


def w4_dequant_f16_t_sym128(qw: torch.Tensor, scales: torch.Tensor,
                            out: torch.Tensor | None = None) -> torch.Tensor:
    """Transposed f16 scratch of the symmetric group-128 format: out[k][n] = RN16(s (q - 8))."""
    n, k = _sym_args(qw, scales)
    if out is None:
        out = torch.empty((k, n), dtype=torch.float16, device=qw.device)
    _dev(out, "out", torch.float16)
    if tuple(out.shape) != (k, n):
        raise ValueError("out must be [K][N]")
    ldwt = _rowmajor(out, "out")
    _check("w4_dequant_f16_t_sym128", lib().w4_dequant_f16_t_sym128(qw.data_ptr(), scales.data_ptr(),
                                                                    out.data_ptr(), ldwt, n, k, _stream()))
    return out


def gemm_f16(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None,
             workspace: torch.Tensor | None = None) -> torch.Tensor:
    """C = A @ B: float16 A [M][K], float16 B [K][N] (rows contiguous) -> float32 [M][N].

    Shapes that split K need a workspace (see gemm_workspace_bytes); one is allocated when
    none (or too small a one) is given.
    """
    _dev(a, "a", torch.float16)
    _dev(b, "b", torch.float16)
    lda, ldb = _rowmajor(a, "a"), _rowmajor(b, "b")
    m, k = a.shape
    k2, n = b.shape
    if k != k2:
        raise ValueError("inner dimensions differ")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=a.device)
    _dev(out, "out", torch.float32)
    if tuple(out.shape) != (m, n):
        raise ValueError("out must be [M][N]")
    ldc = _rowmajor(out, "out")
    need = ctypes.c_size_t(0)
    _check("gemm_f16", lib().gemm_f16(a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc,
                                      m, n, k, None, ctypes.byref(need), None))
    ws_ptr, cap = None, None
    if need.value:
        if workspace is None or workspace.numel() * workspace.element_size() < need.value:
            workspace = torch.empty(need.value, dtype=torch.uint8, device=a.device)
        ws_ptr = workspace.data_ptr()
        cap = ctypes.byref(ctypes.c_size_t(workspace.numel() * workspace.element_size()))
    _check("gemm_f16", lib().gemm_f16(a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc,
                                      m, n, k, ws_ptr, cap, _stream()))
    return out


def gemm_f16_dequant_next(a: torch.Tensor, b: torch.Tensor, qw: torch.Tensor, scales: torch.Tensor,
                          biases: torch.Tensor, out: torch.Tensor | None = None,
                          wt: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """gemm_f16(a, b) and w4_dequant_f16_t(qw, scales, biases) in one call (the dequant rides
    in the CUs the GEMM's last round leaves idle when it fits there): returns (C, wt)."""
    nq, kq = _w4_args(qw, scales, biases)
    return _gemm_dequant_next("gemm_f16_dequant_next", a, b, qw, scales, biases, nq, kq, out, wt, workspace)


def gemm_f16_dequant_next_sym128(a: torch.Tensor, b: torch.Tensor, qw: torch.Tensor, scales: torch.Tensor,
                                 out: torch.Tensor | None = None, wt: torch.Tensor | None = None,
                                 workspace: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """gemm_f16(a, b) and w4_dequant_f16_t_sym128(qw, scales) in one call: returns (C, wt)."""
    nq, kq = _sym_args(qw, scales)
    return _gemm_dequant_next("gemm_f16_dequant_next_sym128", a, b, qw, scales, None, nq, kq, out, wt, workspace)


def _gemm_dequant_next(fn, a, b, qw, scales, biases, nq, kq, out, wt, workspace):
    _dev(a, "a", torch.float16)
    _dev(b, "b", torch.float16)
    lda, ldb = _rowmajor(a, "a"), _rowmajor(b, "b")
    m, k = a.shape
    k2, n = b.shape
    if k != k2:
        raise ValueError("inner dimensions differ")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=a.device)
    _dev(out, "out", torch.float32)
    if tuple(out.shape) != (m, n):
        raise ValueError("out must be [M][N]")
    if wt is None:
        wt = torch.empty((kq, nq), dtype=torch.float16, device=qw.device)
    _dev(wt, "wt", torch.float16)
    if tuple(wt.shape) != (kq, nq):
        raise ValueError("wt must be [Kq][Nq]")
    ldc, ldwt = _rowmajor(out, "out"), _rowmajor(wt, "wt")
    w4q = [qw.data_ptr(), scales.data_ptr()] + ([biases.data_ptr()] if biases is not None else [])

    def call(ws_ptr, cap, stream):
        return getattr(lib(), fn)(a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc, m, n, k, ws_ptr, cap,
                                  *w4q, wt.data_ptr(), ldwt, nq, kq, stream)

    need = ctypes.c_size_t(0)
    _check(fn, call(None, ctypes.byref(need), None))
    ws_ptr, cap = None, None
    if need.value:
        if workspace is None or workspace.numel() * workspace.element_size() < need.value:
            workspace = torch.empty(need.value, dtype=torch.uint8, device=a.device)
        ws_ptr = workspace.data_ptr()
        cap = ctypes.byref(ctypes.c_size_t(workspace.numel() * workspace.element_size()))
    _check(fn, call(ws_ptr, cap, _stream()))
    return out, wt


def gemm_workspace_bytes(a: torch.Tensor, b: torch.Tensor) -> int:
    """Workspace bytes gemm_f16 needs for these operands (0 for most shapes)."""
    need = ctypes.c_size_t(0)
    _check("gemm_f16", lib().gemm_f16(a.data_ptr(), _rowmajor(a, "a"), b.data_ptr(), _rowmajor(b, "b"),
                                      ctypes.c_void_p(16), b.shape[1], a.shape[0], b.shape[1], a.shape[1],
                                      None, ctypes.byref(need), None))
    return int(need.value)


def topk_workspace_bytes(m: int, v: int, k: int) -> int:
    n = ctypes.c_size_t(0)
    _check("logits_argmax_topk", lib().logits_argmax_topk(
        ctypes.c_void_p(16), v, m, v, k, ctypes.c_void_p(16), ctypes.c_void_p(16), None,
        ctypes.byref(n), None))
    return int(n.value)


def logits_argmax_topk(logits: torch.Tensor, k: int, idx: torch.Tensor | None = None,
                       val: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Per row the k largest logits (value desc, ties to lower index): (int32 idx, float32 val)."""
    _dev(logits, "logits", torch.float32)
    ldl = _rowmajor(logits, "logits")
    m, v = logits.shape
    if idx is None:
        idx = torch.empty((m, k), dtype=torch.int32, device=logits.device)
    if val is None:
        val = torch.empty((m, k), dtype=torch.float32, device=logits.device)
    _dev(idx, "idx", torch.int32)
    _dev(val, "val", torch.float32)
    _contig(idx, "idx")
    _contig(val, "val")
    if tuple(idx.shape) != (m, k) or tuple(val.shape) != (m, k):
        raise ValueError("idx and val must be [M][k]")
    need = ctypes.c_size_t(0)
    _check("logits_argmax_topk", lib().logits_argmax_topk(
        logits.data_ptr(), ldl, m, v, k, idx.data_ptr(), val.data_ptr(), None,
        ctypes.byref(need), None))
    if need.value and (workspace is None or workspace.numel() * workspace.element_size() < need.value):
        workspace = torch.empty(need.value, dtype=torch.uint8, device=logits.device)
    ws_ptr = workspace.data_ptr() if need.value else None
    cap = ctypes.c_size_t(workspace.numel() * workspace.element_size() if need.value else 0)
    _check("logits_argmax_topk", lib().logits_argmax_topk(
        logits.data_ptr(), ldl, m, v, k, idx.data_ptr(), val.data_ptr(), ws_ptr,
        ctypes.byref(cap) if need.value else None, _stream()))
    return idx, val


def logits_argmax_topk_noalloc(logits: torch.Tensor, k: int, idx: torch.Tensor | None = None,
                               val: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """logits_argmax_topk without a workspace: the library's own per-device scratch array holds
    the candidates (so the call allocates nothing when idx and val are given).  Calls that
    overlap on one device share that array."""
    _dev(logits, "logits", torch.float32)
    ldl = _rowmajor(logits, "logits")
    m, v = logits.shape
    if idx is None:
        idx = torch.empty((m, k), dtype=torch.int32, device=logits.device)
    if val is None:
        val = torch.empty((m, k), dtype=torch.float32, device=logits.device)
    _dev(idx, "idx", torch.int32)
    _dev(val, "val", torch.float32)
    _contig(idx, "idx")
    _contig(val, "val")
    if tuple(idx.shape) != (m, k) or tuple(val.shape) != (m, k):
        raise ValueError("idx and val must be [M][k]")
    _check("logits_argmax_topk_noalloc", lib().logits_argmax_topk_noalloc(
        logits.data_ptr(), ldl, m, v, k, idx.data_ptr(), val.data_ptr(), _stream()))
    return idx, val


def gemv_topk_workspace_bytes(v: int, k_dim: int, k: int) -> int:
    """Workspace bytes w4_gemv_topk needs for a [v][k_dim] head and top-k."""
    n = ctypes.c_size_t(0)
    p = ctypes.c_void_p(16)
    _check("w4_gemv_topk", lib().w4_gemv_topk(p, p, p, p, v, k_dim, k, p, p, p, None, ctypes.byref(n), None))
    return int(n.value)


def w4_gemv_topk(qw: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, x: torch.Tensor, k: int,
                 logits: torch.Tensor | None = None, idx: torch.Tensor | None = None,
                 val: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """The int4 LM head with top-k on the device, one call: x float16 [K] (or [1][K]) -> (logits float32 [V],
    idx int32 [k], val float32 [k]), the k largest logits, value descending, ties to the lower
    index.  One is allocated for each of the outputs and the workspace not given."""
    v, kdim = _w4_args(qw, scales, biases)
    _dev(x, "x", torch.float16)
    _contig(x, "x")
    if x.numel() != kdim or (x.dim() == 2 and x.shape[0] != 1):
        raise ValueError("x must be [K] or [1][K]")
    outs = []
    for t, name, shape, dt in ((logits, "logits", (v,), torch.float32), (idx, "idx", (k,), torch.int32),
                               (val, "val", (k,), torch.float32)):
        if t is None:
            t = torch.empty(shape, dtype=dt, device=x.device)
        _dev(t, name, dt)
        _contig(t, name)
        if t.numel() != shape[0]:
            raise ValueError(f"{name} must hold {shape[0]} elements")
        outs.append(t)
    logits, idx, val = outs
    need = gemv_topk_workspace_bytes(v, kdim, k)
    ws_ptr, cap = None, None  # no workspace at all when none is needed (a null one would be a query)
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        ws_ptr = workspace.data_ptr()
        cap = ctypes.byref(ctypes.c_size_t(workspace.numel() * workspace.element_size()))
    _check("w4_gemv_topk", lib().w4_gemv_topk(qw.data_ptr(), scales.data_ptr(), biases.data_ptr(), x.data_ptr(),
                                              v, kdim, k, logits.data_ptr(), idx.data_ptr(), val.data_ptr(),
                                              ws_ptr, cap, _stream()))
    return logits, idx, val
