"""Plain CPU reference for the int4 group-wise affine linear layer (test infrastructure).

Nothing here is tuned.  Integers stay integers, floating point is fp64, and
every f16 rounding is a single round-to-nearest-even of an exact value.  The
functions follow the order in which the pages describe the path:

  pack           -- weights are "quantized to int4 at load"
                    ("The inference engine -- Mojo 1.0 on Metal", "Where it fits")
                    into MLX's affine 4-bit layout ("Appendix: the remaining gap,
                    itemized"), group size 64 ("Engineering investigation ...",
                    "Selective quantization ...").
  dequant        -- w = s*q + b per group of 64 along K (the affine format above);
                    also the engine's own symmetric group-128 format, read as
                    w = s*(q - 8) ("The inference engine -- Mojo 1.0 on Metal",
                    "Against MLX, today"; "Appendix: the remaining gap, itemized").
  dequant_f16_t  -- "dequantizes each weight once per prefill into a transposed
                    half-precision scratch" ("Crossing Mojo 1.0").
  gemv_ref       -- the decode GEMV y = x W^T ("Crossing Mojo 1.0", the multi-row
                    GEMV); fp64 sum over exact products.
  gemm_ref       -- the prefill GEMM C = A * Wt on the f16 scratch ("Crossing Mojo
                    1.0") and the f16 LM head ("What's inside the engine today").
  topk_ref       -- greedy / top-k token selection on the logits ("Crossing Mojo
                    1.0"; "What's inside the engine today": bit-exact against a host
                    reference; "engine-mlx", "Tech details": in-graph greedy argmax).
  quantize       -- the load-time step that turns float weights into the int4
                    affine format ("The inference engine -- Mojo 1.0 on Metal",
                    "Where it fits": weights quantized to int4 at load;
                    "Engineering investigation ...", "Selective quantization ...":
                    affine, group size 64).

Readings taken where the pages are silent (each is listed in the design notes):
  * layout: q codes row-major [N][K]; packed words [N][K/8], K contiguous; s and b
    [N][K/64]; element 8j+i of a row sits in bits 4i..4i+3 of word j.
  * rounding of the f16 dequant: one correctly rounded RN-even step from the
    exact value s*q + b, subnormals kept (s*q + b is exact in fp64: both terms are
    multiples of 2**-24 below 2**16, so the sum needs at most 45 bits).
  * "transposed" scratch: [K][N] with N contiguous.
  * the GEMV reference uses the exact (unrounded) weights, since the GEMV never
    materialises f16 weights; the GEMM reference uses the f16 scratch values, which
    are its actual operands.
  * top-k order: value descending, ties to the lower index, -0.0 equal to +0.0;
    logits must be finite.
  * quantizer (the pages give no formula): per group of 64 the plain min/max affine
    fit -- b = min, s = RN16((max - min) / 15), q = clamp(rint_even((w - b) / s), 0, 15),
    q = 0 where s rounds to 0; a zero min or max counts as +0.  Every step that decides
    a code is f32 arithmetic (correctly rounded), the precision the GPU kernel decides
    in, so codes compare bit for bit.  This is the one place the oracle computes in f32.
  * tolerance: |y - y_ref| <= 2e-3 * sum_k |w_k x_k| per output; selection is
    exact on the same f32 logits; against fp64 logits an index must match wherever
    both neighbouring gaps exceed 1e-2, else lie in the near-tie class.
"""

from __future__ import annotations

import struct

import numpy as np

GROUP = 64          # elements of K per (scale, bias) pair
CODES_PER_WORD = 8  # 4-bit codes per uint32 word


# --------------------------------------------------------------------------- pack


def pack(q: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes q (uint8 [N][K], values 0..15) into uint32 [N][K/8].

    Word j of row n holds q[n][8j+i] in bits 4i..4i+3 (low nibble first).  Codes
    above 15 are a precondition violation; only their low four bits are kept.
    """
    q = np.asarray(q)
    assert q.ndim == 2 and q.shape[1] % CODES_PER_WORD == 0, q.shape
    n, k = q.shape
    nib = (q.astype(np.uint32) & np.uint32(0xF)).reshape(n, k // CODES_PER_WORD, CODES_PER_WORD)
    words = np.zeros((n, k // CODES_PER_WORD), dtype=np.uint32)
    for i in range(CODES_PER_WORD):
        words |= nib[:, :, i] << np.uint32(4 * i)
    return words


def pack_loop(q) -> list:
    """Same as :func:`pack` with Python ints, one code at a time (small inputs)."""
    out = []
    for row in q:
        row = [int(v) for v in row]
        assert len(row) % CODES_PER_WORD == 0
        words = []
        for j in range(len(row) // CODES_PER_WORD):
            w = 0
            for i in range(CODES_PER_WORD):
                w += (row[CODES_PER_WORD * j + i] & 0xF) * (16 ** i)
            words.append(w)
        out.append(words)
    return out


def unpack(qw: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack`: uint32 [N][K/8] -> uint8 codes [N][K]."""
    qw = np.asarray(qw, dtype=np.uint32)
    assert qw.ndim == 2
    n, kw = qw.shape
    q = np.empty((n, kw, CODES_PER_WORD), dtype=np.uint8)
    for i in range(CODES_PER_WORD):
        q[:, :, i] = ((qw >> np.uint32(4 * i)) & np.uint32(0xF)).astype(np.uint8)
    return q.reshape(n, kw * CODES_PER_WORD)


def unpack_loop(qw) -> list:
    """Same as :func:`unpack` with Python ints (small inputs)."""
    out = []
    for row in qw:
        codes = []
        for w in row:
            w = int(w)
            for _ in range(CODES_PER_WORD):
                codes.append(w % 16)
                w //= 16
        out.append(codes)
    return out


# ----------------------------------------------------------------- f16 rounding


def f16_bits(v) -> np.ndarray:
    """Round fp64 values to f16 (one RN-even rounding, subnormals kept) -> uint16 bits.

    NumPy converts float64 to float16 directly from the double's bits, so this is a
    single rounding of the fp64 value (pinned against ``struct``'s 'e' encoder and
    against hand-derived cases in the tests).
    """
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def f16_bits_struct(v) -> np.ndarray:
    """Independent encoder: Python's struct 'e' format, one value at a time."""
    flat = np.asarray(v, dtype=np.float64).ravel()
    out = np.empty(flat.shape, dtype=np.uint16)
    for i, x in enumerate(flat):
        out[i] = struct.unpack("<H", struct.pack("<e", float(x)))[0]
    return out.reshape(np.shape(v))


def f16_value(bits) -> np.ndarray:
    """uint16 f16 bit patterns -> exact fp64 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:          # raw f16 bit patterns
        return f16_value(a)
    assert a.dtype == np.float16, a.dtype
    return a.astype(np.float64)       # exact


# ----------------------------------------------------------------------- dequant


def dequant_exact(qw: np.ndarray, s, b, group: int = GROUP) -> np.ndarray:
    """Exact weights in fp64 ([N][K]).

    Affine format (b given): w[n][k] = s[n][k//group] * q[n][k] + b[n][k//group].
    Symmetric format (b is None): the engine's own int4 ("The inference engine -- Mojo 1.0 on
    Metal": group-128 in "Against MLX, today" and "What's inside the engine today",
    symmetric in "Appendix: the remaining gap, itemized"), read as w = s * (q - 8) with
    group = 128 (zero point 8, no bias), an exact zero taken as +0.  s and b are f16 ([N][K/group], np.float16 values or uint16 bits).
    """
    q = unpack(qw).astype(np.float64)
    n, k = q.shape
    assert k % group == 0
    s64 = _f64(s)
    assert s64.shape == (n, k // group)
    grp = np.arange(k) // group
    if b is None:
        return s64[:, grp] * (q - 8.0) + 0.0      # + 0.0 turns -0 into +0
    b64 = _f64(b)
    assert b64.shape == (n, k // group)
    return s64[:, grp] * q + b64[:, grp]


def dequant_f16_t(qw: np.ndarray, s, b, group: int = GROUP) -> np.ndarray:
    """The transposed f16 prefill scratch: uint16 bits [K][N] of RN16(w), w as in
    dequant_exact (one rounding of the exact value)."""
    return f16_bits(dequant_exact(qw, s, b, group)).T.copy()


# ---------------------------------------------------------------------- quantize


def quantize(w) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Float weights -> the affine int4 format: (qw uint32 [N][K/8], s f16 [N][K/64],
    b f16 [N][K/64]) for w f16 [N][K] (np.float16 values or uint16 bit patterns).

    Per (row, group of 64): lo and hi are the group's smallest and largest value (a zero
    becomes +0); b = lo; s = RN16(f32(f32(hi - lo) / 15)); each code is
    q = clamp(rint_even(f32(f32(w - b) / s)), 0, 15), or 0 for the whole group when s is 0.
    NumPy float32 arithmetic is IEEE single precision with round-to-nearest-even.
    """
    w = np.asarray(w)
    if w.dtype == np.uint16:
        w = w.view(np.float16)
    assert w.dtype == np.float16 and w.ndim == 2
    n, k = w.shape
    assert k % GROUP == 0
    assert np.all(np.isfinite(w)), "weights must be finite"
    g = w.reshape(n, k // GROUP, GROUP).astype(np.float32)        # exact
    lo = g.min(axis=2)
    hi = g.max(axis=2)
    lo = np.where(lo == 0, np.float32(0.0), lo)                  # -0 -> +0
    hi = np.where(hi == 0, np.float32(0.0), hi)
    d = (hi - lo).astype(np.float32)
    t = (d / np.float32(15.0)).astype(np.float32)
    s16 = t.astype(np.float16)                                   # one RN-even rounding
    b16 = lo.astype(np.float16)                                  # exact
    sf = s16.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = ((g - b16.astype(np.float32)[:, :, None]).astype(np.float32) / sf).astype(np.float32)
    q = np.where(sf == 0, np.float32(0.0), np.clip(np.rint(r), 0.0, 15.0))
    return pack(q.reshape(n, k).astype(np.uint8)), s16, b16


def _f32(x: float) -> float:
    """Round a Python float (an fp64 value) to the nearest f32, ties to even."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def quantize_loop(w) -> tuple[list, list, list]:
    """Independent scalar restatement of ``quantize`` for small inputs: Python floats with an
    explicit f32 rounding after each operation (the fp64 difference of two f16 values is
    exact, and an fp64 quotient of two f32 values rounds to the correctly rounded f32
    quotient), Python's ``round`` (half to even), ``struct`` for f16.  Returns codes [N][K]
    and s, b as f16 bit patterns [N][K/64]."""
    w = np.asarray(w)
    if w.dtype == np.uint16:
        w = w.view(np.float16)
    n, k = w.shape
    codes, sb, bb = [], [], []
    for row in range(n):
        qrow, srow, brow = [], [], []
        for g0 in range(0, k, GROUP):
            vals = [float(v) for v in w[row, g0:g0 + GROUP]]
            lo, hi = min(vals), max(vals)
            lo = 0.0 if lo == 0 else lo
            hi = 0.0 if hi == 0 else hi
            t = _f32(_f32(hi - lo) / 15.0)
            s_bits = struct.unpack("<H", struct.pack("<e", t))[0]
            s = struct.unpack("<e", struct.pack("<H", s_bits))[0]
            srow.append(s_bits)
            brow.append(struct.unpack("<H", struct.pack("<e", lo))[0])
            for v in vals:
                qrow.append(0 if s == 0 else min(15, max(0, round(_f32(_f32(v - lo) / s)))))
        codes.append(qrow)
        sb.append(srow)
        bb.append(brow)
    return codes, sb, bb


# -------------------------------------------------------------------- products


def gemv_ref(qw: np.ndarray, s, b, x, group: int = GROUP) -> tuple[np.ndarray, np.ndarray]:
    """Decode GEMV: y[m][n] = sum_k w[n][k] * x[m][k] in fp64, with the error scale.

    Returns (y_ref, bound), both fp64 [M][N], where bound = sum_k |w[n][k] x[m][k]|.
    x is f16 [M][K]; w is the exact dequantized weight (either format, see dequant_exact).
    """
    w = dequant_exact(qw, s, b, group)
    x64 = _f64(x)
    assert x64.ndim == 2 and x64.shape[1] == w.shape[1]
    return x64 @ w.T, np.abs(x64) @ np.abs(w).T


def gemm_ref(a, bmat) -> tuple[np.ndarray, np.ndarray]:
    """C[m][n] = sum_k A[m][k] * B[k][n] in fp64 with bound = sum_k |A B| (A, B f16)."""
    a64 = _f64(a)
    b64 = _f64(bmat)
    assert a64.ndim == 2 and b64.ndim == 2 and a64.shape[1] == b64.shape[0]
    return a64 @ b64, np.abs(a64) @ np.abs(b64)


# ---------------------------------------------------------------------- select


def topk_ref(logits: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Per row, the k largest logits: value descending, ties to the lower index.

    Returns (idx int64 [M][k], val [M][k] in the logits' dtype).  Column 0 is the
    greedy argmax.  -0.0 and +0.0 compare equal; logits must be finite.
    """
    v = np.asarray(logits)
    assert v.ndim == 2 and 1 <= k <= v.shape[1]
    assert np.all(np.isfinite(v)), "logits must be finite"
    # A stable sort of the negated values keeps equal values in index order.
    order = np.argsort(-v, axis=1, kind="stable")[:, :k]
    return order.astype(np.int64), np.take_along_axis(v, order, axis=1)


def topk_ref_loop(row, k: int) -> list:
    """Brute force for one row: sort (-value, index) pairs with Python's sort."""
    return [i for _, i in sorted((-float(x), i) for i, x in enumerate(row))][:k]


# ----------------------------------------------------------------------- checks


def check_bound(y, y_ref, bound, rtol: float = 2e-3) -> tuple[bool, float]:
    """Element-wise |y - y_ref| <= rtol * bound.  Returns (ok, worst err/bound).

    Where bound is 0 (e.g. an all-zero x row) y must be exactly 0.
    """
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    lim = rtol * bound
    ok = bool(np.all(err <= lim)) and bool(np.all(np.isfinite(y)))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    worst = float(np.max(ratio)) if ratio.size else 0.0
    return ok, worst


def check_topk_selection(logits, idx, val, k: int) -> bool:
    """Selection is exact: the host selection on the same f32 logits matches bit for bit."""
    ref_idx, ref_val = topk_ref(np.asarray(logits), k)
    return bool(
        np.array_equal(np.asarray(idx, dtype=np.int64), ref_idx)
        and np.array_equal(np.asarray(val, dtype=np.float32).view(np.uint32),
                           ref_val.astype(np.float32).view(np.uint32))
    )


def check_topk_vs_exact(exact_logits, idx, k: int, margin: float = 1e-2) -> tuple[bool, int]:
    """End-to-end check of a GPU top-k against fp64 logits.

    At rank r, if the gaps to ranks r-1 and r+1 of the fp64 order both exceed
    ``margin``, the index must equal the fp64 order's; otherwise it must lie in the
    near-tie class {i : |v[i] - v[order[r]]| <= margin}.  Returns (ok, number of
    ranks decided by the near-tie rule).
    """
    v = np.asarray(exact_logits, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    m, vlen = v.shape
    order = np.argsort(-v, axis=1, kind="stable")
    ok = True
    loose = 0
    for row in range(m):
        vs = v[row, order[row]]
        for r in range(k):
            up = np.inf if r == 0 else vs[r - 1] - vs[r]
            down = np.inf if r + 1 >= vlen else vs[r] - vs[r + 1]
            if up > margin and down > margin:
                ok &= bool(idx[row, r] == order[row, r])
            else:
                loose += 1
                ok &= bool(abs(v[row, idx[row, r]] - vs[r]) <= margin)
        ok &= len(set(idx[row, :k].tolist())) == k
    return ok, loose
