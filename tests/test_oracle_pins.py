"""Pins of the CPU oracle to things other than itself (CPU only).

Each oracle function is checked against hand-derived fixtures (tests/golden),
closed forms, exact rational brute force, an independent encoder, or a textbook
sort.  ``test_mutants_fail`` plants plausible mistakes in copies of the oracle's
functions (on the CPU) and shows that each one fails at least one pin.
"""

from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import w4ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- pin suites
# Each suite takes the implementation under test and returns a list of failures, so the
# same suite judges the real oracle (must be empty) and the planted mutants (must not).


def pins_pack(pack, unpack):
    fails = []
    for c in _gold("pack_worked.json")["cases"]:
        q = np.array([c["codes"]], dtype=np.uint8)
        want = int(c["word"], 16)
        got = int(np.asarray(pack(q))[0, 0])
        if got != want:
            fails.append(f"pack {c['codes']} -> {got:#x} != {want:#x}")
        back = np.asarray(unpack(np.array([[want]], dtype=np.uint32)))[0].tolist()
        if back != c["codes"]:
            fails.append(f"unpack {want:#x} -> {back}")
    return fails


def _pattern(spec, k):
    kind, *arg = spec.split()
    kk = np.arange(k)
    if kind == "const":
        return np.full(k, float(arg[0]))
    if kind == "mod16":
        return (kk % 16).astype(float)
    if kind == "rev16":
        return (15 - kk % 16).astype(float)
    if kind == "alt":
        return np.where(kk % 2 == 0, 1.0, -1.0)
    if kind == "onehot":
        v = np.zeros(k)
        v[int(arg[0])] = 1.0
        return v
    raise ValueError(spec)


def gold_gemv_cases():
    for c in _gold("gemv_handworked.json")["cases"]:
        k = c["K"]
        q = _pattern(c["q"], k).astype(np.uint8)[None, :]
        s = np.array([c["s"]], dtype=np.float16)
        b = np.array([c["b"]], dtype=np.float16)
        x = np.stack([_pattern(p, k) for p in c["x"]]).astype(np.float16)
        yield c["name"], q, s, b, x, np.array(c["y"], dtype=np.float64)[:, None]


def pins_gemv(gemv, pack):
    fails = []
    for name, q, s, b, x, y_want in gold_gemv_cases():
        y, _ = gemv(pack(q), s, b, x)
        if not np.array_equal(np.asarray(y), y_want):
            fails.append(f"{name}: {np.asarray(y).ravel()} != {y_want.ravel()}")
    return fails


def pins_dequant(dequant_f16_t, pack):
    fails = []
    for c in _gold("f16_dequant.json")["cases"]:
        # one row, one group: the case's code sits at k = 5, all other codes are 0
        q = np.zeros((1, 64), dtype=np.uint8)
        q[0, 5] = c["q"]
        s = np.array([[int(c["s"], 16)]], dtype=np.uint16).view(np.float16)
        b = np.array([[int(c["b"], 16)]], dtype=np.uint16).view(np.float16)
        wt = np.asarray(dequant_f16_t(pack(q), s, b))
        if wt.shape != (64, 1):
            fails.append(f"shape {wt.shape}")
            continue
        got = int(wt[5, 0])
        if got != int(c["w"], 16):
            fails.append(f"s={c['s']} q={c['q']} b={c['b']}: {got:#06x} != {c['w']}")
        if int(wt[0, 0]) != int(c["b"], 16):
            fails.append(f"q=0 -> {int(wt[0, 0]):#06x} != b {c['b']}")
    return fails


def pins_topk(topk):
    cases = [
        ([3.0, 1.0, 3.0, 2.0], 2, [0, 2]),
        ([-0.0, 0.0, -1.0], 2, [0, 1]),
        ([0.0, -0.0, 0.0, -0.0], 4, [0, 1, 2, 3]),
        ([5.0] * 5, 3, [0, 1, 2]),
        ([1.0, 2.0, 3.0, 4.0, 5.0], 5, [4, 3, 2, 1, 0]),
        ([5.0, 4.0, 3.0, 2.0, 1.0], 3, [0, 1, 2]),
        ([1.0, 7.0, 7.0, 2.0, 7.0, 3.0], 2, [1, 2]),
        ([-3.0, -1.0, -2.0], 1, [1]),
    ]
    fails = []
    for row, k, want in cases:
        idx, val = topk(np.array([row], dtype=np.float32), k)
        if np.asarray(idx)[0].tolist() != want:
            fails.append(f"{row} k={k}: {np.asarray(idx)[0].tolist()} != {want}")
        if np.asarray(val)[0].tolist() != [row[i] for i in want]:
            fails.append(f"{row} k={k}: values")
    return fails


def pins_sym128(gemv, dequant_f16_t, pack):
    """The symmetric group-128 format: hand-worked GEMVs and dequantized bit patterns."""
    fails = []
    gold = _gold("sym128_handworked.json")
    for c in gold["gemv"]:
        k = c["K"]
        q = _pattern(c["q"], k).astype(np.uint8)[None, :]
        sv = np.array([c["s"]], dtype=np.float16)
        x = np.stack([_pattern(p_, k) for p_ in c["x"]]).astype(np.float16)
        y, _ = gemv(pack(q), sv, None, x, group=128)
        if not np.array_equal(np.asarray(y), np.array(c["y"], dtype=np.float64)[:, None]):
            fails.append(f"{c['name']}: {np.asarray(y).ravel()} != {c['y']}")
    for c in gold["dequant"]:
        q = np.full((1, 128), 8, dtype=np.uint8)
        q[0, 5] = c["q"]
        sv = np.array([[int(c["s"], 16)]], dtype=np.uint16).view(np.float16)
        with np.errstate(over="ignore"):
            wt = np.asarray(dequant_f16_t(pack(q), sv, None, group=128))
        if int(wt[5, 0]) != int(c["w"], 16):
            fails.append(f"s={c['s']} q={c['q']}: {int(wt[5, 0]):#06x} != {c['w']}")
        if int(wt[0, 0]) != 0:
            fails.append(f"s={c['s']} q=8: {int(wt[0, 0]):#06x} != +0")
    return fails


def _quant_group(head, fill):
    bits = [int(h, 16) for h in head] + [int(fill, 16)] * (64 - len(head))
    return np.array([bits], dtype=np.uint16).view(np.float16)


def _grid_groups(n_rows, n_groups, seed):
    """Rows of groups that lie exactly on an affine grid: w = b + s*q with s = 2^-e
    (e = 3..6), b a multiple of 2^-6 in [-2, 2], every group holding a 0 and a 15 code;
    all values are exact f16 and the fit must give back exactly (q, s, b)."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(n_rows, n_groups, 64))
    q[:, :, 3] = 0
    q[:, :, 40] = 15
    s = 2.0 ** -rng.integers(3, 7, size=(n_rows, n_groups))
    b = rng.integers(-128, 129, size=(n_rows, n_groups)) / 64.0
    w = b[:, :, None] + s[:, :, None] * q
    return (w.reshape(n_rows, -1).astype(np.float16), q.reshape(n_rows, -1).astype(np.uint8),
            s.astype(np.float16), b.astype(np.float16))


def pins_quantize(quantize, unpack):
    fails = []
    for c in _gold("quantize_worked.json")["cases"]:
        qw, sv, bv = quantize(_quant_group(c["head"], c["fill"]))
        codes = np.asarray(unpack(np.asarray(qw)))[0]
        s_bits = int(np.asarray(sv, dtype=np.float16).view(np.uint16)[0, 0])
        b_bits = int(np.asarray(bv, dtype=np.float16).view(np.uint16)[0, 0])
        want = c["codes_head"]
        if codes[:len(want)].tolist() != want:
            fails.append(f"{c['name']}: codes {codes[:len(want)].tolist()} != {want}")
        fill_code = 0  # every fixture's fill value is its group minimum (or the constant)
        if np.any(codes[len(c["head"]):] != fill_code):
            fails.append(f"{c['name']}: fill codes {sorted(set(codes[len(c['head']):].tolist()))}")
        if s_bits != int(c["s"], 16):
            fails.append(f"{c['name']}: s {s_bits:#06x} != {c['s']}")
        if b_bits != int(c["b"], 16):
            fails.append(f"{c['name']}: b {b_bits:#06x} != {c['b']}")
    # exact affine grids come back unchanged
    w, q, s_, b_ = _grid_groups(3, 4, seed=41)
    qw, sv, bv = quantize(w)
    if not (np.array_equal(np.asarray(unpack(np.asarray(qw))), q)
            and np.array_equal(np.asarray(sv, np.float16).view(np.uint16), s_.view(np.uint16))
            and np.array_equal(np.asarray(bv, np.float16).view(np.uint16), (b_ + np.float16(0)).view(np.uint16))):
        fails.append("exact grid not reproduced")
    return fails


def test_pins_pass_on_oracle():
    assert pins_pack(oracle.pack, oracle.unpack) == []
    assert pins_gemv(oracle.gemv_ref, oracle.pack) == []
    assert pins_dequant(oracle.dequant_f16_t, oracle.pack) == []
    assert pins_topk(oracle.topk_ref) == []
    assert pins_quantize(oracle.quantize, oracle.unpack) == []
    assert pins_sym128(oracle.gemv_ref, oracle.dequant_f16_t, oracle.pack) == []


# ------------------------------------------------------------------------------- pack


def test_pack_roundtrip_all_nibbles_all_positions():
    # every code value in every position of the word
    q = np.zeros((16 * 8, 8), dtype=np.uint8)
    for v in range(16):
        for i in range(8):
            q[v * 8 + i, i] = v
    w = oracle.pack(q)
    for v in range(16):
        for i in range(8):
            assert int(w[v * 8 + i, 0]) == v << (4 * i)
    assert np.array_equal(oracle.unpack(w), q)


def test_pack_roundtrip_random():
    q = synth.codes(37, 64 * 5, seed=1)
    assert np.array_equal(oracle.unpack(oracle.pack(q)), q)
    words = np.random.default_rng(2).integers(0, 2**32, size=(1000, 1000), dtype=np.uint32)
    assert np.array_equal(oracle.pack(oracle.unpack(words)), words)


def test_pack_numpy_matches_python_loop():
    q = synth.codes(5, 128, seed=3)
    assert oracle.pack(q).tolist() == oracle.pack_loop(q.tolist())
    w = oracle.pack(q)
    assert oracle.unpack(w).tolist() == oracle.unpack_loop(w.tolist())


def test_pack_keeps_low_nibble_only():
    q = np.array([[16, 17, 255, 0, 0, 0, 0, 31]], dtype=np.uint8)
    assert int(oracle.pack(q)[0, 0]) == int(oracle.pack(q & 0xF)[0, 0]) == 0xF0000F10


# ---------------------------------------------------------------------------- f16 + dequant


def test_f16_encoder_matches_struct():
    r = np.random.default_rng(4)
    vals = np.concatenate([
        r.standard_normal(20000) * 10.0 ** r.integers(-8, 4, 20000),
        # exact midpoints between neighbouring f16 values, and points just off them
        (np.arange(-2000, 2000) + 0.5) * 2.0 ** -10,
        (np.arange(-2000, 2000) + 0.5) * 2.0 ** -24,
        (np.arange(1, 4000) + 0.5) * 2.0 ** -24 + 2.0 ** -60,
        [0.0, -0.0, 65504.0, -65504.0, 2.0 ** -24, 2.0 ** -25, 2.0 ** -26, 3 * 2.0 ** -26],
    ])
    assert np.array_equal(oracle.f16_bits(vals), oracle.f16_bits_struct(vals))


def test_dequant_exact_matches_fraction_bruteforce():
    q, s, b = synth.w4_weights(3, 128, seed=5)
    w = oracle.dequant_exact(oracle.pack(q), s, b)
    for n in range(3):
        for k in range(128):
            g = k // 64
            exact = Fraction(float(s[n, g])) * int(q[n, k]) + Fraction(float(b[n, g]))
            assert Fraction(w[n, k]) == exact


def test_dequant_f16_t_is_transposed_rounded_exact():
    q, s, b = synth.w4_weights(7, 192, seed=6)
    qw = oracle.pack(q)
    wt = oracle.dequant_f16_t(qw, s, b)
    assert wt.shape == (192, 7) and wt.dtype == np.uint16
    assert np.array_equal(wt, oracle.f16_bits_struct(oracle.dequant_exact(qw, s, b)).T)
    # closed forms: s = 1, b = 0 -> w = q; b = -8 s -> w = s (q - 8)
    ones = np.ones((7, 3), dtype=np.float16)
    zeros = np.zeros((7, 3), dtype=np.float16)
    assert np.array_equal(oracle.f16_value(oracle.dequant_f16_t(qw, ones, zeros)), q.T.astype(np.float64))
    sym = oracle.dequant_exact(qw, s, (-8.0 * s.astype(np.float64)).astype(np.float16))
    grp = np.arange(192) // 64
    assert np.allclose(sym, s.astype(np.float64)[:, grp] * (q.astype(np.float64) - 8), rtol=0, atol=1e-3)


# ------------------------------------------------------------------------------ GEMV


def test_gemv_closed_forms():
    m, n, k = 3, 9, 192
    x = synth.activations(m, k, seed=7)
    x64 = x.astype(np.float64)
    ones = np.ones((n, k // 64), dtype=np.float16)
    zeros = np.zeros((n, k // 64), dtype=np.float16)
    for c in (0, 1, 7, 15):
        q = np.full((n, k), c, dtype=np.uint8)
        y, bound = oracle.gemv_ref(oracle.pack(q), ones, zeros, x)
        assert np.array_equal(y, np.repeat((c * x64.sum(axis=1))[:, None], n, axis=1))
    # q = 0: y = sum_g b_g X_g with X_g the group sums of x
    _, s, b = synth.w4_weights(n, k, seed=8)
    y, _ = oracle.gemv_ref(oracle.pack(np.zeros((n, k), np.uint8)), s, b, x)
    xg = x64.reshape(m, k // 64, 64).sum(axis=2)
    assert np.allclose(y, xg @ b.astype(np.float64).T, rtol=1e-13, atol=0)
    # x = e_k: y[n] = w[n][k]
    q, s, b = synth.w4_weights(n, k, seed=9)
    qw = oracle.pack(q)
    w = oracle.dequant_exact(qw, s, b)
    for kk in (0, 63, 64, 100, 191):
        e = np.zeros((1, k), dtype=np.float16)
        e[0, kk] = 1.0
        y, bound = oracle.gemv_ref(qw, s, b, e)
        assert np.array_equal(y[0], w[:, kk]) and np.array_equal(bound[0], np.abs(w[:, kk]))
    # x = 0: y = 0 and bound = 0
    y, bound = oracle.gemv_ref(qw, s, b, np.zeros((2, k), np.float16))
    assert not y.any() and not bound.any()


def test_gemv_matches_fraction_bruteforce():
    for k, n, m, seed in ((64, 5, 3, 10), (128, 4, 2, 11)):
        q, s, b = synth.w4_weights(n, k, seed=seed)
        x = synth.activations(m, k, seed=seed)
        y, bound = oracle.gemv_ref(oracle.pack(q), s, b, x)
        for mm in range(m):
            for nn in range(n):
                tot = Fraction(0)
                mag = Fraction(0)
                for kk in range(k):
                    g = kk // 64
                    w = Fraction(float(s[nn, g])) * int(q[nn, kk]) + Fraction(float(b[nn, g]))
                    t = w * Fraction(float(x[mm, kk]))
                    tot += t
                    mag += abs(t)
                assert abs(Fraction(y[mm, nn]) - tot) <= Fraction(1, 10**12) * mag
                assert abs(Fraction(bound[mm, nn]) - mag) <= Fraction(1, 10**12) * mag


def test_check_bound_rule():
    y_ref = np.array([[1.0, -2.0, 0.0]])
    bound = np.array([[10.0, 10.0, 0.0]])
    assert oracle.check_bound(y_ref + np.array([[0.019, -0.0199, 0.0]]), y_ref, bound)[0]
    assert not oracle.check_bound(y_ref + np.array([[0.021, 0, 0]]), y_ref, bound)[0]
    assert not oracle.check_bound(y_ref + np.array([[0, 0, 1e-30]]), y_ref, bound)[0]
    assert not oracle.check_bound(np.array([[np.nan, -2.0, 0.0]]), y_ref, bound)[0]


def test_tolerance_admits_f32_accumulation():
    # Any f32 summation of exact products errs by at most gamma_K * bound with
    # gamma_K ~ K * 2**-24 (Higham); at K = 15360 that is 9.2e-4 < 2e-3.  A sequential
    # f32 sum must therefore pass the rule.
    k = 15360
    q, s, b = synth.w4_weights(4, k, seed=12)
    x = synth.activations(1, k, seed=12)
    qw = oracle.pack(q)
    y_ref, bound = oracle.gemv_ref(qw, s, b, x)
    w32 = oracle.dequant_exact(qw, s, b).astype(np.float32)
    acc = np.zeros(4, dtype=np.float32)
    for kk in range(k):
        acc += w32[:, kk] * np.float32(x[0, kk])
    assert oracle.check_bound(acc[None, :], y_ref, bound)[0]


# ------------------------------------------------------------------------------ GEMM


def test_gemm_identity_and_onehot():
    a = synth.activations(5, 64, seed=13)
    eye = np.eye(64, dtype=np.float16)
    c, bound = oracle.gemm_ref(a, eye)
    assert np.array_equal(c, a.astype(np.float64))
    bmat = synth.activations(64, 7, seed=14)
    onehot = np.zeros((3, 64), dtype=np.float16)
    onehot[0, 0] = onehot[1, 31] = onehot[2, 63] = 1.0
    c, _ = oracle.gemm_ref(onehot, bmat)
    assert np.array_equal(c, bmat.astype(np.float64)[[0, 31, 63]])


def test_gemm_matches_fraction_bruteforce():
    a = synth.activations(3, 16, seed=15)
    bmat = synth.activations(16, 3, seed=16)  # square-ish so a transposed operand would still run
    c, bound = oracle.gemm_ref(a, bmat)
    for i in range(3):
        for j in range(3):
            terms = [Fraction(float(a[i, kk])) * Fraction(float(bmat[kk, j])) for kk in range(16)]
            assert abs(Fraction(c[i, j]) - sum(terms)) <= Fraction(1, 10**12) * sum(abs(t) for t in terms)
            assert Fraction(bound[i, j]) == sum(abs(t) for t in terms)


# ------------------------------------------------------------------------------ top-k


def test_topk_matches_python_sort():
    r = np.random.default_rng(17)
    for v, k in ((1, 1), (7, 7), (50, 10), (300, 64), (2, 1), (1000, 256)):
        rows = r.integers(-4, 4, size=(3, v)).astype(np.float32) * 0.5  # many ties
        rows[:, ::7] = -rows[:, ::7]
        rows[rows == 0] = np.where(r.random((rows == 0).sum()) < 0.5, -0.0, 0.0)
        idx, val = oracle.topk_ref(rows, k)
        for i in range(3):
            assert idx[i].tolist() == oracle.topk_ref_loop(rows[i].tolist(), k)
            assert np.array_equal(val[i], rows[i, idx[i]])
    # k = V is the full stable sort; k = 1 is the argmax
    row = r.standard_normal((1, 999)).astype(np.float32)
    assert oracle.topk_ref(row, 999)[0][0].tolist() == oracle.topk_ref_loop(row[0].tolist(), 999)
    assert oracle.topk_ref(row, 1)[0][0, 0] == int(np.argmax(row[0]))


def test_topk_checks():
    v = np.array([[3.0, 2.995, 1.0, 0.0]], dtype=np.float64)
    # gap 0.005 < 1e-2: ranks 0 and 1 may swap, rank 2 must match
    assert oracle.check_topk_vs_exact(v, np.array([[1, 0, 2]]), 3)[0]
    assert not oracle.check_topk_vs_exact(v, np.array([[1, 0, 3]]), 3)[0]
    assert not oracle.check_topk_vs_exact(np.array([[3.0, 2.0, 1.0]]), np.array([[1, 0]]), 2)[0]
    lg = np.array([[0.5, 2.0, 2.0, -1.0]], dtype=np.float32)
    assert oracle.check_topk_selection(lg, [[1, 2]], [[2.0, 2.0]], 2)
    assert not oracle.check_topk_selection(lg, [[2, 1]], [[2.0, 2.0]], 2)


# -------------------------------------------------------------------- page figures


def test_page_figures_fix_head_and_logit_dtypes():
    g = _gold("page_figures.json")
    assert (g["hidden"], g["vocab"]) == (synth.QWEN25_3B_HIDDEN, synth.QWEN25_3B_VOCAB)
    head_bytes = g["hidden"] * g["vocab"] * 2
    assert round(head_bytes / 1e6) == g["head_mb_per_token"]
    # 4-byte logits are within 2% of the printed size; 2-byte ones are half of it
    assert abs(g["vocab"] * 4 / 1e3 - g["logits_kb_per_token"]) / g["logits_kb_per_token"] < 0.02
    assert abs(g["vocab"] * 2 / 1e3 - g["logits_kb_per_token"]) / g["logits_kb_per_token"] > 0.4


# --------------------------------------------------------------------------- quantize


def test_quantize_matches_scalar_restatement():
    rng = np.random.default_rng(44)
    w = (rng.standard_normal((5, 256)) * 0.02).astype(np.float16)
    w[1, :64] = 0.5                                    # constant group
    w[2, 64:128] = -0.0                                # all negative zeros
    w[3, 128:192] = rng.integers(-3, 4, size=64) * np.float16(2.0 ** -24)  # subnormal range
    w[4, 192:] = rng.standard_normal(64) * 3000        # large magnitudes
    qw, s, b = oracle.quantize(w)
    codes, sb, bb = oracle.quantize_loop(w)
    assert np.array_equal(oracle.unpack(qw), np.array(codes, dtype=np.uint8))
    assert np.array_equal(s.view(np.uint16), np.array(sb, dtype=np.uint16))
    assert np.array_equal(b.view(np.uint16), np.array(bb, dtype=np.uint16))


def test_quantize_error_bound():
    # |w - (s q + b)| <= s/2 away from the clamp; at most 15 |t - s| more where the rounded
    # scale makes the top code overshoot 15 (t = (max - min) / 15 exactly)
    rng = np.random.default_rng(45)
    w = (rng.standard_normal((16, 1024)) * 0.02).astype(np.float16)
    qw, s, b = oracle.quantize(w)
    w_hat = oracle.dequant_exact(qw, s, b)
    g = w.astype(np.float64).reshape(16, 16, 64)
    t = (g.max(axis=2) - g.min(axis=2)) / 15.0
    s64 = s.astype(np.float64)
    bound = 0.5 * s64 * (1 + 2.0 ** -20) + 15 * np.abs(t - s64)
    err = np.abs(w.astype(np.float64) - w_hat).reshape(16, 16, 64).max(axis=2)
    assert np.all(err <= bound)
    assert np.all(oracle.unpack(qw).reshape(16, 16, 64).min(axis=2) == 0)


def test_quantize_then_dequant_is_identity_on_grids():
    w, q, s, b = _grid_groups(8, 8, seed=46)
    qw, s2, b2 = oracle.quantize(w)
    assert np.array_equal(oracle.dequant_exact(qw, s2, b2), w.astype(np.float64))


def test_sym128_equals_affine_with_bias_minus_8s():
    # the symmetric format is the affine one at group 64 with each scale repeated over its two
    # halves and b = -8 s (exact: a power-of-two multiple), dequantized through the other path
    rng = np.random.default_rng(47)
    q = rng.integers(0, 16, size=(6, 512)).astype(np.uint8)
    s128 = (rng.standard_normal((6, 4)) * 0.02).astype(np.float16)
    s64 = np.repeat(s128, 2, axis=1)
    b64 = (-8.0 * s64.astype(np.float64)).astype(np.float16)
    assert np.array_equal(b64.astype(np.float64), -8.0 * s64.astype(np.float64))
    qw = oracle.pack(q)
    assert np.array_equal(oracle.dequant_f16_t(qw, s128, None, group=128), oracle.dequant_f16_t(qw, s64, b64))
    x = synth.activations(3, 512, seed=48)
    y1, b1 = oracle.gemv_ref(qw, s128, None, x, group=128)
    y2, b2 = oracle.gemv_ref(qw, s64, b64, x)
    assert np.allclose(y1, y2, rtol=0, atol=1e-12) and np.allclose(b1, b2, rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------ mutants


def _mut_unpack_high_first(qw):
    q = w4ref.unpack(qw)
    n, k = q.shape
    return q.reshape(n, k // 8, 8)[:, :, ::-1].reshape(n, k).copy()


def _mut_pack_high_first(q):
    n, k = q.shape
    return w4ref.pack(np.asarray(q).reshape(n, k // 8, 8)[:, :, ::-1].reshape(n, k))


def _dequant_with(qw, s, b, group=64, shift=0, use_bias=True, sym=False):
    q = w4ref.unpack(qw).astype(np.float64)
    n, k = q.shape
    grp = np.minimum((np.arange(k) + shift) // group, s.shape[1] - 1)
    s64 = s.astype(np.float64)[:, grp]
    if sym:
        return s64 * (q - 8)
    return s64 * q + (b.astype(np.float64)[:, grp] if use_bias else 0.0)


def _gemv_from(dq):
    def gemv(qw, s, b, x):
        w = dq(qw, s, b)
        x64 = x.astype(np.float64)
        return x64 @ w.T, np.abs(x64) @ np.abs(w).T
    return gemv


def _dequant_t_from(dq):
    return lambda qw, s, b: w4ref.f16_bits(dq(qw, s, b)).T.copy()


def _dequant_t_double_round(qw, s, b):
    return w4ref.f16_bits(w4ref.dequant_exact(qw, s, b).astype(np.float32)).T.copy()


def _dequant_t_ftz(qw, s, b):
    w = w4ref.dequant_exact(qw, s, b)
    w = np.where(np.abs(w) < 2.0 ** -14, 0.0, w)
    return w4ref.f16_bits(w).T.copy()


def _gemv_drop_last_k(qw, s, b, x):
    w = w4ref.dequant_exact(qw, s, b)[:, :-1]
    x64 = x.astype(np.float64)[:, :-1]
    return x64 @ w.T, np.abs(x64) @ np.abs(w).T


def _topk_last_index_ties(v, k):
    v = np.asarray(v)
    rev = v[:, ::-1]
    order = np.argsort(-rev, axis=1, kind="stable")[:, :k]
    idx = v.shape[1] - 1 - order
    return idx, np.take_along_axis(v, idx, axis=1)


def _topk_raw_bits(v, k):
    # orders by the f32 bit pattern read as a signed integer (wrong for negatives)
    v = np.asarray(v, dtype=np.float32)
    order = np.argsort(-v.view(np.int32).astype(np.int64), axis=1, kind="stable")[:, :k]
    return order, np.take_along_axis(v, order, axis=1)


def _topk_ascending(v, k):
    order = np.argsort(np.asarray(v), axis=1, kind="stable")[:, :k]
    return order, np.take_along_axis(np.asarray(v), order, axis=1)


def _quantize_with(w, rnd=np.rint, div=15.0, use_max_as_b=False, clamp=True, wide=False, keep_neg_zero=False,
                   codes_from_t=False):
    w = np.asarray(w)
    n, k = w.shape
    f = np.float64 if wide else np.float32
    g = w.reshape(n, k // 64, 64).astype(f)
    lo, hi = g.min(axis=2), g.max(axis=2)
    if not keep_neg_zero:
        lo = np.where(lo == 0, f(0.0), lo)
    hi = np.where(hi == 0, f(0.0), hi)
    t = ((hi - lo) / f(div)).astype(f)
    s16 = t.astype(np.float16)
    b16 = (hi if use_max_as_b else lo).astype(np.float16)
    sf = (t if codes_from_t else s16.astype(f))[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = ((g - b16.astype(f)[:, :, None]).astype(f) / sf).astype(f)
    r = rnd(r)
    q = np.where(sf == 0, 0.0, np.clip(r, 0, 15) if clamp else np.maximum(r, 0))
    return w4ref.pack(q.reshape(n, k).astype(np.uint8)), s16, b16


def _sym_dequant(zero=8.0, group=128, plus_zero=True, flip=False):
    def dq(qw, sv, b, group_arg=None):
        q = w4ref.unpack(qw).astype(np.float64)
        n, k = q.shape
        grp = np.minimum(np.arange(k) // group, sv.shape[1] - 1)
        w = sv.astype(np.float64)[:, grp] * ((zero - q) if flip else (q - zero))
        return w + 0.0 if plus_zero else w
    return dq


def _sym_pins_with(dq):
    def gemv(qw, sv, b, x, group=128):
        w = dq(qw, sv, b)
        x64 = x.astype(np.float64)
        return x64 @ w.T, np.abs(x64) @ np.abs(w).T

    def deq(qw, sv, b, group=128):
        with np.errstate(over="ignore"):
            return w4ref.f16_bits(dq(qw, sv, b)).T.copy()
    return pins_sym128(gemv, deq, w4ref.pack)


MUTANTS = {
    "unpack high nibble first": lambda: pins_pack(w4ref.pack, _mut_unpack_high_first),
    "pack high nibble first": lambda: pins_pack(_mut_pack_high_first, w4ref.unpack)
    + pins_gemv(w4ref.gemv_ref, _mut_pack_high_first),
    "group size 128": lambda: pins_gemv(_gemv_from(lambda qw, s, b: _dequant_with(qw, s, b, group=128)), w4ref.pack),
    "missing bias": lambda: pins_gemv(_gemv_from(lambda qw, s, b: _dequant_with(qw, s, b, use_bias=False)), w4ref.pack),
    "s*(q-8) without b": lambda: pins_gemv(_gemv_from(lambda qw, s, b: _dequant_with(qw, s, b, sym=True)), w4ref.pack),
    "group index off by one": lambda: pins_gemv(_gemv_from(lambda qw, s, b: _dequant_with(qw, s, b, shift=1)), w4ref.pack),
    "dropped last k term": lambda: pins_gemv(_gemv_drop_last_k, w4ref.pack),
    "f32 then f16 rounding": lambda: pins_dequant(_dequant_t_double_round, w4ref.pack),
    "subnormals flushed": lambda: pins_dequant(_dequant_t_ftz, w4ref.pack),
    "dequant missing bias": lambda: pins_dequant(_dequant_t_from(lambda qw, s, b: _dequant_with(qw, s, b, use_bias=False)), w4ref.pack),
    "argmax ties to last index": lambda: pins_topk(_topk_last_index_ties),
    "raw-bit comparison": lambda: pins_topk(_topk_raw_bits),
    "ascending order": lambda: pins_topk(_topk_ascending),
    "quantize truncates": lambda: pins_quantize(lambda w: _quantize_with(w, rnd=np.floor), w4ref.unpack),
    "quantize ties away from zero": lambda: pins_quantize(lambda w: _quantize_with(w, rnd=lambda r: np.floor(r + 0.5)),
                                                          w4ref.unpack),
    "quantize over 16 steps": lambda: pins_quantize(lambda w: _quantize_with(w, div=16.0), w4ref.unpack),
    "quantize bias from the max": lambda: pins_quantize(lambda w: _quantize_with(w, use_max_as_b=True), w4ref.unpack),
    "quantize without clamp": lambda: pins_quantize(lambda w: _quantize_with(w, clamp=False), w4ref.unpack),
    "quantize in fp64": lambda: pins_quantize(lambda w: _quantize_with(w, wide=True), w4ref.unpack),
    "quantize keeps -0 as bias": lambda: pins_quantize(lambda w: _quantize_with(w, keep_neg_zero=True), w4ref.unpack),
    "quantize codes from unrounded scale": lambda: pins_quantize(lambda w: _quantize_with(w, codes_from_t=True),
                                                                 w4ref.unpack),
    "symmetric zero point 7": lambda: _sym_pins_with(_sym_dequant(zero=7.0)),
    "symmetric over groups of 64": lambda: _sym_pins_with(_sym_dequant(group=64)),
    "symmetric zero keeps its sign": lambda: _sym_pins_with(_sym_dequant(plus_zero=False)),
    "symmetric sign flipped": lambda: _sym_pins_with(_sym_dequant(flip=True)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_fail(name):
    assert MUTANTS[name](), f"planted mistake '{name}' passed every pin"


def test_gemm_transposed_operand_fails_bruteforce():
    a = synth.activations(4, 4, seed=18)
    bmat = synth.activations(4, 4, seed=19)
    c_bad = a.astype(np.float64) @ bmat.astype(np.float64).T
    exact = [[sum(Fraction(float(a[i, kk])) * Fraction(float(bmat[kk, j])) for kk in range(4)) for j in range(4)]
             for i in range(4)]
    assert any(Fraction(c_bad[i, j]) != exact[i][j] for i in range(4) for j in range(4))
    c_ok, _ = oracle.gemm_ref(a, bmat)
    assert all(abs(Fraction(c_ok[i, j]) - exact[i][j]) < Fraction(1, 10**9) for i in range(4) for j in range(4))
