"""GPU parity: every HIP entry point, called through the C ABI, against the CPU oracle.

Integer and byte work (pack, dequant bits, top-k indices) must be bit-exact; f32 products
must satisfy |y - y_ref| <= 2e-3 * sum_k |w_k x_k| per output.  Shapes span several tiles
and ragged tails; the workload shapes run at full size (sampled rows where the fp64
reference would be slow).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

RTOL = 2e-3


@pytest.fixture(scope="module")
def w4():
    import int4_weight_only_group_amd as m
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def upload_layer(w4, q, s, b):
    qw = w4.w4_pack(dev(q))
    return qw, dev(s), dev(b)


# ----------------------------------------------------------------------------- pack


@pytest.mark.parametrize("n,k", [(1, 64), (3, 128), (37, 960), (4864, 896), (257, 2048), (5, 11008), (22016, 2048), (2048, 11008)])
def test_pack_bit_exact(w4, n, k):
    q = synth.codes(n, k, seed=n + k)
    got = to_np(w4.w4_pack(dev(q))).view(np.uint32)
    assert np.array_equal(got, oracle.pack(q))


def test_pack_keeps_low_nibble(w4):
    q = np.random.default_rng(3).integers(0, 256, size=(9, 128), dtype=np.uint8)
    got = to_np(w4.w4_pack(dev(q))).view(np.uint32)
    assert np.array_equal(got, oracle.pack(q))
    assert np.array_equal(oracle.unpack(got), q & 0xF)


# ----------------------------------------------------------------------------- quantize


def quantize_case(w4, w, ldw_pad=0):
    """Run w4_quantize on f16 weights w [N][K] and compare codes, scales and biases bit for bit
    with the oracle."""
    n, k = w.shape
    wd = dev(np.pad(w, ((0, 0), (0, ldw_pad))))[:, :k]
    qw, s, b = w4.w4_quantize(wd)
    qw_ref, s_ref, b_ref = oracle.quantize(w)
    got_q = to_np(qw).view(np.uint32)
    assert np.array_equal(got_q, qw_ref), f"codes differ at {np.argwhere(got_q != qw_ref)[:4].tolist()}"
    assert np.array_equal(to_np(s).view(np.uint16), s_ref.view(np.uint16))
    assert np.array_equal(to_np(b).view(np.uint16), b_ref.view(np.uint16))
    return qw, s, b


@pytest.mark.parametrize("n,k", [(1, 64), (3, 128), (33, 960), (257, 2048), (100, 11008), (31, 64 * 45)])
def test_quantize_bit_exact(w4, n, k):
    rng = np.random.default_rng(n * 1000 + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float16)
    quantize_case(w4, w)


def test_quantize_worked_groups(w4):
    # the hand-worked groups of the oracle's fixture, one per row, on the device
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "quantize_worked.json")) as f:
        cases = json.load(f)["cases"]
    rows = [[int(h, 16) for h in c["head"]] + [int(c["fill"], 16)] * (64 - len(c["head"])) for c in cases]
    w = np.array(rows, dtype=np.uint16).view(np.float16)
    qw, s, b = quantize_case(w4, w)
    codes = oracle.unpack(to_np(qw).view(np.uint32))
    for i, c in enumerate(cases):
        assert codes[i, :len(c["codes_head"])].tolist() == c["codes_head"], c["name"]
        assert int(to_np(s).view(np.uint16)[i, 0]) == int(c["s"], 16), c["name"]
        assert int(to_np(b).view(np.uint16)[i, 0]) == int(c["b"], 16), c["name"]


def test_quantize_edge_values_and_stride(w4):
    rng = np.random.default_rng(77)
    w = (rng.standard_normal((9, 512)) * 0.02).astype(np.float16)
    w[0] = 0.0
    w[1] = -0.0
    w[2, :64] = 0.5
    w[3] = rng.integers(-5, 6, size=512) * np.float16(2.0 ** -24)     # subnormals
    w[4] = (rng.standard_normal(512) * 20000).astype(np.float16)      # near the f16 range
    w[5, ::2] = -0.0
    w[6] = np.float16(65504.0)
    w[6, ::64] = np.float16(-65504.0)
    w[7] = (rng.integers(0, 16, size=512) * 0.125 - 1.0).astype(np.float16)  # exact grid
    quantize_case(w4, w, ldw_pad=24)


def test_quantize_quotients_at_and_near_half_integers(w4):
    # Codes whose f32 quotient (w - b) / s is an exact half-integer (ties to even) or within
    # 4e-5 of one: where a reciprocal product cannot decide the code, the division must.
    rows = []
    for e in (-20, -10, -4, 0, 3):  # s = 2^e exactly: every quotient below is k + 1/2
        sc = 2.0 ** e
        w = np.array([0.0, 15 * sc] + [((i % 15) + 0.5) * sc for i in range(62)])
        rows.append(w.astype(np.float16))
    rng = np.random.default_rng(91)
    cand = (rng.standard_normal((40000, 64)) * 0.02).astype(np.float16)
    wf = cand.astype(np.float32)
    lo, hi = wf.min(1), wf.max(1)
    lo[lo == 0] = 0.0
    hi[hi == 0] = 0.0
    sq = ((hi - lo).astype(np.float32) / np.float32(15)).astype(np.float16).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        qt = ((wf - lo[:, None]).astype(np.float32) / sq[:, None]).astype(np.float32)
    dist = np.abs(qt - np.floor(qt) - np.float32(0.5))
    near = np.nonzero(((dist <= 4e-5) & (sq[:, None] > 0)).any(1))[0]
    assert len(near) >= 20, len(near)
    w = np.concatenate([np.stack(rows), cand[near]])
    qw, _, _ = quantize_case(w4, w)
    codes = oracle.unpack(to_np(qw).view(np.uint32))
    assert codes[0, 2:17].tolist() == [0, 2, 2, 4, 4, 6, 6, 8, 8, 10, 10, 12, 12, 14, 14]  # ties to even


def test_quantize_full_matrix_and_roundtrip(w4):
    # a gate-sized matrix of N(0, 0.02) weights, every code; then dequant of the result
    n, k = 11008, 2048
    w = (np.random.default_rng(5).standard_normal((n, k)) * 0.02).astype(np.float16)
    qw, s, b = quantize_case(w4, w)
    cols = np.arange(0, n, 97)
    wt = to_np(w4.w4_dequant_f16_t(qw, s, b)).view(np.uint16)[:, cols]
    qw_ref, s_ref, b_ref = oracle.quantize(w[cols])
    assert np.array_equal(wt, oracle.dequant_f16_t(qw_ref, s_ref, b_ref))


# ------------------------------------------------------------ symmetric group-128 format


def sym_case(w4, m, n, k, seed, ldx_pad=0, ldy_pad=0):
    q, s = synth.w4_sym128_weights(n, k, seed=seed)
    x = synth.activations(m, k, seed=seed)
    qw, sd = w4.w4_pack(dev(q)), dev(s)
    xd = dev(np.pad(x, ((0, 0), (0, ldx_pad))))[:, :k]
    yd_full = torch.full((m, n + ldy_pad), 7.0, dtype=torch.float32, device="cuda")
    w4.w4_gemv_sym128(qw, sd, xd, out=yd_full[:, :n])
    y = to_np(yd_full)
    assert np.all(y[:, n:] == 7.0), "write outside y"
    y_ref, bound = oracle.gemv_ref(oracle.pack(q), s, None, x, group=128)
    ok, worst = oracle.check_bound(y[:, :n], y_ref, bound, RTOL)
    assert ok, f"(M,N,K)=({m},{n},{k}) worst err/bound {worst:.3g}"
    return q, s, x, qw, sd, y[:, :n]


@pytest.mark.parametrize("m", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("n,k", [(1, 128), (3, 256), (257, 896), (70, 2048), (33, 2176), (5, 11008)])
def test_sym128_gemv(w4, m, n, k):
    sym_case(w4, m, n, k, seed=500 * m + n + k, ldx_pad=8 * (m % 2), ldy_pad=m % 3)


@pytest.mark.parametrize("m", [1, 2, 3, 4, 16])
@pytest.mark.parametrize("n,k", [(2560, 2048), (22016, 2048), (2048, 11008)])
def test_sym128_gemv_equals_affine_kernel_with_bias_minus_8s(w4, m, n, k):
    # w = s (q - 8) is the affine weight with b = -8 s (exact), so with each scale repeated over
    # its two 64-groups the affine kernel must give the same bits
    q, s, x, qw, sd, y = sym_case(w4, m, n, k, seed=n + k + m)
    s64 = np.repeat(s, 2, axis=1)
    b64 = (-8.0 * s64.astype(np.float64)).astype(np.float16)
    y_aff = to_np(w4.w4_gemv(qw, dev(s64), dev(b64), dev(x)))
    assert np.array_equal(y.view(np.uint32), y_aff.view(np.uint32))


@pytest.mark.parametrize("n,k", [(1, 128), (64, 256), (100, 384), (11008, 2048), (2048, 11008)])
def test_sym128_dequant_bit_exact(w4, n, k):
    q, s = synth.w4_sym128_weights(n, k, seed=n * 3 + k)
    got = to_np(w4.w4_dequant_f16_t_sym128(w4.w4_pack(dev(q)), dev(s))).view(np.uint16)
    assert np.array_equal(got, oracle.dequant_f16_t(oracle.pack(q), s, None, group=128))


def test_sym128_worked_values(w4):
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "sym128_handworked.json")) as f:
        gold = json.load(f)
    # bit patterns: one row per case, the case's code at k = 5 and code 8 elsewhere
    cases = gold["dequant"]
    q = np.full((len(cases), 128), 8, dtype=np.uint8)
    s = np.zeros((len(cases), 1), dtype=np.uint16)
    for i, c in enumerate(cases):
        q[i, 5] = c["q"]
        s[i, 0] = int(c["s"], 16)
    wt = to_np(w4.w4_dequant_f16_t_sym128(w4.w4_pack(dev(q)), dev(s.view(np.float16)))).view(np.uint16)
    for i, c in enumerate(cases):
        assert int(wt[5, i]) == int(c["w"], 16), c
        assert int(wt[0, i]) == 0, c
    # hand-worked GEMVs
    pats = {"mod16": lambda k: np.arange(k) % 16, "rev16": lambda k: 15 - np.arange(k) % 16}
    for c in gold["gemv"]:
        k = c["K"]
        kind = c["q"].split()
        qq = (np.full(k, int(kind[1])) if kind[0] == "const" else pats[kind[0]](k)).astype(np.uint8)[None, :]
        xs = []
        for p_ in c["x"]:
            a = p_.split()
            if a[0] == "const":
                xs.append(np.full(k, float(a[1])))
            elif a[0] == "alt":
                xs.append(np.where(np.arange(k) % 2 == 0, 1.0, -1.0))
            else:
                v = np.zeros(k)
                v[int(a[1])] = 1.0
                xs.append(v)
        x = np.stack(xs).astype(np.float16)
        y = to_np(w4.w4_gemv_sym128(w4.w4_pack(dev(qq)), dev(np.array([c["s"]], dtype=np.float16)), dev(x)))
        assert np.array_equal(y[:, 0].astype(np.float64), np.array(c["y"])), c["name"]


# ----------------------------------------------------------------------------- GEMV


def gemv_case(w4, m, n, k, seed, x_override=None, ldx_pad=0, ldy_pad=0):
    q, s, b = synth.w4_weights(n, k, seed=seed)
    x = synth.activations(m, k, seed=seed) if x_override is None else x_override
    qw, sd, bd = upload_layer(w4, q, s, b)
    xd_full = dev(np.pad(x, ((0, 0), (0, ldx_pad))))
    xd = xd_full[:, :k]
    yd_full = torch.full((m, n + ldy_pad), 7.0, dtype=torch.float32, device="cuda")
    yd = yd_full[:, :n]
    w4.w4_gemv(qw, sd, bd, xd, out=yd)
    y = to_np(yd_full)
    if ldy_pad:
        assert np.all(y[:, n:] == 7.0), "write outside y"
    y_ref, bound = oracle.gemv_ref(oracle.pack(q), s, b, x)
    ok, worst = oracle.check_bound(y[:, :n], y_ref, bound, RTOL)
    assert ok, f"(M,N,K)=({m},{n},{k}) worst err/bound {worst:.3g}"
    return worst


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 11, 16])
@pytest.mark.parametrize("n,k", [(1, 64), (3, 128), (257, 960), (70, 2048), (33, 2112), (5, 11008)])
def test_gemv_small_shapes(w4, m, n, k):
    gemv_case(w4, m, n, k, seed=1000 * m + n + k)


@pytest.mark.parametrize("n", [2048, 2049, 2050, 3071, 3072, 3073])
def test_gemv_rows_per_wave_edges(w4, n):
    # one-slice rows at M = 1 take 3 rows per wave from 2049 to 3072 rows, 2 on either side;
    # 2050, 3071 and 3073 end in a partial block of rows
    gemv_case(w4, 1, n, 2048, seed=n)


@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("n,k", [(37, 16448), (9, 20480)])
def test_gemv_rows_past_16384(w4, m, n, k):
    # rows of more than 8 slices of 2048 take the general team kernel (M <= 2) or the matrix
    # cores (M >= 3)
    gemv_case(w4, m, n, k, seed=7 * n + k + m, ldx_pad=8 * (m % 2), ldy_pad=m % 3)


def test_gemv_strided_x_and_y(w4):
    gemv_case(w4, 3, 129, 384, seed=5, ldx_pad=24, ldy_pad=5)
    gemv_case(w4, 1, 64, 1024, seed=6, ldx_pad=8, ldy_pad=1)


def test_gemv_zero_rows_are_exactly_zero(w4):
    x = synth.activations(4, 256, seed=7)
    x[1] = 0
    x[3] = 0
    q, s, b = synth.w4_weights(50, 256, seed=7)
    qw, sd, bd = upload_layer(w4, q, s, b)
    y = to_np(w4.w4_gemv(qw, sd, bd, dev(x)))
    assert not y[1].any() and not y[3].any()


def test_gemv_closed_form_constant_codes(w4):
    # q = c, s = 1, b = 0  ->  y = c * sum(x)
    k, n = 896, 40
    x = synth.activations(2, k, seed=8)
    for c in (0, 5, 15):
        q = np.full((n, k), c, np.uint8)
        s = np.ones((n, k // 64), np.float16)
        b = np.zeros((n, k // 64), np.float16)
        qw, sd, bd = upload_layer(w4, q, s, b)
        y = to_np(w4.w4_gemv(qw, sd, bd, dev(x)))
        want = c * x.astype(np.float64).sum(axis=1)
        bound = c * np.abs(x.astype(np.float64)).sum(axis=1)
        assert np.all(np.abs(y - want[:, None]) <= RTOL * bound[:, None])


def test_gemv_cancelling_weights_are_exactly_zero(w4):
    # q = 8 with b = -8 s: every weight is exactly 0, so y must be exactly 0 (bound 0)
    k, n = 2048, 96
    x = synth.activations(5, k, seed=17)
    _, s, _ = synth.w4_weights(n, k, seed=17)
    b = (-8.0 * s.astype(np.float64)).astype(np.float16)
    q = np.full((n, k), 8, np.uint8)
    qw, sd, bd = upload_layer(w4, q, s, b)
    y = to_np(w4.w4_gemv(qw, sd, bd, dev(x)))
    assert not y.any()
    # and a mix: half the groups cancel, half do not
    q[:, : k // 2] = synth.codes(n, k // 2, seed=18)
    qw, sd, bd = upload_layer(w4, q, s, b)
    y = to_np(w4.w4_gemv(qw, sd, bd, dev(x)))
    y_ref, bound = oracle.gemv_ref(oracle.pack(q), s, b, x)
    assert oracle.check_bound(y, y_ref, bound, RTOL)[0]


def test_gemv_single_config_full(w4):
    # single W4A16 GEMV (M, N, K) = (1, 4864, 896), seed 0
    q, s, b = synth.w4_weights(4864, 896, seed=0, workload=synth.W_SINGLE)
    x = synth.activations(1, 896, seed=0, workload=synth.W_SINGLE)
    qw, sd, bd = upload_layer(w4, q, s, b)
    y = to_np(w4.w4_gemv(qw, sd, bd, dev(x)))
    y_ref, bound = oracle.gemv_ref(oracle.pack(q), s, b, x)
    ok, worst = oracle.check_bound(y, y_ref, bound, RTOL)
    assert ok, worst


def _fused(layer, groups):
    """Row-concatenated shapes of matrices that read the same x (q|k|v, gate|up)."""
    shape = {name: (n, k) for name, n, k in layer}
    return {(sum(shape[g][0] for g in grp), shape[grp[0]][1]) for grp in groups if all(g in shape for g in grp)}


WORKLOAD_SHAPES = sorted({(n, k) for _, n, k in synth.QWEN25_3B_LAYER}
                         | {(n, k) for _, n, k in synth.QWEN3_1P7B_CLASSIFY}
                         | {(n, k) for _, n, k in synth.GEMMA12B_LAYER}
                         | _fused(synth.QWEN25_3B_LAYER, [["q", "k", "v"], ["gate", "up"]])
                         | _fused(synth.QWEN3_1P7B_CLASSIFY, [["q", "k", "v"], ["gate", "up"]])
                         | _fused(synth.GEMMA12B_LAYER, [["gate", "up"]]))


@pytest.mark.parametrize("n,k", WORKLOAD_SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 4, 8, 16])
def test_gemv_workload_shapes_full(w4, m, n, k):
    gemv_case(w4, m, n, k, seed=n * 7 + k + m)


@pytest.mark.parametrize("m", [3, 5, 16])
@pytest.mark.parametrize("n,k", [(12290, 320), (6150, 448), (100, 8256), (17, 64), (383 * 16 + 1, 192)])
def test_gemv_matrix_core_edges(w4, m, n, k):
    # from five rows of x on, the GEMV runs on matrix cores in 16-row blocks grouped by 1, 2 or
    # 4 per wave; these shapes leave the last group partly filled in each grouping, end rows on
    # a half step (K % 128 == 64) and give some waves of the K split no step at all (at M = 3
    # the same shapes run on row slices of 4 rows with three rows of x)
    gemv_case(w4, m, n, k, seed=31 * n + k + m, ldx_pad=8 * (m % 2), ldy_pad=m % 5)


# Long rows on few row blocks split K two ways across workgroups, partial sums added by a
# second launch in split order: the 2048-row down projections (Qwen3-1.7B at M = 16, Qwen2.5-3B
# at M = 8), a ragged one (rows past the last 16-row block, K ending mid-step, 13 rows of x)
# and M = 3 past the row slices' 16384 elements.  Workspaces start filled with 0xFF bytes; a
# second call must give the same bits.
@pytest.mark.parametrize("m,n,k", [(16, 2048, 6144), (8, 2048, 11008), (13, 2000, 6208), (3, 300, 20480)])
def test_gemv_k_split_across_workgroups(w4, m, n, k):
    need = w4.gemv_workspace_bytes(m, n, k)
    assert need == 2 * m * n * 4
    q, s, b = synth.w4_weights(n, k, seed=n + k)
    x = synth.activations(m, k, seed=m + k)
    qw, sd, bd = upload_layer(w4, q, s, b)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    y1 = to_np(w4.w4_gemv(qw, sd, bd, dev(x), workspace=ws))
    y2 = to_np(w4.w4_gemv(qw, sd, bd, dev(x), workspace=ws))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    y_ref, bound = oracle.gemv_ref(oracle.pack(q), s, b, x)
    ok, worst = oracle.check_bound(y1, y_ref, bound, RTOL)
    assert ok, worst


# Matrices of 24 MB of codes and more at 5 <= M <= 8 stage each workgroup's x rows and its
# rows' scales/biases in LDS: ragged rows (the last 16-row block holds one row, in a pair of
# blocks per wave), rows ending on a half step (K % 128 == 64), 13 K-ranges added by a second
# launch (workspace filled with 0xFF first; a repeat must give the same bits), and the
# symmetric group-128 format.  Strided x and y with canary columns.
@pytest.mark.parametrize("m,n,k,sym", [
    (5, 24001, 2112, False), (8, 24001, 2112, False), (7, 1000, 51200, False), (6, 24001, 2176, True),
])
def test_gemv_staged_large_matrices(w4, m, n, k, sym):
    if sym:
        sym_case(w4, m, n, k, seed=n + k + m, ldx_pad=8, ldy_pad=4)
        return
    need = w4.gemv_workspace_bytes(m, n, k)
    q, s, b = synth.w4_weights(n, k, seed=n + k)
    x = synth.activations(m, k, seed=m + k)
    qw, sd, bd = upload_layer(w4, q, s, b)
    ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device="cuda")
    xd = dev(np.pad(x, ((0, 0), (0, 8))))[:, :k]
    yfull = torch.full((m, n + 4), 7.0, dtype=torch.float32, device="cuda")
    w4.w4_gemv(qw, sd, bd, xd, out=yfull[:, :n], workspace=ws)
    y1 = to_np(yfull).copy()
    assert np.all(y1[:, n:] == 7.0), "write outside y"
    w4.w4_gemv(qw, sd, bd, xd, out=yfull[:, :n], workspace=ws)
    assert np.array_equal(y1.view(np.uint32), to_np(yfull).view(np.uint32))
    y_ref, bound = oracle.gemv_ref(oracle.pack(q), s, b, x)
    ok, worst = oracle.check_bound(y1[:, :n], y_ref, bound, RTOL)
    assert ok, f"(M,N,K)=({m},{n},{k}) worst err/bound {worst:.3g}"


def _sampled_rows(n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(min(n, 8)), np.arange(max(0, n - 8), n),
                                     rng.choice(n, min(n, 48), replace=False)]))


# M = 1 runs on row slices of 64 chunks (2048 elements of K), 1 to 8 slices per row in one
# workgroup, with 2, 3 or 4 rows per wave chosen from the number of (row, slice) units.  These
# shapes give every slice count, a partly filled last slice, rows-per-wave tails (N not a
# multiple of the rows per wave) and the unit thresholds of each rows-per-wave choice.
ROW_SLICE_SHAPES = [(5, 1088), (16001, 2048), (30001, 2048), (101, 2112), (4099, 4160), (1000, 6208),
                    (7501, 8256), (3, 10304), (33, 13312), (7, 14400), (257, 16384), (1025, 16320)]


@pytest.mark.parametrize("n,k", ROW_SLICE_SHAPES)
def test_gemv_m1_row_slices(w4, n, k):
    q, s, b = synth.w4_weights(n, k, seed=n + 3 * k)
    x = synth.activations(1, k, seed=n + 3 * k)
    qw, sd, bd = upload_layer(w4, q, s, b)
    y = to_np(w4.w4_gemv(qw, sd, bd, dev(x)))
    rows = _sampled_rows(n, n + k)
    y_ref, bound = oracle.gemv_ref(oracle.pack(q[rows]), s[rows], b[rows], x)
    ok, worst = oracle.check_bound(y[:, rows], y_ref, bound, RTOL)
    assert ok, f"(1,{n},{k}) worst err/bound {worst:.3g}"


def test_gemv_codes_past_2gb(w4):
    # 262147 x 16384: 2.15 GB of packed codes, so the last rows lie past 2^31 bytes (each wave's
    # buffers start at its own rows).  The matrix is drawn on the device (uniform codes, scales
    # and biases as in the workload recipe); sampled rows are checked against the oracle.
    n, k = 262147, 16384
    g = torch.Generator(device="cuda").manual_seed(2024)
    qw = torch.randint(-2 ** 31, 2 ** 31, (n, k // 8), dtype=torch.int32, device="cuda", generator=g)
    s = (torch.randn((n, k // 64), device="cuda", generator=g).abs() * 0.02 + 1e-3).to(torch.float16)
    b = (-8.0 * s.float() + torch.randn((n, k // 64), device="cuda", generator=g) * 0.002).to(torch.float16)
    x = synth.activations(2, k, seed=2024)
    y1 = to_np(w4.w4_gemv(qw, s, b, dev(x[:1])))   # M = 1 and M = 2 (both rows of x per wave)
    y2 = to_np(w4.w4_gemv(qw, s, b, dev(x)))
    rows = _sampled_rows(n, 2024)
    rows_d = torch.from_numpy(rows).cuda()
    q_h = to_np(qw.index_select(0, rows_d)).view(np.uint32)
    y_ref, bound = oracle.gemv_ref(q_h, to_np(s.index_select(0, rows_d)), to_np(b.index_select(0, rows_d)), x)
    del qw, s, b
    ok, worst = oracle.check_bound(y1[:, rows], y_ref[:1], bound[:1], RTOL)
    assert ok, f"M = 1 worst err/bound {worst:.3g}"
    ok, worst = oracle.check_bound(y2[:, rows], y_ref, bound, RTOL)
    assert ok, f"M = 2 worst err/bound {worst:.3g}"


@pytest.mark.parametrize("n,k", [(5, 1152), (16001, 2048), (101, 2176), (7501, 8320), (257, 16384)])
def test_sym128_m1_row_slices_equal_affine_bits(w4, n, k):
    # the symmetric format on the row-slice kernel: against the oracle on sampled rows, and bit
    # for bit against the affine kernel with b = -8 s (the same weights)
    q, s = synth.w4_sym128_weights(n, k, seed=n + k)
    x = synth.activations(1, k, seed=n + k)
    qw, sd = w4.w4_pack(dev(q)), dev(s)
    y = to_np(w4.w4_gemv_sym128(qw, sd, dev(x)))
    rows = _sampled_rows(n, n + 2 * k)
    y_ref, bound = oracle.gemv_ref(oracle.pack(q[rows]), s[rows], None, x, group=128)
    ok, worst = oracle.check_bound(y[:, rows], y_ref, bound, RTOL)
    assert ok, f"(1,{n},{k}) worst err/bound {worst:.3g}"
    s64 = np.repeat(s, 2, axis=1)
    b64 = (-8.0 * s64.astype(np.float64)).astype(np.float16)
    y_aff = to_np(w4.w4_gemv(qw, dev(s64), dev(b64), dev(x)))
    assert np.array_equal(y.view(np.uint32), y_aff.view(np.uint32))


def test_gemv_deterministic(w4):
    q, s, b = synth.w4_weights(2048, 2048, seed=9)
    x = synth.activations(3, 2048, seed=9)
    qw, sd, bd = upload_layer(w4, q, s, b)
    xd = dev(x)
    y1 = to_np(w4.w4_gemv(qw, sd, bd, xd))
    y2 = to_np(w4.w4_gemv(qw, sd, bd, xd))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


# ------------------------------------------------------------------------- dequant


@pytest.mark.parametrize("n,k", [(1, 64), (7, 192), (65, 128), (257, 960), (100, 2112), (2048, 11008), (11008, 2048)])
def test_dequant_bit_exact(w4, n, k):
    q, s, b = synth.w4_weights(n, k, seed=n + 3 * k)
    qw, sd, bd = upload_layer(w4, q, s, b)
    got = to_np(w4.w4_dequant_f16_t(qw, sd, bd)).view(np.uint16)
    assert np.array_equal(got, oracle.dequant_f16_t(oracle.pack(q), s, b))


def test_dequant_strided_output(w4):
    n, k = 40, 256
    q, s, b = synth.w4_weights(n, k, seed=11)
    qw, sd, bd = upload_layer(w4, q, s, b)
    full = torch.full((k, n + 8), -1.0, dtype=torch.float16, device="cuda")
    w4.w4_dequant_f16_t(qw, sd, bd, out=full[:, :n])
    got = to_np(full).view(np.uint16)
    assert np.array_equal(got[:, :n], oracle.dequant_f16_t(oracle.pack(q), s, b))
    assert np.all(got[:, n:] == np.float16(-1.0).view(np.uint16))


def test_dequant_rounding_pins(w4):
    # the hand-derived rounding cases (tests/golden/f16_dequant.json) through the GPU
    import json, os
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "f16_dequant.json")))["cases"]
    n = len(cases)
    q = np.zeros((n, 64), np.uint8)
    s = np.zeros((n, 1), np.uint16)
    b = np.zeros((n, 1), np.uint16)
    for i, c in enumerate(cases):
        q[i, 5] = c["q"]
        s[i, 0] = int(c["s"], 16)
        b[i, 0] = int(c["b"], 16)
    qw, sd, bd = upload_layer(w4, q, s.view(np.float16), b.view(np.float16))
    got = to_np(w4.w4_dequant_f16_t(qw, sd, bd)).view(np.uint16)
    for i, c in enumerate(cases):
        assert got[5, i] == int(c["w"], 16), c
        assert got[0, i] == int(c["b"], 16), c


def test_dequant_random_scales_full_f16_range(w4):
    # scales and biases drawn over the whole finite f16 range with subnormals
    r = np.random.default_rng(12)
    n, k = 300, 128
    q = synth.codes(n, k, seed=12)
    s = r.integers(0, 0x7BFF, size=(n, 2)).astype(np.uint16)
    b = r.integers(0, 0xFBFF, size=(n, 2)).astype(np.uint16)
    b[(b & 0x7C00) == 0x7C00] = 0
    s[:50] = r.integers(0, 0x0400, size=(50, 2))  # subnormal scales
    b[:50] = r.integers(0, 0x0400, size=(50, 2)) | 0x8000
    w = oracle.dequant_exact(oracle.pack(q), s.view(np.float16), b.view(np.float16))
    keep = np.all(np.abs(w) < 65504, axis=1)
    q, s, b = q[keep], s[keep], b[keep]
    qw, sd, bd = upload_layer(w4, q, s.view(np.float16), b.view(np.float16))
    got = to_np(w4.w4_dequant_f16_t(qw, sd, bd)).view(np.uint16)
    assert np.array_equal(got, oracle.dequant_f16_t(oracle.pack(q), s.view(np.float16), b.view(np.float16)))


# ---------------------------------------------------------------------------- GEMM


def gemm_case(w4, m, n, k, seed, lda_pad=0, ldb_pad=0, ldc_pad=0, a=None, bmat=None):
    a = synth.activations(m, k, seed=seed) if a is None else a
    bmat = synth.activations(k, n, seed=seed + 1) if bmat is None else bmat
    ad = dev(np.pad(a, ((0, 0), (0, lda_pad))))[:, :k]
    bd = dev(np.pad(bmat, ((0, 0), (0, ldb_pad))))[:, :n]
    cfull = torch.full((m, n + ldc_pad), 3.0, dtype=torch.float32, device="cuda")
    w4.gemm_f16(ad, bd, out=cfull[:, :n])
    c = to_np(cfull)
    if ldc_pad:
        assert np.all(c[:, n:] == 3.0)
    c_ref, bound = oracle.gemm_ref(a, bmat)
    ok, worst = oracle.check_bound(c[:, :n], c_ref, bound, RTOL)
    assert ok, f"(M,N,K)=({m},{n},{k}) worst {worst:.3g}"
    return c[:, :n]


@pytest.mark.parametrize("m,n,k", [
    (9, 8, 8), (33, 264, 72), (130, 520, 200), (257, 1000, 2056), (128, 256, 32), (1570, 264, 64),
    (300, 2048, 1000), (17, 8, 4096), (300, 1000, 2048), (513, 520, 96), (40, 2056, 32),
])
def test_gemm_mfma_path(w4, m, n, k):
    gemm_case(w4, m, n, k, seed=m + n + k)


# The small-M path gives each lane 8, 4 or 2 columns, whichever spreads the workgroups (64
# lanes x columns each) most evenly over 256 CUs: 131064 columns take 8 (256 workgroups, the
# last one ragged), 65528 take 4, the others 2.
@pytest.mark.parametrize("m,n,k", [(1, 8, 8), (3, 1032, 2048), (8, 4096, 256), (5, 520, 3840), (1, 4752, 2048),
                                   (1, 131064, 64), (4, 131072, 32), (2, 65528, 128), (1, 65536, 72)])
def test_gemm_small_m_path(w4, m, n, k):
    gemm_case(w4, m, n, k, seed=m + n + k)


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (16, 1, 2048), (3, 5, 7), (20, 3, 100), (2, 13, 64),
                                   # 8 consecutive k per thread: several row blocks, a partial
                                   # second round of 2048 k, one thread's worth of k
                                   (40, 2, 4104), (17, 1, 8)])
def test_gemm_plain_path(w4, m, n, k):
    gemm_case(w4, m, n, k, seed=m + n + k)


@pytest.mark.parametrize("lda_pad", [8, 1])
def test_gemm_plain_path_strided_a(w4, lda_pad):
    # rows of A 16-byte aligned (8 consecutive k per thread) or not (k strided by 256)
    gemm_case(w4, 33, 3, 1000, seed=lda_pad, lda_pad=lda_pad, ldc_pad=1)


def test_gemm_strided_operands(w4):
    gemm_case(w4, 40, 128, 96, seed=1, lda_pad=8, ldb_pad=16, ldc_pad=3)
    gemm_case(w4, 2, 256, 64, seed=2, lda_pad=8, ldb_pad=8, ldc_pad=1)


def test_gemm_identity_is_exact(w4):
    a = synth.activations(70, 64, seed=3)
    c = gemm_case(w4, 70, 64, 64, seed=3, a=a, bmat=np.eye(64, dtype=np.float16))
    assert np.array_equal(c, a.astype(np.float32))


def test_gemm_head_column_slice_full_vocabulary(w4):
    # the batched-classify step at full width: 16 rows x the yes/no columns of the
    # [2048][151936] f16 head (B = H + id, ldb = 151936), then the per-row argmax over the two
    k, v, m = synth.QWEN25_3B_HIDDEN, synth.QWEN25_3B_VOCAB, synth.CLASSIFY_ROWS
    h = synth.head_f16(k, v, seed=5)
    ids = synth.class_ids(v)
    x = synth.activations(m, k, seed=5)
    hd, xd = dev(h), dev(x)
    out = torch.empty((m, 2), dtype=torch.float32, device="cuda")
    for j, i in enumerate(ids):
        w4.gemm_f16(xd, hd[:, i:i + 1], out=out[:, j:j + 1])
    idx, _ = w4.logits_argmax_topk(out, 1)
    c = to_np(out)
    c_ref, bound = oracle.gemm_ref(x, h[:, list(ids)])
    assert oracle.check_bound(c, c_ref, bound, RTOL)[0]
    assert oracle.check_topk_vs_exact(c_ref, to_np(idx), 1)[0]


def test_gemm_head_column_slice(w4):
    # two columns of an f16 head read through B = H + id with ldb = V (plain path)
    k, v = 2048, 4099
    h = synth.head_f16(k, v, seed=4)
    x = synth.activations(16, k, seed=4)
    hd, xd = dev(h), dev(x)
    ids = (17, 4098)
    out = torch.empty((16, 2), dtype=torch.float32, device="cuda")
    for j, i in enumerate(ids):
        w4.gemm_f16(xd, hd[:, i:i + 1], out=out[:, j:j + 1])
    c = to_np(out)
    c_ref, bound = oracle.gemm_ref(x, h[:, list(ids)])
    assert oracle.check_bound(c, c_ref, bound, RTOL)[0]


@pytest.mark.parametrize("m,k,v", [(1, 2048, 151936), (8, 2048, 151936), (1, 3840, 262144), (8, 3840, 262144)])
def test_gemm_head_full(w4, m, k, v):
    # Every logit of the f16 LM heads at their real shapes (the decode head, speculative
    # verify's 8 rows, the Gemma-shaped head at M = 1 and 8: the small-M kernel with 2 and 8
    # columns per lane) against fp64, checked in column blocks.
    x = synth.activations(m, k, seed=m + v)
    head = synth.head_f16(k, v, seed=k + v)
    logits = to_np(w4.gemm_f16(dev(x), dev(head)))
    worst = 0.0
    for c0 in range(0, v, 16384):
        c_ref, bound = oracle.gemm_ref(x, head[:, c0:c0 + 16384])
        ok, wr = oracle.check_bound(logits[:, c0:c0 + 16384], c_ref, bound, RTOL)
        assert ok, (c0, wr)
        worst = max(worst, wr)


def test_gemm_prefill_sampled_rows(w4):
    # (M, N, K) = (1570, 11008, 2048): 128 sampled rows incl. the M tail 1536..1569
    m, n, k = 1570, 11008, 2048
    a = synth.activations(m, k, seed=5)
    bmat = synth.activations(k, n, seed=6)
    c = to_np(w4.gemm_f16(dev(a), dev(bmat)))
    rows = np.unique(np.concatenate([np.random.default_rng(5).choice(1536, 94, replace=False),
                                     np.arange(1536, 1570)]))
    c_ref, bound = oracle.gemm_ref(a[rows], bmat)
    ok, worst = oracle.check_bound(c[rows], c_ref, bound, RTOL)
    assert ok, worst


@pytest.mark.parametrize("m,n,k,seed", [(1570, 22016, 2048, 7), (1570, 2048, 11008, 9)])
def test_gemm_prefill_full(w4, m, n, k, seed):
    # Every output of a prefill GEMM at the step's sizes (so the step's launch configuration:
    # 320-row tiles, and split-K with its reduce for the 11008-long K) against fp64, on the
    # dequantized scratch of synthetic int4 weights (the oracle's own dequant as B).
    a = synth.activations(m, k, seed=seed)
    q, sc, b = synth.w4_weights(n, k, seed=seed + 1)
    wt = w4.w4_dequant_f16_t(w4.w4_pack(dev(q)), dev(sc), dev(b))
    c = to_np(w4.gemm_f16(dev(a), wt))
    wt_ref = oracle.dequant_f16_t(oracle.pack(q), sc, b)
    c_ref, bound = oracle.gemm_ref(a, wt_ref.view(np.float16))
    ok, worst = oracle.check_bound(c, c_ref, bound, RTOL)
    assert ok, worst


@pytest.mark.parametrize("m,n,k,sampled", [
    (600, 25608, 64, False),    # 320-row tiles (2 row tiles instead of 3), ragged M and N
    (600, 11000, 2048, True),   # 320-row tiles with K split in two, ragged N
])
def test_gemm_tall_tiles(w4, m, n, k, sampled):
    a = synth.activations(m, k, seed=m + n)
    bmat = synth.activations(k, n, seed=k + 1)
    c = to_np(w4.gemm_f16(dev(a), dev(bmat)))
    rows = np.arange(m)
    if sampled:
        rows = np.unique(np.concatenate([np.random.default_rng(m).choice(576, 40, replace=False),
                                         np.arange(576, m)]))
    c_ref, bound = oracle.gemm_ref(a[rows], bmat)
    ok, worst = oracle.check_bound(c[rows], c_ref, bound, RTOL)
    assert ok, worst


# Several rounds of 256-row output tiles over the 256 CUs (471, 471 and 472 tiles: the last
# round partly filled), ragged in M and N, with 2, 3 and 32 K-tiles of 32 per tile.
@pytest.mark.parametrize("m,n,k,sampled", [
    (600, 40000, 64, False), (700, 40000, 96, False), (1000, 30000, 1024, True),
])
def test_gemm_multi_round(w4, m, n, k, sampled):
    a = synth.activations(m, k, seed=m + k)
    bmat = synth.activations(k, n, seed=n + 3)
    c = to_np(w4.gemm_f16(dev(a), dev(bmat)))
    rows = np.arange(m)
    if sampled:  # the last row tile (768..999) whole, 40 rows of the others
        rows = np.unique(np.concatenate([np.random.default_rng(m).choice(768, 40, replace=False),
                                         np.arange(768, m)]))
    c_ref, bound = oracle.gemm_ref(a[rows], bmat)
    ok, worst = oracle.check_bound(c[rows], c_ref, bound, RTOL)
    assert ok, worst


def test_gemm_prefill_deterministic(w4):
    # the prefill gate|up shape (two rounds of 320-row tiles): bit-identical on repeat
    m, n, k = 1570, 22016, 2048
    a = dev(synth.activations(m, k, seed=11))
    b = dev(synth.activations(k, n, seed=12))
    c1 = to_np(w4.gemm_f16(a, b))
    c2 = to_np(w4.gemm_f16(a, b))
    assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32))


def test_gemm_deterministic(w4):
    a = dev(synth.activations(300, 512, seed=7))
    b = dev(synth.activations(512, 1024, seed=8))
    c1 = to_np(w4.gemm_f16(a, b))
    c2 = to_np(w4.gemm_f16(a, b))
    assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32))


# ---------------------------------------------------------------------------- top-k


def topk_case(w4, logits, k):
    ld = dev(logits)
    idx, val = w4.logits_argmax_topk(ld, k)
    idx, val = to_np(idx), to_np(val)
    ok = oracle.check_topk_selection(logits, idx, val, k)
    assert ok, (logits.shape, k)


@pytest.mark.parametrize("m,v,k", [
    (1, 1, 1), (1, 2, 1), (16, 2, 1), (3, 5, 5), (2, 100, 40), (1, 4096, 64), (2, 4097, 64),
    (1, 151936, 40), (8, 262144, 64), (1, 262144, 256), (4, 9000, 256), (1, 40000, 1),
    # last chunk nearly empty (padding fills most of its top-k), 8192-logit chunks, odd k
    (2, 12293, 64), (3, 4099, 40), (1, 600000, 64), (1, 70000, 63), (2, 8191, 17),
    # either side of the switch to two offered keys per lane (k > 48)
    (1, 300000, 48), (3, 300000, 49), (2, 4096, 49),
    # 8192 group keys after pre-reduction, the most the selection holds in registers
    (1, 1048576, 64),
])
def test_topk_random(w4, m, v, k):
    logits = (np.random.default_rng(m * v + k).standard_normal((m, v)) * 0.9).astype(np.float32)
    topk_case(w4, logits, k)


def test_topk_sorted_and_tied_chunks(w4):
    # logits whose chunk winners arrive as aligned sorted lists (every 4096-chunk a ramp), and a
    # long run of ties: the second pass must stay exact whatever the candidates' layout
    v = 262144
    ramp = np.tile(np.arange(4096, dtype=np.float32) / 4096.0, v // 4096)
    ties = np.full(v, 0.5, np.float32)
    ties[::1000] = 0.75
    lg = np.stack([ramp, ties, ramp[::-1].copy()])
    for k in (40, 64):
        idx, val = w4.logits_argmax_topk(dev(lg), k)
        assert oracle.check_topk_selection(lg, to_np(idx), to_np(val), k)


def test_topk_ties_and_signed_zero(w4):
    r = np.random.default_rng(13)
    v = 10000
    rows = [
        np.zeros(v, np.float32),                                   # all equal
        np.where(r.random(v) < 0.5, np.float32(-0.0), np.float32(0.0)),  # +-0 mixed
        np.round(r.standard_normal(v) * 2).astype(np.float32),     # many duplicates
        np.repeat(np.arange(v // 100, dtype=np.float32), 100)[::-1].copy(),  # runs straddling k
        -np.abs(r.standard_normal(v)).astype(np.float32),           # all negative
    ]
    logits = np.stack(rows)
    for k in (1, 7, 64, 100, 101, 256):
        topk_case(w4, logits, k)


def test_topk_strided_rows(w4):
    logits = np.random.default_rng(14).standard_normal((3, 6000)).astype(np.float32)
    full = dev(np.pad(logits, ((0, 0), (0, 13))))
    idx, val = w4.logits_argmax_topk(full[:, :6000], 33)
    assert oracle.check_topk_selection(logits, to_np(idx), to_np(val), 33)


def test_int4_head_topk(w4):
    # the LM head in the int4 format ([vocab][hidden]), GEMV to logits then top-40
    v, kdim = 151936, 2048
    q, s, b = synth.w4_weights(v, kdim, seed=71)
    x = synth.activations(1, kdim, seed=72)
    qw, sd, bd = upload_layer(w4, q, s, b)
    logits = w4.w4_gemv(qw, sd, bd, dev(x))
    idx, val = w4.logits_argmax_topk(logits, 40)
    lg = to_np(logits)
    rows = np.sort(np.random.default_rng(73).choice(v, 256, replace=False))
    y_ref, bound = oracle.gemv_ref(oracle.pack(q[rows]), s[rows], b[rows], x)
    assert oracle.check_bound(lg[:, rows], y_ref, bound, RTOL)[0]
    assert oracle.check_topk_selection(lg, to_np(idx), to_np(val), 40)


def test_speculative_verify_argmax(w4):
    # draft positions verified greedily: 8 rows through the f16 head, then a per-row argmax
    m, kdim, v = 8, 2048, 151936
    x = synth.activations(m, kdim, seed=61)
    head = synth.head_f16(kdim, v, seed=62)
    logits = w4.gemm_f16(dev(x), dev(head))
    idx, val = w4.logits_argmax_topk(logits, 1)
    lg = to_np(logits)
    assert oracle.check_topk_selection(lg, to_np(idx), to_np(val), 1)
    c_ref, _ = oracle.gemm_ref(x, head)
    assert oracle.check_topk_vs_exact(c_ref, to_np(idx), 1)[0]


def test_topk_deterministic(w4):
    logits = dev(np.round(np.random.default_rng(15).standard_normal((2, 151936)) * 4).astype(np.float32))
    a = [to_np(t) for t in w4.logits_argmax_topk(logits, 40)]
    b = [to_np(t) for t in w4.logits_argmax_topk(logits, 40)]
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def _bound_row(v, groups, per_group, seed):
    # background far below 7; per_group[i] values of [7, 7.25) (ties among them) in group
    # groups[i] (64 logits each)
    r = np.random.default_rng(seed)
    row = (r.standard_normal(v) * 0.1).astype(np.float32)
    j = 0
    for g, c in zip(groups, per_group):
        pos = g * 64 + r.choice(64, c, replace=False)
        row[pos] = 7.0 + (np.arange(j, j + c) % 8) / 32.0
        j += c
    return row


@pytest.mark.parametrize("ngroups,total", [(256, 256), (257, 257), (40, 256), (40, 257)])
def test_topk_group_bound_edges(w4, ngroups, total):
    # the selection's switches on 151936-logit rows at k = 40: every value of [7, 7.5) has the
    # same first radix digit, so the first-digit bound admits `ngroups` groups (up to 256 are
    # taken as they are, more make it find the exact k-th group key) holding `total` candidates
    # (up to 256 are ranked directly, more go through a second radix select); the second row is
    # ordinary logits
    v = 151936
    r = np.random.default_rng(ngroups * 1000 + total)
    groups = np.sort(r.choice(v // 64, ngroups, replace=False))
    per = np.full(ngroups, total // ngroups)
    per[: total % ngroups] += 1
    rows = np.stack([_bound_row(v, groups, per, ngroups + total),
                     (r.standard_normal(v) * 0.9).astype(np.float32)])
    topk_case(w4, rows, 40)


def test_topk_prereduced_groups_adversarial(w4):
    # 600000 logits at k = 64: group keys combined in pairs (128-logit groups) before the
    # selection; all-equal (exact k-th group key, then a second select over 8192 candidates),
    # a ramp (the first-digit bound admits far more than k candidates) and a row whose top
    # values are one repeated value in 70 groups, beside ordinary logits
    v, r = 600000, np.random.default_rng(17)
    ramp = (np.arange(v, dtype=np.float32) / v)[::-1].copy()
    rep = (r.standard_normal(v) * 0.1).astype(np.float32)
    rep[np.sort(r.choice(v // 128, 70, replace=False)) * 128 + 5] = 3.0
    rows = np.stack([np.full(v, 0.25, np.float32), ramp, rep, (r.standard_normal(v) * 0.9).astype(np.float32)])
    topk_case(w4, rows, 64)


# ------------------------------------------------------------- a small decode step


def test_decode_step_small_end_to_end(w4):
    # W4 GEMV -> f16 head -> top-k, checked against fp64 logits with the near-tie rule
    k_hidden, v, n = 512, 5000, 512
    q, s, b = synth.w4_weights(n, k_hidden, seed=16)
    x = synth.activations(1, k_hidden, seed=16)
    h = synth.head_f16(n, v, seed=16)
    qw, sd, bd = upload_layer(w4, q, s, b)
    y = w4.w4_gemv(qw, sd, bd, dev(x))
    y16 = y.to(torch.float16)  # the head consumes f16 activations
    logits = w4.gemm_f16(y16, dev(h))
    idx, val = w4.logits_argmax_topk(logits, 40)
    idx, val, lg = to_np(idx), to_np(val), to_np(logits)
    assert np.array_equal(val.view(np.uint32), lg[0, idx[0]][None].view(np.uint32))
    # the oracle's own chain on the host inputs: fp64 GEMV, f16 rounding, fp64 head
    y_ref, _ = oracle.gemv_ref(oracle.pack(q), s, b, x)
    exact, _ = oracle.gemm_ref(y_ref.astype(np.float16), h)
    ok, loose = oracle.check_topk_vs_exact(exact, idx, 40)
    assert ok, loose
