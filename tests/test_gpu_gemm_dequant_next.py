"""gemm_f16_dequant_next: the GEMM of one prefill weight and the dequant-transpose of the next in
one call.  C must equal gemm_f16's and wt w4_dequant_f16_t's bit for bit; wt is checked against
the oracle bit for bit, C on sampled rows against the oracle's fp64 product within 2e-3 of the
per-output bound.  Outputs start as garbage (NaN / 0xFFFF) and sit inside padded buffers whose
padding must stay untouched.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

RTOL = 2e-3
PAD = 8  # columns of padding right of every output row


@pytest.fixture(scope="module")
def w4():
    import int4_weight_only_group_amd as m
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# (M, N, K) of the GEMM, (Nq, Kq) of the dequant.  On 256 CUs: 430 workgroups of 320 x 256 with
# 82 CUs idle in the second round (the 1570-token prefill: gate|up GEMM beside the down
# projection's dequant, 9 tiles per side group); split-K (192 workgroups, 64 idle) beside a
# dequant of ragged N (2-byte stores); 472 and 471 tiles (40 and 41 idle) beside a single tile
# and beside the 11008 x 2048 dequant (17 tiles per side group, K long enough to hide them);
# then shapes that take two launches: the same dequant beside a short GEMM (it would not finish
# within the last round), 256 tiles (no idle CU), 32-row tiles and the small-M path.
CASES = [
    (1570, 22016, 2048, 2048, 11008),
    (600, 2048, 4096, 1000, 320),
    (1000, 30000, 1024, 64, 64),
    (700, 40000, 4096, 11008, 2048),
    (1000, 30000, 256, 2048, 11008),
    (4096, 4096, 4096, 300, 512),
    (20, 4096, 512, 130, 256),
    (4, 1024, 512, 128, 256),
]


def _run(w4, m, n, k, nq, kq, seed):
    a = synth.activations(m, k, seed=seed)
    bmat = synth.activations(k, n, seed=seed + 1)
    q, s, b = synth.w4_weights(nq, kq, seed=seed + 2)
    ad, bd = dev(a), dev(bmat)
    qw, sd, bd_ = w4.w4_pack(dev(q)), dev(s), dev(b)
    cfull = torch.full((m, n + PAD), float("nan"), dtype=torch.float32, device="cuda")
    wfull = torch.full((kq, nq + PAD), -1, dtype=torch.int16, device="cuda").view(torch.float16)
    c, wt = w4.gemm_f16_dequant_next(ad, bd, qw, sd, bd_, out=cfull[:, :n], wt=wfull[:, :nq])
    c_sep = w4.gemm_f16(ad, bd)
    wt_sep = w4.w4_dequant_f16_t(qw, sd, bd_)
    cf, wf = to_np(cfull), to_np(wfull).view(np.uint16)
    assert np.all(np.isnan(cf[:, n:])), "C padding written"
    assert np.all(wf[:, nq:] == 0xFFFF), "wt padding written"
    c_np, wt_np = cf[:, :n], wf[:, :nq]
    assert np.array_equal(c_np.view(np.uint32), to_np(c_sep).view(np.uint32))
    assert np.array_equal(wt_np, to_np(wt_sep).view(np.uint16))
    return a, bmat, q, s, b, c_np, wt_np


@pytest.mark.parametrize("m,n,k,nq,kq", CASES)
def test_gemm_dequant_next_equals_separate_calls_and_oracle(w4, m, n, k, nq, kq):
    a, bmat, q, s, b, c, wt = _run(w4, m, n, k, nq, kq, seed=m + nq)
    assert np.array_equal(wt, oracle.dequant_f16_t(oracle.pack(q), s, b))
    rng = np.random.default_rng(m + n)
    tail = np.arange(max(0, m - 34), m)  # the last row tile's tail
    rows = np.unique(np.concatenate([rng.choice(m, min(m, 30), replace=False), tail]))
    c_ref, bound = oracle.gemm_ref(a[rows], bmat)
    ok, worst = oracle.check_bound(c[rows], c_ref, bound, RTOL)
    assert ok, f"(M,N,K)=({m},{n},{k}) worst {worst:.3g}"


def test_gemm_dequant_next_repeat_is_bit_identical(w4):
    # twice at the prefill shape, the second over the first call's outputs
    m, n, k, nq, kq = 1570, 22016, 2048, 2048, 11008
    ad = dev(synth.activations(m, k, seed=31))
    bd = dev(synth.activations(k, n, seed=32))
    q, s, b = synth.w4_weights(nq, kq, seed=33)
    qw, sd, bd_ = w4.w4_pack(dev(q)), dev(s), dev(b)
    c1, wt1 = w4.gemm_f16_dequant_next(ad, bd, qw, sd, bd_)
    c1, wt1 = to_np(c1).copy(), to_np(wt1).copy()
    c2 = torch.empty((m, n), dtype=torch.float32, device="cuda")
    wt2 = torch.empty((kq, nq), dtype=torch.float16, device="cuda")
    for _ in range(2):
        w4.gemm_f16_dequant_next(ad, bd, qw, sd, bd_, out=c2, wt=wt2)
    assert np.array_equal(c1.view(np.uint32), to_np(c2).view(np.uint32))
    assert np.array_equal(wt1.view(np.uint16), to_np(wt2).view(np.uint16))


def test_gemm_dequant_next_rejects_overlap(w4):
    # wt inside the GEMM's B operand: refused on the host, nothing written
    m, n, k = 600, 2048, 256
    ad = dev(synth.activations(m, k, seed=41))
    big = dev(synth.activations(k + 64, n, seed=42))
    q, s, b = synth.w4_weights(n, 64, seed=43)
    before = to_np(big).copy()
    with pytest.raises(w4.W4Error):
        w4.gemm_f16_dequant_next(ad, big[:k], w4.w4_pack(dev(q)), dev(s), dev(b), wt=big[k - 32:k + 32])
    assert np.array_equal(to_np(big).view(np.uint16), before.view(np.uint16))


def test_gemm_dequant_next_graph_replays(w4):
    # captured in a HIP graph (as the prefill phase is) and replayed three times with eager work
    # and a synchronisation between the replays; every replay must equal the separate calls
    m, n, k, nq, kq = 700, 40000, 96, 2048, 2048
    ad = dev(synth.activations(m, k, seed=51))
    bd = dev(synth.activations(k, n, seed=52))
    q, s, b = synth.w4_weights(nq, kq, seed=53)
    qw, sd, bd_ = w4.w4_pack(dev(q)), dev(s), dev(b)
    c_ref = to_np(w4.gemm_f16(ad, bd)).copy()
    wt_ref = to_np(w4.w4_dequant_f16_t(qw, sd, bd_)).view(np.uint16).copy()
    c = torch.empty((m, n), dtype=torch.float32, device="cuda")
    wt = torch.empty((kq, nq), dtype=torch.float16, device="cuda")
    ws = torch.empty(max(16, w4.gemm_workspace_bytes(ad, bd)), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        w4.gemm_f16_dequant_next(ad, bd, qw, sd, bd_, out=c, wt=wt, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w4.gemm_f16_dequant_next(ad, bd, qw, sd, bd_, out=c, wt=wt, workspace=ws)
    for r in range(3):
        c.fill_(float("nan"))
        wt.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        got_c, got_wt = to_np(c), to_np(wt).view(np.uint16)
        assert np.array_equal(got_c.view(np.uint32), c_ref.view(np.uint32)), f"replay {r}: C"
        assert np.array_equal(got_wt, wt_ref), f"replay {r}: wt"
        w4.gemm_f16(ad[:64], bd)  # eager work between the replays


@pytest.mark.parametrize("m,n,k,nq,kq", [(1570, 22016, 2048, 2048, 11008), (600, 2048, 4096, 1000, 384),
                                         (1000, 30000, 256, 2048, 11008)])
def test_gemm_dequant_next_sym128(w4, m, n, k, nq, kq):
    # the symmetric group-128 next weight: in the idle CUs (the prefill shape; split-K beside a
    # ragged dequant) or as two launches (a short GEMM); bit-equal to the separate calls, wt
    # bit-exact against the oracle
    a = synth.activations(m, k, seed=m + 61)
    bmat = synth.activations(k, n, seed=62)
    q, s = synth.w4_sym128_weights(nq, kq, seed=63)
    ad, bd = dev(a), dev(bmat)
    qw, sd = w4.w4_pack(dev(q)), dev(s)
    cfull = torch.full((m, n + PAD), float("nan"), dtype=torch.float32, device="cuda")
    wfull = torch.full((kq, nq + PAD), -1, dtype=torch.int16, device="cuda").view(torch.float16)
    w4.gemm_f16_dequant_next_sym128(ad, bd, qw, sd, out=cfull[:, :n], wt=wfull[:, :nq])
    cf, wf = to_np(cfull), to_np(wfull).view(np.uint16)
    assert np.all(np.isnan(cf[:, n:])) and np.all(wf[:, nq:] == 0xFFFF), "padding written"
    assert np.array_equal(cf[:, :n].view(np.uint32), to_np(w4.gemm_f16(ad, bd)).view(np.uint32))
    wt_sep = to_np(w4.w4_dequant_f16_t_sym128(qw, sd)).view(np.uint16)
    assert np.array_equal(wf[:, :nq], wt_sep)
    assert np.array_equal(wf[:, :nq], oracle.dequant_f16_t(oracle.pack(q), s, None, group=128))


@pytest.mark.parametrize("sym", [False, True])
def test_gemm_dequant_next_odd_scratch_pitch(w4, sym):
    # wt rows 1001 elements apart (not 16-byte aligned): the side dequant takes its 2-byte stores;
    # split-K GEMM (64 idle CUs) beside a ragged dequant, bit-equal to the separate calls
    m, n, k, nq, kq = 600, 2048, 4096, 1000, 384
    ad = dev(synth.activations(m, k, seed=71))
    bd = dev(synth.activations(k, n, seed=72))
    if sym:
        q, s = synth.w4_sym128_weights(nq, kq, seed=73)
        qw, sd = w4.w4_pack(dev(q)), dev(s)
    else:
        q, s, b = synth.w4_weights(nq, kq, seed=73)
        qw, sd, bd_ = w4.w4_pack(dev(q)), dev(s), dev(b)
    wfull = torch.full((kq, nq + 1), -1, dtype=torch.int16, device="cuda").view(torch.float16)
    if sym:
        c, _ = w4.gemm_f16_dequant_next_sym128(ad, bd, qw, sd, wt=wfull[:, :nq])
        ref = oracle.dequant_f16_t(oracle.pack(q), s, None, group=128)
    else:
        c, _ = w4.gemm_f16_dequant_next(ad, bd, qw, sd, bd_, wt=wfull[:, :nq])
        ref = oracle.dequant_f16_t(oracle.pack(q), s, b)
    wf = to_np(wfull).view(np.uint16)
    assert np.all(wf[:, nq] == 0xFFFF), "padding column written"
    assert np.array_equal(wf[:, :nq], ref)
    assert np.array_equal(to_np(c).view(np.uint32), to_np(w4.gemm_f16(ad, bd)).view(np.uint32))
