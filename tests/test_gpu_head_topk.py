"""GPU parity of w4_gemv_topk, the int4 LM head with token selection on the device in one call.

Logits: each within 2e-3 * sum |w x| of the oracle's fp64 sum (every row of the small shapes,
sampled rows of the vocabulary-sized ones); the call's GEMV is w4_gemv's M = 1 kernel, so its
logits must equal w4_gemv's bit for bit.  Selection: exact on the logits the call wrote (the oracle's stable top-k of those f32
values, indices and value bits), and against the fp64 logits by the near-tie rule.  Also ties,
a workspace full of garbage, two calls sharing one workspace, and sentinel bands around every
output.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

RTOL = 2e-3
BAND = 256


@pytest.fixture(scope="module")
def w4():
    import int4_weight_only_group_amd as m
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def banded(n, dtype, sentinel):
    full = torch.full((n + 2 * BAND,), sentinel, dtype=dtype, device="cuda")
    return full[BAND:BAND + n], full


def bands_ok(full, n, sentinel):
    f = full.cpu()
    s = torch.full((BAND,), sentinel, dtype=full.dtype)
    return bool(torch.equal(f[:BAND], s) and torch.equal(f[BAND + n:], s))


def head_case(w4, v, kdim, k, seed, rows=None, q=None, s=None, b=None, x=None, ws_fill=None):
    if q is None:
        q, s, b = synth.w4_weights(v, kdim, seed=seed)
    if x is None:
        x = synth.activations(1, kdim, seed=seed + 1)
    qw, sd, bd = w4.w4_pack(dev(q)), dev(s), dev(b)
    logits, fl = banded(v, torch.float32, -77.0)
    idx, fi = banded(k, torch.int32, -3)
    val, fv = banded(k, torch.float32, 55.5)
    need = w4.gemv_topk_workspace_bytes(v, kdim, k)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    if ws_fill is not None:
        ws.copy_(torch.from_numpy(np.random.default_rng(ws_fill).integers(0, 256, need, dtype=np.uint8)).cuda())
    w4.w4_gemv_topk(qw, sd, bd, dev(x), k, logits=logits, idx=idx, val=val, workspace=ws)
    torch.cuda.synchronize()
    assert bands_ok(fl, v, -77.0) and bands_ok(fi, k, -3) and bands_ok(fv, k, 55.5), "write outside an output"
    lg, ix, vl = logits.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy()
    # logits: w4_gemv's at M = 1, bit for bit
    y = w4.w4_gemv(qw, sd, bd, dev(x))
    assert np.array_equal(y.cpu().numpy()[0].view(np.uint32), lg.view(np.uint32))
    # selection: exact on the logits the call wrote
    assert oracle.check_topk_selection(lg[None], ix[None], vl[None], k), (v, kdim, k)
    # logits against fp64 (every row, or a sample)
    r = np.arange(v) if rows is None else rows
    y_ref, bound = oracle.gemv_ref(oracle.pack(q[r]), s[r], b[r], x)
    ok, worst = oracle.check_bound(lg[None, r], y_ref, bound, RTOL)
    assert ok, f"(V,K)=({v},{kdim}) worst err/bound {worst:.3g}"
    return (qw, sd, bd, x), lg, ix, vl


@pytest.mark.parametrize("v,kdim,k", [
    (1, 64, 1), (5, 64, 5), (37, 128, 7), (64, 960, 40), (1000, 2048, 40), (4099, 960, 64),
    (65, 4096, 64), (3001, 3840, 49), (70001, 2112, 17), (16384 + 3, 2048, 48), (262144, 128, 64),
])
def test_head_topk_small_and_ragged(w4, v, kdim, k):
    head_case(w4, v, kdim, k, seed=v + kdim + k)


@pytest.mark.parametrize("k", [1, 40, 64])
def test_head_topk_qwen_head_equals_separate_calls(w4, k):
    # the Qwen2.5-3B-sized int4 head: [151936][2048], k = 40 as in the decode step
    v, kdim = synth.QWEN25_3B_VOCAB, synth.QWEN25_3B_HIDDEN
    rows = np.sort(np.random.default_rng(5).choice(v, 512, replace=False))
    (qw, sd, bd, x), lg, ix, vl = head_case(w4, v, kdim, k, seed=71, rows=rows)
    y = w4.w4_gemv(qw, sd, bd, dev(x))
    i2, v2 = w4.logits_argmax_topk(y, k)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy()[0].view(np.uint32), lg.view(np.uint32))
    assert np.array_equal(i2.cpu().numpy()[0], ix)
    assert np.array_equal(v2.cpu().numpy()[0].view(np.uint32), vl.view(np.uint32))


def test_head_topk_long_rows_and_fp64_margin(w4):
    # rows of two slices (K = 3840, the Gemma-shaped hidden size), k = 64
    v, kdim, k = 65536, 3840, 64
    q, s, b = synth.w4_weights(v, kdim, seed=81)
    x = synth.activations(1, kdim, seed=82)
    rows = np.sort(np.random.default_rng(6).choice(v, 256, replace=False))
    _, lg, ix, _ = head_case(w4, v, kdim, k, seed=81, rows=rows, q=q, s=s, b=b, x=x)
    # end to end against the fp64 logits of the selected rows and their neighbours in rank
    top = np.argsort(-lg, kind="stable")[:k + 64]
    y_ref, _ = oracle.gemv_ref(oracle.pack(q[top]), s[top], b[top], x)
    full = np.full((1, v), -np.inf)
    full[0, top] = y_ref[0]
    ok, _ = oracle.check_topk_vs_exact(full, ix[None], k)
    assert ok


def test_head_topk_ties_go_to_the_lower_index(w4):
    # every row identical: all logits equal, so the top-k are rows 0..k-1 in order
    v, kdim, k = 9000, 256, 64
    q1, s1, b1 = synth.w4_weights(1, kdim, seed=91)
    q, s, b = np.repeat(q1, v, 0), np.repeat(s1, v, 0), np.repeat(b1, v, 0)
    _, lg, ix, vl = head_case(w4, v, kdim, k, seed=91, q=q, s=s, b=b)
    assert np.all(lg == lg[0])
    assert np.array_equal(ix, np.arange(k))
    # runs of equal rows straddling the k-th rank
    q2, s2, b2 = synth.w4_weights(v // 100, kdim, seed=92)
    q, s, b = np.repeat(q2, 100, 0), np.repeat(s2, 100, 0), np.repeat(b2, 100, 0)
    head_case(w4, v, kdim, 40, seed=92, q=q, s=s, b=b)


def test_head_topk_ignores_workspace_contents_and_reuses_it(w4):
    v, kdim, k = 151936, 2048, 40
    a = head_case(w4, 20000, kdim, k, seed=101, ws_fill=1)
    b = head_case(w4, 20000, kdim, k, seed=101, ws_fill=2)
    assert np.array_equal(a[2], b[2]) and np.array_equal(a[3].view(np.uint32), b[3].view(np.uint32))
    # two calls in a row on one workspace, the second smaller
    q, s, bb = synth.w4_weights(v, kdim, seed=102)
    x = synth.activations(1, kdim, seed=103)
    ws = torch.empty(w4.gemv_topk_workspace_bytes(v, kdim, k), dtype=torch.uint8, device="cuda")
    outs = []
    for n in (v, 5003):
        lg, ix, vl = w4.w4_gemv_topk(w4.w4_pack(dev(q[:n])), dev(s[:n]), dev(bb[:n]), dev(x), k, workspace=ws)
        torch.cuda.synchronize()
        assert oracle.check_topk_selection(lg.cpu().numpy()[None], ix.cpu().numpy()[None], vl.cpu().numpy()[None], k)
        outs.append(ix.cpu().numpy())
    ref = np.argsort(-w4.w4_gemv(w4.w4_pack(dev(q[:5003])), dev(s[:5003]), dev(bb[:5003]), dev(x)).cpu().numpy()[0],
                     kind="stable")[:k]
    assert np.array_equal(outs[1], ref)
