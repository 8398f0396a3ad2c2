"""Writes stay inside their outputs: every output of the entry points that has no strided form
(packed codes, the quantizer's codes, scales and biases, top-k indices and values) is placed
inside a larger buffer whose bands before and after it hold a sentinel, and the bands must come
back untouched.  The outputs themselves are checked against the oracle as in the parity tests.
Also the classify head's yes/no columns at the real vocabulary width (B = H + id, ldb = 151936).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BAND = 1024  # elements of sentinel before and after each output


@pytest.fixture(scope="module")
def w4():
    import int4_weight_only_group_amd as m
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def banded(shape, dtype, sentinel):
    """A contiguous view of `shape` in the middle of a buffer with BAND sentinel elements on
    each side; returns (view, full buffer)."""
    n = int(np.prod(shape))
    full = torch.full((n + 2 * BAND,), sentinel, dtype=dtype, device="cuda")
    return full[BAND:BAND + n].view(*shape), full


def bands_intact(full, n, sentinel):
    torch.cuda.synchronize()
    f = full.cpu()
    lo, hi = f[:BAND], f[BAND + n:]
    s = torch.full_like(lo, sentinel)
    return bool(torch.equal(lo, s) and torch.equal(hi, s))


@pytest.mark.parametrize("n,k", [(1, 64), (37, 960), (257, 2048), (2048, 11008)])
def test_pack_output_bands(w4, n, k):
    q = synth.codes(n, k, seed=3 * n + k)
    qw, full = banded((n, k // 8), torch.int32, -0x2A2A2A2B)
    w4.w4_pack(dev(q), out=qw)
    assert bands_intact(full, n * k // 8, -0x2A2A2A2B)
    assert np.array_equal(qw.cpu().numpy().view(np.uint32), oracle.pack(q))


@pytest.mark.parametrize("n,k", [(1, 64), (33, 960), (257, 2048), (100, 11008)])
def test_quantize_output_bands(w4, n, k):
    w = synth.float_weights(n, k, seed=n + k)
    qw, fq = banded((n, k // 8), torch.int32, -0x2A2A2A2B)
    s, fs = banded((n, k // 64), torch.float16, -7.0)
    b, fb = banded((n, k // 64), torch.float16, -7.0)
    w4.w4_quantize(dev(w), out=(qw, s, b))
    assert bands_intact(fq, n * k // 8, -0x2A2A2A2B)
    assert bands_intact(fs, n * k // 64, -7.0)
    assert bands_intact(fb, n * k // 64, -7.0)
    qw_ref, s_ref, b_ref = oracle.quantize(w)
    assert np.array_equal(qw.cpu().numpy().view(np.uint32), qw_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint16), s_ref.view(np.uint16))
    assert np.array_equal(b.cpu().numpy().view(np.uint16), b_ref.view(np.uint16))


@pytest.mark.parametrize("m,v,k", [(1, 5, 5), (1, 4096, 40), (1, 151936, 40), (8, 262144, 64), (3, 9000, 256),
                                   (16, 2, 1)])
def test_topk_output_bands(w4, m, v, k):
    logits = (np.random.default_rng(v + k).standard_normal((m, v)) * 0.9).astype(np.float32)
    idx, fi = banded((m, k), torch.int32, -5)
    val, fv = banded((m, k), torch.float32, 1234.5)
    w4.logits_argmax_topk(dev(logits), k, idx=idx, val=val)
    assert bands_intact(fi, m * k, -5)
    assert bands_intact(fv, m * k, 1234.5)
    assert oracle.check_topk_selection(logits, idx.cpu().numpy(), val.cpu().numpy(), k)


def test_classify_head_columns_at_full_vocabulary(w4):
    # the batched-classify head step: 16 rows x the yes/no columns of the f16 head [2048][151936],
    # each column read through B = H + id with ldb = 151936 (the plain path), then argmax over 2
    k, v = synth.QWEN25_3B_HIDDEN, synth.QWEN25_3B_VOCAB
    h = synth.head_f16(k, v, seed=0, workload=synth.W_CLASSIFY, layer=999)
    x = synth.activations(synth.CLASSIFY_ROWS, k, seed=0, workload=synth.W_CLASSIFY, layer=998)
    ids = synth.class_ids(v)
    hd, xd = dev(h), dev(x)
    out, fo = banded((synth.CLASSIFY_ROWS, 2), torch.float32, -99.0)
    for j, i in enumerate(ids):
        w4.gemm_f16(xd, hd[:, i:i + 1], out=out[:, j:j + 1])
    idx, val = w4.logits_argmax_topk(out, 1)
    assert bands_intact(fo, 2 * synth.CLASSIFY_ROWS, -99.0)
    c = out.cpu().numpy()
    c_ref, bound = oracle.gemm_ref(x, h[:, list(ids)])
    assert oracle.check_bound(c, c_ref, bound, 2e-3)[0]
    assert oracle.check_topk_selection(c, idx.cpu().numpy(), val.cpu().numpy(), 1)
    ok, _ = oracle.check_topk_vs_exact(c_ref, idx.cpu().numpy(), 1)
    assert ok
