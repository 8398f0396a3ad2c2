"""The seeded input generator draws what the workloads specify (CPU only).

The distributions are those of the int4 workloads: x f16 of N(0, 1); codes uniform on 0..15;
scales f16 of |N(0, 0.02)| + 1e-3; biases f16 of -8 s + N(0, 0.002) on the stored s; an f16 head
of N(0, 0.02).  Each is checked against closed-form moments at a few standard errors, and the
head's logits against their closed-form spread sqrt(K) * 0.02 (0.905 at K = 2048, 1.239 at K =
3840).  The generator holds none of the layer's arithmetic, so these pin the inputs, not the
method.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import synth

SQ2PI = math.sqrt(2.0 / math.pi)


def test_codes_are_uniform_on_0_to_15():
    q = synth.codes(4096, 2048, seed=0, workload=synth.W_DECODE, layer=4)
    assert q.dtype == np.uint8 and q.min() == 0 and q.max() == 15
    counts = np.bincount(q.ravel(), minlength=16).astype(np.float64)
    expect = q.size / 16.0
    chi2 = float(((counts - expect) ** 2 / expect).sum())
    # 15 degrees of freedom: P(chi2 > 44.3) = 1e-4
    assert chi2 < 44.3, chi2


def test_scale_and_bias_moments():
    n, k = 8192, 8192  # 1M groups
    s, b = synth.scales_biases(n, k, seed=0, workload=synth.W_DECODE, layer=4)
    assert s.dtype == np.float16 and b.dtype == np.float16 and s.shape == (n, k // 64)
    s64 = s.astype(np.float64)
    cnt = s64.size
    mean_s, sd_s = 0.02 * SQ2PI + 1e-3, 0.02 * math.sqrt(1.0 - 2.0 / math.pi)  # half-normal, shifted
    assert s64.min() >= 1e-3 * (1 - 2.0 ** -11)       # |N| + 1e-3, rounded to f16 once
    assert abs(s64.mean() - mean_s) < 5 * sd_s / math.sqrt(cnt)
    assert abs(s64.std() / sd_s - 1.0) < 0.01
    # b + 8 s is the N(0, 0.002) noise, up to one f16 rounding of b (|error| <= 2^-12 * |b|)
    noise = b.astype(np.float64) + 8.0 * s64
    assert abs(noise.mean()) < 5 * 0.002 / math.sqrt(cnt)
    assert abs(noise.std() / 0.002 - 1.0) < 0.01
    assert np.all(np.abs(noise) < 0.002 * 6 + 2.0 ** -12 * np.abs(b.astype(np.float64)))
    # the bias centres on -8 E[s]
    assert abs(b.astype(np.float64).mean() + 8.0 * mean_s) < 5 * 8.0 * sd_s / math.sqrt(cnt)


def test_activation_and_head_moments():
    x = synth.activations(256, 4096, seed=0, workload=synth.W_PREFILL, layer=1)
    assert x.dtype == np.float16
    xs = x.astype(np.float64)
    assert abs(xs.mean()) < 5 / math.sqrt(xs.size)
    assert abs(xs.std() - 1.0) < 0.005
    h = synth.head_f16(512, 8192, seed=0, workload=synth.W_DECODE, layer=999)
    hs = h.astype(np.float64)
    assert abs(hs.mean()) < 5 * 0.02 / math.sqrt(hs.size)
    assert abs(hs.std() / 0.02 - 1.0) < 0.005


def test_head_rows_regenerate_as_slices():
    full = synth.head_f16(64, 3000, seed=5, workload=synth.W_TEST, layer=2)
    part = synth.head_f16(64, 3000, seed=5, workload=synth.W_TEST, layer=2, rows=slice(17, 40))
    assert np.array_equal(full[17:40], part)


@pytest.mark.parametrize("k", [2048, 3840])
def test_logit_spread_is_sqrt_k_times_0p02(k):
    # logits of one N(0,1) row through an N(0, 0.02) head: given x, each logit is N(0, 0.02^2 |x|^2),
    # and |x|^2 = K within a few sqrt(2K); over 16384 columns the sample spread is within 1 %
    v = 16384
    h = synth.head_f16(k, v, seed=0, workload=synth.W_DECODE, layer=999).astype(np.float64)
    x = synth.activations(1, k, seed=0, workload=synth.W_DECODE, layer=998).astype(np.float64)
    logits = x @ h
    sigma = math.sqrt(k) * 0.02
    assert abs(logits.std() / sigma - 1.0) < 0.04, (logits.std(), sigma)
    assert abs(logits.mean()) < 5 * sigma / math.sqrt(v)
