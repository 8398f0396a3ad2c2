"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and names workload shapes.  It holds none
of the layer's arithmetic (no packing, dequantization, products or selection),
so both the CPU oracle and the GPU library can consume its buffers without
sharing code.

Value distributions (one independent PCG64 stream per tensor, keyed by
``(seed, workload, layer, tensor)``; draw order inside a tensor is fixed):
  * activations x: f16 of N(0, 1);
  * codes q: uniform integers 0..15 (uint8, row-major [N][K]);
  * scales s: f16 of |N(0, 0.02)| + 1e-3, one per (row, 64-group);
  * biases b: f16 of (-8 * s + N(0, 0.002)), using the stored f16 s;
  * f16 head H [K][V]: f16 of N(0, 0.02).
The shapes are those of the int4 Qwen2.5-3B / Qwen3-1.7B / Gemma-12B layers the
pages run ("The inference engine -- Mojo 1.0 on Metal": "Where it fits",
"Crossing Mojo 1.0", "What's inside the engine today").
"""

from __future__ import annotations

import numpy as np

GROUP = 64

# Workload ids used as the second key of every random stream.
W_SINGLE, W_DECODE, W_PREFILL, W_CLASSIFY, W_GEMMA, W_TEST = 0, 1, 2, 3, 4, 9

# Tensor ids (fourth key).
T_Q, T_S, T_B, T_X, T_HEAD, T_IDS, T_W = 0, 1, 2, 3, 4, 5, 6

# (name, N, K) of the int4 projections of one Qwen2.5-3B decoder layer.
QWEN25_3B_LAYER = (
    ("q", 2048, 2048), ("k", 256, 2048), ("v", 256, 2048), ("o", 2048, 2048),
    ("gate", 11008, 2048), ("up", 11008, 2048), ("down", 2048, 11008),
)
QWEN25_3B_LAYERS = 36
QWEN25_3B_VOCAB = 151936
QWEN25_3B_HIDDEN = 2048

PREFILL_TOKENS = 1570
PREFILL_MATS = (("gate", 11008, 2048), ("up", 11008, 2048), ("down", 2048, 11008))

QWEN3_1P7B_CLASSIFY = (
    ("q", 2048, 2048), ("k", 1024, 2048), ("v", 1024, 2048),
    ("gate", 6144, 2048), ("up", 6144, 2048), ("down", 2048, 6144),
)
CLASSIFY_ROWS = 16

GEMMA12B_LAYER = (("gate", 15360, 3840), ("up", 15360, 3840), ("down", 3840, 15360), ("q", 4096, 3840))
GEMMA12B_VOCAB = 262144
GEMMA12B_HIDDEN = 3840


def rng(seed: int, workload: int, layer: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([seed, workload, layer, tensor])


def codes(n: int, k: int, *, seed: int = 0, workload: int = W_TEST, layer: int = 0) -> np.ndarray:
    """Uniform 4-bit codes, uint8 [n][k]."""
    return rng(seed, workload, layer, T_Q).integers(0, 16, size=(n, k), dtype=np.uint8)


def scales_biases(n: int, k: int, *, seed: int = 0, workload: int = W_TEST,
                  layer: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """f16 scales |N(0,0.02)|+1e-3 and biases -8*s+N(0,0.002), each [n][k/64]."""
    assert k % GROUP == 0
    g = k // GROUP
    s = (np.abs(rng(seed, workload, layer, T_S).standard_normal((n, g))) * 0.02 + 1e-3).astype(np.float16)
    noise = rng(seed, workload, layer, T_B).standard_normal((n, g)) * 0.002
    b = (-8.0 * s.astype(np.float64) + noise).astype(np.float16)
    return s, b


def w4_weights(n: int, k: int, *, seed: int = 0, workload: int = W_TEST,
               layer: int = 0) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(q uint8 [n][k], s f16 [n][k/64], b f16 [n][k/64]) for one int4 matrix."""
    q = codes(n, k, seed=seed, workload=workload, layer=layer)
    s, b = scales_biases(n, k, seed=seed, workload=workload, layer=layer)
    return q, s, b


def w4_sym128_weights(n: int, k: int, *, seed: int = 0, workload: int = W_TEST,
                      layer: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """(q uint8 [n][k], s f16 [n][k/128]) of the symmetric group-128 format: uniform codes and
    scales |N(0,0.02)| + 1e-3, the affine format's distributions without the bias."""
    assert k % 128 == 0
    q = codes(n, k, seed=seed, workload=workload, layer=layer)
    s = (np.abs(rng(seed, workload, layer, T_S).standard_normal((n, k // 128))) * 0.02 + 1e-3).astype(np.float16)
    return q, s


def activations(m: int, k: int, *, seed: int = 0, workload: int = W_TEST, layer: int = 0) -> np.ndarray:
    """f16 of N(0,1), [m][k]."""
    return rng(seed, workload, layer, T_X).standard_normal((m, k)).astype(np.float16)


def head_f16(k: int, v: int, *, seed: int = 0, workload: int = W_TEST, layer: int = 0,
             rows: slice | None = None) -> np.ndarray:
    """f16 of N(0, 0.02), [k][v] (V contiguous).  Drawn row by row, so a slice of
    rows can be regenerated without the whole matrix."""
    r = rng(seed, workload, layer, T_HEAD)
    lo, hi = (0, k) if rows is None else (rows.start or 0, rows.stop if rows.stop is not None else k)
    out = np.empty((hi - lo, v), dtype=np.float16)
    chunk = max(1, (1 << 24) // v)
    for r0 in range(0, hi, chunk):
        r1 = min(hi, r0 + chunk)
        block = r.standard_normal((r1 - r0, v), dtype=np.float32)
        a, b = max(r0, lo), r1
        if a < b:
            out[a - lo:b - lo] = (block[a - r0:b - r0] * np.float32(0.02)).astype(np.float16)
    return out


def float_weights(n: int, k: int, *, seed: int = 0, workload: int = W_TEST, layer: int = 0) -> np.ndarray:
    """f16 of N(0, 0.02), [n][k]: unquantized weights, the input of the load-time quantizer."""
    w = rng(seed, workload, layer, T_W).standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    return w.astype(np.float16)


def class_ids(vocab: int, *, seed: int = 0, workload: int = W_CLASSIFY) -> tuple[int, int]:
    """Two distinct token ids standing in for the yes/no answer tokens."""
    a, b = rng(seed, workload, 0, T_IDS).choice(vocab, size=2, replace=False)
    return int(a), int(b)
