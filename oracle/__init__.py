"""CPU oracle for the group-wise affine int4 weight-only linear layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
NumPy/fp64 restatement of what the GPU library computes.  Only the tests, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import it.  The HIP library and its Python binding never import, call or link
anything here, and nothing here imports them: the two share no code.

Sources (page title, then section):
  * "The inference engine -- Mojo 1.0 on Metal" (millfolio):
      - "Crossing Mojo 1.0": the multi-row decode GEMV, the dequantize-once
        prefill into a transposed half-precision scratch followed by an f16
        GEMM, and on-device argmax/top-k that saves the per-token logits
        download.
      - "What's inside the engine today": GPU token selection that is
        bit-exact against a host reference; the LM head that streamed
        bf16 weights of shape [2048 x 151936].
      - "Appendix: the remaining gap, itemized": MLX's affine 4-bit format.
      - "Where it fits": weights quantized to int4 at load (the quantizer).
  * "Engineering investigation: can this MLX port become another 10x faster?"
      - "Selective quantization ...": affine quantization with group size 64.
  * "engine-mlx", "Tech details": in-graph greedy argmax.

The weight format (fixed for this library, the plainest reading of the
affine group-64 format above): 64-element groups along K; 4-bit codes
q in 0..15, eight per little-endian uint32 word with element 8j+i of a row in
bits 4i..4i+3 of word j (low nibble first); one f16 scale s and one f16 bias b
per (row, group); the weight is w = s*q + b.

Every function of :mod:`oracle.w4ref` is pinned by CPU tests to closed forms,
hand-derived fixtures (``tests/golden``), exact rational brute force or
textbook routines; no function is "parity unpinned".
"""

from .w4ref import (  # noqa: F401
    GROUP,
    pack,
    pack_loop,
    unpack,
    unpack_loop,
    f16_bits,
    f16_bits_struct,
    f16_value,
    dequant_exact,
    dequant_f16_t,
    quantize,
    quantize_loop,
    gemv_ref,
    gemm_ref,
    topk_ref,
    topk_ref_loop,
    check_bound,
    check_topk_selection,
    check_topk_vs_exact,
)
