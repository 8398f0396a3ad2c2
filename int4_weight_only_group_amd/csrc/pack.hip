// w4_pack: 4-bit codes (one per byte) -> eight codes per uint32, low nibble first.
//
// The packed layout is the affine 4-bit weight format ("The inference engine -- Mojo 1.0
// on Metal", "Appendix: the remaining gap, itemized": MLX's affine 4-bit; group size 64 in
// "Engineering investigation ...", "Selective quantization").  Packing happens once, at
// load ("Where it fits": "quantized to int4 at load").
//
// Both arrays are row-major with K contiguous and K % 64 == 0, so the whole matrix is one
// flat stream: byte i of q lands in nibble i % 8 of word i / 8.  Each thread turns 32 code
// bytes (two 16-byte loads) into four words (one 16-byte store); HBM-bound.
#include "w4_internal.h"

namespace w4 {

__device__ __forceinline__ uint32_t pack8(uint32_t lo4, uint32_t hi4) {
  // lo4 holds codes 0..3 (one per byte), hi4 codes 4..7.  Keep the low nibble of each
  // byte, then fold byte pairs together: code i goes to bits 4i..4i+3.
  lo4 &= 0x0F0F0F0Fu;
  hi4 &= 0x0F0F0F0Fu;
  // bytes b0 b1 b2 b3 -> nibbles: b0 | b1<<4 in the low byte, b2 | b3<<4 in byte 2.
  uint32_t a = (lo4 | (lo4 >> 4)) & 0x00FF00FFu;  // byte0 = c0|c1<<4, byte2 = c2|c3<<4
  uint32_t b = (hi4 | (hi4 >> 4)) & 0x00FF00FFu;  // byte0 = c4|c5<<4, byte2 = c6|c7<<4
  a = (a | (a >> 8)) & 0x0000FFFFu;               // c0..c3 in bits 0..15
  b = (b | (b >> 8)) & 0x0000FFFFu;               // c4..c7
  return a | (b << 16);
}

__global__ __launch_bounds__(256) void pack_kernel(const uint4* __restrict__ q,
                                                    uint4* __restrict__ qw, int64_t units) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    const uint4 c0 = load_nt(&q[2 * u]);
    const uint4 c1 = load_nt(&q[2 * u + 1]);
    uint4 w;
    w.x = pack8(c0.x, c0.y);
    w.y = pack8(c0.z, c0.w);
    w.z = pack8(c1.x, c1.y);
    w.w = pack8(c1.z, c1.w);
    qw[u] = w;
  }
}

void launch_pack(const uint8_t* q, uint32_t* qw, int64_t N, int64_t K, hipStream_t st) {
  const int64_t units = N * K / 32;  // 32 codes -> 4 words
  int64_t blocks = (units + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(q), reinterpret_cast<uint4*>(qw), units);
}

}  // namespace w4
