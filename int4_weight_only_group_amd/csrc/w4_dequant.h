// Device helpers shared by the GEMV kernels: the weight formats, codes to exact f16 through the
// fp8 converter, one-rounding dequant and the f32 dot products, raw buffer resources.
#pragma once

#include "w4_internal.h"

namespace w4 {

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(hf16x2, a), __builtin_bit_cast(hf16x2, b), c,
                                false);
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// Weight formats: the affine group-64 format (w = s q + b) and the symmetric group-128 one
// (w = s (q - 8), no bias).  For the latter the OR trick's offsets grow by 8, so the exact
// f16 it yields is q - 8, and the FMA's addend is +0 (w = RN(s (q - 8)), an exact zero +0).
template <bool SYM>
struct Fmt {
  static constexpr int kGroupSize = SYM ? 128 : 64;
  static constexpr int kChunkShift = SYM ? 2 : 1;  // 16-byte chunk index -> group index
  static constexpr float kLo = SYM ? 1032.0f : 1024.0f, kHi = SYM ? 72.0f : 64.0f;
};

// Codes of word w as exact f16 pairs through the fp8 converter: in the e4m3 encoding a byte
// holding 0..15 is the number q * 2^-9 exactly (the subnormals and the first normal binade are
// one evenly spaced range), so converting with the scale 2^9 yields q.  The low nibbles
// (w & 0x0F0F0F0F) and high nibbles ((w >> 4) & 0x0F0F0F0F) give the pairs (q0,q2) (q4,q6)
// and (q1,q3) (q5,q7): 7 instructions for 8 codes (the OR trick takes 9).  The symmetric
// format subtracts 8 (exact).
template <bool SYM>
__device__ __forceinline__ void cvt_codes(uint32_t w, h2& q0, h2& q1, h2& q2, h2& q3) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  q0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false);  // (q0, q2)
  q1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true);   // (q4, q6)
  q2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, false);  // (q1, q3)
  q3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, true);   // (q5, q7)
  if constexpr (SYM) {
    const h2 o8 = {(f16)8.0f, (f16)8.0f};
    q0 -= o8;
    q1 -= o8;
    q2 -= o8;
    q3 -= o8;
  }
}

// (x0x1, x2x3, x4x5, x6x7) -> (x0x2, x4x6, x1x3, x5x7): the converter's code order
__device__ __forceinline__ uint4 pair_up_cvt(uint4 d) {
  uint4 p;
  p.x = __builtin_amdgcn_perm(d.y, d.x, 0x05040100u);
  p.y = __builtin_amdgcn_perm(d.w, d.z, 0x05040100u);
  p.z = __builtin_amdgcn_perm(d.y, d.x, 0x07060302u);
  p.w = __builtin_amdgcn_perm(d.w, d.z, 0x07060302u);
  return p;
}

// One word's 8 weights (one FMA rounding each) dotted with x pairs in the converter's order.
template <bool SYM>
__device__ __forceinline__ float word_fma_cvt(uint32_t w, h2 s2, h2 b2, const uint4& xp, float acc) {
  h2 q0, q1, q2, q3;
  cvt_codes<SYM>(w, q0, q1, q2, q3);
  acc = dot2(as_u32(__builtin_elementwise_fma(q0, s2, b2)), xp.x, acc);
  acc = dot2(as_u32(__builtin_elementwise_fma(q1, s2, b2)), xp.y, acc);
  acc = dot2(as_u32(__builtin_elementwise_fma(q2, s2, b2)), xp.z, acc);
  acc = dot2(as_u32(__builtin_elementwise_fma(q3, s2, b2)), xp.w, acc);
  return acc;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* p) {
  // raw buffer (stride 0) over the 31-bit offset range from p; offsets stay far below it
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7FFFFFFF, 0x00020000);
}

}  // namespace w4
