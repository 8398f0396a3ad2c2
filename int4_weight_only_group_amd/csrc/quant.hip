// w4_quantize: f16 weights -> the affine int4 group-64 format, once, at load.
//
// What it computes ("The inference engine -- Mojo 1.0 on Metal", "Where it fits": the
// weights are quantized to int4 at load; "Engineering investigation ...", "Selective
// quantization": affine, group size 64).  The pages give no fitting rule; this is the plain
// min/max fit, per (row, group of 64 along K):
//   lo, hi = the group's smallest and largest value, a zero counting as +0;   b = lo;
//   s = RN16(f32(f32(hi - lo) / 15));
//   q = clamp(rint_even(f32(f32(w - b) / s)), 0, 15),   or q = 0 for the group when s == 0.
// Every step that decides a code is a correctly rounded f32 operation written with the
// explicit _rn intrinsics (no contraction, no reciprocal rewrite), so the codes are a pure
// function of the inputs; the quotient's division is replaced by a reciprocal product wherever
// that provably gives the same code (see the kernel).
//
// Design (HBM-bound: 2 bytes read, 0.5625 written per weight): eight lanes per group, each
// lane one 16-byte load (8 weights) and one packed word; the group's min and max are
// combined across its eight lanes with three DPP moves each (swap neighbours, swap pairs,
// half-row mirror).  A wave covers 8 consecutive groups, i.e. 1 KB of contiguous weights
// (consecutive groups of a row, and rows follow each other when ldw == K), and writes 256
// contiguous bytes of packed words.
#include "w4_internal.h"

namespace w4 {

namespace {

template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xF, 0xF, false));
}

// min and max over the 8 lanes of an aligned lane octet (every lane gets both)
__device__ __forceinline__ void octet_minmax(float& lo, float& hi) {
  lo = fminf(lo, dpp_move<0xB1>(lo));   // quad_perm [1,0,3,2]
  hi = fmaxf(hi, dpp_move<0xB1>(hi));
  lo = fminf(lo, dpp_move<0x4E>(lo));   // quad_perm [2,3,0,1]
  hi = fmaxf(hi, dpp_move<0x4E>(hi));
  lo = fminf(lo, dpp_move<0x141>(lo));  // row_half_mirror: lane i <-> 7 - i (the other quad)
  hi = fmaxf(hi, dpp_move<0x141>(hi));
}

__device__ __forceinline__ float h2f(uint32_t bits) {
  return (float)__builtin_bit_cast(f16, (uint16_t)bits);
}

__global__ __launch_bounds__(256) void quant_kernel(const uint16_t* __restrict__ w, int64_t ldw,
                                                    uint32_t* __restrict__ qw,
                                                    uint16_t* __restrict__ sc,
                                                    uint16_t* __restrict__ bi, int G,
                                                    int64_t ngroups) {
  constexpr int kGroupsPerBlock = 256 / 8;
  const int lane8 = threadIdx.x & 7;
  for (int64_t base = (int64_t)blockIdx.x * kGroupsPerBlock; base < ngroups;
       base += (int64_t)gridDim.x * kGroupsPerBlock) {
    const int64_t gid = base + (threadIdx.x >> 3);
    const int64_t gc = gid < ngroups ? gid : ngroups - 1;  // whole octets clamp together
    const int64_t n = gc / G;
    const int g = (int)(gc - n * G);
    const uint4 raw = load_nt(w + n * ldw + (int64_t)g * kGroup + lane8 * 8);
    float v[8] = {h2f(raw.x & 0xFFFFu), h2f(raw.x >> 16), h2f(raw.y & 0xFFFFu), h2f(raw.y >> 16),
                  h2f(raw.z & 0xFFFFu), h2f(raw.z >> 16), h2f(raw.w & 0xFFFFu), h2f(raw.w >> 16)};
    float lo = v[0], hi = v[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      lo = fminf(lo, v[i]);
      hi = fmaxf(hi, v[i]);
    }
    octet_minmax(lo, hi);
    if (lo == 0.0f) lo = 0.0f;  // -0 -> +0
    if (hi == 0.0f) hi = 0.0f;
    const float t = __fdiv_rn(__fsub_rn(hi, lo), 15.0f);
    const f16 s16 = (f16)t;  // round to nearest even, subnormals kept
    const float s = (float)s16;
    // Codes: only the nearest integer of the correctly rounded quotient RN(d / s) matters.  The
    // quotients stay below 22.5 (s = RN16((hi - lo) / 15) is at least 2/3 of (hi - lo) / 15, the
    // worst case being a subnormal s), so a = RN(d * rcp(s)) is within 1.1e-5 of RN(d / s)
    // (v_rcp_f32 within 2^-22 relative, the product's rounding 2^-24, the quotient's own rounding
    // 2^-20) and rint(a) is the code unless a half-integer lies that close.  Those quotients
    // (about 1 in 12000 on random weights; exact ties always) take the correctly rounded
    // division.  d >= 0 (lo is the group's minimum), so only the upper clamp can act; s == 0
    // (a NaN or infinite a, never within reach of a half-integer) zeroes the word at the end.
    const float rs = __builtin_amdgcn_rcpf(s);
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float d = __fsub_rn(v[i], lo);
      const float a = __fmul_rn(d, rs);
      float r = __builtin_rintf(a);
      if (fabsf(__builtin_amdgcn_fractf(a) - 0.5f) <= 4e-5f) r = __builtin_rintf(__fdiv_rn(d, s));
      word |= (uint32_t)fminf(r, 15.0f) << (4 * i);
    }
    if (s == 0.0f) word = 0u;
    if (gid < ngroups) {
      qw[n * ((int64_t)G * 8) + (int64_t)g * 8 + lane8] = word;
      if (lane8 == 0) {
        sc[gc] = __builtin_bit_cast(uint16_t, s16);
        bi[gc] = __builtin_bit_cast(uint16_t, (f16)lo);  // exact: lo is an f16 value
      }
    }
  }
}

}  // namespace

void launch_quantize(const uint16_t* w, int64_t ldw, uint32_t* qw, uint16_t* s, uint16_t* b,
                     int64_t N, int64_t K, hipStream_t st) {
  const int G = (int)(K / kGroup);
  const int64_t ngroups = N * G;
  int64_t blocks = (ngroups + 31) / 32;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(quant_kernel, dim3((unsigned)blocks), dim3(256), 0, st, w, ldw, qw, s, b, G,
                     ngroups);
}

}  // namespace w4
