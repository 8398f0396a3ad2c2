// One tile of the dequant-transpose (packed int4 -> f16 wt[k][n]) for 256 threads: the body of
// the standalone dequant kernel and of the dequant workgroups that run beside a GEMM.
//
// Tile: 64 rows (n) x 256 codes (k).  Thread (kp, rq) = (tid % 16, tid / 16) loads 16 codes
// (8 bytes) of each of the rows 4rq .. 4rq + 3: a load instruction covers four rows' 128-byte
// lines.  Nibbles become exact f16 pairs (OR into 1024.0 and 64.0, then subtract), one packed
// f16 FMA per pair rounds s*q + b once, and byte permutes transpose the four rows so that each
// k becomes one 8-byte LDS write of four consecutive n.  After a barrier the 256 threads write
// 256 k-rows of 64 contiguous f16 (128 bytes) along N with 16-byte stores (2-byte stores when
// the output rows are not 16-byte aligned, e.g. N not a multiple of 8).  The symmetric
// group-128 format (w = s (q - 8)) stages its scales per 128 codes.
#pragma once

#include "w4_internal.h"

namespace w4 {
namespace dqt {

constexpr int TN = 64;      // n per tile
constexpr int TK = 256;     // k per tile
constexpr int PITCH = 136;  // bytes per LDS k-row: 64 f16 + 8 (see slot())
constexpr int kSB = TN * 4 * 2;                   // bytes of the staged scales (or biases)
constexpr size_t kLds = (size_t)TK * PITCH + 2 * kSB;  // LDS bytes per tile

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// Byte offset of the 8-byte slot holding n = 4*q .. 4*q + 3 of LDS k-row kk.  The XOR with
// (kk / 16) % 16 and the 136-byte pitch make the transposing writes (lanes spread over k-rows
// 16 apart) hit distinct banks.
__device__ __forceinline__ int slot(int kk, int q) { return kk * PITCH + 8 * (q ^ ((kk >> 4) & 15)); }

// Tile (rb, kt) by threads tid = 0..255 of a group whose every thread calls this with the same
// `live`; lds: kLds bytes, 16-byte aligned.  Two workgroup barriers: every thread of the
// workgroup must make the call (a thread whose group has no tile passes live = false and only
// takes the barriers).  A caller that runs tiles back to back reuses lds safely: the next
// call's first LDS write follows its first barrier, which every thread reaches only after its
// stores of the previous tile.
template <bool SYM>
__device__ __forceinline__ void tile(const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                                     const uint16_t* __restrict__ bi, uint16_t* __restrict__ wt, int64_t ldwt,
                                     int N, int K, bool vec, int rb, int kt, int tid, bool live,
                                     unsigned char* lds) {
  constexpr int GRP = SYM ? 128 : kGroup, NGT = TK / GRP;  // groups per tile row
  unsigned char* t = lds;
  uint16_t* ss = reinterpret_cast<uint16_t*>(lds + TK * PITCH);  // [TN][NGT]
  uint16_t* bs = ss + kSB / 2;
  const int n0 = rb * TN;
  const int k0 = kt * TK;
  const int G = K / GRP;

  // this thread's codes: rows n0 + 4rq + i, codes k .. k + 15 (none past the row end: K is a
  // multiple of 64 and the 16 codes never straddle it)
  const int kp = tid & 15, rq = tid >> 4;
  const int k = k0 + kp * 16;
  uint2 w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + 4 * rq + i;
    w[i] = make_uint2(0, 0);
    if (live && n < N && k < K) w[i] = *reinterpret_cast<const uint2*>(qw + (int64_t)n * (K / 8) + k / 8);
  }
  // the tile's scales and biases (64 rows x 4 or 2 groups), zero outside the matrix
  if (live) {
    const int r = tid >> 2, g = tid & 3;
    const int n = n0 + r, gk = k0 / GRP + g;
    uint16_t sv = 0, bv = 0;
    if (g < NGT && n < N && gk < G) {
      sv = sc[(int64_t)n * G + gk];
      bv = SYM ? 0 : bi[(int64_t)n * G + gk];
    }
    if (g < NGT) {
      ss[r * NGT + g] = sv;
      bs[r * NGT + g] = bv;
    }
  }
  __syncthreads();

  if (live) {
    // dequantize: pair p of word wi holds codes 8wi + p and 8wi + p + 4 of a row
    constexpr float kLo = SYM ? 1032.0f : 1024.0f, kHi = SYM ? 72.0f : 64.0f;
    const h2 o1024 = {(f16)kLo, (f16)kLo}, o64 = {(f16)kHi, (f16)kHi};
    uint32_t v[4][2][4];  // [row][word][pair]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16 sv = __builtin_bit_cast(f16, ss[(4 * rq + i) * NGT + kp / (GRP / 16)]);
      const f16 bv = __builtin_bit_cast(f16, bs[(4 * rq + i) * NGT + kp / (GRP / 16)]);
      const h2 s2 = {sv, sv}, b2 = {bv, bv};
      const uint32_t words[2] = {w[i].x, w[i].y};
#pragma unroll
      for (int wi = 0; wi < 2; ++wi) {
        const uint32_t x = words[wi], x8 = x >> 8;
        const h2 q0 = as_h2((x & 0x000F000Fu) | 0x64006400u) - o1024;   // codes 0, 4 (exact)
        const h2 q1 = as_h2((x & 0x00F000F0u) | 0x54005400u) - o64;     // codes 1, 5
        const h2 q2 = as_h2((x8 & 0x000F000Fu) | 0x64006400u) - o1024;  // codes 2, 6
        const h2 q3 = as_h2((x8 & 0x00F000F0u) | 0x54005400u) - o64;    // codes 3, 7
        v[i][wi][0] = as_u32(__builtin_elementwise_fma(q0, s2, b2));     // one rounding each
        v[i][wi][1] = as_u32(__builtin_elementwise_fma(q1, s2, b2));
        v[i][wi][2] = as_u32(__builtin_elementwise_fma(q2, s2, b2));
        v[i][wi][3] = as_u32(__builtin_elementwise_fma(q3, s2, b2));
      }
    }
    // transpose: (row0, row1) and (row2, row3) halves of the same code into one word each
#pragma unroll
    for (int wi = 0; wi < 2; ++wi)
#pragma unroll
      for (int pi = 0; pi < 4; ++pi) {
        const int kk = kp * 16 + wi * 8 + pi;  // code of the low halves; kk + 4 of the high
        const uint32_t lo01 = __builtin_amdgcn_perm(v[1][wi][pi], v[0][wi][pi], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(v[3][wi][pi], v[2][wi][pi], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(v[1][wi][pi], v[0][wi][pi], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(v[3][wi][pi], v[2][wi][pi], 0x07060302u);
        *reinterpret_cast<uint2*>(t + slot(kk, rq)) = make_uint2(lo01, lo23);
        *reinterpret_cast<uint2*>(t + slot(kk + 4, rq)) = make_uint2(hi01, hi23);
      }
  }
  __syncthreads();

  if (!live) return;
  // 256 k-rows x 64 columns = 2048 vectors of 8 f16; 8 per thread, eight lanes per row
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int e = tid + it * 256;
    const int kr = e >> 3;
    const int nb = e & 7;
    const int kk = k0 + kr;
    const int n = n0 + nb * 8;
    if (kk < K && n < N) {
      const uint2 lo = *reinterpret_cast<const uint2*>(t + slot(kr, 2 * nb));
      const uint2 hi = *reinterpret_cast<const uint2*>(t + slot(kr, 2 * nb + 1));
      uint16_t* dst = wt + (int64_t)kk * ldwt + n;
      if (vec && n + 8 <= N) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(lo.x, lo.y, hi.x, hi.y);
      } else {
        const uint32_t h[4] = {lo.x, lo.y, hi.x, hi.y};
        const int cnt = min(8, N - n);  // this thread's 8 columns, fewer at the N tail
        for (int j = 0; j < cnt; ++j) dst[j] = (uint16_t)(h[j >> 1] >> (16 * (j & 1)));
      }
    }
  }
}

// Tiles of an N x K dequant, row block rb = tile / KT, K-tile kt = tile % KT.
__host__ __device__ __forceinline__ int k_tiles(int K) { return (K + TK - 1) / TK; }
__host__ __device__ __forceinline__ int row_blocks(int N) { return (N + TN - 1) / TN; }

}  // namespace dqt
}  // namespace w4
