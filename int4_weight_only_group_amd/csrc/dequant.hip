// w4_dequant_f16_t: packed int4 weights -> transposed f16 scratch wt[k][n].
//
// "The inference engine -- Mojo 1.0 on Metal", "Crossing Mojo 1.0": instead of
// dequantizing inside the GEMM's hot loop, each weight is dequantized once per prefill into
// a transposed half-precision scratch that a plain f16 GEMM then reads.  Transposed here
// means [K][N] with N contiguous, i.e. the B operand of C = A * B for activations A [M][K].
//
// wt[k][n] = RN16(s q + b): q is turned into an exact f16 (OR-ing the nibble into 1024.0
// and subtracting 1024 is exact), and one f16 FMA rounds the exact s*q + b once, with
// subnormals kept (gfx950's f16 denormal mode is on by default).  Bit-exact.
//
// Tile: 64 rows (n) x 256 codes (k) per workgroup of 256 threads, so every row's codes are
// read as whole 128-byte lines by one workgroup.  Thread (kp, rq) = (tid % 16, tid / 16) loads
// 16 codes (8 bytes) of each of the rows 4rq .. 4rq + 3: a load instruction covers four rows'
// 128-byte lines.  Nibbles become exact f16 pairs (OR into 1024.0 and 64.0, then subtract),
// one packed f16 FMA per pair rounds s*q + b once, and byte permutes transpose the four rows
// so that each k becomes one 8-byte LDS write of four consecutive n.  After a barrier the
// workgroup writes 256 k-rows of 64 contiguous f16 (128 bytes) along N with 16-byte stores
// (2-byte stores when the output rows are not 16-byte aligned, e.g. N not a multiple of 8).
// HBM-bound: 0.5625 bytes read and 2 bytes written per weight.  The same kernel serves the
// symmetric group-128 format (w = s (q - 8)), with its scales staged per 128 codes.
#include "w4_internal.h"

namespace w4 {

namespace {

constexpr int TN = 64;      // n per tile
constexpr int TK = 256;     // k per tile
constexpr int PITCH = 136;  // bytes per LDS k-row: 64 f16 + 8 (see slot())

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// Byte offset of the 8-byte slot holding n = 4*q .. 4*q + 3 of LDS k-row kk.  The XOR with
// (kk / 16) % 16 and the 136-byte pitch make the transposing writes (lanes spread over k-rows
// 16 apart) hit distinct banks.
__device__ __forceinline__ int slot(int kk, int q) { return kk * PITCH + 8 * (q ^ ((kk >> 4) & 15)); }

// SYM: the symmetric group-128 format, w = RN16(s (q - 8)) (no bias; the OR trick's offsets
// grow by 8 so the exact f16 is q - 8, and the FMA's addend +0 makes an exact zero +0).
template <bool SYM>
__global__ __launch_bounds__(256) void dequant_t_kernel(const uint32_t* __restrict__ qw,
                                                        const uint16_t* __restrict__ sc,
                                                        const uint16_t* __restrict__ bi,
                                                        uint16_t* __restrict__ wt, int64_t ldwt,
                                                        int N, int K, bool vec) {
  __shared__ __align__(16) unsigned char t[TK * PITCH];
  constexpr int GRP = SYM ? 128 : kGroup, NGT = TK / GRP;  // groups per tile row
  __shared__ uint16_t ss[TN][NGT], bs[TN][NGT];
  // Workgroups are dealt round-robin to the 8 XCDs; all K-tiles of a 64-row block get the
  // same XCD and run back to back there, so the block's scale and bias lines (shared by its
  // K-tiles, 8 bytes of each row per tile) are fetched once into that XCD's L2.
  const int KT = (K + TK - 1) / TK, RB = (N + TN - 1) / TN;
  const int xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
  const int rb = xcd + 8 * (idx / KT), kt = idx % KT;
  if (rb >= RB) return;  // padding of the last group of eight row blocks (whole workgroup)
  const int n0 = rb * TN;
  const int k0 = kt * TK;
  const int tid = threadIdx.x;
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
    if (n < N && k < K)
      w[i] = *reinterpret_cast<const uint2*>(qw + (int64_t)n * (K / 8) + k / 8);
  }
  // the tile's scales and biases (64 rows x 4 or 2 groups), zero outside the matrix
  {
    const int r = tid >> 2, g = tid & 3;
    const int n = n0 + r, gk = k0 / GRP + g;
    uint16_t sv = 0, bv = 0;
    if (g < NGT && n < N && gk < G) {
      sv = sc[(int64_t)n * G + gk];
      bv = SYM ? 0 : bi[(int64_t)n * G + gk];
    }
    if (g < NGT) {
      ss[r][g] = sv;
      bs[r][g] = bv;
    }
  }
  __syncthreads();

  // dequantize: pair p of word wi holds codes 8wi + p and 8wi + p + 4 of a row
  constexpr float kLo = SYM ? 1032.0f : 1024.0f, kHi = SYM ? 72.0f : 64.0f;
  const h2 o1024 = {(f16)kLo, (f16)kLo}, o64 = {(f16)kHi, (f16)kHi};
  uint32_t v[4][2][4];  // [row][word][pair]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16 sv = __builtin_bit_cast(f16, ss[4 * rq + i][kp / (GRP / 16)]);
    const f16 bv = __builtin_bit_cast(f16, bs[4 * rq + i][kp / (GRP / 16)]);
    const h2 s2 = {sv, sv}, b2 = {bv, bv};
    const uint32_t words[2] = {w[i].x, w[i].y};
#pragma unroll
    for (int wi = 0; wi < 2; ++wi) {
      const uint32_t x = words[wi], x8 = x >> 8;
      const h2 q0 = as_h2((x & 0x000F000Fu) | 0x64006400u) - o1024;  // codes 0, 4 (exact)
      const h2 q1 = as_h2((x & 0x00F000F0u) | 0x54005400u) - o64;    // codes 1, 5
      const h2 q2 = as_h2((x8 & 0x000F000Fu) | 0x64006400u) - o1024; // codes 2, 6
      const h2 q3 = as_h2((x8 & 0x00F000F0u) | 0x54005400u) - o64;   // codes 3, 7
      v[i][wi][0] = as_u32(__builtin_elementwise_fma(q0, s2, b2));    // one rounding each
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
  __syncthreads();

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

}  // namespace

template <bool SYM>
void launch_dequant_fmt(const uint32_t* qw, const uint16_t* s, const uint16_t* b, uint16_t* wt,
                        int64_t ldwt, int N, int K, hipStream_t st) {
  const int KT = (K + TK - 1) / TK, RB = (N + TN - 1) / TN;
  const dim3 grid((unsigned)(8 * ((RB + 7) / 8) * KT));  // see the XCD mapping in the kernel
  // 16-byte stores need every output row to start 16-byte aligned
  const bool vec = ldwt % 8 == 0 && ((uintptr_t)wt & 15u) == 0;
  hipLaunchKernelGGL((dequant_t_kernel<SYM>), grid, dim3(256), 0, st, qw, s, b, wt, ldwt, N, K,
                     vec);
}

void launch_dequant_t(const uint32_t* qw, const uint16_t* s, const uint16_t* b, uint16_t* wt,
                      int64_t ldwt, int N, int K, hipStream_t st) {
  launch_dequant_fmt<false>(qw, s, b, wt, ldwt, N, K, st);
}

void launch_dequant_t_sym128(const uint32_t* qw, const uint16_t* s, uint16_t* wt, int64_t ldwt,
                             int N, int K, hipStream_t st) {
  launch_dequant_fmt<true>(qw, s, s, wt, ldwt, N, K, st);
}

}  // namespace w4
