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
// Tile: 64 rows (n) x 128 codes (k) per workgroup of 256 threads.  Each thread loads one
// 16-byte chunk (32 codes of one row) coalesced along K, dequantizes it into LDS at the
// transposed position, and after a barrier the workgroup writes 128 rows of 64 contiguous
// f16 (128 bytes) along N with 16-byte stores (2-byte stores when the output rows are not
// 16-byte aligned, e.g. N not a multiple of 8).  HBM-bound: 0.5625 bytes read and 2 bytes
// written per weight.
#include "w4_internal.h"

namespace w4 {

namespace {

constexpr int TN = 64;    // n per tile
constexpr int TK = 128;   // k per tile
constexpr int PADN = 8;   // f16 of padding per LDS row (keeps rows 16-byte aligned)

__global__ __launch_bounds__(256) void dequant_t_kernel(const uint32_t* __restrict__ qw,
                                                        const uint16_t* __restrict__ sc,
                                                        const uint16_t* __restrict__ bi,
                                                        uint16_t* __restrict__ wt, int64_t ldwt,
                                                        int N, int K, bool vec) {
  __shared__ __align__(16) uint16_t t[TK][TN + PADN];
  const int n0 = blockIdx.y * TN;
  const int k0 = blockIdx.x * TK;
  const int tid = threadIdx.x;

  {
    const int r = tid >> 2;        // row within the tile
    const int part = tid & 3;      // which 32-code chunk of the 128
    const int n = n0 + r;
    const int k = k0 + part * 32;
    if (n < N && k < K) {
      const int64_t KW = K / 8;
      const uint4 w = load_nt(qw + (int64_t)n * KW + k / 8);
      const int g = k / kGroup;
      const f16 s = __builtin_bit_cast(f16, sc[(int64_t)n * (K / kGroup) + g]);
      const f16 b = __builtin_bit_cast(f16, bi[(int64_t)n * (K / kGroup) + g]);
      const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint16_t qb = (uint16_t)(0x6400u | ((words[j] >> (4 * i)) & 0xFu));
          const f16 q = __builtin_bit_cast(f16, qb) - (f16)1024.0f;  // exact
          const f16 v = __builtin_fmaf16(s, q, b);                    // one rounding
          t[part * 32 + j * 8 + i][r] = __builtin_bit_cast(uint16_t, v);
        }
      }
    }
  }
  __syncthreads();

  // 128 rows x 64 columns = 1024 vectors of 8 f16; 4 per thread.
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int v = tid + it * 256;
    const int kr = v >> 3;
    const int nb = (v & 7) * 8;
    const int k = k0 + kr;
    const int n = n0 + nb;
    if (k < K && n < N) {
      uint16_t* dst = wt + (int64_t)k * ldwt + n;
      if (vec && n + 8 <= N) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(&t[kr][nb]);
      } else {
        const int cnt = min(8, N - n);  // this thread's 8 columns, fewer at the N tail
        for (int j = 0; j < cnt; ++j) dst[j] = t[kr][nb + j];
      }
    }
  }
}

}  // namespace

void launch_dequant_t(const uint32_t* qw, const uint16_t* s, const uint16_t* b, uint16_t* wt,
                      int64_t ldwt, int N, int K, hipStream_t st) {
  const dim3 grid((unsigned)((K + TK - 1) / TK), (unsigned)((N + TN - 1) / TN));
  // 16-byte stores need every output row to start 16-byte aligned
  const bool vec = ldwt % 8 == 0 && ((uintptr_t)wt & 15u) == 0;
  hipLaunchKernelGGL(dequant_t_kernel, grid, dim3(256), 0, st, qw, s, b, wt, ldwt, N, K, vec);
}

}  // namespace w4
