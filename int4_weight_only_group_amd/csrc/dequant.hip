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
// The tile (64 rows x 256 codes per workgroup of 256 threads, so every row's codes are read
// as whole 128-byte lines by one workgroup) is in w4_dequant_tile.h.  HBM-bound: 0.5625 bytes
// read and 2 bytes written per weight.  The same kernel serves the symmetric group-128 format
// (w = s (q - 8)).
#include "w4_dequant_tile.h"

namespace w4 {

namespace {

// SYM: the symmetric group-128 format, w = RN16(s (q - 8)) (no bias; the OR trick's offsets
// grow by 8 so the exact f16 is q - 8, and the FMA's addend +0 makes an exact zero +0).
template <bool SYM>
__global__ __launch_bounds__(256) void dequant_t_kernel(const uint32_t* __restrict__ qw,
                                                        const uint16_t* __restrict__ sc,
                                                        const uint16_t* __restrict__ bi,
                                                        uint16_t* __restrict__ wt, int64_t ldwt,
                                                        int N, int K, bool vec) {
  __shared__ __align__(16) unsigned char lds[dqt::kLds];
  // Workgroups are dealt round-robin to the 8 XCDs; all K-tiles of a 64-row block get the
  // same XCD and run back to back there, so the block's scale and bias lines (shared by its
  // K-tiles, 8 bytes of each row per tile) are fetched once into that XCD's L2.
  const int KT = dqt::k_tiles(K), RB = dqt::row_blocks(N);
  const int xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
  const int rb = xcd + 8 * (idx / KT), kt = idx % KT;
  if (rb >= RB) return;  // padding of the last group of eight row blocks (whole workgroup)
  dqt::tile<SYM>(qw, sc, bi, wt, ldwt, N, K, vec, rb, kt, threadIdx.x, true, lds);
}

}  // namespace

template <bool SYM>
void launch_dequant_fmt(const uint32_t* qw, const uint16_t* s, const uint16_t* b, uint16_t* wt,
                        int64_t ldwt, int N, int K, hipStream_t st) {
  const int KT = dqt::k_tiles(K), RB = dqt::row_blocks(N);
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
