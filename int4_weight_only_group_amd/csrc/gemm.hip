// gemm_f16: C[m][n] = sum_k A[m][k] B[k][n], f16 in, f32 accumulate and out.
//
// Two users on the pages' path ("The inference engine -- Mojo 1.0 on Metal"):
//  * the prefill GEMM on the transposed f16 scratch ("Crossing Mojo 1.0": dequantize once,
//    then a half-precision matrix-unit GEMM; edge guards hoisted out of the hot loop);
//  * the f16 LM head at decode, which streams a [hidden x vocab] matrix once per token
//    ("What's inside the engine today").
//
// Paths, chosen per call by shape and alignment:
//  * MFMA (M > 8): 128 x 256 block tile, BK = 32, four waves each owning a 64 x 128 tile of
//    v_mfma_f32_32x32x16_f16.  B arrives [K][N] (N contiguous) but the matrix core wants K
//    contiguous per lane, so each thread loads a 4 (k) x 8 (n) block of B with 16-byte loads
//    and transposes it in registers before writing LDS as [n][k].  Tails: rows of A and
//    column blocks of B are clamped on load (never stored) and the K tail is zero-filled, so
//    the MFMA loop itself has no guards.
//  * small M (M <= 8, decode head): each lane owns 8 contiguous columns and streams B rows
//    with 16-byte loads; the four waves of a workgroup split K and reduce through LDS.  The
//    A values of a k are wave-uniform scalar loads.
//  * plain (any other shape or alignment, e.g. one strided column of a head): a workgroup
//    per (column, 16 rows), threads split K.
#include "w4_internal.h"

namespace w4 {

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(f16, h); }

// ------------------------------------------------------------------------ MFMA path
constexpr int BM = 128, BN = 256, BK = 32;
constexpr int LDS_K = BK + 8;  // f16 per LDS row (padding keeps 16-byte alignment)

__device__ __forceinline__ uint32_t half_of(uint4 v, int j) {
  const uint32_t d = (j >> 1) == 0 ? v.x : (j >> 1) == 1 ? v.y : (j >> 1) == 2 ? v.z : v.w;
  return (j & 1) ? (d >> 16) : (d & 0xFFFFu);
}

__global__ __launch_bounds__(256) void gemm_mfma_kernel(const uint16_t* __restrict__ A,
                                                        int64_t lda,
                                                        const uint16_t* __restrict__ B,
                                                        int64_t ldb, float* __restrict__ C,
                                                        int64_t ldc, int M, int N, int K,
                                                        int tilesN) {
  __shared__ __align__(16) uint16_t As[BM * LDS_K];
  __shared__ __align__(16) uint16_t Bs[BN * LDS_K];

  const int tm = blockIdx.x / tilesN, tn = blockIdx.x % tilesN;
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // global -> register mapping
  const int a_row0 = tid >> 2, a_kc = (tid & 3) * 8;  // + 64 rows for the second chunk
  const int b_nb = tid & 31, b_kb = tid >> 5;         // 8-column block, 4-row block
  const uint16_t* a_src[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int gm = min(m0 + a_row0 + i * 64, M - 1);
    a_src[i] = A + (int64_t)gm * lda + a_kc;
  }
  const int gn = min(n0 + b_nb * 8, N - 8);
  const uint16_t* b_src = B + gn + (int64_t)(b_kb * 4) * ldb;

  uint4 ra[2], rb[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      ra[i] = (k0 + a_kc < K) ? *reinterpret_cast<const uint4*>(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      rb[i] = (k0 + b_kb * 4 + i < K)
                  ? *reinterpret_cast<const uint4*>(b_src + (int64_t)(k0 + i) * ldb)
                  : make_uint4(0, 0, 0, 0);
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<uint4*>(&As[(a_row0 + i * 64) * LDS_K + a_kc]) = ra[i];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint2 v;
      v.x = half_of(rb[0], j) | (half_of(rb[1], j) << 16);
      v.y = half_of(rb[2], j) | (half_of(rb[3], j) << 16);
      *reinterpret_cast<uint2*>(&Bs[(b_nb * 8 + j) * LDS_K + b_kb * 4]) = v;
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  load(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + BK < K) load(k0 + BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kof = ks * 16 + (lane >> 5) * 8;
      f16x8 a[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const f16x8*>(&As[(wm * 64 + i * 32 + (lane & 31)) * LDS_K + kof]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const f16x8*>(&Bs[(wn * 128 + j * 32 + (lane & 31)) * LDS_K + kof]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // D layout of a 32x32 tile: lane l, value r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row < M && col < N) C[(int64_t)row * ldc + col] = acc[i][j][r];
      }
    }
}

// -------------------------------------------------------------------- small-M path
constexpr int SM_COLS = 512;  // 64 lanes x 8 columns

template <int MT>
__global__ __launch_bounds__(256) void gemm_smallm_kernel(const uint16_t* __restrict__ A,
                                                          int64_t lda,
                                                          const uint16_t* __restrict__ B,
                                                          int64_t ldb, float* __restrict__ C,
                                                          int64_t ldc, int M, int N, int K,
                                                          int KS) {
  __shared__ float red[3][MT][SM_COLS];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * SM_COLS + lane * 8;
  const int nn = min(n, N - 8);  // clamp: columns past N are computed, never stored
  const int kb = wave * KS;
  const int ke = min(K, kb + KS);

  float acc[MT][8];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[m][j] = 0.f;

  const uint16_t* bcol = B + nn;
  for (int k = kb; k < ke; k += 8) {
    uint4 h[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      h[kk] = load_nt(bcol + (int64_t)(k + kk) * ldb);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int mm = m < M ? m : M - 1;
      const uint4 a8 = *reinterpret_cast<const uint4*>(A + (int64_t)mm * lda + k);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const float a = h2f((uint16_t)half_of(a8, kk));
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[m][j] = __builtin_fmaf(h2f((uint16_t)half_of(h[kk], j)), a, acc[m][j]);
      }
    }
  }

  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) red[wave - 1][m][lane * 8 + j] = acc[m][j];
  }
  __syncthreads();
  if (wave == 0 && n < N) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= M) break;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = acc[m][j];
        v += red[0][m][lane * 8 + j];
        v += red[1][m][lane * 8 + j];
        v += red[2][m][lane * 8 + j];
        C[(int64_t)m * ldc + n + j] = v;
      }
    }
  }
}

// ------------------------------------------------------------------------ plain path
constexpr int PL_ROWS = 16;

__global__ __launch_bounds__(256) void gemm_plain_kernel(const uint16_t* __restrict__ A,
                                                         int64_t lda,
                                                         const uint16_t* __restrict__ B,
                                                         int64_t ldb, float* __restrict__ C,
                                                         int64_t ldc, int M, int N, int K) {
  __shared__ float red[4][PL_ROWS];
  const int n = blockIdx.x;
  const int m0 = blockIdx.y * PL_ROWS;
  const int rows = min(PL_ROWS, M - m0);
  float acc[PL_ROWS];
#pragma unroll
  for (int i = 0; i < PL_ROWS; ++i) acc[i] = 0.f;
  for (int k = threadIdx.x; k < K; k += 256) {
    const float b = h2f(B[(int64_t)k * ldb + n]);
#pragma unroll
    for (int i = 0; i < PL_ROWS; ++i)
      if (i < rows) acc[i] = __builtin_fmaf(h2f(A[(int64_t)(m0 + i) * lda + k]), b, acc[i]);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < PL_ROWS; ++i) {
    float v = acc[i];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) red[wave][i] = v;
  }
  __syncthreads();
  if (threadIdx.x < rows) {
    const int i = threadIdx.x;
    C[(int64_t)(m0 + i) * ldc + n] = ((red[0][i] + red[1][i]) + red[2][i]) + red[3][i];
  }
}

}  // namespace

GemmPath gemm_path(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M,
                   int64_t N, int64_t K) {
  const bool vec = K % 8 == 0 && N % 8 == 0 && lda % 8 == 0 && ldb % 8 == 0 && aligned16(A) &&
                   aligned16(B);
  if (!vec) return kGemmPlain;
  return M > 8 ? kGemmMfma : kGemmSmallM;
}

void launch_gemm(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C,
                 int64_t ldc, int M, int N, int K, hipStream_t st) {
  switch (gemm_path(A, lda, B, ldb, M, N, K)) {
    case kGemmMfma: {
      const int tilesM = (M + BM - 1) / BM, tilesN = (N + BN - 1) / BN;
      hipLaunchKernelGGL(gemm_mfma_kernel, dim3((unsigned)(tilesM * tilesN)), dim3(256), 0, st, A,
                         lda, B, ldb, C, ldc, M, N, K, tilesN);
      break;
    }
    case kGemmSmallM: {
      int KS = ((K + 3) / 4 + 7) / 8 * 8;
      const dim3 grid((unsigned)((N + SM_COLS - 1) / SM_COLS));
      if (M <= 1)
        hipLaunchKernelGGL(gemm_smallm_kernel<1>, grid, dim3(256), 0, st, A, lda, B, ldb, C, ldc, M, N, K, KS);
      else if (M <= 2)
        hipLaunchKernelGGL(gemm_smallm_kernel<2>, grid, dim3(256), 0, st, A, lda, B, ldb, C, ldc, M, N, K, KS);
      else if (M <= 4)
        hipLaunchKernelGGL(gemm_smallm_kernel<4>, grid, dim3(256), 0, st, A, lda, B, ldb, C, ldc, M, N, K, KS);
      else
        hipLaunchKernelGGL(gemm_smallm_kernel<8>, grid, dim3(256), 0, st, A, lda, B, ldb, C, ldc, M, N, K, KS);
      break;
    }
    default: {
      const dim3 grid((unsigned)N, (unsigned)((M + PL_ROWS - 1) / PL_ROWS));
      hipLaunchKernelGGL(gemm_plain_kernel, grid, dim3(256), 0, st, A, lda, B, ldb, C, ldc, M, N, K);
    }
  }
}

}  // namespace w4
