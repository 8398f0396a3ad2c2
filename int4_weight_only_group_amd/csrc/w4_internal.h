// Internal declarations shared by the kernel files and the C-ABI layer.
// Launchers assume their arguments were validated by abi.hip; they only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <utility>

namespace w4 {

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __fp16 hf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 64;  // elements of K per (scale, bias)

// 16-byte streaming load that is not expected to be re-read (non-temporal hint).
__device__ __forceinline__ uint4 load_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Sum over aligned groups of W lanes (W = 16, 32 or 64) with DPP lane moves instead of LDS
// permutes; the group's total lands in its last lane (lane W - 1 of the group).  Steps: swap
// neighbours, swap pairs (quad sums), half-row mirror (8), row mirror (16: every lane of the
// row), then broadcast row sums forward into rows 1, 3 (32) and rows 2, 3 (64).  The order of
// the additions is fixed, so results are deterministic.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, ROWS, 0xF, false));
}
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(W == 16 || W == 32 || W == 64, "group of 16, 32 or 64 lanes");
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  if constexpr (W >= 32) v += dpp_f<0x142, 0xA>(v);  // row_bcast15 into rows 1 and 3
  if constexpr (W >= 64) v += dpp_f<0x143, 0xC>(v);  // row_bcast31 into rows 2 and 3
  return v;
}

// ---------------------------------------------------------------- launchers
void launch_pack(const uint8_t* q, uint32_t* qw, int64_t N, int64_t K, hipStream_t st);

// ws: gemv_ws_bytes(M, N, K) bytes, 16-byte aligned (nullptr when that is 0)
void launch_gemv(const uint32_t* qw, const uint16_t* s, const uint16_t* b, const uint16_t* x,
                 int64_t ldx, float* y, int64_t ldy, int M, int N, int K, void* ws, hipStream_t st);
size_t gemv_ws_bytes(int64_t M, int64_t N, int64_t K);

void launch_quantize(const uint16_t* w, int64_t ldw, uint32_t* qw, uint16_t* s, uint16_t* b,
                     int64_t N, int64_t K, hipStream_t st);
// The symmetric group-128 format: w = s (q - 8), one scale per 128 elements of K, no bias.
void launch_gemv_sym128(const uint32_t* qw, const uint16_t* s, const uint16_t* x, int64_t ldx,
                        float* y, int64_t ldy, int M, int N, int K, void* ws, hipStream_t st);
void launch_dequant_t_sym128(const uint32_t* qw, const uint16_t* s, uint16_t* wt, int64_t ldwt,
                             int N, int K, hipStream_t st);
void launch_dequant_t(const uint32_t* qw, const uint16_t* s, const uint16_t* b, uint16_t* wt,
                      int64_t ldwt, int N, int K, hipStream_t st);

// Which gemm path a shape takes (exposed for tests through the ABI's behaviour only).
enum GemmPath { kGemmMfma = 0, kGemmSmallM = 1, kGemmPlain = 2 };
GemmPath gemm_path(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M,
                   int64_t N, int64_t K);
size_t gemm_ws_bytes(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M,
                     int64_t N, int64_t K);
void launch_gemm(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C,
                 int64_t ldc, int M, int N, int K, void* ws, hipStream_t st);
// Dequant workgroups that a GEMM of this shape can take beside its own for an Nq x Kq dequant
// (the CUs its last round of workgroups leaves idle on a device of `cus` CUs, when the dequant
// is estimated to finish within that round); 0: the GEMM and the dequant run as two launches.
int gemm_side_workgroups(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M,
                         int64_t N, int64_t K, int64_t Nq, int64_t Kq, int cus);
// launch_gemm and launch_dequant_t (Nq x Kq codes; sym: launch_dequant_t_sym128, b unused) in
// one launch when gemm_side_workgroups allows it, else one after the other; same results
// either way.
void launch_gemm_dequant(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C, int64_t ldc,
                         int M, int N, int K, void* ws, const uint32_t* qw, const uint16_t* s, const uint16_t* b,
                         uint16_t* wt, int64_t ldwt, int Nq, int Kq, bool sym, hipStream_t st);

// Top-k: chunk size (in logits) used for rows longer than one block, and workspace bytes.
int topk_chunk(int64_t V, int k);        // 0 when the shape is unsupported
size_t topk_ws_bytes(int64_t M, int64_t V, int k);
void launch_topk(const float* logits, int64_t ldl, int M, int V, int k, int32_t* idx, float* val,
                 void* ws, hipStream_t st);
// The int4 LM head with token selection (one activation row): shapes it supports, its
// workspace bytes (the GEMV's and the selection's, which run one after the other), and the
// launches.
bool head_topk_supported(int64_t V, int64_t K, int k);
size_t head_topk_ws_bytes(int64_t V, int64_t K, int k);
void launch_head_topk(const uint32_t* qw, const uint16_t* s, const uint16_t* b, const uint16_t* x, float* logits,
                      int32_t* idx, float* val, int V, int K, int k, void* ws, hipStream_t st);

// The allocation-free top-k's file-scope device array: its size, and its device address on
// the current device (fetched once per device; nullptr if the runtime cannot give it).
constexpr size_t kTopkScratchBytes = (size_t)4 << 20;
void* topk_scratch();

// Runs f once for the current device.  Function attributes such as the dynamic LDS limit are
// set per device, so a process that launches on several GPUs sets them on each.
constexpr int kMaxDevices = 64;
template <class F>
void once_per_device(std::once_flag (&flags)[kMaxDevices], F&& f) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    dev = 0;
  }
  std::call_once(flags[dev], std::forward<F>(f));
}

}  // namespace w4
