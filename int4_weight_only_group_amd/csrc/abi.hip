// The C ABI (include/w4.h): argument checks on the host, then one launch path per call.
// Nothing here allocates device memory or keeps per-call state.
#include <atomic>
#include <cstring>

#include "../../include/w4.h"
#include "w4_internal.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;

inline bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
inline bool al2(const void* p) { return ((uintptr_t)p & 1u) == 0; }

std::atomic<int> g_device_ok[w4::kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= w4::kMaxDevices) {
    (void)hipGetLastError();
    return W4_ERR_DEVICE;
  }
  int c = g_device_ok[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
      (void)hipGetLastError();
      c = -1;
    } else {
      c = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    g_device_ok[dev].store(c, std::memory_order_relaxed);
  }
  return c == 1 ? W4_OK : W4_ERR_DEVICE;
}

// Two-phase workspace protocol.  Returns 1 when the call was a size query (already
// answered), 0 to go on, or a negative status.
int workspace(void* ws, size_t* ws_bytes, size_t need) {
  if (ws == nullptr && ws_bytes != nullptr) {
    *ws_bytes = need;
    return 1;
  }
  if (need == 0) return 0;
  if (ws == nullptr || ws_bytes == nullptr || *ws_bytes < need) return W4_ERR_WORKSPACE;
  if (!al16(ws)) return W4_ERR_ALIGN;
  return 0;
}

int launched() { return hipGetLastError() == hipSuccess ? W4_OK : W4_ERR_LAUNCH; }

// [p, p + bytes) as integers, for overlap checks of device ranges
struct Span {
  uintptr_t lo, hi;
};
inline Span span(const void* p, int64_t bytes) { return {(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes}; }
inline bool overlap(Span a, Span b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

int check_w4_shape(int64_t N, int64_t K) {
  if (N < 1 || K < 64 || K % 64 != 0 || N > kMaxDim || K > kMaxDim) return W4_ERR_SHAPE;
  if (N * (K / 8) > ((int64_t)1 << 40)) return W4_ERR_SHAPE;
  return W4_OK;
}

// gemm_f16_dequant_next and its symmetric group-128 twin (sym: no biases, K % 128 == 0, one
// scale per 128 codes): gemm_f16's and the dequant's checks, the GEMM's workspace, then the
// overlap checks (the two operations run at once), then one launch path.
int gemm_dequant_next(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C, int64_t ldc, int64_t M,
                      int64_t N, int64_t K, void* ws, size_t* ws_bytes, const uint32_t* qw, const uint16_t* scales,
                      const uint16_t* biases, uint16_t* wt, int64_t ldwt, int64_t Nq, int64_t Kq, bool sym,
                      w4_stream_t stream) {
  // the GEMM's checks (gemm_f16) ...
  if (!A || !B || !C || !qw || !scales || !wt) return W4_ERR_NULL;
  if (M < 1 || N < 1 || K < 1 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return W4_ERR_SHAPE;
  if (lda < K || ldb < N || ldc < N || lda > kMaxDim || ldb > kMaxDim || ldc > kMaxDim) return W4_ERR_SHAPE;
  if (!al2(A) || !al2(B) || !al4(C)) return W4_ERR_ALIGN;
  if (w4::gemm_path(A, lda, B, ldb, M, N, K) == w4::kGemmPlain && (M + 15) / 16 > 65535) return W4_ERR_SHAPE;
  // ... and the dequant's (w4_dequant_f16_t, w4_dequant_f16_t_sym128)
  if (int e = check_w4_shape(Nq, Kq)) return e;
  if (sym && Kq % 128 != 0) return W4_ERR_SHAPE;
  if (ldwt < Nq || ldwt > kMaxDim || Nq > 65535 * 64) return W4_ERR_SHAPE;
  if (!al16(qw) || !al16(scales) || (!sym && !al16(biases)) || !al2(wt)) return W4_ERR_ALIGN;
  const size_t need = w4::gemm_ws_bytes(A, lda, B, ldb, M, N, K);
  const int w = workspace(ws, ws_bytes, need);
  if (w < 0) return w;
  if (w == 1) return W4_OK;
  // the two run at once: neither's outputs may overlap the other's operands or outputs
  const int64_t groups = Nq * (Kq / (sym ? 128 : 64));
  const Span a = span(A, ((M - 1) * lda + K) * 2), b = span(B, ((K - 1) * ldb + N) * 2);
  const Span c = span(C, ((M - 1) * ldc + N) * 4), wk = span(ws, need ? (int64_t)need : 0);
  const Span q = span(qw, Nq * Kq / 2), sc = span(scales, groups * 2), bi = span(biases, sym ? 0 : groups * 2),
             t = span(wt, ((Kq - 1) * ldwt + Nq) * 2);
  for (const Span& x : {a, b, c, wk, q, sc, bi})
    if (overlap(t, x)) return W4_ERR_OVERLAP;
  for (const Span& x : {q, sc, bi})
    if (overlap(c, x) || overlap(wk, x)) return W4_ERR_OVERLAP;
  if (int e = check_device()) return e;
  (void)hipGetLastError();
  w4::launch_gemm_dequant(A, lda, B, ldb, C, ldc, (int)M, (int)N, (int)K, ws, qw, scales, biases, wt, ldwt, (int)Nq,
                          (int)Kq, sym, (hipStream_t)stream);
  return launched();
}

}  // namespace

extern "C" {

const char* w4_strerror(int status) {
  switch (status) {
    case W4_OK: return "ok";
    case W4_ERR_NULL: return "a required pointer is NULL";
    case W4_ERR_SHAPE: return "a size is out of the supported range";
    case W4_ERR_ALIGN: return "a pointer or leading dimension is misaligned";
    case W4_ERR_WORKSPACE: return "the workspace is too small";
    case W4_ERR_DEVICE: return "no usable gfx950 device is current";
    case W4_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case W4_ERR_INTERNAL: return "internal error";
    case W4_ERR_OVERLAP: return "an output of one operation overlaps an operand of the other";
    default: return "unknown status";
  }
}

int w4_pack(const uint8_t* q, uint32_t* qw, int64_t N, int64_t K, w4_stream_t stream) {
  try {
    if (!q || !qw) return W4_ERR_NULL;
    if (int e = check_w4_shape(N, K)) return e;
    if (!al16(q) || !al16(qw)) return W4_ERR_ALIGN;
    if (int e = check_device()) return e;
    (void)hipGetLastError();
    w4::launch_pack(q, qw, N, K, (hipStream_t)stream);
    return launched();
  } catch (...) {
    return W4_ERR_INTERNAL;
  }
}

int w4_gemv(const uint32_t* qw, const uint16_t* scales, const uint16_t* biases, const uint16_t* x,
            int64_t ldx, float* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* ws,
            size_t* ws_bytes, w4_stream_t stream) {
  try {
    if (!qw || !scales || !biases || !x || !y) return W4_ERR_NULL;
    if (int e = check_w4_shape(N, K)) return e;
    if (M < 1 || M > 16 || ldx < K || ldy < N || ldx > kMaxDim || ldy > kMaxDim) return W4_ERR_SHAPE;
    if (!al16(qw) || !al16(scales) || !al16(biases) || !al16(x) || !al4(y) || ldx % 8 != 0)
      return W4_ERR_ALIGN;
    const int w = workspace(ws, ws_bytes, w4::gemv_ws_bytes(M, N, K));
    if (w < 0) return w;
    if (w == 1) return W4_OK;
    if (int e = check_device()) return e;
    (void)hipGetLastError();
    w4::launch_gemv(qw, scales, biases, x, ldx, y, ldy, (int)M, (int)N, (int)K,
                    w4::gemv_ws_bytes(M, N, K) ? ws : nullptr, (hipStream_t)stream);
    return launched();
  } catch (...) {
    return W4_ERR_INTERNAL;
  }
}

int w4_quantize(const uint16_t* w, int64_t ldw, uint32_t* qw, uint16_t* scales, uint16_t* biases,
                int64_t N, int64_t K, w4_stream_t stream) {
  try {
    if (!w || !qw || !scales || !biases) return W4_ERR_NULL;
    if (int e = check_w4_shape(N, K)) return e;
    if (ldw < K || ldw > kMaxDim) return W4_ERR_SHAPE;
    if (!al16(w) || ldw % 8 != 0 || !al16(qw) || !al2(scales) || !al2(biases)) return W4_ERR_ALIGN;
    if (int e = check_device()) return e;
    (void)hipGetLastError();
    w4::launch_quantize(w, ldw, qw, scales, biases, N, K, (hipStream_t)stream);
    return launched();
  } catch (...) {
    return W4_ERR_INTERNAL;
  }
}

int w4_gemv_sym128(const uint32_t* qw, const uint16_t* scales, const uint16_t* x, int64_t ldx,
                   float* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* ws, size_t* ws_bytes,
                   w4_stream_t stream) {
  try {
    if (!qw || !scales || !x || !y) return W4_ERR_NULL;
    if (int e = check_w4_shape(N, K)) return e;
    if (K % 128 != 0) return W4_ERR_SHAPE;
    if (M < 1 || M > 16 || ldx < K || ldy < N || ldx > kMaxDim || ldy > kMaxDim) return W4_ERR_SHAPE;
    if (!al16(qw) || !al16(scales) || !al16(x) || !al4(y) || ldx % 8 != 0) return W4_ERR_ALIGN;
    const int w = workspace(ws, ws_bytes, w4::gemv_ws_bytes(M, N, K));
    if (w < 0) return w;
    if (w == 1) return W4_OK;
    if (int e = check_device()) return e;
    (void)hipGetLastError();
    w4::launch_gemv_sym128(qw, scales, x, ldx, y, ldy, (int)M, (int)N, (int)K,
                           w4::gemv_ws_bytes(M, N, K) ? ws : nullptr, (hipStream_t)stream);
    return launched();
  } catch (...) {
    return W4_ERR_INTERNAL;
  }
}

int w4_dequant_f16_t_sym128(const uint32_t* qw, const uint16_t* scales, uint16_t* wt, int64_t ldwt,
                            int64_t N, int64_t K, w4_stream_t stream) {
  try {
    if (!qw || !scales || !wt) return W4_ERR_NULL;
    if (int e = check_w4_shape(N, K)) return e;
    if (K % 128 != 0) return W4_ERR_SHAPE;
    if (ldwt < N || ldwt > kMaxDim || N > 65535 * 64) return W4_ERR_SHAPE;
    if (!al16(qw) || !al16(scales) || !al2(wt)) return W4_ERR_ALIGN;
    if (int e = check_device()) return e;
    (void)hipGetLastError();
    w4::launch_dequant_t_sym128(qw, scales, wt, ldwt, (int)N, (int)K, (hipStream_t)stream);
    return launched();
  } catch (...) {
    return W4_ERR_INTERNAL;
  }
}

int w4_dequant_f16_t(const uint32_t* qw, const uint16_t* scales, const uint16_t* biases,
                     uint16_t* wt, int64_t ldwt, int64_t N, int64_t K, w4_stream_t stream) {
  try {
    if (!qw || !scales || !biases || !wt) return W4_ERR_NULL;
    if (int e = check_w4_shape(N, K)) return e;
    if (ldwt < N || ldwt > kMaxDim || N > 65535 * 64) return W4_ERR_SHAPE;
    if (!al16(qw) || !al16(scales) || !al16(biases) || !al2(wt)) return W4_ERR_ALIGN;
    if (int e = check_device()) return e;
    (void)hipGetLastError();
    w4::launch_dequant_t(qw, scales, biases, wt, ldwt, (int)N, (int)K, (hipStream_t)stream);
    return launched();
  } catch (...) {
    return W4_ERR_INTERNAL;
  }
}

int gemm_f16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C, int64_t ldc,
             int64_t M, int64_t N, int64_t K, void* ws, size_t* ws_bytes, w4_stream_t stream) {
  try {
    if (!A || !B || !C) return W4_ERR_NULL;
    if (M < 1 || N < 1 || K < 1 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return W4_ERR_SHAPE;
    if (lda < K || ldb < N || ldc < N || lda > kMaxDim || ldb > kMaxDim || ldc > kMaxDim)
      return W4_ERR_SHAPE;
    if (!al2(A) || !al2(B) || !al4(C)) return W4_ERR_ALIGN;
    if (w4::gemm_path(A, lda, B, ldb, M, N, K) == w4::kGemmPlain && (M + 15) / 16 > 65535)
      return W4_ERR_SHAPE;
    const int w = workspace(ws, ws_bytes, w4::gemm_ws_bytes(A, lda, B, ldb, M, N, K));
    if (w < 0) return w;
    if (w == 1) return W4_OK;
    if (int e = check_device()) return e;
    (void)hipGetLastError();
    w4::launch_gemm(A, lda, B, ldb, C, ldc, (int)M, (int)N, (int)K, ws, (hipStream_t)stream);
    return launched();
  } catch (...) {
    return W4_ERR_INTERNAL;
  }
}

int gemm_f16_dequant_next(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C, int64_t ldc,
                          int64_t M, int64_t N, int64_t K, void* ws, size_t* ws_bytes, const uint32_t* qw,
                          const uint16_t* scales, const uint16_t* biases, uint16_t* wt, int64_t ldwt, int64_t Nq,
                          int64_t Kq, w4_stream_t stream) {
  try {
    if (!biases) return W4_ERR_NULL;
    return gemm_dequant_next(A, lda, B, ldb, C, ldc, M, N, K, ws, ws_bytes, qw, scales, biases, wt, ldwt, Nq, Kq,
                             false, stream);
  } catch (...) {
    return W4_ERR_INTERNAL;
  }
}

int gemm_f16_dequant_next_sym128(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C,
                                 int64_t ldc, int64_t M, int64_t N, int64_t K, void* ws, size_t* ws_bytes,
                                 const uint32_t* qw, const uint16_t* scales, uint16_t* wt, int64_t ldwt, int64_t Nq,
                                 int64_t Kq, w4_stream_t stream) {
  try {
    return gemm_dequant_next(A, lda, B, ldb, C, ldc, M, N, K, ws, ws_bytes, qw, scales, nullptr, wt, ldwt, Nq, Kq,
                             true, stream);
  } catch (...) {
    return W4_ERR_INTERNAL;
  }
}

int logits_argmax_topk(const float* logits, int64_t ldl, int64_t M, int64_t V, int64_t k,
                       int32_t* idx, float* val, void* ws, size_t* ws_bytes, w4_stream_t stream) {
  try {
    if (!logits || !idx || !val) return W4_ERR_NULL;
    if (M < 1 || M > 65535 || V < 1 || V >= ((int64_t)1 << 31) || k < 1 || k > 256 || k > V ||
        ldl < V)
      return W4_ERR_SHAPE;
    if (w4::topk_chunk(V, (int)k) == 0) return W4_ERR_SHAPE;
    if (!al4(logits) || !al4(idx) || !al4(val)) return W4_ERR_ALIGN;
    const int w = workspace(ws, ws_bytes, w4::topk_ws_bytes(M, V, (int)k));
    if (w < 0) return w;
    if (w == 1) return W4_OK;
    if (int e = check_device()) return e;
    (void)hipGetLastError();
    w4::launch_topk(logits, ldl, (int)M, (int)V, (int)k, idx, val, ws, (hipStream_t)stream);
    return launched();
  } catch (...) {
    return W4_ERR_INTERNAL;
  }
}

int w4_gemv_topk(const uint32_t* qw, const uint16_t* scales, const uint16_t* biases, const uint16_t* x,
                 int64_t V, int64_t K, int64_t k, float* logits, int32_t* idx, float* val, void* ws,
                 size_t* ws_bytes, w4_stream_t stream) {
  try {
    if (!qw || !scales || !biases || !x || !logits || !idx || !val) return W4_ERR_NULL;
    if (int e = check_w4_shape(V, K)) return e;
    if (k < 1 || k > 64 || !w4::head_topk_supported(V, K, (int)k)) return W4_ERR_SHAPE;
    if (!al16(qw) || !al16(scales) || !al16(biases) || !al16(x) || !al4(logits) || !al4(idx) || !al4(val))
      return W4_ERR_ALIGN;
    const int w = workspace(ws, ws_bytes, w4::head_topk_ws_bytes(V, K, (int)k));
    if (w < 0) return w;
    if (w == 1) return W4_OK;
    if (int e = check_device()) return e;
    (void)hipGetLastError();
    w4::launch_head_topk(qw, scales, biases, x, logits, idx, val, (int)V, (int)K, (int)k, ws, (hipStream_t)stream);
    return launched();
  } catch (...) {
    return W4_ERR_INTERNAL;
  }
}

int logits_argmax_topk_noalloc(const float* logits, int64_t ldl, int64_t M, int64_t V, int64_t k,
                               int32_t* idx, float* val, w4_stream_t stream) {
  try {
    if (!logits || !idx || !val) return W4_ERR_NULL;
    if (M < 1 || M > 65535 || V < 1 || V >= ((int64_t)1 << 31) || k < 1 || k > 256 || k > V ||
        ldl < V)
      return W4_ERR_SHAPE;
    if (w4::topk_chunk(V, (int)k) == 0) return W4_ERR_SHAPE;
    if (!al4(logits) || !al4(idx) || !al4(val)) return W4_ERR_ALIGN;
    if (w4::topk_ws_bytes(M, V, (int)k) > w4::kTopkScratchBytes) return W4_ERR_WORKSPACE;
    if (int e = check_device()) return e;
    void* scratch = w4::topk_scratch();  // this device's copy of the library's array
    if (scratch == nullptr) return W4_ERR_INTERNAL;
    (void)hipGetLastError();
    w4::launch_topk(logits, ldl, (int)M, (int)V, (int)k, idx, val, scratch, (hipStream_t)stream);
    return launched();
  } catch (...) {
    return W4_ERR_INTERNAL;
  }
}

}  // extern "C"
