// w4_gemv_topk: the int4 LM head at decode (one activation row) with token selection fused into
// the GEMV.
//
// "The inference engine -- Mojo 1.0 on Metal", "What's inside the engine today": the LM head is
// stored in int4 like the other projections (it streamed 622 MB of 2-byte weights per token
// before), and token selection runs on the GPU, bit-exact against the host; "Crossing Mojo 1.0":
// selecting on the device saves downloading the logits every token.
//
// Two launches (the unfused path takes three: the GEMV, then the two top-k passes):
//  * the M = 1 row-slice GEMV (gemv.hip) writes the logits and, in its epilogue, each
//    workgroup's largest selection key: one key per 8-16 rows (2-4 rows when a row spans
//    several waves).
//  * group_select_kernel (w4_select.h), one workgroup: the k-th largest of those keys by radix
//    select, then only the rows of the k workgroups whose keys reach it are read again, and
//    the k best of their logits are selected the same way.  Exact; values are re-read from the
//    logits, so each is the stored logit bit for bit.
#include <mutex>

#include "w4_internal.h"
#include "w4_select.h"

namespace w4 {

namespace {

// group keys combined P at a time so that at most kGsMaxKeys remain; 0: unsupported
int head_prereduce(const HeadGemvPlan& g, int k) { return gs_prereduce(g.nkeys, g.rows_per_key, k); }

}  // namespace

bool head_topk_supported(int64_t V, int64_t K, int k) {
  if (K % 64 != 0 || K < 64 || K > 4096 || V < 1 || V > 524288 || k < 1 || k > 64 || k > V) return false;
  return head_prereduce(head_gemv_plan(V, K), k) != 0;
}

size_t head_topk_ws_bytes(int64_t V, int64_t K, int) {
  return (size_t)head_gemv_plan(V, K).nkeys * sizeof(uint64_t);
}

void launch_head_topk(const uint32_t* qw, const uint16_t* s, const uint16_t* b, const uint16_t* x, float* logits,
                      int32_t* idx, float* val, int V, int K, int k, void* ws, hipStream_t st) {
  static std::once_flag lds_attr[kMaxDevices];
  once_per_device(lds_attr, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(group_select_kernel<>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)gs_lds_bytes(kGsMaxKeys));
  });
  const HeadGemvPlan g = head_gemv_plan(V, K);
  uint64_t* wgmax = reinterpret_cast<uint64_t*>(ws);
  launch_gemv_head(qw, s, b, x, logits, V, K, wgmax, st);
  const int P = head_prereduce(g, k);
  const int G = (g.nkeys + P - 1) / P;
  const int cap = G > k * g.rows_per_key * P ? G : k * g.rows_per_key * P;
  hipLaunchKernelGGL(group_select_kernel<>, dim3(1), dim3(kGsThreads), gs_lds_bytes(cap), st, logits, (int64_t)V, V, k,
                     wgmax, g.nkeys, g.rows_per_key, P, cap, idx, val);
}

}  // namespace w4
