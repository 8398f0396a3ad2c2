// w4_gemv_topk: the int4 LM head at decode (one activation row) with token selection on the
// device, in one call.
//
// "The inference engine -- Mojo 1.0 on Metal", "What's inside the engine today": the LM head is
// stored in int4 like the other projections (it streamed 622 MB of 2-byte weights per token
// before), and token selection runs on the GPU, bit-exact against the host; "Crossing Mojo 1.0":
// selecting on the device saves downloading the logits every token.
//
// The M = 1 GEMV (gemv.hip) writes the logits, then the top-k of logits_argmax_topk (topk.hip)
// selects from them: group maxima of 64 logits, then one selection workgroup.  A variant that
// had the GEMV's workgroups write their largest key directly (saving the group-maxima pass) was
// measured slower: the waves of each GEMV workgroup must meet to combine their keys, and that
// costs the 175 MB head GEMV more (37.3 against 29.2 us) than the 0.6 MB pass it saves.
#include "w4_internal.h"

namespace w4 {

bool head_topk_supported(int64_t V, int64_t K, int k) {
  if (K % 64 != 0 || K < 64 || K > 4096 || V < 1 || V > 524288 || k < 1 || k > 64 || k > V) return false;
  return topk_chunk(V, k) != 0;
}

// the GEMV and the selection run one after the other on the stream and share the workspace
size_t head_topk_ws_bytes(int64_t V, int64_t K, int k) {
  const size_t g = gemv_ws_bytes(1, V, K), t = topk_ws_bytes(1, V, k);
  return g > t ? g : t;
}

void launch_head_topk(const uint32_t* qw, const uint16_t* s, const uint16_t* b, const uint16_t* x, float* logits,
                      int32_t* idx, float* val, int V, int K, int k, void* ws, hipStream_t st) {
  launch_gemv(qw, s, b, x, K, logits, V, 1, V, K, ws, st);
  launch_topk(logits, V, 1, V, k, idx, val, ws, st);
}

}  // namespace w4
