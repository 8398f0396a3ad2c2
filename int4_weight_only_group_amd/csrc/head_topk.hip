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
//    workgroup's largest selection key: a pre-selection of one key per 16 rows (per 2-4 rows
//    when a row spans several waves).
//  * head_select_kernel, one workgroup: T1 = the k-th largest of those group maxima.  A logit
//    in the top k is >= T1 (at least k group maxima reach T1), so its group's maximum is >= T1
//    too: every top-k logit lies in one of the k groups whose maxima are the k largest.  Only
//    those groups' rows (at most 8192 logits) are re-read, their keys >= T1 kept, and the k
//    best of those selected.  Every step is exact; values are re-read from the logits, so each
//    is the stored logit bit for bit.
// Group maxima are pre-reduced P at a time (P consecutive workgroups, so P * rows_per_wg
// consecutive rows) until at most 4096 remain, which bounds the selection's registers.
#include <mutex>

#include "w4_internal.h"
#include "w4_select.h"

namespace w4 {

namespace {

constexpr int kSelWaves = 16;           // one workgroup of 16 waves
constexpr int kSelThreads = kSelWaves * 64;
constexpr int kMaxGroups = 4096;        // group maxima after pre-reduction (4 per lane)
constexpr int kMaxCandRows = 8192;      // rows re-read: k groups x rows per group

// LDS (keys): 1024 level-2 slots; wave 0's area (128 lane maxima, 1024 candidates, 64 survivors:
// it also runs the 1024-slot rounds); the other waves' areas (128 + 64 E0 + 64 each), which the
// pool of kept keys reuses once level 2 is done.
constexpr int kArea0 = 128 + 64 * 16 + 64;
template <int E0>
constexpr int area1() { return 128 + 64 * E0 + 64; }
template <int E0>
constexpr size_t select_lds() {
  constexpr int rest = (kSelWaves - 1) * area1<E0>() > kMaxCandRows ? (kSelWaves - 1) * area1<E0>() : kMaxCandRows;
  return (size_t)(kSelWaves * 64 + kArea0 + rest) * 8;
}

// level-2 slots: survivor j of wave w's sorted list goes to slot w * k + (j + 17 w) % k, so a lane
// gets keys of different ranks (aligned sorted lists make the lane-maxima threshold weak)
__device__ __forceinline__ int rot_slot(int w, int j, int k) { return w * k + (j + 17 * w) % k; }

template <int E0, bool TWO>
__global__ __launch_bounds__(kSelThreads) void head_select_kernel(
    const float* __restrict__ logits, int V, int k, const uint64_t* __restrict__ wgmax, int nwg, int P,
    int rows_per_group, int32_t* __restrict__ idx, float* __restrict__ val) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* slots = reinterpret_cast<uint64_t*>(smem);            // 16 x 64 level-2 slots
  uint64_t* area0 = slots + kSelWaves * 64;
  uint64_t* pool = area0 + kArea0;                                // after level 2: kept keys
  __shared__ uint64_t top_groups[64];
  __shared__ int npool;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ng = (nwg + P - 1) / P;  // groups after pre-reduction

  // 1. group maxima (pre-reduced over P workgroups), E0 per lane; up to 8 rounds' loads together
  uint64_t key[E0];
#pragma unroll
  for (int e = 0; e < E0; ++e) key[e] = 0;
#pragma unroll 8
  for (int p = 0; p < P; ++p) {
    uint64_t v[E0];
#pragma unroll
    for (int e = 0; e < E0; ++e) v[e] = wgmax[min((w * 64 * E0 + e * 64 + lane) * P + p, nwg - 1)];
#pragma unroll
    for (int e = 0; e < E0; ++e) {
      const int g = w * 64 * E0 + e * 64 + lane;
      if (g < ng && g * P + p < nwg) key[e] = v[e] > key[e] ? v[e] : key[e];
    }
  }
#pragma unroll
  for (int e = 0; e < E0; ++e) {  // positions past the groups: distinct padding below every real key
    const int g = w * 64 * E0 + e * 64 + lane;
    if (g >= ng) key[e] = pad_key(~(uint32_t)g & 0x7fffffffu);
  }
  if (tid == 0) npool = 0;

  // 2. level 1: each wave's k largest group maxima; level 2: wave 0 selects the k largest overall
  uint64_t* wm = w == 0 ? area0 : pool + (w - 1) * area1<E0>();
  uint64_t* surv = w == 0 ? area0 + kArea0 - 64 : wm + area1<E0>() - 64;
  wave_topk<E0, TWO>(key, k, wm, wm + 128, surv);
  for (int j = lane; j < k; j += 64) slots[rot_slot(w, j, k)] = surv[j];
  __syncthreads();
  if (w == 0) {
    uint64_t key2[kSelWaves];
#pragma unroll
    for (int e = 0; e < kSelWaves; ++e) {
      const int sidx = e * 64 + lane;
      key2[e] = sidx < kSelWaves * k ? slots[sidx] : pad_key((1u << 30) | (uint32_t)sidx);
    }
    wave_topk<kSelWaves, TWO>(key2, k, wm, wm + 128, top_groups);
  }
  __syncthreads();
  const uint64_t T1 = top_groups[k - 1];

  // 3. re-read the rows of the k groups with the largest maxima, keep keys >= T1.  With fewer
  // than k groups the selected list ends in padding keys (below every real one): only its first
  // min(k, ng) entries are groups.
  const int nsel = min(k, ng);
  const int ncr = nsel * rows_per_group;
  for (int i = tid; i < ncr; i += kSelThreads) {
    const uint32_t g = key_index(top_groups[i / rows_per_group]) / (uint32_t)rows_per_group;  // < ng
    const int64_t row = (int64_t)g * rows_per_group + i % rows_per_group;
    if (g < (uint32_t)ng && row < V) {
      const uint64_t kk = make_key(logits[row], (uint32_t)row);
      if (kk >= T1) pool[atomicAdd(&npool, 1)] = kk;
    }
  }
  __syncthreads();

  // 4. wave 0: the k best of the kept keys, 1024 slots per round (the best so far plus new keys)
  if (w != 0) return;
  const int n = npool;  // >= k: the k group maxima themselves
  uint64_t* best = top_groups;  // reuse: the group list is no longer needed
  int used = 0, have = 0;
  do {
    uint64_t kb[kSelWaves];
#pragma unroll
    for (int e = 0; e < kSelWaves; ++e) {
      const int j = e * 64 + lane;
      const int p = used + j - have;
      kb[e] = j < have ? best[j] : p < n ? pool[p] : pad_key(~(uint32_t)j & 0x7fffffffu);
    }
    used += kSelWaves * 64 - have;
    wave_sync();  // every lane has read `best` before the selection rewrites it
    wave_topk<kSelWaves, TWO>(kb, k, wm, wm + 128, best);
    have = k;
  } while (used < n);
  for (int i = lane; i < k; i += 64) {
    uint32_t j = key_index(best[i]);
    if (j >= (uint32_t)V) j = (uint32_t)V - 1;  // unreachable for k <= V; keeps reads in bounds
    idx[i] = (int32_t)j;
    val[i] = logits[j];
  }
}

struct SelPlan {
  int P, ng, E0, rows_per_group;
};

SelPlan sel_plan(const HeadGemvPlan& g) {
  SelPlan s;
  s.P = 1;
  while ((g.nwg + s.P - 1) / s.P > kMaxGroups) s.P *= 2;
  s.ng = (g.nwg + s.P - 1) / s.P;
  s.rows_per_group = g.rows_per_wg * s.P;
  const int pl = (s.ng + kSelThreads - 1) / kSelThreads;
  s.E0 = pl <= 1 ? 1 : pl <= 2 ? 2 : 4;
  return s;
}

template <int E0>
void launch_select(const float* logits, int V, int k, const uint64_t* wgmax, int nwg, const SelPlan& s, int32_t* idx,
                   float* val, hipStream_t st) {
  static std::once_flag lds_attr[kMaxDevices];
  once_per_device(lds_attr, [] {
    for (const void* f : {reinterpret_cast<const void*>(head_select_kernel<E0, false>),
                          reinterpret_cast<const void*>(head_select_kernel<E0, true>)})
      (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)select_lds<E0>());
  });
  if (k > 48)
    hipLaunchKernelGGL((head_select_kernel<E0, true>), dim3(1), dim3(kSelThreads), select_lds<E0>(), st, logits, V, k,
                       wgmax, nwg, s.P, s.rows_per_group, idx, val);
  else
    hipLaunchKernelGGL((head_select_kernel<E0, false>), dim3(1), dim3(kSelThreads), select_lds<E0>(), st, logits, V,
                       k, wgmax, nwg, s.P, s.rows_per_group, idx, val);
}

}  // namespace

bool head_topk_supported(int64_t V, int64_t K, int k) {
  if (K % 64 != 0 || K < 64 || K > 4096 || V < 1 || V >= ((int64_t)1 << 30) || k < 1 || k > 64 || k > V) return false;
  const SelPlan s = sel_plan(head_gemv_plan(V, K));
  return (int64_t)k * s.rows_per_group <= kMaxCandRows;
}

size_t head_topk_ws_bytes(int64_t V, int64_t K, int) {
  return (size_t)head_gemv_plan(V, K).nwg * sizeof(uint64_t);
}

void launch_head_topk(const uint32_t* qw, const uint16_t* s, const uint16_t* b, const uint16_t* x, float* logits,
                      int32_t* idx, float* val, int V, int K, int k, void* ws, hipStream_t st) {
  const HeadGemvPlan g = head_gemv_plan(V, K);
  uint64_t* wgmax = reinterpret_cast<uint64_t*>(ws);
  launch_gemv_head(qw, s, b, x, logits, V, K, wgmax, st);
  const SelPlan sp = sel_plan(g);
  switch (sp.E0) {
    case 1: launch_select<1>(logits, V, k, wgmax, g.nwg, sp, idx, val, st); break;
    case 2: launch_select<2>(logits, V, k, wgmax, g.nwg, sp, idx, val, st); break;
    default: launch_select<4>(logits, V, k, wgmax, g.nwg, sp, idx, val, st); break;
  }
}

}  // namespace w4
