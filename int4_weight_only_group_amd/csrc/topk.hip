// logits_argmax_topk: per-row greedy argmax and top-k over f32 logits, on the device.
//
// "The inference engine -- Mojo 1.0 on Metal", "Crossing Mojo 1.0": token selection
// (argmax/top-k) runs on the GPU so only the chosen ids cross to the host instead of the
// per-token logits; "What's inside the engine today": it is bit-exact against the host
// reference.  "engine-mlx", "Tech details": greedy argmax inside the graph.
//
// Order: value descending, ties to the lower index, -0.0 equal to +0.0.  Each candidate is
// a 64-bit key  (orderable(value) << 32) | ~index  whose unsigned order is exactly that
// order (keys are unique), so selection is exact and deterministic.
//
// Block selection (block_topk): each of the 256 threads holds E keys in registers.  The
// block sorts only the 256 per-thread maxima; T, the k-th largest of them, is a key that at
// least k keys reach, so the block's k largest keys are all >= T.  Keys >= T are compacted
// into LDS (their order there does not matter) and sorted; the first k are the answer.  On
// random logits only a few k keys pass the threshold; in the worst case (all equal) all of
// them do and the sort covers the whole block, with the same result.
//
// Wave selection (wave_topk, k <= 64, no workgroup barrier): each lane holds E keys; the lane
// whose maximum ranks k-1 among the 64 lane maxima gives the threshold T (at least k keys
// reach it: the k lanes whose maxima do); keys >= T (at most k * E, usually about k) are
// compacted with ballot/mbcnt, and each candidate's rank among them (the count of larger
// candidates) is its output position.  Keys past the end of the data are padding keys that
// are distinct and below every real key, so maxima and ranks never tie.  A workgroup of four
// waves selects from 4 * 64 * E keys: each wave from its quarter, then one wave from the four
// waves' 4k survivors.
//
// Long rows run in two passes: pass 1 selects each chunk's k best keys into the workspace,
// pass 2 selects the row's k best among them.  Rows of at most 4096 logits take pass 2
// straight from the logits.  Values are re-read from the logits at the chosen index, so
// -0.0 stays -0.0.  k > 64 takes the block selection above.
#include <mutex>

#include "w4_internal.h"
#include "w4_select.h"

namespace w4 {

namespace {

constexpr int kWG = 256;
constexpr int kMaxCand = 8192;  // keys per row after pass 1

// Descending bitonic sort of n (a power of two, >= 2) keys in LDS by the whole workgroup.
__device__ void sort_desc(uint64_t* s, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (n >> 1); i += kWG) {
        const int lo = ((i & ~(stride - 1)) << 1) | (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t a = s[lo], b = s[hi];
        if (desc ? (a < b) : (a > b)) {
          s[lo] = b;
          s[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

__host__ __device__ inline int pow2_ceil(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// The k (<= 256) largest of the block's keys (E per thread), sorted, into s[0..k).
// s must hold max(256, 256 * E) keys; *cnt is an LDS counter.
template <int E>
__device__ void block_topk(const uint64_t (&key)[E], int k, uint64_t* s, int* cnt) {
  const int tid = threadIdx.x;
  uint64_t mx = key[0];
#pragma unroll
  for (int e = 1; e < E; ++e) mx = key[e] > mx ? key[e] : mx;
  s[tid] = mx;
  if (tid == 0) *cnt = 0;
  __syncthreads();
  sort_desc(s, kWG);
  const uint64_t T = s[k - 1];
  int mine = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) mine += key[e] >= T;
  __syncthreads();  // every thread has read T before s is overwritten
  int pos = atomicAdd(cnt, mine);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (key[e] >= T) s[pos++] = key[e];
  __syncthreads();
  const int total = *cnt;
  const int n = pow2_ceil(total < 2 ? 2 : total);
  for (int i = total + tid; i < n; i += kWG) s[i] = 0ull;  // pads sort last
  __syncthreads();
  sort_desc(s, n);
}

// Pass 1: the k best keys of logits[m][c*chunk, (c+1)*chunk) into cand[m][c][0:k).
template <int E>
__global__ __launch_bounds__(kWG) void topk_chunk_kernel(const float* __restrict__ logits,
                                                         int64_t ldl, int V, int k,
                                                         uint64_t* __restrict__ cand) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* s = reinterpret_cast<uint64_t*>(smem);
  __shared__ int cnt;
  const int c = blockIdx.x, m = blockIdx.y;
  const int nchunks = gridDim.x;
  const float* row = logits + (int64_t)m * ldl;
  const int base = c * (E * kWG);
  // all loads first (clamped index, no branch around a load, so none waits for another),
  // then the keys; positions past V get 0, below every key
  float lv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) lv[e] = row[min(base + e * kWG + (int)threadIdx.x, V - 1)];
  uint64_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int v = base + e * kWG + threadIdx.x;  // coalesced: one row segment per e
    key[e] = v < V ? make_key(lv[e], (uint32_t)v) : 0ull;
  }
  block_topk<E>(key, k, s, &cnt);
  uint64_t* out = cand + ((int64_t)m * nchunks + c) * k;
  for (int i = threadIdx.x; i < k; i += kWG) out[i] = s[i];
}

// Pass 2: the k best of a row's ncand keys (from cand, or the logits themselves when
// cand == nullptr) -> indices and logits.
template <int E>
__global__ __launch_bounds__(kWG) void topk_final_kernel(const float* __restrict__ logits,
                                                         int64_t ldl, int V, int k,
                                                         const uint64_t* __restrict__ cand,
                                                         int ncand, int32_t* __restrict__ idx,
                                                         float* __restrict__ val) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* s = reinterpret_cast<uint64_t*>(smem);
  __shared__ int cnt;
  const int m = blockIdx.x;
  const float* row = logits + (int64_t)m * ldl;
  uint64_t key[E];
  if (cand) {
    uint64_t cv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) cv[e] = cand[(int64_t)m * ncand + min(e * kWG + (int)threadIdx.x, ncand - 1)];
#pragma unroll
    for (int e = 0; e < E; ++e) key[e] = e * kWG + (int)threadIdx.x < ncand ? cv[e] : 0ull;
  } else {
    float lv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) lv[e] = row[min(e * kWG + (int)threadIdx.x, ncand - 1)];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = e * kWG + threadIdx.x;
      key[e] = i < ncand ? make_key(lv[e], (uint32_t)i) : 0ull;
    }
  }
  block_topk<E>(key, k, s, &cnt);
  for (int i = threadIdx.x; i < k; i += kWG) {
    uint32_t j = key_index(s[i]);
    if (j >= (uint32_t)V) j = (uint32_t)V - 1;  // unreachable for k <= V; keeps reads in bounds
    idx[(int64_t)m * k + i] = (int32_t)j;
    val[(int64_t)m * k + i] = row[j];
  }
}

// ------------------------------------------------------------------ wave selection (k <= 64)

// Pass 1: the k best keys of logits[m][c*chunk, (c+1)*chunk) into cand[m][c][0:k),
// chunk = 4 * 64 * E.
// TWO: k > 48 (two offered keys per lane in the wave selection, lists stored rotated).
template <int E, bool TWO>
__global__ __launch_bounds__(kWG) void wtopk_chunk_kernel(const float* __restrict__ logits,
                                                          int64_t ldl, int V, int k,
                                                          uint64_t* __restrict__ cand) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int c = blockIdx.x, m = blockIdx.y;
  const int nchunks = gridDim.x;
  const float* row = logits + (int64_t)m * ldl;
  const int base = c * (4 * 64 * E) + (threadIdx.x >> 6) * 64 * E + (threadIdx.x & 63);
  float lv[E];  // all loads first: clamped, unconditional, so none waits for another
#pragma unroll
  for (int e = 0; e < E; ++e) lv[e] = row[min(base + e * 64, V - 1)];
  uint64_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int v = base + e * 64;  // coalesced: one 256-byte row segment per e and wave
    key[e] = v < V ? make_key(lv[e], (uint32_t)v) : pad_key(~(uint32_t)v & 0x7fffffffu);
  }
  uint64_t* out = group_out<4, E>(smem);
  group_topk<4, E, TWO>(key, k, smem, out);
  // With TWO the list is stored rotated by 17 c: pass 2 reads candidate i into lane i % 64, so sorted
  // lists stored as-is would give lane l the rank-l key of every list (k = 64: lane 63 then
  // holds a high maximum, the threshold admits almost every key and the rank scan goes
  // quadratic).  Rotated, each lane sees mixed ranks.  Pass 2 selects by key, so the order of
  // the stored keys is free.
  uint64_t* dst = cand + ((int64_t)m * nchunks + c) * k;
  for (int i = threadIdx.x; i < k; i += kWG) dst[TWO ? (i + 17 * c) % k : i] = out[i];
}

// Pass 2: the k best of a row's ncand keys (from cand, or the logits themselves when
// cand == nullptr) -> indices and logits.
template <int E, bool TWO>
__global__ __launch_bounds__(kWG) void wtopk_final_kernel(const float* __restrict__ logits,
                                                          int64_t ldl, int V, int k,
                                                          const uint64_t* __restrict__ cand,
                                                          int ncand, int32_t* __restrict__ idx,
                                                          float* __restrict__ val) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int m = blockIdx.x;
  const float* row = logits + (int64_t)m * ldl;
  const int base = (threadIdx.x >> 6) * 64 * E + (threadIdx.x & 63);
  uint64_t key[E];
  if (cand) {  // all loads first: clamped, unconditional, so none waits for another
    uint64_t cv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) cv[e] = cand[(int64_t)m * ncand + min(base + e * 64, ncand - 1)];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = base + e * 64;
      key[e] = i < ncand ? cv[e] : pad_key(~(uint32_t)i & 0x7fffffffu);
    }
  } else {
    float lv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) lv[e] = row[min(base + e * 64, ncand - 1)];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = base + e * 64;
      key[e] = i < ncand ? make_key(lv[e], (uint32_t)i) : pad_key(~(uint32_t)i & 0x7fffffffu);
    }
  }
  uint64_t* out = group_out<4, E>(smem);
  group_topk<4, E, TWO>(key, k, smem, out);
  for (int i = threadIdx.x; i < k; i += kWG) {
    uint32_t j = key_index(out[i]);
    if (j >= (uint32_t)V) j = (uint32_t)V - 1;  // unreachable for k <= V; keeps reads in bounds
    idx[(int64_t)m * k + i] = (int32_t)j;
    val[(int64_t)m * k + i] = row[j];
  }
}

// Pass 1 of the group-maxima selection (k <= 64): gkeys[m][g] = the largest key among
// logits[m][64 g, 64 g + 64).  A workgroup of 256 threads covers 4096 logits: thread t holds
// 16 consecutive ones (four 16-byte loads when the row allows them), four lanes a group.
__global__ __launch_bounds__(kWG) void group_max_kernel(const float* __restrict__ logits, int64_t ldl, int V,
                                                         int G, uint64_t* __restrict__ gkeys, int vec) {
  const int m = blockIdx.y, t = threadIdx.x;
  const float* row = logits + (int64_t)m * ldl;
  const int base = blockIdx.x * 4096 + t * 16;
  float v[16];
  if (vec && base + 16 <= V) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = reinterpret_cast<const float4*>(row + base)[q];
      v[4 * q] = f.x;
      v[4 * q + 1] = f.y;
      v[4 * q + 2] = f.z;
      v[4 * q + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = row[min(base + j, V - 1)];
  }
  uint64_t mx = 0;  // below every real key
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint64_t x = base + j < V ? make_key(v[j], (uint32_t)(base + j)) : 0ull;
    mx = x > mx ? x : mx;
  }
  // the four lanes of a group are one quad
  uint64_t y = quad_swap64<0xB1>(mx);
  mx = y > mx ? y : mx;
  y = quad_swap64<0x4E>(mx);
  mx = y > mx ? y : mx;
  const int g = base / 64;
  if ((t & 3) == 0 && g < G) gkeys[(int64_t)m * G + g] = mx;
}

template <int E>
void launch_wfinal(const float* logits, int64_t ldl, int M, int V, int k, const uint64_t* cand,
                   int ncand, int32_t* idx, float* val, hipStream_t st) {
  if (k > 48)
    hipLaunchKernelGGL((wtopk_final_kernel<E, true>), dim3(M), dim3(kWG), (group_lds<4, E>()), st, logits,
                       ldl, V, k, cand, ncand, idx, val);
  else
    hipLaunchKernelGGL((wtopk_final_kernel<E, false>), dim3(M), dim3(kWG), (group_lds<4, E>()), st, logits,
                       ldl, V, k, cand, ncand, idx, val);
}

void wfinal_pass(const float* logits, int64_t ldl, int M, int V, int k, const uint64_t* cand,
                 int ncand, int32_t* idx, float* val, hipStream_t st) {
  if (ncand <= 256)
    launch_wfinal<1>(logits, ldl, M, V, k, cand, ncand, idx, val, st);
  else if (ncand <= 1024)
    launch_wfinal<4>(logits, ldl, M, V, k, cand, ncand, idx, val, st);
  else if (ncand <= 2048)
    launch_wfinal<8>(logits, ldl, M, V, k, cand, ncand, idx, val, st);
  else if (ncand <= 4096)
    launch_wfinal<16>(logits, ldl, M, V, k, cand, ncand, idx, val, st);
  else
    launch_wfinal<32>(logits, ldl, M, V, k, cand, ncand, idx, val, st);
}

template <int E>
void launch_final(const float* logits, int64_t ldl, int M, int V, int k, const uint64_t* cand,
                  int ncand, int32_t* idx, float* val, hipStream_t st) {
  hipLaunchKernelGGL((topk_final_kernel<E>), dim3(M), dim3(kWG), (size_t)E * kWG * 8, st, logits,
                     ldl, V, k, cand, ncand, idx, val);
}

void final_pass(const float* logits, int64_t ldl, int M, int V, int k, const uint64_t* cand,
                int ncand, int32_t* idx, float* val, hipStream_t st) {
  if (ncand <= kWG)
    launch_final<1>(logits, ldl, M, V, k, cand, ncand, idx, val, st);
  else if (ncand <= 4 * kWG)
    launch_final<4>(logits, ldl, M, V, k, cand, ncand, idx, val, st);
  else if (ncand <= 8 * kWG)
    launch_final<8>(logits, ldl, M, V, k, cand, ncand, idx, val, st);
  else if (ncand <= 16 * kWG)
    launch_final<16>(logits, ldl, M, V, k, cand, ncand, idx, val, st);
  else
    launch_final<32>(logits, ldl, M, V, k, cand, ncand, idx, val, st);
}

}  // namespace

// Chunk (logits per pass-1 block) for a row of V logits: 4096, or 8192 when 4096-chunks
// would leave more than kMaxCand candidates; 0 when even that is too many.
int topk_chunk(int64_t V, int k) {
  if (V <= 4096) return (int)pow2_ceil((int)V);  // single pass
  for (int chunk = 4096; chunk <= 8192; chunk <<= 1)
    if (((V + chunk - 1) / chunk) * k <= kMaxCand) return chunk;
  return 0;
}

// k <= 64 and rows longer than 4096 logits (every such shape the entry accepts: V k <= 2^26):
// group maxima of 64 logits (pass 1), then one selection workgroup per row
// (group_select_kernel); otherwise chunks of topk_chunk() logits whose k best go to the
// workspace, then a final pass over those.
bool topk_groups(int64_t V, int k) {
  return k <= 64 && V > 4096 && gs_prereduce((V + 63) / 64, 64, k) != 0;
}

size_t topk_ws_bytes(int64_t M, int64_t V, int k) {
  if (V <= 4096) return 0;
  if (topk_groups(V, k)) return (size_t)M * (size_t)((V + 63) / 64) * sizeof(uint64_t);
  const int chunk = topk_chunk(V, k);
  if (chunk == 0) return 0;
  return (size_t)M * (size_t)((V + chunk - 1) / chunk) * (size_t)k * sizeof(uint64_t);
}

void launch_topk(const float* logits, int64_t ldl, int M, int V, int k, int32_t* idx, float* val,
                 void* ws, hipStream_t st) {
  static std::once_flag lds_attr[kMaxDevices];  // several kernels use more than 64 KB of LDS
  once_per_device(lds_attr, [] {
    for (const void* f : {reinterpret_cast<const void*>(wtopk_chunk_kernel<32, false>),
                          reinterpret_cast<const void*>(wtopk_chunk_kernel<32, true>),
                          reinterpret_cast<const void*>(wtopk_final_kernel<32, false>),
                          reinterpret_cast<const void*>(wtopk_final_kernel<32, true>)})
      (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)group_lds<4, 32>());
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(group_select_kernel<>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)gs_lds_bytes(kGsMaxKeys));
  });
  const bool wave = k <= 64;
  if (V <= 4096) {
    if (wave)
      wfinal_pass(logits, ldl, M, V, k, nullptr, V, idx, val, st);
    else
      final_pass(logits, ldl, M, V, k, nullptr, V, idx, val, st);
    return;
  }
  uint64_t* cand = reinterpret_cast<uint64_t*>(ws);
  if (topk_groups(V, k)) {
    const int G0 = (V + 63) / 64;
    const int vec = ((uintptr_t)logits & 15u) == 0 && ldl % 4 == 0;
    hipLaunchKernelGGL(group_max_kernel, dim3((V + 4095) / 4096, M), dim3(kWG), 0, st, logits, ldl, V, G0, cand,
                       vec);
    const int P = gs_prereduce(G0, 64, k);
    const int G = (G0 + P - 1) / P;
    const int cap = gs_cap(G, 64 * P);
    hipLaunchKernelGGL(group_select_kernel<>, dim3(M), dim3(kGsThreads), gs_lds_bytes(cap), st, logits, ldl, V, k,
                       cand, G0, 64, P, cap, idx, val);
    return;
  }
  const int chunk = topk_chunk(V, k);
  const int nchunks = (V + chunk - 1) / chunk;
  if (wave) {
    const dim3 grid(nchunks, M);
    if (chunk == 4096 && k > 48)
      hipLaunchKernelGGL((wtopk_chunk_kernel<16, true>), grid, dim3(kWG), (group_lds<4, 16>()), st, logits,
                         ldl, V, k, cand);
    else if (chunk == 4096)
      hipLaunchKernelGGL((wtopk_chunk_kernel<16, false>), grid, dim3(kWG), (group_lds<4, 16>()), st, logits,
                         ldl, V, k, cand);
    else if (k > 48)
      hipLaunchKernelGGL((wtopk_chunk_kernel<32, true>), grid, dim3(kWG), (group_lds<4, 32>()), st, logits,
                         ldl, V, k, cand);
    else
      hipLaunchKernelGGL((wtopk_chunk_kernel<32, false>), grid, dim3(kWG), (group_lds<4, 32>()), st, logits,
                         ldl, V, k, cand);
    wfinal_pass(logits, ldl, M, V, k, cand, nchunks * k, idx, val, st);
    return;
  }
  if (chunk == 4096)
    hipLaunchKernelGGL((topk_chunk_kernel<16>), dim3(nchunks, M), dim3(kWG), (size_t)chunk * 8, st,
                       logits, ldl, V, k, cand);
  else
    hipLaunchKernelGGL((topk_chunk_kernel<32>), dim3(nchunks, M), dim3(kWG), (size_t)chunk * 8, st,
                       logits, ldl, V, k, cand);
  final_pass(logits, ldl, M, V, k, cand, nchunks * k, idx, val, st);
}

// ------------------------------------------------------------ allocation-free variant
// Callers that cannot allocate device memory (code under graph capture, tight serving loops)
// get the pass-1 candidates in a file-scope device array instead of a workspace.  Host code
// never passes the array's name to a kernel: on the host that name is only a stand-in, so
// the device address is fetched once per device with hipGetSymbolAddress and kept.
namespace {
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
}  // namespace

}  // namespace w4

// One array per device, held until the process ends; calls on one device share it.
static __device__ __align__(256) uint64_t scratch[w4::kTopkScratchBytes / sizeof(uint64_t)];

namespace w4 {

void* topk_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) {
      g_scratch_ptr[dev] = p;
    } else {
      (void)hipGetLastError();
      g_scratch_ptr[dev] = nullptr;
    }
  });
  return g_scratch_ptr[dev];
}

}  // namespace w4
