// logits_argmax_topk: per-row greedy argmax and top-k over f32 logits, on the device.
//
// "The inference engine -- Mojo 1.0 on Metal", "Crossing Mojo 1.0": token selection
// (argmax/top-k) runs on the GPU so only the chosen ids cross to the host instead of the
// per-token logits; "What's inside the engine today": it is bit-exact against the host
// reference.  "engine-mlx", "Tech details": greedy argmax inside the graph.
//
// Order: value descending, ties to the lower index, -0.0 equal to +0.0.  Each candidate is
// a 64-bit key  (orderable(value) << 32) | ~index  whose unsigned order is exactly that
// order, so selection is a plain descending sort of keys (deterministic, exact).
//
// Two passes for long rows: pass 1 splits a row into chunks of `chunk` logits and keeps
// each chunk's k best keys (bitonic sort in LDS); pass 2 sorts a row's chunk winners and
// writes the k best.  Short rows (V <= 4096) take pass 2 straight from the logits.  The
// output values are re-read from the logits at the chosen index, so -0.0 stays -0.0.
#include "w4_internal.h"

namespace w4 {

namespace {

constexpr int kWG = 256;
constexpr int kMaxSort = 8192;  // keys per LDS sort (64 KB)

__device__ __forceinline__ uint64_t make_key(float v, uint32_t i) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;                      // -0.0 == +0.0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // monotone in the value
  return ((uint64_t)u << 32) | (uint64_t)(~i);
}

__device__ __forceinline__ uint32_t key_index(uint64_t key) { return ~(uint32_t)key; }

// Descending bitonic sort of n (power of two) keys in LDS by the whole workgroup.
__device__ void sort_desc(uint64_t* s, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (n >> 1); i += kWG) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
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

// Pass 1: keys of logits[m][c*chunk : (c+1)*chunk) -> k best into cand[m][c][0:k].
__global__ __launch_bounds__(kWG) void topk_chunk_kernel(const float* __restrict__ logits,
                                                         int64_t ldl, int V, int k, int chunk,
                                                         uint64_t* __restrict__ cand) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* s = reinterpret_cast<uint64_t*>(smem);
  const int c = blockIdx.x, m = blockIdx.y;
  const int nchunks = gridDim.x;
  const float* row = logits + (int64_t)m * ldl;
  const int base = c * chunk;
  for (int i = threadIdx.x; i < chunk; i += kWG) {
    const int v = base + i;
    s[i] = (v < V) ? make_key(row[v], (uint32_t)v) : 0ull;  // 0 sorts below every finite key
  }
  __syncthreads();
  sort_desc(s, chunk);
  uint64_t* out = cand + ((int64_t)m * nchunks + c) * k;
  for (int i = threadIdx.x; i < k; i += kWG) out[i] = s[i];
}

// Pass 2: sort n candidate keys per row (from cand, or straight from the logits when
// cand == nullptr) and write the k best indices and their logits.
__global__ __launch_bounds__(kWG) void topk_final_kernel(const float* __restrict__ logits,
                                                         int64_t ldl, int V, int k,
                                                         const uint64_t* __restrict__ cand,
                                                         int ncand, int npow2,
                                                         int32_t* __restrict__ idx,
                                                         float* __restrict__ val) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* s = reinterpret_cast<uint64_t*>(smem);
  const int m = blockIdx.x;
  const float* row = logits + (int64_t)m * ldl;
  for (int i = threadIdx.x; i < npow2; i += kWG) {
    uint64_t key = 0ull;
    if (i < ncand) key = cand ? cand[(int64_t)m * ncand + i] : make_key(row[i], (uint32_t)i);
    s[i] = key;
  }
  __syncthreads();
  sort_desc(s, npow2);
  for (int i = threadIdx.x; i < k; i += kWG) {
    uint32_t j = key_index(s[i]);
    if (j >= (uint32_t)V) j = (uint32_t)V - 1;  // unreachable for k <= V; keeps reads in bounds
    idx[(int64_t)m * k + i] = (int32_t)j;
    val[(int64_t)m * k + i] = row[j];
  }
}

}  // namespace

int topk_chunk(int64_t V, int k) {
  if (V <= 4096) return (int)pow2_ceil((int)V);  // single pass
  int chunk = 4096;
  while (((V + chunk - 1) / chunk) * k > kMaxSort && chunk < kMaxSort) chunk <<= 1;
  if (((V + chunk - 1) / chunk) * k > kMaxSort) return 0;
  return chunk;
}

size_t topk_ws_bytes(int64_t M, int64_t V, int k) {
  if (V <= 4096) return 0;
  const int chunk = topk_chunk(V, k);
  if (chunk == 0) return 0;
  return (size_t)M * (size_t)((V + chunk - 1) / chunk) * (size_t)k * sizeof(uint64_t);
}

void launch_topk(const float* logits, int64_t ldl, int M, int V, int k, int32_t* idx, float* val,
                 void* ws, hipStream_t st) {
  if (V <= 4096) {
    const int np = pow2_ceil(V < 2 ? 2 : V);
    hipLaunchKernelGGL(topk_final_kernel, dim3(M), dim3(kWG), (size_t)np * 8, st, logits, ldl, V,
                       k, (const uint64_t*)nullptr, V, np, idx, val);
    return;
  }
  const int chunk = topk_chunk(V, k);
  const int nchunks = (V + chunk - 1) / chunk;
  uint64_t* cand = reinterpret_cast<uint64_t*>(ws);
  hipLaunchKernelGGL(topk_chunk_kernel, dim3(nchunks, M), dim3(kWG), (size_t)chunk * 8, st,
                     logits, ldl, V, k, chunk, cand);
  const int ncand = nchunks * k;
  const int np = pow2_ceil(ncand < 2 ? 2 : ncand);
  hipLaunchKernelGGL(topk_final_kernel, dim3(M), dim3(kWG), (size_t)np * 8, st, logits, ldl, V, k,
                     (const uint64_t*)cand, ncand, np, idx, val);
}

}  // namespace w4
