// Device helpers for exact top-k selection on 64-bit keys, shared by the top-k kernels and the
// int4 head's fused selection.
//
// Order: value descending, ties to the lower index, -0.0 equal to +0.0.  Each candidate is a
// 64-bit key (orderable(value) << 32) | ~index whose unsigned order is exactly that order (keys
// are unique), so selection is exact and deterministic.
//
// Wave selection (wave_topk, k <= 64, no workgroup barrier): each lane holds E keys; the lane
// whose maximum ranks k-1 among the 64 lane maxima gives the threshold T (at least k keys reach
// it: the k lanes whose maxima do); keys >= T (at most k * E, usually about k) are compacted
// with ballot/mbcnt, and each candidate's rank among them (the count of larger candidates) is
// its output position.  Keys past the end of the data are padding keys that are distinct and
// below every real key, so maxima and ranks never tie.  A workgroup of NW waves selects from
// NW * 64 * E keys: each wave from its share, then the NW sorted lists are merged by rank.
#pragma once

#include "w4_internal.h"

namespace w4 {

__device__ __forceinline__ uint64_t make_key(float v, uint32_t i) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;                      // -0.0 == +0.0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // monotone in the value
  return ((uint64_t)u << 32) | (uint64_t)(~i);
}

__device__ __forceinline__ uint32_t key_index(uint64_t key) { return ~(uint32_t)key; }

// Padding key for position p past the data: high word 0 (every real key's high word is at
// least 0x00800000 for finite logits), low word unique per position.
__device__ __forceinline__ uint64_t pad_key(uint32_t p) { return (uint64_t)p; }

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int src) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, src);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

// 16 keys from 128-byte-aligned LDS with eight 16-byte reads issued back to back.
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void load16(const uint64_t* src, uint64_t (&v)[16]) {
  u64x2 p[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) p[q] = reinterpret_cast<const u64x2*>(src)[q];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    v[2 * q] = p[q][0];
    v[2 * q + 1] = p[q][1];
  }
}

// Number of keys greater than x in a descending list of n <= 64 distinct keys (branchless
// binary search, seven probes).
__device__ __forceinline__ int count_greater(const uint64_t* list, int n, uint64_t x) {
  int lo = 0;
#pragma unroll
  for (int step = 64; step >= 1; step >>= 1) {
    const int probe = min(lo + step, n) - 1;
    if (lo + step <= n && list[probe] > x) lo += step;
  }
  return lo;
}

// The k largest of this wave's 64 * E distinct keys, sorted descending, into out[0..k).
// wm: 128 keys of LDS, cand: 64 * E keys of LDS (both private to the wave).
// Threshold: every lane offers its largest key, or with TWO (k > 48, E > 1) its two largest; the
// one of the offered keys with exactly k - 1 larger ones among them is T, and at least k
// keys reach it.  With one key per lane and k near 64, T is about the smallest lane maximum
// and most keys pass (the rank scan below then goes quadratic); two keys per lane keep the
// candidates near k.  For smaller k one key per lane already does and costs less.
template <int E, bool TWO>
__device__ void wave_topk(const uint64_t (&key)[E], int k, uint64_t* wm, uint64_t* cand,
                          uint64_t* out) {
  const int lane = threadIdx.x & 63;
  constexpr bool two = E > 1 && TWO;
  uint64_t m1 = key[0], m2 = 0;
  if constexpr (two) {
#pragma unroll
    for (int e = 1; e < E; ++e) {
      const uint64_t hi = key[e] > m1 ? key[e] : m1, lo = key[e] > m1 ? m1 : key[e];
      m1 = hi;
      m2 = lo > m2 ? lo : m2;
    }
    wm[64 + lane] = m2;
  } else {
#pragma unroll
    for (int e = 1; e < E; ++e) m1 = key[e] > m1 ? key[e] : m1;
  }
  wm[lane] = m1;
  wave_sync();
  int r1 = 0, r2 = 0;  // LDS reads in batches of 8 x 16 bytes so their latencies overlap
#pragma unroll
  for (int bt = 0; bt < 4; ++bt) {  // the 64 lane maxima
    uint64_t v[16];
    load16(wm + bt * 16, v);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      r1 += v[q] > m1 ? 1 : 0;
      if constexpr (two) r2 += v[q] > m2 ? 1 : 0;
    }
  }
  if constexpr (two) {
#pragma unroll
    for (int bt = 4; bt < 8; ++bt) {  // the 64 second keys
      uint64_t v[16];
      load16(wm + bt * 16, v);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        r1 += v[q] > m1 ? 1 : 0;
        r2 += v[q] > m2 ? 1 : 0;
      }
    }
  }
  // exactly one offered key has rank k - 1: offered keys are distinct
  const bool mine = r1 == k - 1 || (two && r2 == k - 1);
  const uint64_t who = __ballot(mine);
  const uint64_t T = readlane64(r1 == k - 1 ? m1 : m2, (int)__builtin_ctzll(who));
  int c = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool take = key[e] >= T;
    const uint64_t bits = __ballot(take);
    const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0));
    // lanes that drop their key write it to their own dead slot of wm (read before T was
    // chosen), so the write needs no branch
    *(take ? cand + c + before : wm + lane) = key[e];
    c += __builtin_popcountll(bits);
  }
  // pad the candidates to a multiple of 16 with 0, below every real or padding key (c <= 64E,
  // a multiple of 16), so the rank scan reads 16 at a time with its LDS reads overlapped
  const int c16 = (c + 15) & ~15;
  if (lane < c16 - c) cand[c + lane] = 0ull;
  wave_sync();
  for (int i = lane; i < c; i += 64) {
    const uint64_t ki = cand[i];
    int r = 0;
    for (int j = 0; j < c16; j += 16) {
      uint64_t v[16];
      load16(cand + j, v);
#pragma unroll
      for (int q = 0; q < 16; ++q) r += v[q] > ki ? 1 : 0;
    }
    if (r < k) out[r] = ki;
  }
  wave_sync();
}

// A workgroup of NW waves: the k best of NW * 64 * E keys (key[e] of lane l of wave w is element
// w * 64 * E + e * 64 + l of the group's range) into out[0..k) (LDS, read after the final
// barrier).  Each wave selects its sorted k best; the NW sorted lists are then merged by rank:
// survivor i of list w is preceded by the i before it in its own list and by the survivors of
// the other lists that are larger (binary search), and lands at that rank if it is below k.
// LDS layout (keys): NW x 128 lane maxima, NW x 64 survivors, NW x 64 E candidates, 64 out.
template <int NW>
constexpr int grp_surv() { return NW * 128; }
template <int NW>
constexpr int grp_cand() { return NW * 192; }

template <int NW, int E>
constexpr size_t group_lds() {
  return (size_t)(grp_cand<NW>() + NW * 64 * E + 64) * 8;
}

template <int NW, int E>
__device__ __forceinline__ uint64_t* group_out(unsigned char* smem) {
  return reinterpret_cast<uint64_t*>(smem) + grp_cand<NW>() + NW * 64 * E;
}

template <int NW, int E, bool TWO>
__device__ void group_topk(const uint64_t (&key)[E], int k, unsigned char* smem, uint64_t* out) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint64_t* wm = reinterpret_cast<uint64_t*>(smem) + w * 128;
  uint64_t* surv = reinterpret_cast<uint64_t*>(smem) + grp_surv<NW>();
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem) + grp_cand<NW>() + w * 64 * E;
  wave_topk<E, TWO>(key, k, wm, cand, surv + w * 64);
  __syncthreads();
  if (lane < k) {
    const uint64_t x = surv[w * 64 + lane];
    int r = lane;
#pragma unroll
    for (int o = 1; o < NW; ++o) r += count_greater(surv + ((w + o) % NW) * 64, k, x);
    if (r < k) out[r] = x;
  }
  __syncthreads();
}

}  // namespace w4
