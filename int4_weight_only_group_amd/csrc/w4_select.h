// Device helpers for exact top-k selection on 64-bit keys: the wave and workgroup selections and
// the group-maxima selection kernel of topk.hip.
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

// The value of the lane whose index differs in bit 0 (CTRL 0xB1) or bit 1 (0x4E): a DPP
// quad permute, every lane of the wave active.
template <int CTRL>
__device__ __forceinline__ uint32_t quad_swap(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ uint64_t quad_swap64(uint64_t v) {
  return ((uint64_t)quad_swap<CTRL>((uint32_t)(v >> 32)) << 32) | quad_swap<CTRL>((uint32_t)v);
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

// ------------------------------------------------ group-maxima selection (one workgroup)
// Top k (k <= 64) of a row from the largest key of each group of its logits.  T, the k-th
// largest group key, is reached by k distinct keys of the row, so the row's k-th best key is
// >= T and so is every key of its top k; the group of such a key has a maximum >= T, i.e. it is
// one of the k groups whose keys are >= T.  Any lower bound L <= T keeps this true for the
// groups whose keys are >= L: the selection takes L from the first radix digit of the group
// keys (the digit d at which the count from the top reaches k; at least k group keys have a
// top digit >= d, so T >= d << 52) whenever that admits few groups, and the exact T otherwise.
// Only the admitted groups' logits are read again; their keys >= L (at least the k largest
// group maxima) hold the row's top k, ranked directly when there are few, else selected by
// radix select again.  Every step is exact; values come from the logits (-0.0 stays -0.0).
constexpr int kGsThreads = 1024;   // threads of the selection workgroup
constexpr int kGsBins = 4096;      // radix digits of 12 bits (4 bins per thread)
constexpr int kGsRank = 256;       // matching keys ranked directly from this few on
constexpr int kGsMaxKeys = 16384;  // group keys (after pre-reduction) / re-read keys in LDS
constexpr int kGsSel = 256;        // groups admitted by the first-digit bound at most
constexpr int kGsKeyRegs = 8;      // group keys per thread (held in registers)
constexpr int kGsMaxGroups = kGsKeyRegs * kGsThreads;  // group keys after pre-reduction

// LDS bytes of group_select_kernel for cap keys: keys, the rank pool, the histogram, 8 ints
// and kGsThreads / 64 wave totals
__host__ __device__ constexpr size_t gs_lds_bytes(int cap) {
  return (size_t)(((cap + 15) & ~15) + kGsRank) * 8 + (size_t)(kGsBins + 8 + kGsThreads / 64) * 4;
}

// Keys group_select_kernel holds in LDS for G group keys of gsp logits each: the group keys,
// and the re-read logits of up to kGsSel groups (at least k groups: k gsp <= kGsMaxKeys).
__host__ __device__ constexpr int gs_cap(int G, int gsp) {
  const int re = (int64_t)kGsSel * gsp < kGsMaxKeys ? kGsSel * gsp : kGsMaxKeys;
  return G > re ? G : re;
}

// Number of keys of pool[0 .. n) larger than x; pool is padded with zeros (below every real
// key) to a multiple of 16, read 16 at a time so the LDS reads overlap.
__device__ __forceinline__ int rank_in(const uint64_t* pool, int n, uint64_t x) {
  int r = 0;
  for (int j = 0; j < n; j += 16) {
    uint64_t v[16];
    load16(pool + j, v);
#pragma unroll
    for (int q = 0; q < 16; ++q) r += v[q] > x ? 1 : 0;
  }
  return r;
}

// One radix round's crossing: hist holds the counts of the current digit over the keys that
// still match; the digit d at which the count from the top reaches kk goes to misc[0], the keys
// in higher bins to misc[1], the keys in bin d to misc[2].  Every thread calls it; two
// workgroup barriers, after which misc may be read.  wt: kGsThreads / 64 ints of LDS.
__device__ inline void crossing_digit(const int* hist, int kk, int* misc, int* wt) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // thread t holds bins 4t .. 4t + 3 (one 16-byte read); counts from the top digit down
  const int4 hv = reinterpret_cast<const int4*>(hist)[tid];
  const int h0 = hv.x, h1 = hv.y, h2 = hv.z, h3 = hv.w;
  const int s = h0 + h1 + h2 + h3;
  int S = s;  // keys in bins >= 4t within this wave's range
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_down(S, o);
    if (lane + o < 64) S += u;
  }
  if (lane == 0) wt[w] = S;
  __syncthreads();
#pragma unroll
  for (int v = 1; v < kGsThreads / 64; ++v)
    if (v > w) S += wt[v];  // keys in the later waves' bins
  const int above = S - s;  // keys in bins > 4t + 3
  if (above < kk && kk <= S) {  // exactly one thread
    int c = above, d = 4 * tid, cnt = h0;
    if (c + h3 >= kk) {
      d = 4 * tid + 3, cnt = h3;
    } else if ((c += h3) + h2 >= kk) {
      d = 4 * tid + 2, cnt = h2;
    } else if ((c += h2) + h1 >= kk) {
      d = 4 * tid + 1, cnt = h1;
    } else {
      c += h1;
    }
    misc[0] = d;
    misc[1] = c;
    misc[2] = cnt;
  }
  __syncthreads();
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves: shifts by 1, 2, 4, 8
// within each row of 16 lanes (zero from before the row start), then the running total of row
// 0 into rows 1 and 3 and that of rows 0-1 into rows 2 and 3.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, true);
}
__device__ __forceinline__ int wave_prefix_sum(int v) {
  v += dpp_i<0x111>(v);       // row_shr:1
  v += dpp_i<0x112>(v);       // row_shr:2
  v += dpp_i<0x114>(v);       // row_shr:4
  v += dpp_i<0x118>(v);       // row_shr:8
  v += dpp_i<0x142, 0xA>(v);  // row_bcast15 into rows 1 and 3
  v += dpp_i<0x143, 0xC>(v);  // row_bcast31 into rows 2 and 3
  return v;
}

// Slot of a key's first digit (its top 12 bits) in the first-round histogram: its rank from the
// top, 4095 - digit, so that lane l of one wave holds the 64 slots 64 l .. 64 l + 63 (adjacent
// digits, where the counts of a row cluster, are adjacent words in distinct banks).
__device__ __forceinline__ int first_slot(uint64_t x) { return 4095 - (int)(x >> 52); }

// The first round's crossing, by wave 0 alone (no workgroup barrier; hist in the first_slot
// layout): lane l sums the bins of ranks 64 l .. 64 l + 63 (sixteen 16-byte reads, lane l
// starting at its (l mod 16)-th, so that each 16 lanes of a read cover all 64 banks); the lane
// whose prefix sum from the top first reaches kk holds the crossing digit, and the same over
// that lane's 64 bins (one per lane) finds it.  Writes
// misc[0] = digit, misc[1] = keys with higher digits, misc[2] = keys with this digit.  At least
// kk keys must be counted.  Called by the 64 lanes of one wave.
__device__ inline void first_crossing(const int* hist, int kk, int* misc) {
  const int lane = threadIdx.x & 63;
  int s = 0;
  const int4* row = reinterpret_cast<const int4*>(hist + lane * 64);
  int4 v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = row[(j + lane) & 15];  // the sum's order is free
#pragma unroll
  for (int j = 0; j < 16; ++j) s += v[j].x + v[j].y + v[j].z + v[j].w;
  const int pre = wave_prefix_sum(s);
  const uint64_t hit = __ballot(pre >= kk);
  const int L = (int)__builtin_ctzll(hit);  // hit != 0: the total is >= kk
  const int above = __builtin_amdgcn_readlane(pre - s, L);
  const int c = hist[L * 64 + lane];  // rank 64 L + lane
  const int pre2 = above + wave_prefix_sum(c);
  const uint64_t hit2 = __ballot(pre2 >= kk);
  if (lane == (int)__builtin_ctzll(hit2)) {
    misc[0] = 4095 - (64 * L + lane);
    misc[1] = pre2 - c;
    misc[2] = c;
  }
}

// The kk-th largest (1 <= kk <= n) of the n distinct keys A[0..n) in LDS, by the whole
// workgroup (every thread calls it; all get the result).  Radix select from the top, 12 bits a
// round (4 in the last): a histogram of the next digit over the keys matching the digits
// chosen so far, the digit at which the count from the top reaches kk, then the next digit
// among the keys with that one; once at most kGsRank keys match (after at most 6 rounds, keys
// being distinct) they are ranked by counting the larger ones.  hist: kGsBins ints, misc: 8
// ints, wt: kGsThreads / 64 ints, pool: kGsRank keys (16-key aligned), all LDS.
__device__ inline uint64_t block_kth(const uint64_t* A, int n, int kk, int* hist, int* misc, int* wt,
                                     uint64_t* pool) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0, mask = 0;
  int m = n;
  // m is the same in every thread (read from LDS after a barrier); 6 rounds fix all 64 bits
  for (int round = 0; round < 6 && m > kGsRank; ++round) {
    const int shift = round < 5 ? 52 - 12 * round : 0;
    const uint64_t dmask = round < 5 ? 0xFFFull : 0xFull;
#pragma unroll
    for (int q = 0; q < kGsBins / kGsThreads; ++q) hist[q * kGsThreads + tid] = 0;
    __syncthreads();
#pragma unroll 4
    for (int i = tid; i < n; i += kGsThreads) {
      const uint64_t x = A[i];
      if ((x & mask) == prefix) atomicAdd(&hist[(int)((x >> shift) & dmask)], 1);
    }
    __syncthreads();
    crossing_digit(hist, kk, misc, wt);
    const int d = misc[0];
    kk -= misc[1];
    m = misc[2];
    prefix |= (uint64_t)d << shift;
    mask |= dmask << shift;
    __syncthreads();  // hist, wt and misc are rewritten by the next round
  }
  if (tid == 0) misc[3] = 0;
  if (tid < kGsRank) pool[tid] = 0ull;  // padding of the rank reads
  __syncthreads();
#pragma unroll 4
  for (int i = tid; i < n; i += kGsThreads) {
    const uint64_t x = A[i];
    if ((x & mask) == prefix) {
      const int p = atomicAdd(&misc[3], 1);
      if (p < kGsRank) pool[p] = x;  // m <= kGsRank for distinct keys
    }
  }
  __syncthreads();
  m = m < kGsRank ? m : kGsRank;
  if (tid < m) {
    const uint64_t x = pool[tid];
    if (rank_in(pool, m, x) == kk - 1) {  // exactly one key
      misc[4] = (int)(uint32_t)x;
      misc[5] = (int)(uint32_t)(x >> 32);
    }
  }
  __syncthreads();
  const uint64_t T = ((uint64_t)(uint32_t)misc[5] << 32) | (uint32_t)misc[4];
  __syncthreads();  // misc may be rewritten right after the return
  return T;
}

// Logits i = tid, tid + kGsThreads, ... < nre of the listed groups (logit i is offset i % gsp
// of group sel[i / gsp]), UR at a time with their list reads and loads issued together; keys
// >= T are appended to A (the first kGsRank values also to vbits) through the counter *np.
template <bool POW2>
__device__ __forceinline__ void reread_groups(const float* __restrict__ row, int V, const int* sel, int nre, int gsp,
                                              uint64_t T, uint64_t* A, uint32_t* vbits, int cap, int* np) {
  constexpr int UR = 4;
  const int sh = POW2 ? __builtin_ctz((unsigned)gsp) : 0;
  for (int i0 = threadIdx.x; i0 < nre; i0 += UR * kGsThreads) {
    int gi[UR], off[UR], base[UR];
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const int i = i0 + u * kGsThreads < nre ? i0 + u * kGsThreads : nre - 1;
      gi[u] = POW2 ? i >> sh : i / gsp;
      off[u] = POW2 ? i & (gsp - 1) : i - gi[u] * gsp;
    }
#pragma unroll
    for (int u = 0; u < UR; ++u) base[u] = sel[gi[u]];
    float f[UR];
    int64_t r[UR];
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      r[u] = i0 + u * kGsThreads < nre ? (int64_t)base[u] * gsp + off[u] : (int64_t)V;
      f[u] = row[r[u] < V ? r[u] : (int64_t)V - 1];  // always in the row; unused past V
    }
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      if (r[u] < V) {
        const uint64_t x = make_key(f[u], (uint32_t)r[u]);
        if (x >= T) {
          const int p = atomicAdd(np, 1);
          if (p < cap) A[p] = x;  // nre <= cap
          if (p < kGsRank) vbits[p] = __float_as_uint(f[u]);
        }
      }
    }
  }
}

// Row blockIdx.x: gkeys[row][0 .. G0) are the largest keys of consecutive groups of gs logits
// (the last group may be short); P consecutive ones are combined first (groups of gsp = P gs
// logits), so G = ceil(G0 / P) <= kGsMaxGroups and k P gs <= kGsMaxKeys.  Writes the row's top k
// (k <= 64, k <= V) to idx/val in order.  cap = gs_cap(G, gsp); dynamic LDS gs_lds_bytes(cap).
// (A template only so that every file including this header may instantiate it.)
template <int = 0>
__global__ __launch_bounds__(kGsThreads) void group_select_kernel(const float* __restrict__ logits, int64_t ldl,
                                                                  int V, int k, const uint64_t* __restrict__ gkeys,
                                                                  int G0, int gs, int P, int cap,
                                                                  int32_t* __restrict__ idx,
                                                                  float* __restrict__ val) {
  extern __shared__ __align__(16) unsigned char gsmem[];
  uint64_t* A = reinterpret_cast<uint64_t*>(gsmem);
  uint64_t* pool = A + ((cap + 15) & ~15);  // 128-byte aligned for the rank reads
  int* hist = reinterpret_cast<int*>(pool + kGsRank);
  int* misc = hist + kGsBins;
  int* wt = misc + 8;
  __shared__ int sel[kGsSel];
  __shared__ uint32_t vbits[kGsRank];  // values of the first kGsRank re-read candidates
  __shared__ int nsel, npool;
  const int m = blockIdx.x, tid = threadIdx.x, w = tid >> 6;
  const uint64_t* gk = gkeys + (int64_t)m * G0;
  const float* row = logits + (int64_t)m * ldl;
  const int G = (G0 + P - 1) / P, gsp = gs * P;
  const bool some = k <= G;  // else every group is read again
#pragma unroll
  for (int q = 0; q < kGsBins / kGsThreads; ++q) hist[q * kGsThreads + tid] = 0;
  if (tid == 0) {
    nsel = 0;
    npool = 0;
  }
  __syncthreads();
  // group keys: thread t combines the P consecutive keys of groups t + u kGsThreads (u <
  // kGsKeyRegs: G <= kGsMaxGroups), all of them and 4 keys of each in flight at a time, keeps
  // them in registers and counts them in the first-digit histogram
  constexpr int U = kGsKeyRegs;
  uint64_t mine[U];
#pragma unroll
  for (int u = 0; u < U; ++u) mine[u] = 0;
  if (P == 1) {  // one key per group: U loads, no combining
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = tid + u * kGsThreads;
      if (g < G) mine[u] = gk[g];
    }
  } else {
    for (int p0 = 0; p0 < P; p0 += 4) {
      uint64_t y[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int g = tid + u * kGsThreads;
          const int64_t e = (int64_t)g * P + p0 + q;
          y[u][q] = g < G && p0 + q < P && e < G0 ? gk[e] : 0ull;
        }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) mine[u] = y[u][q] > mine[u] ? y[u][q] : mine[u];
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int g = tid + u * kGsThreads;
    if (g < G) {
      A[g] = mine[u];
      if (some) atomicAdd(&hist[first_slot(mine[u])], 1);
    }
  }
  __syncthreads();
  uint64_t T = 0;  // below every real key
  if (some) {
    if (w == 0) first_crossing(hist, k, misc);
    __syncthreads();
    const int d = misc[0], admitted = misc[1] + misc[2];  // group keys with a top digit >= d
    const int capg = cap / gsp < kGsSel ? cap / gsp : kGsSel;
    if (admitted <= capg)
      T = (uint64_t)d << 52;  // <= the k-th largest group key
    else
      T = block_kth(A, G, k, hist, misc, wt, pool);  // exact (its own histogram rounds)
  }
  // the groups whose keys reach T (at most cap / gsp: the admitted ones, k, or G < k)
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int g = tid + u * kGsThreads;
    if (g < G && mine[u] >= T) {
      const int p = atomicAdd(&nsel, 1);
      if (p < kGsSel) sel[p] = g;
    }
  }
  __syncthreads();
  // their logits, read again by the whole workgroup (a shift instead of a division when the
  // group size is a power of two); keys >= T are appended to A
  const int nre = (nsel < kGsSel ? nsel : kGsSel) * gsp;  // <= cap
  if ((gsp & (gsp - 1)) == 0)
    reread_groups<true>(row, V, sel, nre, gsp, T, A, vbits, cap, &npool);
  else
    reread_groups<false>(row, V, sel, nre, gsp, T, A, vbits, cap, &npool);
  __syncthreads();
  const int n2 = npool < cap ? npool : cap;  // >= k: the admitted groups' maxima, or every logit when G < k
  if (n2 <= kGsRank) {
    // few candidates: each one's rank among them (the count of larger ones) is its output
    // position; four threads per candidate, each over every fourth run of 16 keys
    const int c = tid >> 2, part = tid & 3;
    uint64_t x = 0;
    int r = 0;
    if (c < n2) {
      x = A[c];
      for (int j = part * 16; j < n2; j += 64) {
        uint64_t v[16];
        load16(A + j, v);  // within A's (cap + 15) & ~15 keys; those at n2 and past are skipped
#pragma unroll
        for (int q = 0; q < 16; ++q) r += j + q < n2 && v[q] > x ? 1 : 0;
      }
    }
    r += (int)quad_swap<0xB1>((uint32_t)r);  // the four threads of a candidate are one quad
    r += (int)quad_swap<0x4E>((uint32_t)r);
    if (c < n2 && part == 0 && r < k) {
      uint32_t j = key_index(x);
      if (j >= (uint32_t)V) j = (uint32_t)V - 1;  // unreachable: the keys are real logits
      idx[(int64_t)m * k + r] = (int32_t)j;
      val[(int64_t)m * k + r] = __uint_as_float(vbits[c]);
    }
    return;
  }
  const uint64_t T2 = block_kth(A, n2, k, hist, misc, wt, pool);
  if (tid == 0) misc[6] = 0;
  if (tid < 64) pool[tid] = 0ull;  // padding of the rank reads
  __syncthreads();
  for (int i = tid; i < n2; i += kGsThreads) {
    const uint64_t x = A[i];
    if (x >= T2) {
      const int p = atomicAdd(&misc[6], 1);  // exactly k keys
      if (p < kGsRank) pool[p] = x;
    }
  }
  __syncthreads();
  if (tid < k) {
    const uint64_t x = pool[tid];
    const int r = rank_in(pool, k, x);
    uint32_t j = key_index(x);
    if (j >= (uint32_t)V) j = (uint32_t)V - 1;  // unreachable: the keys are real logits
    idx[(int64_t)m * k + r] = (int32_t)j;
    val[(int64_t)m * k + r] = row[j];
  }
}

// Pre-reduction for G0 group keys of gs logits each: the power of two P that minimises the
// keys the selection sweeps, ceil(G0 / P) group keys plus k P gs re-read logits, among those
// with at most kGsMaxGroups group keys and kGsMaxKeys re-read logits; 0 when there is none.  (The int4 head's 9496
// keys of 16 rows at k = 40 take P = 4: 2374 + 2560 keys instead of 9496 + 640.)
__host__ __device__ inline int gs_prereduce(int64_t G0, int gs, int k) {
  int best = 0;
  int64_t cost = 0;
  for (int64_t P = 1; P <= kGsMaxKeys; P *= 2) {
    const int64_t G = (G0 + P - 1) / P, re = (int64_t)k * P * gs;
    if (re > kGsMaxKeys) break;
    if (G <= kGsMaxGroups && (best == 0 || G + re < cost)) {
      best = (int)P;
      cost = G + re;
    }
  }
  return best;
}

}  // namespace w4
