// w4_gemv: decode GEMV over group-wise affine int4 weights (M = 1..16 activation rows).
//
// What it computes ("The inference engine -- Mojo 1.0 on Metal", "Crossing Mojo 1.0" and
// "What's inside the engine today": the multi-row decode GEMV whose weight stream is the
// limit):  y[m][n] = sum_k (s[n][g] q[n][k] + b[n][g]) x[m][k],  g = k / 64.
//
// Design for CDNA4 (wave64, HBM-bound), kernels by the number M of activation rows:
//  * M = 1 with rows longer than 1024 (gemv1s_kernel, "row slices" below): a wave streams
//    whole 1 KB slices of R rows with buffer loads at scalar row offsets, converts codes to
//    f16 through the fp8 converter and splits long rows across the waves of a workgroup.
//  * M = 2..4 (the same kernel with every row of x in registers): each word dequantized once
//    and dotted with each row.
//  * M = 1 with short rows (gemv1_kernel), and what the above do not cover (gemv_kernel:
//    rows beyond 16384): a "team" of P lanes
//    (P = 64, or 32 for short rows) owns R output rows; lane l streams 16-byte chunks (32
//    codes = half a group) c = l, l+P, ... of each row, so every load instruction reads P*16
//    contiguous bytes of one row.  x is staged in LDS (or registers), re-ordered into the f16
//    pairs (x0,x4) (x1,x5) (x2,x6) (x3,x7) that match the order codes come out of a word:
//    OR-ing a nibble into the mantissa of 1024.0 (0x6400) gives exactly 1024 + q, a nibble at
//    bits 4..7 OR-ed into 64.0 (0x5400) gives exactly 64 + q, so one word w yields
//      (w & 0x000F000F) | 0x64006400 = (1024+q0, 1024+q4)
//      (w & 0x00F000F0) | 0x54005400 = (  64+q1,   64+q5)
//    and the same on w >> 8 for (q2,q6), (q3,q7); a packed f16 subtract removes the offset
//    exactly.
//  * 5 <= M <= 16, and 3..4 with rows beyond 16384 (gemv_mf_kernel): dequantized words feed
//    the matrix cores.
// In every kernel a packed f16 FMA forms w = s q + b with one rounding (the value the
// prefill scratch holds) and the products w*x are exact in f32 and summed in f32, blockwise.
// Every term's error is thus relative to |w x|, which keeps each output within
// 2e-3 * sum_k |w x| (and exactly 0 when every w x is 0).  Rows reduce across lanes with DPP
// moves; one lane stores y.
#include "w4_dequant.h"
#include "w4_internal.h"

namespace w4 {

namespace {

constexpr int kWG = 256;
constexpr int kLdsBudget = 64 * 1024;

// The 8 weights of word w as f16 pairs matching the x pair order (see file comment).
template <bool SYM>
__device__ __forceinline__ uint4 word_weights(uint32_t w, h2 s2, h2 b2) {
  const uint32_t w8 = w >> 8;
  const h2 o1024 = {(f16)Fmt<SYM>::kLo, (f16)Fmt<SYM>::kLo}, o64 = {(f16)Fmt<SYM>::kHi, (f16)Fmt<SYM>::kHi};
  const h2 q0 = as_h2((w & 0x000F000Fu) | 0x64006400u) - o1024;   // exact
  const h2 q1 = as_h2((w & 0x00F000F0u) | 0x54005400u) - o64;
  const h2 q2 = as_h2((w8 & 0x000F000Fu) | 0x64006400u) - o1024;
  const h2 q3 = as_h2((w8 & 0x00F000F0u) | 0x54005400u) - o64;
  uint4 r;
  r.x = as_u32(__builtin_elementwise_fma(q0, s2, b2));             // one rounding
  r.y = as_u32(__builtin_elementwise_fma(q1, s2, b2));
  r.z = as_u32(__builtin_elementwise_fma(q2, s2, b2));
  r.w = as_u32(__builtin_elementwise_fma(q3, s2, b2));
  return r;
}

__device__ __forceinline__ float pair_dot(uint4 w, uint4 x, float acc) {
  acc = dot2(w.x, x.x, acc);
  acc = dot2(w.y, x.y, acc);
  acc = dot2(w.z, x.z, acc);
  acc = dot2(w.w, x.w, acc);
  return acc;
}

// (x0x1, x2x3, x4x5, x6x7) -> (x0x4, x1x5, x2x6, x3x7)
__device__ __forceinline__ uint4 pair_up(uint4 d) {
  uint4 p;
  p.x = (d.x & 0xFFFFu) | (d.z << 16);
  p.y = (d.x >> 16) | (d.z & 0xFFFF0000u);
  p.z = (d.y & 0xFFFFu) | (d.w << 16);
  p.w = (d.y >> 16) | (d.w & 0xFFFF0000u);
  return p;
}

template <int MT, int R, int P, bool SYM>
__global__ __launch_bounds__(kWG) void gemv_kernel(const uint32_t* __restrict__ qw,
                                                   const uint16_t* __restrict__ sc,
                                                   const uint16_t* __restrict__ bi,
                                                   const uint16_t* __restrict__ x, int64_t ldx,
                                                   float* __restrict__ y, int64_t ldy, int M,
                                                   int N, int K, int KT) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int TEAMS = kWG / P;
  const int CT = KT / 32;  // chunks per K-tile
  uint4* xs = reinterpret_cast<uint4*>(smem);  // [MT][CT][4]

  const int tid = threadIdx.x;
  const int lane = tid % P;
  const int team = tid / P;
  const int row0 = (blockIdx.x * TEAMS + team) * R;
  const int64_t KW = K / 8;  // words per row
  const int G = K / Fmt<SYM>::kGroupSize;  // groups per row

  const uint4* rowp[R];
  const uint16_t* sp[R];
  const uint16_t* bp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(row0 + r, N - 1);  // clamp: tail rows reload the last row, never stored
    rowp[r] = reinterpret_cast<const uint4*>(qw + (int64_t)n * KW);
    sp[r] = sc + (int64_t)n * G;
    bp[r] = SYM ? sc : bi + (int64_t)n * G;
  }

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;

  for (int k0 = 0; k0 < K; k0 += KT) {
    const int ct = min(CT, (K - k0) / 32);
    if (k0 > 0) __syncthreads();
    // ---- stage x[:, k0 : k0+KT) as re-ordered pairs, one 8-element block per item
    for (int i = tid; i < MT * CT * 4; i += kWG) {
      const int m = i / (CT * 4), cb = i - m * (CT * 4);
      uint4 p = make_uint4(0, 0, 0, 0);
      if (m < M && cb < ct * 4)
        p = pair_up(*reinterpret_cast<const uint4*>(x + (int64_t)m * ldx + k0 + cb * 8));
      xs[m * CT * 4 + cb] = p;
    }
    __syncthreads();

    // ---- stream this tile's chunks of the team's R rows
    const int c0 = k0 / 32;
#pragma unroll 2
    for (int cl = lane; cl < ct; cl += P) {
      const int c = c0 + cl;
      uint4 w[R];
      uint16_t sbits[R], bbits[R];
#pragma unroll
      for (int r = 0; r < R; ++r) w[r] = load_nt(rowp[r] + c);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        sbits[r] = sp[r][c >> Fmt<SYM>::kChunkShift];
        bbits[r] = SYM ? 0 : bp[r][c >> Fmt<SYM>::kChunkShift];
      }
      uint4 wv[R][4];  // dequantized f16 pairs of the chunk, per row and word
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const f16 sv = __builtin_bit_cast(f16, sbits[r]), bv = __builtin_bit_cast(f16, bbits[r]);
        const h2 s2 = {sv, sv}, b2 = {bv, bv};
        wv[r][0] = word_weights<SYM>(w[r].x, s2, b2);
        wv[r][1] = word_weights<SYM>(w[r].y, s2, b2);
        wv[r][2] = word_weights<SYM>(w[r].z, s2, b2);
        wv[r][3] = word_weights<SYM>(w[r].w, s2, b2);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint4* xm = xs + (m * CT + cl) * 4;
        const uint4 x0 = xm[0], x1 = xm[1], x2 = xm[2], x3 = xm[3];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float a = acc[r][m];
          a = pair_dot(wv[r][0], x0, a);
          a = pair_dot(wv[r][1], x1, a);
          a = pair_dot(wv[r][2], x2, a);
          a = pair_dot(wv[r][3], x3, a);
          acc[r][m] = a;
        }
      }
    }
  }

  // ---- team reduction and store
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      acc[r][m] = group_sum<P>(acc[r][m]);
    }
  }
  if (lane == P - 1) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = row0 + r;
      if (n < N) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m < M) y[(int64_t)m * ldy + n] = acc[r][m];
      }
    }
  }
}

// ------------------------------------------------------------------ M = 1 kernel
// Decode at M = 1 needs no LDS: lane l of a team of L lanes always handles the chunks
// c = l + j*L (j < NIT) of whatever row it streams, so its slice of x is loaded once into
// registers (re-ordered into pairs).  Each team walks row blocks of R rows with a grid
// stride, two blocks at a time in ping-pong registers: the next block's loads are in flight
// while the current one is dequantized and reduced.  The first loads are issued before x is
// read.  EXACT means L * NIT == K / 32 (no chunk past the end of a row).

// (w & mask) | magic in one VALU op; GFX9 VOP3 takes no literal, so both constants come in
// as VGPRs.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "v"(mask), "v"(magic));
  return r;
}

struct Consts {
  uint32_t m_lo, m_hi, mag_lo, mag_hi;  // 0x000F000F, 0x00F000F0, 0x64006400, 0x54005400
};

// One word's 8 weights (f16 pairs ordered like the x pairs), accumulated into acc.
template <bool SYM>
__device__ __forceinline__ float word_fma(uint32_t w, h2 s2, h2 b2, const uint4& xp, float acc,
                                          const Consts& k) {
  const uint32_t w8 = w >> 8;
  const h2 o1024 = {(f16)Fmt<SYM>::kLo, (f16)Fmt<SYM>::kLo}, o64 = {(f16)Fmt<SYM>::kHi, (f16)Fmt<SYM>::kHi};
  const h2 q0 = as_h2(and_or(w, k.m_lo, k.mag_lo)) - o1024;   // exact
  const h2 q1 = as_h2(and_or(w, k.m_hi, k.mag_hi)) - o64;
  const h2 q2 = as_h2(and_or(w8, k.m_lo, k.mag_lo)) - o1024;
  const h2 q3 = as_h2(and_or(w8, k.m_hi, k.mag_hi)) - o64;
  acc = dot2(as_u32(__builtin_elementwise_fma(q0, s2, b2)), xp.x, acc);  // one rounding each
  acc = dot2(as_u32(__builtin_elementwise_fma(q1, s2, b2)), xp.y, acc);
  acc = dot2(as_u32(__builtin_elementwise_fma(q2, s2, b2)), xp.z, acc);
  acc = dot2(as_u32(__builtin_elementwise_fma(q3, s2, b2)), xp.w, acc);
  return acc;
}

template <int R, int NIT>
struct Block {
  uint4 w[R][NIT];
  uint32_t s[R][NIT], b[R][NIT];  // f16 bits in the low half (32-bit keeps them in VGPRs)
};

// XL: x is staged once per workgroup in LDS (pairs, K * 2 bytes) and read per chunk instead
// of being held in 16 * NIT registers per lane; fewer registers allow more waves.
template <int L, int NIT, int R, bool EXACT, bool XL, bool SYM>
__global__ __launch_bounds__(kWG) void gemv1_kernel(const uint32_t* __restrict__ qw,
                                                    const uint16_t* __restrict__ sc,
                                                    const uint16_t* __restrict__ bi,
                                                    const uint16_t* __restrict__ x,
                                                    float* __restrict__ y, int N, int K,
                                                    int nblocks) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int TEAMS = kWG / L;
  const int lane = threadIdx.x % L;
  const int team = blockIdx.x * TEAMS + threadIdx.x / L;
  const int T = gridDim.x * TEAMS;
  constexpr int GS = Fmt<SYM>::kChunkShift;
  const int C = K / 32;                    // 16-byte chunks per row
  const int G = K / Fmt<SYM>::kGroupSize;  // groups per row
  const uint4* q4 = reinterpret_cast<const uint4*>(qw) + lane;
  const uint16_t* sl = sc + (lane >> GS);  // L is a multiple of 4: (lane + jL) >> GS splits
  const uint16_t* bl = (SYM ? sc : bi) + (lane >> GS);

  // Every load is unconditional (block and chunk indices are clamped to valid addresses; a
  // chunk past the end of the row is neutralised in the math by a zero scale and bias, never
  // by overwriting the loaded register, which would force a wait for the load).  With no
  // branch around a load and nothing touching a loaded register before its use, the
  // compiler's wait counts stay exact: the math of a chunk waits only for that chunk.
  auto valid = [&](int j) { return EXACT || lane + j * L < C; };
  auto load = [&](int blk, Block<R, NIT>& B) {
    blk = min(blk, nblocks - 1);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = min(blk * R + r, N - 1);  // tail rows reload the last row, never stored
      const uint4* p = q4 + (int64_t)n * C;
      const uint16_t* ps = sl + (int64_t)n * G;
      const uint16_t* pb = bl + (int64_t)n * G;
#pragma unroll
      for (int j = 0; j < NIT; ++j) {
        const int jc = valid(j) ? j * L : (C - 1 - lane);  // in-row chunk for this lane
        B.w[r][j] = load_nt(p + jc);
        B.s[r][j] = ps[jc >> GS];
        B.b[r][j] = SYM ? 0u : pb[jc >> GS];
      }
    }
  };

  // x is loaded first: it is L2-resident and shared by every row, and loads complete in
  // order, so issuing it ahead of the weight stream lets the math wait for x without
  // waiting for the weights.  XL stages it in LDS (NIT 16-byte pieces per thread cover
  // C * 4 >= the row) behind an LDS-only barrier; otherwise each lane keeps its chunks.
  constexpr int XR = XL ? NIT : 1;
  uint4 xr[XR];
  uint4 xv[XL ? 1 : NIT][4];
  if constexpr (XL) {
#pragma unroll
    for (int t = 0; t < XR; ++t) {
      const int i = min((int)threadIdx.x + t * kWG, C * 4 - 1);
      xr[t] = *reinterpret_cast<const uint4*>(x + i * 8);
    }
  } else {
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
      const int c = min(lane + j * L, C - 1);
      const uint4* xp = reinterpret_cast<const uint4*>(x + c * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[j][i] = xp[i];
    }
  }

  Block<R, NIT> A, B;
  int blk = team;
  load(blk, A);
  __builtin_amdgcn_sched_barrier(0);
  uint4* xs = reinterpret_cast<uint4*>(smem);
  if constexpr (XL) {
#pragma unroll
    for (int t = 0; t < XR; ++t) {
      const int i = (int)threadIdx.x + t * kWG;
      if (i < C * 4) xs[i] = pair_up(xr[t]);
    }
    // LDS visibility only: a __syncthreads would also wait for every weight load in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  if (team >= nblocks) return;

  Consts k;
  k.m_lo = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  k.m_hi = __builtin_amdgcn_readfirstlane(0x00F000F0u);
  k.mag_lo = __builtin_amdgcn_readfirstlane(0x64006400u);
  k.mag_hi = __builtin_amdgcn_readfirstlane(0x54005400u);

  auto compute = [&](int blk, const Block<R, NIT>& B) {
    float acc[R];
    float a0[R], a1[R], a2[R], a3[R];  // four independent chains per row (ILP)
#pragma unroll
    for (int r = 0; r < R; ++r) a0[r] = a1[r] = a2[r] = a3[r] = 0.f;
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
      uint4 x0, x1, x2, x3;
      if constexpr (XL) {
        const int c = min(lane + j * L, C - 1);  // chunks past the row end get zero weights
        x0 = xs[c * 4 + 0];
        x1 = xs[c * 4 + 1];
        x2 = xs[c * 4 + 2];
        x3 = xs[c * 4 + 3];
      } else {
        x0 = pair_up(xv[j][0]);
        x1 = pair_up(xv[j][1]);
        x2 = pair_up(xv[j][2]);
        x3 = pair_up(xv[j][3]);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // past the row end: s = b = 0, so every weight is fma(q, 0, 0) = 0 exactly
        const uint32_t sb_on = valid(j) ? 0xFFFFu : 0u;
        const f16 sv = __builtin_bit_cast(f16, (uint16_t)(B.s[r][j] & sb_on));
        const f16 bv = __builtin_bit_cast(f16, (uint16_t)(B.b[r][j] & sb_on));
        const h2 s2 = {sv, sv}, b2 = {bv, bv};
        a0[r] = word_fma<SYM>(B.w[r][j].x, s2, b2, x0, a0[r], k);
        a1[r] = word_fma<SYM>(B.w[r][j].y, s2, b2, x1, a1[r], k);
        a2[r] = word_fma<SYM>(B.w[r][j].z, s2, b2, x2, a2[r], k);
        a3[r] = word_fma<SYM>(B.w[r][j].w, s2, b2, x3, a3[r], k);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc[r] = group_sum<L>((a0[r] + a1[r]) + (a2[r] + a3[r]));
    }
    if (lane == L - 1) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (blk * R + r < N) y[blk * R + r] = acc[r];
    }
  };

  // Every team walks `per` blocks (team, team + T, ...; the same count for all teams, the
  // surplus past nblocks is computed on clamped loads and never stored).  The steady-state
  // loop and the peeled tail contain only unconditional loads, so wait counts are exact on
  // every path; sched_barrier keeps the scheduler from sinking a prefetch below the math of
  // the block before it.
  const int per = (nblocks + T - 1) / T;
  int i = 0;
  for (; i + 2 < per; i += 2) {
    load(blk + (i + 1) * T, B);
    __builtin_amdgcn_sched_barrier(0);
    compute(blk + i * T, A);
    load(blk + (i + 2) * T, A);
    __builtin_amdgcn_sched_barrier(0);
    compute(blk + (i + 1) * T, B);
  }
  if (per - i == 2) {
    load(blk + (i + 1) * T, B);
    __builtin_amdgcn_sched_barrier(0);
    compute(blk + i * T, A);
    compute(blk + (i + 1) * T, B);
  } else {
    compute(blk + i * T, A);
  }
}

// per: blocks each team walks; the grid is sized so that teams * per just covers the blocks
// (no team is left with a surplus block to load and discard).
template <int L, int NIT, int R, bool XL, bool SYM>
void launch_m1(const uint32_t* qw, const uint16_t* s, const uint16_t* b, const uint16_t* x,
               float* y, int N, int K, int per, hipStream_t st) {
  constexpr int teams = kWG / L;
  const int nblocks = (N + R - 1) / R;
  if (per < 1) per = 1;
  const int T = (nblocks + per - 1) / per;
  const int grid = (T + teams - 1) / teams;
  const size_t lds = XL ? (size_t)K * 2 : 0;
  if (L * NIT == K / 32)
    hipLaunchKernelGGL((gemv1_kernel<L, NIT, R, true, XL, SYM>), dim3(grid), dim3(kWG), lds, st, qw, s,
                       b, x, y, N, K, nblocks);
  else
    hipLaunchKernelGGL((gemv1_kernel<L, NIT, R, false, XL, SYM>), dim3(grid), dim3(kWG), lds, st, qw,
                       s, b, x, y, N, K, nblocks);
}

template <int MT, int R, int P, bool SYM>
void launch_t(const uint32_t* qw, const uint16_t* s, const uint16_t* b, const uint16_t* x,
              int64_t ldx, float* y, int64_t ldy, int M, int N, int K, hipStream_t st) {
  // K-tile: as much of x as fits the LDS budget (64 bytes per 32-element chunk and row).
  const int per_chunk = MT * 64;
  int ct = kLdsBudget / per_chunk;
  const int C = K / 32;
  if (ct > C) ct = C;
  const int KT = ct * 32;
  const size_t lds = (size_t)MT * ct * 64;
  constexpr int rows_per_wg = (kWG / P) * R;
  const unsigned grid = (unsigned)((N + rows_per_wg - 1) / rows_per_wg);
  hipLaunchKernelGGL((gemv_kernel<MT, R, P, SYM>), dim3(grid), dim3(kWG), lds, st, qw, s, b, x, ldx,
                     y, ldy, M, N, K, KT);
}

template <int MT, int P, bool SYM>
void launch_r(const uint32_t* qw, const uint16_t* s, const uint16_t* b, const uint16_t* x,
              int64_t ldx, float* y, int64_t ldy, int M, int N, int K, hipStream_t st) {
  // Rows per team: enough workgroups to fill 256 CUs twice before giving a lane more rows.
  constexpr int teams = kWG / P;
  const int64_t want = 512;
  if (MT <= 4 && (int64_t)N / (teams * 4) >= want)
    launch_t<MT, 4, P, SYM>(qw, s, b, x, ldx, y, ldy, M, N, K, st);
  else if ((int64_t)N / (teams * 2) >= want)
    launch_t<MT, 2, P, SYM>(qw, s, b, x, ldx, y, ldy, M, N, K, st);
  else
    launch_t<MT, 1, P, SYM>(qw, s, b, x, ldx, y, ldy, M, N, K, st);
}

template <int MT, bool SYM>
void launch_p(const uint32_t* qw, const uint16_t* s, const uint16_t* b, const uint16_t* x,
              int64_t ldx, float* y, int64_t ldy, int M, int N, int K, hipStream_t st) {
  if (K / 32 <= 32)
    launch_r<MT, 32, SYM>(qw, s, b, x, ldx, y, ldy, M, N, K, st);
  else
    launch_r<MT, 64, SYM>(qw, s, b, x, ldx, y, ldy, M, N, K, st);
}

// ------------------------------------------------------------------ up to 16 rows on MFMA
// With several activation rows the VALU kernels spend 4 dot products per word and row on
// top of the dequant, so at M = 16 the arithmetic, not HBM, would set their speed.
// Here the dequantized weights feed v_mfma_f32_16x16x32_f16 instead: D[n][m] += W[n][k] x[m][k]
// over 16 weight rows n (A operand) and up to 16 activation rows m (B operand), so the only
// per-row VALU work left is the dequant (11 operations per word with the fp8 converter's
// codes), shared by every m.
//
// Lane l = (i = l % 16, g = l / 16) of a wave holds A row i and B column i, k-group g.  At step
// t it loads the 16-byte chunk c = 4t + g of weight row 16*rb + i (so a load instruction reads
// 64 contiguous bytes of each of 16 rows) and the same 32 elements of x row min(i, M - 1).  Word
// j of the chunk dequantizes into one A operand whose 8 f16 sit in the order the converter
// yields the codes, (q0,q2) (q4,q6) (q1,q3) (q5,q7); the B operand holds the x pairs in that
// same order, so every product pairs a weight with its own x whatever order the matrix core
// sums the 32 products in.  D column i, rows 4g..4g+3 come back in the lane's 4 accumulators;
// columns i >= M are computed on a duplicate x row and never stored.
//
// A wave streams RB row blocks (16 RB rows) over one K-range: the NW waves of a workgroup split
// the steps of the same row blocks and their partial sums are added in LDS in wave order
// (deterministic).  Loads are unconditional and clamped (steps past the wave's range or chunks
// past the row end read a valid address, their scale and bias are zeroed so their weights are
// exactly 0) and run in two ping-pong blocks of V steps, as in the M = 1 kernel.

// The 8 weights of word w (f16, the converter's code order) as an MFMA operand.
template <bool SYM>
__device__ __forceinline__ f16x8 word_operand(uint32_t w, h2 s2, h2 b2) {
  h2 q0, q1, q2, q3;
  cvt_codes<SYM>(w, q0, q1, q2, q3);
  const h2 r0 = __builtin_elementwise_fma(q0, s2, b2);  // one rounding each
  const h2 r1 = __builtin_elementwise_fma(q1, s2, b2);
  const h2 r2 = __builtin_elementwise_fma(q2, s2, b2);
  const h2 r3 = __builtin_elementwise_fma(q3, s2, b2);
  return __builtin_bit_cast(f16x8, make_uint4(as_u32(r0), as_u32(r1), as_u32(r2), as_u32(r3)));
}

__device__ __forceinline__ f16x8 as_operand(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(f16x8, make_uint4(a, b, c, d));
}

template <int RB, int V>
struct MfBlock {
  uint4 w[V][RB];
  uint32_t s[V][RB], b[V][RB];  // f16 bits in the low half
  uint4 x[V][4];                // raw x, 32 elements of this lane's chunk
};

template <int NW, int RB, int V, bool SYM>
__global__ __launch_bounds__(NW * 64) void gemv_mf_kernel(const uint32_t* __restrict__ qw,
                                                          const uint16_t* __restrict__ sc,
                                                          const uint16_t* __restrict__ bi,
                                                          const uint16_t* __restrict__ x,
                                                          int64_t ldx, float* __restrict__ y,
                                                          int64_t ldy, int M, int N, int K,
                                                          int U, float* __restrict__ part) {
  __shared__ f32x4 red[NW][RB][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  constexpr int GS = Fmt<SYM>::kChunkShift;
  const int C = K / 32, G = K / Fmt<SYM>::kGroupSize, T = (C + 3) / 4;
  const int rb0 = blockIdx.x * RB;
  const int t0 = (blockIdx.y * NW + wv) * U, tend = min(T, t0 + U);  // K-range blockIdx.y
  const int nb = (U + V - 1) / V;  // blocks per wave, the same for every wave

  const uint4* wrow[RB];
  const uint16_t* srow[RB];
  const uint16_t* brow[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int n = min(16 * (rb0 + r) + i, N - 1);  // tail rows reload the last row, never stored
    wrow[r] = reinterpret_cast<const uint4*>(qw) + (int64_t)n * C;
    srow[r] = sc + (int64_t)n * G;
    brow[r] = (SYM ? sc : bi) + (int64_t)n * G;
  }
  const uint4* xrow = reinterpret_cast<const uint4*>(x + (int64_t)min(i, M - 1) * ldx);

  auto chunk = [&](int t) { return min(4 * min(t, T - 1) + g, C - 1); };
  auto valid = [&](int t) { return t < tend && 4 * t + g < C; };
  auto load = [&](int blk, MfBlock<RB, V>& B) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int c = chunk(t0 + blk * V + v);
#pragma unroll
      for (int j = 0; j < 4; ++j) B.x[v][j] = xrow[c * 4 + j];
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        B.w[v][r] = load_nt(wrow[r] + c);
        B.s[v][r] = srow[r][c >> GS];
        B.b[v][r] = SYM ? 0u : brow[r][c >> GS];
      }
    }
  };

  f32x4 acc[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int blk, const MfBlock<RB, V>& B) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const uint32_t sb_on = valid(t0 + blk * V + v) ? 0xFFFFu : 0u;
      uint4 xp[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) xp[j] = pair_up_cvt(B.x[v][j]);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const f16 sv = __builtin_bit_cast(f16, (uint16_t)(B.s[v][r] & sb_on));
        const f16 bv = __builtin_bit_cast(f16, (uint16_t)(B.b[v][r] & sb_on));
        const h2 s2 = {sv, sv}, b2 = {bv, bv};
        const uint32_t wd[4] = {B.w[v][r].x, B.w[v][r].y, B.w[v][r].z, B.w[v][r].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              word_operand<SYM>(wd[j], s2, b2), as_operand(xp[j].x, xp[j].y, xp[j].z, xp[j].w),
              acc[r], 0, 0, 0);
      }
    }
  };

  MfBlock<RB, V> A, B;
  load(0, A);
  __builtin_amdgcn_sched_barrier(0);
  int bk = 0;
  for (; bk + 2 < nb; bk += 2) {
    load(bk + 1, B);
    __builtin_amdgcn_sched_barrier(0);
    compute(bk, A);
    load(bk + 2, A);
    __builtin_amdgcn_sched_barrier(0);
    compute(bk + 1, B);
  }
  if (nb - bk == 2) {
    load(bk + 1, B);
    __builtin_amdgcn_sched_barrier(0);
    compute(bk, A);
    compute(bk + 1, B);
  } else {
    compute(bk, A);
  }

  // ---- add the NW partial sums in wave order and store: output (r, m, g, e) is row
  // n = 16 (rb0 + r) + 4 g + e, column m, held by lane 16 g + m of every wave
#pragma unroll
  for (int r = 0; r < RB; ++r) red[wv][r][lane] = acc[r];
  __syncthreads();
  for (int o = threadIdx.x; o < RB * 256; o += NW * 64) {
    const int e = o & 3, gg = (o >> 2) & 3, m = (o >> 4) & 15, r = o >> 8;
    const int n = 16 * (rb0 + r) + 4 * gg + e;
    if (m < M && n < N) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += red[w][r][16 * gg + m][e];
      if (part)  // one K-range of several: its partial sum, added by mf_reduce_kernel
        part[((int64_t)blockIdx.y * M + m) * N + n] = sum;
      else
        y[(int64_t)m * ldy + n] = sum;
    }
  }
}

// y[m][n] = the S partial sums part[s][m][n] added in split order (deterministic)
__global__ __launch_bounds__(256) void mf_reduce_kernel(const float* __restrict__ part, float* __restrict__ y,
                                                        int64_t ldy, int M, int N, int S) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x, MN = (int64_t)M * N;
  if (e >= MN) return;
  const int m = (int)(e / N), n = (int)(e - (int64_t)m * N);
  float v = part[e];
  for (int s = 1; s < S; ++s) v += part[s * MN + e];
  y[(int64_t)m * ldy + n] = v;
}

// Large matrices (24 MB of codes and more) at 5 <= M <= 8: the same matrix-core GEMV with each workgroup's
// x rows over its K-range (already in the converter's pair order) and its rows' (scale | bias
// << 16) words staged in LDS once, so that the loop issues only the weight loads (RB per step
// instead of RB + 4 + 2 RB load instructions).  Measured at M = 8, graph-replayed over distinct
// weights: the 30720 x 3840 gate|up 29.9 -> 24.8 us, the 3840 x 15360 down 22.2 -> 16.5 us (with
// four K-ranges); on 4096 x 3840 and on the Qwen3 M = 16 shapes (5-13 MB) the staging does not
// pay (6.9 -> 8.6 us on the former).  Tiles, steps, masking and the wave-order reduction are
// those of gemv_mf_kernel; the staged x row of lane i is min(i, M - 1).
template <int NW, int RB, int V, bool SYM>
__global__ __launch_bounds__(NW * 64) void gemv_mfs_kernel(const uint32_t* __restrict__ qw,
                                                           const uint16_t* __restrict__ sc,
                                                           const uint16_t* __restrict__ bi,
                                                           const uint16_t* __restrict__ x, int64_t ldx,
                                                           float* __restrict__ y, int64_t ldy, int M, int N,
                                                           int K, int U, float* __restrict__ part, int xpitch,
                                                           int gr) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  constexpr int GS = Fmt<SYM>::kChunkShift;
  const int C = K / 32, G = K / Fmt<SYM>::kGroupSize, T = (C + 3) / 4;
  const int rb0 = blockIdx.x * RB;
  const int s0 = blockIdx.y * NW * U, send = min(T, s0 + NW * U);  // this K-range's steps
  const int c0 = 4 * s0, cend = min(C, 4 * send);                   // and chunks
  const int g0 = c0 >> GS, ng = ((cend - 1) >> GS) - g0 + 1;        // and groups
  unsigned char* lx = smem;                                          // [M][xpitch] bytes
  uint32_t* lsb = reinterpret_cast<uint32_t*>(smem + M * xpitch);   // [16 RB][gr]
  const int n8 = (cend - c0) * 4;  // 16-byte pieces of one x row in the range
  for (int e = threadIdx.x; e < M * n8; e += NW * 64) {
    const int m = e / n8, c8 = e - m * n8;
    const uint4 v = *reinterpret_cast<const uint4*>(x + (int64_t)m * ldx + c0 * 32 + c8 * 8);
    *reinterpret_cast<uint4*>(lx + m * xpitch + c8 * 16) = pair_up_cvt(v);
  }
  for (int e = threadIdx.x; e < 16 * RB * ng; e += NW * 64) {
    const int r = e / ng, gg = e - r * ng;
    const int64_t o = (int64_t)min(16 * rb0 + r, N - 1) * G + g0 + gg;
    lsb[r * gr + gg] = (uint32_t)sc[o] | (SYM ? 0u : (uint32_t)bi[o] << 16);
  }
  const int t0 = s0 + wv * U, tend = min(send, t0 + U);
  const int nb = (U + V - 1) / V;
  const uint4* wrow[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
    wrow[r] = reinterpret_cast<const uint4*>(qw) + (int64_t)min(16 * (rb0 + r) + i, N - 1) * C;
  const int xrow = min(i, M - 1) * xpitch;
  auto chunk = [&](int t) { return min(4 * min(t, send - 1) + g, cend - 1); };
  auto valid = [&](int t) { return t < tend && 4 * t + g < cend; };
  struct Blk {
    uint4 w[V][RB];
  };
  auto load = [&](int blk, Blk& B) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int c = chunk(t0 + blk * V + v);
#pragma unroll
      for (int r = 0; r < RB; ++r) B.w[v][r] = load_nt(wrow[r] + c);
    }
  };
  f32x4 acc[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int blk, const Blk& B) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int t = t0 + blk * V + v;
      const int c = chunk(t);
      const uint32_t sb_on = valid(t) ? 0xFFFFFFFFu : 0u;
      const uint4* xq = reinterpret_cast<const uint4*>(lx + xrow + (c - c0) * 64);
      uint4 xp[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) xp[j] = xq[j];
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const uint32_t sb = lsb[(16 * r + i) * gr + (c >> GS) - g0] & sb_on;
        const f16 sv = __builtin_bit_cast(f16, (uint16_t)(sb & 0xFFFFu));
        const f16 bv = __builtin_bit_cast(f16, (uint16_t)(sb >> 16));
        const h2 s2 = {sv, sv}, b2 = {bv, bv};
        const uint32_t wd[4] = {B.w[v][r].x, B.w[v][r].y, B.w[v][r].z, B.w[v][r].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              word_operand<SYM>(wd[j], s2, b2), as_operand(xp[j].x, xp[j].y, xp[j].z, xp[j].w), acc[r], 0, 0, 0);
      }
    }
  };
  Blk A, B;
  load(0, A);
  __syncthreads();  // x, scales and biases staged
  __builtin_amdgcn_sched_barrier(0);
  int bk = 0;
  for (; bk + 2 < nb; bk += 2) {
    load(bk + 1, B);
    __builtin_amdgcn_sched_barrier(0);
    compute(bk, A);
    load(bk + 2, A);
    __builtin_amdgcn_sched_barrier(0);
    compute(bk + 1, B);
  }
  if (nb - bk == 2) {
    load(bk + 1, B);
    __builtin_amdgcn_sched_barrier(0);
    compute(bk, A);
    compute(bk + 1, B);
  } else {
    compute(bk, A);
  }
  __syncthreads();  // the staged data is dead: the reduction reuses the LDS
  f32x4* red = reinterpret_cast<f32x4*>(smem);  // [NW][RB][64]
#pragma unroll
  for (int r = 0; r < RB; ++r) red[(wv * RB + r) * 64 + lane] = acc[r];
  __syncthreads();
  for (int o = threadIdx.x; o < RB * 256; o += NW * 64) {
    const int e = o & 3, gg = (o >> 2) & 3, m = (o >> 4) & 15, r = o >> 8;
    const int n = 16 * (rb0 + r) + 4 * gg + e;
    if (m < M && n < N) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += red[(w * RB + r) * 64 + 16 * gg + m][e];
      if (part)
        part[((int64_t)blockIdx.y * M + m) * N + n] = sum;
      else
        y[(int64_t)m * ldy + n] = sum;
    }
  }
}

// The staged kernel's launch shape: K-ranges S and LDS bytes; S = 0 when it does not apply.
constexpr int kMfsNW = 8, kMfsRB = 2, kMfsV = 2;
constexpr size_t kMfsMaxLds = 80 * 1024;  // two workgroups per CU
struct MfsPlan {
  int S, U, xpitch, gr;
  size_t lds;
};
MfsPlan mfs_plan(int64_t M, int64_t N, int64_t K, bool sym) {
  MfsPlan p{0, 0, 0, 0, 0};
  if (M < 5 || M > 8 || N * K / 2 < ((int64_t)24 << 20)) return p;  // measured at M = 8
  const int T = (int)((K / 32 + 3) / 4);
  const int64_t gx = ((N + 15) / 16 + kMfsRB - 1) / kMfsRB;
  int S = 1;  // K-ranges: about two workgroups per CU
  while (S < 16 && gx * S * 2 <= 512) S *= 2;
  for (; S <= 16; S *= 2) {
    const int U = (T + S * kMfsNW - 1) / (S * kMfsNW);
    const int rc = kMfsNW * U * 4;                   // chunks of one K-range, at most
    const int xpitch = rc * 64 + 16;                 // 16 bytes apart in the LDS banks per x row
    const int gr = rc / (sym ? 4 : 2) + 1;           // groups of one K-range, at most
    size_t lds = (size_t)M * xpitch + (size_t)16 * kMfsRB * gr * 4;
    const size_t red = (size_t)kMfsNW * kMfsRB * 64 * 16;
    if (lds < red) lds = red;
    if (lds <= kMfsMaxLds) {
      p.S = (T + kMfsNW * U - 1) / (kMfsNW * U);     // no empty K-range
      p.U = U;
      p.xpitch = xpitch;
      p.gr = gr;
      p.lds = lds;
      return p;
    }
  }
  return p;
}

template <bool SYM>
void launch_mfs(const uint32_t* qw, const uint16_t* s, const uint16_t* b, const uint16_t* x, int64_t ldx,
                float* y, int64_t ldy, int M, int N, int K, const MfsPlan& p, float* part, hipStream_t st) {
  static std::once_flag lds_attr[kMaxDevices];
  once_per_device(lds_attr, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_mfs_kernel<kMfsNW, kMfsRB, kMfsV, SYM>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMfsMaxLds);
  });
  const int grid = ((N + 15) / 16 + kMfsRB - 1) / kMfsRB;
  hipLaunchKernelGGL((gemv_mfs_kernel<kMfsNW, kMfsRB, kMfsV, SYM>), dim3(grid, p.S), dim3(kMfsNW * 64), p.lds, st,
                     qw, s, b, x, ldx, y, ldy, M, N, K, p.U, p.S > 1 ? part : nullptr, p.xpitch, p.gr);
  if (p.S > 1) {
    const int64_t MN = (int64_t)M * N;
    hipLaunchKernelGGL(mf_reduce_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, st, part, y, ldy, M, N,
                       p.S);
  }
}

// S > 1: S K-ranges on separate workgroups, partial sums in part ([S][M][N] f32), then added
template <int NW, int RB, int V, bool SYM>
void launch_mf(const uint32_t* qw, const uint16_t* s, const uint16_t* b, const uint16_t* x,
               int64_t ldx, float* y, int64_t ldy, int M, int N, int K, int S, float* part, hipStream_t st) {
  const int T = (K / 32 + 3) / 4;            // steps of 4 chunks (128 elements) per row
  const int U = (T + S * NW - 1) / (S * NW); // steps per wave
  const int grid = ((N + 15) / 16 + RB - 1) / RB;
  hipLaunchKernelGGL((gemv_mf_kernel<NW, RB, V, SYM>), dim3(grid, S), dim3(NW * 64), 0, st, qw, s, b, x,
                     ldx, y, ldy, M, N, K, U, S > 1 ? part : nullptr);
  if (S > 1) {
    const int64_t MN = (int64_t)M * N;
    hipLaunchKernelGGL(mf_reduce_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, st, part, y, ldy, M, N,
                       S);
  }
}

// ------------------------------------------------------------------ M = 1 on row slices
// The M = 1 GEMV is bound by its VALU work as much as by HBM: with the weights already in
// cache the arithmetic alone takes most of a launch.  This kernel cuts the instructions per
// weight and the per-row overhead:
//  * Work unit = one row x one slice of 64 chunks (2048 elements) of K: lane l of the wave on
//    slice j holds chunk 64 j + l of the row, so a load instruction reads 1 KB of one row.
//    KS = ceil(C / 64) slices of the same R rows run as the KS waves of one workgroup and
//    their row sums are added through LDS in slice order (deterministic); with KS = 1 a
//    workgroup holds four independent waves.  Each lane keeps the 32 x values of its chunk
//    in registers.  Lanes past the row end load a clamped chunk with a zero scale and bias.
//  * Loads are buffer loads whose row offset is wave-uniform and sits in a scalar register,
//    so no vector instruction computes an address.
//  * Codes become exact f16 through the fp8 converter: in the e4m3 encoding a byte holding
//    0..15 is the number q * 2^-9 exactly (the subnormals and the first normal binade are one
//    evenly spaced range), so converting with the scale 2^9 yields q.  The word's low
//    nibbles (w & 0x0F0F0F0F) and high nibbles ((w >> 4) & 0x0F0F0F0F) give the pairs
//    (q0,q2) (q4,q6) and (q1,q3) (q5,q7): 7 instructions for 8 codes instead of 9, so 15 per
//    word with the FMA and the dot products.  The symmetric format subtracts 8 (exact) before
//    its FMA, so both formats pair and sum their products in the same order and give the same
//    bits where their weights agree (b = -8 s).
// BIG: 2 GB of codes or more -- the buffers then start at each wave's own rows (64-bit base,
// offsets below R rows); otherwise one buffer per array and the row offset in the scalar
// register (measured 1-2 % faster).
template <int R, int KS, bool SYM, bool BIG, int MT>
__global__ __launch_bounds__(KS == 1 ? kWG : KS * 64) void gemv1s_kernel(
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc, const uint16_t* __restrict__ bi,
    const uint16_t* __restrict__ x, int64_t ldx, float* __restrict__ y, int64_t ldy, int N, int K,
    int nblocks, uint32_t qblk, uint32_t sblk) {  // bytes of codes / of scales per block of R rows
  __shared__ float red[KS][R * MT];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slice = KS == 1 ? 0 : wave;
  const int blk = KS == 1 ? (int)blockIdx.x * (kWG / 64) + wave : (int)blockIdx.x;
  const int C = K / 32, G = K / Fmt<SYM>::kGroupSize;
  const int c = slice * 64 + lane;
  const int cc = min(c, C - 1);
  const uint32_t sb_on = c < C ? 0xFFFFu : 0u;  // past the row end: s = b = 0, every weight 0
  const int voff_q = cc * 16, voff_s = (cc >> Fmt<SYM>::kChunkShift) * 2;

  // x first: loads complete in order, so the math can wait for x without the weights
  uint4 xv[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const uint4* xp = reinterpret_cast<const uint4*>(x + m * ldx + cc * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[m][i] = xp[i];
  }
  uint4 w[R];
  uint32_t sv[R], bv[R];
  const int b0 = min(blk, nblocks - 1);
  const int nbase = BIG ? b0 * R : 0;  // first row of the buffers
  const uint64_t qoff = BIG ? (uint64_t)(uint32_t)b0 * qblk : 0, soff = BIG ? (uint64_t)(uint32_t)b0 * sblk : 0;
  const __amdgpu_buffer_rsrc_t rq = buffer_of(reinterpret_cast<const char*>(qw) + qoff);
  const __amdgpu_buffer_rsrc_t rs = buffer_of(reinterpret_cast<const char*>(sc) + soff);
  const __amdgpu_buffer_rsrc_t rb = buffer_of(reinterpret_cast<const char*>(SYM ? sc : bi) + soff);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int dn = min(b0 * R + r, N - 1) - nbase;  // tail rows reload the last row, never stored
    w[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, voff_q, dn * C * 16, 2));
    sv[r] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff_s, dn * G * 2, 0);
    bv[r] = SYM ? 0u : __builtin_amdgcn_raw_buffer_load_b16(rb, voff_s, dn * G * 2, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (KS == 1 && blk >= nblocks) return;

  uint4 xp[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) xp[m][i] = pair_up_cvt(xv[m][i]);
  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const h2 s2 = __builtin_bit_cast(h2, (sv[r] & sb_on) * 0x10001u);
    const h2 b2 = __builtin_bit_cast(h2, (bv[r] & sb_on) * 0x10001u);
    if constexpr (MT == 1) {
      float a0 = word_fma_cvt<SYM>(w[r].x, s2, b2, xp[0][0], 0.f);
      float a1 = word_fma_cvt<SYM>(w[r].y, s2, b2, xp[0][1], 0.f);
      a0 = word_fma_cvt<SYM>(w[r].z, s2, b2, xp[0][2], a0);
      a1 = word_fma_cvt<SYM>(w[r].w, s2, b2, xp[0][3], a1);
      acc[r][0] = group_sum<64>(a0 + a1);
    } else {
      // each word dequantized once, its weight pairs dotted with every row of x (the same
      // pairing and chaining per row as at M = 1)
      float a[MT][2];
#pragma unroll
      for (int m = 0; m < MT; ++m) a[m][0] = a[m][1] = 0.f;
      const uint32_t wd[4] = {w[r].x, w[r].y, w[r].z, w[r].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h2 q0, q1, q2, q3;
        cvt_codes<SYM>(wd[j], q0, q1, q2, q3);
        const uint32_t p0 = as_u32(__builtin_elementwise_fma(q0, s2, b2));
        const uint32_t p1 = as_u32(__builtin_elementwise_fma(q1, s2, b2));
        const uint32_t p2 = as_u32(__builtin_elementwise_fma(q2, s2, b2));
        const uint32_t p3 = as_u32(__builtin_elementwise_fma(q3, s2, b2));
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float t = a[m][j & 1];
          t = dot2(p0, xp[m][j].x, t);
          t = dot2(p1, xp[m][j].y, t);
          t = dot2(p2, xp[m][j].z, t);
          t = dot2(p3, xp[m][j].w, t);
          a[m][j & 1] = t;
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[r][m] = group_sum<64>(a[m][0] + a[m][1]);
    }
  }
  if constexpr (KS == 1) {
    if (lane == 63) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (blk * R + r < N) y[m * ldy + blk * R + r] = acc[r][m];
    }
  } else {
    if (lane == 63) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) red[slice][r * MT + m] = acc[r][m];
    }
    __syncthreads();
    if (wave == 0 && lane < R * MT && blk * R + lane / MT < N) {
      float v = red[0][lane];
#pragma unroll
      for (int j = 1; j < KS; ++j) v += red[j][lane];
      y[(lane % MT) * ldy + blk * R + lane / MT] = v;
    }
  }
}

template <int R, int KS, bool SYM, int MT>
void launch_rs(const uint32_t* qw, const uint16_t* s, const uint16_t* b, const uint16_t* x,
               int64_t ldx, float* y, int64_t ldy, int N, int K, hipStream_t st) {
  const int nblocks = (N + R - 1) / R;
  const int grid = KS == 1 ? (nblocks + kWG / 64 - 1) / (kWG / 64) : nblocks;
  const uint32_t qblk = (uint32_t)R * (uint32_t)(K / 2);
  const uint32_t sblk = (uint32_t)R * (uint32_t)(K / Fmt<SYM>::kGroupSize) * 2;
  const dim3 block(KS == 1 ? kWG : KS * 64);
  if ((int64_t)N * (K / 2) >= ((int64_t)1 << 31))
    hipLaunchKernelGGL((gemv1s_kernel<R, KS, SYM, true, MT>), dim3(grid), block, 0, st, qw, s, b, x, ldx,
                       y, ldy, N, K, nblocks, qblk, sblk);
  else
    hipLaunchKernelGGL((gemv1s_kernel<R, KS, SYM, false, MT>), dim3(grid), block, 0, st, qw, s, b, x, ldx,
                       y, ldy, N, K, nblocks, qblk, sblk);
}

template <int KS, bool SYM, int MT>
void launch_rs_r(int R, const uint32_t* qw, const uint16_t* s, const uint16_t* b,
                 const uint16_t* x, int64_t ldx, float* y, int64_t ldy, int N, int K, hipStream_t st) {
  if (R >= 4)
    launch_rs<4, KS, SYM, MT>(qw, s, b, x, ldx, y, ldy, N, K, st);
  else if (KS == 1 && R == 3)
    launch_rs<3, KS, SYM, MT>(qw, s, b, x, ldx, y, ldy, N, K, st);
  else
    launch_rs<2, KS, SYM, MT>(qw, s, b, x, ldx, y, ldy, N, K, st);
}

template <bool SYM, int MT>
void launch_rs_ks(int KS, int R, const uint32_t* qw, const uint16_t* s, const uint16_t* b,
                  const uint16_t* x, int64_t ldx, float* y, int64_t ldy, int N, int K, hipStream_t st) {
  switch (KS) {
    case 1: launch_rs_r<1, SYM, MT>(R, qw, s, b, x, ldx, y, ldy, N, K, st); break;
    case 2: launch_rs_r<2, SYM, MT>(R, qw, s, b, x, ldx, y, ldy, N, K, st); break;
    case 3: launch_rs_r<3, SYM, MT>(R, qw, s, b, x, ldx, y, ldy, N, K, st); break;
    case 4: launch_rs_r<4, SYM, MT>(R, qw, s, b, x, ldx, y, ldy, N, K, st); break;
    case 5: launch_rs_r<5, SYM, MT>(R, qw, s, b, x, ldx, y, ldy, N, K, st); break;
    case 6: launch_rs_r<6, SYM, MT>(R, qw, s, b, x, ldx, y, ldy, N, K, st); break;
    case 7: launch_rs_r<7, SYM, MT>(R, qw, s, b, x, ldx, y, ldy, N, K, st); break;
    default: launch_rs_r<8, SYM, MT>(R, qw, s, b, x, ldx, y, ldy, N, K, st); break;
  }
}

// three or four rows of x: 4 rows per wave on every shape measured
template <bool SYM, int MT>
void launch_rs_ks4(int KS, const uint32_t* qw, const uint16_t* s, const uint16_t* b,
                   const uint16_t* x, int64_t ldx, float* y, int64_t ldy, int N, int K, hipStream_t st) {
  switch (KS) {
    case 1: launch_rs<4, 1, SYM, MT>(qw, s, b, x, ldx, y, ldy, N, K, st); break;
    case 2: launch_rs<4, 2, SYM, MT>(qw, s, b, x, ldx, y, ldy, N, K, st); break;
    case 3: launch_rs<4, 3, SYM, MT>(qw, s, b, x, ldx, y, ldy, N, K, st); break;
    case 4: launch_rs<4, 4, SYM, MT>(qw, s, b, x, ldx, y, ldy, N, K, st); break;
    case 5: launch_rs<4, 5, SYM, MT>(qw, s, b, x, ldx, y, ldy, N, K, st); break;
    case 6: launch_rs<4, 6, SYM, MT>(qw, s, b, x, ldx, y, ldy, N, K, st); break;
    case 7: launch_rs<4, 7, SYM, MT>(qw, s, b, x, ldx, y, ldy, N, K, st); break;
    default: launch_rs<4, 8, SYM, MT>(qw, s, b, x, ldx, y, ldy, N, K, st); break;
  }
}

// Row-slice policy, measured on MI355X (graph launches on distinct weights), rows per wave
// from the number of (row, slice) units: at M = 1, 4 from 30000 units, 3 from 16000 when rows
// are one slice long, else 2, except that one-slice rows that fit one wave per SIMD at 3 rows
// per wave but not at 2 take 3, so no SIMD carries 4 rows (2560 x 2048: 2.83 vs 3.00 us); at
// M = 2, 4 from 12000, 3 from 2304 for one-slice rows, else 2
// (22016 x 2048: 8.3 us; 2560 x 2048: 3.05; 2048 x 2048: 2.76; 2048 x 11008: 6.25); at M = 3
// and 4, 4 (faster than the matrix cores on every decode, classify and Gemma-shaped matrix:
// 22016 x 2048 10.0 vs 15.8 us at M = 3, 11.3 vs 16.0 at M = 4; from M = 6 the matrix cores
// win on most).  Returns false when the shape is not covered: M outside 1..4, more than 8
// slices, or at M = 1 rows of at most 32 chunks (a half-empty slice; the 32-lane team kernel
// is faster there).
template <bool SYM>
bool launch_gemv_rs(int M, const uint32_t* qw, const uint16_t* s, const uint16_t* b,
                    const uint16_t* x, int64_t ldx, float* y, int64_t ldy, int N, int K,
                    hipStream_t st) {
  const int C = K / 32;
  const int KS = (C + 63) / 64;
  if (KS > 8 || M < 1 || M > 4 || (M == 1 && C <= 32)) return false;
  const int64_t units = (int64_t)N * KS;
  if (M == 1) {
    constexpr int kSimds = 256 * 4;  // MI355X: 256 CUs of 4 SIMDs
    const bool fits3 = KS == 1 && N > 2 * kSimds && N <= 3 * kSimds;
    const int R = units >= 30000 ? 4 : ((units >= 16000 && KS == 1) || fits3) ? 3 : 2;
    launch_rs_ks<SYM, 1>(KS, R, qw, s, b, x, ldx, y, ldy, N, K, st);
  } else if (M == 2) {
    const int R = units >= 12000 ? 4 : (units >= 2304 && KS == 1) ? 3 : 2;
    launch_rs_ks<SYM, 2>(KS, R, qw, s, b, x, ldx, y, ldy, N, K, st);
  } else if (M == 3) {
    launch_rs_ks4<SYM, 3>(KS, qw, s, b, x, ldx, y, ldy, N, K, st);
  } else {
    launch_rs_ks4<SYM, 4>(KS, qw, s, b, x, ldx, y, ldy, N, K, st);
  }
  return true;
}

// M = 1: rows of more than 32 chunks (K > 1024) and up to 8 slices (K <= 16384) on row
// slices; shorter rows on 32-lane teams of the OR-trick kernel (one chunk per lane, x in
// LDS); longer rows fall through to the general kernel.
template <bool SYM>
bool launch_gemv_m1(const uint32_t* qw, const uint16_t* s, const uint16_t* b, const uint16_t* x,
                    float* y, int N, int K, hipStream_t st) {
  if (launch_gemv_rs<SYM>(1, qw, s, b, x, K, y, N, N, K, st)) return true;
  if (K / 32 <= 32) {
    launch_m1<32, 1, 1, true, SYM>(qw, s, b, x, y, N, K, 1, st);
    return true;
  }
  return false;
}

// Row blocks per wave of the matrix-core path for N rows.
int mf_rb(int N) {
  const int nrb = (N + 15) / 16;
  return nrb >= 768 ? 4 : nrb >= 384 ? 2 : 1;
}

// Whether (M, K) takes the matrix-core path: 5 <= M, or M = 3..4 past the row slices' 16384
// elements (mirrors launch_gemv_fmt).
bool uses_mf(int64_t M, int64_t K) { return M >= 5 || (M >= 3 && (K / 32 + 63) / 64 > 8); }

// K-ranges on separate workgroups for the matrix-core path: long rows (K >= 6144) that give at
// most 128 workgroups (the 2048-row down projections) run as 2 K-ranges on 256 workgroups; a
// second launch adds the two partial sums.  Measured (graph-replayed, distinct weights; one /
// two / four K-ranges): 2048 x 6144 at M = 16 11.8 / 9.4 / 10.1 us, 2048 x 11008 at M = 16
// 18.0 / 13.4 / 13.8 us and at M = 8 13.8 / 11.4 / 11.5 us; the 240 workgroups of the 3840-row
// Gemma down lose with any split (M = 8: 22.8 / 25.8 / 26.8 us).
int mf_splits(int64_t M, int64_t N, int64_t K) {
  if (!uses_mf(M, K) || K < 6144) return 1;
  const int64_t grid = ((N + 15) / 16 + mf_rb((int)N) - 1) / mf_rb((int)N);
  return grid <= 128 ? 2 : 1;
}

// Matrix-core policy (5 <= M <= 16, and M = 3..4 past 16384 elements), measured on MI355X
// (back-to-back graph launches on distinct weights):
// four row blocks per wave once there are >= 768 of them, two from 384, otherwise one with
// eight waves splitting K when rows are long.  Up to 4 rows of x the row slices are ahead.
// part: mf_splits(M, N, K) * M * N floats, or nullptr (then one K-range).
template <bool SYM>
void launch_gemv_mf(const uint32_t* qw, const uint16_t* s, const uint16_t* b, const uint16_t* x,
                    int64_t ldx, float* y, int64_t ldy, int M, int N, int K, float* part, hipStream_t st) {
  const MfsPlan ps = mfs_plan(M, N, K, SYM);
  if (ps.S == 1 || (ps.S > 1 && part)) {
    launch_mfs<SYM>(qw, s, b, x, ldx, y, ldy, M, N, K, ps, part, st);
    return;
  }
  const int S = part ? mf_splits(M, N, K) : 1;
  const int rb = mf_rb(N);
  if (rb == 4)
    launch_mf<8, 4, 1, SYM>(qw, s, b, x, ldx, y, ldy, M, N, K, S, part, st);
  else if (rb == 2)
    launch_mf<8, 2, 1, SYM>(qw, s, b, x, ldx, y, ldy, M, N, K, S, part, st);
  else if (K >= 8192)
    launch_mf<8, 1, 1, SYM>(qw, s, b, x, ldx, y, ldy, M, N, K, S, part, st);
  else
    launch_mf<4, 1, 1, SYM>(qw, s, b, x, ldx, y, ldy, M, N, K, S, part, st);
}

template <bool SYM>
void launch_gemv_fmt(const uint32_t* qw, const uint16_t* s, const uint16_t* b, const uint16_t* x,
                     int64_t ldx, float* y, int64_t ldy, int M, int N, int K, float* part, hipStream_t st) {
  if (M <= 1 && launch_gemv_m1<SYM>(qw, s, b, x, y, N, K, st)) return;
  if (M >= 2 && M <= 4 && launch_gemv_rs<SYM>(M, qw, s, b, x, ldx, y, ldy, N, K, st)) return;
  if (M >= 3) {
    launch_gemv_mf<SYM>(qw, s, b, x, ldx, y, ldy, M, N, K, part, st);
    return;
  }
  if (M <= 1)
    launch_p<1, SYM>(qw, s, b, x, ldx, y, ldy, M, N, K, st);
  else
    launch_p<2, SYM>(qw, s, b, x, ldx, y, ldy, M, N, K, st);
}

}  // namespace

void launch_gemv(const uint32_t* qw, const uint16_t* s, const uint16_t* b, const uint16_t* x,
                 int64_t ldx, float* y, int64_t ldy, int M, int N, int K, void* ws, hipStream_t st) {
  launch_gemv_fmt<false>(qw, s, b, x, ldx, y, ldy, M, N, K, reinterpret_cast<float*>(ws), st);
}

size_t gemv_ws_bytes(int64_t M, int64_t N, int64_t K) {
  // the staged kernel's plan is the same for both formats except for its LDS bytes, which do not
  // change S on the shapes it takes (checked by the affine plan, the larger one)
  const MfsPlan ps = uses_mf(M, K) ? mfs_plan(M, N, K, false) : MfsPlan{0, 0, 0, 0, 0};
  const int S = ps.S ? ps.S : mf_splits(M, N, K);
  return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

void launch_gemv_sym128(const uint32_t* qw, const uint16_t* s, const uint16_t* x, int64_t ldx,
                        float* y, int64_t ldy, int M, int N, int K, void* ws, hipStream_t st) {
  launch_gemv_fmt<true>(qw, s, nullptr, x, ldx, y, ldy, M, N, K, reinterpret_cast<float*>(ws), st);
}

}  // namespace w4
