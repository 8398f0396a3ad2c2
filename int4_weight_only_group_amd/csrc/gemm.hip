// gemm_f16: C[m][n] = sum_k A[m][k] B[k][n], f16 in, f32 accumulate and out.
//
// Two users on the pages' path ("The inference engine -- Mojo 1.0 on Metal"):
//  * the prefill GEMM on the transposed f16 scratch ("Crossing Mojo 1.0": dequantize once,
//    then a half-precision matrix-unit GEMM; edge guards hoisted out of the hot loop);
//  * the f16 LM head at decode, which streams a [hidden x vocab] matrix once per token
//    ("What's inside the engine today").
//
// Paths, chosen per call by shape and alignment:
//  * MFMA (M > 8; 16-byte aligned operands): 256- or 320-row x
//    256-column block tiles, operands moved HBM -> LDS by LDS DMA through a 4-stage ring,
//    eight waves (two per SIMD) each owning a 128 (160) x 64 tile of v_mfma_f32_32x32x16_f16;
//    up to 32 rows, 32-row tiles with every wave on 32 x 32 (a stream of B, e.g. a head read
//    by 16 rows).  B is read from its [K][N] layout with transposing LDS reads.  K % 32 != 0
//    takes a register-staged variant.  Tails: rows of A
//    and column blocks of B are clamped on load (never stored) and the K tail is zero-filled,
//    so the MFMA loop itself has no guards.  Too few tiles for the CUs: K is split and the
//    slices summed in a fixed order by a second kernel.
//  * small M (M <= 8: the decode head, speculative-verify rows): each lane owns 8, 4 or 2
//    contiguous columns and streams B rows with 16-, 8- or 4-byte loads; byte permutes pair
//    the values of two k and v_dot2_f32_f16 multiplies them with the wave-uniform A pair; the
//    four waves of a workgroup split K and reduce through LDS.
//  * plain (any other shape or alignment, e.g. one strided column of a head): a workgroup
//    per (column, 16 rows), threads split K.
#include <atomic>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "w4_dequant_tile.h"
#include "w4_internal.h"

namespace w4 {

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(f16, h); }

// ------------------------------------------------------------------------ MFMA path
// 256 x 256 block tile, BK = 64, four waves each owning a 128 x 128 tile: 4 x 4
// v_mfma_f32_32x32x16_f16 accumulators (256 f32 per lane, in AGPRs), one wave per SIMD.
// LDS holds two stages of A [256][64] and B^T [256][64] (K contiguous, padded rows), so
// each K-tile costs one barrier and the next tile's global loads are in flight while the
// matrix cores work on the current one.  B arrives [K][N] (N contiguous); each thread loads
// an 8 (k) x 8 (n) block with eight 16-byte loads and transposes it in registers with
// v_perm_b32 before a 16-byte LDS store per column.  Tails: A rows and B column blocks are
// clamped on load and never stored, the K tail is zero-filled, so the MFMA loop has no
// guards.  Tiles are ordered so that each XCD works on a contiguous range of them (its own
// L2 then holds the A and B panels they share).  Shapes with too few tiles for 256 CUs split
// K; the slices' partial tiles go to the workspace and a second kernel adds them in a fixed
// order (deterministic).
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LDK = BK + 8;                      // f16 per LDS row (144 B)
// B^T rows get 16 extra bytes every 8 rows: the transposed stores put consecutive lanes 8
// rows apart, which with 144-byte rows would land them all in the same LDS banks.
__device__ __forceinline__ int brow(int n) { return n * LDK + (n >> 3) * 8; }
constexpr int STAGE = BM * LDK + BN * LDK + (BN / 8) * 8;  // f16 per stage
constexpr size_t kGemmLds = 2 * STAGE * sizeof(uint16_t);

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int d) {
  return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

struct GemmArgs {
  const uint16_t* A;
  const uint16_t* B;
  float* C;
  float* ws;
  int64_t lda, ldb, ldc;
  int M, N, K;
  int tilesM, tilesN, ksplit, kslice;
  int wide;  // C rows take 16-byte stores (C 16-byte aligned, ldc a multiple of 4)
  int nwg;   // the GEMM's workgroups: blockIdx.x < nwg; dequant workgroups follow (SIDE)
  // the dequant-transpose that runs in the same launch (N x K codes; dq_sym: the symmetric
  // group-128 format, dq_b unused)
  const uint32_t* dq_qw;
  const uint16_t* dq_s;
  const uint16_t* dq_b;
  uint16_t* dq_wt;
  int64_t dq_ld;
  int dq_N, dq_K, dq_vec, dq_sym;
};

__device__ __forceinline__ void tile_of(const GemmArgs& g, int bid, int& tm, int& tn, int& split) {
  // XCD-aware order: the hardware deals workgroups round-robin to 8 XCDs; give each XCD a
  // contiguous range of the linear order below.
  const int total = g.nwg;
  const int q = total / 8, rem = total % 8, xcd = bid % 8, idx = bid / 8;
  const int lin = xcd * q + min(xcd, rem) + idx;
  const int nt = g.tilesM * g.tilesN;
  split = lin / nt;
  const int t = lin - split * nt;
  // groups of 4 tile-rows, column-major inside a group: consecutive tiles share B panels
  constexpr int GM = 4;
  const int group = t / (GM * g.tilesN);
  const int first_m = group * GM;
  const int gsize = min(g.tilesM - first_m, GM);
  const int in = t - group * GM * g.tilesN;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

__global__ __launch_bounds__(256, 1) void gemm_mfma_kernel(GemmArgs g) {
  extern __shared__ __align__(16) uint16_t lds[];
  int tm, tn, split;
  tile_of(g, blockIdx.x, tm, tn, split);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = split * g.kslice;
  const int kend = min(g.K, kbeg + g.kslice);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // global -> register mapping: A rows a_r + 32 i, 8-element chunk a_kc; B 8x8 block
  const int a_r = tid >> 3, a_kc = (tid & 7) * 8;
  const int b_nb = tid & 31, b_kb = tid >> 5;
  const uint16_t* a_src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    a_src[i] = g.A + (int64_t)min(m0 + a_r + 32 * i, g.M - 1) * g.lda + a_kc;
  const uint16_t* b_src = g.B + min(n0 + b_nb * 8, g.N - 8) + (int64_t)(b_kb * 8) * g.ldb;

  uint4 ra[8], rb[8];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      ra[i] = (k0 + a_kc < kend) ? *reinterpret_cast<const uint4*>(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rb[i] = (k0 + b_kb * 8 + i < kend)
                  ? *reinterpret_cast<const uint4*>(b_src + (int64_t)(k0 + i) * g.ldb)
                  : make_uint4(0, 0, 0, 0);
  };
  auto store = [&](int stage) {
    uint16_t* As = lds + stage * STAGE;
    uint16_t* Bs = As + BM * LDK;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint4*>(&As[(a_r + 32 * i) * LDK + a_kc]) = ra[i];
    // 8x8 transpose of 16-bit values: column j of the block becomes 8 contiguous k
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      const int d = j >> 1;
      uint4 o;
      o.x = __builtin_amdgcn_perm(dword_of(rb[1], d), dword_of(rb[0], d), sel);
      o.y = __builtin_amdgcn_perm(dword_of(rb[3], d), dword_of(rb[2], d), sel);
      o.z = __builtin_amdgcn_perm(dword_of(rb[5], d), dword_of(rb[4], d), sel);
      o.w = __builtin_amdgcn_perm(dword_of(rb[7], d), dword_of(rb[6], d), sel);
      *reinterpret_cast<uint4*>(&Bs[brow(b_nb * 8 + j) + b_kb * 8]) = o;
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (kend - kbeg + BK - 1) / BK;
  load(kbeg);
  store(0);
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    if (t + 1 < nk) load(kbeg + (t + 1) * BK);
    const uint16_t* As = lds + (t & 1) * STAGE;
    const uint16_t* Bs = As + BM * LDK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kof = ks * 16 + (lane >> 5) * 8;
      f16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const f16x8*>(&As[(wm * 128 + i * 32 + (lane & 31)) * LDK + kof]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const f16x8*>(&Bs[brow(wn * 128 + j * 32 + (lane & 31)) + kof]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (t + 1 < nk) store((t + 1) & 1);
    __syncthreads();
  }

  // D layout of a 32x32 tile: lane l, value r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  float* out = g.ksplit == 1 ? g.C : g.ws + (int64_t)split * g.M * g.N;
  const int64_t ldo = g.ksplit == 1 ? g.ldc : g.N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row < g.M && col < g.N) out[(int64_t)row * ldo + col] = acc[i][j][r];
      }
    }
}

// ------------------------------------------------------------- MFMA path, LDS DMA
// Same 256 x 256 tile as above, but both operands travel HBM -> LDS with gfx950's 16-byte
// LDS DMA (global_load_lds_dwordx4: lane l's 16 bytes land at the instruction's LDS base +
// 16 l), so no registers hold tiles in flight.  Four LDS stages of BK = 32 (32 KB each) keep
// three K-tiles in flight while the matrix cores work on the fourth.  Eight waves, two per
// SIMD, each own 128 x 64 of the tile (4 x 2 accumulators): while one wave of a SIMD waits
// on its DMA issue or a barrier, the other issues MFMAs (measured 7-13 % faster than four
// waves of 128 x 128).  B stays [k][n] in LDS and its MFMA operand (8 consecutive k of one
// column per lane) is read with two ds_read_b64_tr_b16: within each 16-lane group, result
// lane i gets element i mod 4 of source lanes 4e + i / 4 (e = 0..3), so source lane L
// pointing at B[k0 + L / 4][n0 + 4 (L mod 4)] hands lane i the column B[k0 .. k0 + 3][n0 + i].
// The 16-byte chunks are permuted in LDS (a_rot, b_swz below).  Waits are explicit
// (vmcnt for this wave's DMA, then a plain s_barrier): a __syncthreads() would drain every
// K-tile in flight.  Requires K % 32 == 0 (split-K slices are multiples of 32); other K take
// the register-staged kernel above.
constexpr int DBK = 32;
constexpr int DSTAGES = 4;
constexpr size_t dma_lds(int bm) { return (size_t)DSTAGES * (bm + BN) * DBK * 2; }  // 128 / 144 KB
constexpr int kDmaWaves = 8;  // waves per workgroup (4 also builds: one per SIMD, 128 x 128)

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));

// One 16-byte-per-lane LDS DMA (lds: wave-uniform LDS byte address of the 1 KB destination,
// passed in m0, which the compiler sets).  Issued as inline asm: through the builtin, the
// compiler would protect every later LDS read with a wait for all DMA in flight, which
// serializes the K-tile pipeline; the kernel waits explicitly instead (W4_SYNC).  The s_nop
// gives the wait states an LDS DMA needs after an m0 write, which the compiler does not
// insert for an asm statement.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds) {
  asm volatile("s_nop 1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds) : "memory");
}

// wait for this wave's DMA down to n outstanding instructions and for all of its LDS reads
// (a stage may be refilled right after the barrier), then barrier
#define W4_SYNC(n) asm volatile("s_waitcnt vmcnt(" #n ") lgkmcnt(0)\n\ts_barrier" ::: "memory")

// LDS layouts of the DMA kernel's stages (bank conflicts counted with SQ_LDS_BANK_CONFLICT
// on in-bounds probes of exactly these read patterns: a 16-byte read of 64 lanes takes 4 LDS
// cycles when conflict-free, a transposing 8-byte read 2).
//  A stage: row r holds 64 B = four 16-B chunks; logical chunk c sits at physical chunk
//  (c + a_rot(r)) & 3, a_rot(r) = (r + (r >> 2)) & 3.  A fragment read takes 32 consecutive
//  rows (r0 % 32 == 0) at logical chunk c for lanes 0-31 and c + 1 for lanes 32-63; the
//  rotation gives each of any 4 rows of equal r & 3 (r0 + j + 4t, t = 0..3) a different
//  chunk, and measured 4 cycles per read, where an XOR layout bijective over the same row
//  sets took 8 and the plain layout 16.
//  B stage: k-row holds 512 B = 32 chunks; chunk c sits at c ^ b_swz(k).  A transposing b64
//  read takes, per 16 lanes, 4 consecutive k-rows x 2 chunks and, per 32 lanes, 4 k-rows x
//  4 chunks; b_swz(k) = 2 * h(k & 3) with h(x) = (x ^ 2x) & 7, whose bits 1..2 and 2..3 are
//  both bijective in k & 3, spreads either phase over distinct banks (measured 2 cycles per
//  read).
__device__ __forceinline__ int a_rot(int r) { return (r + (r >> 2)) & 3; }
__device__ __forceinline__ int b_swz(int k) {
  const int x = k & 3;
  return ((x ^ (x << 1)) & 7) << 1;
}

// W4_SYNC with a compile-time count
template <int N>
__device__ __forceinline__ void dma_sync_n() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 0..63");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// W4_SYNC with a wave-uniform count of DMA instructions allowed to stay in flight
__device__ __forceinline__ void dma_sync(int n) {
  switch (n) {  // per-wave instructions per K-tile (2 to 5) times 0 .. 3 K-tiles
    case 24: W4_SYNC(24); break;
    case 16: W4_SYNC(16); break;
    case 15: W4_SYNC(15); break;
    case 12: W4_SYNC(12); break;
    case 10: W4_SYNC(10); break;
    case 9: W4_SYNC(9); break;
    case 8: W4_SYNC(8); break;
    case 6: W4_SYNC(6); break;
    case 5: W4_SYNC(5); break;
    case 4: W4_SYNC(4); break;
    case 3: W4_SYNC(3); break;
    case 2: W4_SYNC(2); break;
    default: W4_SYNC(0); break;
  }
}

// WMW waves along M and NW / WMW along N (two along M for the prefill tiles; one for the
// 32-row tiles of small M, where every wave takes 32 rows x 32 columns).
// The dequant workgroups of a SIDE launch: workgroup j of the nside that follow the GEMM's
// is two groups of 256 threads; group u = 2j + half takes the u-th of 2 nside equal runs of
// consecutive dequant tiles (tile t: row block t / KT, K-tile t % KT, so a run stays on a row
// block and re-reads its scale and bias lines from cache).  Every thread makes the same number
// of tile calls (two barriers each); a group whose run is shorter passes live = false.
__device__ __forceinline__ void side_dequant(const GemmArgs& g, int j, int nside, unsigned char* lds) {
  const int tid = threadIdx.x, half = tid >> 8;
  const int KT = dqt::k_tiles(g.dq_K), T = dqt::row_blocks(g.dq_N) * KT;
  const int U = 2 * nside, u = 2 * j + half;
  const int beg = (int)((int64_t)T * u / U), end = (int)((int64_t)T * (u + 1) / U);
  const int iters = (T + U - 1) / U;  // >= end - beg for every u
  for (int it = 0; it < iters; ++it) {
    const int t = beg + it;
    const bool live = t < end;
    const int rb = live ? t / KT : 0, kt = live ? t % KT : 0;
    if (g.dq_sym)  // the same for the whole launch
      dqt::tile<true>(g.dq_qw, g.dq_s, g.dq_s, g.dq_wt, g.dq_ld, g.dq_N, g.dq_K, g.dq_vec != 0, rb, kt, tid & 255,
                      live, lds + half * dqt::kLds);
    else
      dqt::tile<false>(g.dq_qw, g.dq_s, g.dq_b, g.dq_wt, g.dq_ld, g.dq_N, g.dq_K, g.dq_vec != 0, rb, kt, tid & 255,
                       live, lds + half * dqt::kLds);
  }
}

// SIDE: workgroups from g.nwg on run side_dequant instead of a tile (whole workgroups, before
// any barrier of the GEMM's code).
template <int NW, int BMT, int WMW, bool SIDE = false>
__global__ __launch_bounds__(64 * NW, 1) void gemm_dma_kernel(GemmArgs g) {
  constexpr int WN = NW / WMW;          // waves along N
  constexpr int WTN = BN / WN;          // columns per wave
  constexpr int NJ = WTN / 32;          // 32-column MFMA blocks per wave
  constexpr int WTM = BMT / WMW;        // rows per wave
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tiles of whole 32 x 32 blocks");
  constexpr int MI = WTM / 32;          // 32-row MFMA blocks per wave
  constexpr int DI = 16 / NW;           // B DMA instructions per wave and K-tile
  constexpr int AI = BMT / 16;          // A DMA instructions per K-tile (16 rows each)
  constexpr int AW = (AI + NW - 1) / NW;  // A DMA instructions per wave, at most
  constexpr int STAGE = (BMT + BN) * DBK * 2;
  extern __shared__ __align__(16) unsigned char dlds[];
  if constexpr (SIDE) {
    static_assert(NW == 8 && 2 * dqt::kLds <= (size_t)DSTAGES * (BMT + BN) * DBK * 2,
                  "two 256-thread dequant groups and their LDS");
    if ((int)blockIdx.x >= g.nwg) {
      side_dequant(g, (int)blockIdx.x - g.nwg, (int)gridDim.x - g.nwg, dlds);
      return;
    }
  }
  int tm, tn, split;
  tile_of(g, blockIdx.x, tm, tn, split);
  const int m0 = tm * BMT, n0 = tn * BN;
  const int kbeg = split * g.kslice;
  const int kend = min(g.K, kbeg + g.kslice);
  const int nk = (kend - kbeg) / DBK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // DMA source addresses (this lane, K-tile 0): wave w issues A instructions w, w + NW, ...
  // (below AI; na of them, wave-uniform) and B instructions DI*w .. DI*w + DI - 1 of 16
  const int na = (AI - wave + NW - 1) / NW;
  const int per_tile = na + DI;  // this wave's DMA instructions per K-tile
  const uint16_t* a_src[AW];
  const uint16_t* b_src[DI];
#pragma unroll
  for (int ta = 0; ta < AW; ++ta) {
    const int i = min(wave + NW * ta, AI - 1);
    const int row = 16 * i + (lane >> 2);
    const int ca = ((lane & 3) - a_rot(row)) & 3;  // the logical chunk that lands at chunk lane & 3
    a_src[ta] = g.A + (int64_t)min(m0 + row, g.M - 1) * g.lda + kbeg + ca * 8;
  }
#pragma unroll
  for (int ii = 0; ii < DI; ++ii) {
    const int i = wave * DI + ii;
    const int krow = 2 * i + (lane >> 5);
    const int cb = (lane & 31) ^ b_swz(krow);
    b_src[ii] = g.B + (int64_t)(kbeg + krow) * g.ldb + min(n0 + cb * 8, g.N - 8);
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void_t*)dlds;
  auto issue = [&](int t) {
    const uint32_t st = lds_base + (uint32_t)((t % DSTAGES) * STAGE);
#pragma unroll
    for (int ta = 0; ta < AW; ++ta)
      if (ta < na) dma16(a_src[ta] + t * DBK, st + (uint32_t)((wave + NW * ta) * 1024));
#pragma unroll
    for (int ii = 0; ii < DI; ++ii)
      dma16(b_src[ii] + (int64_t)t * DBK * g.ldb,
            st + (uint32_t)(BMT * DBK * 2 + (wave * DI + ii) * 1024));
  };

  // DMA instruction d of this wave for tile t: d < AW the A rows of instruction wave + NW d
  // (when d < na), else B k-rows 2 (DI wave + d - AW) .. + 1
  auto dma_one = [&](int t, int d) {
    const uint32_t st = lds_base + (uint32_t)((t % DSTAGES) * STAGE);
    if (d < AW) {
      if (AI % NW == 0 || d < na)  // every wave issues AW A instructions when NW divides AI
        dma16(a_src[d] + t * DBK, st + (uint32_t)((wave + NW * d) * 1024));
    } else {
      const int ii = d - AW;
      dma16(b_src[ii] + (int64_t)t * DBK * g.ldb, st + (uint32_t)(BMT * DBK * 2 + (wave * DI + ii) * 1024));
    }
  };

  // per-lane LDS read offsets (bytes within a stage)
  // a_rot depends on r mod 16 only, so the row blocks mi differ by a constant 2 KB
  int a_off[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int r = wm * WTM + (lane & 31);
    const int c = 2 * ks + (lane >> 5);
    a_off[ks] = r * 64 + (((c + a_rot(r)) & 3) * 16);
  }
  int b_off[NJ][2][2];
  {
    const int grp = lane >> 4, L = lane & 15;
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int krow = 16 * ks + 8 * (grp >> 1) + 4 * h + (L >> 2);
          const int ncol = wn * WTN + nj * 32 + (grp & 1) * 16 + 4 * (L & 3);
          const int c = ncol >> 3;
          b_off[nj][ks][h] = BMT * DBK * 2 + krow * 512 + ((c ^ b_swz(krow)) * 16) + (L & 1) * 8;
        }
  }

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Operand fragments of one 16-wide k-step: A rows (b128 reads) and B columns (two
  // transposing b64 reads each).  Two sets alternate so that the reads of the next k-step
  // are in flight while the 16 MFMAs of the current one run.
  struct Frag {
    f16x8 a[MI];
    s16x4 blo[NJ], bhi[NJ];
  };
  // LDS read r of a fragment set: r < MI the A rows of block r, else half (r - MI) & 1 of the
  // B columns of block (r - MI) / 2
  auto load_one = [&](const unsigned char* st, int ks, Frag& f, int r) {
    if (r < MI) {
      f.a[r] = *reinterpret_cast<const f16x8*>(st + a_off[ks] + r * 2048);
    } else {
      const int nj = (r - MI) >> 1, h = (r - MI) & 1;
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(st + b_off[nj][ks][h]));
      if (h == 0)
        f.blo[nj] = v;
      else
        f.bhi[nj] = v;
    }
  };
  auto load = [&](const unsigned char* st, int ks, Frag& f) {
#pragma unroll
    for (int r = 0; r < MI + 2 * NJ; ++r) load_one(st, ks, f, r);
  };
  auto mma_one = [&](const Frag& f, int j) {
    const int mi = j / NJ, nj = j % NJ;
    const f16x8 b = __builtin_bit_cast(f16x8, __builtin_shufflevector(f.blo[nj], f.bhi[nj], 0, 1, 2, 3, 4, 5, 6, 7));
    acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, f.a[mi], acc[mi][nj], 0, 0, 0);
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int j = 0; j < MI * NJ; ++j) mma_one(f, j);
  };
  // the MI + 2 * NJ LDS reads of the next fragments interleaved one-to-one with the first
  // of the MI * NJ MFMAs
  constexpr int RD = MI + 2 * NJ, MF = MI * NJ;
  constexpr int PAIRS = RD < MF ? RD : MF;
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < PAIRS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    }
    if constexpr (MF > RD) __builtin_amdgcn_sched_group_barrier(0x008, MF - RD, 0);
    if constexpr (RD > MF) __builtin_amdgcn_sched_group_barrier(0x100, RD - MF, 0);
  };

  // Pipeline: the DMA runs up to 3 K-tiles ahead into a ring of 4 stages.  Iteration t
  // reads k-step 1 of tile t while computing k-step 0, meets the other waves at a barrier
  // (after it tile t + 1 has landed and no wave reads tile t's stage any more, so the DMA of
  // tile t + 4 may overwrite it), then reads k-step 0 of tile t + 1 while computing k-step 1
  // of tile t, with this wave's DMA instructions for tile t + 4 issued one after every second
  // MFMA.  (Issued together right after the barrier, the eight waves' DMA instructions queue
  // for the vector memory path at once and every wave stalls there while the matrix cores
  // idle: ~20 % of each K-tile.)
  Frag f0, f1;
  constexpr int NDMA = AW + DI;  // DMA instructions per wave and K-tile, at most
  constexpr int STEPS = (MF > RD ? MF : RD) > 2 * NDMA ? (MF > RD ? MF : RD) : 2 * NDMA;
  auto iter = [&](int t, auto refill_c) {
    constexpr bool REFILL = decltype(refill_c)::value;
    load(dlds + (t % DSTAGES) * STAGE, 1, f1);
    mma(f0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (REFILL) {
      // tiles t + 2 and t + 3 may fly: 2 per_tile instructions, per_tile = na + DI
      if (na == AW)
        dma_sync_n<2 * (AW + DI)>();
      else
        dma_sync_n<2 * (AW - 1 + DI)>();
    } else {
      dma_sync(min(2, nk - 2 - t) * per_tile);  // tiles after t + 1 already issued may fly
    }
    const unsigned char* nst = dlds + ((t + 1) % DSTAGES) * STAGE;
#pragma unroll
    for (int j = 0; j < STEPS; ++j) {
      if (j < RD) load_one(nst, 0, f0, j);
      if (j < MF) mma_one(f1, j);
      if constexpr (REFILL)
        if ((j & 1) && (j >> 1) < NDMA) dma_one(t + DSTAGES, j >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const int pre = min(DSTAGES, nk);
  for (int t = 0; t < pre; ++t) issue(t);
  dma_sync((pre - 1) * per_tile);  // tile 0 landed; tiles 1 .. pre-1 may be in flight
  load(dlds, 0, f0);
  int t = 0;
  for (; t + DSTAGES < nk; ++t) iter(t, std::true_type{});
  for (; t + 1 < nk; ++t) iter(t, std::false_type{});
  load(dlds + ((nk - 1) % DSTAGES) * STAGE, 1, f1);
  mma(f0);
  interleave();
  __builtin_amdgcn_sched_barrier(0);
  mma(f1);

  // The MFMAs compute the transposed tile (A and B operands swapped): lane l holds C row
  // m = l mod 32 of each 32 x 32 block and, for each group q of four accumulators, the
  // four consecutive columns 8 q + 4 (l / 32) .. + 3 -- one 16-byte store instead of four.
  // N is a multiple of 8, so a group is either wholly inside N or wholly past it.
  float* out = g.ksplit == 1 ? g.C : g.ws + (int64_t)split * g.M * g.N;
  const int64_t ldo = g.ksplit == 1 ? g.ldc : g.N;
  const bool wide = g.ksplit > 1 || g.wide;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int row = m0 + wm * WTM + i * 32 + (lane & 31);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + wn * WTN + j * 32 + 8 * q + 4 * (lane >> 5);
        if (row < g.M && col < g.N) {
          float* dst = out + (int64_t)row * ldo + col;
          if (wide) {
            *reinterpret_cast<f32x4*>(dst) =
                f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[e] = acc[i][j][4 * q + e];
          }
        }
      }
    }
}

// C[m][n] = sum over s (in order) of ws[s][m][n], four consecutive elements of a row per
// thread (N is a multiple of 8); 16-byte stores when C allows them
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws,
                                                            float* __restrict__ C, int64_t ldc,
                                                            int M, int N, int S, int wide) {
  const int64_t MN = (int64_t)M * N, MN4 = MN / 4;
  for (int64_t e4 = (int64_t)blockIdx.x * 256 + threadIdx.x; e4 < MN4; e4 += (int64_t)gridDim.x * 256) {
    f32x4 v = reinterpret_cast<const f32x4*>(ws)[e4];
    for (int s = 1; s < S; ++s) v += reinterpret_cast<const f32x4*>(ws + s * MN)[e4];
    const int64_t e = 4 * e4, m = e / N, n = e - m * N;
    float* dst = C + m * ldc + n;
    if (wide) {
      *reinterpret_cast<f32x4*>(dst) = v;
    } else {
      dst[0] = v[0];
      dst[1] = v[1];
      dst[2] = v[2];
      dst[3] = v[3];
    }
  }
}

struct GemmPlan {
  int tilesM, tilesN, ksplit, kslice, bm;
};

GemmPlan plan_mfma(int64_t M, int64_t N, int64_t K, int bm) {
  GemmPlan p;
  p.bm = bm;
  p.tilesM = (int)((M + bm - 1) / bm);
  p.tilesN = (int)((N + BN - 1) / BN);
  const int tiles = p.tilesM * p.tilesN;
  const int kt = (int)((K + BK - 1) / BK);
  int s = 1;
  // when fewer than half the CUs would have a tile, split K into as many slices as fill the
  // CUs once, keeping >= 8 K-tiles per slice
  if (tiles * 2 <= 256) {
    s = 256 / tiles;
    while (s > 1 && kt / s < 8) --s;
  }
  p.ksplit = s;
  p.kslice = ((kt + s - 1) / s) * BK;
  p.ksplit = (int)((K + p.kslice - 1) / p.kslice);
  return p;
}

// The LDS-DMA kernel (K % 32 == 0) takes 256- or 320-row tiles, whichever gives the shorter
// critical path: rounds of workgroups over 256 CUs times the work of one (rows x K-slice).
// 1570-row prefills take 320 (5 row tiles instead of 7, 2 rounds instead of 3 for 22016
// columns); the register-staged kernel has 256-row tiles only.
GemmPlan choose_plan(int64_t M, int64_t N, int64_t K) {
  // up to 32 rows (with the LDS-DMA kernel): 32-row tiles, every wave 32 x 32, so the B
  // stream is not spread over mostly padding rows
  if (M <= 32 && K % DBK == 0) return plan_mfma(M, N, K, 32);
  const GemmPlan p256 = plan_mfma(M, N, K, 256);
  if (K % DBK != 0) return p256;
  const GemmPlan p320 = plan_mfma(M, N, K, 320);
  auto cost = [](const GemmPlan& p) {
    const int64_t wgs = (int64_t)p.tilesM * p.tilesN * p.ksplit;
    return ((wgs + 255) / 256) * (int64_t)p.bm * p.kslice;
  };
  return cost(p320) < cost(p256) ? p320 : p256;
}
__device__ __forceinline__ uint32_t half_of(uint4 v, int j) {
  const uint32_t d = dword_of(v, j >> 1);
  return (j & 1) ? (d >> 16) : (d & 0xFFFFu);
}

// -------------------------------------------------------------------- small-M path
// Each lane owns CPL contiguous columns (CPL = 8, 4 or 2: 16-, 8- or 4-byte loads of a B row),
// so a workgroup covers 64 CPL columns; the launcher picks CPL so that the workgroups spread
// evenly over the CUs (a head of 151936 columns in 512-column blocks leaves 41 CUs with twice
// the work of the others).
template <int CPL>
struct BRow;  // CPL f16 of one B row, loaded with one non-temporal load
template <>
struct BRow<8> {
  u32x4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
  __device__ __forceinline__ uint32_t dw(int i) const { return v[i]; }
};
template <>
struct BRow<4> {
  u32x2 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p)); }
  __device__ __forceinline__ uint32_t dw(int i) const { return v[i]; }
};
template <>
struct BRow<2> {
  uint32_t v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)); }
  __device__ __forceinline__ uint32_t dw(int) const { return v; }
};

template <int MT, int CPL>
__global__ __launch_bounds__(256) void gemm_smallm_kernel(const uint16_t* __restrict__ A,
                                                          int64_t lda,
                                                          const uint16_t* __restrict__ B,
                                                          int64_t ldb, float* __restrict__ C,
                                                          int64_t ldc, int M, int N, int K,
                                                          int KS) {
  constexpr int COLS = 64 * CPL;
  __shared__ float red[3][MT][COLS];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * COLS + lane * CPL;
  const int nn = min(n, N - CPL);  // clamp: columns past N are computed, never stored
  const int kb = wave * KS;
  const int ke = min(K, kb + KS);

  float acc[MT][CPL];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < CPL; ++j) acc[m][j] = 0.f;

  // Eight k-rows per step.  Byte permutes pair each column's values of rows k and k + 1
  // (one permute per two values), and v_dot2_f32_f16 multiplies such a pair with the pair
  // (A[m][k], A[m][k + 1]), wave-uniform: one instruction per two products and row of A.
  const uint16_t* bcol = B + nn;
  for (int k = kb; k < ke; k += 8) {
    BRow<CPL> h[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) h[kk].load(bcol + (int64_t)(k + kk) * ldb);
    uint32_t pr[4][CPL];  // pr[kp][j] = (B[k + 2 kp][j], B[k + 2 kp + 1][j])
#pragma unroll
    for (int kp = 0; kp < 4; ++kp)
#pragma unroll
      for (int j2 = 0; j2 < CPL / 2; ++j2) {
        const uint32_t lo = h[2 * kp].dw(j2), hi = h[2 * kp + 1].dw(j2);
        pr[kp][2 * j2] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        pr[kp][2 * j2 + 1] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
      }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int mm = m < M ? m : M - 1;
      const uint4 a8 = *reinterpret_cast<const uint4*>(A + (int64_t)mm * lda + k);
      const uint32_t ap[4] = {a8.x, a8.y, a8.z, a8.w};  // (A[m][k + 2 kp], A[m][k + 2 kp + 1])
#pragma unroll
      for (int kp = 0; kp < 4; ++kp)
#pragma unroll
        for (int j = 0; j < CPL; ++j)
          acc[m][j] = __builtin_amdgcn_fdot2(__builtin_bit_cast(hf16x2, pr[kp][j]),
                                             __builtin_bit_cast(hf16x2, ap[kp]), acc[m][j], false);
    }
  }

  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < CPL; ++j) red[wave - 1][m][lane * CPL + j] = acc[m][j];
  }
  __syncthreads();
  if (wave == 0 && n < N) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= M) break;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        float v = acc[m][j];
        v += red[0][m][lane * CPL + j];
        v += red[1][m][lane * CPL + j];
        v += red[2][m][lane * CPL + j];
        C[(int64_t)m * ldc + n + j] = v;
      }
    }
  }
}

template <int MT>
void launch_smallm(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C,
                   int64_t ldc, int M, int N, int K, hipStream_t st) {
  const int KS = ((K + 3) / 4 + 7) / 8 * 8;  // k-rows per wave, a multiple of 8
  // columns per lane: the largest whose busiest CU holds at most 10 % more workgroups than the
  // average (measured: the 151936-column head 111 -> 92 us at 2 columns per lane; a
  // 262144-column head is fastest at 8, two workgroups on every CU)
  int cpl = 2;
  for (int c : {8, 4}) {
    const double wgs = (double)((N + 64 * c - 1) / (64 * c));
    const double per_cu = wgs / 256.0;
    if (std::ceil(per_cu) <= 1.10 * per_cu) {
      cpl = c;
      break;
    }
  }
  const dim3 grid((unsigned)((N + 64 * cpl - 1) / (64 * cpl)));
  if (cpl == 8)
    hipLaunchKernelGGL((gemm_smallm_kernel<MT, 8>), grid, dim3(256), 0, st, A, lda, B, ldb, C, ldc, M, N, K, KS);
  else if (cpl == 4)
    hipLaunchKernelGGL((gemm_smallm_kernel<MT, 4>), grid, dim3(256), 0, st, A, lda, B, ldb, C, ldc, M, N, K, KS);
  else
    hipLaunchKernelGGL((gemm_smallm_kernel<MT, 2>), grid, dim3(256), 0, st, A, lda, B, ldb, C, ldc, M, N, K, KS);
}

// ------------------------------------------------------------------------ plain path
constexpr int PL_ROWS = 16;

__global__ __launch_bounds__(256) void gemm_plain_kernel(const uint16_t* __restrict__ A,
                                                         int64_t lda,
                                                         const uint16_t* __restrict__ B,
                                                         int64_t ldb, float* __restrict__ C,
                                                         int64_t ldc, int M, int N, int K) {
  __shared__ float red[4][PL_ROWS];
  const int n = blockIdx.x;
  const int m0 = blockIdx.y * PL_ROWS;
  const int rows = min(PL_ROWS, M - m0);
  float acc[PL_ROWS];
#pragma unroll
  for (int i = 0; i < PL_ROWS; ++i) acc[i] = 0.f;
  // PL_KU k-values per thread per round, every load unconditional (clamped row and k, the
  // clamped terms zeroed through b) so that a round's loads are all in flight together: a
  // column of B has one element per cache line, and loads behind a branch would wait in turn
  constexpr int PL_KU = 8;
  for (int k0 = threadIdx.x; k0 < K; k0 += 256 * PL_KU) {
    float b[PL_KU];
    uint16_t a[PL_KU][PL_ROWS];
#pragma unroll
    for (int u = 0; u < PL_KU; ++u) {
      const int k = min(k0 + u * 256, K - 1);
      b[u] = h2f(B[(int64_t)k * ldb + n]);
#pragma unroll
      for (int i = 0; i < PL_ROWS; ++i) a[u][i] = A[(int64_t)(m0 + min(i, rows - 1)) * lda + k];
    }
#pragma unroll
    for (int u = 0; u < PL_KU; ++u) {
      const float bu = k0 + u * 256 < K ? b[u] : 0.f;
#pragma unroll
      for (int i = 0; i < PL_ROWS; ++i) acc[i] = __builtin_fmaf(h2f(a[u][i]), bu, acc[i]);
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < PL_ROWS; ++i) {
    const float v = group_sum<64>(acc[i]);
    if (lane == 63) red[wave][i] = v;
  }
  __syncthreads();
  if (threadIdx.x < rows) {
    const int i = threadIdx.x;
    C[(int64_t)(m0 + i) * ldc + n] = ((red[0][i] + red[1][i]) + red[2][i]) + red[3][i];
  }
}

}  // namespace

size_t gemm_ws_bytes(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M,
                     int64_t N, int64_t K) {
  if (gemm_path(A, lda, B, ldb, M, N, K) != kGemmMfma) return 0;
  const GemmPlan p = choose_plan(M, N, K);
  return p.ksplit > 1 ? (size_t)p.ksplit * (size_t)M * (size_t)N * sizeof(float) : 0;
}

GemmPath gemm_path(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M,
                   int64_t N, int64_t K) {
  const bool vec = K % 8 == 0 && N % 8 == 0 && lda % 8 == 0 && ldb % 8 == 0 && aligned16(A) &&
                   aligned16(B);
  if (!vec) return kGemmPlain;
  // up to 8 rows the VALU kernel (dot2 over pairs of k) streams B faster than 32-row MFMA tiles
  // (measured at M = 8: 2048 x 151936 head 100 vs 114 us, 3840 x 262144 head 295 vs 346 us)
  if (M > 8) return kGemmMfma;
  return kGemmSmallM;
}

namespace {

void set_dma_lds_limits() {
  static std::once_flag lds_attr[kMaxDevices];
  once_per_device(lds_attr, [] {
    auto set = [](const void* f, size_t bytes) {
      (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    };
    set(reinterpret_cast<const void*>(gemm_mfma_kernel), kGemmLds);
    set(reinterpret_cast<const void*>(gemm_dma_kernel<kDmaWaves, 256, 2>), dma_lds(256));
    set(reinterpret_cast<const void*>(gemm_dma_kernel<kDmaWaves, 320, 2>), dma_lds(320));
    set(reinterpret_cast<const void*>(gemm_dma_kernel<kDmaWaves, 32, 1>), dma_lds(32));
    set(reinterpret_cast<const void*>(gemm_dma_kernel<kDmaWaves, 256, 2, true>), dma_lds(256));
    set(reinterpret_cast<const void*>(gemm_dma_kernel<kDmaWaves, 320, 2, true>), dma_lds(320));
  });
}

// The current device's compute units, queried once per device (256 on MI355X).
int device_cus() {
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
      (void)hipGetLastError();
      n = 256;
    }
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The MFMA path: the tile kernel (plus nside dequant workgroups after its own, SIDE), then the
// split-K reduce when K is split.
void launch_mfma(GemmArgs g, const GemmPlan& p, int nside, hipStream_t st) {
  set_dma_lds_limits();
  const dim3 grid((unsigned)(g.nwg + nside)), block(64 * kDmaWaves);
  const bool dma = g.K % DBK == 0;
  if (nside > 0 && p.bm == 320)
    hipLaunchKernelGGL((gemm_dma_kernel<kDmaWaves, 320, 2, true>), grid, block, dma_lds(320), st, g);
  else if (nside > 0)
    hipLaunchKernelGGL((gemm_dma_kernel<kDmaWaves, 256, 2, true>), grid, block, dma_lds(256), st, g);
  else if (dma && p.bm == 32)
    hipLaunchKernelGGL((gemm_dma_kernel<kDmaWaves, 32, 1>), grid, block, dma_lds(32), st, g);
  else if (dma && p.bm == 320)
    hipLaunchKernelGGL((gemm_dma_kernel<kDmaWaves, 320, 2>), grid, block, dma_lds(320), st, g);
  else if (dma)
    hipLaunchKernelGGL((gemm_dma_kernel<kDmaWaves, 256, 2>), grid, block, dma_lds(256), st, g);
  else
    hipLaunchKernelGGL(gemm_mfma_kernel, grid, dim3(256), kGemmLds, st, g);
  if (p.ksplit > 1) {
    const int64_t MN4 = (int64_t)g.M * g.N / 4;
    int64_t blocks = (MN4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                       reinterpret_cast<const float*>(g.ws), g.C, g.ldc, g.M, g.N, p.ksplit, g.wide);
  }
}

GemmArgs mfma_args(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C, int64_t ldc,
                   int M, int N, int K, void* ws, const GemmPlan& p) {
  GemmArgs g{};
  g.A = A;
  g.B = B;
  g.C = C;
  g.ws = reinterpret_cast<float*>(ws);
  g.lda = lda;
  g.ldb = ldb;
  g.ldc = ldc;
  g.M = M;
  g.N = N;
  g.K = K;
  g.tilesM = p.tilesM;
  g.tilesN = p.tilesN;
  g.ksplit = p.ksplit;
  g.kslice = p.kslice;
  g.wide = aligned16(C) && ldc % 4 == 0;
  g.nwg = p.tilesM * p.tilesN * p.ksplit;
  return g;
}

// Fewest CUs left idle by the last round of GEMM workgroups for a dequant to ride along, and
// the estimates that decide whether it finishes within that round: a side group takes about
// 4.5 us per dequant tile (measured beside a GEMM of K = 64: 18 tiles per group in 63-75 us),
// and a GEMM tile takes at least its MFMA work at about 5 TFLOP/s per CU (the 1570-token gate|up
// GEMM's second round: 320 x 256 x 2048 tiles in about 61 us).  Beside shorter tiles the dequant
// would run long on a few CUs after the GEMM (75 against 44 us as two launches at K = 64).
constexpr int kMinSide = 32;
constexpr double kSideTileNs = 4500.0;
constexpr double kCuFlopPerNs = 5000.0;

}  // namespace

int gemm_side_workgroups(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M,
                         int64_t N, int64_t K, int64_t Nq, int64_t Kq, int cus) {
  if (gemm_path(A, lda, B, ldb, M, N, K) != kGemmMfma || K % DBK != 0) return 0;
  const GemmPlan p = choose_plan(M, N, K);
  if (p.bm != 256 && p.bm != 320) return 0;
  // one GEMM workgroup per CU (the DMA ring holds 128 or 144 KB of LDS)
  const int nwg = p.tilesM * p.tilesN * p.ksplit;
  const int idle = (nwg + cus - 1) / cus * cus - nwg;
  if (idle < kMinSide) return 0;
  const int64_t tiles = (int64_t)dqt::row_blocks((int)Nq) * dqt::k_tiles((int)Kq);
  const int64_t iters = (tiles + 2 * idle - 1) / (2 * idle);  // tiles per side group
  const double tile_ns = 2.0 * p.bm * BN * p.kslice / kCuFlopPerNs;
  return (double)iters * kSideTileNs <= tile_ns ? idle : 0;
}

void launch_gemm(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C,
                 int64_t ldc, int M, int N, int K, void* ws, hipStream_t st) {
  switch (gemm_path(A, lda, B, ldb, M, N, K)) {
    case kGemmMfma: {
      const GemmPlan p = choose_plan(M, N, K);
      launch_mfma(mfma_args(A, lda, B, ldb, C, ldc, M, N, K, ws, p), p, 0, st);
      break;
    }
    case kGemmSmallM: {
      if (M <= 1)
        launch_smallm<1>(A, lda, B, ldb, C, ldc, M, N, K, st);
      else if (M <= 2)
        launch_smallm<2>(A, lda, B, ldb, C, ldc, M, N, K, st);
      else if (M <= 4)
        launch_smallm<4>(A, lda, B, ldb, C, ldc, M, N, K, st);
      else
        launch_smallm<8>(A, lda, B, ldb, C, ldc, M, N, K, st);
      break;
    }
    default: {
      const dim3 grid((unsigned)N, (unsigned)((M + PL_ROWS - 1) / PL_ROWS));
      hipLaunchKernelGGL(gemm_plain_kernel, grid, dim3(256), 0, st, A, lda, B, ldb, C, ldc, M, N, K);
    }
  }
}

}  // namespace w4

namespace w4 {

void launch_gemm_dequant(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C, int64_t ldc,
                         int M, int N, int K, void* ws, const uint32_t* qw, const uint16_t* s, const uint16_t* b,
                         uint16_t* wt, int64_t ldwt, int Nq, int Kq, bool sym, hipStream_t st) {
  const int nside = gemm_side_workgroups(A, lda, B, ldb, M, N, K, Nq, Kq, device_cus());
  if (nside == 0) {
    launch_gemm(A, lda, B, ldb, C, ldc, M, N, K, ws, st);
    if (sym)
      launch_dequant_t_sym128(qw, s, wt, ldwt, Nq, Kq, st);
    else
      launch_dequant_t(qw, s, b, wt, ldwt, Nq, Kq, st);
    return;
  }
  const GemmPlan p = choose_plan(M, N, K);
  GemmArgs g = mfma_args(A, lda, B, ldb, C, ldc, M, N, K, ws, p);
  g.dq_qw = qw;
  g.dq_s = s;
  g.dq_b = b;
  g.dq_wt = wt;
  g.dq_ld = ldwt;
  g.dq_N = Nq;
  g.dq_K = Kq;
  g.dq_vec = ldwt % 8 == 0 && aligned16(wt);  // 16-byte stores need 16-byte aligned rows
  g.dq_sym = sym;
  launch_mfma(g, p, nside, st);
}

}  // namespace w4
