/*
 * w4.h -- C ABI of the MI355X (gfx950) group-wise affine int4 weight-only linear layer.
 *
 * The operations are those of a local LLM engine's int4 linear layer as described on
 * "The inference engine -- Mojo 1.0 on Metal" (millfolio), section "Crossing Mojo 1.0":
 * a multi-row decode GEMV that streams the packed weights, a prefill that dequantizes
 * every weight once into a transposed half-precision scratch and then runs an f16 GEMM,
 * and on-device argmax/top-k over the logits.  The weight format is MLX's affine 4-bit
 * format (same page, "Appendix: the remaining gap, itemized") with group size 64
 * ("Engineering investigation: can this MLX port become another 10x faster?",
 * section "Selective quantization").
 *
 * Weight format (fixed):
 *   codes    q[n][k] in 0..15, n < N output features, k < K input features, K % 64 == 0;
 *   packed   qw[n][j], uint32, row-major [N][K/8]; code q[n][8j+i] in bits 4i..4i+3
 *            (low nibble first, little-endian words);
 *   scales   s[n][g], biases b[n][g], f16 bit patterns, row-major [N][K/64], g = k / 64;
 *   weight   w[n][k] = s[n][g] * q[n][k] + b[n][g].
 *
 * Conventions for every function:
 *   - f16 values travel as uint16_t bit patterns; f32 as float.
 *   - Every pointer is a DEVICE pointer owned by the caller.  The library never allocates,
 *     frees or retains device memory and keeps no per-call state; inputs are read-only;
 *     outputs are fully overwritten (no accumulation) and must not alias inputs.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the default stream) and the call
 *     returns without waiting for it.
 *   - Every argument check runs on the host before anything is launched; on a non-zero
 *     return nothing was launched and no output was touched.  Faults inside a kernel
 *     surface as a HIP error at the caller's next synchronisation.
 *   - Functions with a workspace use a two-phase protocol: with ws == NULL the required
 *     byte count is written to *ws_bytes and W4_OK is returned without launching;
 *     otherwise *ws_bytes is the capacity of ws (16-byte aligned) and too little returns
 *     W4_ERR_WORKSPACE.  A required size of 0 means ws may be NULL-or-anything once queried.
 *   - Alignment: the base pointers named below must be 16-byte aligned and the leading
 *     dimensions of f16 operands multiples of 8 elements, else W4_ERR_ALIGN.
 *   - The functions are reentrant; calls on different streams may run concurrently.
 *   - No C++ exception crosses the ABI (an internal failure returns W4_ERR_INTERNAL).
 *   - Only gfx950 devices are accepted (W4_ERR_DEVICE otherwise, or with no device).
 */
#ifndef W4_H
#define W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* w4_stream_t; /* == hipStream_t */

enum {
  W4_OK = 0,
  W4_ERR_NULL = -1,      /* a required pointer is NULL */
  W4_ERR_SHAPE = -2,     /* a size is out of the supported range */
  W4_ERR_ALIGN = -3,     /* a pointer or leading dimension is misaligned */
  W4_ERR_WORKSPACE = -4, /* the workspace is too small */
  W4_ERR_DEVICE = -5,    /* no usable gfx950 device is current */
  W4_ERR_LAUNCH = -6,    /* the HIP runtime rejected a launch */
  W4_ERR_INTERNAL = -7,  /* unexpected internal failure */
  W4_ERR_OVERLAP = -8    /* gemm_f16_dequant_next: one operation's output overlaps the other's data */
};

/* Static string describing a status code (never NULL). */
const char* w4_strerror(int status);

/*
 * w4_pack -- pack 4-bit codes into the weight format ("quantized to int4 at load":
 * "The inference engine -- Mojo 1.0 on Metal", "Where it fits").
 *   q   uint8 [N][K], row-major, values 0..15 (only the low 4 bits of each byte are kept);
 *   qw  uint32 [N][K/8] output.
 * Requires N >= 1, K >= 64, K % 64 == 0; q and qw 16-byte aligned.  Bit-exact.
 */
int w4_pack(const uint8_t* q, uint32_t* qw, int64_t N, int64_t K, w4_stream_t stream);

/*
 * w4_quantize -- the load-time step that produces the format ("The inference engine -- Mojo
 * 1.0 on Metal", "Where it fits": weights quantized to int4 at load; "Engineering
 * investigation ...", "Selective quantization": affine, group size 64).  The pages give no
 * fitting rule; per (row n, group g of 64) this is the min/max fit:
 *   lo, hi = min, max of w[n][64g .. 64g+63] (a zero counts as +0);  biases[n][g] = lo;
 *   scales[n][g] = RN16(f32(f32(hi - lo) / 15));
 *   q = clamp(rint_even(f32(f32(w - lo) / s)), 0, 15), or 0 for the group when s == 0,
 * with every operation a correctly rounded f32 operation; q is packed as by w4_pack.
 *   w f16 [N][K] with row stride ldw; qw [N][K/8]; scales, biases f16 [N][K/64].
 * Requires N >= 1, K >= 64, K % 64 == 0, ldw >= K, ldw % 8 == 0; w and qw 16-byte aligned,
 * scales and biases 2-byte aligned.  w must be finite (not checked).  Deterministic.
 */
int w4_quantize(const uint16_t* w, int64_t ldw, uint32_t* qw, uint16_t* scales, uint16_t* biases,
                int64_t N, int64_t K, w4_stream_t stream);

/*
 * w4_gemv -- decode GEMV over the packed weights ("Crossing Mojo 1.0": the multi-row
 * GEMV that keeps several weight streams in flight; "What's inside the engine today"):
 *   y[m][n] = sum_k (s[n][k/64] * q[n][k] + b[n][k/64]) * x[m][k]      (f32 accumulation)
 *   qw [N][K/8], scales/biases [N][K/64] (f16 bits), x f16 [M][K] with row stride ldx,
 *   y  f32 [M][N] with row stride ldy.
 * Requires 1 <= M <= 16, N >= 1, K >= 64, K % 64 == 0, ldx >= K, ldy >= N, ldx % 8 == 0;
 * qw, scales, biases, x 16-byte aligned; y 4-byte aligned.  The result is deterministic;
 * per output it is within 2e-3 * sum_k |w[n][k] x[m][k]| of the exact sum.
 * Workspace (query it: ws = NULL and ws_bytes set returns the size): 0 for most shapes, when
 * ws/ws_bytes may be NULL; on the matrix-core path (5 <= M, or M = 3..4 with K > 16384) rows
 * of K >= 6144 elements that would give at most 128 workgroups (N <= 2048 rows, e.g. the
 * 2048 x 6144 and 2048 x 11008 down projections) split K two ways across workgroups and need
 * 2 * M * N * 4 bytes for the partial sums, 16-byte aligned.  Contents need no initialisation.
 */
int w4_gemv(const uint32_t* qw, const uint16_t* scales, const uint16_t* biases,
            const uint16_t* x, int64_t ldx, float* y, int64_t ldy,
            int64_t M, int64_t N, int64_t K, void* ws, size_t* ws_bytes, w4_stream_t stream);

/*
 * w4_dequant_f16_t -- the prefill's "transposed half-precision scratch" ("Crossing Mojo
 * 1.0": each weight dequantized once per prefill):
 *   wt[k][n] = RN16(s[n][k/64] * q[n][k] + b[n][k/64])
 * with one round-to-nearest-even step from the exact value (subnormals kept).
 *   wt f16 [K][N] with row stride ldwt (N contiguous).
 * Requires N >= 1, K >= 64, K % 64 == 0, ldwt >= N; qw, scales, biases 16-byte aligned,
 * wt 2-byte aligned (16-byte aligned with ldwt % 8 == 0 for full-speed stores).  Bit-exact.
 */
int w4_dequant_f16_t(const uint32_t* qw, const uint16_t* scales, const uint16_t* biases,
                     uint16_t* wt, int64_t ldwt, int64_t N, int64_t K, w4_stream_t stream);

/*
 * The engine's own symmetric group-128 int4 ("The inference engine -- Mojo 1.0 on Metal":
 * group-128 int4 in "Against MLX, today" and "What's inside the engine today", symmetric in
 * "Appendix: the remaining gap, itemized"), read as
 *   w[n][k] = s[n][k/128] * (q[n][k] - 8)      (zero point 8, no bias),
 * with the same packed codes as above and scales f16 [N][K/128].  These two calls are
 * w4_gemv and w4_dequant_f16_t for that format: same arguments without the biases (the GEMV
 * takes w4_gemv's workspace, of the same size for the same M, N, K), same requirements plus
 * K % 128 == 0; the dequant rounds s (q - 8) once (an exact zero is +0) and is bit-exact;
 * the GEMV meets the same per-output bound.
 */
int w4_gemv_sym128(const uint32_t* qw, const uint16_t* scales, const uint16_t* x, int64_t ldx,
                   float* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* ws, size_t* ws_bytes,
                   w4_stream_t stream);
int w4_dequant_f16_t_sym128(const uint32_t* qw, const uint16_t* scales, uint16_t* wt, int64_t ldwt,
                            int64_t N, int64_t K, w4_stream_t stream);

/*
 * gemm_f16 -- C = A * B with f16 inputs and f32 accumulation and output: the prefill GEMM
 * on the f16 scratch ("Crossing Mojo 1.0") and the f16 LM head ("What's inside the engine
 * today": the head streamed as a [hidden x vocab] matrix per token).
 *   A f16 [M][K] (row stride lda), B f16 [K][N] (row stride ldb, N contiguous),
 *   C f32 [M][N] (row stride ldc).
 * Requires M, N, K >= 1, lda >= K, ldb >= N, ldc >= N; A, B 2-byte aligned, C 4-byte
 * aligned.  M >= 9 uses matrix cores (needs K % 8 == 0, N % 8 == 0, lda and ldb multiples
 * of 8, A and B 16-byte aligned; M <= 32 in 32-row tiles that stream B once); M <= 8 with
 * the same layout streams B once on the vector ALUs;
 * any other shape or alignment (e.g. one column of a head, B = H + id, ldb = V) takes a
 * plain path.  Per output within 2e-3 * sum_k |A[m][k] B[k][n]| of the exact sum; the result
 * is deterministic.  Workspace: shapes whose output tiles would leave most of the 256 CUs
 * idle split K and need ksplit * M * N * 4 bytes for the partial tiles (query it); 0 otherwise.
 */
int gemm_f16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C, int64_t ldc,
             int64_t M, int64_t N, int64_t K, void* ws, size_t* ws_bytes, w4_stream_t stream);

/*
 * gemm_f16_dequant_next -- one step of the prefill ("Crossing Mojo 1.0": every weight is
 * dequantized once per prefill into the transposed f16 scratch, then the f16 GEMM runs on it):
 * the GEMM of one weight together with the dequant of the next weight, which does not depend
 * on it.  Results are exactly those of
 *   gemm_f16(A, lda, B, ldb, C, ldc, M, N, K, ws, ws_bytes, stream) and
 *   w4_dequant_f16_t(qw, scales, biases, wt, ldwt, Nq, Kq, stream)
 * (C and wt bit for bit), with the same arguments, requirements, workspace (the GEMM's, same
 * size query) and errors as those two calls.  When the GEMM's last round of workgroups leaves
 * at least 32 CUs idle (e.g. 430 tiles of 320 x 256 on 256 CUs for a 1570-token gate|up
 * projection) and the dequant is estimated to finish within that round, it runs in those CUs
 * in the same launch; otherwise the two are launched one after the other on `stream`.  The two run concurrently, so wt must not overlap
 * A, B, C, the workspace or the dequant's own inputs, and C and the workspace must not overlap
 * qw, scales or biases: W4_ERR_OVERLAP otherwise (checked on the host).  Deterministic.
 */
int gemm_f16_dequant_next(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C,
                          int64_t ldc, int64_t M, int64_t N, int64_t K, void* ws, size_t* ws_bytes,
                          const uint32_t* qw, const uint16_t* scales, const uint16_t* biases,
                          uint16_t* wt, int64_t ldwt, int64_t Nq, int64_t Kq, w4_stream_t stream);

/*
 * gemm_f16_dequant_next_sym128 -- the same for a next weight in the symmetric group-128 format
 * (see w4_gemv_sym128): gemm_f16 and w4_dequant_f16_t_sym128 in one call, with their arguments,
 * requirements (Kq % 128 == 0), workspace and errors, and the same overlap rule (scales
 * f16 [Nq][Kq/128]).  C and wt are bit-identical to the two separate calls.
 */
int gemm_f16_dequant_next_sym128(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                 float* C, int64_t ldc, int64_t M, int64_t N, int64_t K, void* ws,
                                 size_t* ws_bytes, const uint32_t* qw, const uint16_t* scales,
                                 uint16_t* wt, int64_t ldwt, int64_t Nq, int64_t Kq,
                                 w4_stream_t stream);

/*
 * logits_argmax_topk -- on-device token selection ("Crossing Mojo 1.0": argmax/top-k on
 * the GPU instead of downloading the logits; "What's inside the engine today": bit-exact
 * against the host reference; "engine-mlx", "Tech details": in-graph greedy argmax).
 *   logits f32 [M][V] (row stride ldl); idx int32 [M][k] and val f32 [M][k] outputs.
 * Per row: the k largest logits ordered by value descending, ties to the lower index,
 * -0.0 equal to +0.0; idx[m][0] is the argmax; val[m][r] == logits[m][idx[m][r]] bit for bit.
 * Requires 1 <= M, 1 <= k <= min(V, 256), V < 2^31, ldl >= V, ceil(V / 8192) * k <= 8192;
 * logits 4-byte aligned, idx/val 4-byte aligned.  Logits must be finite (unchecked).
 * Workspace (query it; 0 when V <= 4096): k <= 64: one 8-byte key per 64 logits,
 * M * ceil(V / 64) * 8 bytes (19 KB for one 151936-logit row); k > 64: M * ceil(V / chunk) * k * 8
 * bytes with chunk = 4096 or 8192 logits.  Contents need no initialisation.
 */
int logits_argmax_topk(const float* logits, int64_t ldl, int64_t M, int64_t V, int64_t k,
                       int32_t* idx, float* val, void* ws, size_t* ws_bytes, w4_stream_t stream);

/*
 * w4_gemv_topk -- the int4 LM head at decode with token selection on the device, in one call
 * ("The inference engine -- Mojo 1.0 on Metal", "What's inside the engine today": the LM head
 * stored in int4 and token selection on the GPU, bit-exact against the host; "Crossing Mojo
 * 1.0": the logits stay on the device):
 *   logits[v] = sum_k (s[v][k/64] * q[v][k] + b[v][k/64]) * x[k]      (one activation row)
 *   idx[0..k), val[0..k): the k largest logits, value descending, ties to the lower index,
 *   -0.0 equal to +0.0; val[r] == logits[idx[r]] bit for bit; idx[0] is the argmax.
 *   qw [V][K/8], scales/biases [V][K/64] (the weight format above, V vocabulary rows), x f16 [K],
 *   logits f32 [V] (written in full), idx int32 [k], val f32 [k].
 * Each logit is within 2e-3 * sum_k |w[v][k] x[k]| of the exact sum, and bit-identical to
 * w4_gemv's at M = 1; the selection is exact on the logits it writes and equals
 * logits_argmax_topk's on them.  Launches: the M = 1 GEMV, then logits_argmax_topk's passes
 * (for V > 4096 the largest key of every 64 logits, then one workgroup that selects from the
 * groups whose keys can hold the top k and re-reads only those).
 * Requires 1 <= k <= 64, k <= V <= 524288, 64 <= K <= 4096, K % 64 == 0; qw, scales, biases, x
 * 16-byte aligned; logits, idx, val 4-byte aligned.  Workspace: 8 bytes per 64 logits for
 * V > 4096, none up to 4096 (query it; 18.5 KiB for 151936 rows); nothing in it has to be
 * initialised.  Deterministic.
 */
int w4_gemv_topk(const uint32_t* qw, const uint16_t* scales, const uint16_t* biases, const uint16_t* x,
                 int64_t V, int64_t K, int64_t k, float* logits, int32_t* idx, float* val, void* ws,
                 size_t* ws_bytes, w4_stream_t stream);

/*
 * logits_argmax_topk_noalloc -- logits_argmax_topk for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, requirements, results and errors as logits_argmax_topk, minus
 * the workspace: what logits_argmax_topk would keep there (the size it would ask for) goes
 * to a 4 MiB array that the library holds on each device
 * until the process ends.  Needing more than 4 MiB returns W4_ERR_WORKSPACE without launching
 * (e.g. top-64 of 262144 logits needs 32 KiB per row, so up to 128 such rows per call).  The
 * call allocates nothing.  Calls that overlap on one device (concurrent streams, or host
 * threads) share that array and race: serialise them.  Nothing in the array has to start at
 * zero; every call overwrites what it reads.
 */
int logits_argmax_topk_noalloc(const float* logits, int64_t ldl, int64_t M, int64_t V, int64_t k,
                               int32_t* idx, float* val, w4_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W4_H */
