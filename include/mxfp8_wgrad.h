/*
 * mxfp8_wgrad.h -- C ABI of the MI355X (gfx950) MXFP8 ragged weight-gradient
 * grouped GEMM.
 *
 * The operation (blog post "Ragged MXFP8 Weight Gradients: A FlyDSL Grouped
 * GEMM on MI355X", section 1): after expert-parallel dispatch the routed tokens
 * are sorted by expert, and offs[g] is where expert g's run of tokens ends.
 * For every expert g the weight gradient is
 *
 *     dW[g] = dY[g]^T * X[g]          (contraction over expert g's tokens)
 *
 * so the ragged axis is the contraction axis and the output [E, N, K] is
 * dense.  The operands are MXFP8 and quantised along tokens (same section):
 * FP8 E4M3 codes with one E8M0 scale per 32 tokens, passed as A = dY^T [N, M]
 * and B = X^T [K, M] with the token axis contiguous, plus row-major scale
 * planes [N, M/32] and [K, M/32].  Element by element:
 *
 *     dW[g][n][k] = sum_{m = start_g}^{end_g - 1}
 *                     e4m3(A[n][m]) 2^(sA[n][m/32] - 127) *
 *                     e4m3(B[k][m]) 2^(sB[k][m/32] - 127)
 *
 * with start_0 = 0, start_g = offs[g-1], end_g = offs[g] (the XLA blog
 * "Group-GEMM in XLA", section "Contracting": group start = exclusive prefix,
 * end = inclusive prefix).  E4M3 is the OCP E4M3FN flavour; E8M0 is 2^(s-127),
 * 0xFF = NaN.  Accumulation is FP32 on the block-scaled MFMA; the result is
 * rounded once to bfloat16, round-to-nearest-even (blog section 5.5).
 *
 * Every function is callable from C; no exception crosses the boundary.
 */
#ifndef MXFP8_WGRAD_H
#define MXFP8_WGRAD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MXW_OK 0
#define MXW_ERR_NULL (-1)   /* a required pointer is NULL */
#define MXW_ERR_DIM (-2)    /* a size outside the supported range */
#define MXW_ERR_ALIGN (-3)  /* A, B or out not 16-byte aligned */
#define MXW_ERR_DEVICE (-4) /* current device is not gfx950, or no device */
#define MXW_ERR_LAUNCH (-5) /* a kernel launch failed (hipGetLastError), or a
                               workspace could not be allocated */

/* Supported ranges (checked on the host, no device access). */
#define MXW_MAX_EXPERTS 256
#define MXW_MAX_TOKENS (8 * 1024 * 1024)
#define MXW_MAX_ROWS (8 * 1024 * 1024)

/*
 * mxfp8_wgrad_grouped -- the weight-gradient grouped GEMM above.
 *
 * Arguments (every pointer is caller-owned DEVICE memory on the current HIP
 * device):
 *   A     uint8  [N, M]    E4M3 codes of dY^T, row stride M bytes.
 *   sA    uint8  [N, M/32] E8M0 scales of A, row stride M/32 bytes.
 *   B     uint8  [K, M]    E4M3 codes of X^T, row stride M bytes.
 *   sB    uint8  [K, M/32] E8M0 scales of B, row stride M/32 bytes.
 *   offs  int32  [E]       cumulative end of each expert's token run.
 *   E     number of experts, 1 <= E <= MXW_MAX_EXPERTS.
 *   M     token-axis length of A and B (routed tokens plus any padding),
 *         0 <= M <= MXW_MAX_TOKENS, M % 32 == 0.
 *   N, K  output dimensions, each >= 16 and a multiple of 16.
 *   out   bf16 bit patterns [E, N, K], row-major (k contiguous).
 *   stream  a hipStream_t (NULL = the default stream), passed as void*.
 *
 * Host-checked preconditions (violations return an error code and launch
 * nothing): non-NULL pointers; A, B and out 16-byte aligned; the ranges above;
 * the current device is gfx950.
 *
 * Device-data preconditions (not checked on the host, which never reads
 * offs): offs non-decreasing, every offs[g] a multiple of 32, offs[E-1] <= M.
 * Tokens in [offs[E-1], M) belong to no expert and may hold anything (NaN
 * codes, 0xFF scales): they never reach the result.  Malformed offs give
 * unspecified values but no out-of-bounds access: windows are clamped to
 * [0, M] and every load is range-checked.
 *
 * Effects: enqueues the kernel (after the scale pre-shuffle below, when it
 * runs) on `stream` and returns without synchronising.  `out` is completely
 * overwritten; an expert with no tokens gets exact +0.0.
 * Inputs are never written.  The result is bitwise reproducible run to run:
 * for given (E, M, N, K, offs) every output element is summed in a fixed
 * order, whatever the timing (no atomics on data).
 *
 * Scheduling and state: with few output tiles per compute unit and long
 * experts (mxw_columns() > 0) the launch runs in column mode, one workgroup
 * per CU, and a region of tiles cut between columns is summed through FP32
 * partial tiles in a device workspace plus one arrival counter per region:
 * the last piece of a region to finish adds the others' partials, so no
 * workgroup ever waits for another and the kernel needs no co-residency.
 * The library allocates that workspace (128 MiB on a 256-CU device) with
 * hipMalloc on the first column-mode call on a device, synchronising the
 * device once, and keeps it until the process ends; every launch leaves the
 * counters at zero.
 *
 * Scale pre-shuffle: when the experts are long (M >= 4096 E) or the scale
 * rows are not 16-byte aligned (M % 512 != 0), the call first launches a
 * short kernel that rewrites sA and sB into a device workspace, each 256-row
 * band's 16-byte groups of 8 K-steps made contiguous (and the scales of
 * tokens past offs[E-1] cleared), so that the main kernel's scale loads read
 * consecutive bytes.  The workspace holds (ceil(N/256) + ceil(K/256)) *
 * ceil(M/512) * 4 KiB (21 MiB at the 16B shape with 196,608 tokens, 88 MiB
 * at 671B gate/up with 262,144); it is allocated with hipMalloc on the first
 * such call on a device and replaced by a buffer of the next power of two
 * when a later call needs more.  Replaced buffers are not freed (a HIP graph
 * captured earlier may still use them; what is kept stays below twice the
 * largest size), and all are kept until the process ends.
 *
 * Launches of mxfp8_wgrad_grouped or bf16_wgrad_grouped that use a workspace
 * (column mode, or the scale pre-shuffle) must not overlap in time on one
 * device: launches on different streams would race on it.  A call that uses
 * neither allocates nothing and keeps no state.  Capture into a HIP graph
 * after one eager call of the same or a larger shape (the capture must not
 * allocate).
 *
 * Returns MXW_OK or a negative MXW_ERR_* code.
 */
int mxfp8_wgrad_grouped(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                        const int32_t* offs, int E, int M, int N, int K, uint16_t* out, void* stream);

/*
 * bf16_wgrad_grouped -- the same weight gradient on plain bfloat16 operands:
 * the "contracting" ragged dot of the XLA blog ("Group-GEMM in XLA", Table 1,
 * and the bfloat16 wgrad_wi / wgrad_wo classes of its Table 7, which contract
 * the ragged token axis into one slab per expert).  For every expert g,
 * n < N, k < K:
 *
 *     out[g][n][k] = sum_{m = start_g}^{end_g - 1} bf16(A[n][m]) * bf16(B[k][m])
 *
 * accumulated in FP32 on the bf16 MFMA (every product is exact in FP32) and
 * rounded once to bf16, round-to-nearest-even.  Same windows as above.
 *
 * Arguments (caller-owned DEVICE memory on the current HIP device):
 *   A     bf16 bit patterns [N, M] (dY^T), token-contiguous, row stride M.
 *   B     bf16 bit patterns [K, M] (X^T), token-contiguous, row stride M.
 *   offs  int32 [E] cumulative ends.  E, N, K, out, stream: as above.
 *   M     0 <= M <= MXW_MAX_TOKENS / 2, M % 16 == 0.
 * The pages give the classes' dimension numbers, not a storage order; the
 * operands are taken with the contracted (token) axis innermost, as for the
 * MXFP8 path.  Device-data preconditions: offs non-decreasing, every offs[g]
 * a multiple of 16, offs[E-1] <= M (malformed offs: unspecified values, no
 * out-of-bounds access).  Tokens in [offs[E-1], M) may hold anything, NaN and
 * infinity included: they never reach the result.
 *
 * Effects, reproducibility, scheduling and workspace: as mxfp8_wgrad_grouped,
 * planned on the token axis in bytes: the launch runs in column mode exactly
 * when mxw_columns(E, 2 M, N, K) > 0, and shares the device's column-mode
 * workspace with mxfp8_wgrad_grouped (launches of either on one device must
 * not overlap in time when both run in column mode).
 *
 * Returns MXW_OK or a negative MXW_ERR_* code.
 */
int bf16_wgrad_grouped(const uint16_t* A, const uint16_t* B, const int32_t* offs, int E, int M, int N, int K,
                       uint16_t* out, void* stream);

/*
 * mxw_grid_size -- the number of (expert, 256 x 256 output tile) work items
 * of (E, N, K), E * ceil(N/256) * ceil(K/256) (blog section 4: one block per
 * expert per output tile).  Outside column mode this is also the number of
 * workgroups launched.  Returns 0 for invalid sizes.
 */
int64_t mxw_grid_size(int E, int N, int K);

/*
 * mxw_columns -- the number of columns mxfp8_wgrad_grouped uses for
 * (E, M, N, K) on the current device: 0 when it launches one workgroup per
 * work item, otherwise the column count of column mode (16 workgroups per
 * column, one per compute unit).  Column mode is chosen when the work items
 * fill the device at most 4 times over and M >= 8192 * E.  Reads device
 * properties only; returns MXW_ERR_DIM or MXW_ERR_DEVICE on invalid input or
 * no gfx950 device.
 */
int mxw_columns(int E, int M, int N, int K);

/*
 * mxw_scale_shuffle -- 1 if mxfp8_wgrad_grouped with (E, M) runs the scale
 * pre-shuffle kernel before the main kernel (M >= 4096 E or M % 512 != 0),
 * 0 if it launches the main kernel alone, MXW_ERR_DIM for invalid sizes.
 * Host-only: no device access.
 */
int mxw_scale_shuffle(int E, int M);

/*
 * mxfp8_grouped_fwd -- the row-ragged MXFP8 grouped GEMM: the forward and
 * data-gradient GEMMs of the same MoE layer.  (Blog section 1: the weight
 * gradient is one of three grouped GEMMs per expert layer; the other two keep
 * the contraction over the fixed hidden dimension and carry the raggedness
 * in their rows.  XLA blog: the "non-contracting" ragged dot and its forward
 * and data-gradient classes.)  For every expert g, every row m in
 * [start_g, end_g) (start_0 = 0, start_g = offs[g-1], end_g = offs[g]) and
 * every n < N:
 *
 *   out[m][n] = sum over c in [0, C) of
 *               e4m3(A[m][c]) 2^(sA[m][c/32] - 127) * e4m3(B[g][n][c]) 2^(sB[g][n][c/32] - 127)
 *
 * accumulated in FP32 and rounded to bf16 (round to nearest even).  Forward:
 * A = the routed tokens' activations (C = the layer's input width), B = the
 * expert weights.  Data gradient: A = the output gradient, B = the weights
 * quantized along their other axis.  MXFP8 puts its 32-element blocks along
 * the contraction axis, so both operands are stored with C innermost.
 *
 * Arguments (caller-owned DEVICE memory on the current HIP device):
 *   A     uint8  [R, C]       E4M3 codes, row stride C bytes.
 *   sA    uint8  [R, C/32]    E8M0 scales of A.
 *   B     uint8  [E, N, C]    E4M3 codes of each expert's [N, C] operand.
 *   sB    uint8  [E, N, C/32] E8M0 scales of B.
 *   offs  int32  [E]          cumulative end of each expert's run of rows.
 *   E     1 <= E <= MXW_MAX_EXPERTS.
 *   R     rows of A and out, 0 <= R <= MXW_MAX_ROWS.
 *   C     contraction length, 32 <= C <= 65536, C % 32 == 0.
 *   N     output columns, 16 <= N <= 65536, N % 16 == 0.
 *   out   bf16 bit patterns [R, N], row-major.
 *   stream  a hipStream_t (NULL = the default stream), passed as void*.
 *
 * Host-checked preconditions return an error code and launch nothing:
 * non-NULL pointers; A, B and out 16-byte aligned; the ranges above; a
 * gfx950 device.  Device-data preconditions (never read on the host): offs
 * non-decreasing and offs[E-1] <= R; row boundaries need no alignment.
 * Rows in [offs[E-1], R) belong to no expert: they are neither read as
 * values nor written.  Malformed offs give unspecified values but no
 * out-of-bounds access (windows are clamped to [0, R], loads range-checked,
 * stores confined to the clamped windows).
 *
 * Effects: enqueues one kernel on `stream`; allocates nothing, keeps no
 * state, never writes its inputs.  Each output element is one workgroup's
 * fixed-order sum: bitwise reproducible run to run.
 *
 * Returns MXW_OK or a negative MXW_ERR_* code.
 */
int mxfp8_grouped_fwd(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                      const int32_t* offs, int E, int R, int C, int N, uint16_t* out, void* stream);

/*
 * mxw_fwd_grid_size -- the workgroups mxfp8_grouped_fwd launches for
 * (E, R, N): (R / 256 + E) * ceil(N / 256) work items at most (each expert
 * adds at most one partial 256-row tile), rounded up to a multiple of 8.
 * Workgroups past the actual number of work items exit at once.  Returns 0
 * for invalid sizes.
 */
int64_t mxw_fwd_grid_size(int E, int R, int N);

/*
 * mxfp8_quantize_tokens -- the token-axis MXFP8 quantiser that produces the
 * weight gradient's operands (blog section 1: both operands are quantised
 * along the token axis and handed over token-contiguous, with one E8M0
 * scale per 32 tokens; the blog times its operator without this step,
 * section 7).  From bf16 x [M, H] (tokens x hidden, hidden contiguous) to
 * E4M3 codes q [H, M] and E8M0 scales s [H, M/32]; for every hidden column
 * h and 32-token block b:
 *
 *   amax    = max |x[m][h]| over the block's tokens below `used`
 *   s[h][b] = clamp(floor(log2 amax) - 8 + 127, 0, 254), 127 if amax == 0
 *   q[h][m] = E4M3FN(x[m][h] / 2^(s[h][b] - 127)): round to nearest, ties to
 *             the even code, saturated to +-448, zero encoded as +0; 0 for
 *             m >= used
 *
 * (8 = floor(log2 448), the largest E4M3 binade: the OCP MX shared scale.)
 * Call it on dY for A and on X for B.  `used` is offs[E-1] read on the
 * device (tokens past the last expert become finite zeros, whatever x holds
 * there), or M when offs is NULL.
 *
 * Arguments (caller-owned DEVICE memory on the current HIP device):
 *   x     uint16 [M, H]    bf16 bit patterns.
 *   offs  int32  [E]       cumulative expert ends (may be NULL: all tokens).
 *   E     1 <= E <= MXW_MAX_EXPERTS when offs is not NULL.
 *   M     0 <= M <= MXW_MAX_TOKENS, M % 32 == 0.
 *   H     16 <= H <= 65536, H % 16 == 0.
 *   q     uint8  [H, M]    codes, row stride M bytes.
 *   s     uint8  [H, M/32] scales, row stride M/32 bytes.
 *   stream  a hipStream_t, passed as void*.
 *
 * Host-checked preconditions return an error code and launch nothing:
 * non-NULL x, q, s; x and q 16-byte aligned; the ranges above; a gfx950
 * device.  Effects: one kernel on `stream`; allocates nothing; q and s are
 * fully overwritten; the result depends only on x and `used`.
 *
 * Returns MXW_OK or a negative MXW_ERR_* code.
 */
int mxfp8_quantize_tokens(const uint16_t* x, const int32_t* offs, int E, int M, int H, uint8_t* q, uint8_t* s,
                          void* stream);

/* mxw_strerror -- a static, human-readable message for a return code. */
const char* mxw_strerror(int code);

/* mxw_version -- library ABI version (major * 10000 + minor * 100 + patch). */
int mxw_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_WGRAD_H */
