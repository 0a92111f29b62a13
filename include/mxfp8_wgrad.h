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

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MXW_OK 0
#define MXW_ERR_NULL (-1)      /* a required pointer is NULL */
#define MXW_ERR_DIM (-2)       /* a size outside the supported range */
#define MXW_ERR_ALIGN (-3)     /* A, B or out not 16-byte aligned, or sA / sB
                                  not 4-byte aligned */
#define MXW_ERR_DEVICE (-4)    /* current device is not gfx950, or no device */
#define MXW_ERR_LAUNCH (-5)    /* a kernel launch failed (hipGetLastError) */
#define MXW_ERR_WORKSPACE (-6) /* workspace NULL, smaller than its size query,
                                  or not 256-byte aligned */
#define MXW_ERR_SCRATCH (-7)   /* the shape needs more workspace than
                                  MXW_SCRATCH_BYTES (no-allocation entry) */

/* Size of the static device scratch of mxfp8_wgrad_grouped_noalloc. */
#define MXW_SCRATCH_BYTES (160u * 1024u * 1024u)

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
 *   N, K  output dimensions, each >= 16 and a multiple of 16, <= 65536.
 *   out   bf16 bit patterns [E, N, K], row-major (k contiguous).
 *   stream  a hipStream_t (NULL = the default stream), passed as void*.
 *
 * Host-checked preconditions (violations return an error code and launch
 * nothing): non-NULL pointers; A, B and out 16-byte aligned, sA and sB
 * 4-byte aligned; the ranges above; the current device is gfx950.
 *
 * Device-data preconditions (not checked on the host, which never reads
 * offs): offs non-decreasing, every offs[g] a multiple of 32, offs[E-1] <= M.
 * Tokens in [offs[E-1], M) belong to no expert and may hold anything (NaN
 * codes, 0xFF scales): they never reach the result.  Malformed offs give
 * unspecified values but no out-of-bounds access: windows are clamped to
 * [0, M] and made monotone, every load is range-checked, and every store
 * lands inside out.
 *
 * Effects: enqueues one kernel on `stream` and returns without
 * synchronising.  It allocates nothing, keeps no state between calls, takes
 * no lock (the first call on a device reads its properties once, under a
 * host mutex) and never writes its inputs, so it may run concurrently on any
 * number of streams and be captured into a HIP graph at any time, the very
 * first call included.  `out` is completely overwritten; an expert with no
 * tokens gets exact +0.0.
 *
 * Scheduling and bits: one workgroup per (expert, 256 x 256 output tile)
 * (blog section 4), experts taken longest first (section 5.4), no atomics;
 * when N % 256 == 128 the last 384 rows of N are two tiles of 192 rows
 * instead of a whole one and one half past N (the same tile count); with
 * short experts and a partly filled last round, that round's tiles run
 * as two half-tile workgroups each (mxw_tail_split; such a launch keeps
 * whole 256-row tiles), computing every element exactly as the whole tile
 * does.
 * Each output element is one workgroup's sum over its expert's window in
 * token order, so the result depends only on that expert's window of A, sA,
 * B and sB: it is bitwise reproducible run to run, and unchanged by the
 * other experts' sizes, by the padding past offs[E-1] and by M.
 *
 * Returns MXW_OK or a negative MXW_ERR_* code.
 */
int mxfp8_wgrad_grouped(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                        const int32_t* offs, int E, int M, int N, int K, uint16_t* out, void* stream);

/*
 * mxfp8_wgrad_workspace_size -- bytes of device workspace that
 * mxfp8_wgrad_grouped_ws needs for (E, M, ld, N, K) on the current device (0
 * if it needs none), or a negative MXW_ERR_* code.  ld is the row stride
 * described there (0 = M).  Reads device properties only.  128 MiB of FP32
 * partial tiles on a 256-CU device when the launch runs in column mode
 * (mxw_columns() > 0), plus (ceil(N/256) + ceil(K/256)) * ceil(M/512) * 4 KiB
 * of shuffled scales when it pre-shuffles (M >= 4096 E):
 * 149 MiB at the 16B shape with 196,608 tokens, 88 MiB at 671B gate/up with
 * 262,144.
 */
int64_t mxfp8_wgrad_workspace_size(int E, int M, int ld, int N, int K);

/*
 * mxfp8_wgrad_grouped_ws -- the same weight gradient, given a caller-owned
 * device workspace, which lets the launch use two faster schedules where they
 * pay (the blog does not describe either):
 *  - column mode (few output tiles per compute unit, long experts): one
 *    workgroup per CU; 16 workgroups on one XCD form a column that streams
 *    regions of up to 16 tiles of one expert together through that XCD's L2.
 *    The K-step-weighted sequence of (expert, region) pieces is cut into one
 *    equal span per column, and a region cut between columns is summed in a
 *    fixed order through FP32 partial tiles in the workspace: the last of
 *    its pieces to finish (found with a device-scope counter) adds the
 *    others' partials.  No workgroup ever waits for another.
 *  - the scale pre-shuffle (M >= 4096 E): a short first
 *    kernel rewrites sA and sB into the workspace so that the main kernel's
 *    scale loads read consecutive bytes (the blog has a per-call pre-shuffle
 *    too, section 5.6).
 *
 * Arguments: as mxfp8_wgrad_grouped, plus
 *   ld               the row stride of A and B in bytes (tokens), M <= ld <=
 *                    MXW_MAX_TOKENS, ld % 32 == 0, or 0 for M; the scale
 *                    planes' rows are then ld / 32 bytes apart.  A is
 *                    [N, ld] storage holding the [N, M] matrix in its first M
 *                    columns (likewise sA, B, sB); columns [M, ld) are never
 *                    read.  Rows whose stride is a multiple of 64 KiB (the
 *                    16B shape's M = 3 * 2^16, the 671B shapes' 2^18) put the
 *                    lines a tile needs at once into few L2 sets; a stride
 *                    padded by an odd number of 128-token lines
 *                    (ld = M + 128) avoids that at long experts (16B shape,
 *                    196,608 tokens: 35% fewer HBM bytes, 3-4% faster;
 *                    671B: 13% fewer reads, 2-3% faster; within 2% of
 *                    contiguous rows at ~1,000 tokens per expert).
 *                    mxfp8_quantize_tokens writes such padded rows.
 *   workspace        caller-owned device memory, 256-byte aligned, of at
 *                    least mxfp8_wgrad_workspace_size(E, M, ld, N, K) bytes
 *                    (may be NULL when that size is 0).  Its contents are
 *                    undefined on entry and on exit: the call's first kernel
 *                    initialises what the others read.
 *   workspace_bytes  its size.
 *
 * Effects: enqueues one or two kernels on `stream`, returns without
 * synchronising, allocates nothing and keeps no state; graph-capturable at
 * any time.  The workspace is in use until the call's work on `stream` has
 * finished: calls that run concurrently (other streams, overlapping graph
 * replays) need workspaces of their own.  `out` is completely overwritten.
 *
 * Bits: bitwise reproducible run to run for the same (offs, M) on the same
 * device, but in column mode an output element is the sum of FP32 partials
 * whose cut points depend on the whole of offs, on M (through the mode
 * choice) and on the device's CU count: dW[g] may then differ, within the
 * tolerance of FP32 summation order, from mxfp8_wgrad_grouped's result and
 * from the result of a call whose other experts or padding differ.  Without
 * column mode the bits equal mxfp8_wgrad_grouped's.
 *
 * Returns MXW_OK or a negative MXW_ERR_* code (MXW_ERR_WORKSPACE for a
 * missing, short or misaligned workspace).
 */
int mxfp8_wgrad_grouped_ws(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                           const int32_t* offs, int E, int M, int ld, int N, int K, uint16_t* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * mxfp8_wgrad_grouped_noalloc -- for callers that cannot allocate device
 * memory (code under HIP-graph capture, tight serving loops, harnesses that
 * forbid allocation): mxfp8_wgrad_grouped_ws with its workspace taken from a
 * static device array of MXW_SCRATCH_BYTES (160 MiB) inside the library, which
 * every device the library runs on holds until the process ends.
 *
 * Arguments and results: as mxfp8_wgrad_grouped_ws (row stride ld included)
 * without the workspace arguments; the same plan, kernels and bits.  The
 * caller still passes the operands and out.  A shape whose workspace size
 * (mxfp8_wgrad_workspace_size) exceeds MXW_SCRATCH_BYTES returns
 * MXW_ERR_SCRATCH and launches nothing (the 16B shape with 196,608 tokens
 * needs 149 MiB, 671B gate/up with 262,144 tokens 88 MiB).  It calls no
 * allocating routine; the first call on a device looks up that device's
 * scratch address (hipGetSymbolAddress) once.
 *
 * Every call on a device shares that device's scratch: calls that overlap in
 * time on one device (other streams, overlapping graph replays) race on it
 * and give wrong results.  Each call initialises what it reads; the scratch
 * keeps the last call's contents.
 */
int mxfp8_wgrad_grouped_noalloc(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                                const int32_t* offs, int E, int M, int ld, int N, int K, uint16_t* out,
                                void* stream);

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
 * Effects, reproducibility and scheduling: as mxfp8_wgrad_grouped (one
 * kernel, allocates nothing, keeps no state; each output element one
 * workgroup's sum in token order).
 *
 * Returns MXW_OK or a negative MXW_ERR_* code.
 */
int bf16_wgrad_grouped(const uint16_t* A, const uint16_t* B, const int32_t* offs, int E, int M, int N, int K,
                       uint16_t* out, void* stream);

/*
 * bf16_wgrad_workspace_size -- bytes of device workspace bf16_wgrad_grouped_ws
 * needs for (E, M, N, K) on the current device (0 if none), or a negative
 * MXW_ERR_* code.  Planned on the token axis in bytes: column mode exactly
 * when mxw_columns(E, 2 M, N, K) > 0; there are no scales to shuffle.
 */
int64_t bf16_wgrad_workspace_size(int E, int M, int N, int K);

/*
 * bf16_wgrad_grouped_ws -- bf16_wgrad_grouped with a caller-owned workspace
 * for column mode, with the workspace contract, effects and bits of
 * mxfp8_wgrad_grouped_ws (a first one-workgroup kernel clears the counters).
 */
int bf16_wgrad_grouped_ws(const uint16_t* A, const uint16_t* B, const int32_t* offs, int E, int M, int N, int K,
                          uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mxw_grid_size -- the number of (expert, 256 x 256 output tile) work items
 * of (E, N, K), E * ceil(N/256) * ceil(K/256) (blog section 4: one block per
 * expert per output tile): the workgroups mxfp8_wgrad_grouped launches, and
 * mxfp8_wgrad_grouped_ws outside column mode.  Returns 0 for invalid sizes.
 */
int64_t mxw_grid_size(int E, int N, int K);

/*
 * mxw_columns -- the number of columns mxfp8_wgrad_grouped_ws uses for
 * (E, M, N, K) on the current device: 0 when it launches one workgroup per
 * work item, otherwise the column count of column mode (16 workgroups per
 * column, one per compute unit).  Column mode is chosen when the work items
 * fill the device at most 4 times over and M >= 8192 * E.  Reads device
 * properties only; returns MXW_ERR_DIM or MXW_ERR_DEVICE on invalid input or
 * no gfx950 device.
 */
int mxw_columns(int E, int M, int N, int K);

/*
 * mxw_tail_split -- how many output tiles mxfp8_wgrad_grouped runs as two
 * half tiles for (E, M, N, K) on the current device (0: none); the same
 * holds for mxfp8_wgrad_grouped_ws when it runs one workgroup per tile
 * without the scale pre-shuffle (mxw_columns() == 0, mxw_scale_shuffle() ==
 * 0), and for the bf16 entries with M tokens when they run one workgroup per
 * tile (mxw_columns(E, 2 M, N, K) == 0).  When the tiles fill the device only a few times over (more than once,
 * under 4 times) and experts are short (M <= 2048 E), the tiles of the last,
 * partly filled round (the last in longest-first order) each run as two
 * workgroups, one for the even and one for the odd 32-row blocks of the
 * tile's 256 rows of N, so that round has twice as many workgroups of a
 * little over half the length.  Each output element is computed exactly as
 * in the whole tile: the bits do not change.  Returns MXW_ERR_DIM or
 * MXW_ERR_DEVICE on invalid input or no gfx950 device.
 */
int mxw_tail_split(int E, int M, int N, int K);

/*
 * mxw_scale_shuffle -- 1 if mxfp8_wgrad_grouped_ws with (E, M) runs the scale
 * pre-shuffle kernel before the main kernel (M >= 4096 E),
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
 * non-NULL pointers; A, B and out 16-byte aligned, sA and sB 4-byte
 * aligned; the ranges above; a gfx950 device.  Device-data preconditions
 * (never read on the host): offs non-decreasing and offs[E-1] <= R; row boundaries need no alignment.
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
 *   ld    row stride of q in bytes (tokens), M <= ld <= MXW_MAX_TOKENS,
 *         ld % 32 == 0, or 0 for M; s's rows are ld / 32 bytes apart.  A
 *         padded stride (ld = M + 128) is the layout mxfp8_wgrad_grouped_ws
 *         reads best (see there); columns [M, ld) of q and [M/32, ld/32) of
 *         s are not written.
 *   H     16 <= H <= 65536, H % 16 == 0.
 *   q     uint8  [H, ld]   codes (the first M bytes of each row).
 *   s     uint8  [H, ld/32] scales (the first M/32 bytes of each row); any
 *         alignment, but with s 8-byte aligned and ld % 256 == 0 every
 *         whole 256-token tile's scale bytes go out as one 8-byte store
 *         per row, and with s 4-byte aligned and ld % 128 == 0 as two
 *         4-byte stores (either way faster than byte stores).
 *   stream  a hipStream_t, passed as void*.
 *
 * Host-checked preconditions return an error code and launch nothing:
 * non-NULL x, q, s; x and q 16-byte aligned; the ranges above; a gfx950
 * device.  Effects: one kernel on `stream`; allocates nothing; the [H, M]
 * codes and [H, M/32] scales are fully overwritten; the result depends only
 * on x and `used`.
 *
 * Returns MXW_OK or a negative MXW_ERR_* code.
 */
int mxfp8_quantize_tokens(const uint16_t* x, const int32_t* offs, int E, int M, int ld, int H, uint8_t* q,
                          uint8_t* s, void* stream);

/* mxw_strerror -- a static, human-readable message for a return code. */
const char* mxw_strerror(int code);

/* mxw_version -- library ABI version (major * 10000 + minor * 100 + patch). */
int mxw_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_WGRAD_H */
