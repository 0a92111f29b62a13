// mxfp8_wgrad.hip -- MXFP8 ragged weight-gradient grouped GEMM for MI355X
// (gfx950), and its C ABI (declared in include/mxfp8_wgrad.h).
//
// dW[g][n][k] = sum over expert g's tokens m of
//               e4m3(A[n][m]) 2^(sA[n][m/32]-127) * e4m3(B[k][m]) 2^(sB[k][m/32]-127)
// (blog "Ragged MXFP8 Weight Gradients: A FlyDSL Grouped GEMM on MI355X",
// section 1).  A = dY^T [N, M], B = X^T [K, M], token axis contiguous.
//
// The same tile body also serves the row-ragged GEMM of the layer (forward
// and data gradient: out[m] = A[m] B[g]^T over the rows m of expert g,
// rows_kernel), and the file holds the token-axis quantiser that produces
// the weight gradient's operands (quant_kernel); both are described where
// they are defined.
//
// Structure of one weight-gradient launch:
//   * work item = (expert, 256 x 256 output tile), computed by one 256-thread
//     workgroup (4 wave64) that walks the expert's tokens in 64-token K-steps,
//     keeps the tile's 65,536 FP32 sums in accumulator registers and stores
//     once (blog section 4).  No atomics on data: bit-reproducible.
//   * tile scheduler, two modes:
//     - one workgroup per work item (many tiles): every workgroup reads offs
//       itself, ranks the experts by window length with one lane per expert
//       (longest first, ties to the lower index; blog section 5.4), and
//       numbers tiles so that the workgroups the dispatcher deals to one XCD
//       (block index mod 8, blog section 3) cover a compact rectangle of the
//       same expert's tiles (blog section 5.5); with short experts and a
//       partly filled last round, that round's tiles run as two half-tile
//       workgroups each (the even and the odd 32-row blocks, same bits);
//     - column mode (few tiles per CU, long experts): one workgroup per CU;
//       16 workgroups on one XCD form a column that works through regions of
//       up to 16 tiles (4 x 4) of one expert, all members on the same tokens
//       at the same time so that they share the region's A and B stripes in
//       the XCD's L2.  The sequence of (expert, region) pieces, weighted by
//       K-steps, is cut into equal spans, one per column (whole tiles pack
//       unevenly: 1.3x the ideal span at 1.5 tiles per CU).  A region cut
//       between columns is summed in a fixed order: its pieces count
//       themselves in on a counter and the last to finish adds the others'
//       FP32 partial tiles (no workgroup waits for another).  The tiles of a
//       column that share a stripe split an L2 prefetch of it between them,
//       one pair ahead of their loads.
//     In both modes, when N % 256 == 128 the last 384 rows of N are two short
//     tiles of 192 rows (three 32-row blocks per wave) rather than a whole
//     tile and one with half its rows past N.
//   * staging: an LDS stage holds a pair of K-steps (256 rows x 128 tokens of
//     A and of B, 64 KiB), filled by 16-byte LDS-direct buffer loads, 8 rows x
//     128 bytes per instruction, so every memory request is one whole cache
//     line (half-line requests halve the miss bandwidth, measured); two stages
//     ping-pong (blog section 4).  The 16-byte chunk c of row r sits at
//     position c ^ ((r / 2) % 8): the MFMA fragment reads, served 16 lanes
//     (256 bytes of banks) at a time, are free of LDS bank conflicts.
//   * software pipeline: the fragments of K-step j + 1 are read from LDS into
//     a second register set while K-step j's 16 MFMAs run, one read per MFMA,
//     so the MFMAs never wait on LDS and the LDS stays evenly loaded.  One
//     barrier per pair of K-steps, at the odd step: it certifies that the
//     next pair has landed and that the current pair has been read, and that
//     pair's stage is then refilled with the pair after next, its loads
//     spread over the MFMAs of this odd step and the first ones of the next
//     even step (a CU's vector memory path takes a 1 KiB load per ~16
//     clocks: issued all at once they would hold up the MFMAs).
//   * ragged head/tail: a 32-token sub-block is live iff it lies inside
//     [start, end) (group boundaries are 32-aligned, blog section 1).  Dead
//     sub-blocks are removed twice: their data loads are pointed out of the
//     buffer range, so the hardware writes zeros (padding that holds NaN never
//     reaches the MFMA, blog section 5.3), and both operands' scales are set
//     to 0x00.
//   * scales: the raw E8M0 bytes arrive by LDS-direct loads; once per pair of
//     K-steps each lane reads, for each of its 32-row blocks, the dword of
//     its row that holds the pair's 4 bytes (2 K-steps x 2 sub-blocks), shifts
//     its own sub-block's bytes to bytes 0 and 2, clears dead sub-blocks, and
//     the MFMA picks byte 0 or 2 with op_sel (blog sections 5.2 and 5.6): no
//     unpacking and no relayout through LDS.  One 16-byte load per row brings
//     8 K-steps of scales (GROUP = true).  In the caller's planes those 16
//     bytes of 256 rows lie in 256 cache lines, and at long experts that
//     costs the weight gradient ~6%; it then first rewrites the planes so that
//     a band's groups are contiguous (scale_shuffle_kernel).  Scale rows that
//     are not a whole number of dwords (M % 128 != 0) are read a dword early
//     and each word is joined from two.  The row-ragged GEMM reads its planes
//     directly: a tile's whole scale blocks
//     once, in the prologue, when C <= 1,504, otherwise 16-byte groups
//     (C % 128 == 0) or the two aligned dwords around a row's 4 bytes of 2
//     K-steps.  A scale load per row per
//     step would double the number of L1 -> L2 requests of a step (every lane
//     hits a different row), which measurably slows the data stream.
//   * contraction: v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x E4M3 with
//     per-32 E8M0 scales, FP32 accumulation (blog section 3).  Operand roles
//     are swapped (B feeds the instruction's first operand) so that each lane
//     ends with 4 consecutive k of one output row (ROCm/aiter PR 6605,
//     section 1).
//   * epilogue: FP32 -> bf16 round-to-nearest-even in registers (blog
//     section 5.5), staged through LDS so that every global store writes
//     whole 128-byte lines (8-byte stores straight from the MFMA layout touch
//     32 lines per instruction and took ~19k clocks per tile); the stores are
//     non-temporal, so the output streams past the L2.
//
// MFMA lane layout used here (32x32x64, FP8 operands, checked on gfx950): lane
// l holds row l % 32 and tokens {16(l/32) + p : p < 16} in bytes 0..15 and
// {32 + 16(l/32) + p} in bytes 16..31; the scale word of lane l carries the
// E8M0 of row l % 32 and 32-token block l / 32 (byte picked by op_sel); the
// result's lane l register r holds row 8(r/4) + 4(l/32) + r%4 of column l % 32.
//
// Every global read in the K-loop is an LDS-direct load issued through asm,
// and the kernel waits on vmcnt itself: the compiler's wait insertion cannot
// tell the stages apart and would drain the prefetch before each LDS read.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "mxfp8_wgrad.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kTile = 256;                   // output tile edge, N and K
// short tiles: when N % 256 == 128 the last 384 rows of N are cut into two
// tiles of 192 rows (96 per wave) instead of a whole and a half-empty one
constexpr int kShort = 192;
constexpr int kStep = 64;                    // tokens per K-step (two 32-token sub-blocks)
constexpr int kPair = 2 * kStep;             // tokens per LDS stage (two K-steps)
constexpr int kThreads = 256;                // 4 wave64
constexpr int kRowBytes = kPair;             // one staged row = 128 E4M3 codes (one cache line)
constexpr int kOpBytes = kTile * kRowBytes;  // 32 KiB per operand per stage
constexpr uint32_t kOob = 0x80000000u;       // a buffer offset past any range used here
// DMA instructions per wave per pair of K-steps for operand data: 8 row groups
// (8 rows x 128 B = 1 KiB each) of A and 8 of B.
constexpr int kDataDma = 16;
// column mode: L2 prefetch loads per wave per even K-step
constexpr int kPrefetch = 4;
// raw buffer descriptor word 3 for gfx9-family: 32-bit data format, no swizzle,
// range checking on the byte offset
constexpr int kRsrcWord3 = 0x00020000;
// cache-policy operand of the buffer builtins: sc1 = device-scope coherence
constexpr int kSc1 = 16;

// Column mode (see Params): workgroups per column = tiles per region.
constexpr int kMem = 16;
// fixed cost of a region piece (prologue and epilogue), in K-steps, charged
// when the work sequence is cut into columns
constexpr int kColHov = 3;
// column mode is used when the (expert, tile) work items fill the chip at
// most this many times over and the mean expert has at least kColTokens
// tokens; below that the per-piece costs outweigh the better packing
constexpr int kColWaves = 4;
constexpr int kColTokens = 8192;
// the weight gradient shuffles its scale planes when M >= kShufTokens * E
constexpr int kShufTokens = 4096;
// row-ragged GEMM: whole-tile scale blocks in the raw area when C <= kWholeC
// (256 rows x C / 32 bytes per operand, plus the dword read past a row's last
// pair, within kWholeOp dwords each)
constexpr int kWholeC = 1504;
constexpr int kWholeOp = 3072;
static_assert(kTile * (kWholeC / 32) / 4 + 2 <= kWholeOp, "whole-tile scale block fits");

// LDS layout (159 KiB of the 160 KiB per CU).
struct Smem {
  // [stage][0 = A n-rows, 1 = B k-rows]: 256 rows x 128 tokens, chunk-swizzled
  uint8_t data[2][2][kOpBytes];
  // raw E8M0 scale bytes as loaded, 24 KiB, in one of three layouts:
  //  grouped (scale rows a whole number of dwords): [group % 3][op][row][4 dwords], the
  //    2 sub-block bytes of 8 consecutive K-steps of a row;
  //  paired (any row alignment): [pair % 4][op][dword][row], the two aligned
  //    dwords that hold a row's 4 bytes of 2 consecutive K-steps (16 KiB),
  //    then 1 KiB taking the out-of-range scale-slot loads of steps that
  //    have no scale pair to fetch (written with zeros, never read);
  //  whole (row-ragged GEMM, C <= kWholeC): [op][kWholeOp dwords], the tile's
  //    whole scale block of 256 consecutive rows per operand
  uint32_t raw[6144];
  int start[MXW_MAX_EXPERTS];
  int len[MXW_MAX_EXPERTS];
  int order[MXW_MAX_EXPERTS];
  // column mode: non-empty experts in index order (expert, loop iterations,
  // exclusive prefix of region costs), the empty ones, and their counts; one
  // workgroup per tile: the experts' ranking keys in place of the first list
  union {
    int ne[MXW_MAX_EXPERTS];
    uint32_t key[MXW_MAX_EXPERTS];
  };
  int nit[MXW_MAX_EXPERTS];
  int pre[MXW_MAX_EXPERTS];
  int ee[MXW_MAX_EXPERTS];
  int cnt[4];
  uint32_t pfd[64];  // landing place of the L2 prefetch loads (never read)
};

// 16-byte chunk c of staged row r sits at chunk position c ^ swz(r).  A
// ds_read_b128 is served 16 lanes (256 bytes of banks) at a time; a fragment
// read's 16 lanes take rows r .. r+15 at one chunk index, and with 128-byte
// rows two rows share a 256-byte bank line, so swz must differ across the 8
// rows of each parity: (r / 2) % 8 (r % 8 left rows r and r + 8 on the same
// banks, measured with SQ_LDS_BANK_CONFLICT)
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// LDS-direct loads: lane l's 16 (or 4) bytes from the buffer at voff (range
// checked against the descriptor; out-of-range lanes write zeros) land at LDS
// byte lds + 16 l (or 4 l).  M0 carries the wave-uniform LDS base and needs
// one instruction before the load.  (M0 has no other user in this kernel.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const __amdgpu_buffer_rsrc_t& rsrc, uint32_t lds, uint32_t voff,
                                      uint32_t soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "m0");
}
__device__ __forceinline__ void dma4(const __amdgpu_buffer_rsrc_t& rsrc, uint32_t lds, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// the same for 4 bytes per lane (lane l's dword lands at lds + 4 l), with a
// scalar offset added after the range check
__device__ __forceinline__ void dma4s(const __amdgpu_buffer_rsrc_t& rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, %3 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "m0");
}
// counter waits (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; the counters not waited on are left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lgkm_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Inclusive prefix sum over the 64 lanes of a wave, all of which must be
// active: log-step shifts inside each row of 16 lanes (DPP row_shr 1, 2, 4, 8;
// lanes with no source add 0), then lane 15 of rows 0 and 2 added to rows 1
// and 3 (row_bcast:15) and lane 31 to rows 2 and 3 (row_bcast:31).  Six
// VALU operations, against six LDS-crossbar round trips for a shuffle scan.
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return v;
}

// live-sub-block mask of K-step s for window [start, end): bit b set iff tokens
// [64 s + 32 b, 64 s + 32 b + 32) lie inside the window.
__device__ __forceinline__ uint32_t live_mask(int s, int start, int end) {
  uint32_t m = 0;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int t0 = s * kStep + 32 * b;
    m |= (uint32_t)(t0 >= start && t0 + 32 <= end) << b;
  }
  return m;
}
// 4-bit live mask of the 128-token pair P from sub-block indices qs, qn
__device__ __forceinline__ uint32_t live_mask_pair(int P, int qs, int qn) {
  uint32_t m = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) m |= (uint32_t)((uint32_t)(4 * P + b - qs) < (uint32_t)qn) << b;
  return m;
}
// the same from sub-block indices qs = start / 32, qn = (end - start) / 32
__device__ __forceinline__ uint32_t live_mask_q(int s, int qs, int qn) {
  const uint32_t q = (uint32_t)(2 * s - qs);
  return (uint32_t)(q < (uint32_t)qn) | ((uint32_t)(q + 1u < (uint32_t)qn) << 1);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 h = __builtin_convertvector(f, bf16x2);  // round-to-nearest-even
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

// v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands (format code 0) and the
// scale byte selectors as template constants.
template <int OA, int OB>
__device__ __forceinline__ v16f mfma_e4m3(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OA, sa, OB, sb);
}

// same, selectors given as values that are constant after unrolling
__device__ __forceinline__ v16f mfma_e4m3_sel(int oa, int ob, const v8i& a, const v8i& b, const v16f& c, int sa,
                                             int sb) {
  switch (oa * 4 + ob) {
#define MXW_SEL(A_, B_) \
  case A_ * 4 + B_:     \
    return mfma_e4m3<A_, B_>(a, b, c, sa, sb);
    MXW_SEL(0, 0) MXW_SEL(0, 1) MXW_SEL(0, 2) MXW_SEL(0, 3)
    MXW_SEL(1, 0) MXW_SEL(1, 1) MXW_SEL(1, 2) MXW_SEL(1, 3)
    MXW_SEL(2, 0) MXW_SEL(2, 1) MXW_SEL(2, 2) MXW_SEL(2, 3)
    MXW_SEL(3, 0) MXW_SEL(3, 1) MXW_SEL(3, 2) MXW_SEL(3, 3)
#undef MXW_SEL
    default:
      __builtin_unreachable();
  }
}

// v_mfma_f32_32x32x16_bf16 on half H of two fragments: bytes 16 H .. 16 H + 15
// of each lane's 32 (8 bf16 values per lane and operand)
template <int H>
__device__ __forceinline__ v16f mfma_bf16(const v8i& a, const v8i& b, const v16f& c) {
  const v4i ah = __builtin_shufflevector(a, a, 4 * H, 4 * H + 1, 4 * H + 2, 4 * H + 3);
  const v4i bh = __builtin_shufflevector(b, b, 4 * H, 4 * H + 1, 4 * H + 2, 4 * H + 3);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, ah), __builtin_bit_cast(v8bf, bh), c, 0, 0, 0);
}

// one MFMA operand fragment: the lane's two 16-byte runs of a 32-row block
__device__ __forceinline__ v8i frag(const uint8_t* blk, int lo, int hi) {
  const v4i a = *(const v4i*)(blk + lo);
  const v4i b = *(const v4i*)(blk + hi);
  return (v8i){a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}

struct Params {
  const uint8_t* A;
  const uint8_t* sA;
  const uint8_t* B;
  const uint8_t* sB;
  const int32_t* offs;
  uint16_t* out;
  // weight gradient: A [N, M], B [K, M], out [E, N, K] (contraction M);
  // row-ragged GEMM: A [R, M], B [E, N, M], out [R, N] (contraction M, K unused)
  int E, M, N, K;
  // row stride of A and B in bytes (>= M; the scale planes' rows are ld / 32
  // bytes apart): M unless the caller pads its rows
  int ld;
  int R;  // row-ragged GEMM: rows of A and out
  // log2 of the bytes per token of A and B: 0 for E4M3 codes, 1 for bf16 (M,
  // the row stride and every window are then in bytes: offs are shifted)
  int tshift;
  int tilesN, tilesK;
  // XCD regions (0 = off): each expert's tilesN x tilesK grid is cut into 8
  // rectangles of regN x regK tiles, regB of them across the K direction;
  // rectangle x is walked in bands of `band` rows, column by column
  int regN, regK, regB, band;
  // column mode (ncol > 0): the grid is ncol columns of kMem workgroups,
  // each column on one XCD (one workgroup per CU); the (expert, region) work
  // sequence is cut into ncol equal spans, one per column, and a region cut
  // between columns is summed through FP32 partial tiles
  // weight gradient on E4M3 operands: the scale planes rewritten per call by
  // scale_shuffle_kernel as [256-row band][group of 8 K-steps][256 rows][16
  // bytes], sgroups groups per band (see there)
  const uint8_t* sAs;
  const uint8_t* sBs;
  int sgroups;
  float* part;      // [ncol][2][kMem][kTile * kTile] partial tiles (a column's first / last piece)
  uint32_t* flags;  // [ncol][kMem] arrival counters of cut regions, cleared by the call's first kernel
  int ncol;
  int regions;  // regions of up to kMem tiles per expert
  int rband;    // tile rows per band of regions (see region_tile)
  int hov;      // per-region cost, in K-steps, added to the split's weights
  // tiles along N of 256 rows; tiles tn >= tall have kShort rows (starting at
  // 256 tall + 192 (tn - tall)); tall = tilesN when N has no short tiles
  int tall;
  // one workgroup per tile: blocks [nfull, grid) are half tiles, two per tile
  // of blocks [nfull, nfull + (grid - nfull) / 2) of the plain dealing (the
  // last tiles in longest-first order); nfull = grid for no split
  int nfull;
};

// loop iterations (4 K-steps each) of an expert's window [start, start + len)
__device__ __forceinline__ int window_iters(int start, int len) {
  const int s0 = (start / kPair) * 2;
  const int s_end = (start + len + kStep - 1) / kStep;
  return ((s_end - s0 + 3) & ~3) >> 2;
}

// Region r of an expert's tile grid and its member j (0 .. kMem-1): bands of
// H tile rows hold H x (kMem / H) regions; a last band of h < H rows holds
// h x (kMem / h) regions (3 x 5 for h = 3).  A region's tiles share H (or h)
// A stripes and kMem / H (or kMem / h) B stripes, which its members stream
// together through their XCD's L2.  H (4, 8 or 2) is chosen on the host so
// that the regions leave the fewest members without a tile (region_band).
// Returns false if member j has no tile.
__device__ __forceinline__ bool region_tile(int tN, int tK, int H, int r, int j, int& tn, int& tk) {
  const int wf = kMem / H;
  const int full = tN / H, rpf = (tK + wf - 1) / wf;
  int band, c, h, w;
  if (r < full * rpf) {
    band = r / rpf;
    c = r - band * rpf;
    h = H;
    w = wf;
  } else {
    band = full;
    c = r - full * rpf;
    h = tN - H * full;
    w = kMem / h;
  }
  if (j >= h * w) return false;
  tn = H * band + j % h;
  tk = c * w + j / h;
  return tk < tK;
}

// One workgroup per tile: block b's expert rank d (index into the
// longest-first order) and tile (tn, tk).  The dispatcher deals block b to
// XCD b % 8 and each XCD starts its blocks in order.  With regions, XCD x
// owns the same rectangle of every expert's tile grid and works through the
// experts longest first, so its co-resident workgroups cover a compact block
// of one expert's tiles and share their A and B stripes in that XCD's L2.
__device__ __forceinline__ int tile_of_block(const Params& p, int bid, int& tn, int& tk) {
  int d;
  if (p.regN) {
    const int per = p.regN * p.regK;  // = T / 8
    const int x = bid & 7, i = bid >> 3;
    d = i / per;
    const int v = i - d * per;
    const int bandsz = p.band * p.regK;
    const int bnd = v / bandsz, w = v - bnd * bandsz;
    const int hb = min(p.band, p.regN - bnd * p.band);  // rows in this band
    const int c = w / hb;
    tn = (x / p.regB) * p.regN + bnd * p.band + (w - c * hb);
    tk = (x % p.regB) * p.regK + c;
  } else {
    const int T = p.tilesN * p.tilesK;
    d = bid / T;
    const int u = bid - d * T;
    tn = u / p.tilesK;
    tk = u - tn * p.tilesK;
  }
  return d;
}

// exact +0 over tile (tn, tk) of expert g's output (non-temporal stores, as
// for the computed tiles)
__device__ __forceinline__ void zero_tile(const Params& p, int g, int tn, int tk) {
  const int N = p.N, K = p.K;
  const int n0 = tn * kTile, k0 = tk * kTile;
  const int rows = min(kTile, N - n0), cols = min(kTile, K - k0);
  const int chunks = cols / 8;  // 16-byte chunks per row (K % 16 == 0)
  const v4i z = {0, 0, 0, 0};
  uint16_t* o = p.out + (size_t)g * N * K;
  for (int i = threadIdx.x; i < rows * chunks; i += kThreads) {
    const int r = i / chunks, c = i - r * chunks;
    __builtin_nontemporal_store(z, (v4i*)(o + (size_t)(n0 + r) * K + k0 + 8 * c));
  }
}

// One tile piece: contraction [start, end) of expert g into tile (tn, tk).
// Row-ragged GEMM: tile (tn = row tile, tk = column tile) of rows
// [ar0, ar0 + ra) of A, all of expert g.
struct Piece {
  int g, tn, tk, start, end;
  int role;  // 0: whole tile; 1, 2: a piece of a region cut between columns (2: its first)
  int col, member, Q, ra_lin, r_it;  // column mode: position, column quota, the region's place and length
  int ar0, ra;                       // row-ragged GEMM: first row of A and rows in the tile
  int half;                          // HALF: which half of the tile (the A band starts 32 h rows lower)
};

// ROWS: the row-ragged GEMM (out rows = A rows of one expert, out columns =
// that expert's B rows); otherwise the weight gradient.  BF: the weight
// gradient on bf16 operands.  Everything along the token axis is then counted
// in bytes (a staged 128-byte row holds 64 tokens, a "K-step" 32 and a
// "sub-block" 16), there are no scales, and each MFMA slot runs two
// v_mfma_f32_32x32x16_bf16 on the halves of the fragments that the E4M3
// instruction takes whole: the same bytes per clock, at twice the
// instruction count and half the FLOP per byte.
// WHOLE (row-ragged GEMM with C <= kWholeC): the tile's whole scale blocks
// (its 256 A rows and 256 B rows are consecutive rows of the planes, so each
// block is one contiguous range of 256 C / 32 bytes) are DMA'd once, in the
// prologue, with 16-byte LDS-direct loads (dword loads when a block is not
// 4-byte aligned); the K-loop then loads no scales.
// HALF (weight gradient, one workgroup per tile): a half tile.  The
// workgroup computes only the even 32-row A blocks of each wave's quarter, on
// an A band that starts 32 pc.half rows below the tile's, so the two halves
// of a tile cover its even and its odd blocks.  Each computed block is the
// same MFMA sequence on the same fragments and scales as in the whole tile,
// so the output bits are the whole tile's.  The A row groups of the odd
// blocks are neither loaded nor read, and their MFMAs are not issued: half
// the MFMA work and a quarter less staging per K-step.
template <bool GROUP, bool COL, bool ROWS, bool BF = false, bool WHOLE = false, bool HALF = false, bool SHORT = false,
          bool WALIGN = false, bool GUNAL = false>
__device__ __forceinline__ void run_piece(const Params& p, Smem& sm, const Piece& pc) {
  static_assert(!HALF || (!COL && !ROWS && !WHOLE), "half tiles: weight gradient, one workgroup per tile");
  static_assert(!SHORT || (!ROWS && !WHOLE && !HALF), "short tiles: weight gradient");
  static_assert(!WALIGN || WHOLE, "dword-aligned scale rows: whole-tile scale blocks");
  static_assert(!GUNAL || (GROUP && !COL && !ROWS && !BF), "grouped loads from unaligned rows: weight gradient, per tile");
  // A rows per wave: its 32-row blocks t < (SHORT ? 3 : 4)
  constexpr int kWaveA = SHORT ? kShort / 2 : kTile / 2;
  int tid = threadIdx.x;
  // opaque per piece: nothing derived from the thread index is hoisted out of
  // the column loop (it would stay live through the K-loop)
  if (COL) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = p.M, N = p.N, K = p.K, ld = p.ld;
  const int g = pc.g, start = pc.start, end = pc.end, role = pc.role;
  const int col = pc.col, member = pc.member, Q = pc.Q, ra_lin = pc.ra_lin, r_it = pc.r_it;
  // the tile: rows [arow, arow + rowsA) of A, [brow, brow + rowsB) of B, and
  // its place in out (row stride ldo)
  size_t arow, brow;
  int rowsA, rowsB, ldo;
  uint16_t* otile;
  if constexpr (ROWS) {
    const int c0 = pc.tk * kTile;
    arow = (size_t)pc.ar0;
    rowsA = pc.ra;
    brow = (size_t)g * N + c0;
    rowsB = min(kTile, N - c0);
    ldo = N;
    otile = p.out + arow * N + c0;
  } else {
    const int n0 = (SHORT ? p.tall * kTile + (pc.tn - p.tall) * kShort : pc.tn * kTile) + (HALF ? 32 * pc.half : 0),
              k0 = pc.tk * kTile;
    arow = (size_t)n0;
    rowsA = min(SHORT ? kShort : kTile, N - n0);
    // a half band may start past N (none of its rows then exist); the
    // clamp is done in a scalar register, which the descriptors need
    if (HALF) rowsA = __builtin_amdgcn_readfirstlane(rowsA < 0 ? 0 : rowsA);
    brow = (size_t)k0;
    rowsB = min(kTile, K - k0);
    ldo = K;
    otile = p.out + (size_t)g * N * K + (size_t)n0 * K + k0;
  }

  // ---- buffer resources, rebased to this tile's 256-row bands ----------------
  // SHUF: the weight gradient's grouped scale loads read the shuffled planes,
  // in which the 16-byte groups of a band's 256 rows are contiguous (when
  // the host made them: p.sAs != null)
  const bool SHUF = GROUP && !ROWS && !BF && p.sAs != nullptr;
  const uint32_t sbytes = (uint32_t)ld >> 5;  // scale bytes from one row to the next
  // (a short tile's A rows past its 192 are out of range: loaded as zeros,
  // never read)
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A + arow * ld, (uint32_t)rowsA * (uint32_t)ld);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.B + brow * ld, (uint32_t)rowsB * (uint32_t)ld);
  // scale planes are read as whole dwords; rounding the range up to 4 bytes
  // keeps every dword entirely inside or outside it (bytes past the plane
  // belong to tokens >= M, which are always masked)
  const uint32_t band_bytes = (uint32_t)p.sgroups * (uint32_t)(kTile * 16);
  const __amdgpu_buffer_rsrc_t rsA =
      SHUF ? make_rsrc(p.sAs + (size_t)pc.tn * band_bytes, band_bytes)
           : make_rsrc(p.sA + arow * sbytes, ((uint32_t)rowsA * sbytes + 3u) & ~3u);
  const __amdgpu_buffer_rsrc_t rsB =
      SHUF ? make_rsrc(p.sBs + (size_t)pc.tk * band_bytes, band_bytes)
           : make_rsrc(p.sB + brow * sbytes, ((uint32_t)rowsB * sbytes + 3u) & ~3u);

  // ---- per-lane DMA geometry -------------------------------------------------
  // Data: a stage holds a pair of K-steps (128 tokens, one cache line per row).
  // Wave w fills row groups 8w .. 8w+7 (8 rows x 128 B = 1 KiB each) of both
  // stripes.  Lane i of a group writes LDS bytes [16 i, 16 i + 16) of the group:
  // row i / 8, chunk position i % 8, which holds global chunk (i % 8) ^ swz(row).
  const int lrow = lane >> 3;
  // swz of the wave's rows depends on lrow and the parity of the row group q
  const int ch_e = (lane & 7) ^ swz(lrow), ch_o = (lane & 7) ^ swz(8 + lrow);
  // The lane's offset for each of the wave's 8 row groups, in a register (so
  // the descriptor's range check sees the row: rows past the operand's end
  // read nothing).  One workgroup per tile: the row groups go out in a
  // rotated order, load q taking group (q + rot) % 8: the tiles that share an
  // A (B) stripe rotate by different even amounts, so each tile's first loads
  // of a pair are the likely misses, with the most lead, and its last ones
  // mostly hit lines another tile requested earlier.  (Column mode's in-step
  // tiles lose with the rotation.)
  const int rot = (COL || HALF) ? 0 : 2 * ((pc.tk + pc.tn) & 3);
  uint32_t vrow[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    vrow[q] = (uint32_t)((wave * 8 + ((q + rot) & 7)) * 8 + lrow) * (uint32_t)ld + (uint32_t)(((q & 1) ? ch_o : ch_e) * 16);
  // Scales: lane l of wave w fetches scale row 64 w + l (shuffled planes: the
  // 16 bytes of that row in each group of 4 KiB)
  const uint32_t srow_off = (uint32_t)(wave * 64 + lane) * (SHUF ? 16u : sbytes);
  const int sbl_e = ch_e >> 1, sbl_o = ch_o >> 1;  // this lane's 32-token sub-block within a pair
  const uint32_t dbase = __builtin_amdgcn_readfirstlane(lds_addr(&sm.data[0][0][wave * 8 * 1024]));
  // Column mode L2 prefetch.  The tiles of a region that share an A (B) stripe
  // run in step and would all wait out the same misses; instead, at each even
  // step every tile touches its share of the stripe lines of the pair after
  // the one the next odd step loads (one dword per line, 8 lines per
  // instruction), so that pair's loads mostly hit in L2.  Sharer i of a stripe with
  // S sharers takes row groups i and i + S (if < 8) of every wave's 8, of A
  // and of B: two instructions per operand per wave.
  int pfa = 8, pfb = 8, pfsa = 8, pfsb = 8;
  if constexpr (COL) {
    const int full = p.tilesN / p.rband, band = pc.tn / p.rband;
    const int rh = band < full ? p.rband : p.tilesN - p.rband * full;  // region height (tiles along N)
    pfa = __builtin_amdgcn_readfirstlane(member / rh);      // index among the A stripe's sharers
    pfb = __builtin_amdgcn_readfirstlane(member % rh);      // among the B stripe's
    pfsa = __builtin_amdgcn_readfirstlane(kMem / rh);       // A stripe sharers = region width
    pfsb = __builtin_amdgcn_readfirstlane(rh);
  }
  const uint32_t pfdst = __builtin_amdgcn_readfirstlane(lds_addr(&sm.pfd[0]));
  // pair P into stage buf: load i of 16 (row group 8w + i/2 of A for even i,
  // of B for odd i); dead sub-blocks are forced out of range
  auto dma_pair = [&](int i, int buf, int P, uint32_t live) {
    const int qi = i >> 1, op = i & 1;
    if (HALF && op == 0 && qi >= 4) return;  // an odd A block's rows
    const bool ok = (live >> ((qi & 1) ? sbl_o : sbl_e)) & 1u;
    const int q = (qi + rot) & 7;  // same parity as qi
    dma16(op ? rB : rA, dbase + (uint32_t)((buf * 2 + op) * kOpBytes + q * 1024), ok ? vrow[qi] : kOob,
          (uint32_t)(P * kPair));
  };

  // Scale loads.  A K-step needs 2 bytes of each of 512 rows; fetching them
  // step by step presents one cache line per row per step to the memory path,
  // as many requests as all of the step's operand data.  So when scale rows
  // are a whole number of dwords (M % 128 == 0; a 16-byte LDS-direct load
  // takes a 4-byte-aligned start; GUNAL: any rows, each load starting at the
  // dword boundary below the group) each row's 16 bytes of 8 consecutive
  // K-steps ("group" G = steps 8G .. 8G+7) come in one 16-byte load per lane
  // and operand, into 3 buffers by G % 3: one load per loop iteration (4
  // K-steps), operand k % 2 of group (s0 + 4 (k - k % 2)) / 8 + 2 in
  // iteration k, so no step carries a load with nothing to fetch.  Otherwise
  // (the row-ragged GEMM at C % 128 != 0) the two aligned dwords around each row's 4 bytes of 2 consecutive K-steps
  // ("pair" G = steps 2G, 2G+1) are fetched, 4 loads per wave per pair, into
  // 4 buffers by pair % 4; pair G + 3 is fetched at step 2G, and loads with
  // real == false are out of range (no memory traffic, but address-unit
  // time) so that every step issues the same count.
  constexpr int kGroupSteps = GROUP ? 8 : 2;
  constexpr int kAhead = GROUP ? 1 : 3;
  constexpr int kScaleDma = (BF || WHOLE) ? 0 : (GROUP ? 2 : 4);
  // grouped: one operand's 16 bytes of group g for this lane's row, into
  // slot g % 3 (groups past the row's end read other rows' bytes or nothing;
  // they only reach steps past M, whose sub-blocks are all dead)
  // (GUNAL: scale rows not a whole number of dwords; each row's group is
  // loaded from the dword boundary at or below its start, (row offset) % 4
  // bytes early, and its last bytes are the first of the next group's load)
  const uint32_t sgrp_off = GUNAL ? (srow_off & ~3u) : srow_off;
  auto dma_scale_grp = [&](int g, int op) {
    const uint32_t dst = lds_addr(&sm.raw[(((g % 3) * 2 + op) * kTile + wave * 64) * 4]);
    dma16(op ? rsB : rsA, __builtin_amdgcn_readfirstlane(dst),
          sgrp_off + (SHUF ? (uint32_t)(kTile * 16) : 16u) * (uint32_t)g, 0u);
  };
  auto dma_scales = [&](int grp_idx, bool real) {
    {
#pragma unroll
      for (int k = 0; k < 4; ++k) {  // A lo, A hi, B lo, B hi
        const int op = k >> 1;
        const uint32_t so = real ? (srow_off & ~3u) + 4u * (uint32_t)grp_idx + 4u * (uint32_t)(k & 1) : kOob;
        const uint32_t dst = real ? lds_addr(&sm.raw[(((grp_idx & 3) * 2 + op) * 2 + (k & 1)) * kTile + wave * 64])
                                  : lds_addr(&sm.raw[4096]);
        dma4(op ? rsB : rsA, __builtin_amdgcn_readfirstlane(dst), so);
      }
    }
  };

  // ---- MFMA geometry -----------------------------------------------------------
  // wave (wn, wk) owns A rows 128 wn .. +128 and B rows 128 wk .. +128: 4 x 4
  // blocks of 32 x 32 outputs.  Fragment of a 32-row block for the first
  // K-step of a pair: lane l reads row l % 32, chunks l / 32 and l / 32 + 2
  // (tokens 16 (l / 32) + 0..15 and 32 + 16 (l / 32) + 0..15); for the second
  // K-step, chunks 4 further on.
  const int wn = wave >> 1, wk = wave & 1;
  const int fr = lane & 31, fq = lane >> 5;
  const int frag_lo0 = fr * kRowBytes + ((fq ^ swz(fr)) << 4);
  const int frag_hi0 = fr * kRowBytes + (((fq + 2) ^ swz(fr)) << 4);
  const int frag_lo1 = fr * kRowBytes + (((fq + 4) ^ swz(fr)) << 4);
  const int frag_hi1 = fr * kRowBytes + (((fq + 6) ^ swz(fr)) << 4);

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v16f){};

  // ---- the K-loop ----------------------------------------------------------------
  // K-step j of the window (tokens [64 (s0 + j), +64)) is half j % 2 of pair
  // (s0 + j) / 2, which sits in stage (j / 2) % 2.  A pair is DMA'd as whole
  // 128-byte row segments (one cache line per row, so every memory request
  // carries a full line).  Step j + 1's fragments and scale words are read into
  // register set (j + 1) % 2 during step j, so step j's MFMAs never wait on
  // LDS.  Odd steps have one barrier (after their first two MFMAs): it
  // certifies that the next pair has landed and that every wave has read the
  // current pair, whose stage then takes the pair after next (loaded during
  // this step and the next).
  const int s0 = (start / kPair) * 2;
  const int s_end = (end + kStep - 1) / kStep;
  const int nsteps = (s_end - s0 + 3) & ~3;  // a multiple of 4: the loop body is unrolled by 4

  // The 16 loads of a pair go out in two parts: kOddLoads at the odd step
  // whose barrier freed its stage (two steps ahead of its use), the rest in
  // the first MFMA slots of the next (even) step.  Spreading them keeps the
  // address unit below its full rate (one 1 KiB load per ~16 clk per CU,
  // that is one per MFMA from each of the 4 waves), so load issue does not
  // hold up the MFMAs, while the even step's part still lands well before
  // the next odd barrier.  Then the scale loads (paired: kScaleDma per step;
  // grouped: one per 4-step iteration, at its first step) and, in column
  // mode, the even step's prefetches.  At the barrier of odd step j the pair
  // issued at steps j - 2 and j - 1 must have landed: only the loads issued
  // after step j - 1's data loads may still be in flight.
  constexpr int kSlot = kScaleDma;
  constexpr int kOddLoads = 10;

  // Prologue: the scale groups the first steps need, pair s0/2, the odd-step
  // part of pair s0/2 + 1 (the first step issues the rest), and (paired) one
  // dummy scale slot.
  const int qs = start >> 5, qn = (end - start) >> 5;
  {
    const int G0 = s0 / kGroupSteps;
    if (BF) {
      // no scales
    } else if (WHOLE) {
      // A's block into raw[0 ..), B's into raw[kWholeOp ..).  The range check
      // works per dword (each dword entirely inside or outside the checked
      // range, which is rounded up to 4 bytes), so with 4-byte-aligned blocks
      // (C % 128 == 0 and 4-byte-aligned planes) 1 KiB per instruction, 16
      // bytes per lane: a quarter of the instructions of the dword loads
      // (256 bytes per instruction) that other blocks take
      const bool wide = ((sbytes & 3u) | ((uint32_t)(uintptr_t)p.sA & 3u) | ((uint32_t)(uintptr_t)p.sB & 3u)) == 0u;
      const int shift = wide ? 10 : 8;
      const int nA = (int)((kTile * sbytes + (1u << shift) - 1u) >> shift);
      for (int k = wave; k < 2 * nA; k += 4) {
        const int op = k >= nA, kk = k - op * nA;
        const uint32_t dst = lds_addr(&sm.raw[op * kWholeOp + (kk << (shift - 2))]);
        if (wide)
          dma16(op ? rsB : rsA, __builtin_amdgcn_readfirstlane(dst), (uint32_t)kk * 1024u + 16u * (uint32_t)lane, 0u);
        else
          dma4(op ? rsB : rsA, __builtin_amdgcn_readfirstlane(dst), (uint32_t)kk * 256u + 4u * (uint32_t)lane);
      }
    } else if (GROUP) {
      // groups G0 and G0 + 1; the loop fetches group G + 2 for both operands
      // during the two iterations that start in group G
#pragma unroll
      for (int a = 0; a < 4; ++a) dma_scale_grp(G0 + (a >> 1), a & 1);
    } else {
#pragma unroll
      for (int a = 0; a <= kAhead; ++a) dma_scales(G0 + a, true);
    }
    const int P0 = s0 >> 1;
    const uint32_t l0 = live_mask_pair(P0, qs, qn), l1 = live_mask_pair(P0 + 1, qs, qn);
#pragma unroll
    for (int i = 0; i < kDataDma; ++i) dma_pair(i, 0, P0, l0);
#pragma unroll
    for (int i = 0; i < kOddLoads; ++i) dma_pair(i, 1, P0 + 1, l1);
    if (!GROUP && !BF && !WHOLE) dma_scales(0, false);
  }
  // (a half tile skips one of the kOddLoads: A row group 4)
  wait_vm<((GROUP || BF || WHOLE) ? kOddLoads : kOddLoads + kSlot) - (HALF ? 1 : 0)>();  // scales and pair s0/2 landed (this wave)
  __syncthreads();

  // Scale registers.  In lane l the MFMA takes the E8M0 byte of row l % 32 and
  // 32-token sub-block l / 32 of each 32-row block, from the byte op_sel
  // picks.  A row's raw dword for a pair of K-steps holds sub-blocks 0, 1 of
  // the first K-step, then of the second; shifted right by 8 (l / 32) bits,
  // its byte 0 is this lane's byte of the first K-step and byte 2 that of the
  // second.  So a lane keeps one dword per 32-row block and operand for a
  // whole pair, with the bytes of dead sub-blocks cleared.
  const int msb = lane >> 5;
  const uint32_t mshift = 8u * (uint32_t)msb;
  auto load_sregs = [&](int x, uint32_t* ra4, uint32_t* rb4) {  // x: first K-step of the pair
    const uint32_t pm = (((live_mask_q(x, qs, qn) >> msb) & 1u) ? 0xFFu : 0u) |
                        (((live_mask_q(x + 1, qs, qn) >> msb) & 1u) ? 0xFF0000u : 0u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int RA = wn * kWaveA + 32 * i + fr, RB = wk * 128 + 32 * i + fr;
      uint32_t a, b;
      if (WHOLE) {
        // the 4 bytes of steps x, x + 1 of each row (x is even; one aligned
        // dword when the rows are, WALIGN)
        const uint32_t ba = (uint32_t)RA * sbytes + 2u * (uint32_t)x, bb = (uint32_t)RB * sbytes + 2u * (uint32_t)x;
        if (WALIGN) {
          a = sm.raw[ba >> 2];
          b = sm.raw[kWholeOp + (bb >> 2)];
        } else {
          a = __builtin_amdgcn_alignbit(sm.raw[(ba >> 2) + 1], sm.raw[ba >> 2], (ba & 3u) * 8u);
          b = __builtin_amdgcn_alignbit(sm.raw[kWholeOp + (bb >> 2) + 1], sm.raw[kWholeOp + (bb >> 2)], (bb & 3u) * 8u);
        }
      } else if (GROUP) {
        const int slot = (x >> 3) % 3, dw = (x & 7) >> 1;
        a = sm.raw[((slot * 2 + 0) * kTile + RA) * 4 + dw];
        b = sm.raw[((slot * 2 + 1) * kTile + RB) * 4 + dw];
        if (GUNAL) {
          // the dword after, in this group's load or the next group's
          const int ns = dw < 3 ? slot : (slot + 1) % 3, nd = dw < 3 ? dw + 1 : 0;
          a = __builtin_amdgcn_alignbit(sm.raw[((ns * 2 + 0) * kTile + RA) * 4 + nd], a,
                                        (((uint32_t)RA * sbytes) & 3u) * 8u);
          b = __builtin_amdgcn_alignbit(sm.raw[((ns * 2 + 1) * kTile + RB) * 4 + nd], b,
                                        (((uint32_t)RB * sbytes) & 3u) * 8u);
        }
      } else {
        const int slot = (x >> 1) & 3;
        a = __builtin_amdgcn_alignbit(sm.raw[((slot * 2 + 0) * 2 + 1) * kTile + RA],
                                      sm.raw[((slot * 2 + 0) * 2 + 0) * kTile + RA], (((uint32_t)RA * sbytes) & 3u) * 8u);
        b = __builtin_amdgcn_alignbit(sm.raw[((slot * 2 + 1) * 2 + 1) * kTile + RB],
                                      sm.raw[((slot * 2 + 1) * 2 + 0) * kTile + RB], (((uint32_t)RB * sbytes) & 3u) * 8u);
      }
      ra4[i] = (a >> mshift) & pm;
      rb4[i] = (b >> mshift) & pm;
    }
  };

  // grouped: the raw dwords are read a few MFMAs before they are shifted and
  // masked, so the wave does not wait on the LDS between two MFMAs
  auto read_raw = [&](int x, uint32_t* a4, uint32_t* b4, uint32_t* an4, uint32_t* bn4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int RA = wn * kWaveA + 32 * i + fr, RB = wk * 128 + 32 * i + fr;
      const int slot = (x >> 3) % 3, dw = (x & 7) >> 1;
      a4[i] = sm.raw[((slot * 2 + 0) * kTile + RA) * 4 + dw];
      b4[i] = sm.raw[((slot * 2 + 1) * kTile + RB) * 4 + dw];
      if (GUNAL) {
        const int ns = dw < 3 ? slot : (slot + 1) % 3, nd = dw < 3 ? dw + 1 : 0;
        an4[i] = sm.raw[((ns * 2 + 0) * kTile + RA) * 4 + nd];
        bn4[i] = sm.raw[((ns * 2 + 1) * kTile + RB) * 4 + nd];
      }
    }
  };
  auto finish_sregs = [&](int x, const uint32_t* a4, const uint32_t* b4, const uint32_t* an4, const uint32_t* bn4,
                          uint32_t* ra4, uint32_t* rb4) {
    const uint32_t pm = (((live_mask_q(x, qs, qn) >> msb) & 1u) ? 0xFFu : 0u) |
                        (((live_mask_q(x + 1, qs, qn) >> msb) & 1u) ? 0xFF0000u : 0u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t a = a4[i], b = b4[i];
      if (GUNAL) {
        const uint32_t RA = (uint32_t)(wn * kWaveA + 32 * i + fr), RB = (uint32_t)(wk * 128 + 32 * i + fr);
        a = __builtin_amdgcn_alignbit(an4[i], a, ((RA * sbytes) & 3u) * 8u);
        b = __builtin_amdgcn_alignbit(bn4[i], b, ((RB * sbytes) & 3u) * 8u);
      }
      ra4[i] = (a >> mshift) & pm;
      rb4[i] = (b >> mshift) & pm;
    }
  };

  // whole-tile scale blocks (WHOLE): the next pair's two dwords per row and
  // operand are read one 32-row block per MFMA slot right after the odd
  // step's barrier (m = 2 .. 5), and joined, shifted and masked one block per
  // slot (m = 11 .. 14); formed all at once, the 16 LDS reads, their waits and
  // ~60 vector instructions sat between two MFMAs (+2.0% at C = 1,408).  The
  // other scale paths keep the placement below, which measured best for them.
  uint32_t wlo[8], whi[8];  // [operand * 4 + block]
  uint32_t wpm = 0;
  auto whole_read = [&](int x, int i) {
    const int RA = wn * 128 + 32 * i + fr, RB = wk * 128 + 32 * i + fr;
    const uint32_t ba = (uint32_t)RA * sbytes + 2u * (uint32_t)x, bb = (uint32_t)RB * sbytes + 2u * (uint32_t)x;
    wlo[i] = sm.raw[ba >> 2];
    wlo[4 + i] = sm.raw[kWholeOp + (bb >> 2)];
    if (!WALIGN) {  // rows of C / 32 bytes not a multiple of 4: the dword after too
      whi[i] = sm.raw[(ba >> 2) + 1];
      whi[4 + i] = sm.raw[kWholeOp + (bb >> 2) + 1];
    }
  };

  v8i fa[2][4], fb[2][4];
  uint32_t sra[2][4], srb[2][4];  // [pair parity][32-row block]
  uint32_t rawa[4], rawb[4], rawan[4], rawbn[4];
  if (!BF) load_sregs(s0, sra[0], srb[0]);
  {
    const uint8_t* ta = sm.data[0][0] + (wn * kWaveA) * kRowBytes;
    const uint8_t* tb = sm.data[0][1] + (wk * 128) * kRowBytes;
#pragma unroll
    for (int t = 0; t < 4; ++t) fb[0][t] = frag(tb + t * 32 * kRowBytes, frag_lo0, frag_hi0);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (!(HALF && (t & 1)) && !(SHORT && t == 3)) fa[0][t] = frag(ta + t * 32 * kRowBytes, frag_lo0, frag_hi0);
  }

  // per-step scalars of the first step; later steps compute theirs one step ahead
  uint32_t livep = live_mask_pair((s0 >> 1) + 2, qs, qn);  // pair issued at the next odd step
  // per row group: the lane's load offset in the pair being issued, or out of
  // range for a dead sub-block (set at odd steps, used again by the next
  // even step; the first even step issues the rest of pair s0/2 + 1)
  uint32_t va[8];
  {
    const uint32_t l1 = live_mask_pair((s0 >> 1) + 1, qs, qn);
    const bool lok_e = (l1 >> sbl_e) & 1u, lok_o = (l1 >> sbl_o) & 1u;
#pragma unroll
    for (int q = 0; q < 8; ++q) va[q] = ((q & 1) ? lok_o : lok_e) ? vrow[q] : kOob;
  }
  int sgrp = s0 / kGroupSteps + kAhead;
  bool sreal = false;  // s0 never issues a real scale load

// load D of a pair's 16 (operand D % 2, row group D / 2): odd step U issues
// the pair after next into stage U / 2, even step U the same pair into stage
// (U / 2 + 1) % 2
#define MXW_DMA_ODD(D, U)                                                                                    \
  if (!(HALF && !((D) & 1) && ((D) >> 1) >= 4))                                                              \
  dma16(((D) & 1) ? rB : rA,                                                                                 \
        dbase + (uint32_t)((((U) >> 1) * 2 + ((D) & 1)) * kOpBytes + (((((D) >> 1) + rot) & 7) * 1024)), \
        va[(D) >> 1], soffp)
#define MXW_DMA_EVEN(D, U)                                                                                         \
  if (!(HALF && !((D) & 1) && ((D) >> 1) >= 4))                                                                    \
  dma16(((D) & 1) ? rB : rA,                                                                                       \
        dbase + (uint32_t)((((((U) >> 1) + 1) & 1) * 2 + ((D) & 1)) * kOpBytes + (((((D) >> 1) + rot) & 7) * 1024)), \
        va[(D) >> 1], soffb)
  for (int jj = 0;; jj += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = jj + u;
      const int s = s0 + j;
      const int cur = u & 1, nxt = cur ^ 1;
      const int nst = ((u + 1) >> 1) & 1, nhalf = (u + 1) & 1;  // stage and half of step j + 1
      const uint8_t* na = sm.data[nst][0] + (wn * kWaveA) * kRowBytes;
      const uint8_t* nb = sm.data[nst][1] + (wk * 128) * kRowBytes;
      const int flo = nhalf ? frag_lo1 : frag_lo0, fhi = nhalf ? frag_hi1 : frag_hi0;
      __builtin_amdgcn_sched_barrier(0);
      wait_lgkm_all();  // this step's fragments and words are in registers
      __builtin_amdgcn_sched_barrier(0);
      uint32_t soffp = 0;  // odd step: token offset of the pair after next
      uint32_t soffb = 0;  // even step: of the next pair
      if (!(u & 1)) {
        int sb = s;
        asm volatile("" : "+s"(sb));
        soffb = (uint32_t)(((sb >> 1) + 1) * kPair);
      }
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int i = m >> 2, t = m & 3;  // B block i, A block t
        if constexpr (BF) {
          // first halves into block m, second halves into block (m + 8) % 16:
          // MFMAs on one accumulator stay 16 instructions apart
          const int i2 = i ^ 2;
          if (!(HALF && (t & 1)) && !(SHORT && t == 3)) {
            acc[i][t] = mfma_bf16<0>(fb[cur][i], fa[cur][t], acc[i][t]);
            acc[i2][t] = mfma_bf16<1>(fb[cur][i2], fa[cur][t], acc[i2][t]);
          }
        } else if (!(HALF && (t & 1)) && !(SHORT && t == 3)) {
          acc[i][t] = mfma_e4m3_sel(2 * (u & 1), 2 * (u & 1), fb[cur][i], fa[cur][t], acc[i][t], (int)srb[u >> 1][i],
                                    (int)sra[u >> 1][t]);
        }
        if (m == 0 && (u & 1)) {
          const bool lok_e = (livep >> sbl_e) & 1u, lok_o = (livep >> sbl_o) & 1u;
#pragma unroll
          for (int q = 0; q < 8; ++q) va[q] = ((q & 1) ? lok_o : lok_e) ? vrow[q] : kOob;
        }
        if (m == 1 && (u & 1)) {
          __builtin_amdgcn_sched_barrier(0);
          // after the previous (even) step's data loads: its scale loads
          // (paired: kSlot; grouped: one at u = 0) and, in column mode, its
          // kPrefetch prefetches
          if (BF || WHOLE) wait_vm<COL ? kPrefetch : 0>();
          else if (!GROUP) wait_vm<kSlot + (COL ? kPrefetch : 0)>();
          else if (u == 1) wait_vm<1 + (COL ? kPrefetch : 0)>();
          else wait_vm<COL ? kPrefetch : 0>();
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
        if (m == 2) {
          int sp = s;
          asm volatile("" : "+s"(sp));
          soffp = (uint32_t)(((sp >> 1) + 2) * kPair);
        }
        {
          // odd step: loads 0 .. 9 after the MFMAs m = 2, 3, 5, 6, 8, 9, 11, 12,
          // 14, 15; even step: loads 10 .. 15 after m = 0 .. 5
          constexpr int odd_load[16] = {-1, -1, 0, 1, -1, 2, 3, -1, 4, 5, -1, 6, 7, -1, 8, 9};
          constexpr int even_load[16] = {10, 11, 12, 13, 14, 15, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1};
          static_assert(odd_load[15] == kOddLoads - 1 && even_load[0] == kOddLoads, "load split");
          if ((u & 1) && odd_load[m] >= 0) MXW_DMA_ODD(odd_load[m], u);
          if (!(u & 1) && even_load[m] >= 0) MXW_DMA_EVEN(even_load[m], u);
        }
        if (COL && !(u & 1) && m >= 8 && m < 12) {
          // prefetch slot k: row group pfa + k pfsa of A (k = 0, 1), pfb + (k - 2) pfsb
          // of B (k = 2, 3), of pair s / 2 + 3; always issued (an unused slot
          // is out of range) so the load count per step is fixed
          int sq = s;
          asm volatile("" : "+s"(sq));
          const int pp = (sq >> 1) + 3;
          const int k = m - 8;
          const int q = k < 2 ? pfa + (k & 1) * pfsa : pfb + (k & 1) * pfsb;
          const bool ok = 2 * pp < s0 + nsteps && q < 8 && (pp + 1) * kPair <= M;
          // the row group goes into the range-checked (VGPR) offset, the
          // token offset (inside the row) into the scalar one
          const uint32_t rq = __builtin_amdgcn_readfirstlane(ok ? (uint32_t)q * 8u * (uint32_t)ld : kOob);
          dma4s(k < 2 ? rA : rB, pfdst, vrow[0] + rq, __builtin_amdgcn_readfirstlane(ok ? (uint32_t)(pp * kPair) : 0u));
        }
        if (m >= 3 && m < 7) fb[nxt][m - 3] = frag(nb + (m - 3) * 32 * kRowBytes, flo, fhi);
        if (m >= 7 && m < 11 && !(HALF && ((m - 7) & 1)) && !(SHORT && m == 10))
          fa[nxt][m - 7] = frag(na + (m - 7) * 32 * kRowBytes, flo, fhi);
        if (!BF && GROUP && (u & 1) && m == 10) {
          int sq = s;
          asm volatile("" : "+s"(sq));
          read_raw(sq + 1, rawa, rawb, rawan, rawbn);
        }
        if (WHOLE && (u & 1) && m >= 2 && m < 6) {
          int sq = s;
          asm volatile("" : "+s"(sq));
          whole_read(sq + 1, m - 2);
        }
        if (WHOLE && (u & 1) && m >= 11 && m < 15) {
          // the 4 bytes of steps x, x + 1 sit at the row's own byte
          // alignment (x is even)
          int sq = s;
          asm volatile("" : "+s"(sq));
          const int i = m - 11, nb = ((u >> 1) + 1) & 1;
          if (m == 11)
            wpm = (((live_mask_q(sq + 1, qs, qn) >> msb) & 1u) ? 0xFFu : 0u) |
                  (((live_mask_q(sq + 2, qs, qn) >> msb) & 1u) ? 0xFF0000u : 0u);
          const uint32_t RA = (uint32_t)(wn * 128 + 32 * i + fr), RB = (uint32_t)(wk * 128 + 32 * i + fr);
          if (WALIGN) {
            sra[nb][i] = (wlo[i] >> mshift) & wpm;
            srb[nb][i] = (wlo[4 + i] >> mshift) & wpm;
          } else {
            sra[nb][i] = (__builtin_amdgcn_alignbit(whi[i], wlo[i], ((RA * sbytes) & 3u) * 8u) >> mshift) & wpm;
            srb[nb][i] = (__builtin_amdgcn_alignbit(whi[4 + i], wlo[4 + i], ((RB * sbytes) & 3u) * 8u) >> mshift) & wpm;
          }
        }
        if (!BF && !WHOLE && m == 15) {  // after the step's data loads (vmcnt order)
          if (!GROUP) {
            dma_scales(sgrp, sreal);
          } else if (u == 0) {
            // iteration k fetches operand k % 2 of group (s0 + 4 (k - k % 2)) / 8 + 2
            const int kk = jj >> 2;
            dma_scale_grp(((s0 + 4 * (kk & ~1)) >> 3) + 2, kk & 1);
          }
        }
        if (m == 13) {
          int sp = s;
          asm volatile("" : "+s"(sp));
          // odd step: the next pair's scale registers (its raw bytes landed
          // with the pair, certified by this step's barrier)
          if (!BF && (u & 1)) {
            if (GROUP) finish_sregs(sp + 1, rawa, rawb, rawan, rawbn, sra[((u >> 1) + 1) & 1], srb[((u >> 1) + 1) & 1]);
            else if (!WHOLE) load_sregs(sp + 1, sra[((u >> 1) + 1) & 1], srb[((u >> 1) + 1) & 1]);
          }
          if (!(u & 1)) livep = live_mask_pair(((sp + 1) >> 1) + 2, qs, qn);
          sreal = ((sp + 1) % kGroupSteps) == 0;
          sgrp = (sp + 1) / kGroupSteps + kAhead;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (jj + 4 >= nsteps) break;
  }
#undef MXW_DMA_ODD
#undef MXW_DMA_EVEN
  wait_vm_all();  // no LDS-direct load may outlive the workgroup

  // ---- column mode: regions cut between columns ------------------------------
  // Such a region has one piece in each column that holds part of it (column
  // order = token order).  When its K-loop is done, every piece counts itself
  // in on the region's counter (a device-scope atomic); the last one to arrive
  // finishes the region.  With two pieces it adds the other piece's FP32
  // partial tile to its own sums -- IEEE addition is commutative, so the bits
  // do not depend on which piece arrives last; with more, every piece stores
  // its partial and the last one adds them all, in column order, from zero.
  // No workgroup ever waits for another.  Partial tiles move between XCDs,
  // whose L2s are not coherent with each other: they are written and read
  // with device-scope (sc1) accesses, which go to memory rather than a local
  // cache, and a piece counts itself in only after its stores have completed.
  // Layout of a slot: [wave][block i][block t][quad q][lane], 16 bytes each
  // (the accumulator registers as they sit); slot [column][0 / 1][member]
  // holds the column's first / last piece (a region's first piece is the last
  // piece of its column, its other pieces are first pieces).
  const __amdgpu_buffer_rsrc_t rP = make_rsrc(p.part, (uint32_t)(p.ncol * 2 * kMem) * (uint32_t)(kTile * kTile * 4));
  const uint32_t pidx = (uint32_t)(wave * 64 * 64 + lane) * 16u;  // + (((i * 4 + t) * 4 + q) * 64) * 16
  bool finish = true;  // this piece writes the bf16 result
  if (COL && role != 0) {
    uint64_t pmask = 0;  // columns holding a piece of this region
    for (int cc = 0; cc < p.ncol; ++cc) {
      const int lo = min(max((cc * Q - ra_lin + 2) >> 2, 0), r_it);
      const int hi = min(max(((cc + 1) * Q - ra_lin + 2) >> 2, 0), r_it);
      if (lo >= r_it) break;
      if (lo < hi) pmask |= 1ull << cc;
    }
    pmask |= 1ull << col;  // never empty, whatever the arithmetic above says
    const int c0 = __builtin_ctzll(pmask), np = __builtin_popcountll(pmask);
    uint32_t* ctr = &p.flags[c0 * kMem + member];
    auto slot = [&](int cc) {
      return (uint32_t)((cc * 2 + (cc == c0 ? 1 : 0)) * kMem + member) * (uint32_t)(kTile * kTile * 4) + pidx;
    };
    auto store_mine = [&]() {
      const uint32_t dst = slot(col);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const v4f v = {acc[i][t][4 * q], acc[i][t][4 * q + 1], acc[i][t][4 * q + 2], acc[i][t][4 * q + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(v, rP, dst + (uint32_t)(((i * 4 + t) * 4 + q) * 64) * 16u, 0, kSc1);
          }
      wait_vm_all();  // this wave's partial has reached memory
    };
    // tid 0 performs op on the counter; every thread gets its result
    auto counter = [&](bool add) {
      __syncthreads();
      if (tid == 0)
        sm.cnt[3] = add ? (int)__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                        : (int)__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      return __builtin_amdgcn_readfirstlane(sm.cnt[3]);
    };
    // acc (+)= the partial in slot src, 16 loads in flight
    auto add_partial = [&](uint32_t src, auto add) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v4f w[16];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < 16; ++x)
          w[x] = __builtin_amdgcn_raw_buffer_load_b128(rP, src + (uint32_t)((i * 16 + x) * 64) * 16u, 0, kSc1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int t = x >> 2, q = x & 3;
          acc[i][t][4 * q] = add ? acc[i][t][4 * q] + w[x].x : w[x].x;
          acc[i][t][4 * q + 1] = add ? acc[i][t][4 * q + 1] + w[x].y : w[x].y;
          acc[i][t][4 * q + 2] = add ? acc[i][t][4 * q + 2] + w[x].z : w[x].z;
          acc[i][t][4 * q + 3] = add ? acc[i][t][4 * q + 3] + w[x].w : w[x].w;
        }
      }
    };
    // two pieces: if the other one is done already, finish without storing
    if (np == 2 && counter(false) != 0) {
      finish = true;
    } else {
      store_mine();
      finish = counter(true) == np - 1;
    }
    if (finish) {
      uint64_t todo = pmask & ~(1ull << col);  // two pieces: mine + the other's
      if (np != 2) {                            // more: all, in column order
        add_partial(slot(c0), std::false_type{});
        todo = pmask & (pmask - 1);
      }
      for (uint64_t m = todo; m; m &= m - 1) add_partial(slot(__builtin_ctzll(m)), std::true_type{});
    }
  }

  // ---- epilogue ------------------------------------------------------------------
  // block (i, t): lane l register r holds k = 32 i + 8 (r / 4) + 4 (l / 32) + r % 4,
  // n = 32 t + l % 32 (within the wave's 128 x 128 quarter).
  if (finish) {
    // bf16 RNE in registers, then through this wave's 32 KiB of the (now idle)
    // stage area so that every global store writes whole 128-byte lines: the
    // quarter is laid out as 128 rows of 256 bytes, 16-byte chunk c of row n
    // at position c ^ (n % 16), its two 8-byte halves swapped when n / 16 is
    // odd.  The 8-byte writes of 32 lanes (rows n .. n+31, one half each) and
    // the 16-byte reads of 16 lanes then all hit distinct banks.
    __syncthreads();  // every wave is done with the stages
    uint8_t* ep = &sm.data[0][0][0] + wave * 32768;
    const int rsub = lane >> 4, cl = lane & 15;
    const int kk = wk * 128 + cl * 8;  // within the tile
    // One 32-row block at a time: its 16 8-byte writes, then its rows read
    // back (8 reads in flight before their stores: one read, wait, store at a
    // time left the wave waiting on the LDS 32 times) and stored, so the
    // first stores go out after a quarter of the writes (a wave's LDS
    // operations run in order; no other wave touches this area).  The stores
    // are non-temporal: the output is written once and never read here, and
    // streaming it past the L2 keeps the operand stripes there (row-ragged
    // GEMM, whose output is the larger part of its traffic: +2.7% to +4.3%;
    // weight gradient: within +-0.4%; same bits).
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (HALF && (t & 1)) continue;  // a half tile's odd blocks belong to the other half
      if (SHORT && t == 3) continue;  // a short tile has 3 blocks per wave
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v4f v = {acc[i][t][4 * q], acc[i][t][4 * q + 1], acc[i][t][4 * q + 2], acc[i][t][4 * q + 3]};
          const int nl = 32 * t + fr, c = 4 * i + q;
          uint2 w;
          w.x = pack_bf16x2(v.x, v.y);
          w.y = pack_bf16x2(v.z, v.w);
          *(uint2*)(ep + nl * 256 + ((c ^ (nl & 15)) << 4) + ((fq ^ (nl >> 4)) & 1) * 8) = w;
        }
      v4i d[8];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int nl = 4 * (8 * t + x) + rsub;
        d[x] = *(const v4i*)(ep + nl * 256 + ((cl ^ (nl & 15)) << 4));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int nl = 4 * (8 * t + x) + rsub;
        if ((nl >> 4) & 1) d[x] = (v4i){d[x].z, d[x].w, d[x].x, d[x].y};  // a constant after unrolling
        const int n = wn * kWaveA + nl;
        if (n < rowsA && kk < rowsB) __builtin_nontemporal_store(d[x], (v4i*)(otile + (size_t)n * ldo + kk));
      }
    }
  }
}

// GROUP: scales are loaded 8 K-steps (16 bytes per row) at a time, from rows
// that are a whole number of dwords (M % 128 == 0) or, GUNAL, from the dword
// boundary below any row's group; otherwise 2 K-steps at a time (the paired
// path, which only the row-ragged GEMM still takes).  COL: column mode (see
// Params); otherwise one workgroup per (expert, tile).  BF: bf16 operands.
template <bool GROUP, bool COL, bool BF = false, bool GUNAL = false>
__global__ __launch_bounds__(kThreads, 1) void wgrad_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = p.E, M = p.M;
  const int T = p.tilesN * p.tilesK;
  const int bid = blockIdx.x;

  // ---- windows from offs (clamped to [0, M], monotone; in bytes) -------------
  if (tid < E) {
    const int Mt = M >> p.tshift;  // tokens
    int e = min(max(p.offs[tid], 0), Mt) << p.tshift;
    const int s = tid ? min(max(p.offs[tid - 1], 0), Mt) << p.tshift : 0;
    if (e < s) e = s;
    sm.start[tid] = s;
    sm.len[tid] = e - s;
    static_assert(MXW_MAX_TOKENS < (1 << 24) && MXW_MAX_EXPERTS <= 256, "ranking key fields");
    // ranking key: window bytes (< 2^24) above 255 - g, so keys are distinct
    // and a larger key means a longer window, or an equal one of a lower index
    if (!COL) sm.key[tid] = ((uint32_t)(e - s) << 8) | (uint32_t)(255 - tid);
  }
  __syncthreads();
  if (!COL) {
    // ---- longest-first ranking: lane g counts the experts ahead of it -------
    // (one compare and one add per expert)
    if (tid < E) {
      const uint32_t mine = sm.key[tid];
      int r = 0;
      for (int u = 0; u < E; ++u) r += sm.key[u] > mine;
      sm.order[r] = tid;
    }
  } else if (wave == 0) {
    // ---- compact lists of non-empty and empty experts (wave scans) ----------
    int cn = 0, ce = 0, acc_cost = 0;
    for (int base = 0; base < E; base += 64) {
      const int e = base + lane;
      const int it = (e < E && sm.len[e] > 0) ? window_iters(sm.start[e], sm.len[e]) : 0;
      const int cost = it ? 4 * it + p.hov : 0;
      const int sc = wave_scan_incl(cost);
      const int sn = wave_scan_incl(it > 0);
      const int sz = wave_scan_incl(e < E && it == 0);
      if (it) {
        sm.ne[cn + sn - 1] = e;
        sm.nit[cn + sn - 1] = it;
        sm.pre[cn + sn - 1] = acc_cost + sc - cost;
      } else if (e < E) {
        sm.ee[ce + sz - 1] = e;
      }
      cn += __builtin_amdgcn_readlane(sn, 63);
      ce += __builtin_amdgcn_readlane(sz, 63);
      acc_cost += __builtin_amdgcn_readlane(sc, 63);
    }
    if (lane == 0) {
      sm.cnt[0] = cn;
      sm.cnt[1] = ce;
      sm.cnt[2] = acc_cost;
    }
  }
  __syncthreads();

  // ---- column mode: walk state -----------------------------------------------
  // Block b sits on XCD b % 8 (the dispatcher's round robin); with i = b / 8
  // its column is (i / kMem, b % 8) -- kMem members i % kMem on one XCD --
  // numbered from the top (later spans are dispatched first; the numbering
  // only places spans on XCDs, since no column ever waits for another).
  const int col = COL ? p.ncol - 1 - (((bid >> 3) / kMem) * 8 + (bid & 7)) : 0;
  const int member = (bid >> 3) % kMem;
  int nne = 0, kx = 0, rx = 0, Q = 0, x0 = 0, x1 = 0;
  const int Rg = p.regions;
  if (COL) {
    // tiles of experts with no tokens: exact +0, dealt round robin
    const int nemp = __builtin_amdgcn_readfirstlane(sm.cnt[1]);
    for (int z = bid; z < nemp * T; z += gridDim.x) {
      const int ez = __builtin_amdgcn_readfirstlane(sm.ee[z / T]);
      const int tz = z - (z / T) * T;
      const int tnz = tz / p.tilesK;
      zero_tile(p, ez, tnz, tz - tnz * p.tilesK);
    }
    nne = __builtin_amdgcn_readfirstlane(sm.cnt[0]);
    const int W = Rg * __builtin_amdgcn_readfirstlane(sm.cnt[2]);
    Q = (W + p.ncol - 1) / p.ncol;
    x0 = col * Q;
    x1 = x0 + Q;
    // first non-empty expert whose regions reach past x0
    kx = nne;
    for (int base = 0; base < nne; base += 64) {
      const int k = base + lane;
      const bool hit = k < nne && Rg * (sm.pre[k] + 4 * sm.nit[k] + p.hov) > x0;
      const uint64_t bal = __ballot(hit);
      if (bal) {
        kx = base + (int)__builtin_ctzll(bal);
        break;
      }
    }
    kx = __builtin_amdgcn_readfirstlane(kx);
    if (kx < nne) {
      const int pk = __builtin_amdgcn_readfirstlane(sm.pre[kx]);
      const int ck = 4 * __builtin_amdgcn_readfirstlane(sm.nit[kx]) + p.hov;
      rx = x0 > Rg * pk ? (x0 - Rg * pk) / ck : 0;
    }
  }

  if constexpr (!COL) {
    // ---- block -> (expert rank d, tile) -> (expert g, tile tn, tk) -----------
    // (tile_of_block); blocks past p.nfull are half tiles, two per tile of the
    // blocks that follow p.nfull in that dealing
    Piece pc = {};
    int bt = bid, half = -1;
    if (bid >= p.nfull) {
      const int j = bid - p.nfull;
      bt = p.nfull + (j >> 1);
      half = j & 1;
    }
    const int d = tile_of_block(p, bt, pc.tn, pc.tk);
    pc.g = __builtin_amdgcn_readfirstlane(sm.order[d]);
    pc.start = __builtin_amdgcn_readfirstlane(sm.start[pc.g]);
    const int len = __builtin_amdgcn_readfirstlane(sm.len[pc.g]);
    pc.end = pc.start + len;
    // ---- empty expert: exact +0 over the tile (once, by half 0) -----------------
    if (len == 0) {
      if (half <= 0) zero_tile(p, pc.g, pc.tn, pc.tk);
      return;
    }
    const bool shrt = pc.tn >= p.tall;
    if (half >= 0) {
      // a short tile is not split: half 0 computes all of it
      if (shrt) {
        if (half == 0) run_piece<GROUP, false, false, BF, false, false, true, false, GUNAL>(p, sm, pc);
        return;
      }
      pc.half = half;
      run_piece<GROUP, false, false, BF, false, true, false, false, GUNAL>(p, sm, pc);
      return;
    }
    if (shrt)
      run_piece<GROUP, false, false, BF, false, false, true, false, GUNAL>(p, sm, pc);
    else
      run_piece<GROUP, false, false, BF, false, false, false, false, GUNAL>(p, sm, pc);
  } else {
    // ---- column mode: the pieces of this column, in sequence order -------------
    for (;;) {
      if (kx >= nne) break;
      const int it = __builtin_amdgcn_readfirstlane(sm.nit[kx]);
      const int cost = 4 * it + p.hov;
      const int a = Rg * __builtin_amdgcn_readfirstlane(sm.pre[kx]) + rx * cost;
      if (a >= x1) break;
      // iteration boundary of a sequence position, clamped to [0, it]
      const int lo = min(max((x0 - a + 2) >> 2, 0), it);
      const int hi = min(max((x1 - a + 2) >> 2, 0), it);
      Piece pc;
      pc.g = __builtin_amdgcn_readfirstlane(sm.ne[kx]);
      const int rcur = rx;
      if (++rx == Rg) {
        rx = 0;
        ++kx;
      }
      if (lo >= hi) continue;
      if (!region_tile(p.tilesN, p.tilesK, p.rband, rcur, member, pc.tn, pc.tk)) continue;
      const int es = __builtin_amdgcn_readfirstlane(sm.start[pc.g]);
      const int ee = es + __builtin_amdgcn_readfirstlane(sm.len[pc.g]);
      const int es0 = (es / kPair) * 2;
      pc.start = max(es, (es0 + 4 * lo) * kStep);
      pc.end = min(ee, (es0 + 4 * hi) * kStep);
      pc.role = lo > 0 ? 1 : (hi < it ? 2 : 0);
      pc.col = col;
      pc.member = member;
      pc.Q = Q;
      pc.ra_lin = a;
      pc.r_it = it;
      // the previous piece's stores have completed (vmcnt starts at 0) and its
      // LDS reads are done in every wave before new loads land
      wait_vm_all();
      __syncthreads();
      if (pc.tn >= p.tall)
        run_piece<GROUP, true, false, BF, false, false, true>(p, sm, pc);
      else
        run_piece<GROUP, true, false, BF>(p, sm, pc);
    }
  }
}

// Row-ragged grouped GEMM (the forward and data-gradient GEMMs of the layer):
// out[m][n] = sum_c A[m][c] B[g][n][c] for the rows m of expert g.  Expert
// g's rows [start_g, end_g) are cut into 256-row tiles (the last one
// partial), never crossing into another expert; work item t = (row tile,
// column tile) in expert order, column tile fastest.  XCD x (blocks x,
// x + 8, ...) takes a contiguous range of work items, so the column tiles of
// a row tile (sharing its A rows) and the row tiles of an expert (sharing its
// B) meet in one L2.  The grid is sized on the host for the most row tiles
// any offs can give (R / 256 + E); blocks past the actual count exit.
template <bool GROUP, bool WHOLE = false, bool WALIGN = false>
__global__ __launch_bounds__(kThreads, 1) void rows_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int E = p.E, R = p.R;
  const int bid = blockIdx.x;
  // ---- row windows from offs (clamped to [0, R], monotone) -------------------
  if (tid < E) {
    int e = min(max(p.offs[tid], 0), R);
    const int st = tid ? min(max(p.offs[tid - 1], 0), R) : 0;
    if (e < st) e = st;
    sm.start[tid] = st;
    sm.len[tid] = e - st;
  }
  __syncthreads();
  // ---- exclusive prefix of the experts' row-tile counts, in registers --------
  // Every wave computes it for itself (one scan per 64 experts), so no further
  // barrier and no LDS round trip stand between the windows and the tile.
  static_assert(MXW_MAX_EXPERTS <= 4 * 64, "at most four 64-expert chunks");
  int cst[4], cln[4], cpre[4];
  int total = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    cst[c] = cln[c] = cpre[c] = 0;
    if (64 * c < E) {
      const int e = 64 * c + lane;
      const int st = e < E ? sm.start[e] : 0;
      const int ln = e < E ? sm.len[e] : 0;
      const int ntl = (ln + kTile - 1) / kTile;
      const int inc = wave_scan_incl(ntl);
      cst[c] = st;
      cln[c] = ln;
      cpre[c] = total + inc - ntl;
      total += __builtin_amdgcn_readlane(inc, 63);
    }
  }
  const int tiles = total * p.tilesN;
  const int per = (tiles + 7) >> 3;  // work items per XCD
  const int t = (bid & 7) * per + (bid >> 3);
  if ((bid >> 3) >= per || t >= tiles) return;
  const int mt = t / p.tilesN, nt = t - mt * p.tilesN;
  // the expert whose row tiles hold mt: the last non-empty one starting at or
  // before it, and its window and prefix, read from the lane that holds them
  int g = 0, gs = 0, gl = 0, gp = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (64 * c < E) {
      const uint64_t bal = __ballot(64 * c + lane < E && cln[c] > 0 && cpre[c] <= mt);
      if (bal) {
        const int l = 63 - (int)__builtin_clzll(bal);
        g = 64 * c + l;
        gs = __builtin_amdgcn_readlane(cst[c], l);
        gl = __builtin_amdgcn_readlane(cln[c], l);
        gp = __builtin_amdgcn_readlane(cpre[c], l);
      }
    }
  }
  Piece pc = {};
  pc.g = g;
  pc.tn = mt;
  pc.tk = nt;
  pc.start = 0;
  pc.end = p.M;
  pc.ar0 = gs + (mt - gp) * kTile;
  pc.ra = min(kTile, gs + gl - pc.ar0);
  run_piece<GROUP, false, true, false, WHOLE, false, false, WALIGN>(p, sm, pc);
}

// ---- token-axis MXFP8 quantiser --------------------------------------------------
// bf16 x [M, H] (tokens x hidden, hidden contiguous) -> E4M3 codes q [H, M]
// (token-contiguous) and E8M0 scales s [H, M/32], the operand layout of the
// weight gradient (blog section 1).  Per (hidden column h, 32-token block):
// amax over the block (tokens at or past `used` count as 0 and get code 0),
// scale byte clamp(floor(log2 amax) - 8 + 127, 0, 254) (127 for amax = 0),
// codes = E4M3 round-to-nearest-even of x / 2^(byte - 127), saturated to
// +-448, zero always encoded as +0.  HBM-bound: each element is read once
// (2 bytes) and written once (1 byte plus 1/32 of a scale byte).
//
// A workgroup takes a tile of 128 tokens x 64 hidden: coalesced 16-byte
// loads of the token rows (128 bytes each, one line) into LDS; thread (h, b)
// reduces and encodes hidden column h of 32-token block b straight from LDS
// (the 64 lanes of a wave read one 128-byte row segment at a time); the codes
// then overwrite the tile in LDS as 64 hidden rows of 128 bytes, 16-byte chunk
// c of row r at position c ^ ((r / 2) % 8) (the 16-byte writes of 16 lanes,
// rows r .. r+15 at one chunk, then hit 16 distinct bank groups), so that
// every global store writes whole 128-byte lines of q.
// Per-call scale pre-shuffle for the weight gradient (blog section 5.6 names
// a per-call scale pre-shuffle; this one exists for the memory path).  In the
// caller's planes [R, M/32] a workgroup's 16-byte group of 8 K-steps sits in
// 256 different rows, so each scale load of the K-loop touches 64 cache lines
// per wave for 1 KiB (its data loads touch 8), and the address unit and the L1
// fill path pay per line: measured, that costs the weight gradient ~6% at the
// 16B shape.  Rewritten as [band b = r / 256][group G][r % 256][16 bytes],
// the same loads read 1 KiB of consecutive bytes.  Rows past R, bytes past
// M/32 and the sub-blocks of tokens past offs[E-1] (padding, which may hold
// 0xFF = NaN scales; past the largest offs value, so that malformed offs
// still keep every window's scales) become 0.  One workgroup per (operand,
// band, 8 groups):
// each wave reads 8 rows x 128 bytes at a time (consecutive lanes, consecutive
// bytes) and writes, per group, 8 rows x 16 bytes contiguous.
struct ShufArgs {
  const uint8_t* s[2];  // A, B scale planes [R, M/32]
  uint8_t* out[2];
  int R[2];             // rows of A, B
  int bands[2];         // ceil(R / 256)
  int tall[2];          // 256-row bands; bands b >= tall start at 256 tall + 192 (b - tall)
  int M, groups, octets;
  int sstride;  // bytes from one scale row to the next (ld / 32)
  const int32_t* offs;
  int E;
  // column mode's arrival counters, cleared here for the main kernel that
  // follows on the stream (nullptr when it does not run in column mode)
  uint32_t* flags;
  int nflags;
};

__global__ __launch_bounds__(256) void scale_shuffle_kernel(ShufArgs a) {
  int blk = blockIdx.x;
  if (blk == 0 && a.flags)
    for (int i = (int)threadIdx.x; i < a.nflags; i += 256) a.flags[i] = 0u;
  const int op = blk >= a.bands[0] * a.octets;
  if (op) blk -= a.bands[0] * a.octets;
  const int b = blk / a.octets, o = blk - b * a.octets;
  const uint32_t sb = (uint32_t)a.sstride;  // bytes from one row to the next
  const int R = a.R[op];
  // tokens past the largest clamped offs belong to no expert's window
  // (offs[E-1] when offs is well formed)
  __shared__ int used_max;
  if (threadIdx.x == 0) used_max = 0;
  __syncthreads();
  for (int g = (int)threadIdx.x; g < a.E; g += 256) atomicMax(&used_max, min(max(a.offs[g], 0), a.M));
  __syncthreads();
  const int qlim = used_max >> 5;  // sub-blocks (bytes) of a row that may belong to an expert
  // this band's rows of the plane, the size rounded up to a dword (offsets
  // below are dword-aligned from this base: every dword is entirely inside
  // or outside the checked range)
  // the band of a short tile holds its 192 rows (the rest of its 256 are zero)
  const int tall = a.tall[op];
  const int r0 = b < tall ? b * kTile : tall * kTile + (b - tall) * kShort;
  const int rows = min(b < tall ? kTile : kShort, R - r0);
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(a.s[op] + (size_t)r0 * sb, ((uint32_t)rows * sb + 3u) & ~3u);
  auto keep_bytes = [](uint32_t x, int keep) { return keep >= 4 ? x : (keep <= 0 ? 0u : x & ((1u << (8 * keep)) - 1u)); };
  if ((sb & 15u) == 0) {
    // 16-byte aligned rows (ld % 512 == 0): one load per chunk, all eight in
    // flight before any store (the compiler cannot tell the buffer loads from
    // the global stores, so a load-store loop would wait out each load)
    v4i v[8];
    int nv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i * 256 + (int)threadIdx.x;  // chunk: row c / 8, group 8 o + c % 8
      const int r = c >> 3, G = 8 * o + (c & 7), q0 = 16 * G;
      nv[i] = (r < rows && G < a.groups) ? min(max(qlim - q0, 0), 16) : 0;
      const uint32_t off = nv[i] > 0 ? (uint32_t)r * sb + (uint32_t)q0 : kOob;
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i * 256 + (int)threadIdx.x;
      const int r = c >> 3, G = 8 * o + (c & 7);
      if (G >= a.groups) continue;
      const v4i w = {(int)keep_bytes((uint32_t)v[i].x, nv[i]), (int)keep_bytes((uint32_t)v[i].y, nv[i] - 4),
                     (int)keep_bytes((uint32_t)v[i].z, nv[i] - 8), (int)keep_bytes((uint32_t)v[i].w, nv[i] - 12)};
      *(v4i*)(a.out[op] + (((size_t)b * a.groups + G) * kTile + r) * 16) = w;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = i * 256 + (int)threadIdx.x;  // chunk: row c / 8, group 8 o + c % 8
    const int r = c >> 3, G = 8 * o + (c & 7);
    if (G >= a.groups) continue;
    const int q0 = 16 * G;  // first sub-block of the chunk
    const int nvalid = r < rows ? min(max(qlim - q0, 0), 16) : 0;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (nvalid > 0) {
      const uint32_t off = (uint32_t)r * sb + (uint32_t)q0;
      // unaligned rows: the 5 dwords around the chunk, funnel-shifted
      const uint32_t al = off & ~3u, sh = (off & 3u) * 8u;
      uint32_t v[5];
#pragma unroll
      for (int d = 0; d < 5; ++d) v[d] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, (int)(al + 4u * d), 0, 0);
#pragma unroll
      for (int d = 0; d < 4; ++d) w[d] = keep_bytes(__builtin_amdgcn_alignbit(v[d + 1], v[d], sh), nvalid - 4 * d);
    }
    *(v4i*)(a.out[op] + (((size_t)b * a.groups + G) * kTile + r) * 16) = (v4i){(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
  }
}

// Clears column mode's arrival counters before a launch that has no scale
// pre-shuffle to do it (the bf16 weight gradient).
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int n) {
  for (int i = (int)threadIdx.x; i < n; i += 256) p[i] = 0u;
}

constexpr int kQTok = 256, kQHid = 64;
// The codes overwrite the bf16 tile once every thread holds its encoded
// blocks in registers: 32 KiB per workgroup, 5 workgroups per CU.  (256
// tokens per tile rather than 128: +2.1% at the 16B shape, +2.6% at 671B.)
union QSmem {
  uint16_t x[kQTok][kQHid];  // the bf16 tile, token rows (32 KiB)
  uint8_t q[kQHid][kQTok];   // the codes, hidden rows, swizzled chunks (16 KiB)
};

__global__ __launch_bounds__(256) void quant_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ offs,
                                                    int E, int M, int ld, int H, uint8_t* __restrict__ q,
                                                    uint8_t* __restrict__ s) {
  __shared__ __attribute__((aligned(16))) QSmem sm;
  __shared__ uint2 sbw[kQHid];  // the 8 scale bytes of each hidden row
  const int tid = threadIdx.x;
  // Workgroups are dealt to the 8 XCDs in turn. Each XCD gets one contiguous
  // run of tiles (token tiles fastest), so the 16 token tiles whose scale
  // bytes share a 128-byte line of s write it through one L2, which writes
  // it back whole rather than as up to 8 partly dirty copies (+5% at 671B,
  // +6% at the 16B shape, against tiles in launch order).
  const uint32_t gx = gridDim.x, nt = gx * gridDim.y, lin = blockIdx.y * gx + blockIdx.x;
  const uint32_t xc = lin & 7, per = nt >> 3, tile = xc * per + min(xc, nt & 7) + (lin >> 3);
  const int m0 = (int)(tile % gx) * kQTok, h0 = (int)(tile / gx) * kQHid;
  int used = M;
  if (offs) used = min(max(offs[E - 1], 0), M);
  used = __builtin_amdgcn_readfirstlane(used);
  // ---- load: chunk c = 256 k + tid is token row c / 8, hidden h0 + 8 (c % 8)
  // (one 128-byte line per row); rows at or past `used` are outside the
  // descriptor's range and read as 0. Non-temporal (each line is read once):
  // +1% at the 16B shape, +4% at 671B.
  {
    const int rows = max(0, min(kQTok, used - m0));
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (size_t)m0 * H, (uint32_t)rows * (uint32_t)H * 2u);
    v4i v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = k * 256 + tid, r = c >> 3, h = h0 + (c & 7) * 8;
      const uint32_t off = h < H ? ((uint32_t)r * (uint32_t)H + (uint32_t)h) * 2u : kOob;
      v[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 2);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = k * 256 + tid;
      *(v4i*)&sm.x[c >> 3][(c & 7) * 8] = v[k];
    }
  }
  __syncthreads();
  // ---- encode: thread (h, b) does column h of 32-token blocks b and b + 4 ----
  {
    const int h = tid & 63, b = tid >> 6;
    uint32_t wq[2][8];
    int sbp[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int bb = b + 4 * p;
      float v[32];
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        v[i] = __builtin_bit_cast(float, (uint32_t)sm.x[bb * 32 + i][h] << 16);
        amax = fmaxf(amax, fabsf(v[i]));
      }
      // floor(log2 amax) = frexp exponent - 1 (exact, subnormals included)
      int sb = amax == 0.0f ? 127 : __builtin_amdgcn_frexp_expf(amax) - 1 - 8 + 127;
      sb = min(max(sb, 0), 254);
      sbp[p] = sb;
      const int sh = 127 - sb;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float y[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) y[t] = fminf(fmaxf(__builtin_ldexpf(v[4 * j + t], sh), -448.0f), 448.0f);
        int c = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        c = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], c, true);
        // a code of magnitude 0 (including -0) becomes +0
        const uint32_t z = (uint32_t)c & 0x7F7F7F7Fu;
        const uint32_t nz = ((z + 0x7F7F7F7Fu) & 0x80808080u) >> 7;
        wq[p][j] = (uint32_t)c & (nz * 0xFFu);
      }
    }
    __syncthreads();  // every thread has read its columns of the bf16 tile
    // 256-byte code rows span all 64 banks: chunk c of row h sits at c ^ (h % 16)
    const int sw = h & 15;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int bb = b + 4 * p;
      *(v4i*)&sm.q[h][((2 * bb) ^ sw) * 16] = (v4i){(int)wq[p][0], (int)wq[p][1], (int)wq[p][2], (int)wq[p][3]};
      *(v4i*)&sm.q[h][((2 * bb + 1) ^ sw) * 16] = (v4i){(int)wq[p][4], (int)wq[p][5], (int)wq[p][6], (int)wq[p][7]};
      ((uint8_t*)sbw)[h * 8 + bb] = (uint8_t)sbp[p];
    }
  }
  __syncthreads();
  // ---- scales: where the tile is whole, one 8-byte store per hidden row if
  // the row's 8 bytes are 8-byte aligned, two 4-byte stores if they are
  // 4-byte aligned (rows ld = M + 128 tokens apart), else byte stores (byte
  // stores from the waves, at 128-token tiles, measured 3 to 6% slower than
  // one store)
  if (tid < kQHid && h0 + tid < H) {
    uint8_t* srow = s + (size_t)(h0 + tid) * (size_t)(ld >> 5) + (m0 >> 5);
    const uint32_t mis = (uint32_t)(((uintptr_t)s) | (uintptr_t)(ld >> 5));
    if (m0 + kQTok <= M && (mis & 7) == 0) {
      *(uint2*)srow = sbw[tid];
    } else if (m0 + kQTok <= M && (mis & 3) == 0) {
      ((uint32_t*)srow)[0] = sbw[tid].x;
      ((uint32_t*)srow)[1] = sbw[tid].y;
    } else {
      for (int b = 0; b < 8 && m0 + 32 * b < M; ++b) srow[b] = ((const uint8_t*)sbw)[tid * 8 + b];
    }
  }
  // ---- store: chunk c = 256 k + tid is hidden row c / 16, tokens 16 (c % 16) .. +15
  // (non-temporal: the codes are not read again by this kernel, and keeping
  // them out of the L2 leaves it to the input rows: +4.0% at the 16B shape,
  // +1.2% at 671B, same bytes)
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = k * 256 + tid, r = c >> 4, c16 = c & 15;
    const int h = h0 + r, m = m0 + c16 * 16;
    if (h < H && m < M) __builtin_nontemporal_store(*(const v4i*)&sm.q[r][(c16 ^ (r & 15)) * 16], (v4i*)(q + (size_t)h * ld + m));
  }
}

struct DeviceInfo {
  std::atomic<int> state;  // 0: not read yet, 1: gfx950, 2: another device
  int cus;                 // compute units (written before state)
};
DeviceInfo g_dev[64];
std::mutex g_dev_mutex;  // taken only by the first check of a device

// Reads device properties once per device (no allocation, no stream work);
// after that a check is one atomic load, so calls take no lock.
int check_device(int* cus = nullptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MXW_ERR_DEVICE;
  DeviceInfo& d = g_dev[dev];
  int st = d.state.load(std::memory_order_acquire);
  if (st == 0) {
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    st = d.state.load(std::memory_order_relaxed);
    if (st == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MXW_ERR_DEVICE;
      d.cus = prop.multiProcessorCount;
      st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
      d.state.store(st, std::memory_order_release);
    }
  }
  if (cus) *cus = d.cus;
  return st == 1 ? MXW_OK : MXW_ERR_DEVICE;
}

// whether an E4M3 weight-gradient call with a workspace pre-shuffles its
// scales for (E, M) and row stride ld
bool uses_scale_shuffle(int E, int M, int ld) { return (int64_t)M >= (int64_t)kShufTokens * E; }

// One workgroup per tile (operands and scales read from the caller's buffers): how
// many of the last tiles of the dealing (the shortest experts', longest
// first) run as two half tiles.  When the tiles fill the device only a few
// times over, the last round leaves compute units idle; with short experts
// (at most 2,048 tokens per expert on average), where a tile's fixed costs
// are a large share of it, the tiles of that round are split, so it has twice
// as many workgroups of a little over half the length: +4.0% and +4.8% at
// 1,024 tokens per expert (measured interleaved, same bits).  At long experts
// the halves' fragment-read-bound K-loop loses (up to -7% at 24,576), so they
// stay whole.
int tail_split(int64_t tiles, int cus, int E, int M) {
  if (tiles <= cus || tiles >= 4LL * cus || (int64_t)M > 2048LL * E) return 0;
  return (int)(tiles % cus);
}

// Columns of a column-mode launch (0: one workgroup per work item) and the
// regions per expert.  Column mode when the work items fill the chip only a
// few times over (whole tiles then pack unevenly onto the compute units) and
// experts are long enough to amortise the per-piece costs; it needs whole
// 8-column groups (one column per XCD each), a column mask of at most 64
// columns and a work sequence that fits in int.
// Tile rows per band of column mode's regions (region_tile): the H in
// {4, 8, 2} whose regions leave the fewest members without a tile, 4 (the
// squarest regions) on ties.  (16 x 6 tiles: 4-row bands make two 4 x 4 and
// two 4 x 2 regions per 8 rows, a third of the members idle in the latter;
// 8-row bands make three full 8 x 2 regions.)
int region_band(int tN, int tK, int* regions) {
  int best = 0, idle_best = 1 << 30, r_best = 0;
  for (const int H : {4, 8, 2}) {
    const int full = tN / H, h = tN - H * full, wf = kMem / H;
    const int rpf = (tK + wf - 1) / wf;
    int R = full * rpf, idle = full * (rpf * kMem - H * tK);
    if (h) {
      const int w = kMem / h, rl = (tK + w - 1) / w;
      R += rl;
      idle += rl * kMem - h * tK;
    }
    if (idle < idle_best) {
      idle_best = idle;
      best = H;
      r_best = R;
    }
  }
  *regions = r_best;
  return best;
}

int plan_columns(int E, int M, int N, int K, int cus, int* regions, int* rband = nullptr) {
  const int tN = (N + kTile - 1) / kTile, tK = (K + kTile - 1) / kTile;
  int R = 0;
  const int H = region_band(tN, tK, &R);
  *regions = R;
  if (rband) *rband = H;
  const int ncol = (cus / kMem) & ~7;
  const int64_t items = (int64_t)E * tN * tK;
  const int64_t wmax = (int64_t)R * (4 * ((int64_t)M / 256 + 2 * E) + (int64_t)E * kColHov);
  if (ncol >= 8 && ncol <= 64 && items <= (int64_t)kColWaves * cus && (int64_t)M >= (int64_t)kColTokens * E &&
      wmax < (1LL << 30))
    return ncol;
  return 0;
}

// Tiles along N of 256 rows in a weight-gradient launch; the rest (two) are
// short tiles of 192 rows.  With N % 256 == 128 the last 384 rows are two
// short tiles rather than a whole tile and one with half its rows past N (whose
// MFMAs would work on nothing): the same tile count, a quarter less MFMA work
// per short tile.
int short_tiles_from(int N) {
  const int tN = (N + kTile - 1) / kTile;
  return (N % kTile == kTile / 2 && tN >= 2) ? tN - 2 : tN;
}

constexpr size_t kWsAlign = 4096;
size_t round_ws(size_t x) { return (x + kWsAlign - 1) & ~(kWsAlign - 1); }

// The plan of one weight-gradient launch.  Without a workspace: one workgroup
// per (expert, tile), scales read from the caller's planes.  With one (the
// _ws entry points): column mode and the scale pre-shuffle where they pay,
// their buffers carved from the workspace as
//   [arrival counters: ncol * kMem words][FP32 partial tiles: ncol * 2 * kMem
//    * 256 KiB][shuffled scale planes of A, then of B]
// each part starting on a 4 KiB boundary.
struct Plan {
  int ncol, regions, rband;
  bool shuffle;
  int sgroups;
  size_t flags_off, part_off, scaleA_off, scaleB_off, bytes;
};

Plan make_plan(int E, int Mb, int ldb, int tshift, int N, int K, int cus, bool ws) {
  Plan pl = {};
  const int tN = (N + kTile - 1) / kTile, tK = (K + kTile - 1) / kTile;
  if (!ws) {
    int regions = 0;
    (void)plan_columns(E, Mb, N, K, cus, &regions, &pl.rband);
    pl.regions = regions;
    return pl;
  }
  pl.ncol = plan_columns(E, Mb, N, K, cus, &pl.regions, &pl.rband);
  pl.shuffle = tshift == 0 && uses_scale_shuffle(E, Mb, ldb);
  size_t off = 0;
  if (pl.ncol) {
    pl.flags_off = off;
    off = round_ws(off + (size_t)pl.ncol * kMem * sizeof(uint32_t));
    pl.part_off = off;
    off = round_ws(off + (size_t)pl.ncol * 2 * kMem * kTile * kTile * sizeof(float));
  }
  if (pl.shuffle) {
    pl.sgroups = (Mb + 511) / 512 > 0 ? (Mb + 511) / 512 : 1;
    pl.scaleA_off = off;
    off = round_ws(off + (size_t)tN * pl.sgroups * kTile * 16);
    pl.scaleB_off = off;
    off = round_ws(off + (size_t)tK * pl.sgroups * kTile * 16);
  }
  pl.bytes = off;
  return pl;
}

// Bytes of workspace a _ws call of this shape needs on the current device
// (0: none), or a negative MXW_ERR_* code.
int64_t wgrad_ws_bytes(int E, int Mb, int ldb, int tshift, int N, int K) {
  int cus = 0;
  const int rc = check_device(&cus);
  if (rc) return rc;
  return (int64_t)make_plan(E, Mb, ldb, tshift, N, K, cus, true).bytes;
}

// One weight-gradient launch (E4M3 operands with scales when tshift = 0,
// bf16 operands when tshift = 1).  Mb: bytes of the token axis of A and B,
// ldb: bytes from one of their rows to the next (>= Mb).  use_ws:
// the _ws plan on workspace ws of ws_bytes bytes; otherwise the plain plan,
// which touches no memory but the operands and out.  Sizes and operand
// pointers are validated by the caller.
int launch_wgrad(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, const int32_t* offs,
                 int E, int Mb, int ldb, int tshift, int N, int K, uint16_t* out, bool use_ws, void* ws,
                 size_t ws_bytes, void* stream) {
  const int64_t grid = (int64_t)E * ((N + kTile - 1) / kTile) * ((K + kTile - 1) / kTile);
  if (grid <= 0 || grid * kThreads > 0xFFFFFFFFLL) return MXW_ERR_DIM;
  int cus = 0;
  int rc = check_device(&cus);
  if (rc) return rc;
  const Plan pl = make_plan(E, Mb, ldb, tshift, N, K, cus, use_ws);
  if (use_ws && pl.bytes) {
    if (!ws || ws_bytes < pl.bytes || ((uintptr_t)ws & 255)) return MXW_ERR_WORKSPACE;
  }
  uint8_t* wsb = (uint8_t*)ws;
  Params p = {};
  p.A = A;
  p.sA = sA;
  p.B = B;
  p.sB = sB;
  p.offs = offs;
  p.out = out;
  p.E = E;
  p.M = Mb;
  p.ld = ldb;
  p.N = N;
  p.K = K;
  p.tshift = tshift;
  p.tilesN = (N + kTile - 1) / kTile;
  p.tall = short_tiles_from(N);
  p.tilesK = (K + kTile - 1) / kTile;
  // XCD regions: split the tile grid a x b = 8 ways into equal rectangles,
  // the most square split (fewest distinct A + B stripes per rectangle)
  p.regN = p.regK = p.regB = p.band = 0;
  int best = 1 << 30;
  for (int a = 1; a <= 8; a *= 2) {
    const int b = 8 / a;
    if (p.tilesN % a || p.tilesK % b) continue;
    const int rn = p.tilesN / a, rk = p.tilesK / b;
    if (rn + rk < best) {
      best = rn + rk;
      p.regN = rn;
      p.regK = rk;
      p.regB = b;
    }
  }
  if (p.regN) {
    // about 32 co-resident workgroups per XCD: bands of ~32 / regK rows
    p.band = (32 + p.regK - 1) / p.regK;
    if (p.band > p.regN) p.band = p.regN;
  }
  p.hov = kColHov;
  p.regions = pl.regions;
  p.rband = pl.rband;
  p.ncol = pl.ncol;
  if (pl.ncol) {
    p.flags = (uint32_t*)(wsb + pl.flags_off);
    p.part = (float*)(wsb + pl.part_off);
  }
  // one workgroup per tile with operands (and scales) read from the caller's
  // buffers: the last tiles of the dealing as half tiles (blocks [nfull, grid))
  const int nsplit = (!pl.ncol && !pl.shuffle) ? tail_split(grid, cus, E, Mb >> tshift) : 0;
  p.nfull = (int)grid - nsplit;
  // a launch with half tiles keeps whole 256-row tiles: a short tile cannot be
  // halved, and run whole in the last round it delays the round
  if (nsplit) p.tall = p.tilesN;
  const dim3 g((unsigned)(pl.ncol ? pl.ncol * kMem : grid + nsplit)), blk(kThreads);
  hipStream_t st = (hipStream_t)stream;
  if (tshift) {
    // bf16: no scales; column mode's counters are cleared by a first kernel
    if (pl.ncol) {
      hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(256), 0, st, p.flags, pl.ncol * kMem);
      hipLaunchKernelGGL((wgrad_kernel<false, true, true>), g, blk, 0, st, p);
    } else {
      hipLaunchKernelGGL((wgrad_kernel<false, false, true>), g, blk, 0, st, p);
    }
  } else if (!pl.shuffle) {
    // the caller's scale planes, 16-byte groups of 8 K-steps per row: from the
    // row's own offset when scale rows are a whole number of dwords (ld % 128
    // == 0; the 16-byte LDS-direct loads then start on 4-byte boundaries,
    // which they take, the range check working per dword), else from the
    // dword boundary below it, each scale word then joined from two
    // consecutive dwords (GUNAL).  (Column mode always shuffles: it needs
    // M >= 8192 E.)
    p.sAs = p.sBs = nullptr;
    p.sgroups = 0;
    if (pl.ncol) return MXW_ERR_DIM;  // unreachable by construction of the plan
    if ((ldb & 127) == 0) hipLaunchKernelGGL((wgrad_kernel<true, false>), g, blk, 0, st, p);
    else hipLaunchKernelGGL((wgrad_kernel<true, false, false, true>), g, blk, 0, st, p);
  } else {
    // long experts (M >= 4096 E): rewrite the scale planes into the workspace
    // so that the K-loop's grouped scale loads read consecutive bytes (the same
    // kernel clears column mode's counters); at short experts the extra pass
    // costs more than the scattered scale loads do (~4 us against ~1 us at
    // 1,024 tokens per expert, whatever the row alignment)
    ShufArgs sa;
    sa.s[0] = sA;
    sa.s[1] = sB;
    sa.R[0] = N;
    sa.R[1] = K;
    sa.bands[0] = p.tilesN;
    sa.bands[1] = p.tilesK;
    sa.tall[0] = p.tall;
    sa.tall[1] = p.tilesK;
    sa.M = Mb;
    sa.sstride = ldb >> 5;
    sa.groups = pl.sgroups;
    sa.octets = (sa.groups + 7) / 8;
    sa.offs = offs;
    sa.E = E;
    sa.out[0] = wsb + pl.scaleA_off;
    sa.out[1] = wsb + pl.scaleB_off;
    sa.flags = p.flags;
    sa.nflags = pl.ncol * kMem;
    p.sAs = sa.out[0];
    p.sBs = sa.out[1];
    p.sgroups = sa.groups;
    hipLaunchKernelGGL(scale_shuffle_kernel, dim3((unsigned)((sa.bands[0] + sa.bands[1]) * sa.octets)), dim3(256), 0, st,
                       sa);
    if (pl.ncol) hipLaunchKernelGGL((wgrad_kernel<true, true>), g, blk, 0, st, p);
    else hipLaunchKernelGGL((wgrad_kernel<true, false>), g, blk, 0, st, p);
  }
  if (hipGetLastError() != hipSuccess) return MXW_ERR_LAUNCH;
  return MXW_OK;
}

// The no-allocation entry point's scratch: the workspace of a _ws call, held
// in a static device array instead (each device the library runs on holds
// its own copy until the process ends).  Its host-side name is not a device
// address: host code uses only the address hipGetSymbolAddress returns for
// the current device, looked up once per device.
static_assert(MXW_SCRATCH_BYTES % kWsAlign == 0, "scratch size");
__device__ __align__(256) uint8_t scratch[MXW_SCRATCH_BYTES];
void* g_scratch[64];
std::mutex g_scratch_mutex;

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MXW_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MXW_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MXW_OK;
}

int check_wgrad_args(const void* A, const void* sA, const void* B, const void* sB, const void* offs, const void* out,
                     int E, int M, int N, int K, bool bf, int ld = -1) {
  if (!A || (!bf && !sA) || !B || (!bf && !sB) || !offs || !out) return MXW_ERR_NULL;
  const int mmax = bf ? MXW_MAX_TOKENS / 2 : MXW_MAX_TOKENS;
  const int mal = bf ? 15 : 31;
  if (E < 1 || E > MXW_MAX_EXPERTS || M < 0 || M > mmax || (M & mal) || N < 16 || K < 16 || (N & 15) ||
      (K & 15) || N > 65536 || K > 65536)
    return MXW_ERR_DIM;
  if (ld >= 0 && (ld < M || ld > MXW_MAX_TOKENS || (ld & 31))) return MXW_ERR_DIM;
  if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)out) & 15) return MXW_ERR_ALIGN;
  if (!bf && (((uintptr_t)sA | (uintptr_t)sB) & 3)) return MXW_ERR_ALIGN;
  return MXW_OK;
}

}  // namespace

extern "C" {

int mxw_columns(int E, int M, int N, int K) {
  if (E < 1 || E > MXW_MAX_EXPERTS || M < 0 || M > MXW_MAX_TOKENS || N < 16 || K < 16) return MXW_ERR_DIM;
  int cus = 0;
  const int rc = check_device(&cus);
  if (rc) return rc;
  int regions = 0;
  return plan_columns(E, M, N, K, cus, &regions);
}

int mxw_tail_split(int E, int M, int N, int K) {
  if (E < 1 || E > MXW_MAX_EXPERTS || M < 0 || M > MXW_MAX_TOKENS || (M & 31) || N < 16 || K < 16) return MXW_ERR_DIM;
  int cus = 0;
  const int rc = check_device(&cus);
  if (rc) return rc;
  return tail_split((int64_t)E * ((N + kTile - 1) / kTile) * ((K + kTile - 1) / kTile), cus, E, M);
}

int mxw_scale_shuffle(int E, int M) {
  if (E < 1 || E > MXW_MAX_EXPERTS || M < 0 || M > MXW_MAX_TOKENS || (M & 31)) return MXW_ERR_DIM;
  return uses_scale_shuffle(E, M, M) ? 1 : 0;
}

int64_t mxw_grid_size(int E, int N, int K) {
  if (E < 1 || E > MXW_MAX_EXPERTS || N < 16 || K < 16) return 0;
  return (int64_t)E * ((N + kTile - 1) / kTile) * ((K + kTile - 1) / kTile);
}

int mxfp8_wgrad_grouped(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                        const int32_t* offs, int E, int M, int N, int K, uint16_t* out, void* stream) {
  const int rc = check_wgrad_args(A, sA, B, sB, offs, out, E, M, N, K, false);
  if (rc) return rc;
  return launch_wgrad(A, sA, B, sB, offs, E, M, M, 0, N, K, out, false, nullptr, 0, stream);
}

int64_t mxfp8_wgrad_workspace_size(int E, int M, int ld, int N, int K) {
  if (ld == 0) ld = M;
  if (E < 1 || E > MXW_MAX_EXPERTS || M < 0 || M > MXW_MAX_TOKENS || (M & 31) || N < 16 || K < 16 || (N & 15) ||
      (K & 15) || N > 65536 || K > 65536 || ld < M || ld > MXW_MAX_TOKENS || (ld & 31))
    return MXW_ERR_DIM;
  return wgrad_ws_bytes(E, M, ld, 0, N, K);
}

int mxfp8_wgrad_grouped_ws(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                           const int32_t* offs, int E, int M, int ld, int N, int K, uint16_t* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (ld == 0) ld = M;
  const int rc = check_wgrad_args(A, sA, B, sB, offs, out, E, M, N, K, false, ld);
  if (rc) return rc;
  return launch_wgrad(A, sA, B, sB, offs, E, M, ld, 0, N, K, out, true, workspace, workspace_bytes, stream);
}

int mxfp8_wgrad_grouped_noalloc(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                                const int32_t* offs, int E, int M, int ld, int N, int K, uint16_t* out, void* stream) {
  if (ld == 0) ld = M;
  int rc = check_wgrad_args(A, sA, B, sB, offs, out, E, M, N, K, false, ld);
  if (rc) return rc;
  int cus = 0;
  rc = check_device(&cus);
  if (rc) return rc;
  if (make_plan(E, M, ld, 0, N, K, cus, true).bytes > (size_t)MXW_SCRATCH_BYTES) return MXW_ERR_SCRATCH;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  return launch_wgrad(A, sA, B, sB, offs, E, M, ld, 0, N, K, out, true, ws, MXW_SCRATCH_BYTES, stream);
}

int bf16_wgrad_grouped(const uint16_t* A, const uint16_t* B, const int32_t* offs, int E, int M, int N, int K,
                       uint16_t* out, void* stream) {
  const int rc = check_wgrad_args(A, nullptr, B, nullptr, offs, out, E, M, N, K, true);
  if (rc) return rc;
  // planned and run in bytes along the token axis: 2 M per row
  return launch_wgrad((const uint8_t*)A, nullptr, (const uint8_t*)B, nullptr, offs, E, 2 * M, 2 * M, 1, N, K, out,
                      false, nullptr, 0, stream);
}

int64_t bf16_wgrad_workspace_size(int E, int M, int N, int K) {
  if (E < 1 || E > MXW_MAX_EXPERTS || M < 0 || M > MXW_MAX_TOKENS / 2 || (M & 15) || N < 16 || K < 16 ||
      (N & 15) || (K & 15) || N > 65536 || K > 65536)
    return MXW_ERR_DIM;
  return wgrad_ws_bytes(E, 2 * M, 2 * M, 1, N, K);
}

int bf16_wgrad_grouped_ws(const uint16_t* A, const uint16_t* B, const int32_t* offs, int E, int M, int N, int K,
                          uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = check_wgrad_args(A, nullptr, B, nullptr, offs, out, E, M, N, K, true);
  if (rc) return rc;
  return launch_wgrad((const uint8_t*)A, nullptr, (const uint8_t*)B, nullptr, offs, E, 2 * M, 2 * M, 1, N, K, out,
                      true, workspace, workspace_bytes, stream);
}

int64_t mxw_fwd_grid_size(int E, int R, int N) {
  if (E < 1 || E > MXW_MAX_EXPERTS || R < 0 || R > MXW_MAX_ROWS || N < 16) return 0;
  const int64_t items = ((int64_t)R / kTile + E) * ((N + kTile - 1) / kTile);
  return ((items + 7) / 8) * 8;
}

int mxfp8_grouped_fwd(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                      const int32_t* offs, int E, int R, int C, int N, uint16_t* out, void* stream) {
  if (!A || !sA || !B || !sB || !offs || !out) return MXW_ERR_NULL;
  if (E < 1 || E > MXW_MAX_EXPERTS || R < 0 || R > MXW_MAX_ROWS || C < 32 || (C & 31) || C > 65536 || N < 16 ||
      (N & 15) || N > 65536)
    return MXW_ERR_DIM;
  if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)out) & 15) return MXW_ERR_ALIGN;
  if (((uintptr_t)sA | (uintptr_t)sB) & 3) return MXW_ERR_ALIGN;
  const int64_t grid = mxw_fwd_grid_size(E, R, N);
  if (grid <= 0 || grid * kThreads > 0xFFFFFFFFLL) return MXW_ERR_DIM;
  int rc = check_device();
  if (rc) return rc;
  Params p = {};
  p.A = A;
  p.sA = sA;
  p.B = B;
  p.sB = sB;
  p.offs = offs;
  p.out = out;
  p.E = E;
  p.M = C;  // the contraction length
  p.ld = C;  // and the row stride of A and B
  p.N = N;
  p.K = 0;
  p.R = R;
  p.tilesN = (N + kTile - 1) / kTile;
  p.tilesK = 0;
  if (C <= kWholeC && (C & 127) == 0)  // scale rows a whole number of dwords
    hipLaunchKernelGGL((rows_kernel<false, true, true>), dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream, p);
  else if (C <= kWholeC)
    hipLaunchKernelGGL((rows_kernel<false, true>), dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream, p);
  else if ((C & 127) == 0)  // 16-byte scale groups from dword-aligned rows
    hipLaunchKernelGGL((rows_kernel<true>), dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL((rows_kernel<false>), dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream, p);
  if (hipGetLastError() != hipSuccess) return MXW_ERR_LAUNCH;
  return MXW_OK;
}

int mxfp8_quantize_tokens(const uint16_t* x, const int32_t* offs, int E, int M, int ld, int H, uint8_t* q,
                          uint8_t* s, void* stream) {
  if (!x || !q || !s) return MXW_ERR_NULL;
  if (ld == 0) ld = M;
  if (M < 0 || M > MXW_MAX_TOKENS || (M & 31) || H < 16 || (H & 15) || H > 65536 ||
      (offs && (E < 1 || E > MXW_MAX_EXPERTS)) || ld < M || ld > MXW_MAX_TOKENS || (ld & 31))
    return MXW_ERR_DIM;
  if (((uintptr_t)x | (uintptr_t)q) & 15) return MXW_ERR_ALIGN;
  int rc = check_device();
  if (rc) return rc;
  if (M == 0) return MXW_OK;
  const dim3 grid((unsigned)((M + kQTok - 1) / kQTok), (unsigned)((H + kQHid - 1) / kQHid));
  hipLaunchKernelGGL(quant_kernel, grid, dim3(256), 0, (hipStream_t)stream, x, offs, E, M, ld, H, q, s);
  if (hipGetLastError() != hipSuccess) return MXW_ERR_LAUNCH;
  return MXW_OK;
}

const char* mxw_strerror(int code) {
  switch (code) {
    case MXW_OK: return "ok";
    case MXW_ERR_NULL: return "a required pointer is NULL";
    case MXW_ERR_DIM: return "a size (E, M, N, K, R or C) outside the supported range";
    case MXW_ERR_ALIGN: return "A, B or out is not 16-byte aligned, or sA or sB not 4-byte aligned";
    case MXW_ERR_DEVICE: return "the current device is not gfx950 (or no device)";
    case MXW_ERR_LAUNCH: return "kernel launch failed";
    case MXW_ERR_WORKSPACE: return "workspace missing, smaller than the size query returned, or not 256-byte aligned";
    case MXW_ERR_SCRATCH: return "the shape needs more workspace than the library's static scratch (MXW_SCRATCH_BYTES)";
    default: return "unknown error";
  }
}

int mxw_version(void) { return 500; }

}  // extern "C"
