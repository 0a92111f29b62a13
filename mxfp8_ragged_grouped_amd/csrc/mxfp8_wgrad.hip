// mxfp8_wgrad.hip -- MXFP8 ragged weight-gradient grouped GEMM for MI355X
// (gfx950), and its C ABI (declared in include/mxfp8_wgrad.h).
//
// dW[g][n][k] = sum over expert g's tokens m of
//               e4m3(A[n][m]) 2^(sA[n][m/32]-127) * e4m3(B[k][m]) 2^(sB[k][m/32]-127)
// (blog "Ragged MXFP8 Weight Gradients: A FlyDSL Grouped GEMM on MI355X",
// section 1).  A = dY^T [N, M], B = X^T [K, M], token axis contiguous.
//
// Structure of one launch:
//   * grid = one 256-thread workgroup (4 wave64) per (expert, 256 x 256 output
//     tile); a workgroup owns its tile for life, walks its expert's tokens in
//     128-token K-steps, keeps the tile's 65,536 FP32 sums in accumulator
//     registers and stores once (blog section 4).  No atomics:
//     bit-reproducible.
//   * tile scheduler: every workgroup reads offs itself, ranks the experts by
//     window length with one lane per expert (longest first, ties to the lower
//     index; blog section 5.4), and numbers tiles so that the workgroups the
//     dispatcher deals to one XCD (block index mod 8, blog section 3) cover a
//     compact group of 2 x 2 supertiles of the same expert (blog section 5.5).
//   * staging: each K-step's operand stripes (256 rows x 128 tokens of A and
//     of B, 64 KiB) go HBM -> LDS with 16-byte LDS-direct buffer loads into a
//     ping-pong pair of stages (blog section 4); the 16-byte chunk c of row r
//     sits at position c ^ (r & 7), which makes the MFMA fragment reads free
//     of LDS bank conflicts on gfx950 (measured with SQ_LDS_BANK_CONFLICT).  Each wave pulls all
//     of a step's fragments into registers at the top of the step; a
//     mid-step barrier then frees the stage, which is refilled for the step
//     after next while this step's MFMAs run.  Up to two steps are in flight
//     while one computes (the blog's "refill as soon as read", section 4).
//   * ragged head/tail: a 32-token sub-block of a step is live iff it lies
//     inside [start, end) (group boundaries are 32-aligned, blog section 1).
//     Dead sub-blocks are removed twice: their data loads are pointed out of
//     the buffer range, so the hardware writes zeros (padding that holds NaN
//     never reaches the MFMA, blog section 5.3), and both operands' scales are
//     set to 0x00.
//   * scales: the raw E8M0 bytes arrive by LDS-direct loads and each thread
//     re-lays its row's 4 bytes of a step into MFMA-ready words (blog
//     sections 5.2 and 5.6): byte i of a word is 16-row tile i of one K-step,
//     picked by op_sel, so the MFMA loop reads two dwords per operand per step
//     and unpacks nothing.  When every row of the scale planes starts 16-byte
//     aligned (M a multiple of 512) one 16-byte load per row brings four
//     steps of scales into a double-buffered group area (GROUP = true);
//     otherwise each step loads its own 4-byte dword per row, three steps
//     ahead.  A scale dword per row per step would double the number of
//     L1 -> L2 requests of a step (every lane hits a different row), which
//     measurably slows the data stream; the grouped form issues 8x fewer.
//   * contraction: v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 x E4M3 with
//     per-32 E8M0 scales, FP32 accumulation (blog section 3).  Operand roles
//     are swapped (B feeds the instruction's first operand) so that each lane
//     ends with 4 consecutive k of one output row (ROCm/aiter PR 6605,
//     section 1).
//   * epilogue: FP32 -> bf16 round-to-nearest-even in registers, 8-byte
//     stores (blog section 5.5).
//
// MFMA lane layout used here (16x16x128, FP8 operands): lane l holds row
// l % 16 and tokens {16(l/16) + p : p < 16} in bytes 0..15 and
// {64 + 16(l/16) + p} in bytes 16..31 (two runs of 16, 64 apart, blog
// section 3); the scale word of lane l carries the E8M0 of row l % 16 and
// 32-token block l / 16; the result's lane l holds rows 4(l/16) .. 4(l/16)+3
// of column l % 16.
//
// Every global read in the K-loop is an LDS-direct load issued through asm,
// and the kernel waits on vmcnt itself: the compiler's wait insertion cannot
// tell the stages apart and would drain the prefetch before each LDS read.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "mxfp8_wgrad.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 256;                   // output tile edge, N and K
constexpr int kStep = 128;                   // tokens per K-step
constexpr int kThreads = 256;                // 4 wave64
constexpr int kRowBytes = kStep;             // one staged row = 128 E4M3 codes
constexpr int kOpBytes = kTile * kRowBytes;  // 32 KiB per operand per stage
constexpr uint32_t kOob = 0x80000000u;       // a buffer offset past any range used here
// DMA instructions per wave per batch of operand data: 8 row groups of A and
// of B.  Scale loads come on top (see the two scale paths below).
constexpr int kDataDma = 16;
// raw buffer descriptor word 3 for gfx9-family: 32-bit data format, no swizzle,
// range checking on the byte offset
constexpr int kRsrcWord3 = 0x00020000;

// LDS layout (152 KiB of the 160 KiB per CU).
struct Smem {
  // [stage][0 = A n-rows, 1 = B k-rows]: 256 rows x 128 tokens, chunk-swizzled
  uint8_t data[2][2][kOpBytes];
  // raw E8M0 scale bytes as loaded, 16 KiB, in one of two layouts:
  //  grouped (scale rows 16-byte aligned): [group % 2][op][row][4 dwords], the
  //    4 sub-block bytes of 4 consecutive K-steps of a row;
  //  per step (any row alignment): [step % 4][op][dword at floor4(addr), next][row]
  uint32_t raw[4096];
  // destination of the out-of-range scale-slot loads on steps that have no
  // scale group to fetch (always written with zeros, never read)
  uint32_t dummy[256];
  // MFMA-ready scale words [buf][op][(half * 64 + lane) * 2 + word]: byte i of
  // word w is 16-row tile 4w + i of that half's 128 rows, for sub-block
  // lane / 16 and row lane % 16
  uint32_t words[2][2][256];
  int start[MXW_MAX_EXPERTS];
  int len[MXW_MAX_EXPERTS];
  int order[MXW_MAX_EXPERTS];
};

__device__ __forceinline__ int swz(int row) { return row & 7; }

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

// counter waits (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; the counters not waited on are left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lgkm_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// live-sub-block mask of K-step s for window [start, end): bit b set iff tokens
// [128 s + 32 b, 128 s + 32 b + 32) lie inside the window.
__device__ __forceinline__ uint32_t live_mask(int s, int start, int end) {
  uint32_t m = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int t0 = s * kStep + 32 * b;
    m |= (uint32_t)(t0 >= start && t0 + 32 <= end) << b;
  }
  return m;
}

// byte mask with 0xFF in byte b iff bit b of the live mask is set
__device__ __forceinline__ uint32_t byte_mask(uint32_t live) {
  uint32_t m = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) m |= ((live >> b) & 1u) ? (0xFFu << (8 * b)) : 0u;
  return m;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 h = __builtin_convertvector(f, bf16x2);  // round-to-nearest-even
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

// v_mfma_scale_f32_16x16x128_f8f6f4 with E4M3 operands (format code 0) and the
// scale byte selectors as template constants.
template <int OA, int OB>
__device__ __forceinline__ v4f mfma_e4m3(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, OA, sa, OB, sb);
}

// same, selectors given as values that are constant after unrolling
__device__ __forceinline__ v4f mfma_e4m3_sel(int oa, int ob, const v8i& a, const v8i& b, const v4f& c, int sa,
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

// one MFMA operand fragment: the lane's two 16-byte runs of a 16-row tile
__device__ __forceinline__ v8i frag(const uint8_t* tile, int lo, int hi) {
  const v4i a = *(const v4i*)(tile + lo);
  const v4i b = *(const v4i*)(tile + hi);
  return (v8i){a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}

struct Params {
  const uint8_t* A;
  const uint8_t* sA;
  const uint8_t* B;
  const uint8_t* sB;
  const int32_t* offs;
  uint16_t* out;
  int E, M, N, K;
  int tilesN, tilesK;
  // XCD regions (0 = off): each expert's tilesN x tilesK grid is cut into 8
  // rectangles of regN x regK tiles, regB of them across the K direction;
  // rectangle x is walked in bands of `band` rows, column by column
  int regN, regK, regB, band;
};

// GROUP: scale rows are 16-byte aligned (M % 512 == 0) and scales are loaded
// 4 K-steps at a time; otherwise step by step.
template <bool GROUP>
__global__ __launch_bounds__(kThreads, 1) void wgrad_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = p.E, M = p.M, N = p.N, K = p.K;

  // ---- windows from offs (clamped to [0, M], monotone) ----------------------
  if (tid < E) {
    int e = min(max(p.offs[tid], 0), M);
    const int s = tid ? min(max(p.offs[tid - 1], 0), M) : 0;
    if (e < s) e = s;
    sm.start[tid] = s;
    sm.len[tid] = e - s;
  }
  __syncthreads();
  // ---- longest-first ranking: lane g counts the experts ahead of it ---------
  if (tid < E) {
    const int mine = sm.len[tid];
    int r = 0;
    for (int u = 0; u < E; ++u) {
      const int l = sm.len[u];
      r += (l > mine) || (l == mine && u < tid);
    }
    sm.order[r] = tid;
  }
  __syncthreads();

  // ---- block -> (expert rank d, tile) -> (expert g, tile tn, tk) -------------
  // The dispatcher deals block b to XCD b % 8 and each XCD starts its blocks in
  // order.  With regions, XCD x owns the same rectangle of every expert's tile
  // grid and works through the experts longest first, so its co-resident
  // workgroups cover a compact block of one expert's tiles and share their A
  // and B stripes in that XCD's L2.
  const int T = p.tilesN * p.tilesK;
  const int bid = blockIdx.x;
  int d, tn, tk;
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
    d = bid / T;
    const int u = bid - d * T;
    tn = u / p.tilesK;
    tk = u - tn * p.tilesK;
  }
  const int g = __builtin_amdgcn_readfirstlane(sm.order[d]);
  const int start = __builtin_amdgcn_readfirstlane(sm.start[g]);
  const int len = __builtin_amdgcn_readfirstlane(sm.len[g]);
  const int end = start + len;
  const int n0 = tn * kTile, k0 = tk * kTile;
  uint16_t* outg = p.out + (size_t)g * N * K;

  // ---- empty expert: exact +0 over the tile ----------------------------------
  if (len == 0) {
    const int rows = min(kTile, N - n0), cols = min(kTile, K - k0);
    const int chunks = cols / 8;  // 16-byte chunks per row (K % 16 == 0)
    const v4i z = {0, 0, 0, 0};
    for (int i = tid; i < rows * chunks; i += kThreads) {
      const int r = i / chunks, c = i - r * chunks;
      *(v4i*)(outg + (size_t)(n0 + r) * K + k0 + 8 * c) = z;
    }
    return;
  }

  // ---- buffer resources, rebased to this tile's 256-row bands ----------------
  const int rowsA = min(kTile, N - n0), rowsB = min(kTile, K - k0);
  const uint32_t sbytes = (uint32_t)M >> 5;  // scale bytes per row
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A + (size_t)n0 * M, (uint32_t)rowsA * (uint32_t)M);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.B + (size_t)k0 * M, (uint32_t)rowsB * (uint32_t)M);
  // scale planes are read as whole dwords; rounding the range up to 4 bytes
  // keeps every dword entirely inside or outside it (bytes past the plane
  // belong to tokens >= M, which are always masked)
  const __amdgpu_buffer_rsrc_t rsA =
      make_rsrc(p.sA + (size_t)n0 * sbytes, ((uint32_t)rowsA * sbytes + 3u) & ~3u);
  const __amdgpu_buffer_rsrc_t rsB =
      make_rsrc(p.sB + (size_t)k0 * sbytes, ((uint32_t)rowsB * sbytes + 3u) & ~3u);

  // ---- per-lane DMA geometry -------------------------------------------------
  // Data: wave w fills row groups 8w .. 8w+7 (8 rows x 128 B = 1 KiB each) of
  // both stripes.  Lane i of a group writes LDS bytes [16 i, 16 i + 16) of the
  // group: row i / 8, chunk position i % 8, which holds global chunk
  // (i % 8) ^ swz(row).
  const int lrow = lane >> 3;
  const int ch = (lane & 7) ^ swz(lrow);  // global chunk (row groups are 8-aligned)
  // Scales: lane l of wave w fetches scale row 64 w + l.
  const uint32_t srow_off = (uint32_t)(wave * 64 + lane) * sbytes;

  // data of step sdata into stage buf, load i of 16 (row group 8w + i/2 of A
  // for even i, of B for odd i); dead sub-blocks are forced out of range
  auto dma_data = [&](int i, int buf, int sdata, uint32_t live) {
    const int grp = wave * 8 + (i >> 1), op = i & 1;
    const int row = grp * 8 + lrow;
    const bool ok = (live >> (ch >> 1)) & 1u;
    const uint32_t va = ok ? (uint32_t)row * (uint32_t)M + (uint32_t)(ch * 16) : kOob;
    dma16(op ? rB : rA, __builtin_amdgcn_readfirstlane(lds_addr(&sm.data[buf][op][grp * 1024])), va,
          (uint32_t)(sdata * kStep));
  };

  // Scale loads.  A K-step needs 4 bytes of each of 512 rows; fetching them
  // step by step presents one cache line per row per step to the memory path,
  // as many requests as all of the step's operand data.  So when scale rows
  // are 16-byte aligned (M % 512 == 0) each row's 16 bytes of 4 consecutive
  // K-steps ("group" g = steps 4g .. 4g+3) come in one 16-byte load per lane,
  // 2 per wave per group, double-buffered by group parity.  Otherwise the
  // two dwords around each row's 4 bytes are fetched every step (4 loads per
  // wave per step, 4 buffers by step % 4).
  // GROUP layout; with real == false the load is out of range (no memory
  // traffic) and lands in the dummy area, so every step issues the same count
  auto dma_group = [&](int grp_idx, int op, bool real) {
    const uint32_t so = real ? srow_off + 16u * (uint32_t)grp_idx : kOob;
    const uint32_t dst = real ? lds_addr(&sm.raw[(((grp_idx & 1) * 2 + op) * kTile + wave * 64) * 4])
                              : lds_addr(&sm.dummy[0]);
    dma16(op ? rsB : rsA, __builtin_amdgcn_readfirstlane(dst), so, 0u);
  };
  auto dma_raw = [&](int sraw, int k) {  // per-step layout, k = A lo, A hi, B lo, B hi
    const uint32_t so = (srow_off & ~3u) + 4u * (uint32_t)sraw + 4u * (uint32_t)(k & 1);
    dma4((k >> 1) ? rsB : rsA,
         __builtin_amdgcn_readfirstlane(
             lds_addr(&sm.raw[(((sraw & 3) * 2 + (k >> 1)) * 2 + (k & 1)) * kTile + wave * 64])),
         so);
  };

  // Relayout of thread t's scale row (row t of A and of B) for step s into
  // words buffer wb: byte b (sub-block b) -> lane (t % 16) + 16 b of half
  // t / 128, word ((t % 128) / 16) / 4, byte ((t % 128) / 16) % 4.
  const int rh = tid >> 7, rt = (tid & 127) >> 4, rj = tid & 15;
  const int wbyte = ((rh * 64 + rj) * 2 + (rt >> 2)) * 4 + (rt & 3);  // + 128 per sub-block
  const uint32_t tshift = (((uint32_t)tid * sbytes) & 3u) * 8u;
  auto relayout = [&](int s, int wb) {
    const uint32_t bm = byte_mask(live_mask(s, start, end));
    uint32_t a, b;
    if (GROUP) {
      const int gb = (s >> 2) & 1, d = s & 3;
      a = sm.raw[((gb * 2 + 0) * kTile + tid) * 4 + d];
      b = sm.raw[((gb * 2 + 1) * kTile + tid) * 4 + d];
    } else {
      const int rb = s & 3;
      a = __builtin_amdgcn_alignbit(sm.raw[((rb * 2 + 0) * 2 + 1) * kTile + tid],
                                    sm.raw[((rb * 2 + 0) * 2 + 0) * kTile + tid], tshift);
      b = __builtin_amdgcn_alignbit(sm.raw[((rb * 2 + 1) * 2 + 1) * kTile + tid],
                                    sm.raw[((rb * 2 + 1) * 2 + 0) * kTile + tid], tshift);
    }
    a &= bm;
    b &= bm;
    uint8_t* pa = (uint8_t*)sm.words[wb][0] + wbyte;
    uint8_t* pb = (uint8_t*)sm.words[wb][1] + wbyte;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pa[i * 128] = (uint8_t)(a >> (8 * i));
      pb[i * 128] = (uint8_t)(b >> (8 * i));
    }
  };

  // ---- MFMA geometry -----------------------------------------------------------
  const int wn = wave >> 1, wk = wave & 1;
  const int fr = lane & 15, fq = lane >> 4;
  // byte offsets of this lane's two 16-byte runs inside a 16-row tile: chunk
  // fq (tokens 16 fq ..) and chunk fq + 4 (tokens 64 + 16 fq ..), swizzled
  const int frag_lo = fr * kRowBytes + ((fq ^ swz(fr)) << 4);
  const int frag_hi = fr * kRowBytes + (((fq + 4) ^ swz(fr)) << 4);

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  // ---- the K-loop ----------------------------------------------------------------
  const int s0 = start / kStep;
  const int s_end = (end + kStep - 1) / kStep;
  const int nsteps = s_end - s0;
  // Loads issued at step x (after its barrier 2): the data of step x + 2, plus
  //   grouped:  2 scale-slot loads, which fetch group x / 4 + 1 (A, B) when
  //             x % 4 == 0 and x > s0 and are out-of-range dummies otherwise;
  //   per step: the raw scales of step x + 3 (4 loads);
  // so a batch is always kBatch loads (the prologue covers the scales the loop
  // starts with).
  constexpr int kBatch = GROUP ? kDataDma + 2 : kDataDma + 4;
  // Prologue.  Batches past the window are still issued, with every data load
  // out of range (no memory traffic; the stage they zero is never read again),
  // so that exactly one batch is in flight at each barrier 1 and the loop body
  // has no data-dependent branch for the compiler to sink MFMAs into.
  if (GROUP) {
    dma_group(s0 >> 2, 0, true);
    dma_group(s0 >> 2, 1, true);
    dma_group((s0 >> 2) + 1, 0, true);
    dma_group((s0 >> 2) + 1, 1, true);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) dma_raw(s0, k);
#pragma unroll
    for (int k = 0; k < 4; ++k) dma_raw(s0 + 1, k);
#pragma unroll
    for (int k = 0; k < 4; ++k) dma_raw(s0 + 2, k);
  }
  {
    const uint32_t live = live_mask(s0, start, end);
#pragma unroll
    for (int i = 0; i < kDataDma; ++i) dma_data(i, 0, s0, live);
  }
  wait_vm<kDataDma>();  // the prologue's scale loads landed
  __syncthreads();
  relayout(s0, 0);
  __syncthreads();  // words of s0 written
  {
    const uint32_t live = live_mask(s0 + 1, start, end);
#pragma unroll
    for (int i = 0; i < kDataDma; ++i) dma_data(i, 1, s0 + 1, live);
  }

  for (int j = 0; j < nsteps; ++j) {
    const int s = s0 + j;
    const int P = j & 1;
    // barrier 1: this step's data (and every scale load issued before it) has
    // landed everywhere; only the loads issued at step s - 1 may still be in
    // flight.  This step's words were written during the last step.
    __builtin_amdgcn_sched_barrier(0);
    if (j == 0)
      wait_vm<kDataDma>();
    else
      wait_vm<kBatch>();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);

    const uint8_t* ta = sm.data[P][0] + (wn * 128) * kRowBytes;
    const uint8_t* tb = sm.data[P][1] + (wk * 128) * kRowBytes;
    const uint32_t* wa = sm.words[P][0] + (wn * 64 + lane) * 2;
    const uint32_t* wbw = sm.words[P][1] + (wk * 64 + lane) * 2;
    const int sa0 = (int)wa[0], sa1 = (int)wa[1];
    const int sb0 = (int)wbw[0], sb1 = (int)wbw[1];
    // all of this step's fragments, in the order the MFMAs below consume them
    v8i fa[8], fb[8];
    fa[0] = frag(ta, frag_lo, frag_hi);
#pragma unroll
    for (int t = 0; t < 8; ++t) fb[t] = frag(tb + t * 16 * kRowBytes, frag_lo, frag_hi);
#pragma unroll
    for (int t = 1; t < 8; ++t) fa[t] = frag(ta + t * 16 * kRowBytes, frag_lo, frag_hi);
    __builtin_amdgcn_sched_barrier(0);

    const uint32_t live2 = live_mask(s + 2, start, end);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const int m = nt * 8 + kt;
        acc[kt][nt] = mfma_e4m3_sel(kt & 3, nt & 3, fb[kt], fa[nt], acc[kt][nt], kt < 4 ? sb0 : sb1,
                                    nt < 4 ? sa0 : sa1);
        if (m == 15) {
          // barrier 2: every wave holds this step's fragments and scale words
          // in registers, so this stage may be refilled (step after next).
          __builtin_amdgcn_sched_barrier(0);
          wait_lgkm_all();
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
        if (m >= 16 && m < 16 + kDataDma) {
          // one refill load between consecutive MFMAs
          dma_data(m - 16, P, s + 2, live2);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (m == 16 + kDataDma) {
          // this step's scale loads (see batch_size)
          if (GROUP) {
            const bool real = (s & 3) == 0 && s > s0;
            dma_group((s >> 2) + 1, 0, real);
            dma_group((s >> 2) + 1, 1, real);
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) dma_raw(s + 3, k);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (m == 44) {
          // the next step's scale words (their raw bytes landed before
          // barrier 1; past the window they are all-zero and never read)
          relayout(s + 1, P ^ 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vm_all();  // no LDS-direct load may outlive the workgroup

  // ---- epilogue: bf16 RNE in registers, 8-byte stores -----------------------------
  const int on = n0 + wn * 128 + fr;      // + 16 nt
  const int ok = k0 + wk * 128 + 4 * fq;  // + 16 kt
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int n = on + 16 * nt, k = ok + 16 * kt;
      if (n < N && k < K) {
        const v4f v = acc[kt][nt];
        uint2 w;
        w.x = pack_bf16x2(v.x, v.y);
        w.y = pack_bf16x2(v.z, v.w);
        *(uint2*)(outg + (size_t)n * K + k) = w;
      }
    }
  }
}

struct DeviceInfo {
  int checked;
  int ok;
};
DeviceInfo g_dev[64];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MXW_ERR_DEVICE;
  if (dev < 64 && g_dev[dev].checked) return g_dev[dev].ok ? MXW_OK : MXW_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MXW_ERR_DEVICE;
  const int ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) {
    g_dev[dev].ok = ok;
    g_dev[dev].checked = 1;
  }
  return ok ? MXW_OK : MXW_ERR_DEVICE;
}

}  // namespace

extern "C" {

int64_t mxw_grid_size(int E, int N, int K) {
  if (E < 1 || E > MXW_MAX_EXPERTS || N < 16 || K < 16) return 0;
  return (int64_t)E * ((N + kTile - 1) / kTile) * ((K + kTile - 1) / kTile);
}

int mxfp8_wgrad_grouped(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                        const int32_t* offs, int E, int M, int N, int K, uint16_t* out, void* stream) {
  if (!A || !sA || !B || !sB || !offs || !out) return MXW_ERR_NULL;
  if (E < 1 || E > MXW_MAX_EXPERTS || M < 0 || M > MXW_MAX_TOKENS || (M & 31) || N < 16 || K < 16 ||
      (N & 15) || (K & 15) || N > 65536 || K > 65536)
    return MXW_ERR_DIM;
  if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)out) & 15) return MXW_ERR_ALIGN;
  const int64_t grid = mxw_grid_size(E, N, K);
  if (grid <= 0 || grid * kThreads > 0xFFFFFFFFLL) return MXW_ERR_DIM;
  int rc = check_device();
  if (rc) return rc;
  Params p;
  p.A = A;
  p.sA = sA;
  p.B = B;
  p.sB = sB;
  p.offs = offs;
  p.out = out;
  p.E = E;
  p.M = M;
  p.N = N;
  p.K = K;
  p.tilesN = (N + kTile - 1) / kTile;
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
  if ((M & 511) == 0)
    hipLaunchKernelGGL(wgrad_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL(wgrad_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream, p);
  if (hipGetLastError() != hipSuccess) return MXW_ERR_LAUNCH;
  return MXW_OK;
}

const char* mxw_strerror(int code) {
  switch (code) {
    case MXW_OK: return "ok";
    case MXW_ERR_NULL: return "a required pointer is NULL";
    case MXW_ERR_DIM: return "E, M, N or K outside the supported range";
    case MXW_ERR_ALIGN: return "A, B or out is not 16-byte aligned";
    case MXW_ERR_DEVICE: return "the current device is not gfx950 (or no device)";
    case MXW_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown error";
  }
}

int mxw_version(void) { return 100; }

}  // extern "C"
