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
//     128-token K-steps, keeps the tile's 65,536 FP32 sums in registers and
//     stores once (blog section 4).  No atomics: bit-reproducible.
//   * tile scheduler: every workgroup reads offs itself, ranks the experts by
//     window length with one lane per expert (longest first, ties to the lower
//     index; blog section 5.4), and numbers tiles so that the workgroups the
//     dispatcher deals to one XCD (block index mod 8, blog section 3) cover a
//     compact group of 2 x 2 supertiles of the same expert (blog section 5.5).
//   * staging: each K-step's operand stripes (256 rows x 128 tokens of A and
//     of B) go HBM -> LDS with 16-byte LDS-direct buffer loads into a
//     ping-pong pair of stages (blog section 4), laid out with an XOR swizzle
//     of the 16-byte chunk index so that MFMA fragment reads are free of bank
//     conflicts.
//   * ragged head/tail: a 32-token sub-block of a step is live iff it lies
//     inside [start, end) (group boundaries are 32-aligned, blog section 1).
//     Dead sub-blocks are removed twice: their data loads are pointed out of
//     the buffer range, so the hardware returns zeros (NaN padding never
//     reaches the MFMA, blog section 5.3), and both operands' scales are set
//     to 0x00.
//   * scales: one dword per row per K-step (4 sub-blocks) is loaded
//     cooperatively (lane <-> row) and re-laid in LDS into MFMA-ready words:
//     byte i of a word is 16-row tile i of one K-step, picked with op_sel
//     (blog sections 3, 5.2 and 5.6), so the hot loop reads two dwords per
//     operand per K-step and does no unpacking.
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
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kTile = 256;              // output tile edge, N and K
constexpr int kStep = 128;              // tokens per K-step
constexpr int kThreads = 256;           // 4 wave64
constexpr int kRowBytes = kStep;        // one staged row = 128 E4M3 codes
constexpr int kOpBytes = kTile * kRowBytes;  // 32 KiB per operand per stage
constexpr uint32_t kOob = 0x80000000u;  // a buffer offset past any range used here
// raw buffer descriptor word 3 for gfx9-family: 32-bit data format, no swizzle,
// range checking on the byte offset
constexpr int kRsrcWord3 = 0x00020000;

// One pipeline stage in LDS.
struct Stage {
  uint8_t a[kOpBytes];  // A stripe: 256 n-rows x 128 tokens (swizzled chunks)
  uint8_t b[kOpBytes];  // B stripe: 256 k-rows x 128 tokens
  // MFMA-ready scale words, index (half * 64 + lane) * 2 + word: byte i of
  // word w is 16-row tile 4w + i of that half's 128 rows, for the sub-block
  // lane / 16 and row lane % 16.
  uint32_t sa[256];
  uint32_t sb[256];
};

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// 16-byte LDS-direct load: lane l's 16 bytes from the buffer at voff (range
// checked; out-of-range lanes write zeros) land at LDS byte lds + 16 l.  Issued
// through asm so that the compiler's alias-blind wait insertion does not drain
// the prefetch before every LDS read; the kernel waits on vmcnt itself.  M0
// carries the LDS base and needs one instruction before the load.
// (M0 has no other user in this kernel, so clobbering it is safe.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_load16(const __amdgpu_buffer_rsrc_t& rsrc, uint32_t lds, uint32_t voff,
                                           uint32_t soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// live-sub-block mask of K-step s for window [start, end): bit b set iff tokens
// [128 s + 32 b, 128 s + 32 b + 32) lie inside the window.
__device__ __forceinline__ uint32_t live_mask(int s, int start, int end) {
  uint32_t m = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    int t0 = s * kStep + 32 * b;
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

struct Params {
  const uint8_t* A;
  const uint8_t* sA;
  const uint8_t* B;
  const uint8_t* sB;
  const int32_t* offs;
  uint16_t* out;
  int E, M, N, K;
  int tilesN, tilesK;
  int xcd_map;  // 1: XCD-aware tile numbering (tiles per expert % 8 == 0)
  int super2;   // 1: tilesN and tilesK even -> 2 x 2 supertile order
};

__global__ __launch_bounds__(kThreads, 1) void wgrad_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) Stage stages[2];
  __shared__ int s_start[MXW_MAX_EXPERTS];
  __shared__ int s_len[MXW_MAX_EXPERTS];
  __shared__ int s_order[MXW_MAX_EXPERTS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = p.E, M = p.M, N = p.N, K = p.K;

  // ---- windows from offs (clamped to [0, M], monotone) ----------------------
  if (tid < E) {
    int e = min(max(p.offs[tid], 0), M);
    int s = tid ? min(max(p.offs[tid - 1], 0), M) : 0;
    if (e < s) e = s;
    s_start[tid] = s;
    s_len[tid] = e - s;
  }
  __syncthreads();
  // ---- longest-first ranking: lane g counts the experts ahead of it ---------
  if (tid < E) {
    int mine = s_len[tid], r = 0;
    for (int u = 0; u < E; ++u) {
      int l = s_len[u];
      r += (l > mine) || (l == mine && u < tid);
    }
    s_order[r] = tid;
  }
  __syncthreads();

  // ---- block -> (expert rank d, tile u) -> (expert g, tile tn, tk) ----------
  const int T = p.tilesN * p.tilesK;
  const int bid = blockIdx.x;
  int d, u;
  if (p.xcd_map) {
    const int per = T >> 3;          // tiles of one expert dealt to one XCD
    const int x = bid & 7, i = bid >> 3;
    d = i / per;
    u = x * per + (i - d * per);
  } else {
    d = bid / T;
    u = bid - d * T;
  }
  int tn, tk;
  if (p.super2) {
    const int sq = u >> 2, q = u & 3, sk = p.tilesK >> 1;
    tn = 2 * (sq / sk) + (q >> 1);
    tk = 2 * (sq % sk) + (q & 1);
  } else {
    tn = u / p.tilesK;
    tk = u - tn * p.tilesK;
  }
  const int g = __builtin_amdgcn_readfirstlane(s_order[d]);
  const int start = __builtin_amdgcn_readfirstlane(s_start[g]);
  const int len = __builtin_amdgcn_readfirstlane(s_len[g]);
  const int end = start + len;
  const int n0 = tn * kTile, k0 = tk * kTile;
  uint16_t* outg = p.out + (size_t)g * N * K;

  // ---- empty expert: exact +0 over the tile ----------------------------------
  if (len == 0) {
    const int rows = min(kTile, N - n0), cols = min(kTile, K - k0);
    const int chunks = cols / 8;  // 16-byte chunks per row (K % 16 == 0)
    const v4i z = {0, 0, 0, 0};
    for (int i = tid; i < rows * chunks; i += kThreads) {
      int r = i / chunks, c = i - r * chunks;
      *(v4i*)(outg + (size_t)(n0 + r) * K + k0 + 8 * c) = z;
    }
    return;
  }

  // ---- buffer resources, rebased to this tile's 256-row bands ----------------
  const int rowsA = min(kTile, N - n0), rowsB = min(kTile, K - k0);
  const int sbytes = M >> 5;  // scale bytes per row
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A + (size_t)n0 * M, (uint32_t)rowsA * (uint32_t)M);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.B + (size_t)k0 * M, (uint32_t)rowsB * (uint32_t)M);
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(p.sA + (size_t)n0 * sbytes, (uint32_t)rowsA * (uint32_t)sbytes);
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(p.sB + (size_t)k0 * sbytes, (uint32_t)rowsB * (uint32_t)sbytes);

  // ---- per-lane load geometry ------------------------------------------------
  // Data: wave w fills row groups 8w .. 8w+7 (8 rows x 128 B = 1 KiB each) of
  // both stripes.  Lane i of a group writes LDS bytes [16 i, 16 i + 16) of the
  // group, i.e. row i / 8, chunk position i % 8, which holds global chunk
  // (i % 8) ^ swz(row).
  const int lrow = lane >> 3;                 // row within a group of 8
  const int cpos = lane & 7;                  // LDS chunk position
  const int chunk_even = cpos ^ swz(lrow);    // global chunk for an even group
  const int chunk_odd = cpos ^ swz(lrow + 8); // ... odd group (row bit 3 set)
  // Scales: thread t loads the dword of tile row t (4 sub-blocks of a step).
  const uint32_t sc_off = (uint32_t)tid * (uint32_t)sbytes;
  const bool sc_dword = (sbytes & 3) == 0;

  // Relayout destination of thread t's scale bytes: row t -> half t/128,
  // 16-row tile (t%128)/16 -> word ((t%128)/16)/4, byte ((t%128)/16)%4, lane
  // (t%16) + 16 * sub-block.
  const int rh = tid >> 7, rt = (tid & 127) >> 4, rj = tid & 15;
  const int sc_word = ((rh * 64 + rj) * 2 + (rt >> 2));  // + 32 per sub-block
  const int sc_byte = rt & 3;

  auto load_scale = [&](const __amdgpu_buffer_rsrc_t& r, int s) -> uint32_t {
    const uint32_t off = sc_off + (uint32_t)(4 * s);
    if (sc_dword) return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      v |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)(off + b), 0, 0) << (8 * b);
    return v;
  };

  auto issue_data = [&](Stage& S, int s, uint32_t live) {
    const int soff = s * kStep;  // token offset of the step (wave-uniform)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int grp = wave * 8 + j;  // row group
      const int row = grp * 8 + lrow;
      const int ch = (grp & 1) ? chunk_odd : chunk_even;
      const bool ok = (live >> (ch >> 1)) & 1u;
      const uint32_t base = (uint32_t)row * (uint32_t)M + (uint32_t)(ch * 16);
      const uint32_t va = ok ? base : kOob;
      const uint32_t da = (uint32_t)(uintptr_t)(S.a + grp * 1024);
      const uint32_t db = (uint32_t)(uintptr_t)(S.b + grp * 1024);
      lds_load16(rA, __builtin_amdgcn_readfirstlane(da), va, (uint32_t)soff);
      lds_load16(rB, __builtin_amdgcn_readfirstlane(db), va, (uint32_t)soff);
    }
  };

  auto write_scales = [&](Stage& S, uint32_t wa, uint32_t wb) {
    uint8_t* pa = (uint8_t*)S.sa + sc_word * 4 + sc_byte;
    uint8_t* pb = (uint8_t*)S.sb + sc_word * 4 + sc_byte;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      pa[b * 128] = (uint8_t)(wa >> (8 * b));
      pb[b * 128] = (uint8_t)(wb >> (8 * b));
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

  // One K-step of MFMAs on stage S: the wave's 8 B-fragments (16-row k tiles)
  // stay in registers while the 8 A-fragments (16-row n tiles) stream through,
  // one n tile per cluster of 8 MFMAs.
  auto compute = [&](Stage& S) {
    const uint32_t* wsb = S.sb + (wk * 64 + lane) * 2;
    const uint32_t* wsa = S.sa + (wn * 64 + lane) * 2;
    const int sb0 = (int)wsb[0], sb1 = (int)wsb[1];
    const int sa0 = (int)wsa[0], sa1 = (int)wsa[1];
    const uint8_t* bb = S.b + (wk * 128) * kRowBytes;
    const uint8_t* ba = S.a + (wn * 128) * kRowBytes;
    v8i fb[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const v4i lo = *(const v4i*)(bb + t * 16 * kRowBytes + frag_lo);
      const v4i hi = *(const v4i*)(bb + t * 16 * kRowBytes + frag_hi);
      fb[t] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const v4i lo = *(const v4i*)(ba + nt * 16 * kRowBytes + frag_lo);
      const v4i hi = *(const v4i*)(ba + nt * 16 * kRowBytes + frag_hi);
      const v8i fa = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      const int saw = nt < 4 ? sa0 : sa1;
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const int sbw = kt < 4 ? sb0 : sb1;
        acc[kt][nt] = mfma_e4m3_sel(kt & 3, nt & 3, fb[kt], fa, acc[kt][nt], sbw, saw);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- the K-loop ----------------------------------------------------------------
  const int s_lo = start / kStep;
  const int s_hi = (end + kStep - 1) / kStep;
  const int nsteps = s_hi - s_lo;

  uint32_t live = live_mask(s_lo, start, end);
  issue_data(stages[0], s_lo, live);
  uint32_t scA = load_scale(rsA, s_lo), scB = load_scale(rsB, s_lo);

  for (int j = 0; j < nsteps; ++j) {
    const int s = s_lo + j;
    Stage& cur = stages[j & 1];
    Stage& nxt = stages[(j & 1) ^ 1];
    const uint32_t bm = byte_mask(live);
    __builtin_amdgcn_sched_barrier(0);
    write_scales(cur, scA & bm, scB & bm);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's fills of `cur` landed
    __syncthreads();                     // all fills + scale words visible; `nxt` free
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < s_hi) {
      live = live_mask(s + 1, start, end);
      issue_data(nxt, s + 1, live);
      scA = load_scale(rsA, s + 1);
      scB = load_scale(rsB, s + 1);
    }
    compute(cur);
  }

  // ---- epilogue: bf16 RNE in registers, 8-byte stores -----------------------------
  const int on = n0 + wn * 128 + fr;        // + 16 nt
  const int ok = k0 + wk * 128 + 4 * fq;    // + 16 kt
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
  const int T = p.tilesN * p.tilesK;
  p.xcd_map = (T % 8) == 0;
  p.super2 = (p.tilesN % 2 == 0) && (p.tilesK % 2 == 0);
  hipLaunchKernelGGL(wgrad_kernel, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream, p);
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
