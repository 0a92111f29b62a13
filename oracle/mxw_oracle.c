/*
 * mxw_oracle.c -- plain CPU reference for the MXFP8 ragged weight-gradient
 * grouped GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP path is
 * checked against.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or helper
 * with the GPU library, and the GPU library never calls it.
 *
 * What it computes (blog post "Ragged MXFP8 Weight Gradients: A FlyDSL
 * Grouped GEMM on MI355X", section 1, and the ROCm blog "Group-GEMM in XLA",
 * section "Contracting"): for every expert g, every n < N and every k < K,
 *
 *   dW[g][n][k] = sum over tokens m in [start_g, end_g) of
 *                 dec(A[n][m], sA[n][m/32]) * dec(B[k][m], sB[k][m/32])
 *
 *   dec(q, s)   = e4m3(q) * 2^(s - 127)
 *
 * with A = dY^T [N, M] and B = X^T [K, M] stored token-contiguous (row
 * stride M bytes), scale planes sA [N, M/32] and sB [K, M/32] row-major
 * (row stride M/32 bytes), and offs[g] the cumulative END of expert g's run
 * of tokens (start_0 = 0, start_g = offs[g-1]).
 *
 * Everything is evaluated in IEEE binary64.  Decoding is exact (an E4M3
 * value times a power of two), every product of two decoded values is exact
 * (4 + 4 significant bits), and the sum runs in ascending token order, so the
 * only rounding is the fp64 accumulation itself.  No blocking, no
 * reordering, no fused multiply-add (built with -ffp-contract=off).
 *
 * Formats (readings stated where the pages leave them open):
 *   - E4M3 is the OCP "E4M3FN" flavour used by MXFP8: 1 sign, 4 exponent
 *     bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal
 *     (m * 2^-9); S.1111.111 is NaN; there is no infinity; max 448.
 *     (The blog names FP8 E4M3 for MXFP8 on gfx950 and mentions FP8 NaN in
 *     section 5.3; the OCP MX format fixes the flavour.)
 *   - E8M0 is an unsigned biased exponent: 2^(s-127) for s in 0..254, and
 *     s = 255 is NaN (section 5.3 of the blog: 0x00 is 2^-127, an
 *     out-of-range read of 0xFF is NaN).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define MXWO_OK 0
#define MXWO_ERR_NULL (-1)
#define MXWO_ERR_DIM (-2)
#define MXWO_ERR_OFFS (-3)
#define MXWO_ERR_NOMEM (-4)

/* OCP E4M3FN decode, written from the bit fields. */
double mxw_oracle_e4m3(unsigned code) {
  code &= 0xFFu;
  unsigned sign = code >> 7;
  unsigned expo = (code >> 3) & 0xFu;
  unsigned mant = code & 0x7u;
  double mag;
  if (expo == 0xFu && mant == 0x7u) return NAN; /* S.1111.111 */
  if (expo == 0)
    mag = ldexp((double)mant, -9); /* subnormal: 0.mmm * 2^(1-7) */
  else
    mag = ldexp(8.0 + (double)mant, (int)expo - 7 - 3); /* 1.mmm * 2^(e-7) */
  return sign ? -mag : mag;
}

/* E8M0 decode: a pure power of two with bias 127; 0xFF is NaN. */
double mxw_oracle_e8m0(unsigned code) {
  code &= 0xFFu;
  if (code == 0xFFu) return NAN;
  return ldexp(1.0, (int)code - 127);
}

/*
 * Token windows from the cumulative ends (blog section 1; XLA blog,
 * "Contracting": the start is the exclusive prefix, the end the inclusive
 * prefix).  Validates the device-data preconditions the pages imply: the
 * ends never decrease and never pass M, and every boundary is a multiple of
 * `align` -- 32 for MXFP8 operands, whose groups start on the 32-token scale
 * block (blog sections 1 and 5.3); 1 for plain decoded operands.
 */
int mxw_oracle_windows(const int32_t* offs, int E, int64_t M, int align, int64_t* start, int64_t* end) {
  if (!offs || !start || !end) return MXWO_ERR_NULL;
  if (E < 1 || M < 0 || align < 1) return MXWO_ERR_DIM;
  int64_t prev = 0;
  for (int g = 0; g < E; ++g) {
    int64_t e = offs[g];
    if (e < prev || e > M || (e % align) != 0) return MXWO_ERR_OFFS;
    start[g] = prev;
    end[g] = e;
    prev = e;
  }
  return MXWO_OK;
}

/*
 * The contraction itself on already-decoded fp64 operands:
 *   out[g][n][k] = sum_{m = start_g}^{end_g - 1} Ad[n][m] * Bd[k][m]
 * (ascending m).  Ad is [N, M] and Bd is [K, M], both row-major.  An empty
 * window gives exactly +0.  No alignment requirement at this level, so the
 * small decimal example of the XLA blog can be fed to it directly.
 */
int mxw_oracle_ragged_contract_f64(const double* Ad, const double* Bd, const int64_t* start,
                                   const int64_t* end, int E, int64_t M, int N, int K, double* out) {
  if (!Ad || !Bd || !start || !end || !out) return MXWO_ERR_NULL;
  if (E < 1 || M < 0 || N < 1 || K < 1) return MXWO_ERR_DIM;
  for (int g = 0; g < E; ++g)
    if (start[g] < 0 || end[g] < start[g] || end[g] > M) return MXWO_ERR_OFFS;
  int64_t rows = (int64_t)E * N;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t gn = 0; gn < rows; ++gn) {
    int g = (int)(gn / N);
    int n = (int)(gn % N);
    const double* arow = Ad + (int64_t)n * M;
    double* orow = out + ((int64_t)g * N + n) * K;
    for (int k = 0; k < K; ++k) {
      const double* brow = Bd + (int64_t)k * M;
      double acc = 0.0;
      for (int64_t m = start[g]; m < end[g]; ++m) acc += arow[m] * brow[m];
      orow[k] = acc;
    }
  }
  return MXWO_OK;
}

/* Decode a token-contiguous MXFP8 plane [rows, M] with its scale plane
 * [rows, M/32] into fp64: value = e4m3(q) * 2^(s - 127).  Tokens at or past
 * `used` are written as 0 without being read as values: past the last
 * expert's end they belong to no expert and may hold NaN codes. */
int mxw_oracle_decode_plane(const uint8_t* q, const uint8_t* s, int rows, int64_t M, int64_t used, double* out) {
  if (!q || !s || !out) return MXWO_ERR_NULL;
  if (rows < 0 || M < 0 || (M % 32) != 0 || used < 0 || used > M) return MXWO_ERR_DIM;
  double e4m3[256], e8m0[256];
  for (unsigned c = 0; c < 256; ++c) {
    e4m3[c] = mxw_oracle_e4m3(c);
    e8m0[c] = mxw_oracle_e8m0(c);
  }
  int64_t nb = M / 32;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r)
    for (int64_t m = 0; m < M; ++m)
      out[(int64_t)r * M + m] = m < used ? e4m3[q[(int64_t)r * M + m]] * e8m0[s[(int64_t)r * nb + m / 32]] : 0.0;
  return MXWO_OK;
}

/*
 * Full weight gradient: validate, decode both operands to fp64, contract.
 * out is fp64 [E, N, K].  Tokens at or past offs[E-1] are never read as
 * values (they belong to no expert), whatever their bytes.
 */
int mxw_oracle_wgrad_f64(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                         const int32_t* offs, int E, int64_t M, int N, int K, double* out) {
  if (!A || !sA || !B || !sB || !offs || !out) return MXWO_ERR_NULL;
  if (E < 1 || M < 0 || (M % 32) != 0 || N < 1 || K < 1) return MXWO_ERR_DIM;
  int64_t* start = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  int64_t* end = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  double* Ad = (double*)malloc(sizeof(double) * (size_t)N * (size_t)(M > 0 ? M : 1));
  double* Bd = (double*)malloc(sizeof(double) * (size_t)K * (size_t)(M > 0 ? M : 1));
  int rc = MXWO_OK;
  if (!start || !end || !Ad || !Bd) {
    rc = MXWO_ERR_NOMEM;
    goto done;
  }
  rc = mxw_oracle_windows(offs, E, M, 32, start, end);
  if (rc) goto done;
  rc = mxw_oracle_decode_plane(A, sA, N, M, end[E - 1], Ad);
  if (rc) goto done;
  rc = mxw_oracle_decode_plane(B, sB, K, M, end[E - 1], Bd);
  if (rc) goto done;
  rc = mxw_oracle_ragged_contract_f64(Ad, Bd, start, end, E, M, N, K, out);
done:
  free(start);
  free(end);
  free(Ad);
  free(Bd);
  return rc;
}

/*
 * Selected outputs only, each evaluated straight from the definition (decode
 * every term, ascending m).  Used where the full tensor is too large for the
 * CPU: (pg[i], pn[i], pk[i]) -> out[i].
 */
int mxw_oracle_wgrad_points(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                            const int32_t* offs, int E, int64_t M, int N, int K, const int32_t* pg,
                            const int32_t* pn, const int32_t* pk, int64_t npts, double* out) {
  if (!A || !sA || !B || !sB || !offs || !pg || !pn || !pk || !out) return MXWO_ERR_NULL;
  if (E < 1 || M < 0 || (M % 32) != 0 || N < 1 || K < 1 || npts < 0) return MXWO_ERR_DIM;
  int64_t* start = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  int64_t* end = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  if (!start || !end) {
    free(start);
    free(end);
    return MXWO_ERR_NOMEM;
  }
  int rc = mxw_oracle_windows(offs, E, M, 32, start, end);
  for (int64_t i = 0; rc == MXWO_OK && i < npts; ++i)
    if (pg[i] < 0 || pg[i] >= E || pn[i] < 0 || pn[i] >= N || pk[i] < 0 || pk[i] >= K) rc = MXWO_ERR_DIM;
  if (rc == MXWO_OK) {
    int64_t nb = M / 32;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < npts; ++i) {
      int g = pg[i];
      const uint8_t* arow = A + (int64_t)pn[i] * M;
      const uint8_t* brow = B + (int64_t)pk[i] * M;
      const uint8_t* sarow = sA + (int64_t)pn[i] * nb;
      const uint8_t* sbrow = sB + (int64_t)pk[i] * nb;
      double acc = 0.0;
      for (int64_t m = start[g]; m < end[g]; ++m) {
        double a = mxw_oracle_e4m3(arow[m]) * mxw_oracle_e8m0(sarow[m / 32]);
        double b = mxw_oracle_e4m3(brow[m]) * mxw_oracle_e8m0(sbrow[m / 32]);
        acc += a * b;
      }
      out[i] = acc;
    }
  }
  free(start);
  free(end);
  return rc;
}

/*
 * Row-ragged grouped GEMM: the forward and data-gradient GEMMs of the same
 * MoE layer (blog section 1: the weight gradient is one of three grouped
 * GEMMs per expert layer, the other two keep the contraction over the fixed
 * hidden dimension and carry the raggedness in their rows; XLA blog, the
 * "non-contracting" ragged dot and its forward / data-gradient classes).
 * For every expert g, every row m in [start_g, end_g) and every n < Nw:
 *
 *   out[m][n] = sum over c in [0, C) of
 *               dec(X[m][c], sX[m][c/32]) * dec(W[g][n][c], sW[g][n][c/32])
 *
 * X is [M, C] and W is [E, Nw, C], both contraction-contiguous (MXFP8
 * carries its 32-element blocks along the contraction axis, so both operands
 * are stored with it innermost), scale planes sX [M, C/32] and sW
 * [E, Nw, C/32].  offs[g] is the cumulative END of expert g's rows; rows
 * past offs[E-1] belong to no expert and are not written.  This first level
 * works on already-decoded fp64 operands Xd [M, C] and Wd [E, Nw, C]
 * (ascending c; no alignment requirement, so the XLA blog's decimal example
 * can be fed to it directly).
 */
int mxw_oracle_rows_contract_f64(const double* Xd, const double* Wd, const int64_t* start, const int64_t* end,
                                 int E, int64_t M, int C, int Nw, double* out) {
  if (!Xd || !Wd || !start || !end || !out) return MXWO_ERR_NULL;
  if (E < 1 || M < 0 || C < 1 || Nw < 1) return MXWO_ERR_DIM;
  for (int g = 0; g < E; ++g)
    if (start[g] < 0 || end[g] < start[g] || end[g] > M || (g > 0 && start[g] != end[g - 1])) return MXWO_ERR_OFFS;
  for (int g = 0; g < E; ++g) {
    const double* wg = Wd + (int64_t)g * Nw * C;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t m = start[g]; m < end[g]; ++m) {
      const double* xrow = Xd + m * C;
      double* orow = out + m * Nw;
      for (int n = 0; n < Nw; ++n) {
        const double* wrow = wg + (int64_t)n * C;
        double acc = 0.0;
        for (int c = 0; c < C; ++c) acc += xrow[c] * wrow[c];
        orow[n] = acc;
      }
    }
  }
  return MXWO_OK;
}

/* The full row-ragged GEMM from MXFP8 operands: validate, decode, contract.
 * out is fp64 [M, Nw]; rows past offs[E-1] are left as the caller set them. */
int mxw_oracle_rows_f64(const uint8_t* X, const uint8_t* sX, const uint8_t* W, const uint8_t* sW,
                        const int32_t* offs, int E, int64_t M, int C, int Nw, double* out) {
  if (!X || !sX || !W || !sW || !offs || !out) return MXWO_ERR_NULL;
  if (E < 1 || M < 0 || C < 32 || (C % 32) != 0 || Nw < 1) return MXWO_ERR_DIM;
  int64_t* start = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  int64_t* end = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  double* Xd = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1) * (size_t)C);
  double* Wd = (double*)malloc(sizeof(double) * (size_t)E * (size_t)Nw * (size_t)C);
  int rc = MXWO_OK;
  if (!start || !end || !Xd || !Wd) {
    rc = MXWO_ERR_NOMEM;
    goto done;
  }
  rc = mxw_oracle_windows(offs, E, M, 1, start, end);
  if (rc) goto done;
  /* rows past the last expert are decoded as zeros (never read as values) */
  rc = mxw_oracle_decode_plane(X, sX, (int)end[E - 1], C, C, Xd);
  if (rc) goto done;
  rc = mxw_oracle_decode_plane(W, sW, E * Nw, C, C, Wd);
  if (rc) goto done;
  rc = mxw_oracle_rows_contract_f64(Xd, Wd, start, end, E, M, C, Nw, out);
done:
  free(start);
  free(end);
  free(Xd);
  free(Wd);
  return rc;
}

/* Selected outputs of the row-ragged GEMM, each straight from the
 * definition: (pm[i], pn[i]) -> out[i]; a row past offs[E-1] gives NaN. */
int mxw_oracle_rows_points(const uint8_t* X, const uint8_t* sX, const uint8_t* W, const uint8_t* sW,
                           const int32_t* offs, int E, int64_t M, int C, int Nw, const int64_t* pm,
                           const int32_t* pn, int64_t npts, double* out) {
  if (!X || !sX || !W || !sW || !offs || !pm || !pn || !out) return MXWO_ERR_NULL;
  if (E < 1 || M < 0 || C < 32 || (C % 32) != 0 || Nw < 1 || npts < 0) return MXWO_ERR_DIM;
  int64_t* start = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  int64_t* end = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  if (!start || !end) {
    free(start);
    free(end);
    return MXWO_ERR_NOMEM;
  }
  int rc = mxw_oracle_windows(offs, E, M, 1, start, end);
  for (int64_t i = 0; rc == MXWO_OK && i < npts; ++i)
    if (pm[i] < 0 || pm[i] >= M || pn[i] < 0 || pn[i] >= Nw) rc = MXWO_ERR_DIM;
  if (rc == MXWO_OK) {
    const int64_t nb = C / 32;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < npts; ++i) {
      int g = -1;
      for (int h = 0; h < E; ++h)
        if (start[h] <= pm[i] && pm[i] < end[h]) g = h;
      if (g < 0) {
        out[i] = NAN;
        continue;
      }
      const uint8_t* xrow = X + pm[i] * C;
      const uint8_t* sxrow = sX + pm[i] * nb;
      const uint8_t* wrow = W + ((int64_t)g * Nw + pn[i]) * C;
      const uint8_t* swrow = sW + ((int64_t)g * Nw + pn[i]) * nb;
      double acc = 0.0;
      for (int c = 0; c < C; ++c) {
        double a = mxw_oracle_e4m3(xrow[c]) * mxw_oracle_e8m0(sxrow[c / 32]);
        double b = mxw_oracle_e4m3(wrow[c]) * mxw_oracle_e8m0(swrow[c / 32]);
        acc += a * b;
      }
      out[i] = acc;
    }
  }
  free(start);
  free(end);
  return rc;
}

/*
 * Token-axis MXFP8 quantiser (the step that produces the weight gradient's
 * operands; blog section 1: both operands are quantised along the token
 * axis, token-contiguous, one E8M0 scale per 32 tokens; the blog excludes
 * this step from its timing, section 7).  From bf16 x [M, H] (tokens x
 * hidden, hidden contiguous) to codes q [H, M] and scales s [H, M/32]:
 *
 *   amax   = max |x[m][h]| over the block's 32 tokens (tokens at or past
 *            `used` count as 0: they belong to no expert)
 *   s      = clamp(floor(log2 amax) - 8 + 127, 0, 254), and 127 when amax = 0
 *            (8 = floor(log2 448), the largest E4M3 power of two)
 *   q[h][m] = E4M3FN(x[m][h] / 2^(s - 127)), round to nearest, ties to the
 *            even code, saturated to +-448; 0 for a token at or past `used`
 *
 * (OCP MX definition of the shared scale; the reading and its basis are in
 * the notes: scale exponent = floor(log2 amax) - emax of the element type,
 * saturating conversion.)  floor(log2) is taken exactly from frexp.  The
 * rounding is done on the exact binary64 value by searching the E4M3 grid.
 */
static unsigned mxwo_e4m3_rne(double y) {
  /* nearest of the 127 non-negative finite codes 0x00..0x7E to |y|; ties to
   * the even code (the one whose mantissa LSB is 0) */
  double a = fabs(y);
  unsigned best = 0;
  double bd = a;
  for (unsigned c = 1; c <= 0x7E; ++c) {
    double d = fabs(mxw_oracle_e4m3(c) - a);
    if (d < bd || (d == bd && (c & 1u) == 0 && (best & 1u) != 0)) {
      bd = d;
      best = c;
    }
  }
  if (a > 448.0) best = 0x7E; /* saturate */
  if (best != 0 && y < 0) best |= 0x80u;
  return best;
}

int mxw_oracle_quantize_tokens(const uint16_t* x, int64_t M, int H, int64_t used, uint8_t* q, uint8_t* s) {
  if (!x || !q || !s) return MXWO_ERR_NULL;
  if (M < 0 || (M % 32) != 0 || H < 1 || used < 0 || used > M) return MXWO_ERR_DIM;
  const int64_t nb = M / 32;
#pragma omp parallel for schedule(static)
  for (int h = 0; h < H; ++h) {
    for (int64_t b = 0; b < nb; ++b) {
      double v[32];
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) {
        const int64_t m = b * 32 + i;
        double xv = 0.0;
        if (m < used) {
          uint32_t bits = (uint32_t)x[m * H + h] << 16;
          float f;
          memcpy(&f, &bits, 4);
          xv = (double)f;
        }
        v[i] = xv;
        if (fabs(xv) > amax) amax = fabs(xv);
      }
      int sb;
      if (amax == 0.0) {
        sb = 127;
      } else {
        int e2;
        frexp(amax, &e2); /* amax = f 2^e2, f in [0.5, 1): floor(log2 amax) = e2 - 1 */
        sb = (e2 - 1) - 8 + 127;
        if (sb < 0) sb = 0;
        if (sb > 254) sb = 254;
      }
      s[(int64_t)h * nb + b] = (uint8_t)sb;
      for (int i = 0; i < 32; ++i) {
        const int64_t m = b * 32 + i;
        q[(int64_t)h * M + m] = m < used ? (uint8_t)mxwo_e4m3_rne(ldexp(v[i], 127 - sb)) : 0;
      }
    }
  }
  return MXWO_OK;
}

/*
 * Round a binary64 value to bfloat16 (1 sign, 8 exponent, 7 mantissa bits),
 * round-to-nearest, ties-to-even, in one step from the exact fp64 value
 * (no intermediate fp32).  The blog's epilogue narrows to bf16 with
 * round-to-nearest-even (section 5.5).  NaN -> 0x7FC0 (sign kept).
 */
uint16_t mxw_oracle_bf16_rne(double x) {
  if (isnan(x)) return (uint16_t)(signbit(x) ? 0xFFC0u : 0x7FC0u);
  uint16_t sign = signbit(x) ? 0x8000u : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
  /* bf16 grid spacing at a: ulp = 2^(e-7) for normals (e = floor(log2 a),
   * e >= -126); 2^-133 in the subnormal range. */
  int e;
  frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) -> floor(log2 a) = e - 1 */
  int fl = e - 1;
  int q = fl < -126 ? -133 : fl - 7;
  double scaled = ldexp(a, -q); /* exact: power-of-two scaling of a binary64 */
  double r = nearbyint(scaled); /* current mode is round-to-nearest-even */
  double v = ldexp(r, q);
  if (v >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u); /* overflow to inf */
  /* encode v exactly */
  if (v < ldexp(1.0, -126)) {
    unsigned m = (unsigned)ldexp(v, 133); /* subnormal mantissa (may reach 128 -> min normal) */
    return (uint16_t)(sign | m);
  }
  int ev;
  double f = frexp(v, &ev); /* v = f * 2^ev, f in [0.5,1) */
  unsigned biased = (unsigned)(ev - 1 + 127);
  unsigned mant = (unsigned)ldexp(f * 2.0 - 1.0, 7);
  return (uint16_t)(sign | (biased << 7) | mant);
}

void mxw_oracle_to_bf16(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = mxw_oracle_bf16_rne(x[i]);
}

int mxw_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void mxw_oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/*
 * BF16 contracting ragged dot: the same weight gradient on plain bfloat16
 * operands (ROCm blog "Group-GEMM in XLA": the "Contracting" variant of
 * Table 1, and the wgrad_wi / wgrad_wo classes of Table 7, which are
 * bfloat16 throughout).  For every expert g, n < N, k < K:
 *
 *   out[g][n][k] = sum over tokens m in [start_g, end_g) of bf16(A[n][m]) * bf16(B[k][m])
 *
 * A [N, M] and B [K, M] hold bf16 bit patterns, token-contiguous (row stride
 * M elements).  The pages fix the classes' dimension numbers, not the
 * storage order; this is the storage with the contracted axis innermost,
 * the same as the MXFP8 operands.  The XLA ragged dot puts no alignment on
 * the group sizes, so windows are checked with align = 1.
 *
 * bf16 is decoded from its bit fields: 1 sign bit, 8 exponent bits with bias
 * 127 and 7 fraction bits; exponent field 0 holds zero and the subnormals
 * f * 2^-133, field 255 holds infinity (f = 0) and NaN.  Every product of two
 * decoded values is exact in fp64 (8 + 8 significant bits); the sum runs in
 * ascending token order.
 */
double mxw_oracle_bf16(unsigned bits) {
  bits &= 0xFFFFu;
  unsigned sign = bits >> 15;
  unsigned expo = (bits >> 7) & 0xFFu;
  unsigned frac = bits & 0x7Fu;
  double mag;
  if (expo == 0xFFu) {
    mag = frac ? NAN : INFINITY;
  } else if (expo == 0) {
    mag = ldexp((double)frac, -133); /* 0.fffffff * 2^-126 */
  } else {
    mag = ldexp(128.0 + (double)frac, (int)expo - 127 - 7); /* 1.fffffff * 2^(e-127) */
  }
  return sign ? -mag : mag;
}

/* Decode a bf16 plane [rows, M] to fp64; tokens at or past `used` become 0
 * without being read as values (they belong to no expert). */
int mxw_oracle_decode_bf16_plane(const uint16_t* x, int rows, int64_t M, int64_t used, double* out) {
  if (!x || !out) return MXWO_ERR_NULL;
  if (rows < 0 || M < 0 || used < 0 || used > M) return MXWO_ERR_DIM;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r)
    for (int64_t m = 0; m < M; ++m)
      out[(int64_t)r * M + m] = m < used ? mxw_oracle_bf16(x[(int64_t)r * M + m]) : 0.0;
  return MXWO_OK;
}

/* Full BF16 weight gradient [E, N, K] in fp64: windows, decode, contract. */
int mxw_oracle_bf16_wgrad_f64(const uint16_t* A, const uint16_t* B, const int32_t* offs, int E, int64_t M, int N,
                              int K, double* out) {
  if (!A || !B || !offs || !out) return MXWO_ERR_NULL;
  if (E < 1 || M < 0 || N < 1 || K < 1) return MXWO_ERR_DIM;
  int64_t* start = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  int64_t* end = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  double* Ad = (double*)malloc(sizeof(double) * (size_t)N * (size_t)(M > 0 ? M : 1));
  double* Bd = (double*)malloc(sizeof(double) * (size_t)K * (size_t)(M > 0 ? M : 1));
  int rc = MXWO_OK;
  if (!start || !end || !Ad || !Bd) {
    rc = MXWO_ERR_NOMEM;
    goto done;
  }
  rc = mxw_oracle_windows(offs, E, M, 1, start, end);
  if (rc) goto done;
  rc = mxw_oracle_decode_bf16_plane(A, N, M, end[E - 1], Ad);
  if (rc) goto done;
  rc = mxw_oracle_decode_bf16_plane(B, K, M, end[E - 1], Bd);
  if (rc) goto done;
  rc = mxw_oracle_ragged_contract_f64(Ad, Bd, start, end, E, M, N, K, out);
done:
  free(start);
  free(end);
  free(Ad);
  free(Bd);
  return rc;
}

/* Selected outputs of the BF16 weight gradient, each straight from the
 * definition (decode every term, ascending m): (pg[i], pn[i], pk[i]) -> out[i]. */
int mxw_oracle_bf16_wgrad_points(const uint16_t* A, const uint16_t* B, const int32_t* offs, int E, int64_t M, int N,
                                 int K, const int32_t* pg, const int32_t* pn, const int32_t* pk, int64_t npts,
                                 double* out) {
  if (!A || !B || !offs || !pg || !pn || !pk || !out) return MXWO_ERR_NULL;
  if (E < 1 || M < 0 || N < 1 || K < 1 || npts < 0) return MXWO_ERR_DIM;
  int64_t* start = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  int64_t* end = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  if (!start || !end) {
    free(start);
    free(end);
    return MXWO_ERR_NOMEM;
  }
  int rc = mxw_oracle_windows(offs, E, M, 1, start, end);
  for (int64_t i = 0; rc == MXWO_OK && i < npts; ++i)
    if (pg[i] < 0 || pg[i] >= E || pn[i] < 0 || pn[i] >= N || pk[i] < 0 || pk[i] >= K) rc = MXWO_ERR_DIM;
  if (rc == MXWO_OK) {
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < npts; ++i) {
      const int g = pg[i];
      const uint16_t* arow = A + (int64_t)pn[i] * M;
      const uint16_t* brow = B + (int64_t)pk[i] * M;
      double acc = 0.0;
      for (int64_t m = start[g]; m < end[g]; ++m) acc += mxw_oracle_bf16(arow[m]) * mxw_oracle_bf16(brow[m]);
      out[i] = acc;
    }
  }
  free(start);
  free(end);
  return rc;
}
