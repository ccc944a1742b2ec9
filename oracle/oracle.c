/*
 * CPU oracle for the tiled dense GEMM.  TEST INFRASTRUCTURE ONLY: the tests,
 * the smoke check and the benchmark's CPU-baseline leg use it; the library
 * path never does.  It shares no source with the GPU path.
 *
 * What it computes is the plain definition of the product that the pages
 * tile:
 *   C[i,j] = sum_{k=0}^{K-1} a[i,k] * b[k,j]            (fp64, k ascending)
 *   S[i,j] = sum_{k=0}^{K-1} |a[i,k]| * |b[k,j]|         (magnitude sum for
 *                                                         the error bound)
 * "Getting to know TileLang", first-GEMM section: fp16 operands, an fp32
 * fragment accumulator cleared before the K loop and copied (cast) to C once
 * after it; "TileKernels deep dive" section 3.1: the 128x128 tile loop that
 * accumulates C tile += A tile * B tile over K; section 2.1: element
 * addressing through per-dimension strides (stride_am, stride_ak, stride_bk,
 * stride_bn).  Here a and b are the exact values of the stored input codes,
 * decoded into fp64; the oracle evaluates the sum in fp64 rather than fp32,
 * so it is the reference the fp32 GPU result is held to.
 *
 * For the fp8 block-scaled product (e4m3fn codes, one fp32 scale per 1x128
 * slice of each A row and per 128x128 block of B, the block-scaled GEMM that
 * the TileLang example list names), each operand element is its decoded code
 * times the scale of the block holding it:
 *   a[i,k] = e4m3(QA[i,k]) * SA[i, k/128],  b[k,j] = e4m3(QB[j,k]) * SB[j/128, k/128]
 *
 * Loop order: for B with unit stride along k the loop is i-j-k; otherwise
 * i-k-j with a row of accumulators.  Each output element sees exactly the same
 * additions in the same ascending-k order either way.  Rows run in parallel
 * (OpenMP), so the result does not depend on the thread count.  Build without
 * fast-math and with -ffp-contract=off (no fused multiply-add contraction).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>

/* ---- decoders, written from the format definitions ---------------------- */

/* binary format with `ebits` exponent bits, `mbits` fraction bits, IEEE
 * special values (all-ones exponent = inf / NaN). */
static double decode_ieee(uint32_t code, int ebits, int mbits) {
  int bias = (1 << (ebits - 1)) - 1;
  uint32_t m = code & ((1u << mbits) - 1);
  uint32_t e = (code >> mbits) & ((1u << ebits) - 1);
  int neg = (code >> (mbits + ebits)) & 1;
  double v;
  if (e == (1u << ebits) - 1)
    v = m ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)m, 1 - bias - mbits);              /* subnormal */
  else
    v = ldexp((double)((1u << mbits) | m), (int)e - bias - mbits);
  return neg ? -v : v;
}

/* OCP E4M3FN: 4 exponent bits (bias 7), 3 fraction bits, no infinities; the
 * single NaN pattern per sign is exponent 1111 with fraction 111; max 448. */
static double decode_e4m3fn(uint32_t code) {
  uint32_t m = code & 7u, e = (code >> 3) & 15u;
  int neg = (code >> 7) & 1;
  double v;
  if (e == 15u && m == 7u)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, 1 - 7 - 3);
  else
    v = ldexp((double)(8u | m), (int)e - 7 - 3);
  return neg ? -v : v;
}

static double tab_f16[65536], tab_bf16[65536], tab_e4m3[256];
static int tabs_ready = 0;

static void build_tables(void) {
  if (tabs_ready) return;
  for (uint32_t c = 0; c < 65536; ++c) {
    tab_f16[c] = decode_ieee(c, 5, 10);
    tab_bf16[c] = decode_ieee(c, 8, 7);
  }
  for (uint32_t c = 0; c < 256; ++c) tab_e4m3[c] = decode_e4m3fn(c);
  tabs_ready = 1;
}

void tg_oracle_init(void) { build_tables(); }

/* Threads of the parallel row loops (n <= 0: every available core).  The
 * result does not depend on it: each output row is one thread's work. */
void tg_oracle_threads(int n) { omp_set_num_threads(n > 0 ? n : omp_get_num_procs()); }

/* Decode n codes of a format (1 = fp16, 2 = bf16, 3 = e4m3fn) for tests. */
void tg_oracle_decode(int fmt, const void* codes, int64_t n, double* out) {
  build_tables();
  for (int64_t t = 0; t < n; ++t) {
    if (fmt == 1) out[t] = tab_f16[((const uint16_t*)codes)[t]];
    else if (fmt == 2) out[t] = tab_bf16[((const uint16_t*)codes)[t]];
    else out[t] = tab_e4m3[((const uint8_t*)codes)[t]];
  }
}

/* ---- the product --------------------------------------------------------- */

enum { FMT_F16 = 1, FMT_BF16 = 2 };

/* A[i,k] at A[i*sam + k*sak], B[k,j] at B[k*sbk + j*sbn] (element strides).
 * rows: the nrows row indices of C to compute (NULL: rows 0..M-1).
 * C, S: nrows x N, row-major.  Returns 0, or -1 on bad arguments. */
int tg_oracle_gemm(int fmt, int64_t M, int64_t N, int64_t K,
                   const uint16_t* A, int64_t sam, int64_t sak,
                   const uint16_t* B, int64_t sbk, int64_t sbn,
                   const int64_t* rows, int64_t nrows, double* C, double* S) {
  if (fmt != FMT_F16 && fmt != FMT_BF16) return -1;
  if (M < 0 || N < 0 || K < 0) return -1;
  build_tables();
  const double* tab = fmt == FMT_F16 ? tab_f16 : tab_bf16;
  if (!rows) nrows = M;
  for (int64_t r = 0; rows && r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= M) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t i = rows ? rows[r] : r;
    double* c = C + r * N;
    double* s = S + r * N;
    if (sbk == 1) {
      for (int64_t j = 0; j < N; ++j) {
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
          double a = tab[A[i * sam + k * sak]];
          double b = tab[B[k + j * sbn]];
          acc += a * b;
          mag += fabs(a) * fabs(b);
        }
        c[j] = acc;
        s[j] = mag;
      }
    } else {
      for (int64_t j = 0; j < N; ++j) { c[j] = 0.0; s[j] = 0.0; }
      for (int64_t k = 0; k < K; ++k) {
        double a = tab[A[i * sam + k * sak]];
        const uint16_t* brow = B + k * sbk;
        for (int64_t j = 0; j < N; ++j) {
          double b = tab[brow[j * sbn]];
          c[j] += a * b;
          s[j] += fabs(a) * fabs(b);
        }
      }
    }
  }
  return 0;
}

/* fp8 e4m3fn block-scaled product.  QA[i,k] at QA[i*sam + k*sak];
 * QB[k,j] at QB[k*sbk + j*sbn]; SA[i, kb] at SA[i*ssam + kb*ssak];
 * SB[jb, kb] at SB[jb*ssbn + kb*ssbk]; kb = k/128, jb = j/128. */
int tg_oracle_gemm_fp8_blockscaled(int64_t M, int64_t N, int64_t K,
                                   const uint8_t* QA, int64_t sam, int64_t sak,
                                   const float* SA, int64_t ssam, int64_t ssak,
                                   const uint8_t* QB, int64_t sbk, int64_t sbn,
                                   const float* SB, int64_t ssbn, int64_t ssbk,
                                   const int64_t* rows, int64_t nrows, double* C, double* S) {
  if (M < 0 || N < 0 || K < 0) return -1;
  build_tables();
  if (!rows) nrows = M;
  for (int64_t r = 0; rows && r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= M) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t i = rows ? rows[r] : r;
    double* c = C + r * N;
    double* s = S + r * N;
    if (sbk == 1) {
      for (int64_t j = 0; j < N; ++j) {
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
          double a = tab_e4m3[QA[i * sam + k * sak]] * (double)SA[i * ssam + (k / 128) * ssak];
          double b = tab_e4m3[QB[k + j * sbn]] * (double)SB[(j / 128) * ssbn + (k / 128) * ssbk];
          acc += a * b;
          mag += fabs(a) * fabs(b);
        }
        c[j] = acc;
        s[j] = mag;
      }
    } else {
      for (int64_t j = 0; j < N; ++j) { c[j] = 0.0; s[j] = 0.0; }
      for (int64_t k = 0; k < K; ++k) {
        double a = tab_e4m3[QA[i * sam + k * sak]] * (double)SA[i * ssam + (k / 128) * ssak];
        for (int64_t j = 0; j < N; ++j) {
          double b = tab_e4m3[QB[k * sbk + j * sbn]] * (double)SB[(j / 128) * ssbn + (k / 128) * ssbk];
          c[j] += a * b;
          s[j] += fabs(a) * fabs(b);
        }
      }
    }
  }
  return 0;
}

/* ---- rounding of the fp64 reference to the output format ----------------- */

/* Round-to-nearest-even of x onto a binary format with p significant bits
 * (including the implicit one), minimum normal exponent emin and largest
 * finite value maxf.  x = f * 2^e with f in [0.5, 1); the representable
 * neighbours near x are multiples of 2^(q) with q = max(e, emin + 1) - p, so
 * x * 2^-q is rounded to an integer with nearbyint (ties to even in the
 * default mode) and scaled back.  Results above maxf after rounding are inf. */
static double round_to_format(double x, int p, int emin, double maxf) {
  if (x != x || x == 0.0 || isinf(x)) return x;
  int e;
  frexp(x, &e);
  int q = (e > emin + 1 ? e : emin + 1) - p;
  double r = ldexp(nearbyint(ldexp(x, -q)), q);
  if (fabs(r) > maxf) return x > 0 ? INFINITY : -INFINITY;
  return r;
}

static uint16_t encode_exact(double v, int ebits, int mbits) {
  /* v is exactly representable in the format (or inf / NaN). */
  int bias = (1 << (ebits - 1)) - 1;
  uint16_t sign = signbit(v) ? (uint16_t)(1u << (ebits + mbits)) : 0;
  double a = fabs(v);
  uint32_t emax = (1u << ebits) - 1;
  if (a != a) return (uint16_t)(sign | (emax << mbits) | (1u << (mbits - 1)));
  if (isinf(a)) return (uint16_t)(sign | (emax << mbits));
  if (a == 0.0) return sign;
  int e;
  double f = frexp(a, &e); /* a = f * 2^e, f in [0.5,1) */
  int E = e - 1 + bias;     /* biased exponent of a */
  if (E <= 0) /* subnormal: a = m * 2^(1 - bias - mbits) */
    return (uint16_t)(sign | (uint32_t)ldexp(a, bias - 1 + mbits));
  uint32_t m = (uint32_t)(ldexp(f, mbits + 1)) - (1u << mbits);
  return (uint16_t)(sign | ((uint32_t)E << mbits) | m);
}

/* ---- fp8 block quantisation ---------------------------------------------
 * "TileKernels deep dive", section 7.2 (the fused RMSNorm + FP8 quantisation
 * listing) and section 4.3 (E4M3 FN): per block the scale is the absolute
 * maximum over 448, and the stored code is x / scale cast to E4M3.  Read
 * here as:
 *   amax = max |x| over the block (exact in fp32);
 *   s    = amax / 448 rounded once to fp32 (the fp64 quotient rounded to
 *          fp32 is the correctly rounded fp32 quotient: 53 >= 2 * 24 + 2);
 *   if s = 0 (amax = 0, or the quotient underflows): s := 1, all codes 0;
 *   y    = x / s rounded once to fp32 (same argument), clamped to
 *          [-448, 448] (a subnormal s is coarse, so x / s can pass 448);
 *   code = y rounded to the nearest e4m3fn value, ties to the even
 *          fraction, sign kept (-0 and negatives that round to 0 give 0x80).
 * Blocks are br x 128 (br = 1: one scale per 128-wide slice of a row; br =
 * 128: one per 128 x 128 block); partial blocks at the edges have scales of
 * their own.  X is R x K fp32 with leading dimension ldx, Q is R x K bytes
 * with leading dimension ldq, S[ib, kb] at S[ib * ssr + kb * ssk]. */

/* the code of v, a finite value on the e4m3fn grid: binary search of the
 * decoded non-negative codes 0 .. 126 (increasing values) */
static uint8_t e4m3_code_of(double v) {
  double a = fabs(v);
  int lo = 0, hi = 126;
  while (lo < hi) {
    int mid = (lo + hi) / 2;
    if (tab_e4m3[mid] < a) lo = mid + 1;
    else hi = mid;
  }
  return (uint8_t)(lo | (signbit(v) ? 0x80 : 0));
}

static double round_to_format(double x, int p, int emin, double maxf);

int tg_oracle_quant_fp8(int64_t R, int64_t K, const float* X, int64_t ldx, int64_t br,
                        uint8_t* Q, int64_t ldq, float* S, int64_t ssr, int64_t ssk) {
  if (R < 0 || K < 0 || (br != 1 && br != 128)) return -1;
  build_tables();
  const int64_t nrb = (R + br - 1) / br, nkb = (K + 127) / 128;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t ib = 0; ib < nrb; ++ib) {
    const int64_t r0 = ib * br, r1 = r0 + br < R ? r0 + br : R;
    for (int64_t kb = 0; kb < nkb; ++kb) {
      const int64_t k0 = kb * 128, k1 = k0 + 128 < K ? k0 + 128 : K;
      float amax = 0.0f;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t k = k0; k < k1; ++k) {
          float a = fabsf(X[r * ldx + k]);
          if (a > amax) amax = a;
        }
      float sc = (float)((double)amax / 448.0);
      const int zero = sc == 0.0f;
      S[ib * ssr + kb * ssk] = zero ? 1.0f : sc;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t k = k0; k < k1; ++k) {
          if (zero) {
            Q[r * ldq + k] = 0;
            continue;
          }
          double y = (double)(float)((double)X[r * ldx + k] / (double)sc);
          if (y > 448.0) y = 448.0;
          if (y < -448.0) y = -448.0;
          Q[r * ldq + k] = e4m3_code_of(round_to_format(y, 4, -6, 448.0));
        }
    }
  }
  return 0;
}

/* fmt 1: fp16 (p = 11, emin = -14, max 65504); fmt 2: bf16 (p = 8,
 * emin = -126, max (2 - 2^-7) * 2^127). */
/* ---- SwiGLU of a gate and an up product ----------------------------------
 * "TileKernels deep dive", section 4.3 (the fused SwiGLU + FP8 quantisation
 * example): the gate and up projections of one input are combined by the
 * SwiGLU activation, and the combination, not the two products, is what is
 * quantised.  Read here as, element by element,
 *   h = silu(g) * u,   silu(g) = g / (1 + e^(-g)),
 * in fp64 from the fp64 products g (gate) and u (up); n values. */
int tg_oracle_swiglu(int64_t n, const double* G, const double* U, double* H) {
  if (n < 0) return -1;
  for (int64_t t = 0; t < n; ++t) H[t] = G[t] / (1.0 + exp(-G[t])) * U[t];
  return 0;
}

void tg_oracle_round(int fmt, const double* x, int64_t n, uint16_t* out) {
  for (int64_t t = 0; t < n; ++t) {
    if (fmt == FMT_F16)
      out[t] = encode_exact(round_to_format(x[t], 11, -14, 65504.0), 5, 10);
    else
      out[t] = encode_exact(round_to_format(x[t], 8, -126, ldexp(255.0, 120)), 8, 7);
  }
}

/* ---- the acceptance bound -------------------------------------------------
 * Per-element tolerance on |C_gpu - C_ref| for a product accumulated in fp32
 * and rounded once to the output format: four unit roundoffs of the output
 * format times S = sum_k |a||b|.  A binary format with p significant bits
 * (the implicit one included) has unit roundoff 2^-p: bf16 has p = 8, fp16
 * p = 11, so the tolerance is 4 * 2^-8 * S and 4 * 2^-11 * S.  It covers the
 * output rounding (at most 2^-p |C| <= 2^-p S) plus fp32 summation in any
 * order (at most about K * 2^-24 * S, 2^-10 S at K = 16384) with room left;
 * S = 0 gives 0, so an all-zero sum must come out exactly zero. */
void tg_oracle_bound(int fmt, const double* S, int64_t n, double* out) {
  const int p = fmt == FMT_F16 ? 11 : 8;
  for (int64_t t = 0; t < n; ++t) out[t] = ldexp(4.0, -p) * S[t];
}
