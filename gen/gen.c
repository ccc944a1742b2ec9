/*
 * Seeded synthetic inputs for the tiled GEMM C = A*B.
 *
 * This module holds none of the GEMM's arithmetic.  It draws the input
 * matrices (uniform[-1,1], N(0,1), N(0,1)/sqrt(K), small integers), rounds
 * them once to the storage format the kernels read (fp64 -> bf16 / fp16 /
 * fp32, round-to-nearest-even), and block-quantises fp32 matrices to OCP
 * e4m3fn with one fp32 scale per block (scale = amax/448, q = x/scale cast
 * to e4m3), the per-block convention of the fused RMSNorm + FP8 quantisation
 * listing in "TileKernels deep dive" (section 7.2) and its E4M3 FN format
 * (section 4.3).  Both the CPU oracle and the GPU path read these bytes.
 *
 * Random numbers: a counter-based generator.  Draw i of (seed, stream) is the
 * SplitMix64 output function (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) applied to
 * key(seed, stream) + (i + 1) * 0x9E3779B97F4A7C15, so any element can be
 * computed on its own and the bytes do not depend on the thread count.
 *
 *   uniform u in [0,1)    : (draw >> 11) * 2^-53
 *   uniform[-1,1]         : 2u - 1
 *   normal (Box-Muller)   : element i uses draws 2i and 2i+1:
 *                           sqrt(-2 ln(1 - u0)) * cos(2 pi u1), in fp64
 *   integer in [-r, r]    : floor(u * (2r + 1)) - r
 *
 * The value is divided by `divisor` in fp64 (sqrt(K) for N(0,1)/sqrt(K)) and
 * then rounded once to the output format.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t splitmix_out(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return splitmix_out(splitmix_out(seed + GOLDEN) + stream * GOLDEN);
}

static inline uint64_t draw(uint64_t key, uint64_t i) {
  return splitmix_out(key + (i + 1) * GOLDEN);
}

static inline double unit(uint64_t key, uint64_t i) {
  return (double)(draw(key, i) >> 11) * 0x1p-53;
}

enum { DIST_UNIFORM = 0, DIST_NORMAL = 1, DIST_INT = 2 };
enum { OUT_F64 = 0, OUT_F32 = 1, OUT_BF16 = 2, OUT_F16 = 3 };

static double sample(int dist, uint64_t key, uint64_t i, double param) {
  switch (dist) {
    case DIST_UNIFORM:
      return 2.0 * unit(key, i) - 1.0;
    case DIST_NORMAL: {
      double u0 = 1.0 - unit(key, 2 * i);   /* in (0, 1] */
      double u1 = unit(key, 2 * i + 1);
      return sqrt(-2.0 * log(u0)) * cos(6.283185307179586 * u1);
    }
    default: { /* DIST_INT, param = r */
      double r = param;
      return floor(unit(key, i) * (2.0 * r + 1.0)) - r;
    }
  }
}

/* fp64 -> bf16 bits, one round-to-nearest-even.  Normal results round the
 * 52-bit fraction to 7 bits on the integer (exponent | fraction) pattern, so a
 * carry moves into the exponent by itself; results below 2^-126 are multiples
 * of 2^-133 and are rounded with rint (ties to even in the default mode). */
static uint16_t to_bf16(double d) {
  uint64_t u;
  memcpy(&u, &d, 8);
  uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  uint64_t mag = u & 0x7FFFFFFFFFFFFFFFULL;
  if (mag > 0x7FF0000000000000ULL) return (uint16_t)(sign | 0x7FC0u); /* NaN */
  int e = (int)(mag >> 52) - 1023;
  if (e > 127) return (uint16_t)(sign | 0x7F80u);                     /* inf */
  if (e >= -126) {
    uint64_t t = ((uint64_t)(e + 127) << 52) | (mag & 0xFFFFFFFFFFFFFULL);
    uint64_t r = (t + ((1ULL << 44) - 1) + ((t >> 45) & 1)) >> 45;
    if (r >= 0x7F80u) r = 0x7F80u;
    return (uint16_t)(sign | r);
  }
  double q = rint(fabs(d) * 0x1p133);
  return (uint16_t)(sign | (uint16_t)q);
}

/* fp64 -> fp16 bits, one round-to-nearest-even (same scheme: 10-bit fraction,
 * subnormal unit 2^-24). */
static uint16_t to_f16(double d) {
  uint64_t u;
  memcpy(&u, &d, 8);
  uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  uint64_t mag = u & 0x7FFFFFFFFFFFFFFFULL;
  if (mag > 0x7FF0000000000000ULL) return (uint16_t)(sign | 0x7E00u);
  int e = (int)(mag >> 52) - 1023;
  if (e > 15) return (uint16_t)(sign | 0x7C00u);
  if (e >= -14) {
    uint64_t t = ((uint64_t)(e + 15) << 52) | (mag & 0xFFFFFFFFFFFFFULL);
    uint64_t r = (t + ((1ULL << 41) - 1) + ((t >> 42) & 1)) >> 42;
    if (r >= 0x7C00u) r = 0x7C00u;
    return (uint16_t)(sign | r);
  }
  double q = rint(fabs(d) * 0x1p24);
  return (uint16_t)(sign | (uint16_t)q);
}

/* Fill out[0..n) with elements offset..offset+n of (seed, stream). */
void tg_gen_fill(int dist, uint64_t seed, uint64_t stream, int64_t offset, int64_t n,
                 double param, double divisor, int out_fmt, void* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) {
    double v = sample(dist, key, (uint64_t)(offset + t), param) / divisor;
    switch (out_fmt) {
      case OUT_F64: ((double*)out)[t] = v; break;
      case OUT_F32: ((float*)out)[t] = (float)v; break;
      case OUT_BF16: ((uint16_t*)out)[t] = to_bf16(v); break;
      default: ((uint16_t*)out)[t] = to_f16(v); break;
    }
  }
}

/* Raw 64-bit draws (for tests of the generator and for row sampling). */
void tg_gen_draws(uint64_t seed, uint64_t stream, int64_t offset, int64_t n, uint64_t* out) {
  uint64_t key = stream_key(seed, stream);
  for (int64_t t = 0; t < n; ++t) out[t] = draw(key, (uint64_t)(offset + t));
}

/* Rounding helpers exposed for the codec tests. */
void tg_gen_round_bf16(const double* x, int64_t n, uint16_t* out) {
  for (int64_t t = 0; t < n; ++t) out[t] = to_bf16(x[t]);
}
void tg_gen_round_f16(const double* x, int64_t n, uint16_t* out) {
  for (int64_t t = 0; t < n; ++t) out[t] = to_f16(x[t]);
}

/* fp32 -> e4m3fn code, round-to-nearest-even, for |v| <= 448 (the caller
 * clamps first, so no NaN code is produced).  Below 2^-6 the grid is the
 * subnormal one, multiples of 2^-9; at and above 2^-6 the value is scaled so
 * that its significand lies in [8, 16) and rounded to an integer there. */
static uint8_t to_e4m3fn(float v) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  float a = fabsf(v);
  if (!(a == a)) return 0x7F; /* NaN stays NaN */
  if (a < 0x1p-6f) return (uint8_t)(sign | (uint8_t)rintf(a * 0x1p9f));
  int e;
  (void)frexpf(a, &e);       /* a = f * 2^e, f in [0.5, 1) */
  e -= 1;                    /* a in [2^e, 2^(e+1)) */
  float t = rintf(ldexpf(a, 3 - e)); /* in [8, 16] */
  if (t == 16.0f) { t = 8.0f; e += 1; }
  return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | ((int)t - 8)));
}

void tg_gen_round_e4m3fn(const float* x, int64_t n, uint8_t* out) {
  for (int64_t t = 0; t < n; ++t) out[t] = to_e4m3fn(x[t]);
}

/* Block quantiser.  X is rows x cols fp32, row-major.  Blocks are br x bc
 * (1 x 128 for the activation operand, 128 x 128 for the weight operand);
 * trailing partial blocks keep their own scale.  For each block:
 *   amax = max |x|  (fp32), s = amax / 448 (fp32 division), or s = 1 if amax = 0
 *   q    = e4m3fn_rne(clamp(x / s, -448, 448))
 * Q is rows x cols codes, row-major; S is ceil(rows/br) x ceil(cols/bc), row-major. */
void tg_gen_quant_e4m3fn(const float* X, int64_t rows, int64_t cols, int64_t br, int64_t bc,
                         uint8_t* Q, float* S) {
  int64_t nbr = (rows + br - 1) / br, nbc = (cols + bc - 1) / bc;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nbr * nbc; ++b) {
    int64_t r0 = (b / nbc) * br, c0 = (b % nbc) * bc;
    int64_t r1 = r0 + br < rows ? r0 + br : rows;
    int64_t c1 = c0 + bc < cols ? c0 + bc : cols;
    float amax = 0.0f;
    for (int64_t r = r0; r < r1; ++r)
      for (int64_t c = c0; c < c1; ++c) {
        float a = fabsf(X[r * cols + c]);
        if (a > amax) amax = a;
      }
    float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    S[b] = s;
    for (int64_t r = r0; r < r1; ++r)
      for (int64_t c = c0; c < c1; ++c) {
        float y = X[r * cols + c] / s;
        if (y > 448.0f) y = 448.0f;
        if (y < -448.0f) y = -448.0f;
        Q[r * cols + c] = amax > 0.0f ? to_e4m3fn(y) : 0;
      }
  }
}
