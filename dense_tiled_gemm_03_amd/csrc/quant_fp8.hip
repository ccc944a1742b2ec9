// Block quantisation of fp32 matrices to OCP E4M3FN codes plus fp32 scales,
// the step that produces the operands of the block-scaled fp8 product:
// "TileKernels deep dive", section 7.2 (per block, scale = absolute maximum
// over 448 and code = x / scale cast to E4M3) and section 4.3 (the E4M3 FN
// format).  Per block of 1 x 128 (a row slice, the A operand's scales) or
// 128 x 128 (the B operand's scales):
//   amax = max |x|;  s = amax / 448 (fp32, correctly rounded);
//   s = 0 (zero block, or the quotient underflows): s := 1, all codes 0;
//   code = e4m3fn round-to-nearest-even of clamp(x / s, -448, 448), where
//          x / s is the correctly rounded fp32 quotient; the sign is kept.
// Both kernels are bound by HBM (4 bytes read and 1 written per element):
// every element is loaded once into registers, reduced for the block's
// maximum and converted from there.  The quotient x / s comes from the
// block's reciprocal with one FMA correction (quotient_by, fp8_codec.hpp),
// exact for the scales nearly every block has; blocks with extreme scales
// divide.
#include "../../include/tg_gemm.h"

#include <hip/hip_runtime.h>

#include "common.hpp"
#include "fp8_codec.hpp"

namespace tg {
namespace {

// Element mapping inside a 128-wide row segment: lane t (of 16) holds
// columns 4t .. 4t+3 and 64 + 4t .. 64 + 4t + 3, so each 16-byte load (and
// each 4-byte code store) of 16 lanes covers one contiguous run.  Every
// element is read once and every code written once, so the vector paths use
// the non-temporal cache policy: streaming through the caches without it
// measured 12-15% slower (4096 x 16384 with 1 x 128 scales: 61.8 against
// 52.8 us; 7168 x 16384 with 128 x 128 scales: 109.5 against 96.0 us).
__device__ __forceinline__ void load_seg(const float* x, int t, int64_t k0, int64_t K, bool full,
                                         bool vec, float* v) {
  if (full && vec) {
    const f32x4 lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x + 4 * t));
    const f32x4 hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x + 64 + 4 * t));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = lo[e];
      v[4 + e] = hi[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = k0 + 4 * t + e < K ? x[4 * t + e] : 0.0f;
      v[4 + e] = k0 + 64 + 4 * t + e < K ? x[64 + 4 * t + e] : 0.0f;
    }
  }
}

__device__ __forceinline__ void store_seg(uint8_t* q, int t, int64_t k0, int64_t K, bool full,
                                          bool vec, const uint32_t* w) {
  if (full && vec) {
    __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(q + 4 * t));
    __builtin_nontemporal_store(w[1], reinterpret_cast<uint32_t*>(q + 64 + 4 * t));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (k0 + 4 * t + e < K) q[4 * t + e] = (uint8_t)(w[0] >> (8 * e));
      if (k0 + 64 + 4 * t + e < K) q[64 + 4 * t + e] = (uint8_t)(w[1] >> (8 * e));
    }
  }
}

// The eight codes of a lane's segment, packed as store_seg() writes them.
template <bool FAST>
__device__ __forceinline__ void codes_of(const float* v, float s, float r, bool zero,
                                         uint32_t* w) {
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = FAST ? scaled_fast(v[e], s, r) : scaled(v[e], s);
  w[0] = zero ? 0u : e4m3x4(y[0], y[1], y[2], y[3]);
  w[1] = zero ? 0u : e4m3x4(y[4], y[5], y[6], y[7]);
}

// 1 x 128 blocks, numbered row-major (consecutive blocks of a row are
// adjacent in memory): each 16-lane group takes QNB consecutive blocks and
// loads all of them before reducing any, 16 groups per workgroup.
constexpr int QNB = 4;

__global__ __launch_bounds__(256) void quant_1x128(int64_t R, int64_t K, const float* X,
                                                   int64_t ldx, uint8_t* Q, int64_t ldq, float* S,
                                                   int64_t ssr, int64_t ssk, int64_t nkb,
                                                   bool vec) {
  const int t16 = threadIdx.x & 15;
  const int64_t first = ((int64_t)blockIdx.x * 16 + (threadIdx.x >> 4)) * QNB;
  const int64_t nblk = R * nkb;
  int64_t i = first / nkb, kb = first % nkb;
  int64_t row[QNB], col[QNB];
  float v[QNB][8];
#pragma unroll
  for (int b = 0; b < QNB; ++b) {
    row[b] = i;
    col[b] = kb * 128;
    const bool live = first + b < nblk;
    const bool full = live && col[b] + 128 <= K;
    if (live) {
      load_seg(X + i * ldx + col[b], t16, col[b], K, full, vec, v[b]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[b][e] = 0.0f;
    }
    if (++kb == nkb) {
      kb = 0;
      ++i;
    }
  }
#pragma unroll
  for (int b = 0; b < QNB; ++b) {
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[b][e]));
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
    if (first + b >= nblk) continue;
    bool zero;
    const float s = block_scale(amax, zero);
    const float rs = 1.0f / s;
    uint32_t w[2];
    if (__all(scale_in_fast_range(s)))
      codes_of<true>(v[b], s, rs, zero, w);
    else
      codes_of<false>(v[b], s, rs, zero, w);
    const bool full = col[b] + 128 <= K;
    store_seg(Q + row[b] * ldq + col[b], t16, col[b], K, full, vec, w);
    if (t16 == 0) S[row[b] * ssr + (col[b] / 128) * ssk] = s;
  }
}

// 128 x 128 blocks: one workgroup per block; thread t takes rows t / 16 +
// 16 j (j < 8) of the block, lane t % 16 of each: 64 elements in registers.
__global__ __launch_bounds__(256) void quant_128x128(int64_t R, int64_t K, const float* X,
                                                     int64_t ldx, uint8_t* Q, int64_t ldq,
                                                     float* S, int64_t ssr, int64_t ssk,
                                                     int64_t nkb, bool vec) {
  __shared__ float wmax[4];
  const int64_t ib = blockIdx.x / nkb, kb = blockIdx.x % nkb;
  const int t = threadIdx.x, t16 = t & 15, rg = t >> 4;
  const int64_t k0 = kb * 128;
  const bool kfull = k0 + 128 <= K;
  float v[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t r = ib * 128 + rg + 16 * j;
    if (r < R) {
      load_seg(X + r * ldx + k0, t16, k0, K, kfull, vec, v[j]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[j][e]));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  if ((t & 63) == 0) wmax[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  bool zero;
  const float s = block_scale(amax, zero);
  const float rs = 1.0f / s;
  const bool fast = scale_in_fast_range(s);  // uniform over the workgroup
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t r = ib * 128 + rg + 16 * j;
    if (r >= R) continue;
    uint32_t w[2];
    if (fast)
      codes_of<true>(v[j], s, rs, zero, w);
    else
      codes_of<false>(v[j], s, rs, zero, w);
    store_seg(Q + r * ldq + k0, t16, k0, K, kfull, vec, w);
  }
  if (t == 0) S[ib * ssr + kb * ssk] = s;
}

bool ext_ok(int64_t n, int64_t stride) {
  int64_t r;
  return n <= 1 || !__builtin_mul_overflow(n - 1, stride, &r);
}

tg_status quant(int64_t br, int64_t R, int64_t K, const float* X, int64_t ldx, void* Q,
                int64_t ldq, float* S, int64_t ssr, int64_t ssk, tg_stream_t stream) {
  if (R < 0 || K < 0 || ldx < 0 || ldq < 0 || ssr < 0 || ssk < 0) return TG_ERR_INVALID_VALUE;
  if (R == 0 || K == 0) return TG_SUCCESS;
  if (X == nullptr || Q == nullptr || S == nullptr) return TG_ERR_INVALID_VALUE;
  const int64_t nrb = cdiv(R, br), nkb = cdiv(K, 128);
  if (R > 1 && (ldx < K || ldq < K)) return TG_ERR_INVALID_VALUE;  // rows would overlap
  if ((nrb > 1 && ssr == 0) || (nkb > 1 && ssk == 0)) return TG_ERR_INVALID_VALUE;
  if (!ext_ok(R, ldx) || !ext_ok(R, ldq) || !ext_ok(nrb, ssr) || !ext_ok(nkb, ssk))
    return TG_ERR_INVALID_VALUE;
  {
    // element extents; their byte addresses must not overflow either
    const int64_t lim = int64_t(1) << 60;
    int64_t ex, eq, es;
    if (__builtin_add_overflow((R - 1) * ldx, K, &ex) || __builtin_add_overflow((R - 1) * ldq, K, &eq) ||
        __builtin_add_overflow((nrb - 1) * ssr, (nkb - 1) * ssk, &es) || ex >= lim || eq >= lim ||
        es >= lim)
      return TG_ERR_INVALID_VALUE;
  }
  const int64_t groups = br == 1 ? cdiv(R * nkb, 16 * QNB) : nrb * nkb;
  if (groups >= (int64_t(1) << 31)) return TG_ERR_UNSUPPORTED;
  // 16-byte fp32 reads and 4-byte code writes when every full block's rows
  // are aligned so
  const bool vec = ((reinterpret_cast<uintptr_t>(X) & 15) == 0) && ldx % 4 == 0 &&
                   ((reinterpret_cast<uintptr_t>(Q) & 3) == 0) && ldq % 4 == 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (br == 1)
    hipLaunchKernelGGL(quant_1x128, dim3((unsigned)groups), dim3(256), 0, s, R, K, X, ldx,
                       static_cast<uint8_t*>(Q), ldq, S, ssr, ssk, nkb, vec);
  else
    hipLaunchKernelGGL(quant_128x128, dim3((unsigned)groups), dim3(256), 0, s, R, K, X, ldx,
                       static_cast<uint8_t*>(Q), ldq, S, ssr, ssk, nkb, vec);
  return hipGetLastError() == hipSuccess ? TG_SUCCESS : TG_ERR_LAUNCH;
}

}  // namespace
}  // namespace tg

extern "C" {

tg_status tg_quant_fp8_1x128(int64_t R, int64_t K, const float* X, int64_t ldx, void* Q,
                             int64_t ldq, float* S, int64_t ssr, int64_t ssk, tg_stream_t stream) {
  return tg::quant(1, R, K, X, ldx, Q, ldq, S, ssr, ssk, stream);
}

tg_status tg_quant_fp8_128x128(int64_t R, int64_t K, const float* X, int64_t ldx, void* Q,
                               int64_t ldq, float* S, int64_t ssr, int64_t ssk,
                               tg_stream_t stream) {
  return tg::quant(128, R, K, X, ldx, Q, ldq, S, ssr, ssk, stream);
}

}  // extern "C"
