// General masked GEMM kernels: any shape, any non-negative strides, any
// alignment.  They take every call the tuned kernels refuse (small or ragged
// shapes, padded or transposed views, K = 0) and are written for clarity of
// indexing rather than speed: one 64x64 output tile per workgroup, operands
// gathered element by element into LDS with bounds masks, MFMA on the tile.
//
// The tile loop is the one of "TileKernels deep dive" section 3.1 and the
// first-GEMM listing of "Getting to know TileLang": clear an fp32 tile
// accumulator, for each K slice copy the A and B tiles to on-chip memory and
// accumulate their product, then round the accumulator into C.
#include "common.hpp"

namespace tg {
namespace {

constexpr int GT = 64;       // output tile edge
constexpr int GK = 32;       // K slice per step (16-bit inputs)
constexpr int GPAD = 8;      // LDS row padding (elements): keeps 16 B alignment, spreads banks

// 256 threads = 4 waves in a 2 x 2 grid; wave w owns the 32 x 32 block
// (w / 2, w % 2) of the tile and accumulates it with 32x32x16 MFMAs.
template <typename T>
__global__ __launch_bounds__(256) void gemm16_generic(GemmArgs a, int64_t tiles_n) {
  typedef typename Elem<T>::x8 T8;
  __shared__ __attribute__((aligned(16))) T As[GT][GK + GPAD];  // [m][k]
  __shared__ __attribute__((aligned(16))) T Bs[GT][GK + GPAD];  // [n][k]

  const T* A = static_cast<const T*>(a.A);
  const T* B = static_cast<const T*>(a.B);
  T* C = static_cast<T*>(a.C);
  const int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = tm * GT, n0 = tn * GT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;

  f32x16 acc;
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;

  for (int64_t k0 = 0; k0 < a.K; k0 += GK) {
    for (int e = tid; e < GT * GK; e += 256) {
      const int r = e / GK, kk = e % GK;
      const int64_t gk = k0 + kk;
      const int64_t gi = m0 + r, gj = n0 + r;
      As[r][kk] = (gi < a.M && gk < a.K) ? A[gi * a.sam + gk * a.sak] : (T)0.0f;
      Bs[r][kk] = (gj < a.N && gk < a.K) ? B[gk * a.sbk + gj * a.sbn] : (T)0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < GK; kk += 16) {
      const int ko = kk + 8 * (lane >> 5);
      T8 av = *reinterpret_cast<const T8*>(&As[wm * 32 + (lane & 31)][ko]);
      T8 bv = *reinterpret_cast<const T8*>(&Bs[wn * 32 + (lane & 31)][ko]);
      acc = mfma32x32x16(av, bv, acc);
    }
    __syncthreads();
  }

  const int64_t j = n0 + wn * 32 + (lane & 31);
  for (int v = 0; v < 16; ++v) {
    const int64_t i = m0 + wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (i < a.M && j < a.N) C[i * a.scm + j] = to_out<T>(acc[v]);
  }
}

// fp8 block-scaled: the K step is one 128-wide scale block.  The block's code
// products are summed from zero in fp32 by the MFMA (two 32x32x64 steps), then
// folded into the accumulator with that block's scale product SA * SB.
constexpr int FK = 128;
constexpr int FPAD = 16;

__global__ __launch_bounds__(256) void gemm_fp8_generic(GemmArgs a, int64_t tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t As[GT][FK + FPAD];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[GT][FK + FPAD];

  const uint8_t* A = static_cast<const uint8_t*>(a.A);
  const uint8_t* B = static_cast<const uint8_t*>(a.B);
  __bf16* C = static_cast<__bf16*>(a.C);
  const int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = tm * GT, n0 = tn * GT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int64_t j = n0 + wn * 32 + (lane & 31);

  f32x16 acc;
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;

  for (int64_t k0 = 0; k0 < a.K; k0 += FK) {
    const int64_t kb = k0 / FK;
    for (int e = tid; e < GT * FK; e += 256) {
      const int r = e / FK, kk = e % FK;
      const int64_t gk = k0 + kk;
      const int64_t gi = m0 + r, gj = n0 + r;
      As[r][kk] = (gi < a.M && gk < a.K) ? A[gi * a.sam + gk * a.sak] : (uint8_t)0;
      Bs[r][kk] = (gj < a.N && gk < a.K) ? B[gk * a.sbk + gj * a.sbn] : (uint8_t)0;
    }
    __syncthreads();
    f32x16 part;
    for (int v = 0; v < 16; ++v) part[v] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < FK; kk += 64) {
      const int ko = kk + 32 * (lane >> 5);
      i32x8 av = *reinterpret_cast<const i32x8*>(&As[wm * 32 + (lane & 31)][ko]);
      i32x8 bv = *reinterpret_cast<const i32x8*>(&Bs[wn * 32 + (lane & 31)][ko]);
      part = mfma32x32x64_e4m3(av, bv, part);
    }
    const float sb = (j < a.N) ? a.SB[(j / 128) * a.ssbn + kb * a.ssbk] : 0.0f;
    for (int v = 0; v < 16; ++v) {
      const int64_t i = m0 + wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      const float sa = (i < a.M) ? a.SA[i * a.ssam + kb * a.ssak] : 0.0f;
      acc[v] += (sa * sb) * part[v];
    }
    __syncthreads();
  }

  for (int v = 0; v < 16; ++v) {
    const int64_t i = m0 + wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (i < a.M && j < a.N) C[i * a.scm + j] = to_out<__bf16>(acc[v]);
  }
}

bool accepts_any(Op, const GemmArgs&) { return true; }

hipError_t launch16(Op op, const GemmArgs& a, const Scratch&, hipStream_t s) {
  const int64_t tn = cdiv(a.N, GT), tiles = cdiv(a.M, GT) * tn;
  if (op == Op::BF16)
    hipLaunchKernelGGL(gemm16_generic<__bf16>, dim3(tiles), dim3(256), 0, s, a, tn);
  else
    hipLaunchKernelGGL(gemm16_generic<_Float16>, dim3(tiles), dim3(256), 0, s, a, tn);
  return hipGetLastError();
}

hipError_t launch_fp8(Op, const GemmArgs& a, const Scratch&, hipStream_t s) {
  const int64_t tn = cdiv(a.N, GT), tiles = cdiv(a.M, GT) * tn;
  hipLaunchKernelGGL(gemm_fp8_generic, dim3(tiles), dim3(256), 0, s, a, tn);
  return hipGetLastError();
}

}  // namespace

const Variant* variant_generic16() {
  static const Variant v = {"generic16_64x64", accepts_any, launch16, nullptr, nullptr};
  return &v;
}
const Variant* variant_generic_fp8() {
  static const Variant v = {"generic_fp8_64x64", accepts_any, launch_fp8, nullptr, nullptr};
  return &v;
}

}  // namespace tg
