// Product with an fp8 output: C = A * B (fp16 / bf16 inputs, fp32
// accumulation) quantised in the epilogue, straight from the accumulators,
// to OCP E4M3FN codes with one fp32 scale per 1 x 128 row slice of C.  That
// is the layout of the block-scaled product's A operand, so one product
// writes the next one's input without a round trip through a wider type:
// the fusion of "TileKernels deep dive" section 7.2 (the result quantised to
// FP8 in the kernel that computes it, scale = row maximum over 448) and of
// its fused SwiGLU + FP8 example (no full write and read of the wide
// result).  Per slice the arithmetic is that of tg_quant_fp8_1x128
// (fp8_codec.hpp) applied to the fp32 product.
//
// Kernels: the 256 x 256 tile kernel in its eight-wave ping-pong form (B
// stored N x K or K x N, 64 x 128 per wave) with the quantising epilogue --
// each wave's 128 columns are one slice, so a row's maximum is a reduction
// inside one wave -- and, for every call it does not take, a fully masked
// kernel with one 32 x 128 tile per workgroup.
#include "../../include/tg_gemm.h"

#include "tile_mfma.hpp"
#include "tile_pp.hpp"

namespace tg {
namespace {

using tile::QuantOut;
typedef tile::PPTile<256> Tile256;

constexpr int QTM = 32, QTN = 128;  // general kernel's output tile: one slice per row
constexpr int QK = 32;              // K per step
constexpr int QPAD = 8;             // LDS row padding (elements), keeps 16-byte alignment

// 256 threads = 4 waves side by side; wave w owns columns 32w .. 32w+31 of
// the tile and accumulates them with 32x32x16 MFMAs.  The row maxima of the
// four waves meet in LDS.
template <typename T>
__global__ __launch_bounds__(256) void gemm16_generic_q8(GemmArgs a, QuantOut qo,
                                                         int64_t tiles_n) {
  typedef typename Elem<T>::x8 T8;
  typedef tile::Mfma32 MMA;
  __shared__ __attribute__((aligned(16))) T As[QTM][QK + QPAD];  // [m][k]
  __shared__ __attribute__((aligned(16))) T Bs[QTN][QK + QPAD];  // [n][k]
  __shared__ float rmax[4][QTM];

  const T* A = static_cast<const T*>(a.A);
  const T* B = static_cast<const T*>(a.B);
  const int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = tm * QTM, n0 = tn * QTN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  f32x16 acc;
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;

  for (int64_t k0 = 0; k0 < a.K; k0 += QK) {
    for (int e = tid; e < QTM * QK; e += 256) {
      const int r = e / QK, kk = e % QK;
      const int64_t gi = m0 + r, gk = k0 + kk;
      As[r][kk] = (gi < a.M && gk < a.K) ? A[gi * a.sam + gk * a.sak] : (T)0.0f;
    }
    for (int e = tid; e < QTN * QK; e += 256) {
      const int r = e / QK, kk = e % QK;
      const int64_t gj = n0 + r, gk = k0 + kk;
      Bs[r][kk] = (gj < a.N && gk < a.K) ? B[gk * a.sbk + gj * a.sbn] : (T)0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < QK; kk += 16) {
      const int ko = kk + 8 * (lane >> 5);
      const T8 av = *reinterpret_cast<const T8*>(&As[lane & 31][ko]);
      const T8 bv = *reinterpret_cast<const T8*>(&Bs[w * 32 + (lane & 31)][ko]);
      acc = mfma32x32x16(av, bv, acc);
    }
    __syncthreads();
  }

  // Row maxima over the wave's 32 columns (columns past N hold zeros), then
  // over the four waves.
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float m = fabsf(acc[v]);
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((lane & 31) == 0) rmax[w][MMA::out_row(lane, v)] = m;
  }
  __syncthreads();
  const int64_t c = n0 + w * 32 + (lane & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = MMA::out_row(lane, v);
    const float amax = fmaxf(fmaxf(rmax[0][row], rmax[1][row]), fmaxf(rmax[2][row], rmax[3][row]));
    bool zero;
    const float sc = block_scale(amax, zero);
    const int64_t r = m0 + row;
    if (r < a.M) {
      if (c < a.N) qo.Q[r * qo.sqm + c] = (uint8_t)code_of(acc[v], sc, zero);
      if (w == 0 && (lane & 31) == 0) qo.S[r * qo.ssm + tn * qo.ssj] = sc;
    }
  }
}

struct Call {
  Op op;
  GemmArgs a;  // C and scm stand for Q and sqm
  QuantOut qo;
};

// The product's checks with Q in place of C (row stride sqm, in bytes), then
// the scales': non-negative strides, a non-zero stride along a dimension of
// more than one slice, and address ranges that do not overflow.
tg_status validate(const Call& c) {
  tg_status st = validate_args(c.op, c.a, 1);
  if (st != TG_SUCCESS) return st;
  if (c.qo.ssm < 0 || c.qo.ssj < 0) return TG_ERR_INVALID_VALUE;
  const int64_t M = c.a.M, N = c.a.N;
  if (M == 0 || N == 0) return TG_SUCCESS;
  if (c.qo.S == nullptr) return TG_ERR_INVALID_VALUE;
  const int64_t nb = cdiv(N, 128);
  if ((M > 1 && c.qo.ssm == 0) || (nb > 1 && c.qo.ssj == 0)) return TG_ERR_INVALID_VALUE;
  int64_t r1, r2, r;
  if (__builtin_mul_overflow(M - 1, c.qo.ssm, &r1) || __builtin_mul_overflow(nb - 1, c.qo.ssj, &r2) ||
      __builtin_add_overflow(r1, r2, &r) || r >= (int64_t(1) << 61))
    return TG_ERR_INVALID_VALUE;
  return TG_SUCCESS;
}

enum class Path { TileNT, TileNN, Generic };

Path path_of(const Call& c) {
  if (variant_tile_nt16()->accepts(c.op, c.a)) return Path::TileNT;
  if (variant_tile_nn16()->accepts(c.op, c.a)) return Path::TileNN;
  return Path::Generic;
}

template <typename T>
hipError_t launch_t(const Call& c, Path p, hipStream_t s) {
  const GemmArgs& a = c.a;
  if (p == Path::Generic) {
    const int64_t tn = cdiv(a.N, QTN), tiles = cdiv(a.M, QTM) * tn;
    if (tiles >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gemm16_generic_q8<T>, dim3((unsigned)tiles), dim3(256), 0, s, a, c.qo, tn);
    return hipGetLastError();
  }
  const int tm = (int)cdiv(a.M, Tile256::BM), tn = (int)cdiv(a.N, Tile256::BN);
  if (p == Path::TileNT)
    // B stored N x K: the eight-wave ping-pong form (each wave's 64 x 128
    // block holds whole 1 x 128 slices)
    hipLaunchKernelGGL((tile::gemm16_pp_q8<T, tile::PPTile<256>>), dim3(tm * tn), dim3(512), 0, s,
                       a, tm, tn, c.qo);
  else
    hipLaunchKernelGGL((tile::gemm16_pp_q8<T, tile::PPTile<256>, true>), dim3(tm * tn), dim3(512),
                       0, s, a, tm, tn, c.qo);
  return hipGetLastError();
}

tg_status run(const Call& c, tg_stream_t stream) {
  tg_status st = validate(c);
  if (st != TG_SUCCESS) return st;
  if (c.a.M == 0 || c.a.N == 0) return TG_SUCCESS;
  const Path p = path_of(c);
  if (p == Path::Generic && cdiv(c.a.M, QTM) * cdiv(c.a.N, QTN) >= (int64_t(1) << 31))
    return TG_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = c.op == Op::BF16 ? launch_t<__bf16>(c, p, s) : launch_t<_Float16>(c, p, s);
  return e == hipSuccess ? TG_SUCCESS : TG_ERR_LAUNCH;
}

Call make(Op op, int64_t M, int64_t N, int64_t K, const void* A, int64_t sam, int64_t sak,
          const void* B, int64_t sbk, int64_t sbn, void* Q, int64_t sqm, float* S, int64_t ssm,
          int64_t ssj) {
  Call c;
  c.op = op;
  c.a = GemmArgs{M, N, K, A, sam, sak, B, sbk, sbn, nullptr, 0, 0, nullptr, 0, 0, Q, sqm};
  c.qo = QuantOut{static_cast<uint8_t*>(Q), sqm, S, ssm, ssj};
  return c;
}

}  // namespace
}  // namespace tg

extern "C" {

tg_status tg_gemm_f16_quant_fp8(int64_t M, int64_t N, int64_t K, const void* A, int64_t sam,
                                int64_t sak, const void* B, int64_t sbk, int64_t sbn, void* Q,
                                int64_t sqm, float* S, int64_t ssm, int64_t ssj,
                                tg_stream_t stream) {
  return tg::run(tg::make(tg::Op::F16, M, N, K, A, sam, sak, B, sbk, sbn, Q, sqm, S, ssm, ssj),
                 stream);
}

tg_status tg_gemm_bf16_quant_fp8(int64_t M, int64_t N, int64_t K, const void* A, int64_t sam,
                                 int64_t sak, const void* B, int64_t sbk, int64_t sbn, void* Q,
                                 int64_t sqm, float* S, int64_t ssm, int64_t ssj,
                                 tg_stream_t stream) {
  return tg::run(tg::make(tg::Op::BF16, M, N, K, A, sam, sak, B, sbk, sbn, Q, sqm, S, ssm, ssj),
                 stream);
}

const char* tg_gemm_quant_fp8_plan(int op, int64_t M, int64_t N, int64_t K, const void* A,
                                   int64_t sam, int64_t sak, const void* B, int64_t sbk,
                                   int64_t sbn, void* Q, int64_t sqm, float* S, int64_t ssm,
                                   int64_t ssj) {
  if (op != 0 && op != 1) return nullptr;
  const tg::Call c = tg::make(static_cast<tg::Op>(op), M, N, K, A, sam, sak, B, sbk, sbn, Q, sqm,
                              S, ssm, ssj);
  if (tg::validate(c) != TG_SUCCESS) return nullptr;
  if (M == 0 || N == 0) return "none";
  switch (tg::path_of(c)) {
    case tg::Path::TileNT: return "tile_nt_256x256_q8";
    case tg::Path::TileNN: return "tile_nn_256x256_q8";
    default: return "generic16_32x128_q8";
  }
}

}  // extern "C"
