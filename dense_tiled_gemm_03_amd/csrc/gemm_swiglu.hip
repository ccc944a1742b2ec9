// Fused SwiGLU with an fp8 output: the gate product G = A * Bg and the up
// product U = A * Bu of one input (fp16 / bf16, fp32 accumulation), combined
// by the SwiGLU activation h = silu(g) * u, silu(g) = g / (1 + e^-g), and h
// quantised in the epilogue to OCP E4M3FN codes with one fp32 scale per
// 1 x 128 row slice -- "TileKernels deep dive" section 4.3 (the fused SwiGLU
// + FP8 quantisation: the SwiGLU result is quantised without being written
// back in a wider type; the down projection then reads it as the A operand
// of the block-scaled product).  Neither product nor h reaches memory.
//
// Kernels: the 256 x 256 tile kernel in its eight-wave ping-pong form, each
// tile over 128 output columns (B stage rows 0 .. 127 from the gate weights,
// 128 .. 255 from the up weights, so the two wave groups hold g and u of the
// same block and meet through LDS in the epilogue), and, for every call it
// does not take, a fully masked kernel with one 32 x 128 tile per workgroup.
#include "../../include/tg_gemm.h"

#include "tile_mfma.hpp"
#include "tile_pp.hpp"

namespace tg {
namespace {

using tile::QuantOut;

constexpr int WTM = 32, WTN = 128;  // general kernel's output tile: one slice per row
constexpr int WK = 32;              // K per step
constexpr int WPAD = 8;             // LDS row padding (elements), keeps 16-byte alignment

// 256 threads = 4 waves side by side; wave w owns columns 32w .. 32w+31 of
// the tile and accumulates their gate and up products with 32x32x16 MFMAs.
// The row maxima of h over the four waves meet in LDS.
template <typename T>
__global__ __launch_bounds__(256) void gemm16_generic_swiglu_q8(GemmArgs a, const void* up,
                                                                QuantOut qo, int64_t tiles_n) {
  typedef typename Elem<T>::x8 T8;
  typedef tile::Mfma32 MMA;
  __shared__ __attribute__((aligned(16))) T As[WTM][WK + WPAD];   // [m][k]
  __shared__ __attribute__((aligned(16))) T Bgs[WTN][WK + WPAD];  // [n][k], gate
  __shared__ __attribute__((aligned(16))) T Bus[WTN][WK + WPAD];  // [n][k], up
  __shared__ float rmax[4][WTM];

  const T* A = static_cast<const T*>(a.A);
  const T* Bg = static_cast<const T*>(a.B);
  const T* Bu = static_cast<const T*>(up);
  const int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = tm * WTM, n0 = tn * WTN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  f32x16 accg, accu;
  for (int v = 0; v < 16; ++v) accg[v] = accu[v] = 0.0f;

  for (int64_t k0 = 0; k0 < a.K; k0 += WK) {
    for (int e = tid; e < WTM * WK; e += 256) {
      const int r = e / WK, kk = e % WK;
      const int64_t gi = m0 + r, gk = k0 + kk;
      As[r][kk] = (gi < a.M && gk < a.K) ? A[gi * a.sam + gk * a.sak] : (T)0.0f;
    }
    for (int e = tid; e < WTN * WK; e += 256) {
      const int r = e / WK, kk = e % WK;
      const int64_t gj = n0 + r, gk = k0 + kk;
      const bool in = gj < a.N && gk < a.K;
      Bgs[r][kk] = in ? Bg[gk * a.sbk + gj * a.sbn] : (T)0.0f;
      Bus[r][kk] = in ? Bu[gk * a.sbk + gj * a.sbn] : (T)0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < WK; kk += 16) {
      const int ko = kk + 8 * (lane >> 5);
      const T8 av = *reinterpret_cast<const T8*>(&As[lane & 31][ko]);
      const T8 gv = *reinterpret_cast<const T8*>(&Bgs[w * 32 + (lane & 31)][ko]);
      const T8 uv = *reinterpret_cast<const T8*>(&Bus[w * 32 + (lane & 31)][ko]);
      accg = mfma32x32x16(av, gv, accg);
      accu = mfma32x32x16(av, uv, accu);
    }
    __syncthreads();
  }

  // h = silu(g) u (columns past N hold zeros in both products, so h = 0 there)
  f32x16 h;
#pragma unroll
  for (int v = 0; v < 16; ++v) h[v] = accg[v] * accu[v] / (1.0f + expf(-accg[v]));

  // Row maxima over the wave's 32 columns, then over the four waves.
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float m = fabsf(h[v]);
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
      if (c < a.N) qo.Q[r * qo.sqm + c] = (uint8_t)code_of(h[v], sc, zero);
      if (w == 0 && (lane & 31) == 0) qo.S[r * qo.ssm + tn * qo.ssj] = sc;
    }
  }
}

struct Call {
  Op op;
  GemmArgs a;       // B is the gate weights; C and scm stand for Q and sqm
  const void* up;   // the up weights, with B's strides
  QuantOut qo;
};

// The checks of the product with an fp8 output (the gate weights as B, Q for
// C), then the up weights' pointer; the two weight matrices share strides,
// so their address ranges are checked alike.
tg_status validate(const Call& c) {
  tg_status st = validate_args(c.op, c.a, 1);
  if (st != TG_SUCCESS) return st;
  if (c.qo.ssm < 0 || c.qo.ssj < 0) return TG_ERR_INVALID_VALUE;
  const int64_t M = c.a.M, N = c.a.N;
  if (M == 0 || N == 0) return TG_SUCCESS;
  if (c.a.K > 0 && c.up == nullptr) return TG_ERR_INVALID_VALUE;
  if (c.qo.S == nullptr) return TG_ERR_INVALID_VALUE;
  const int64_t nb = cdiv(N, 128);
  if ((M > 1 && c.qo.ssm == 0) || (nb > 1 && c.qo.ssj == 0)) return TG_ERR_INVALID_VALUE;
  int64_t r1, r2, r;
  if (__builtin_mul_overflow(M - 1, c.qo.ssm, &r1) || __builtin_mul_overflow(nb - 1, c.qo.ssj, &r2) ||
      __builtin_add_overflow(r1, r2, &r) || r >= (int64_t(1) << 61))
    return TG_ERR_INVALID_VALUE;
  return TG_SUCCESS;
}

// The tiled kernel takes the calls the N x K tile kernel takes for both
// weight matrices (K-contiguous, 16-byte aligned rows, descriptor ranges).
bool tiled(const Call& c) {
  GemmArgs u = c.a;
  u.B = c.up;
  return variant_tile_nt16()->accepts(c.op, c.a) && variant_tile_nt16()->accepts(c.op, u);
}

template <typename T>
hipError_t launch_t(const Call& c, bool tile, hipStream_t s) {
  const GemmArgs& a = c.a;
  if (!tile) {
    const int64_t tn = cdiv(a.N, WTN), tiles = cdiv(a.M, WTM) * tn;
    hipLaunchKernelGGL(gemm16_generic_swiglu_q8<T>, dim3((unsigned)tiles), dim3(256), 0, s, a,
                       c.up, c.qo, tn);
    return hipGetLastError();
  }
  typedef tile::PPTile<256> Cfg;
  const int tm = (int)cdiv(a.M, Cfg::BM), tn = (int)cdiv(a.N, Cfg::BN / 2);
  hipLaunchKernelGGL((tile::gemm16_pp_swiglu<T, Cfg>), dim3(tm * tn), dim3(512), 0, s, a, tm, tn,
                     c.qo, c.up);
  return hipGetLastError();
}

tg_status run(const Call& c, tg_stream_t stream) {
  tg_status st = validate(c);
  if (st != TG_SUCCESS) return st;
  if (c.a.M == 0 || c.a.N == 0) return TG_SUCCESS;
  const bool tile = tiled(c);
  const int64_t tiles = tile ? cdiv(c.a.M, 256) * cdiv(c.a.N, 128)
                             : cdiv(c.a.M, WTM) * cdiv(c.a.N, WTN);
  if (tiles >= (int64_t(1) << 31)) return TG_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      c.op == Op::BF16 ? launch_t<__bf16>(c, tile, s) : launch_t<_Float16>(c, tile, s);
  return e == hipSuccess ? TG_SUCCESS : TG_ERR_LAUNCH;
}

Call make(Op op, int64_t M, int64_t N, int64_t K, const void* A, int64_t sam, int64_t sak,
          const void* Bg, const void* Bu, int64_t sbk, int64_t sbn, void* Q, int64_t sqm,
          float* S, int64_t ssm, int64_t ssj) {
  Call c;
  c.op = op;
  c.a = GemmArgs{M, N, K, A, sam, sak, Bg, sbk, sbn, nullptr, 0, 0, nullptr, 0, 0, Q, sqm};
  c.up = Bu;
  c.qo = QuantOut{static_cast<uint8_t*>(Q), sqm, S, ssm, ssj};
  return c;
}

}  // namespace
}  // namespace tg

extern "C" {

tg_status tg_gemm_f16_swiglu_quant_fp8(int64_t M, int64_t N, int64_t K, const void* A,
                                       int64_t sam, int64_t sak, const void* Bg, const void* Bu,
                                       int64_t sbk, int64_t sbn, void* Q, int64_t sqm, float* S,
                                       int64_t ssm, int64_t ssj, tg_stream_t stream) {
  return tg::run(tg::make(tg::Op::F16, M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q, sqm, S, ssm,
                          ssj),
                 stream);
}

tg_status tg_gemm_bf16_swiglu_quant_fp8(int64_t M, int64_t N, int64_t K, const void* A,
                                        int64_t sam, int64_t sak, const void* Bg, const void* Bu,
                                        int64_t sbk, int64_t sbn, void* Q, int64_t sqm, float* S,
                                        int64_t ssm, int64_t ssj, tg_stream_t stream) {
  return tg::run(tg::make(tg::Op::BF16, M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q, sqm, S, ssm,
                          ssj),
                 stream);
}

const char* tg_gemm_swiglu_quant_fp8_plan(int op, int64_t M, int64_t N, int64_t K, const void* A,
                                          int64_t sam, int64_t sak, const void* Bg,
                                          const void* Bu, int64_t sbk, int64_t sbn, void* Q,
                                          int64_t sqm, float* S, int64_t ssm, int64_t ssj) {
  if (op != 0 && op != 1) return nullptr;
  const tg::Call c = tg::make(static_cast<tg::Op>(op), M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q,
                              sqm, S, ssm, ssj);
  if (tg::validate(c) != TG_SUCCESS) return nullptr;
  if (M == 0 || N == 0) return "none";
  return tg::tiled(c) ? "tile_nt_256x256_swiglu_q8" : "generic16_32x128_swiglu_q8";
}

}  // extern "C"
