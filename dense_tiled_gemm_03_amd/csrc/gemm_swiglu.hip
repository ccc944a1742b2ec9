// Fused SwiGLU with an fp8 output: the gate product G = A * Bg and the up
// product U = A * Bu of one input (fp16 / bf16, fp32 accumulation), combined
// by the SwiGLU activation h = silu(g) * u, silu(g) = g / (1 + e^-g), and h
// quantised in the epilogue to OCP E4M3FN codes with one fp32 scale per
// 1 x 128 row slice -- "TileKernels deep dive" section 4.3 (the fused SwiGLU
// + FP8 quantisation: the SwiGLU result is quantised without being written
// back in a wider type; the down projection then reads it as the A operand
// of the block-scaled product).  Neither product nor h reaches memory.
//
// Kernels: for M <= 64 a skinny kernel, one 128-column slice per workgroup
// over the whole of K (below); otherwise the 256 x 256 tile kernel in its
// eight-wave ping-pong form, each tile over 128 output columns (B stage rows
// 0 .. 127 from the gate weights, 128 .. 255 from the up weights, so the two
// wave groups hold g and u of the same block and meet through LDS in the
// epilogue); and, for every call neither takes, a fully masked kernel with
// one 32 x 128 tile per workgroup.
#include "../../include/tg_gemm.h"

#include "tile_mfma.hpp"
#include "tile_pp.hpp"

namespace tg {
namespace {

using tile::QuantOut;
using tile::kOutOfRange;
using tile::load_lds16;
using tile::load_lds16_nt;
using tile::make_desc;

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

// Decode-sized calls (M <= 64, both operands K-contiguous): the products are
// bound by streaming the two weight matrices from HBM, which the 256-row tile
// does with most of its rows empty.  One workgroup of 4 waves owns one
// 128-column output slice (so the slice's row maxima stay in the workgroup)
// over the whole of K -- or, with a caller's workspace, over one of `splits`
// ranges of the K slices, so that there are about as many workgroups as CUs:
//  - 64-wide K slices go HBM -> LDS by LDS-direct loads into a 4-stage ring;
//    a stage holds the slice of A (64 rows), then the slice's 128 gate rows
//    and its 128 up rows (40 KiB; the weights non-temporal, as they are read
//    once); one barrier per slice; slice i + 1's fragments are read while
//    slice i's MFMAs run;
//  - wave w owns columns 32w .. 32w + 31 of both products: per k16 step two
//    32x32x16 MFMAs (rows 0-31, 32-63) of the gate and two of the up
//    weights, so g and u of an element sit in the same lane and h = silu(g) u
//    is formed in registers;
//  - split: each workgroup writes its fp32 g and u partial tiles to the
//    workspace in the accumulators' register layout (rows below M only);
//    the last of a slice's workgroups to finish (a device-scope counter, the
//    protocol of the skinny product) adds them in split order, so g and u
//    are whole before the activation, and clears the counter;
//  - the epilogue takes each row's maximum |h| over the wave's 32 columns by
//    shuffles and over the four waves through LDS, then quantises as the
//    fp8-output epilogue does.
// Chunk swizzle, descriptors and edges as in the skinny product: chunk c of
// stage row r at position c ^ ((r >> 1) & 7); rows past M or N read as zero
// through the descriptor bounds; chunks past K get an out-of-range offset.
constexpr int DM = 64;                         // rows of C per workgroup (all of M)
constexpr int DN = 128;                        // output columns per workgroup (one slice)
constexpr int DK = 64;                         // k per slice
constexpr int DROW = DK * 2;                   // 128 bytes per stage row
constexpr int D_STAGE = (DM + 2 * DN) * DROW;  // 40 KiB: A, gate rows, up rows
constexpr int D_ST = 4;                        // ring depth
constexpr int D_ALD = DM / 8 / 4;              // 1 KiB loads per wave per slice: A
constexpr int D_BLD = DN / 8 / 4;              // each of the gate and up weights
constexpr int D_NLD = D_ALD + 2 * D_BLD;       // 10
static_assert(D_ST * D_STAGE <= 160 * 1024, "the ring must fit the LDS");
static_assert(D_ST * D_NLD <= 63, "loads in flight must fit the vmcnt counter");
static_assert(4 * DM * 4 <= D_STAGE, "the row maxima fit the first stage");
constexpr int D_PART = 256 * 64;               // floats of a split's g and u partial tiles
constexpr int D_LAST = 4096;                   // LDS byte offset of the last-split flag
static_assert(D_LAST >= 4 * DM * 4 && D_LAST + 4 <= D_STAGE, "the flag clears the row maxima");
constexpr int kCoherent = 0x10;                // sc1: device-coherent buffer access
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__global__ __launch_bounds__(256) void gemm16_swiglu_skinny(GemmArgs a, const void* up,
                                                            QuantOut qo, int splits, float* part,
                                                            int* counters) {
  typedef typename Elem<T>::x8 T8;
  typedef tile::Mfma32 MMA;
  __shared__ __attribute__((aligned(1024))) char lds[D_ST * D_STAGE];
  const uint32_t lds32 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t strip = blockIdx.x / splits, n0 = strip * DN;
  const int split = blockIdx.x % splits;
  const int K = (int)a.K;
  const uint32_t lda = (uint32_t)a.sam, ldb = (uint32_t)a.sbn;
  const int rows_a = (int)a.M;  // <= 64
  const int rows_b = (int)min<int64_t>(DN, a.N - n0);
  const i32x4 ra = make_desc(a.A, (uint32_t)(((rows_a - 1) * lda + K) * 2));
  const uint32_t b_range = (uint32_t)(((rows_b - 1) * ldb + K) * 2);
  const i32x4 rg = make_desc(static_cast<const T*>(a.B) + n0 * a.sbn, b_range);
  const i32x4 ru = make_desc(static_cast<const T*>(up) + n0 * a.sbn, b_range);
  // This workgroup's slices [s_begin, s_end) of the nk 64-wide K slices.
  const int nk = (K + DK - 1) / DK;
  const int s_begin = (int)((int64_t)split * nk / splits);
  const int s_end = (int)((int64_t)(split + 1) * nk / splits);
  const int count = s_end - s_begin;

  // Wave w's j-th load of a stage fills 8-row group G of the stage: A rows
  // 16w + 8j (G = 2w + j), gate rows 32w + 8j' (G = 8 + 4w + j'), up rows
  // 32w + 8j' (G = 24 + 4w + j'); lane l writes stage row 8G + (l >> 3) at
  // chunk position l & 7, i.e. logical chunk (l & 7) ^ (4 (G & 1) + (l >> 4)).
  const uint32_t lrow = lane >> 3;
  const uint32_t lc0 = (lane & 7) ^ (lane >> 4), lc1 = (lane & 7) ^ (4 + (lane >> 4));
  auto load_slice = [&](int slot, int slice) {
    if (slice >= s_end) return;  // nothing past the range (an empty load still costs an issue)
    const int k0 = slice * DK;
    const uint32_t stage = lds32 + slot * D_STAGE;
#pragma unroll
    for (int j = 0; j < D_ALD; ++j) {
      const uint32_t c = (j & 1) ? lc1 : lc0;
      const uint32_t off = (16 * w + 8 * j + lrow) * lda * 2 + 2 * k0 + 16 * c;
      load_lds16(ra, stage + (2 * w + j) * 1024, k0 + 8 * (int)c < K ? off : kOutOfRange);
    }
#pragma unroll
    for (int j = 0; j < D_BLD; ++j) {
      const uint32_t c = (j & 1) ? lc1 : lc0;
      const uint32_t off = (32 * w + 8 * j + lrow) * ldb * 2 + 2 * k0 + 16 * c;
      const bool kin = k0 + 8 * (int)c < K;
      load_lds16_nt(rg, stage + (8 + 4 * w + j) * 1024, kin ? off : kOutOfRange);
      load_lds16_nt(ru, stage + (24 + 4 * w + j) * 1024, kin ? off : kOutOfRange);
    }
  };

  // Fragment reads (32x32x16): row (32-aligned base) + (l & 31), chunk
  // 2s + (l >> 5) for k16 step s, at position chunk ^ ((l >> 1) & 7).
  const int sw = (lane >> 1) & 7;
  int rd[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) rd[s] = (lane & 31) * DROW + (((2 * s + (lane >> 5)) ^ sw) * 16);
  const int g_rows = (DM + 32 * w) * DROW, u_rows = (DM + DN + 32 * w) * DROW;

  f32x16 acc_g[2], acc_u[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc_g[i][v] = acc_u[i][v] = 0.0f;

  T8 fa0[2][4], fa1[2][4], fg[2][4], fu[2][4];
  auto read_slice = [&](int buf, int slot) {
    const char* base = lds + slot * D_STAGE;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      fa0[buf][s] = *reinterpret_cast<const T8*>(base + rd[s]);
      fa1[buf][s] = *reinterpret_cast<const T8*>(base + 32 * DROW + rd[s]);
      fg[buf][s] = *reinterpret_cast<const T8*>(base + g_rows + rd[s]);
      fu[buf][s] = *reinterpret_cast<const T8*>(base + u_rows + rd[s]);
    }
  };
  // One slice: wait until slice i + 1 has landed (at most the loads of the
  // D_ST - 2 slices issued after it outstanding; near the end, where fewer
  // follow, every load) and every wave's reads of slice i are done; refill
  // slice i's slot with slice i + D_ST; read slice i + 1; multiply slice i.
  auto step = [&](int i, int cur) {
    if (i + D_ST - 1 < count)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((D_ST - 2) * D_NLD) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");
    load_slice(i % D_ST, s_begin + i + D_ST);
    read_slice(cur ^ 1, (i + 1) % D_ST);
    __builtin_amdgcn_sched_barrier(0);  // reads ahead of the MFMAs
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      acc_g[0] = mfma32x32x16(fa0[cur][s], fg[cur][s], acc_g[0]);
      acc_g[1] = mfma32x32x16(fa1[cur][s], fg[cur][s], acc_g[1]);
      acc_u[0] = mfma32x32x16(fa0[cur][s], fu[cur][s], acc_u[0]);
      acc_u[1] = mfma32x32x16(fa1[cur][s], fu[cur][s], acc_u[1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int p = 0; p < D_ST; ++p) load_slice(p, s_begin + p);
  if (D_ST <= count)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((D_ST - 1) * D_NLD) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  asm volatile("s_barrier" ::: "memory");
  read_slice(0, 0);
  int i = 0;
  for (; i + 1 < count; i += 2) {
    step(i, 0);
    step(i + 1, 1);
  }
  if (i < count) step(i, 0);
  // every load has landed; once every wave is past its last reads the LDS
  // holds the flag and the row maxima
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  if (splits > 1) {
    // Thread t's float4 e (0 .. 15) of a split's partial tiles: acc_g[e / 4]
    // (e < 8) or acc_u[e / 4 - 2], values 4 (e % 4) .. + 3, i.e. rows 32 b +
    // 8 (e % 4) + 4 (l >> 5) .. + 3 (b = (e / 4) % 2) of column 32 w + (l & 31);
    // float4s of rows past M are neither stored nor read.
    const int t = threadIdx.x;
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        part + strip * splits * D_PART, (short)0, splits * D_PART * 4, 0x00020000);
    auto row0 = [&](int e) { return 32 * ((e >> 2) & 1) + 8 * (e & 3) + 4 * (lane >> 5); };
    auto acc_of = [&](int e) -> f32x16& { return e < 8 ? acc_g[e >> 2] : acc_u[(e >> 2) - 2]; };
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (row0(e) < a.M) {
        const f32x16& v = acc_of(e);
        const int q = 4 * (e & 3);
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, f32x4{v[q], v[q + 1], v[q + 2], v[q + 3]}), rp,
            ((split * 16 + e) * 256 + t) * 16, 0, kCoherent);
      }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    int* last = reinterpret_cast<int*>(lds + D_LAST);
    __syncthreads();
    if (t == 0) *last = atomicAdd(counters + strip, 1) == splits - 1;
    __syncthreads();
    if (!*last) return;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc_g[b][v] = acc_u[b][v] = 0.0f;
    // two splits' tiles in flight at a time, added in split order
    for (int sp0 = 0; sp0 < splits; sp0 += 2) {
      u32x4 y[2][16];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          y[j][e] = row0(e) < a.M && sp0 + j < splits
                        ? __builtin_amdgcn_raw_buffer_load_b128(
                              rp, (((sp0 + j) * 16 + e) * 256 + t) * 16, 0, kCoherent)
                        : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (sp0 + j < splits)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            f32x16& v = acc_of(e);
            const f32x4 x = __builtin_bit_cast(f32x4, y[j][e]);
            const int q = 4 * (e & 3);
#pragma unroll
            for (int r = 0; r < 4; ++r) v[q + r] += x[r];
          }
    }
    if (t == 0) __hip_atomic_store(counters + strip, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // h = silu(g) u; lane l holds column 32w + (l & 31), rows 32i + out_row(l, v)
  f32x16 h[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      h[b][v] = acc_g[b][v] * acc_u[b][v] / (1.0f + expf(-acc_g[b][v]));
  // Columns past N are left out of the maxima explicitly: with weight rows
  // closer than K apart, the rows past N are not all outside the descriptor.
  float* rmax = reinterpret_cast<float*>(lds);  // [wave][row]
  const int64_t c = n0 + 32 * w + (lane & 31);
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float m = c < a.N ? fabsf(h[b][v]) : 0.0f;
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
      if ((lane & 31) == 0) rmax[w * DM + 32 * b + MMA::out_row(lane, v)] = m;
    }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = 32 * b + MMA::out_row(lane, v);
      const float amax = fmaxf(fmaxf(rmax[row], rmax[DM + row]),
                               fmaxf(rmax[2 * DM + row], rmax[3 * DM + row]));
      bool zero;
      const float sc = block_scale(amax, zero);
      if (row < a.M) {
        if (c < a.N) qo.Q[row * qo.sqm + c] = (uint8_t)code_of(h[b][v], sc, zero);
        if (w == 0 && (lane & 31) == 0) qo.S[row * qo.ssm + strip * qo.ssj] = sc;
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

enum class Path { Skinny, Tile, Generic };

// Decode-sized calls take the skinny kernel and the rest of the N x K calls
// the tile kernel, when the skinny / N x K tile product takes the call with
// each weight matrix as B (K-contiguous, 16-byte aligned rows, descriptor
// ranges); everything else the masked kernel.
Path path_of(const Call& c) {
  GemmArgs u = c.a;
  u.B = c.up;
  if (variant_skinny16()->accepts(c.op, c.a) && variant_skinny16()->accepts(c.op, u))
    return Path::Skinny;
  if (variant_tile_nt16()->accepts(c.op, c.a) && variant_tile_nt16()->accepts(c.op, u))
    return Path::Tile;
  return Path::Generic;
}

int64_t grid_of(const Call& c, Path p) {
  switch (p) {
    case Path::Skinny: return cdiv(c.a.N, DN);
    case Path::Tile: return cdiv(c.a.M, 256) * cdiv(c.a.N, 128);
    default: return cdiv(c.a.M, WTM) * cdiv(c.a.N, WTN);
  }
}

// Splits of the skinny kernel's K slices with a workspace: about one
// workgroup per CU, at least 8 slices and at most 8 splits (the last
// workgroup of a slice reads every split's 64 KiB of partial tiles); 1: no
// split plan.  When the output slices already fill half the CUs and a split
// would get fewer than 16 K slices, the combine costs more than the second
// half of the CUs gains (64 x 16384 x 1024: 33.3 us split against 30.1).
constexpr int kCus = 256;
int choose_splits(const Call& c) {
  const int64_t slices = cdiv(c.a.N, DN), nk = cdiv(c.a.K, DK);
  int64_t sp = kCus / slices;
  if (sp > nk / 8) sp = nk / 8;
  if (sp > 8) sp = 8;
  if (sp < 2 || (slices > kCus / 4 && nk / sp < 16)) return 1;
  return (int)sp;
}

// Workspace of the split plan: a counter per slice in the fixed counter
// area, then every split's g and u partial tiles (0: no split plan).
size_t scratch_bytes(const Call& c) {
  if (path_of(c) != Path::Skinny) return 0;
  const int64_t slices = cdiv(c.a.N, DN);
  const int splits = choose_splits(c);
  if (splits == 1 || slices > kWorkspaceCounters) return 0;
  return kWorkspaceCounterBytes + (size_t)slices * splits * D_PART * 4;
}

template <typename T>
hipError_t launch_t(const Call& c, Path p, const Scratch& ws, hipStream_t s) {
  const GemmArgs& a = c.a;
  const unsigned grid = (unsigned)grid_of(c, p);
  if (p == Path::Skinny) {
    if (scratch_fits(ws, scratch_bytes(c))) {
      const int splits = choose_splits(c);
      hipLaunchKernelGGL(gemm16_swiglu_skinny<T>, dim3(grid * splits), dim3(256), 0, s, a, c.up,
                         c.qo, splits, reinterpret_cast<float*>(ws.ptr + kWorkspaceCounterBytes),
                         reinterpret_cast<int*>(ws.ptr));
    } else {
      hipLaunchKernelGGL(gemm16_swiglu_skinny<T>, dim3(grid), dim3(256), 0, s, a, c.up, c.qo, 1,
                         nullptr, nullptr);
    }
  } else if (p == Path::Generic) {
    hipLaunchKernelGGL(gemm16_generic_swiglu_q8<T>, dim3(grid), dim3(256), 0, s, a, c.up, c.qo,
                       cdiv(a.N, WTN));
  } else {
    typedef tile::PPTile<256> Cfg;
    const int tm = (int)cdiv(a.M, Cfg::BM), tn = (int)cdiv(a.N, Cfg::BN / 2);
    hipLaunchKernelGGL((tile::gemm16_pp_swiglu<T, Cfg>), dim3(grid), dim3(512), 0, s, a, tm, tn,
                       c.qo, c.up);
  }
  return hipGetLastError();
}

tg_status run(const Call& c, const Scratch& ws, tg_stream_t stream) {
  tg_status st = validate(c);
  if (st != TG_SUCCESS) return st;
  if (c.a.M == 0 || c.a.N == 0) return TG_SUCCESS;
  const Path p = path_of(c);
  if (grid_of(c, p) >= (int64_t(1) << 31)) return TG_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      c.op == Op::BF16 ? launch_t<__bf16>(c, p, ws, s) : launch_t<_Float16>(c, p, ws, s);
  return e == hipSuccess ? TG_SUCCESS : TG_ERR_LAUNCH;
}

// The workspace entry points: a NULL or unaligned workspace of nonzero size
// is rejected before anything runs.
tg_status run_ws(const Call& c, void* workspace, size_t workspace_bytes, tg_stream_t stream) {
  tg_status st = validate(c);
  if (st != TG_SUCCESS) return st;
  if (workspace_bytes > 0 &&
      (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0))
    return TG_ERR_INVALID_VALUE;
  return run(c, Scratch{static_cast<char*>(workspace), workspace_bytes}, stream);
}

const char* const kSplitNames[] = {
    "skinny_64x128_swiglu_q8",         "skinny_64x128_swiglu_q8",
    "skinny_64x128_swiglu_q8_splitk2", "skinny_64x128_swiglu_q8_splitk3",
    "skinny_64x128_swiglu_q8_splitk4", "skinny_64x128_swiglu_q8_splitk5",
    "skinny_64x128_swiglu_q8_splitk6", "skinny_64x128_swiglu_q8_splitk7",
    "skinny_64x128_swiglu_q8_splitk8"};

const char* plan_name(const Call& c, size_t workspace_bytes) {
  switch (path_of(c)) {
    case Path::Skinny: {
      const size_t need = scratch_bytes(c);
      return need > 0 && workspace_bytes >= need ? kSplitNames[choose_splits(c)]
                                                 : "skinny_64x128_swiglu_q8";
    }
    case Path::Tile: return "tile_nt_256x256_swiglu_q8";
    default: return "generic16_32x128_swiglu_q8";
  }
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
                 tg::Scratch{nullptr, 0}, stream);
}

tg_status tg_gemm_bf16_swiglu_quant_fp8(int64_t M, int64_t N, int64_t K, const void* A,
                                        int64_t sam, int64_t sak, const void* Bg, const void* Bu,
                                        int64_t sbk, int64_t sbn, void* Q, int64_t sqm, float* S,
                                        int64_t ssm, int64_t ssj, tg_stream_t stream) {
  return tg::run(tg::make(tg::Op::BF16, M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q, sqm, S, ssm,
                          ssj),
                 tg::Scratch{nullptr, 0}, stream);
}

tg_status tg_gemm_f16_swiglu_quant_fp8_ws(int64_t M, int64_t N, int64_t K, const void* A,
                                          int64_t sam, int64_t sak, const void* Bg,
                                          const void* Bu, int64_t sbk, int64_t sbn, void* Q,
                                          int64_t sqm, float* S, int64_t ssm, int64_t ssj,
                                          void* workspace, size_t workspace_bytes,
                                          tg_stream_t stream) {
  return tg::run_ws(tg::make(tg::Op::F16, M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q, sqm, S, ssm,
                             ssj),
                    workspace, workspace_bytes, stream);
}

tg_status tg_gemm_bf16_swiglu_quant_fp8_ws(int64_t M, int64_t N, int64_t K, const void* A,
                                           int64_t sam, int64_t sak, const void* Bg,
                                           const void* Bu, int64_t sbk, int64_t sbn, void* Q,
                                           int64_t sqm, float* S, int64_t ssm, int64_t ssj,
                                           void* workspace, size_t workspace_bytes,
                                           tg_stream_t stream) {
  return tg::run_ws(tg::make(tg::Op::BF16, M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q, sqm, S,
                             ssm, ssj),
                    workspace, workspace_bytes, stream);
}

tg_status tg_gemm_swiglu_quant_fp8_workspace_size(int op, int64_t M, int64_t N, int64_t K,
                                                  const void* A, int64_t sam, int64_t sak,
                                                  const void* Bg, const void* Bu, int64_t sbk,
                                                  int64_t sbn, void* Q, int64_t sqm, float* S,
                                                  int64_t ssm, int64_t ssj, size_t* bytes) {
  if (bytes == nullptr || (op != 0 && op != 1)) return TG_ERR_INVALID_VALUE;
  const tg::Call c = tg::make(static_cast<tg::Op>(op), M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q,
                              sqm, S, ssm, ssj);
  const tg_status st = tg::validate(c);
  if (st != TG_SUCCESS) return st;
  *bytes = M == 0 || N == 0 ? 0 : tg::scratch_bytes(c);
  return TG_SUCCESS;
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
  return tg::plan_name(c, 0);
}

const char* tg_gemm_swiglu_quant_fp8_plan_ws(int op, int64_t M, int64_t N, int64_t K,
                                             const void* A, int64_t sam, int64_t sak,
                                             const void* Bg, const void* Bu, int64_t sbk,
                                             int64_t sbn, void* Q, int64_t sqm, float* S,
                                             int64_t ssm, int64_t ssj, size_t workspace_bytes) {
  if (op != 0 && op != 1) return nullptr;
  const tg::Call c = tg::make(static_cast<tg::Op>(op), M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q,
                              sqm, S, ssm, ssj);
  if (tg::validate(c) != TG_SUCCESS) return nullptr;
  if (M == 0 || N == 0) return "none";
  return tg::plan_name(c, workspace_bytes);
}

}  // extern "C"
