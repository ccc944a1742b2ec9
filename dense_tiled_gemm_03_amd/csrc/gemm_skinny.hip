// Skinny fp16 / bf16 C = A * B for M <= 64 with both operands K-contiguous
// (A row-major, B stored N x K): the decode-like 64 x 7168 x 7168 shape on
// the 7168 hidden size of "TileKernels deep dive" (sections 5.1, 8.1).
//
// Here the product is bound by HBM: B (N x K) is read exactly once and is
// ~98% of the bytes; A (64 x K) is re-read from L2 by every workgroup.  The
// tile loop of "TileKernels deep dive" section 3.1 (clear an fp32 tile,
// accumulate C tile += A tile * B tile over K, round once) is laid out so
// that as many bytes as possible are in flight:
//  - one workgroup per 32 columns of C, all (up to 64) rows;
//  - K is split across the 4 waves by 64-wide slices (slice s goes to wave
//    s % 4), each wave with its own 3-stage LDS ring filled by
//    buffer_load_dwordx4 ... lds, so waves never wait on each other in the
//    main loop and every wave keeps two slices (24 KiB) of loads in flight;
//  - loads cover whole 128-byte lines (8 rows x 64 k per instruction);
//    partial-line loads move far fewer bytes per clock on gfx950;
//  - 32x32x16 MFMAs: per 64-wide slice, 2 x 1 blocks per wave;
//  - the four partial 64 x 32 fp32 tiles are summed through LDS, rounded
//    once and stored 16 bytes per lane.
// LDS chunk swizzle, edges and descriptors as in the N x K tile kernel:
// chunk c of row r at position c ^ ((r >> 1) & 7); rows past M / N read as
// zero through the descriptor bounds; chunks past K get an out-of-range
// offset; stores are masked.
#include "common.hpp"

namespace tg {
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int SM = 64;          // rows of C per workgroup (all of M)
constexpr int SN = 32;          // columns of C per workgroup
constexpr int SK = 64;          // k per slice
constexpr int SSTAGES = 3;      // LDS ring depth per wave
constexpr int ROWB = SK * 2;    // 128 bytes per LDS row
constexpr int SLICE_BYTES = (SM + SN) * ROWB;  // 12 KiB
constexpr int A_LD = SM / 8, B_LD = SN / 8;    // 1 KiB loads per slice
constexpr int NLD = A_LD + B_LD;               // 12

// Raw buffer descriptor over [base, base + bytes).  The fields go through
// readfirstlane: they are wave-uniform, and saying so keeps the descriptor in
// scalar registers (otherwise every load can become a per-lane waterfall).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* q = reinterpret_cast<void*>((uint64_t)hi << 32 | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

template <typename T>
__global__ __launch_bounds__(256) void gemm16_skinny(GemmArgs a) {
  typedef typename Elem<T>::x8 T8;
  __shared__ __attribute__((aligned(1024))) char lds[4 * SSTAGES * SLICE_BYTES];  // 144 KiB

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * SN;
  const int K = (int)a.K;
  const uint32_t lda = (uint32_t)a.sam, ldb = (uint32_t)a.sbn;
  const int rows_a = (int)a.M;                                 // <= 64
  const int rows_b = (int)min<int64_t>(SN, a.N - n0);
  const T* Bb = static_cast<const T*>(a.B) + n0 * a.sbn;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, (uint32_t)(((rows_a - 1) * lda + K) * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb, (uint32_t)(((rows_b - 1) * ldb + K) * 2));
  char* ring = lds + w * SSTAGES * SLICE_BYTES;

  // Load j (0 .. NLD-1) of a slice fills LDS rows 8j .. 8j+7 of the slice
  // (A rows 0..63, then B rows 64..95); lane l writes row 8j + (l >> 3),
  // chunk position l & 7, i.e. logical chunk (l & 7) ^ ((row >> 1) & 7)
  // = (l & 7) ^ (4 * (j & 1) + (l >> 4)).
  const uint32_t lrow = lane >> 3;
  const uint32_t lc0 = (lane & 7) ^ (lane >> 4), lc1 = (lane & 7) ^ (4 + (lane >> 4));
  auto load_slice = [&](int slot, int k0) {
    char* base = ring + slot * SLICE_BYTES;
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const uint32_t c = (j & 1) ? lc1 : lc0;
      const bool kin = k0 + 8 * (int)c < K;
      const uint32_t row = 8 * (j < A_LD ? j : j - A_LD) + lrow;
      const uint32_t off = row * (j < A_LD ? lda : ldb) * 2 + 2 * k0 + 16 * c;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(j < A_LD ? ra : rb, (lds_ptr_t)(base + j * 1024), 16,
                                               kin ? off : kOutOfRange, 0, 0, 0);
    }
  };

  // Fragment reads (32x32x16): row (32-aligned base) + (l & 31), chunk
  // 2s + (l >> 5) for k16 step s, at position chunk ^ ((l >> 1) & 7).
  const int sw = (lane >> 1) & 7;
  int rd[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) rd[s] = (lane & 31) * ROWB + (((2 * s + (lane >> 5)) ^ sw) * 16);

  // Four accumulators (row block i, k16-step parity p) keep the dependent
  // MFMA chains short; the parities are added before the reduction.
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][p][v] = 0.0f;

  // Wave w takes slices w, w + 4, w + 8, ...; its ring holds slices i (being
  // read), i + 1 and i + 2 (in flight).  Slices past K fetch out of range
  // (no traffic, zeros), so every wave runs the same uniform loop.  Per
  // slice all twelve fragments are read before the MFMAs, so the slice
  // costs one LDS round trip.
  const int nk = (K + SK - 1) / SK;
  const int my = (nk - w + 3) / 4;   // slices of this wave
#pragma unroll
  for (int s = 0; s < SSTAGES - 1; ++s) load_slice(s, (w + 4 * s) * SK);
  for (int i = 0; i < my; ++i) {
    // the slot refilled here held slice i - 1, whose reads this wave has
    // already consumed in MFMAs
    load_slice((i + SSTAGES - 1) % SSTAGES, (w + 4 * (i + SSTAGES - 1)) * SK);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((SSTAGES - 1) * NLD) : "memory");
    const char* base = ring + (i % SSTAGES) * SLICE_BYTES;
    T8 fa0[4], fa1[4], fb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      fa0[s] = *reinterpret_cast<const T8*>(base + rd[s]);
      fa1[s] = *reinterpret_cast<const T8*>(base + 32 * ROWB + rd[s]);
      fb[s] = *reinterpret_cast<const T8*>(base + SM * ROWB + rd[s]);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      acc[0][s & 1] = mfma32x32x16(fa0[s], fb[s], acc[0][s & 1]);
      acc[1][s & 1] = mfma32x32x16(fa1[s], fb[s], acc[1][s & 1]);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Sum the four partial tiles: wave w stores its 64 x 32 fp32 tile at
  // red[w][row][col]; lane l holds column l & 31, rows 32i + 8(v/4) +
  // 4(l >> 5) + (v % 4).
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      red[(w * SM + row) * SN + (lane & 31)] = acc[i][0][v] + acc[i][1][v];
    }
  __syncthreads();
  // thread t: row t >> 2, columns 8 * (t & 3) .. +7
  const int t = threadIdx.x, row = t >> 2, c0 = 8 * (t & 3);
  float sum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sum[e] = 0.0f;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const f32x4* src = reinterpret_cast<const f32x4*>(red + (p * SM + row) * SN + c0);
    const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sum[e] += x0[e];
      sum[4 + e] += x1[e];
    }
  }
  if (row < a.M) {
    T* C = static_cast<T*>(a.C) + (int64_t)row * a.scm + n0 + c0;
    if (n0 + c0 + 8 <= a.N && (reinterpret_cast<uintptr_t>(C) & 15) == 0) {
      typename Elem<T>::x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = to_out<T>(sum[e]);
      *reinterpret_cast<typename Elem<T>::x8*>(C) = o;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n0 + c0 + e < a.N) C[e] = to_out<T>(sum[e]);
    }
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// At most 64 rows, both operands K-contiguous with 16-byte aligned rows;
// offsets inside one operand tile fit the 31-bit range the descriptors use.
bool accepts(Op op, const GemmArgs& a) {
  if (op == Op::FP8) return false;
  if (a.M > SM || a.K == 0 || a.K % 8 != 0) return false;
  if (a.sak != 1 || a.sbk != 1) return false;
  if (a.sam % 8 != 0 || a.sbn % 8 != 0) return false;
  if (!aligned16(a.A) || !aligned16(a.B)) return false;
  const int64_t lim = int64_t(1) << 30;
  if (SM * a.sam * 2 + 2 * a.K >= lim || SN * a.sbn * 2 + 2 * a.K >= lim) return false;
  if (a.N > (int64_t(1) << 30)) return false;
  return true;
}

hipError_t launch(Op op, const GemmArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)cdiv(a.N, SN)), block(256);
  if (op == Op::BF16)
    hipLaunchKernelGGL(gemm16_skinny<__bf16>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(gemm16_skinny<_Float16>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

const Variant* variant_skinny16() {
  static const Variant v = {"skinny_64x32", accepts, launch, nullptr};
  return &v;
}

}  // namespace tg
