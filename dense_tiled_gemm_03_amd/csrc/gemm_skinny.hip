// Skinny fp16 / bf16 C = A * B for M <= 64 with both operands K-contiguous
// (A row-major, B stored N x K): the decode-like 64 x 7168 x 7168 shape on
// the 7168 hidden size of "TileKernels deep dive" (sections 5.1, 8.1).
//
// Here the product is bound by HBM: B (N x K) is read exactly once and is
// ~98% of the bytes, so the kernel is laid out to keep as many B bytes in
// flight as the LDS holds, using the tile loop of "TileKernels deep dive"
// section 3.1 (clear an fp32 tile, accumulate C tile += A tile * B tile over
// K, round once):
//  - a workgroup owns 128 columns of C and all (up to 64) rows, over one of
//    `splits` equal ranges of K (split-K across workgroups, so that there
//    are about as many workgroups as CUs); its 4 waves each own 32 columns
//    and share the A slice;
//  - 64-wide K slices go HBM -> LDS with buffer_load_dwordx4 ... lds (whole
//    128-byte lines; B with the non-temporal policy, since it is read once
//    while A is read by every strip) into a 6-stage ring shared by the 4
//    waves: five slices (80 KiB of B) in flight per workgroup; one barrier
//    per slice; each slice's fragments are read from LDS while the previous
//    slice's MFMAs run; nothing is loaded past the workgroup's K range;
//  - 32x32x16 MFMAs: per slice, 2 x 1 blocks x 4 k-steps per wave;
//  - each workgroup writes its fp32 64 x 128 partial tile to scratch; the
//    last of a column strip's workgroups to finish (a device-scope counter)
//    adds the strip's partial tiles in split order, rounds once and stores C,
//    and clears the counter for the next call.  With one split the partial
//    tile is rounded and stored directly.
// LDS chunk swizzle, edges and descriptors as in the N x K tile kernel:
// chunk c of row r at position c ^ ((r >> 1) & 7); rows past M / N read as
// zero through the descriptor bounds; chunks past K (or past the
// workgroup's K range) get an out-of-range offset; stores are masked.
#include "tile_mfma.hpp"

namespace tg {
namespace {

using tile::kOutOfRange;
using tile::load_lds16;
using tile::load_lds16_nt;
using tile::make_desc;

constexpr int SM = 64;                     // rows of C per workgroup (all of M)
constexpr int SN = 128;                    // columns of C per workgroup (32 per wave)
constexpr int SK = 64;                     // k per slice
constexpr int SSTAGES = 6;                 // LDS ring depth
constexpr int ROWB = SK * 2;               // 128 bytes per LDS row
constexpr int STAGE = (SM + SN) * ROWB;    // 24 KiB
constexpr int A_LD = SM / 8 / 4;           // 1 KiB loads per wave per slice (A)
constexpr int B_LD = SN / 8 / 4;           // (B)
constexpr int NLD = A_LD + B_LD;           // 6
constexpr int RED_PITCH = SN + 4;          // fp32 tile row pitch in LDS (words)
constexpr int kCus = 256;
constexpr int kMinSlices = 8;              // fewest K slices per split
constexpr int kCoherent = 0x10;            // sc1: device-coherent buffer access
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
static_assert(SSTAGES * NLD <= 63, "loads in flight must fit the vmcnt counter");
static_assert(SM * RED_PITCH * 4 <= SSTAGES * STAGE, "reduction tile must fit the ring");

template <typename T>
__global__ __launch_bounds__(256) void gemm16_skinny(GemmArgs a, int splits, float* part,
                                                     int* counters) {
  typedef typename Elem<T>::x8 T8;
  __shared__ __attribute__((aligned(1024))) char lds[SSTAGES * STAGE];  // 144 KiB
  __shared__ int last;  // this workgroup is the strip's last to finish
  const uint32_t lds32 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int strip = blockIdx.x / splits, split = blockIdx.x % splits;
  const int64_t n0 = (int64_t)strip * SN;
  const int K = (int)a.K;
  const uint32_t lda = (uint32_t)a.sam, ldb = (uint32_t)a.sbn;
  const int rows_a = (int)a.M;  // <= 64
  const int rows_b = (int)min<int64_t>(SN, a.N - n0);
  const T* Bb = static_cast<const T*>(a.B) + n0 * a.sbn;
  const i32x4 ra = make_desc(a.A, (uint32_t)(((rows_a - 1) * lda + K) * 2));
  const i32x4 rb = make_desc(Bb, (uint32_t)(((rows_b - 1) * ldb + K) * 2));

  // This workgroup's slices [s_begin, s_end) of the nk 64-wide K slices.
  const int nk = (K + SK - 1) / SK;
  const int s_begin = (int)((int64_t)split * nk / splits);
  const int s_end = (int)((int64_t)(split + 1) * nk / splits);
  const int k_end = min(K, s_end * SK);

  // Wave w fills stage rows 16w .. 16w+15 (A) and 64 + 32w .. 64+32w+31 (B),
  // eight rows per load; lane l writes row 8m + (l >> 3) of the stage at
  // chunk position l & 7, i.e. logical chunk (l & 7) ^ (4 (m & 1) + (l >> 4)).
  const uint32_t lrow = lane >> 3;
  const uint32_t lc0 = (lane & 7) ^ (lane >> 4), lc1 = (lane & 7) ^ (4 + (lane >> 4));
  auto load_slice = [&](int slot, int slice) {
    // past this workgroup's range there is nothing to load (a load that
    // would fetch nothing still costs the CU's load pipe a full issue)
    if (slice >= s_end) return;
    const int k0 = slice * SK;
    const uint32_t stage = lds32 + slot * STAGE;
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const bool is_a = j < A_LD;
      const int jj = is_a ? j : j - A_LD;
      const uint32_t c = (jj & 1) ? lc1 : lc0;
      const uint32_t row = (is_a ? 16 * w : 32 * w) + 8 * jj + lrow;  // row of A or of the B strip
      const uint32_t group = is_a ? 2 * w + jj : 8 + 4 * w + jj;     // 8-row group in the stage
      const bool kin = k0 + 8 * (int)c < k_end;
      const uint32_t off = row * (is_a ? lda : ldb) * 2 + 2 * k0 + 16 * c;
      // B is read once (non-temporal); A is shared by every strip
      if (is_a)
        load_lds16(ra, stage + group * 1024, kin ? off : kOutOfRange);
      else
        load_lds16_nt(rb, stage + group * 1024, kin ? off : kOutOfRange);
    }
  };

  // Fragment reads (32x32x16): row (32-aligned base) + (l & 31), chunk
  // 2s + (l >> 5) for k16 step s, at position chunk ^ ((l >> 1) & 7).
  const int sw = (lane >> 1) & 7;
  int rd[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) rd[s] = (lane & 31) * ROWB + (((2 * s + (lane >> 5)) ^ sw) * 16);
  const int b_rows = (SM + 32 * w) * ROWB;

  // Two accumulators per row block (k16-step parity) keep the dependent MFMA
  // chains short; they are added before the epilogue.
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][p][v] = 0.0f;

  const int count = s_end - s_begin;
  // Fragments of two slices alternate: slice i + 1 is read from LDS while
  // slice i's MFMAs run.
  T8 fa0[2][4], fa1[2][4], fb[2][4];
  auto read_slice = [&](int buf, int slot) {
    const char* base = lds + slot * STAGE;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      fa0[buf][s] = *reinterpret_cast<const T8*>(base + rd[s]);
      fa1[buf][s] = *reinterpret_cast<const T8*>(base + 32 * ROWB + rd[s]);
      fb[buf][s] = *reinterpret_cast<const T8*>(base + b_rows + rd[s]);
    }
  };
  // One slice: wait until slice i + 1 has landed and every wave's reads of
  // slice i are done; refill slice i's slot with slice i + SSTAGES; read
  // slice i + 1; multiply slice i.
  // The waits count loads: slice i + 1 is complete once at most the loads
  // of the SSTAGES - 2 slices issued after it are outstanding.  Near the end
  // of the range fewer slices follow (nothing is loaded past it), so there
  // the wait is for every load.
  auto step = [&](int i, int cur) {
    if (i + SSTAGES - 1 < count)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((SSTAGES - 2) * NLD) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");
    load_slice(i % SSTAGES, s_begin + i + SSTAGES);
    read_slice(cur ^ 1, (i + 1) % SSTAGES);
    __builtin_amdgcn_sched_barrier(0);  // reads ahead of the MFMAs
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      acc[0][s & 1] = mfma32x32x16(fa0[cur][s], fb[cur][s], acc[0][s & 1]);
      acc[1][s & 1] = mfma32x32x16(fa1[cur][s], fb[cur][s], acc[1][s & 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int p = 0; p < SSTAGES; ++p) load_slice(p, s_begin + p);
  if (SSTAGES <= count)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((SSTAGES - 1) * NLD) : "memory");
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
  // every load has landed (the last steps wait for all); once every wave is
  // past its last reads the LDS is reused for the fp32 tile
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // The 64 x 128 fp32 tile through LDS: wave w's lane l holds column
  // 32w + (l & 31), rows 32i + 8(v/4) + 4(l >> 5) + (v % 4).
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      red[row * RED_PITCH + 32 * w + (lane & 31)] = acc[i][0][v] + acc[i][1][v];
    }
  __syncthreads();
  // Thread t, step e handles float4 q = 256 e + t of the tile (row q >> 5,
  // columns 4 (q & 31) .. + 3): consecutive lanes touch consecutive 16 bytes
  // in LDS, in scratch and (8 bytes) in C.
  const int t = threadIdx.x;
  f32x4 x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int q = 256 * e + t;
    x[e] = *reinterpret_cast<const f32x4*>(red + (q >> 5) * RED_PITCH + 4 * (q & 31));
  }

  if (splits > 1) {
    // Publish this split's partial tile, then count the strip's finished
    // splits; the last one sums all partial tiles in split order (so the
    // result does not depend on which finishes last).  The tiles are written
    // and read with device-coherent (sc1) accesses, and every wave waits for
    // its writes to complete before the barrier that precedes the counter
    // increment, so the last workgroup reads every tile whole.
    // Only the rows of C are stored and read (row (256 e + t) >> 5 < M).
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        part + (int64_t)strip * splits * SM * SN, (short)0, splits * SM * SN * 4, 0x00020000);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (8 * e + (t >> 5) < a.M)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x[e]), rp,
                                               (split * SM * SN + 4 * (256 * e + t)) * 4, 0,
                                               kCoherent);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t == 0) last = atomicAdd(counters + strip, 1) == splits - 1;
    __syncthreads();
    if (!last) return;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // four splits' tiles in flight at a time, added in split order
    for (int sp0 = 0; sp0 < splits; sp0 += 4) {
      u32x4 y[4][8];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          y[j][e] = 8 * e + (t >> 5) < a.M && sp0 + j < splits
                        ? __builtin_amdgcn_raw_buffer_load_b128(
                              rp, ((sp0 + j) * SM * SN + 4 * (256 * e + t)) * 4, 0, kCoherent)
                        : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (sp0 + j < splits)
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] += __builtin_bit_cast(f32x4, y[j][e]);
    }
    if (t == 0) __hip_atomic_store(counters + strip, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  typedef typename Elem<T>::x4 T4;
  T* Cb = static_cast<T*>(a.C);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int q = 256 * e + t, row = q >> 5, col = 4 * (q & 31);
    if (row >= a.M) continue;
    T* C = Cb + (int64_t)row * a.scm + n0 + col;
    T4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = to_out<T>(x[e][j]);
    if (n0 + col + 4 <= a.N && (reinterpret_cast<uintptr_t>(C) & 7) == 0) {
      *reinterpret_cast<T4*>(C) = o;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n0 + col + j < a.N) C[j] = o[j];
    }
  }
}

// The allocation-free skinny plan: each workgroup owns a 32-column strip of
// C (all rows, up to 64) over the whole of K, so nothing is combined across
// workgroups; its 4 waves split each 64-wide K slice instead, wave w taking
// the slice's k16 step w, and their four fp32 partial tiles are added in
// wave order through LDS at the end.  Same loads, swizzle, descriptors and
// edges as gemm16_skinny.  Every workgroup reads all of A (from L2, shared
// by every strip) and its 32 rows of B (from HBM), so the two streams have
// different latencies: A and B have LDS rings of their own (WA_ST stages of
// MT rows of A, WB_ST of 4 KiB of B), waves 0-1 load only A and waves 2-3
// only B, so that each wave's wait counts one stream.  Slices go in groups
// of WP per barrier (a slice is only 2 MFMAs per wave; the barrier, the
// fragment reads and their LDS latency are paid once per group).  The kernel
// takes MT = 32 rows of A per stage for M <= 32 and 64 otherwise: the B ring
// gets the LDS the smaller A stages free (28 stages against 16), so a decode
// step with few rows keeps more of B, the stream from HBM, in flight.
constexpr int WN = 32;                          // columns of C per workgroup
constexpr int WA_ST = 12;                       // stages of the A ring
constexpr int WP = 4;                           // slices per barrier
constexpr int WB_BYTES = WN * ROWB;             // 4 KiB: one B slice
constexpr int WRED_PITCH = WN + 4;              // fp32 row pitch of the partial tiles in LDS

template <int MT>
struct WCfg {
  static constexpr int A_BYTES = MT * ROWB;    // one A slice
  static constexpr int A_LD = MT / 16;         // loads per slice of an A wave
  static constexpr int B_ST = (160 * 1024 - WA_ST * A_BYTES) / WB_BYTES / WP * WP;
  static constexpr int LDS = WA_ST * A_BYTES + B_ST * WB_BYTES;
  static_assert(MT == 32 || MT == 64, "32 or 64 rows");
  static_assert(LDS <= 160 * 1024, "rings must fit the LDS");
  static_assert(WA_ST % WP == 0 && B_ST % WP == 0 && WA_ST >= 2 * WP && B_ST >= 2 * WP,
                "rings hold whole groups, two groups at least");
  static_assert((WA_ST - WP) * A_LD <= 63 && (B_ST - WP) * 2 <= 63,
                "loads in flight must fit the vmcnt counter");
  static_assert(4 * MT * WRED_PITCH * 4 <= LDS, "partial tiles must fit the rings");
};

template <typename T, int MT>
__global__ __launch_bounds__(256) void gemm16_skinny_wsplit(GemmArgs a) {
  typedef typename Elem<T>::x8 T8;
  typedef WCfg<MT> Cfg;
  constexpr int WA_BYTES = Cfg::A_BYTES, WB_ST = Cfg::B_ST, A_LD = Cfg::A_LD;
  constexpr int NI = MT / 32;                  // 32-row blocks
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS];
  const uint32_t lds32 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * WN;
  const int K = (int)a.K;
  const uint32_t lda = (uint32_t)a.sam, ldb = (uint32_t)a.sbn;
  const int rows_b = (int)min<int64_t>(WN, a.N - n0);
  const T* Bb = static_cast<const T*>(a.B) + n0 * a.sbn;
  const i32x4 ra = make_desc(a.A, (uint32_t)((((int)a.M - 1) * lda + K) * 2));
  const i32x4 rb = make_desc(Bb, (uint32_t)(((rows_b - 1) * ldb + K) * 2));
  const int count = (K + SK - 1) / SK;
  const bool loads_a = w < 2;  // wave-uniform

  // Slot s of the A ring at s * WA_BYTES, of the B ring after the A ring.
  // A slice's 8-row groups: wave w (0, 1) loads A groups A_LD w .. A_LD w +
  // A_LD - 1, wave w (2, 3) B groups 2(w - 2) .. + 1.  Lane l writes group
  // row l >> 3 at chunk position l & 7, i.e. logical chunk (l & 7) ^ (4 (g &
  // 1) + (l >> 4)).
  const uint32_t lrow = lane >> 3;
  const uint32_t lc0 = (lane & 7) ^ (lane >> 4), lc1 = (lane & 7) ^ (4 + (lane >> 4));
  auto load_a = [&](int slice) {
    if (slice >= count) return;  // nothing past K
    const int k0 = slice * SK;
    const uint32_t stage = lds32 + (slice % WA_ST) * WA_BYTES;
#pragma unroll
    for (int j = 0; j < A_LD; ++j) {
      const int g = A_LD * w + j;
      const uint32_t c = (g & 1) ? lc1 : lc0;
      const bool kin = k0 + 8 * (int)c < K;
      const uint32_t off = (8 * g + lrow) * lda * 2 + 2 * k0 + 16 * c;
      load_lds16(ra, stage + g * 1024, kin ? off : kOutOfRange);
    }
  };
  auto load_b = [&](int slice) {
    if (slice >= count) return;
    const int k0 = slice * SK;
    const uint32_t stage = lds32 + WA_ST * WA_BYTES + (slice % WB_ST) * WB_BYTES;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int g = 2 * (w - 2) + j;
      const uint32_t c = (g & 1) ? lc1 : lc0;
      const bool kin = k0 + 8 * (int)c < K;
      const uint32_t off = (8 * g + lrow) * ldb * 2 + 2 * k0 + 16 * c;
      load_lds16_nt(rb, stage + g * 1024, kin ? off : kOutOfRange);
    }
  };
  // Waits for this wave's stream.  Before the first group: slices 0 .. WP - 1
  // landed, the ring's other ST - WP slices may be in flight.  Before the
  // group after slices i .. i + WP - 1 is read: slices .. i + 2 WP - 1 landed,
  // the ST - 2 WP issued after them may be in flight (all of them near the
  // end of K, where fewer were issued).
  auto wait_first = [&]() {
    if (loads_a) {
      if (WA_ST <= count) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((WA_ST - WP) * A_LD) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      if (WB_ST <= count) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((WB_ST - WP) * 2) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  };
  auto wait_next = [&](int i) {
    if (loads_a) {
      if (i + WA_ST <= count)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((WA_ST - 2 * WP) * A_LD) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    } else {
      if (i + WB_ST <= count)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((WB_ST - 2 * WP) * 2) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    }
  };

  // Wave w's fragments of a slice (32x32x16, its k16 step w): A rows
  // (l & 31) and 32 + (l & 31), B rows (l & 31), chunk 2w + (l >> 5) at
  // position chunk ^ ((l >> 1) & 7).
  const int rd = (lane & 31) * ROWB + (((2 * w + (lane >> 5)) ^ ((lane >> 1) & 7)) * 16);
  f32x16 acc[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
  T8 fa[2][WP][NI], fb[2][WP];  // [buffer][slice of the group][32-row block]
  auto read_group = [&](int buf, int first) {
#pragma unroll
    for (int h = 0; h < WP; ++h) {
      const char* ab = lds + ((first + h) % WA_ST) * WA_BYTES;
      const char* bb = lds + WA_ST * WA_BYTES + ((first + h) % WB_ST) * WB_BYTES;
#pragma unroll
      for (int i = 0; i < NI; ++i) fa[buf][h][i] = *reinterpret_cast<const T8*>(ab + 32 * i * ROWB + rd);
      fb[buf][h] = *reinterpret_cast<const T8*>(bb + rd);
    }
  };
  // The group of slices i .. i + WP - 1 (read into buffer cur): wait for the
  // next group and for every wave's reads of this one, refill this group's
  // slots with the slices a ring's depth later, read the next group,
  // multiply this one (slices past K are skipped; their fragments are stale).
  auto step = [&](int i, int cur) {
    wait_next(i);
    asm volatile("s_barrier" ::: "memory");
#pragma unroll
    for (int h = 0; h < WP; ++h) {
      if (loads_a) load_a(i + h + WA_ST);
      else load_b(i + h + WB_ST);
    }
    if (i + WP < count) read_group(cur ^ 1, i + WP);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 0; h < WP; ++h)
      if (i + h < count) {
#pragma unroll
        for (int ii = 0; ii < NI; ++ii) acc[ii] = mfma32x32x16(fa[cur][h][ii], fb[cur][h], acc[ii]);
      }
    __builtin_amdgcn_sched_barrier(0);
  };
  if (loads_a) {
#pragma unroll
    for (int p = 0; p < WA_ST; ++p) load_a(p);
  } else {
#pragma unroll
    for (int p = 0; p < WB_ST; ++p) load_b(p);
  }
  wait_first();
  asm volatile("s_barrier" ::: "memory");
  read_group(0, 0);
  int i = 0;
  for (; i + WP < count; i += 2 * WP) {
    step(i, 0);
    step(i + WP, 1);
  }
  if (i < count) step(i, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // The four waves' partial tiles through LDS: wave w's lane l holds column
  // l & 31, rows 32i + 8(v/4) + 4(l >> 5) + (v % 4).
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int i2 = 0; i2 < NI; ++i2)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = 32 * i2 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      red[(w * MT + row) * WRED_PITCH + (lane & 31)] = acc[i2][v];
    }
  __syncthreads();
  // Thread t, step e: float4 q = 256 e + t of the MT x 32 tile (row q >> 3,
  // columns 4 (q & 7) .. + 3), the sum of the four partials in wave order.
  typedef typename Elem<T>::x4 T4;
  T* Cb = static_cast<T*>(a.C);
  const int t = threadIdx.x;
#pragma unroll
  for (int e = 0; e < MT / 32; ++e) {
    const int q = 256 * e + t, row = q >> 3, col = 4 * (q & 7);
    f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ww = 0; ww < 4; ++ww)
      x += *reinterpret_cast<const f32x4*>(red + (ww * MT + row) * WRED_PITCH + col);
    if (row >= a.M) continue;
    T* C = Cb + (int64_t)row * a.scm + n0 + col;
    T4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = to_out<T>(x[j]);
    if (n0 + col + 4 <= a.N && (reinterpret_cast<uintptr_t>(C) & 7) == 0) {
      *reinterpret_cast<T4*>(C) = o;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n0 + col + j < a.N) C[j] = o[j];
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

// Split K so that the grid is about one workgroup per CU, keeping at least
// kMinSlices slices per split.
int choose_splits(const GemmArgs& a) {
  const int64_t strips = cdiv(a.N, SN), nk = cdiv(a.K, SK);
  int64_t s = kCus / strips;
  if (s > nk / kMinSlices) s = nk / kMinSlices;
  return s < 1 ? 1 : (int)s;
}

// Whether the split plan beats the 32-column strips over all of K (both
// stream the same B bytes per CU; the split saves A bytes and fills the CUs
// when the strip grid does not, but pays a fixed cost for the combine).  As
// measured: when each strip workgroup has a long run of K slices (strip
// rounds x slices >= 96), or when the strip grid fills at most half the
// CUs.  Short K on a full strip grid (64 x 7168 x 2048: 15.8 us split
// against 11.1) stays on the strips.
constexpr int kLongSlices = 96;
bool split_pays(const GemmArgs& a) {
  const int64_t strip_wgs = cdiv(a.N, WN), nk = cdiv(a.K, SK);
  return cdiv(strip_wgs, kCus) * nk >= kLongSlices || strip_wgs <= kCus / 2;
}

// Scratch of the split plan: one counter per strip in the fixed counter
// area, then each split's 64 x 128 fp32 partial tile (0: no split).
size_t scratch_bytes(const GemmArgs& a) {
  const int64_t strips = cdiv(a.N, SN);
  const int splits = choose_splits(a);
  if (splits == 1 || !split_pays(a) || strips > kWorkspaceCounters) return 0;
  return kWorkspaceCounterBytes + (size_t)strips * splits * SM * SN * 4;
}

// Plans: with scratch for the split where it pays, 64 x 128 strips split K
// across workgroups; otherwise 32-column strips over all of K (waves split
// each slice); when K is too short to split or the strips alone fill the
// CUs, 64 x 128 strips unsplit.
enum class Skinny { Strip128, Split128, Strip32 };
Skinny choose(const GemmArgs& a, const Scratch& ws, int& splits) {
  splits = choose_splits(a);
  if (splits == 1) return Skinny::Strip128;
  if (split_pays(a) && scratch_fits(ws, scratch_bytes(a))) return Skinny::Split128;
  splits = 1;
  return Skinny::Strip32;
}

hipError_t launch(Op op, const GemmArgs& a, const Scratch& ws, hipStream_t stream) {
  int splits;
  const Skinny plan = choose(a, ws, splits);
  const dim3 block(256);
  if (plan == Skinny::Strip32) {
    const dim3 grid((unsigned)cdiv(a.N, WN));
    if (a.M <= 32) {
      if (op == Op::BF16)
        hipLaunchKernelGGL((gemm16_skinny_wsplit<__bf16, 32>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((gemm16_skinny_wsplit<_Float16, 32>), grid, block, 0, stream, a);
    } else {
      if (op == Op::BF16)
        hipLaunchKernelGGL((gemm16_skinny_wsplit<__bf16, 64>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((gemm16_skinny_wsplit<_Float16, 64>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
  }
  int* counters = nullptr;
  float* part = nullptr;
  if (plan == Skinny::Split128) {
    counters = reinterpret_cast<int*>(ws.ptr);
    part = reinterpret_cast<float*>(ws.ptr + kWorkspaceCounterBytes);
  }
  const dim3 grid((unsigned)(cdiv(a.N, SN) * splits));
  if (op == Op::BF16)
    hipLaunchKernelGGL(gemm16_skinny<__bf16>, grid, block, 0, stream, a, splits, part, counters);
  else
    hipLaunchKernelGGL(gemm16_skinny<_Float16>, grid, block, 0, stream, a, splits, part,
                       counters);
  return hipGetLastError();
}

const char* const kSplitNames[] = {"", "skinny_64x128", "skinny_64x128_splitk2",
                                   "skinny_64x128_splitk3", "skinny_64x128_splitk4",
                                   "skinny_64x128_splitk5", "skinny_64x128_splitk6",
                                   "skinny_64x128_splitk7", "skinny_64x128_splitk8"};
const char* name_of(const GemmArgs& a, const Scratch& ws) {
  int splits;
  const Skinny plan = choose(a, ws, splits);
  if (plan == Skinny::Strip32) return "skinny_64x32";
  return splits <= 8 ? kSplitNames[splits] : "skinny_64x128_splitk";
}

}  // namespace

const Variant* variant_skinny16() {
  static const Variant v = {"skinny", accepts, launch, name_of, scratch_bytes};
  return &v;
}

}  // namespace tg
