// Shared definitions of the gfx950 GEMM kernels: argument block, vector
// types, MFMA wrappers and the fp32 -> output rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tg_gemm.h"

namespace tg {

enum class Op : int { F16 = 0, BF16 = 1, FP8 = 2 };

// One GEMM call after host validation (element strides, device pointers).
struct GemmArgs {
  int64_t M, N, K;
  const void* A;
  int64_t sam, sak;
  const void* B;
  int64_t sbk, sbn;
  const float* SA;  // fp8 only
  int64_t ssam, ssak;
  const float* SB;  // fp8 only
  int64_t ssbn, ssbk;
  void* C;
  int64_t scm;
};

// Device scratch a call may use to combine the partial results of several
// workgroups (split K): `bytes` bytes at `ptr`, owned by the caller, or none
// (ptr == nullptr).  Layout shared by every kernel that uses it: the first
// kWorkspaceCounterBytes hold up to kWorkspaceCounters completion counters
// (ints), which must be zero when a kernel starts and which every kernel
// leaves zero; partial results start at kWorkspaceCounterBytes, so no call's
// partials can land on a later call's counters.
struct Scratch {
  char* ptr;
  size_t bytes;
};
constexpr int kWorkspaceCounters = 4096;
constexpr size_t kWorkspaceCounterBytes = kWorkspaceCounters * sizeof(int);

// A kernel family: whether it takes a call, and how to launch it.  Families
// with a split-K plan run it when `ws` holds at least scratch_bytes(a)
// bytes, and their allocation-free plan otherwise.
struct Variant {
  const char* name;
  bool (*accepts)(Op op, const GemmArgs& a);
  hipError_t (*launch)(Op op, const GemmArgs& a, const Scratch& ws, hipStream_t s);
  // Name of the plan a call would run with scratch `ws`; NULL: `name`.
  const char* (*plan_name)(const GemmArgs& a, const Scratch& ws);
  // Scratch bytes of the split-K plan (0: the family has none for this
  // call); NULL: never any.
  size_t (*scratch_bytes)(const GemmArgs& a);
};

// True when `ws` can hold `need` bytes of scratch (need > 0).
inline bool scratch_fits(const Scratch& ws, size_t need) {
  return need > 0 && ws.ptr != nullptr && ws.bytes >= need;
}

// Defined by each kernel source file (host functions; see the tables in api.cpp).
const Variant* variant_generic16();
const Variant* variant_generic_fp8();
const Variant* variant_tile_nt16();
const Variant* variant_tile_nn16();
const Variant* variant_skinny16();
const Variant* variant_tile_fp8();

// Group table of a grouped product, passed with the kernel arguments: the
// groups' first rows (in A and C) and first tile ids, and the strides from
// one group's B (and B scales) to the next.
constexpr int kMaxGroups = 128;
struct GroupTable {
  int G;
  int tiles_n;
  int64_t sbg;                        // elements between consecutive groups' B
  int64_t ssbg;                       // fp32 scales between consecutive groups' B scales
  int64_t row0[kMaxGroups + 1];
  int tile0[kMaxGroups + 1];
};

// Host-side checks of a product's sizes, strides and pointers (C with row
// stride scm and column stride scn); TG_SUCCESS when the call is valid.
tg_status validate_args(Op op, const GemmArgs& a, int64_t scn);

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

// 16-bit element type traits: storage is raw 16-bit codes.
template <typename T> struct Elem;
template <> struct Elem<__bf16> {
  typedef bf16x8 x8;
  typedef bf16x4 x4;
};
template <> struct Elem<_Float16> {
  typedef f16x8 x8;
  typedef f16x4 x4;
};

// D = A(32x16) * B(16x32) + C on one wave.  Lane l supplies row (l % 32) of A
// and column (l % 32) of B, eight k values each; A and B use the same k
// assignment, so any consistent assignment gives the same sum.  D: lane l
// holds column l % 32, rows 8*(v/4) + 4*(l/32) + (v%4), v = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// D = A(16x32) * B(32x16) + C.  Lane l: row / column l % 16, eight k values.
// D: lane l holds column l % 16, rows 4*(l/16) + v, v = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// fp8 (OCP E4M3FN) products with unit block exponents (E8M0 code 127 = 2^0),
// i.e. plain fp8 MFMAs.  32x32x64: lane l supplies row / column l % 32 and
// 32 k values (32 bytes); 16x16x128: row / column l % 16 and 32 k values.
__device__ __forceinline__ f32x16 mfma32x32x64_e4m3(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ f32x4 mfma16x16x128_e4m3(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// fp32 -> output type, round-to-nearest-even (v_cvt_pk_bf16_f32 for bf16,
// v_cvt_f16_f32 for fp16; both RNE, NaN preserved, overflow to inf).
template <typename T> __device__ __forceinline__ T to_out(float x) { return (T)x; }

__host__ __device__ constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace tg
