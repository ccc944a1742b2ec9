// The C-ABI entry points: host-side validation (no HIP call before it
// passes), kernel selection, launch and error mapping.
#include "../../include/tg_gemm.h"

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace tg {

// M <= 64 block-scaled fp8 products (gemm_skinny_fp8.hip)
const Variant* variant_skinny_fp8();

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

// (n - 1) * stride without int64 overflow; false if it overflows.
bool extent_ok(int64_t n, int64_t stride) {
  if (n <= 1 || stride == 0) return true;
  int64_t r;
  return !__builtin_mul_overflow(n - 1, stride, &r);
}

}  // namespace

// Returns TG_SUCCESS when the call is valid (it may still be a no-op).
tg_status validate_args(Op op, const GemmArgs& a, int64_t scn) {
  if (a.M < 0 || a.N < 0 || a.K < 0) return TG_ERR_INVALID_VALUE;
  if (a.sam < 0 || a.sak < 0 || a.sbk < 0 || a.sbn < 0 || a.scm < 0 || scn < 0)
    return TG_ERR_INVALID_VALUE;
  if (op == Op::FP8 && (a.ssam < 0 || a.ssak < 0 || a.ssbn < 0 || a.ssbk < 0))
    return TG_ERR_INVALID_VALUE;
  if (a.M == 0 || a.N == 0) return TG_SUCCESS;  // nothing to compute, nothing to check
  if (a.C == nullptr) return TG_ERR_INVALID_VALUE;
  if (a.K > 0) {
    if (a.A == nullptr || a.B == nullptr) return TG_ERR_INVALID_VALUE;
    if (op == Op::FP8 && (a.SA == nullptr || a.SB == nullptr)) return TG_ERR_INVALID_VALUE;
  }
  if (a.M > 1 && a.scm < a.N) return TG_ERR_INVALID_VALUE;  // rows of C would overlap
  if (!extent_ok(a.M, a.sam) || !extent_ok(a.K, a.sak) || !extent_ok(a.K, a.sbk) ||
      !extent_ok(a.N, a.sbn) || !extent_ok(a.M, a.scm))
    return TG_ERR_INVALID_VALUE;
  {
    // largest element offsets; their byte addresses must not overflow either
    const int64_t lim = int64_t(1) << 61;
    int64_t ra, rb, rc;
    if (__builtin_add_overflow((a.M - 1) * a.sam, (a.K > 0 ? a.K - 1 : 0) * a.sak, &ra) ||
        __builtin_add_overflow((a.K > 0 ? a.K - 1 : 0) * a.sbk, (a.N - 1) * a.sbn, &rb) ||
        __builtin_add_overflow((a.M - 1) * a.scm, a.N - 1, &rc) || ra >= lim || rb >= lim ||
        rc >= lim)
      return TG_ERR_INVALID_VALUE;
  }
  if (op == Op::FP8) {
    const int64_t kb = cdiv(a.K, 128), nb = cdiv(a.N, 128);
    if (!extent_ok(a.M, a.ssam) || !extent_ok(kb, a.ssak) || !extent_ok(nb, a.ssbn) ||
        !extent_ok(kb, a.ssbk))
      return TG_ERR_INVALID_VALUE;
  }
  if (scn != 1) return TG_ERR_UNSUPPORTED;
  if (a.M > kMaxDim || a.N > kMaxDim || a.K > kMaxDim) return TG_ERR_UNSUPPORTED;
  return TG_SUCCESS;
}

namespace {

struct Call {
  Op op;
  GemmArgs a;
  int64_t scn;
};

tg_status validate(const Call& c) { return validate_args(c.op, c.a, c.scn); }

// Kernel tables, most specialised first; the last entry takes every call.
const Variant* (*const kTable16[])() = {variant_skinny16, variant_tile_nt16, variant_tile_nn16,
                                          variant_generic16};
const Variant* (*const kTableFp8[])() = {variant_skinny_fp8, variant_tile_fp8,
                                           variant_generic_fp8};

const Variant* select(const Call& c) {
  if (c.op == Op::FP8) {
    for (auto get : kTableFp8)
      if (get()->accepts(c.op, c.a)) return get();
  } else {
    for (auto get : kTable16)
      if (get()->accepts(c.op, c.a)) return get();
  }
  return nullptr;  // unreachable: the generic kernels accept every call
}

// A caller's workspace: none (bytes == 0), or a 256-byte aligned device
// buffer.  TG_SUCCESS when usable.
tg_status check_workspace(const void* ws, size_t bytes) {
  if (bytes == 0) return TG_SUCCESS;
  if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 255) != 0) return TG_ERR_INVALID_VALUE;
  return TG_SUCCESS;
}

tg_status run(const Call& c, const Scratch& ws, tg_stream_t stream) {
  tg_status st = validate(c);
  if (st != TG_SUCCESS) return st;
  if (c.a.M == 0 || c.a.N == 0) return TG_SUCCESS;
  const Variant* v = select(c);
  if (v == nullptr) return TG_ERR_UNSUPPORTED;
  hipError_t e = v->launch(c.op, c.a, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TG_SUCCESS : TG_ERR_LAUNCH;
}

Call make16(Op op, int64_t M, int64_t N, int64_t K, const void* A, int64_t sam, int64_t sak,
            const void* B, int64_t sbk, int64_t sbn, void* C, int64_t scm, int64_t scn) {
  Call c;
  c.op = op;
  c.a = GemmArgs{M, N, K, A, sam, sak, B, sbk, sbn, nullptr, 0, 0, nullptr, 0, 0, C, scm};
  c.scn = scn;
  return c;
}

// The call tg_gemm_plan / tg_gemm_workspace_size describe (op 0..2); false
// for an unknown op.
bool describe(int op, int64_t M, int64_t N, int64_t K, const void* A, int64_t sam, int64_t sak,
              const void* B, int64_t sbk, int64_t sbn, void* C, int64_t scm, int64_t scn,
              Call& c) {
  if (op < 0 || op > 2) return false;
  c = make16(static_cast<Op>(op), M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn);
  if (c.op == Op::FP8) {
    // scale pointers do not affect the choice; stand-ins pass the null checks
    static const float dummy = 0.0f;
    c.a.SA = &dummy;
    c.a.SB = &dummy;
  }
  return true;
}

}  // namespace
}  // namespace tg

extern "C" {

const char* tg_status_string(tg_status s) {
  switch (s) {
    case TG_SUCCESS: return "TG_SUCCESS: success";
    case TG_ERR_INVALID_VALUE: return "TG_ERR_INVALID_VALUE: invalid argument";
    case TG_ERR_UNSUPPORTED: return "TG_ERR_UNSUPPORTED: unsupported layout or size";
    case TG_ERR_LAUNCH: return "TG_ERR_LAUNCH: kernel launch failed";
    case TG_ERR_SCRATCH_LIMIT:
      return "TG_ERR_SCRATCH_LIMIT: the call's split plan needs more scratch than the fixed "
             "64 MiB array holds";
    default: return "unknown tg_status";
  }
}

tg_status tg_gemm_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t sam, int64_t sak,
                      const void* B, int64_t sbk, int64_t sbn, void* C, int64_t scm, int64_t scn,
                      tg_stream_t stream) {
  return tg::run(tg::make16(tg::Op::F16, M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn),
                 tg::Scratch{nullptr, 0}, stream);
}

tg_status tg_gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t sam, int64_t sak,
                       const void* B, int64_t sbk, int64_t sbn, void* C, int64_t scm, int64_t scn,
                       tg_stream_t stream) {
  return tg::run(tg::make16(tg::Op::BF16, M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn),
                 tg::Scratch{nullptr, 0}, stream);
}

tg_status tg_gemm_fp8_blockscaled(int64_t M, int64_t N, int64_t K, const void* A, int64_t sam,
                                  int64_t sak, const float* SA, int64_t ssam, int64_t ssak,
                                  const void* B, int64_t sbk, int64_t sbn, const float* SB,
                                  int64_t ssbn, int64_t ssbk, void* C, int64_t scm, int64_t scn,
                                  tg_stream_t stream) {
  tg::Call c;
  c.op = tg::Op::FP8;
  c.a = tg::GemmArgs{M, N, K, A, sam, sak, B, sbk, sbn, SA, ssam, ssak, SB, ssbn, ssbk, C, scm};
  c.scn = scn;
  return tg::run(c, tg::Scratch{nullptr, 0}, stream);
}

tg_status tg_gemm_f16_ws(int64_t M, int64_t N, int64_t K, const void* A, int64_t sam,
                         int64_t sak, const void* B, int64_t sbk, int64_t sbn, void* C,
                         int64_t scm, int64_t scn, void* workspace, size_t workspace_bytes,
                         tg_stream_t stream) {
  const tg::Call c = tg::make16(tg::Op::F16, M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn);
  tg_status st = tg::validate(c);
  if (st == TG_SUCCESS) st = tg::check_workspace(workspace, workspace_bytes);
  if (st != TG_SUCCESS) return st;
  return tg::run(c, tg::Scratch{static_cast<char*>(workspace), workspace_bytes}, stream);
}

tg_status tg_gemm_bf16_ws(int64_t M, int64_t N, int64_t K, const void* A, int64_t sam,
                          int64_t sak, const void* B, int64_t sbk, int64_t sbn, void* C,
                          int64_t scm, int64_t scn, void* workspace, size_t workspace_bytes,
                          tg_stream_t stream) {
  const tg::Call c = tg::make16(tg::Op::BF16, M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn);
  tg_status st = tg::validate(c);
  if (st == TG_SUCCESS) st = tg::check_workspace(workspace, workspace_bytes);
  if (st != TG_SUCCESS) return st;
  return tg::run(c, tg::Scratch{static_cast<char*>(workspace), workspace_bytes}, stream);
}

tg_status tg_gemm_fp8_blockscaled_ws(int64_t M, int64_t N, int64_t K, const void* A,
                                     int64_t sam, int64_t sak, const float* SA, int64_t ssam,
                                     int64_t ssak, const void* B, int64_t sbk, int64_t sbn,
                                     const float* SB, int64_t ssbn, int64_t ssbk, void* C,
                                     int64_t scm, int64_t scn, void* workspace,
                                     size_t workspace_bytes, tg_stream_t stream) {
  tg::Call c;
  c.op = tg::Op::FP8;
  c.a = tg::GemmArgs{M, N, K, A, sam, sak, B, sbk, sbn, SA, ssam, ssak, SB, ssbn, ssbk, C, scm};
  c.scn = scn;
  tg_status st = tg::validate(c);
  if (st == TG_SUCCESS) st = tg::check_workspace(workspace, workspace_bytes);
  if (st != TG_SUCCESS) return st;
  return tg::run(c, tg::Scratch{static_cast<char*>(workspace), workspace_bytes}, stream);
}

tg_status tg_gemm_workspace_size(int op, int64_t M, int64_t N, int64_t K, const void* A,
                                 int64_t sam, int64_t sak, const void* B, int64_t sbk,
                                 int64_t sbn, void* C, int64_t scm, int64_t scn, size_t* bytes) {
  tg::Call c;
  if (bytes == nullptr || !tg::describe(op, M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, c))
    return TG_ERR_INVALID_VALUE;
  const tg_status st = tg::validate(c);
  if (st != TG_SUCCESS) return st;
  *bytes = 0;
  if (M == 0 || N == 0) return TG_SUCCESS;
  const tg::Variant* v = tg::select(c);
  if (v != nullptr && v->scratch_bytes != nullptr) *bytes = v->scratch_bytes(c.a);
  return TG_SUCCESS;
}

const char* tg_gemm_plan_ws(int op, int64_t M, int64_t N, int64_t K, const void* A, int64_t sam,
                            int64_t sak, const void* B, int64_t sbk, int64_t sbn, void* C,
                            int64_t scm, int64_t scn, size_t workspace_bytes) {
  tg::Call c;
  if (!tg::describe(op, M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, c)) return nullptr;
  if (tg::validate(c) != TG_SUCCESS) return nullptr;
  if (M == 0 || N == 0) return "none";
  const tg::Variant* v = tg::select(c);
  if (v == nullptr) return nullptr;
  // a stand-in address: only the size decides the plan
  alignas(256) static char stand_in;
  const tg::Scratch ws{workspace_bytes > 0 ? &stand_in : nullptr, workspace_bytes};
  return v->plan_name ? v->plan_name(c.a, ws) : v->name;
}

const char* tg_gemm_plan(int op, int64_t M, int64_t N, int64_t K, const void* A, int64_t sam,
                         int64_t sak, const void* B, int64_t sbk, int64_t sbn, void* C,
                         int64_t scm, int64_t scn) {
  return tg_gemm_plan_ws(op, M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, 0);
}

}  // extern "C"
