// tg_gemm_bf16_static_scratch: the workspace product tg_gemm_bf16_ws with
// its scratch in a fixed device array of the library instead of a caller's
// buffer, for callers that cannot allocate at all.
//
// The array `scratch` is a file-scope __device__ variable: each GPU the
// library runs on holds its own copy, at its own address, until the process
// ends.  Host code never passes the array's name to a kernel (on the host
// it names a stand-in, not device memory): the first call on a device, with
// that device current, takes the copy's device address with
// hipGetSymbolAddress, clears its counter area with a fill kernel on the
// call's stream (the split kernels need those counters zero when they start
// and leave them zero when they end), and keeps the address for the device.
// Every call on a device shares that device's array: calls whose work may
// overlap in time on one GPU race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "common.hpp"

namespace tg {

constexpr size_t kStaticScratchBytes = size_t(64) << 20;  // 64 MiB per GPU
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
char* g_ptr[kMaxDevices];  // per-device address of `scratch`, null until set up

__global__ void clear_counters(int* counters, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) counters[i] = 0;
}

// The device address of this device's `scratch`, set up on first use (null
// on failure, with the HIP error in `err`).
char* device_scratch(hipStream_t stream, hipError_t& err) {
  int dev = 0;
  err = hipGetDevice(&dev);
  if (err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] != nullptr) return g_ptr[dev];
  void* p = nullptr;
  err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (err != hipSuccess || p == nullptr) return nullptr;
  const int n = kWorkspaceCounters;
  hipLaunchKernelGGL(clear_counters, dim3((n + 255) / 256), dim3(256), 0, stream,
                     static_cast<int*>(p), n);
  err = hipGetLastError();
  if (err != hipSuccess) return nullptr;
  g_ptr[dev] = static_cast<char*>(p);
  return g_ptr[dev];
}

}  // namespace

// The call on the static scratch: TG_ERR_SCRATCH_LIMIT when its split plan
// needs more than the array holds (checked on the host before any HIP call).
static tg_status run_static_scratch(int64_t M, int64_t N, int64_t K, const void* A, int64_t sam,
                                    int64_t sak, const void* B, int64_t sbk, int64_t sbn, void* C,
                                    int64_t scm, int64_t scn, tg_stream_t stream) {
  size_t need = 0;
  const int iop = static_cast<int>(Op::BF16);
  tg_status st = tg_gemm_workspace_size(iop, M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, &need);
  if (st != TG_SUCCESS) return st;
  if (need > kStaticScratchBytes) return TG_ERR_SCRATCH_LIMIT;
  if (M == 0 || N == 0) return TG_SUCCESS;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = hipSuccess;
  char* p = device_scratch(s, err);
  if (p == nullptr) return TG_ERR_LAUNCH;
  return tg_gemm_bf16_ws(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, p, kStaticScratchBytes,
                         stream);
}

}  // namespace tg

extern "C" {

tg_status tg_gemm_bf16_static_scratch(int64_t M, int64_t N, int64_t K, const void* A,
                                      int64_t sam, int64_t sak, const void* B, int64_t sbk,
                                      int64_t sbn, void* C, int64_t scm, int64_t scn,
                                      tg_stream_t stream) {
  return tg::run_static_scratch(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn,
                                stream);
}

}  // extern "C"
