// awq_gemm_noalloc: awq_gemm with its split-K workspace in a fixed
// library-owned device array instead of a caller buffer, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The contract is in include/awq.h.
//
// The array lives in this file as a file-scope __device__ variable; every GPU
// the library runs on holds its own copy (loaded with the code object, zero
// before first use) until the process ends.  In host code the array's name
// is only a stand-in for the symbol, not a device address, so its address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and only that pointer is handed to kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/awq.h"
#include "awq_launch.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceScratch {
  void* ptr = nullptr;  // device address of this device's copy of `scratch`
};
DeviceScratch g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// Zero the leading counter region (the only part a call needs at zero; every
// call leaves it zero again).  A fill kernel rather than hipMemsetAsync, so
// that a call recorded into a graph holds only kernel nodes.
__global__ __launch_bounds__(256) void clear_words(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

// The current device's scratch pointer, looked up (and its counters cleared
// on `stream`) on the first call on that device.  NULL on failure.
void* device_scratch(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  DeviceScratch& d = g_scratch[dev];
  if (d.ptr == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    const size_t words = awq::gemm_counter_bytes() / 4;
    hipLaunchKernelGGL(clear_words, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                       static_cast<uint32_t*>(p), words);
    if (hipGetLastError() != hipSuccess) return nullptr;
    d.ptr = p;
  }
  return d.ptr;
}

}  // namespace

extern "C" {

size_t awq_gemm_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

int awq_gemm_noalloc(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* y,
                     int32_t M, int32_t N, int32_t K, int32_t group_size, int32_t zero_point, void* stream) {
  // the same validation as awq_gemm, by calling it with no workspace: any
  // error other than a missing workspace is returned as it is
  const size_t need = awq_gemm_workspace_bytes(M, N, K, group_size);
  if (need == 0)
    return awq_gemm(x, qweight, scales, qzeros, y, M, N, K, group_size, zero_point, nullptr, 0, stream);
  const int st = awq_gemm(x, qweight, scales, qzeros, y, M, N, K, group_size, zero_point, nullptr, 0, stream);
  if (st != AWQ_ERR_WORKSPACE) return st;  // a validation error (nothing was launched)
  if (need > kScratchBytes) return AWQ_ERR_SCRATCH;
  void* ws = device_scratch(static_cast<hipStream_t>(stream));
  if (ws == nullptr) return AWQ_ERR_HIP;
  return awq_gemm(x, qweight, scales, qzeros, y, M, N, K, group_size, zero_point, ws, kScratchBytes, stream);
}

}  // extern "C"
