// Host-side launchers of the gfx950 kernels.  Arguments are validated by the
// C ABI layer before any of these is called; each returns hipGetLastError()
// after enqueueing its kernel(s) on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

hipError_t launch_pack(const void* w, int N, int K, int group_size, bool zero_point, uint32_t* qweight,
                       void* scales, uint32_t* qzeros, hipStream_t stream);

hipError_t launch_dequant(const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* w_out,
                          int N, int K, int group_size, bool zero_point, hipStream_t stream);

hipError_t launch_gemv(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros,
                       void* y, int N, int K, int group_size, bool zero_point, hipStream_t stream);

// Workspace bytes launch_gemm needs for an M x N x K product (0: none).
size_t gemm_workspace_bytes(int M, int N, int K);

// `workspace` holds gemm_workspace_bytes(M, N, K) bytes whose leading
// per-tile counters are zero; the call leaves them zero again.
hipError_t launch_gemm(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros,
                       void* y, int M, int N, int K, int group_size, bool zero_point, void* workspace,
                       hipStream_t stream);

}  // namespace awq
