// Measurement aid, not a step of the method: a streaming read of a device
// buffer, used as the achievable HBM read rate beside the spec-sheet peak.
// The shape is the fastest of a sweep over loads in flight (2-16), work-groups
// per CU (1-32) and cached versus non-temporal loads on MI355X: 16-byte
// non-temporal loads, eight in flight per thread, one 256-thread work-group
// per CU.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fg.h"

extern "C" int fg_internal_device_cu_count(void);

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeThreads = 256;
constexpr int kProbeInFlight = 8;

// Grid-stride loop over n16 16-byte words; every index stays below n16.  The
// XOR of what a thread read goes to its sink word so the loads stay live.
__global__ __launch_bounds__(kProbeThreads) void read_stream_kernel(const u32x4* __restrict__ src,
                                                                    size_t n16, uint32_t* sink) {
  const size_t tid = size_t(blockIdx.x) * kProbeThreads + threadIdx.x;
  const size_t stride = size_t(gridDim.x) * kProbeThreads;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = tid;
  for (; i + (kProbeInFlight - 1) * stride < n16; i += kProbeInFlight * stride) {
    u32x4 v[kProbeInFlight];
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  sink[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

extern "C" fg_status fg_probe_read_stream(const void* buf, size_t bytes, void* sink,
                                          size_t sink_bytes, void* stream) {
  if (!buf || !sink || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return FG_E_INVALID;
  const int cus = fg_internal_device_cu_count();
  if (cus <= 0) return FG_E_HIP;
  if (sink_bytes < size_t(cus) * kProbeThreads * sizeof(uint32_t)) return FG_E_WORKSPACE;
  if (bytes == 0) return FG_OK;
  hipLaunchKernelGGL(read_stream_kernel, dim3(cus), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), bytes / 16,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? FG_OK : FG_E_HIP;
}
