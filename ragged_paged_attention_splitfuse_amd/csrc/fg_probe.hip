// Measurement aids, not steps of the method: a streaming read of a device
// buffer, used as the achievable HBM read rate beside the spec-sheet peak, and
// a matrix-core loop giving the achievable MFMA rate and the shader clock
// under matrix-core load.
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
constexpr int kProbeMfmaGroupsPerCu = 2;
constexpr int kProbeMfmaMaxIters = 2048;

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

// Matrix-core rate and shader clock under matrix-core load.  Every wavefront
// issues `iters` rounds of 32 v_mfma_f32_32x32x16_bf16 on register operands
// (all ones, four independent accumulators, so no MFMA waits on the one
// before it); thread 0 of each work-group records the work-group's elapsed
// s_memtime count (shader clock) and s_memrealtime count (100 MHz).  Every
// accumulator element ends at 16 * 8 * iters, so each thread's sink word is
// 8192 * iters exactly (iters <= 2048 keeps it exact in fp32).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(kProbeThreads) void mfma_loop_kernel(int iters, float* sink,
                                                                  long long* clocks) {
  bf16x8 a;
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = __bf16(1.0f);
  f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
  __syncthreads();
  const long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc1, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc2, 0, 0, 0);
      acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc3, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += acc0[v] + acc1[v] + acc2[v] + acc3[v];
  __syncthreads();
  const long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  sink[size_t(blockIdx.x) * kProbeThreads + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clocks[2 * size_t(blockIdx.x)] = c1 - c0;
    clocks[2 * size_t(blockIdx.x) + 1] = r1 - r0;
  }
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

extern "C" fg_status fg_probe_mfma_loop(int32_t iters, void* sink, size_t sink_bytes, void* clocks,
                                        size_t clocks_bytes, void* stream) {
  if (iters < 1 || iters > kProbeMfmaMaxIters || !sink || !clocks ||
      reinterpret_cast<uintptr_t>(sink) % 4 != 0 || reinterpret_cast<uintptr_t>(clocks) % 8 != 0)
    return FG_E_INVALID;
  const int cus = fg_internal_device_cu_count();
  if (cus <= 0) return FG_E_HIP;
  const size_t groups = size_t(cus) * kProbeMfmaGroupsPerCu;
  if (sink_bytes < groups * kProbeThreads * sizeof(float) || clocks_bytes < groups * 2 * sizeof(long long))
    return FG_E_WORKSPACE;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(unsigned(groups)), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), int(iters), static_cast<float*>(sink),
                     static_cast<long long*>(clocks));
  return hipGetLastError() == hipSuccess ? FG_OK : FG_E_HIP;
}
