// Small service kernels of the C ABI: reading and clearing the workspace's
// sticky error word, and a plain streaming read used to measure the read
// rate the memory system delivers to a launch of a given size (the practical
// ceiling for the weight stream of a decode call).
#include "device_common.h"
#include "internal.h"

namespace spear {

namespace {

__global__ void take_error_kernel(uint32_t* sync, uint32_t* out) {
  if (threadIdx.x == 0) {
    const uint32_t v = __hip_atomic_exchange(&sync[kSyncError], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(out, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Workgroup b reads 16-byte units [b * per, (b + 1) * per) of src, kUnroll
// loads per lane in flight, and folds them into one word so the loads stay
// live; the word is stored only in the (practically impossible) case that it
// equals a magic value.  sink holds one word per workgroup.
constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;
__global__ void __launch_bounds__(kReadThreads) stream_read_kernel(const u32x4_t* __restrict__ src, uint64_t units,
                                                                  uint32_t* sink) {
  const uint64_t per = (units + gridDim.x - 1) / gridDim.x;
  const uint64_t beg = (uint64_t)blockIdx.x * per;
  const uint64_t end = beg + per < units ? beg + per : units;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (uint64_t i = beg + threadIdx.x; i < end; i += (uint64_t)kReadThreads * kReadUnroll) {
    u32x4_t v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const uint64_t j = i + (uint64_t)u * kReadThreads;
      v[u] = j < end ? __builtin_nontemporal_load(&src[j]) : (u32x4_t){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}

}  // namespace

hipError_t launch_take_error(void* workspace, void* out, void* stream) {
  uint32_t* sync = (uint32_t*)((char*)workspace + kGemmSyncOffset);
  hipLaunchKernelGGL(take_error_kernel, dim3(1), dim3(kWave), 0, (hipStream_t)stream, sync, (uint32_t*)out);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, size_t bytes, int grid, void* sink, void* stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kReadThreads), 0, (hipStream_t)stream,
                     (const u32x4_t*)src, (uint64_t)(bytes / 16), (uint32_t*)sink);
  return hipGetLastError();
}

}  // namespace spear
