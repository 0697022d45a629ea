// Small service kernels of the C ABI: reading and clearing the workspace's
// sticky error word, a plain streaming read used to measure the read rate
// the memory system delivers to a launch of a given size (the practical
// ceiling for the weight stream of a decode call), and back-to-back matrix
// instructions on register operands, the matrix cores' practical ceiling.
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

// Every wave issues `iterations` rounds of independent matrix instructions on
// register operands (no memory in the loop): 8 accumulators of
// v_mfma_f32_16x16x32_f16 (SHAPE 0) or 4 of v_mfma_f32_32x32x16_f16
// (SHAPE 1).  The accumulators are folded into one value that is stored only
// if it equals a magic value, so the work stays live.
typedef float float16_t __attribute__((ext_vector_type(16)));
template <int SHAPE>
__global__ void __launch_bounds__(1024) mfma_rate_kernel(int iterations, float* sink) {
  half8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (half_t)((float)((threadIdx.x + i) & 7) * 0.125f);
    b[i] = (half_t)((float)((threadIdx.x * 3 + i) & 7) * 0.0625f);
  }
  float x = 0.0f;
  if (SHAPE == 0) {
    float4_t acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
    for (int it = 0; it < iterations; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) x += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  } else {
    float16_t acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
    for (int it = 0; it < iterations; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) x += acc[j][e];
  }
  if (x == 1234567.0f) sink[blockIdx.x] = x;
}

}  // namespace

hipError_t launch_mfma_rate(int shape, int waves_per_simd, int iterations, int grid, void* sink, void* stream) {
  const dim3 block(4 * kWave * waves_per_simd);
  if (shape == 0)
    hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(grid), block, 0, (hipStream_t)stream, iterations, (float*)sink);
  else
    hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3(grid), block, 0, (hipStream_t)stream, iterations, (float*)sink);
  return hipGetLastError();
}

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
