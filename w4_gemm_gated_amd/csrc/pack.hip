// Weight quantization and packing (SPEAR abstract: 4-bit per-channel
// weights), and the debug decode used by the bit-exactness tests.
//
// Quantizer: s[n] = fp16(max_k |W[k,n]| / 7) with a float32 division rounded
// to nearest even, q = clamp(rint(W / s), -7, 7) with a float32 division and
// ties to even, q = 0 where s = 0, code u = q + 8.  Output layout id 2 (see
// device_common.h and spear_w4ec.h).
#include "device_common.h"
#include "internal.h"

namespace spear {

namespace {

constexpr int kPackCols = 64;     // columns per workgroup (four panels)
constexpr int kPackThreads = 256;
// k-offset held by bit field i of a packed word.
__constant__ int kNibbleK[8] = {0, 2, 4, 6, 1, 3, 5, 7};

__device__ __forceinline__ uint32_t quant_code(half_t w, float s) {
  if (s == 0.0f) return 8u;
  float r = rintf(__fdiv_rn((float)w, s));
  r = fminf(fmaxf(r, -7.0f), 7.0f);
  return (uint32_t)((int)r + 8);
}

__global__ void __launch_bounds__(kPackThreads)
pack_w4_kernel(const half_t* __restrict__ W, int K, int N, int KC, int NP,
               uint32_t* __restrict__ Wq, half_t* __restrict__ scales) {
  __shared__ float red[kPackThreads / kPackCols][kPackCols];
  __shared__ float s_col[kPackCols];
  const int c = threadIdx.x % kPackCols;
  const int rg = threadIdx.x / kPackCols;
  const int n = blockIdx.x * kPackCols + c;
  const bool real_col = n < N;

  // Column max of |W| (exact in float32).
  float m = 0.0f;
  if (real_col)
    for (int k = rg; k < K; k += kPackThreads / kPackCols)
      m = fmaxf(m, fabsf((float)W[(size_t)k * N + n]));
  red[rg][c] = m;
  __syncthreads();
  if (rg == 0) {
    float mm = red[0][c];
#pragma unroll
    for (int i = 1; i < kPackThreads / kPackCols; ++i) mm = fmaxf(mm, red[i][c]);
    const half_t s = (half_t)__fdiv_rn(mm, 7.0f);   // float32 -> fp16, nearest even
    s_col[c] = (float)s;
    if (real_col) scales[n] = s;
  }
  __syncthreads();
  if (n >= NP) return;
  const float s = real_col ? s_col[c] : 0.0f;
  const int nb = n / kNBlock, cc = n % kNBlock;
  const int K8P = KC * (kKChunk / 8);
  for (int k8 = rg; k8 < K8P; k8 += kPackThreads / kPackCols) {
    uint32_t word = 0;
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int k = k8 * 8 + kNibbleK[f];
      const uint32_t u = (real_col && k < K) ? quant_code(W[(size_t)k * N + n], s) : 8u;
      word |= u << (4 * f);
    }
    const int kc = k8 / 16, j = (k8 % 16) / 4, t = k8 % 4;
    const size_t idx = ((size_t)(nb * KC + kc) * kWave + t * kNBlock + cc) * 4 + j;
    Wq[idx] = word;
  }
}

// Group-wise scales: workgroup (column block of 64, 128-k group kc) takes the
// group's column maxima (four partial maxima of 32 rows per column), the
// scales s[kc][n], and the group's 16 k-octets of codes per column, written
// at their tiled positions (codes past K, and columns past N, are u = 8).
__global__ void __launch_bounds__(kPackThreads)
pack_w4g_kernel(const half_t* __restrict__ W, int K, int N, int KC, int NP, uint32_t* __restrict__ Wq,
                half_t* __restrict__ scales) {
  __shared__ float red[kPackThreads / kPackCols][kPackCols];
  __shared__ float s_col[kPackCols];
  const int c = threadIdx.x % kPackCols;
  const int rg = threadIdx.x / kPackCols;
  const int n = blockIdx.x * kPackCols + c;
  const int kc = blockIdx.y;
  const bool real_col = n < N;
  const int k0 = kc * kKChunk, k1 = min(K, k0 + kKChunk);
  float m = 0.0f;
  if (real_col)
    for (int k = k0 + rg; k < k1; k += kPackThreads / kPackCols) m = fmaxf(m, fabsf((float)W[(size_t)k * N + n]));
  red[rg][c] = m;
  __syncthreads();
  if (rg == 0) {
    float mm = red[0][c];
#pragma unroll
    for (int i = 1; i < kPackThreads / kPackCols; ++i) mm = fmaxf(mm, red[i][c]);
    const half_t s = (half_t)__fdiv_rn(mm, 7.0f);
    s_col[c] = (float)s;
    if (n < NP) scales[(size_t)kc * NP + n] = real_col ? s : (half_t)0.0f;
  }
  __syncthreads();
  if (n >= NP) return;
  const float s = real_col ? s_col[c] : 0.0f;
  const int nb = n / kNBlock, cc = n % kNBlock;
  for (int i = rg; i < kKChunk / 8; i += kPackThreads / kPackCols) {
    const int k8 = kc * (kKChunk / 8) + i;
    uint32_t word = 0;
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int k = k8 * 8 + kNibbleK[f];
      const uint32_t u = (real_col && k < K) ? quant_code(W[(size_t)k * N + n], s) : 8u;
      word |= u << (4 * f);
    }
    const int j = (k8 % 16) / 4, t = k8 % 4;
    Wq[((size_t)(nb * KC + kc) * kWave + t * kNBlock + cc) * 4 + j] = word;
  }
}

__global__ void __launch_bounds__(256)
unpack_w4_kernel(const uint32_t* __restrict__ Wq, int K, int N, int KC, int8_t* __restrict__ q) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)(K / 8) * N;
  if (gid >= total) return;
  const int n = (int)(gid % N);
  const int k8 = (int)(gid / N);
  const int nb = n / kNBlock, cc = n % kNBlock;
  const int kc = k8 / 16, j = (k8 % 16) / 4, t = k8 % 4;
  const uint32_t w = Wq[((size_t)(nb * KC + kc) * kWave + t * kNBlock + cc) * 4 + j];
  const half8_t h = decode_w4(w);
#pragma unroll
  for (int e = 0; e < 8; ++e) q[(size_t)(k8 * 8 + e) * N + n] = (int8_t)(int)(float)h[e];
}

}  // namespace

hipError_t launch_pack_w4(const void* W, int32_t K, int32_t N, void* Wq, void* scales, void* stream) {
  const int KC = (int)(k_pad(K) / kKChunk);
  const int NP = (int)n_pad(N);
  const int blocks = (int)ceil_div(NP, kPackCols);
  hipLaunchKernelGGL(pack_w4_kernel, dim3(blocks), dim3(kPackThreads), 0, (hipStream_t)stream,
                     (const half_t*)W, K, N, KC, NP, (uint32_t*)Wq, (half_t*)scales);
  return hipGetLastError();
}

hipError_t launch_pack_w4_grouped(const void* W, int32_t K, int32_t N, void* Wq, void* scales, void* stream) {
  const int KC = (int)(k_pad(K) / kKChunk);
  const int NP = (int)n_pad(N);
  const dim3 grid((unsigned)ceil_div(NP, kPackCols), (unsigned)KC);
  hipLaunchKernelGGL(pack_w4g_kernel, grid, dim3(kPackThreads), 0, (hipStream_t)stream, (const half_t*)W, K, N, KC,
                     NP, (uint32_t*)Wq, (half_t*)scales);
  return hipGetLastError();
}

hipError_t launch_unpack_w4(const void* Wq, int32_t K, int32_t N, void* q_out, void* stream) {
  const int KC = (int)(k_pad(K) / kKChunk);
  const int64_t total = (int64_t)(K / 8) * N;
  const int blocks = (int)ceil_div(total, 256);
  hipLaunchKernelGGL(unpack_w4_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const uint32_t*)Wq, K, N, KC, (int8_t*)q_out);
  return hipGetLastError();
}

}  // namespace spear
