// W4 GEMM with the gated EC term in its epilogue (SPEAR abstract: "fuse the
// post-EC computation into low-bit GEMMs"):
//
//   acc[m, n] = sum_k X[m, k] q[k, n]                  (fp16 x fp16 -> fp32 MFMA)
//   Y[m, n]   = fp16( s[n] acc[m, n] + sum_j (g'[m] P[m, j]) B[j, n] )
//
// The per-channel scale factors out of the k-sum, so q stays an exact small
// integer in fp16 and s is applied once in the epilogue.  The EC term runs on
// the matrix cores too: g' P is rounded to fp16 (relative error 2^-11 on a
// term two orders of magnitude below Y) and multiplied by B with fp32
// accumulation.  A wave whose rows all have g' = 0 skips the EC term (the
// device-side gate-value decision of the dispatcher).
#include "device_common.h"
#include "internal.h"

namespace spear {

namespace {

constexpr int kGemmThreads = 256;

struct GemmKArgs {
  const half_t* X;
  const u32x4_t* Wq;
  const half_t* scales;
  const half_t* B;
  const float* P;
  const float* g;
  half_t* Y;
  int M, K, N, rank, KC, NBLK, ps, ec;
};

// Wave tile MB x NB blocks of 16 x 16; workgroup WM x WN wave tiles; WK waves
// share the K range of one tile and add their sums through LDS.
template <int MB, int NB, int WM, int WN, int WK>
__global__ void __launch_bounds__(kGemmThreads) w4_gemm_kernel(GemmKArgs a) {
  static_assert(WM * WN * WK * kWave == kGemmThreads, "four waves");
  constexpr int TM = 16 * MB * WM;
  constexpr int NBW = NB * WN;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int c16 = lane % 16, t = lane / 16;
  const int wm = wave % WM, wn = (wave / WM) % WN, wk = wave / (WM * WN);
  const int row0 = blockIdx.y * TM + wm * MB * 16;
  const int nb0 = blockIdx.x * NBW + wn * NB;

  float4_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = zero_float4();

  for (int kc = wk; kc < a.KC; kc += WK) {
    u32x4_t bw[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int gnb = nb0 + nb;
      if (gnb < a.NBLK) {
        bw[nb] = a.Wq[((size_t)gnb * a.KC + kc) * kWave + lane];
      } else {
        bw[nb] = (u32x4_t){kZeroCodeWord, kZeroCodeWord, kZeroCodeWord, kZeroCodeWord};
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kx = kc * kKChunk + j * 32 + t * 8;
      half8_t xa[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int row = row0 + mb * 16 + c16;
        xa[mb] = (row < a.M && kx < a.K) ? load_half8(a.X + (size_t)row * a.K + kx) : zero_half8();
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const half8_t b = decode_w4(bw[nb][j]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb][nb] = mfma16x16x32(xa[mb], b, acc[mb][nb]);
      }
    }
  }

  if constexpr (WK > 1) {
    __shared__ float4_t red[WK - 1][WM * WN][kWave][MB * NB];
    const int slot = wm + WM * wn;
    if (wk > 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) red[wk - 1][slot][lane][mb * NB + nb] = acc[mb][nb];
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int w = 0; w < WK - 1; ++w)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] += red[w][slot][lane][mb * NB + nb];
  }

  // ---------------------------------------------------------------- epilogue
  const int jblocks = a.ps / 32;
  bool any_gate = false;
  if (a.ec) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int row = row0 + mb * 16 + c16;
      any_gate |= (row < a.M) && (a.g[row] != 0.0f);
    }
  }
  any_gate = __any(any_gate);

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int col = (nb0 + nb) * 16 + c16;
    const float s = col < a.N ? (float)a.scales[col] : 0.0f;
    float4_t ecacc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) ecacc[mb] = zero_float4();
    if (any_gate) {
      for (int jb = 0; jb < jblocks; ++jb) {
        half8_t bb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = jb * 32 + t * 8 + e;
          bb[e] = (j < a.rank && col < a.N) ? a.B[(size_t)j * a.N + col] : (half_t)0.0f;
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int row = row0 + mb * 16 + c16;
          half8_t pa = zero_half8();
          if (row < a.M) {
            const float gv = a.g[row];
            const float* pr = a.P + (size_t)row * a.ps + jb * 32 + t * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) pa[e] = (half_t)(gv * pr[e]);
          }
          ecacc[mb] = mfma16x16x32(pa, bb, ecacc[mb]);
        }
      }
    }
    if (col < a.N) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = row0 + mb * 16 + 4 * t + v;
          if (row < a.M) a.Y[(size_t)row * a.N + col] = (half_t)fmaf(s, acc[mb][nb][v], ecacc[mb][v]);
        }
    }
  }
}

template <int MB, int NB, int WM, int WN, int WK>
hipError_t launch_cfg(const GemmKArgs& k, void* stream) {
  constexpr int TM = 16 * MB * WM, NBW = NB * WN;
  const dim3 grid((unsigned)ceil_div(k.NBLK, NBW), (unsigned)ceil_div(k.M, TM));
  hipLaunchKernelGGL((w4_gemm_kernel<MB, NB, WM, WN, WK>), grid, dim3(kGemmThreads), 0,
                     (hipStream_t)stream, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, const spear_plan_t& plan, void* stream) {
  GemmKArgs k;
  k.X = (const half_t*)a.X;
  k.Wq = (const u32x4_t*)a.Wq;
  k.scales = (const half_t*)a.scales;
  k.B = (const half_t*)a.B;
  k.P = a.P;
  k.g = a.g;
  k.Y = (half_t*)a.Y;
  k.M = a.M; k.K = a.K; k.N = a.N; k.rank = a.rank;
  k.KC = (int)(k_pad(a.K) / kKChunk);
  k.NBLK = (int)(n_pad(a.N) / kNBlock);
  k.ps = a.ec ? (int)p_stride(a.rank) : 0;
  k.ec = a.ec;
  if (plan.kernel == 0) return launch_cfg<1, 1, 1, 1, 4>(k, stream);
  return launch_cfg<4, 4, 2, 2, 1>(k, stream);
}

}  // namespace spear
