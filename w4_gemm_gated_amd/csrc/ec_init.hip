// Data-free initialisation of the Error Compensator: A B = the rank-r
// truncated SVD of the quantization residual E = W - dequant(Wq, s), with the
// singular values split evenly (A = U_r sqrt(S_r), B = sqrt(S_r) V_r^T).
// Sources: the SPEAR page, abstract (lightweight error compensators that
// recover the quantization error); the SERQ page ("Saliency-Aware Low-Rank
// Error Reconstruction for LLM Quantization"), Figure 1 and Table 8 (a
// low-rank reconstruction of the quantization error from its SVD).
//
// A weight-preparation step, run once per weight, in fp32 on the vector
// units:
//   1. E [K][N] fp32 from W and the packed codes and scales (per channel or
//      per 128-row group);
//   2. randomized subspace iteration with l = r + 16 columns: V0 from a
//      counter hash, then `iterations` times Y = E V, orthonormalize, Z = E^T Y,
//      orthonormalize -> V; each orthonormalization is Y <- Y W L^-1/2 from the
//      eigen-decomposition Y^T Y = W L W^T, applied twice (the second pass
//      mends what fp32 loses on a poorly conditioned block);
//   3. Rayleigh-Ritz: Y = E V, Y^T Y = W L W^T (eigenvalues descending),
//      s_j = sqrt(L_j), A = Y W_r diag(s^-1/2), B^T = V W_r diag(s^1/2);
//   4. each singular pair's sign so that the largest-magnitude entry of A's
//      column is positive (ties: the lowest row), then fp16 A [K][r], B [r][N].
// Eigen-decompositions: parallel cyclic Jacobi on one workgroup, the l x l
// matrix and its eigenvectors in LDS (l <= 128), round-robin pairing so the
// l/2 rotations of a step touch disjoint rows and columns.
#include <algorithm>
#include <cmath>

#include "device_common.h"
#include "internal.h"

namespace spear {

namespace {

constexpr int kEiThreads = 256;
constexpr int kMaxL = 128;                 // l = rank + 16 (even), at most this
constexpr int kOversample = 16;
constexpr int kTile = 64;                  // rows and inner extent of one product tile
constexpr int kJacobiSweeps = 14;

// -------------------------------------------------------------- residual
// One thread per packed word (8 k of one column): E[k][n] = W[k][n] - q s.
__global__ void __launch_bounds__(kEiThreads)
ec_residual_kernel(const half_t* __restrict__ W, const uint32_t* __restrict__ Wq, const half_t* __restrict__ scales,
                   int K, int N, int KC, int NP, int grouped, float* __restrict__ E) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t words = (int64_t)(K / 8) * N;
  if (gid >= words) return;
  const int n = (int)(gid % N), k8 = (int)(gid / N);
  const int nb = n / kNBlock, cc = n % kNBlock;
  const int kc = k8 / 16, j = (k8 % 16) / 4, t = k8 % 4;
  const uint32_t w = Wq[((size_t)(nb * KC + kc) * kWave + t * kNBlock + cc) * 4 + j];
  const half8_t q = decode_w4(w);
  const float s = (float)(grouped ? scales[(size_t)kc * NP + n] : scales[n]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const size_t idx = (size_t)(k8 * 8 + e) * N + n;
    E[idx] = (float)W[idx] - (float)q[e] * s;
  }
}

// -------------------------------------------------------------- start block
// V0[n][c] uniform in (-1, 1) from the SplitMix64 finalizer (Steele, Lea and
// Flood, "Fast splittable pseudorandom number generators") of the index.
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}
__global__ void ec_start_kernel(float* V, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const uint64_t h = splitmix64((uint64_t)i);
  V[i] = (float)((double)(h >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0);
}

// -------------------------------------------------------------- products
// C[R][l] = op(E) D[L][l] with op(E) = E [R][L] (TRANS false, E stored
// [R][L]) or E^T (TRANS true, E stored [L][R]).  A workgroup owns 64 rows of
// C; per 64-wide slice of the inner dimension the E tile (64 x 64) and the D
// slice (64 x l) go through LDS; thread t computes row t % 64 of C for the
// columns c = t / 64 + 4 i.
template <bool TRANS>
__global__ void __launch_bounds__(kEiThreads)
ec_product_kernel(const float* __restrict__ E, const float* __restrict__ D, float* __restrict__ C, int R, int L, int l) {
  __shared__ float et[kTile][kTile + 1];
  __shared__ float dt[kTile][kMaxL];
  const int tid = threadIdx.x, r_loc = tid % kTile, cg = tid / kTile;
  const int r0 = blockIdx.x * kTile;
  float acc[kMaxL / 4];
#pragma unroll
  for (int i = 0; i < kMaxL / 4; ++i) acc[i] = 0.0f;
  for (int c0 = 0; c0 < L; c0 += kTile) {
    // E tile: et[row][inner]
    for (int idx = tid; idx < kTile * kTile; idx += kEiThreads) {
      const int a = idx / kTile, b = idx % kTile;      // coalesced along b
      float v = 0.0f;
      if (!TRANS) {
        const int row = r0 + a, in = c0 + b;
        if (row < R && in < L) v = E[(size_t)row * L + in];
        et[a][b] = v;
      } else {
        const int in = c0 + a, row = r0 + b;
        if (row < R && in < L) v = E[(size_t)in * R + row];
        et[b][a] = v;
      }
    }
    for (int idx = tid; idx < kTile * l; idx += kEiThreads) {
      const int a = idx / l, b = idx % l;
      dt[a][b] = c0 + a < L ? D[(size_t)(c0 + a) * l + b] : 0.0f;
    }
    __syncthreads();
    for (int k = 0; k < kTile; ++k) {
      const float e = et[r_loc][k];
#pragma unroll
      for (int i = 0; i < kMaxL / 4; ++i) {
        const int c = cg + 4 * i;
        if (c < l) acc[i] = fmaf(e, dt[k][c], acc[i]);
      }
    }
    __syncthreads();
  }
  const int row = r0 + r_loc;
  if (row < R) {
#pragma unroll
    for (int i = 0; i < kMaxL / 4; ++i) {
      const int c = cg + 4 * i;
      if (c < l) C[(size_t)row * l + c] = acc[i];
    }
  }
}

// Out[R][c] = In[R][l] T[l][c] (T [l][c] with c <= l, in LDS); one thread per row.
__global__ void __launch_bounds__(kEiThreads)
ec_apply_kernel(const float* __restrict__ In, const float* __restrict__ T, float* __restrict__ Out, int R, int l, int c) {
  __shared__ float ts[kMaxL * kMaxL];
  for (int idx = threadIdx.x; idx < l * c; idx += kEiThreads) ts[idx] = T[idx];
  __syncthreads();
  const int row = blockIdx.x * kEiThreads + threadIdx.x;
  if (row >= R) return;
  float x[kMaxL];
#pragma unroll
  for (int i = 0; i < kMaxL; ++i) x[i] = i < l ? In[(size_t)row * l + i] : 0.0f;
  for (int j = 0; j < c; ++j) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxL; ++i)
      if (i < l) s = fmaf(x[i], ts[i * c + j], s);
    Out[(size_t)row * c + j] = s;
  }
}

// Gram matrix G = Y^T Y of Y [R][l]: workgroup b sums rows [b * rows_per, ...)
// into part[b][l][l]; the sum over workgroups is taken in fixed order.
__global__ void __launch_bounds__(kEiThreads)
ec_gram_part_kernel(const float* __restrict__ Y, int R, int l, int rows_per, float* __restrict__ part) {
  const int b = blockIdx.x;
  const int rbeg = b * rows_per, rend = min(R, rbeg + rows_per);
  for (int e = threadIdx.x; e < l * l; e += kEiThreads) {
    const int i = e / l, j = e % l;
    float s = 0.0f;
    if (i <= j)
      for (int r = rbeg; r < rend; ++r) s = fmaf(Y[(size_t)r * l + i], Y[(size_t)r * l + j], s);
    part[(size_t)b * l * l + e] = s;
  }
}
__global__ void ec_gram_sum_kernel(const float* __restrict__ part, int parts, int l, float* __restrict__ G) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= l * l) return;
  const int i = e / l, j = e % l;
  const int src = i <= j ? e : j * l + i;                 // the upper triangle, mirrored
  float s = 0.0f;
  for (int b = 0; b < parts; ++b) s += part[(size_t)b * l * l + src];
  G[e] = s;
}

// -------------------------------------------------------------- Jacobi
// Eigen-decomposition of the symmetric G [l][l] (l even, <= 128): cyclic
// Jacobi with round-robin pairs.  Output: the transform T [l][c] for one of
// three uses, with the eigenpairs ordered by decreasing eigenvalue:
//   mode 0 (orthonormalize): T = W diag(L^-1/2), c = l, eigenvalues below
//          1e-12 of the largest give zero columns;
//   mode 1 (factor A):       T = W_r diag(L_r^-1/4), c = r;
//   mode 2 (factor B^T):     T = W_r diag(L_r^+1/4), c = r.
// (L_j = s_j^2, so L^-1/4 = s^-1/2 and L^+1/4 = s^+1/2.)
__global__ void __launch_bounds__(kEiThreads)
ec_jacobi_kernel(const float* __restrict__ G, int l, int mode, int r, float* __restrict__ T, float* __restrict__ evals) {
  extern __shared__ float sm[];
  float* a = sm;                        // [l][l]
  float* v = sm + l * l;                // [l][l] eigenvectors (columns)
  float* cs = v + l * l;                // [l/2][2] rotation c, s
  int* pr = reinterpret_cast<int*>(cs + l);     // [l] current round-robin order
  int* ord = pr + l;                             // [l] eigenpair order
  __shared__ float red[kEiThreads];
  const int tid = threadIdx.x, half = l / 2;
  for (int e = tid; e < l * l; e += kEiThreads) {
    a[e] = G[e];
    v[e] = (e / l == e % l) ? 1.0f : 0.0f;
  }
  for (int i = tid; i < l; i += kEiThreads) pr[i] = i;
  __syncthreads();
  for (int sweep = 0; sweep < kJacobiSweeps; ++sweep) {
    // Off-diagonal and diagonal norms: stop when the off part is negligible.
    float off = 0.0f, dia = 0.0f;
    for (int e = tid; e < l * l; e += kEiThreads) {
      const float x = a[e] * a[e];
      if (e / l == e % l) dia += x; else off += x;
    }
    red[tid] = off;
    __syncthreads();
    for (int st = kEiThreads / 2; st > 0; st /= 2) {
      if (tid < st) red[tid] += red[tid + st];
      __syncthreads();
    }
    const float off_all = red[0];
    __syncthreads();
    red[tid] = dia;
    __syncthreads();
    for (int st = kEiThreads / 2; st > 0; st /= 2) {
      if (tid < st) red[tid] += red[tid + st];
      __syncthreads();
    }
    const float dia_all = red[0];
    __syncthreads();
    if (!(off_all > 1e-14f * dia_all)) break;
    for (int step = 0; step < l - 1; ++step) {
      // pairs k: (pr[k], pr[l - 1 - k])
      for (int k = tid; k < half; k += kEiThreads) {
        const int p = pr[k], q = pr[l - 1 - k];
        const float apq = a[p * l + q], app = a[p * l + p], aqq = a[q * l + q];
        float c = 1.0f, s = 0.0f;
        if (fabsf(apq) > 1e-30f) {
          const float th = (aqq - app) / (2.0f * apq);
          const float t = (th >= 0.0f ? 1.0f : -1.0f) / (fabsf(th) + sqrtf(th * th + 1.0f));
          c = 1.0f / sqrtf(t * t + 1.0f);
          s = t * c;
        }
        cs[2 * k] = c;
        cs[2 * k + 1] = s;
      }
      __syncthreads();
      // columns p, q of a and v:  (x_p, x_q) <- (c x_p - s x_q, s x_p + c x_q)
      for (int e = tid; e < half * l; e += kEiThreads) {
        const int k = e / l, i = e % l;
        const int p = pr[k], q = pr[l - 1 - k];
        const float c = cs[2 * k], s = cs[2 * k + 1];
        const float xp = a[i * l + p], xq = a[i * l + q];
        a[i * l + p] = c * xp - s * xq;
        a[i * l + q] = s * xp + c * xq;
        const float vp = v[i * l + p], vq = v[i * l + q];
        v[i * l + p] = c * vp - s * vq;
        v[i * l + q] = s * vp + c * vq;
      }
      __syncthreads();
      // rows p, q of a
      for (int e = tid; e < half * l; e += kEiThreads) {
        const int k = e / l, j = e % l;
        const int p = pr[k], q = pr[l - 1 - k];
        const float c = cs[2 * k], s = cs[2 * k + 1];
        const float xp = a[p * l + j], xq = a[q * l + j];
        a[p * l + j] = c * xp - s * xq;
        a[q * l + j] = s * xp + c * xq;
      }
      __syncthreads();
      // next round-robin order: position 0 fixed, the others rotate by one
      if (tid == 0) {
        const int last = pr[l - 1];
        for (int i = l - 1; i > 1; --i) pr[i] = pr[i - 1];
        pr[1] = last;
      }
      __syncthreads();
    }
  }
  // order the eigenpairs by decreasing eigenvalue (ties: lower index first)
  for (int i = tid; i < l; i += kEiThreads) {
    const float li = a[i * l + i];
    int rank_i = 0;
    for (int j = 0; j < l; ++j) {
      const float lj = a[j * l + j];
      rank_i += (lj > li) || (lj == li && j < i);
    }
    ord[rank_i] = i;
  }
  __syncthreads();
  float lmax = 0.0f;
  for (int j = 0; j < l; ++j) lmax = fmaxf(lmax, a[j * l + j]);
  const int c = mode == 0 ? l : r;
  for (int e = tid; e < l * c; e += kEiThreads) {
    const int i = e / c, jj = e % c;
    const int src = ord[jj];
    const float lam = a[src * l + src];
    float f = 0.0f;
    if (lam > 1e-12f * lmax && lam > 0.0f) {
      f = mode == 0 ? rsqrtf(lam) : mode == 1 ? rsqrtf(sqrtf(lam)) : sqrtf(sqrtf(lam));
    }
    T[e] = v[i * l + src] * f;
  }
  if (evals)
    for (int jj = tid; jj < l; jj += kEiThreads) evals[jj] = a[ord[jj] * l + ord[jj]];
}

// -------------------------------------------------------------- output
// Sign of each of the r columns of A32 [K][r]: the largest-magnitude entry
// (ties: lowest row) made positive.  One workgroup per column.
__global__ void __launch_bounds__(kEiThreads) ec_sign_kernel(const float* __restrict__ A32, int K, int r, float* sign) {
  __shared__ float bv[kEiThreads];
  __shared__ int bi[kEiThreads];
  const int j = blockIdx.x, tid = threadIdx.x;
  float best = -1.0f;
  int besti = 0x7fffffff;
  for (int k = tid; k < K; k += kEiThreads) {
    const float x = fabsf(A32[(size_t)k * r + j]);
    if (x > best) { best = x; besti = k; }
  }
  bv[tid] = best;
  bi[tid] = besti;
  __syncthreads();
  for (int st = kEiThreads / 2; st > 0; st /= 2) {
    if (tid < st && (bv[tid + st] > bv[tid] || (bv[tid + st] == bv[tid] && bi[tid + st] < bi[tid]))) {
      bv[tid] = bv[tid + st];
      bi[tid] = bi[tid + st];
    }
    __syncthreads();
  }
  if (tid == 0) sign[j] = A32[(size_t)bi[0] * r + j] < 0.0f ? -1.0f : 1.0f;
}

__global__ void ec_write_kernel(const float* __restrict__ A32, const float* __restrict__ Bt32,
                                const float* __restrict__ sign, int K, int N, int r, half_t* __restrict__ A,
                                half_t* __restrict__ B) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t na = (int64_t)K * r, nb = (int64_t)r * N;
  if (i < na) A[i] = (half_t)(A32[i] * sign[i % r]);
  if (i < nb) {
    const int j = (int)(i / N), n = (int)(i % N);
    B[i] = (half_t)(Bt32[(size_t)n * r + j] * sign[j]);
  }
}

}  // namespace

EcInitLayout ec_init_layout(int64_t K, int64_t N, int64_t rank) {
  EcInitLayout L;
  L.l = (int)round_up(std::min<int64_t>(rank + kOversample, std::min(K, N)), 2);
  if (L.l > std::min(K, N)) L.l -= 2;
  L.gram_parts = (int)std::min<int64_t>(64, ceil_div(std::max(K, N), 256));
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = (size_t)round_up((int64_t)(off + bytes), 256); return o; };
  L.E = take((size_t)K * N * 4);
  L.Y = take((size_t)K * L.l * 4);
  L.Y2 = take((size_t)std::max(K, N) * L.l * 4);
  L.V = take((size_t)N * L.l * 4);
  L.part = take((size_t)L.gram_parts * L.l * L.l * 4);
  L.G = take((size_t)L.l * L.l * 4);
  L.T = take((size_t)L.l * L.l * 4);
  L.evals = take((size_t)L.l * 4);
  L.A32 = take((size_t)K * rank * 4);
  L.Bt32 = take((size_t)N * rank * 4);
  L.sign = take((size_t)rank * 4);
  L.bytes = off;
  L.fits = L.l <= kMaxL && L.l >= rank && rank >= 1;
  return L;
}

hipError_t launch_ec_init(const EcInitArgs& a, void* stream) {
  const hipStream_t s = (hipStream_t)stream;
  const EcInitLayout& L = a.layout;
  char* ws = (char*)a.workspace;
  float* E = (float*)(ws + L.E);
  float* Y = (float*)(ws + L.Y);
  float* Y2 = (float*)(ws + L.Y2);
  float* V = (float*)(ws + L.V);
  float* part = (float*)(ws + L.part);
  float* G = (float*)(ws + L.G);
  float* T = (float*)(ws + L.T);
  float* A32 = (float*)(ws + L.A32);
  float* Bt32 = (float*)(ws + L.Bt32);
  float* sign = (float*)(ws + L.sign);
  const int K = a.K, N = a.N, l = L.l, r = a.rank;
  const int KC = (int)(k_pad(K) / kKChunk), NP = (int)n_pad(N);
  const size_t jacobi_lds = (size_t)2 * l * l * 4 + (size_t)l * 4 + (size_t)2 * l * 4;
  hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void*>(&ec_jacobi_kernel), (int)jacobi_lds);
  if (e != hipSuccess) return e;
  const int64_t words = (int64_t)(K / 8) * N;
  hipLaunchKernelGGL(ec_residual_kernel, dim3((unsigned)ceil_div(words, kEiThreads)), dim3(kEiThreads), 0, s,
                     (const half_t*)a.W, (const uint32_t*)a.Wq, (const half_t*)a.scales, K, N, KC, NP, a.grouped, E);
  hipLaunchKernelGGL(ec_start_kernel, dim3((unsigned)ceil_div((int64_t)N * l, 256)), dim3(256), 0, s, V,
                     (int64_t)N * l);
  // X <- X W L^-1/2 twice, for a block of R rows held in X: the first pass
  // writes the scratch block Y2, the second writes X again.
  auto orthonormalize = [&](float* X, int R) {
    const int rows_per = (int)ceil_div(R, L.gram_parts);
    const int parts = (int)ceil_div(R, rows_per);
    for (int pass = 0; pass < 2; ++pass) {
      const float* src = pass == 0 ? X : Y2;
      float* dst = pass == 0 ? Y2 : X;
      hipLaunchKernelGGL(ec_gram_part_kernel, dim3(parts), dim3(kEiThreads), 0, s, src, R, l, rows_per, part);
      hipLaunchKernelGGL(ec_gram_sum_kernel, dim3((unsigned)ceil_div(l * l, 256)), dim3(256), 0, s, part, parts, l, G);
      hipLaunchKernelGGL(ec_jacobi_kernel, dim3(1), dim3(kEiThreads), jacobi_lds, s, G, l, 0, l, T, (float*)nullptr);
      hipLaunchKernelGGL(ec_apply_kernel, dim3((unsigned)ceil_div(R, kEiThreads)), dim3(kEiThreads), 0, s, src, T, dst,
                         R, l, l);
    }
  };
  orthonormalize(V, N);
  for (int it = 0; it < a.iterations; ++it) {
    hipLaunchKernelGGL(ec_product_kernel<false>, dim3((unsigned)ceil_div(K, kTile)), dim3(kEiThreads), 0, s, E, V, Y, K,
                       N, l);
    orthonormalize(Y, K);
    hipLaunchKernelGGL(ec_product_kernel<true>, dim3((unsigned)ceil_div(N, kTile)), dim3(kEiThreads), 0, s, E, Y, V, N,
                       K, l);
    orthonormalize(V, N);
  }
  // Rayleigh-Ritz on the final basis V.
  hipLaunchKernelGGL(ec_product_kernel<false>, dim3((unsigned)ceil_div(K, kTile)), dim3(kEiThreads), 0, s, E, V, Y, K, N,
                     l);
  {
    const int rows_per = (int)ceil_div(K, L.gram_parts);
    const int parts = (int)ceil_div(K, rows_per);
    hipLaunchKernelGGL(ec_gram_part_kernel, dim3(parts), dim3(kEiThreads), 0, s, Y, K, l, rows_per, part);
    hipLaunchKernelGGL(ec_gram_sum_kernel, dim3((unsigned)ceil_div(l * l, 256)), dim3(256), 0, s, part, parts, l, G);
  }
  hipLaunchKernelGGL(ec_jacobi_kernel, dim3(1), dim3(kEiThreads), jacobi_lds, s, G, l, 1, r, T,
                     (float*)(ws + L.evals));
  hipLaunchKernelGGL(ec_apply_kernel, dim3((unsigned)ceil_div(K, kEiThreads)), dim3(kEiThreads), 0, s, Y, T, A32, K, l, r);
  hipLaunchKernelGGL(ec_jacobi_kernel, dim3(1), dim3(kEiThreads), jacobi_lds, s, G, l, 2, r, T, (float*)nullptr);
  hipLaunchKernelGGL(ec_apply_kernel, dim3((unsigned)ceil_div(N, kEiThreads)), dim3(kEiThreads), 0, s, V, T, Bt32, N, l, r);
  hipLaunchKernelGGL(ec_sign_kernel, dim3(r), dim3(kEiThreads), 0, s, A32, K, r, sign);
  const int64_t outs = std::max((int64_t)K * r, (int64_t)r * N);
  hipLaunchKernelGGL(ec_write_kernel, dim3((unsigned)ceil_div(outs, 256)), dim3(256), 0, s, A32, Bt32, sign, K, N, r,
                     (half_t*)a.A, (half_t*)a.B);
  return hipGetLastError();
}

}  // namespace spear
