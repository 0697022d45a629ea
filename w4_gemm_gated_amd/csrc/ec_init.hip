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
//      orthonormalize -> V; each orthonormalization is Y <- Y L^-T from the
//      Cholesky factor Y^T Y = L L^T, applied twice (CholeskyQR2: the second
//      pass mends what fp32 loses on a poorly conditioned block);
//   3. Rayleigh-Ritz: Y = E V, Y^T Y = W L W^T (eigenvalues descending),
//      s_j = sqrt(L_j), A = Y W_r diag(s^-1/2), B^T = V W_r diag(s^1/2);
//   4. each singular pair's sign so that the largest-magnitude entry of A's
//      column is positive (ties: the lowest row), then fp16 A [K][r], B [r][N].
// Products (E V, E^T Y, Gram matrices, basis changes) share one tiled fp32
// kernel, K-split where its tiles alone would not fill the CUs.  The Cholesky
// factor and the eigen-decomposition of the l x l Gram matrices run on one
// workgroup each (l <= 128): Cholesky by columns with the triangle in
// registers, the eigenpairs by parallel cyclic Jacobi in LDS.
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
// C[R][n] = op(E) D with op(E) = E [R][L] (TRANS false, E stored [R][L]) or
// E^T (TRANS true, E stored [L][R]) and D [L][n], n <= 128.  Workgroup
// (x, y, z) owns rows 64x.., columns 64y.. of C and the z-th range of
// `slices` 64-wide steps of the inner dimension (a K split: each range writes
// its own partial C, summed afterwards in fixed order).  Per step the E tile
// (held k-major, et[k][row]) and the D tile (dt[k][col]) go through LDS, the
// next step's tiles are loaded into registers meanwhile, and thread t computes
// a 4 x 4 block of C: rows 4 (t / 16).., columns 4 (t % 16)...
constexpr int kEtStride = kTile + 1;   // transposing E stores (TRANS false) conflict-free

template <bool TRANS>
__global__ void __launch_bounds__(kEiThreads)
ec_mm_kernel(const float* __restrict__ E, const float* __restrict__ D, float* __restrict__ C, int R, int L, int n,
             int slices) {
  __shared__ float et[kTile * kEtStride];
  __shared__ __align__(16) float dt[kTile * kTile];
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * kTile, c0 = blockIdx.y * kTile;
  const int k_first = blockIdx.z * slices * kTile;
  const int k_end = min(L, k_first + slices * kTile);
  C += (size_t)blockIdx.z * R * n;
  // Loads: element i of the 4096 in a tile is (a = i / 64, b = i % 64); lanes
  // run along b, which is contiguous in memory for both operands.
  float er[16], dr[16];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = tid + u * kEiThreads, a = i / kTile, b = i % kTile;
      if (!TRANS) {            // E[row = r0 + a][k = k0 + b]
        const int row = r0 + a, k = k0 + b;
        er[u] = (row < R && k < k_end) ? E[(size_t)row * L + k] : 0.0f;
      } else {                 // E[k = k0 + a][row = r0 + b]
        const int k = k0 + a, row = r0 + b;
        er[u] = (row < R && k < k_end) ? E[(size_t)k * R + row] : 0.0f;
      }
      const int k = k0 + a, c = c0 + b;
      dr[u] = (k < k_end && c < n) ? D[(size_t)k * n + c] : 0.0f;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = tid + u * kEiThreads, a = i / kTile, b = i % kTile;
      if (!TRANS) et[b * kEtStride + a] = er[u];
      else et[a * kEtStride + b] = er[u];
      dt[a * kTile + b] = dr[u];
    }
  };
  const int tr = tid / 16, tc = tid % 16;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  if (k_first < k_end) load(k_first);
  for (int k0 = k_first; k0 < k_end; k0 += kTile) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + kTile < k_end) load(k0 + kTile);
#pragma unroll 8
    for (int k = 0; k < kTile; ++k) {
      float av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = et[k * kEtStride + tr * 4 + i];
      const float4 bv = *reinterpret_cast<const float4*>(&dt[k * kTile + tc * 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i][0] = fmaf(av[i], bv.x, acc[i][0]);
        acc[i][1] = fmaf(av[i], bv.y, acc[i][1]);
        acc[i][2] = fmaf(av[i], bv.z, acc[i][2]);
        acc[i][3] = fmaf(av[i], bv.w, acc[i][3]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = r0 + tr * 4 + i;
    if (row >= R) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = c0 + tc * 4 + j;
      if (c < n) C[(size_t)row * n + c] = acc[i][j];
    }
  }
}

// C[i] = sum over the `parts` partial results part[p][i], in order of p.
__global__ void ec_reduce_kernel(const float* __restrict__ part, int parts, int64_t count, float* __restrict__ C) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float s = 0.0f;
  for (int p = 0; p < parts; ++p) s += part[(size_t)p * count + i];
  C[i] = s;
}

// -------------------------------------------------------------- Cholesky QR
// T = L^-T from the Cholesky factor of the Gram matrix G = Y^T Y = L L^T
// (l x l, one workgroup), so that Y T has orthonormal columns: one
// pass of Cholesky QR (applied twice, it is CholeskyQR2: Fukaya, Nakatsukasa,
// Yanagisawa and Yamamoto, "CholeskyQR2: a simple and communication-avoiding
// algorithm for computing a tall-skinny QR factorization", 2014).  A column
// whose pivot is not above 1e-12 of the largest diagonal entry (a direction
// the block does not span: a zero or rank-deficient residual) is dropped: its
// column of L is zeroed and its column of T is zero.
// Thread t owns the lower-triangle positions e = t, t + 256, ... (row i,
// column k, e = i (i + 1) / 2 + k) of both L (from G) and X = L^-1 (from the
// identity) in registers; only the current column of L and row of X pass
// through LDS.  Column j: the owner of (j, j) publishes the pivot; the owners
// of column j of L and of row j of X scale them by its inverse square root
// and publish them; every thread then takes column j out of its trailing
// positions of L (k > j) and row j out of its positions of X below it
// (i > j, k <= j).
// kCholElems positions per thread cover l (l + 1) / 2 <= 256 kCholElems; the
// launch takes the smallest instance that covers l.
constexpr int chol_elems(int l) { return (l * (l + 1) / 2 + kEiThreads - 1) / kEiThreads; }

template <int kCholElems>
__global__ void __launch_bounds__(kEiThreads) ec_cholinv_kernel(const float* __restrict__ G, int l, float* __restrict__ T) {
  // col[0, kMaxL): column j of L; col[kMaxL, 2 kMaxL): row j of X.
  __shared__ float col[2 * kMaxL];
  __shared__ float red[kEiThreads];
  __shared__ float piv;
  static_assert(kMaxL == 128, "row and column indexes in 8 bits, i & 127 in range");
  const int tid = threadIdx.x;
  const int count = l * (l + 1) / 2;
  float a[kCholElems], x[kCholElems];
  int ik[kCholElems];    // (i << 8) | k; -1 past the triangle (row -1: never below, column 255: never j)
  float dm = 0.0f;
#pragma unroll
  for (int u = 0; u < kCholElems; ++u) {
    const int e = tid + u * kEiThreads;
    int i = (int)((sqrtf(8.0f * (float)e + 1.0f) - 1.0f) * 0.5f);
    while (i * (i + 1) / 2 > e) --i;
    while ((i + 1) * (i + 2) / 2 <= e) ++i;
    const int k = e - i * (i + 1) / 2;
    const bool valid = e < count;
    ik[u] = valid ? (i << 8) | k : -1;
    a[u] = valid ? G[i * l + k] : 0.0f;
    x[u] = (valid && i == k) ? 1.0f : 0.0f;
    if (valid && i == k) dm = fmaxf(dm, a[u]);
  }
  red[tid] = dm;
  __syncthreads();
  for (int st = kEiThreads / 2; st > 0; st /= 2) {
    if (tid < st) red[tid] = fmaxf(red[tid], red[tid + st]);
    __syncthreads();
  }
  const float tol = 1e-12f * red[0];
  for (int j = 0; j < l; ++j) {
    const int jj = (j << 8) | j;
#pragma unroll
    for (int u = 0; u < kCholElems; ++u)
      if (ik[u] == jj) piv = a[u];
    __syncthreads();
    const float d = piv;
    const bool ok = d > tol && d > 0.0f;
    const float inv = ok ? rsqrtf(d) : 0.0f;
    // Publish column j of L (its diagonal: sqrt(d), or 0 when dropped) and
    // row j of X, scaled; masked stores, no loads.
#pragma unroll
    for (int u = 0; u < kCholElems; ++u) {
      const int i = ik[u] >> 8, k = ik[u] & 255;
      if (k == j) {
        a[u] = i == j ? (ok ? d * inv : 0.0f) : a[u] * inv;
        col[i] = a[u];
      }
      if (i == j) {
        x[u] *= inv;
        col[kMaxL + k] = x[u];
      }
    }
    __syncthreads();
    // Trailing update, branch-free so that all the loads issue together:
    // L positions (i > j, k > j) take L[i][j] L[k][j] off, X positions
    // (i > j, k <= j) take L[i][j] X[j][k] off; the others get a zero factor
    // (every slot a position above row j reads was written this column).
    float li[kCholElems], ck[kCholElems];
#pragma unroll
    for (int u = 0; u < kCholElems; ++u) {
      const int i = ik[u] >> 8, k = ik[u] & 255;
      li[u] = col[i & (kMaxL - 1)];
      ck[u] = col[k > j ? k : kMaxL + k];
    }
#pragma unroll
    for (int u = 0; u < kCholElems; ++u) {
      const int i = ik[u] >> 8, k = ik[u] & 255;
      const float fa = i > j && k > j ? li[u] : 0.0f;
      const float fx = i > j && k <= j ? li[u] : 0.0f;
      a[u] = fmaf(-fa, ck[u], a[u]);
      x[u] = fmaf(-fx, ck[u], x[u]);
    }
  }
  // T = X^T: zeros where X is zero (above its diagonal), the owned values elsewhere.
  for (int e = tid; e < l * l; e += kEiThreads)
    if (e % l < e / l) T[e] = 0.0f;
#pragma unroll
  for (int u = 0; u < kCholElems; ++u)
    if (ik[u] >= 0) T[(ik[u] & 255) * l + (ik[u] >> 8)] = x[u];
}

// -------------------------------------------------------------- Jacobi
// Rayleigh-Ritz step: eigen-decomposition of the symmetric G [l][l] (l even,
// <= 128) by cyclic Jacobi, with the l/2 rotations of a step on disjoint
// row/column pairs (the round-robin "circle" schedule: index l - 1 fixed,
// the others rotating, so l - 1 steps pair every two indexes once; a step
// rotates every 2 x 2 block of a on both sides in one pass).  Outputs,
// eigenpairs ordered by decreasing eigenvalue L_j = s_j^2:
//   TA = W_r diag(L_r^-1/4) [l][r]   (A = Y TA)
//   TB = W_r diag(L_r^+1/4) [l][r]   (B^T = V TB)
// and the eigenvalues.  Eigenvalues not above 1e-12 of the largest give zero
// columns.
__global__ void __launch_bounds__(kEiThreads)
ec_jacobi_kernel(const float* __restrict__ G, int l, int r, float* __restrict__ TA, float* __restrict__ TB,
                 float* __restrict__ evals) {
  extern __shared__ float sm[];
  float* a = sm;                        // [l][l]
  float* v = sm + l * l;                // [l][l] eigenvectors (columns)
  float* cs = v + l * l;                // [l/2][2] rotation c, s
  int* ord = reinterpret_cast<int*>(cs + l);     // [l] eigenpair order
  __shared__ float red[kEiThreads];
  __shared__ int pq[kMaxL];             // the step's pairs (p, q)
  const int tid = threadIdx.x, half = l / 2, m = l - 1;
  for (int e = tid; e < l * l; e += kEiThreads) {
    a[e] = G[e];
    v[e] = (e / l == e % l) ? 1.0f : 0.0f;
  }
  __syncthreads();
  auto pair = [&](int step, int k, int& p, int& q) {
    if (k == 0) { p = step; q = m; return; }
    p = step + k;
    if (p >= m) p -= m;
    q = step - k + m;
    if (q >= m) q -= m;
  };
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
    // Converged when the off-diagonal part is below (1e-6)^2 of the diagonal
    // (fp32 leaves about 1e-7 l of rounding there).
    if (!(off_all > 1e-12f * dia_all)) break;
    for (int step = 0; step < m; ++step) {
      for (int k = tid; k < half; k += kEiThreads) {
        int p, q;
        pair(step, k, p, q);
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
        pq[2 * k] = p;
        pq[2 * k + 1] = q;
      }
      __syncthreads();
      // Every 2 x 2 block (rows p1, q1 of pair k1, columns p2, q2 of pair
      // k2) in one pass: columns (x_p, x_q) <- (c x_p - s x_q, s x_p + c x_q)
      // with pair k2's rotation, then rows the same way with pair k1's; the
      // pairs are disjoint, so the blocks are too.  Then the columns of v.
      const int tx = tid % 16, ty = tid / 16;
      for (int k1 = ty; k1 < half; k1 += 16) {
        const int p1 = pq[2 * k1], q1 = pq[2 * k1 + 1];
        const float c1 = cs[2 * k1], s1 = cs[2 * k1 + 1];
        for (int k2 = tx; k2 < half; k2 += 16) {
          const int p2 = pq[2 * k2], q2 = pq[2 * k2 + 1];
          const float c2 = cs[2 * k2], s2 = cs[2 * k2 + 1];
          const float xpp = a[p1 * l + p2], xpq = a[p1 * l + q2], xqp = a[q1 * l + p2], xqq = a[q1 * l + q2];
          const float ypp = c2 * xpp - s2 * xpq, ypq = s2 * xpp + c2 * xpq;   // row p1, columns rotated
          const float yqp = c2 * xqp - s2 * xqq, yqq = s2 * xqp + c2 * xqq;   // row q1
          a[p1 * l + p2] = c1 * ypp - s1 * yqp;
          a[q1 * l + p2] = s1 * ypp + c1 * yqp;
          a[p1 * l + q2] = c1 * ypq - s1 * yqq;
          a[q1 * l + q2] = s1 * ypq + c1 * yqq;
        }
      }
      for (int i = ty; i < l; i += 16) {
        for (int k2 = tx; k2 < half; k2 += 16) {
          const int p2 = pq[2 * k2], q2 = pq[2 * k2 + 1];
          const float c2 = cs[2 * k2], s2 = cs[2 * k2 + 1];
          const float vp = v[i * l + p2], vq = v[i * l + q2];
          v[i * l + p2] = c2 * vp - s2 * vq;
          v[i * l + q2] = s2 * vp + c2 * vq;
        }
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
  for (int e = tid; e < l * r; e += kEiThreads) {
    const int i = e / r, jj = e % r;
    const int src = ord[jj];
    const float lam = a[src * l + src];
    const bool ok = lam > 1e-12f * lmax && lam > 0.0f;
    TA[e] = ok ? v[i * l + src] * rsqrtf(sqrtf(lam)) : 0.0f;
    TB[e] = ok ? v[i * l + src] * sqrtf(sqrtf(lam)) : 0.0f;
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

namespace {

constexpr int64_t kTargetGroups = 512;   // workgroups a product aims for (two per CU)
constexpr int64_t kMaxParts = 128;       // K-split ranges of one product at most

// K split of the product C[R][n] = op(E) D over an inner extent L: `slices`
// 64-wide steps per range, `parts` ranges.
struct MmSplit {
  int slices, parts;
};
MmSplit mm_split(int64_t R, int64_t L, int64_t n) {
  R = std::max<int64_t>(R, 1);
  n = std::max<int64_t>(n, 1);
  const int64_t steps = std::max<int64_t>(1, ceil_div(L, kTile));
  const int64_t tiles = ceil_div(R, kTile) * ceil_div(n, kTile);
  const int64_t want = std::max<int64_t>(1, std::min({steps, kMaxParts, ceil_div(kTargetGroups, tiles)}));
  const int64_t slices = ceil_div(steps, want);
  return {(int)slices, (int)ceil_div(steps, slices)};
}
size_t mm_part_floats(int64_t R, int64_t L, int64_t n) {
  const MmSplit p = mm_split(R, L, n);
  return p.parts > 1 ? (size_t)p.parts * R * n : 0;
}

// The Cholesky-inverse instance whose positions per thread cover l (l is at
// most kMaxL).
void launch_cholinv(const float* G, int l, float* T, hipStream_t s) {
  const dim3 one(1), threads(kEiThreads);
  if (l <= 32)
    hipLaunchKernelGGL(ec_cholinv_kernel<chol_elems(32)>, one, threads, 0, s, G, l, T);
  else if (l <= 48)
    hipLaunchKernelGGL(ec_cholinv_kernel<chol_elems(48)>, one, threads, 0, s, G, l, T);
  else if (l <= 64)
    hipLaunchKernelGGL(ec_cholinv_kernel<chol_elems(64)>, one, threads, 0, s, G, l, T);
  else if (l <= 80)
    hipLaunchKernelGGL(ec_cholinv_kernel<chol_elems(80)>, one, threads, 0, s, G, l, T);
  else if (l <= 96)
    hipLaunchKernelGGL(ec_cholinv_kernel<chol_elems(96)>, one, threads, 0, s, G, l, T);
  else
    hipLaunchKernelGGL(ec_cholinv_kernel<chol_elems(kMaxL)>, one, threads, 0, s, G, l, T);
}

}  // namespace

EcInitLayout ec_init_layout(int64_t K, int64_t N, int64_t rank) {
  EcInitLayout L;
  L.l = (int)round_up(std::min<int64_t>(rank + kOversample, std::min(K, N)), 2);
  if (L.l > std::min(K, N)) L.l -= 2;
  L.fits = L.l <= kMaxL && L.l >= rank && rank >= 1;
  if (!L.fits) return L;
  const int64_t l = L.l;
  // partial sums of the largest split product
  const size_t part = std::max({mm_part_floats(K, N, l), mm_part_floats(N, K, l), mm_part_floats(l, K, l),
                                mm_part_floats(l, N, l), mm_part_floats(K, l, l), mm_part_floats(N, l, l),
                                mm_part_floats(K, l, rank), mm_part_floats(N, l, rank), (size_t)1});
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = (size_t)round_up((int64_t)(off + bytes), 256); return o; };
  L.E = take((size_t)K * N * 4);
  L.Y = take((size_t)K * l * 4);
  L.Y2 = take((size_t)std::max(K, N) * l * 4);
  L.V = take((size_t)N * l * 4);
  L.part = take(part * 4);
  L.G = take((size_t)l * l * 4);
  L.T = take((size_t)l * l * 4);
  L.T2 = take((size_t)l * l * 4);
  L.evals = take((size_t)l * 4);
  L.A32 = take((size_t)K * rank * 4);
  L.Bt32 = take((size_t)N * rank * 4);
  L.sign = take((size_t)rank * 4);
  L.bytes = off;
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
  float* T2 = (float*)(ws + L.T2);
  float* A32 = (float*)(ws + L.A32);
  float* Bt32 = (float*)(ws + L.Bt32);
  float* sign = (float*)(ws + L.sign);
  const int K = a.K, N = a.N, l = L.l, r = a.rank;
  const int KC = (int)(k_pad(K) / kKChunk), NP = (int)n_pad(N);
  const size_t jacobi_lds = (size_t)2 * l * l * 4 + (size_t)2 * l * 4;
  hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void*>(&ec_jacobi_kernel), (int)jacobi_lds);
  if (e != hipSuccess) return e;
  // C[R][n] = op(E) D, K-split into the partial-sum buffer where that fills the CUs.
  auto mm = [&](bool trans, const float* Ein, const float* D, float* C, int R, int Lin, int n) {
    const MmSplit p = mm_split(R, Lin, n);
    float* out = p.parts > 1 ? part : C;
    const dim3 grid((unsigned)ceil_div(R, kTile), (unsigned)ceil_div(n, kTile), (unsigned)p.parts);
    if (trans)
      hipLaunchKernelGGL(ec_mm_kernel<true>, grid, dim3(kEiThreads), 0, s, Ein, D, out, R, Lin, n, p.slices);
    else
      hipLaunchKernelGGL(ec_mm_kernel<false>, grid, dim3(kEiThreads), 0, s, Ein, D, out, R, Lin, n, p.slices);
    if (p.parts > 1) {
      const int64_t count = (int64_t)R * n;
      hipLaunchKernelGGL(ec_reduce_kernel, dim3((unsigned)ceil_div(count, 256)), dim3(256), 0, s, part, p.parts, count,
                         C);
    }
  };
  const int64_t words = (int64_t)(K / 8) * N;
  hipLaunchKernelGGL(ec_residual_kernel, dim3((unsigned)ceil_div(words, kEiThreads)), dim3(kEiThreads), 0, s,
                     (const half_t*)a.W, (const uint32_t*)a.Wq, (const half_t*)a.scales, K, N, KC, NP, a.grouped, E);
  hipLaunchKernelGGL(ec_start_kernel, dim3((unsigned)ceil_div((int64_t)N * l, 256)), dim3(256), 0, s, V,
                     (int64_t)N * l);
  // X [R][l] <- X L^-T twice (CholeskyQR2): the first pass writes the scratch
  // block Y2, the second writes X again.
  auto orthonormalize = [&](float* X, int R) {
    for (int pass = 0; pass < 2; ++pass) {
      const float* src = pass == 0 ? X : Y2;
      float* dst = pass == 0 ? Y2 : X;
      mm(true, src, src, G, l, R, l);
      launch_cholinv(G, l, T, s);
      mm(false, src, T, dst, R, l, l);
    }
  };
  orthonormalize(V, N);
  for (int it = 0; it < a.iterations; ++it) {
    mm(false, E, V, Y, K, N, l);
    orthonormalize(Y, K);
    mm(true, E, Y, V, N, K, l);
    orthonormalize(V, N);
  }
  // Rayleigh-Ritz on the final basis V.
  mm(false, E, V, Y, K, N, l);
  mm(true, Y, Y, G, l, K, l);
  hipLaunchKernelGGL(ec_jacobi_kernel, dim3(1), dim3(kEiThreads), jacobi_lds, s, G, l, r, T, T2,
                     (float*)(ws + L.evals));
  mm(false, Y, T, A32, K, l, r);
  mm(false, V, T2, Bt32, N, l, r);
  hipLaunchKernelGGL(ec_sign_kernel, dim3(r), dim3(kEiThreads), 0, s, A32, K, r, sign);
  const int64_t outs = std::max((int64_t)K * r, (int64_t)r * N);
  hipLaunchKernelGGL(ec_write_kernel, dim3((unsigned)ceil_div(outs, 256)), dim3(256), 0, s, A32, Bt32, sign, K, N, r,
                     (half_t*)a.A, (half_t*)a.B);
  return hipGetLastError();
}

}  // namespace spear
