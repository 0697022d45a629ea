// EC projection and per-token gate in one pass over X (SPEAR abstract:
// "lightweight Error Compensators (ECs) modulated by per-token gates"):
//
//   [P | z] = X . [A | w_g]      (fp32 accumulation on the matrix cores)
//   g'      = sigmoid(z + b_g), set to 0 when tau > 0 and g < tau
//
// The K dimension is cut into slices; each workgroup computes one
// (row tile, K slice) partial and stores it in the workspace.  The last
// workgroup of a row tile to finish (a device-scope counter; partials move
// through device-coherent stores and loads) adds the slices in fixed order,
// so the result does not depend on scheduling, applies the gate, writes P and
// g', and resets the counter.
#include "device_common.h"
#include "internal.h"

namespace spear {

EcWorkspace ec_workspace_layout(int64_t M, int64_t K, int64_t rank) {
  EcWorkspace w;
  if (rank <= 0 || M <= 0) return w;
  w.tile_rows = M <= 16 ? 16 : 64;
  w.m_tiles = (int32_t)ceil_div(M, w.tile_rows);
  w.k_slice = 256;
  w.splits = (int32_t)ceil_div(K, w.k_slice);
  const int64_t cols = ec_cols(rank);
  size_t off = kSyncHeaderBytes;
  auto take = [&](size_t bytes) { size_t o = off; off = (size_t)round_up((int64_t)(off + bytes), 256); return o; };
  w.counters = 0;   // in the counter header
  w.partials = take(sizeof(float) * (size_t)w.splits * (size_t)w.m_tiles * w.tile_rows * cols);
  w.p = take(sizeof(float) * (size_t)M * (size_t)p_stride(rank));
  w.g = take(sizeof(float) * (size_t)M);
  w.bytes = off;
  return w;
}

namespace {

constexpr int kEcThreads = 256;
constexpr int kEcMaxBlocks = 17;   // ec_cols(256) / 16
constexpr int kEsPitch = 40;       // halves per LDS row (32 k + 8 padding)

struct EcKArgs {
  const half_t* X;
  const half_t* A;
  const half_t* w_g;
  int M, K, rank, cols, k_slice, splits, m_tiles, tile_rows;
  float* partials;
  uint32_t* counters;
  float* P_out;
  int p_out_stride;
  int zero_pad;  // also write zeros in P_out columns [rank, p_out_stride)
  float* g_out;
  float gate_bias, skip_tau;
};

// WM = waves along rows (4: 64-row tiles; 1: one 16-row block, the waves
// share the column blocks instead).
template <int WM>
__global__ void __launch_bounds__(kEcThreads) ec_project_kernel(EcKArgs a) {
  __shared__ half_t Es[kEcMaxBlocks * 16][kEsPitch];
  __shared__ uint32_t last_flag;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int c16 = lane % 16, t = lane / 16;
  const int m_tile = blockIdx.x, split = blockIdx.y;
  const int nblocks = a.cols / 16;
  const int row_block = m_tile * a.tile_rows + (WM == 4 ? wave * 16 : 0);
  const int my_row = row_block + c16;

  float4_t acc[kEcMaxBlocks];
#pragma unroll
  for (int i = 0; i < kEcMaxBlocks; ++i) acc[i] = zero_float4();

  const int k_begin = split * a.k_slice;
  const int k_end = min(a.K, k_begin + a.k_slice);
  for (int k0 = k_begin; k0 < k_end; k0 += 32) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < 32 * a.cols; idx += kEcThreads) {
      const int kk = idx / a.cols, c = idx % a.cols, k = k0 + kk;
      half_t v = (half_t)0.0f;
      if (k < a.K) {
        if (c < a.rank) v = a.A[(size_t)k * a.rank + c];
        else if (c == a.rank) v = a.w_g[k];
      }
      Es[c][kk] = v;
    }
    __syncthreads();
    const int kx = k0 + t * 8;
    const half8_t xa = (my_row < a.M && kx < a.K) ? load_half8(a.X + (size_t)my_row * a.K + kx) : zero_half8();
#pragma unroll
    for (int nb = 0; nb < kEcMaxBlocks; ++nb) {
      const bool mine = (WM == 4) ? (nb < nblocks) : (nb < nblocks && nb % 4 == wave);
      if (mine) {
        const half8_t b = *reinterpret_cast<const half8_t*>(&Es[nb * 16 + c16][t * 8]);
        acc[nb] = mfma16x16x32(xa, b, acc[nb]);
      }
    }
  }

  // Partial of this (row tile, slice): rows 4t..4t+3 of column c16 per block.
  const size_t part_base = ((size_t)split * a.m_tiles + m_tile) * a.tile_rows;
#pragma unroll
  for (int nb = 0; nb < kEcMaxBlocks; ++nb) {
    const bool mine = (WM == 4) ? (nb < nblocks) : (nb < nblocks && nb % 4 == wave);
    if (mine) {
      const int lr0 = (WM == 4 ? wave * 16 : 0) + 4 * t;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        st_dev(&a.partials[(part_base + lr0 + v) * a.cols + nb * 16 + c16], acc[nb][v]);
    }
  }
  drain_vm();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = add_dev_u32(&a.counters[m_tile], 1u);
    last_flag = (prev == (uint32_t)(a.splits - 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (!last_flag) return;

  // Last arriver: fixed-order sum over the slices, gate, publish.
  const int rows_here = min(a.tile_rows, a.M - m_tile * a.tile_rows);
  for (int idx = threadIdx.x; idx < rows_here * a.cols; idx += kEcThreads) {
    const int lr = idx / a.cols, c = idx % a.cols;
    if (c > a.rank) continue;
    float s = 0.0f;
    for (int sp = 0; sp < a.splits; ++sp)
      s += ld_dev(&a.partials[(((size_t)sp * a.m_tiles + m_tile) * a.tile_rows + lr) * a.cols + c]);
    const int row = m_tile * a.tile_rows + lr;
    if (c < a.rank) {
      a.P_out[(size_t)row * a.p_out_stride + c] = s;
    } else {
      float g = sigmoidf_(s + a.gate_bias);
      if (a.skip_tau > 0.0f && !(g >= a.skip_tau)) g = 0.0f;
      a.g_out[row] = g;
    }
  }
  if (a.zero_pad) {
    const int padc = a.p_out_stride - a.rank;
    for (int idx = threadIdx.x; idx < rows_here * padc; idx += kEcThreads) {
      const int lr = idx / padc, c = a.rank + idx % padc;
      a.P_out[(size_t)(m_tile * a.tile_rows + lr) * a.p_out_stride + c] = 0.0f;
    }
  }
  if (threadIdx.x == 0) st_dev_u32(&a.counters[m_tile], 0u);
}

}  // namespace

hipError_t launch_ec_project(const EcArgs& e, void* stream) {
  const EcWorkspace L = ec_workspace_layout(e.M, e.K, e.rank);
  char* base = (char*)e.workspace;
  EcKArgs a;
  a.X = (const half_t*)e.X;
  a.A = (const half_t*)e.A;
  a.w_g = (const half_t*)e.w_g;
  a.M = e.M; a.K = e.K; a.rank = e.rank;
  a.cols = (int)ec_cols(e.rank);
  a.k_slice = L.k_slice; a.splits = L.splits; a.m_tiles = L.m_tiles; a.tile_rows = L.tile_rows;
  a.partials = (float*)(base + L.partials);
  a.counters = (uint32_t*)(base + L.counters);
  a.P_out = e.P_out ? (float*)e.P_out : (float*)(base + L.p);
  a.g_out = e.g_out ? (float*)e.g_out : (float*)(base + L.g);
  a.p_out_stride = e.P_out ? e.p_out_stride : (int)p_stride(e.rank);
  a.zero_pad = e.P_out ? 0 : 1;
  a.gate_bias = e.gate_bias; a.skip_tau = e.skip_tau;
  const dim3 grid(L.m_tiles, L.splits);
  if (L.tile_rows == 16)
    hipLaunchKernelGGL(ec_project_kernel<1>, grid, dim3(kEcThreads), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(ec_project_kernel<4>, grid, dim3(kEcThreads), 0, (hipStream_t)stream, a);
  return hipGetLastError();
}

}  // namespace spear
