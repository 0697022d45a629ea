// EC projection and per-token gate in one pass over X (SPEAR page, abstract:
// the small error compensators are scaled per token by a gate):
//
//   [P | z] = X . [A | w_g]      (fp32 accumulation on the matrix cores)
//   g'      = sigmoid(z + b_g), set to 0 when tau > 0 and g < tau
//
// This is the first launch of the split variant.  It is bound by reading X
// once (M K 2 bytes); [A | w_g] is small and stays in L2.
//
// Grid: 64-row tiles x K slices.  A workgroup's four waves own 16 rows each;
// its K slice is walked in sub-slabs of SS k (two LDS stages): the A sub-slab
// [SS][rank] is copied to LDS (row-major, row stride rank rounded up to 4)
// and the gate column w_g to Wg[SS][4] (w_g in column 0), while each wave
// keeps its X fragments of the next sub-slab in registers.  B fragments of
// the row-major A come from two transposing LDS reads (ds_read_b64_tr_b16):
// within each 16-lane group, lane 4e + c supplies the address of
// A[k + e][j + 4c .. j + 4c + 3], and lane i then holds A[k .. k + 3][j + i].
//
// Each (row tile, K slice) partial goes to the workspace with device-coherent
// stores; the last workgroup of a row tile to arrive (device-scope counter)
// adds the slices in fixed order, so the result does not depend on
// scheduling, applies the gate, writes P and g', and resets the counter.
#include "device_common.h"
#include "internal.h"

namespace spear {

namespace {

constexpr int kEcThreads = 256;
constexpr int kTileRows = 64;             // four waves x 16 rows
constexpr int kMaxBlocks = 17;            // ec_cols(256) / 16
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4_t;

inline int rank_pad(int64_t rank) { return (int)round_up(rank, 4); }

// Sub-slab k: A sub-slab of at most 32 KiB.
inline int sub_slab(int64_t rank) {
  const int rp = rank_pad(rank);
  return rp <= 64 ? 256 : rp <= 128 ? 128 : 64;
}

}  // namespace

EcWorkspace ec_workspace_layout(int64_t M, int64_t K, int64_t rank) {
  EcWorkspace w;
  if (rank <= 0 || M <= 0) return w;
  w.tile_rows = kTileRows;
  w.m_tiles = (int32_t)ceil_div(M, kTileRows);
  // K slices: enough workgroups to spread the read of X over the GPU (about
  // 256), at most 16 slices (the last arriver of a row tile adds them all).
  const int ss = sub_slab(rank);
  const int64_t max_splits = ceil_div(K, ss);
  int64_t splits = ceil_div(256, w.m_tiles);
  if (splits > 16) splits = 16;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  w.k_slice = (int32_t)round_up(ceil_div(K, splits), ss);
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

struct EcKArgs {
  const half_t* X;
  const half_t* A;
  const half_t* w_g;
  int M, K, rank, rp, cols, k_slice, splits, m_tiles, ss;
  float* partials;
  uint32_t* counters;
  float* P_out;
  int p_out_stride;
  int zero_pad;  // also write zeros in P_out columns [rank, p_out_stride)
  float* g_out;
  float gate_bias, skip_tau;
};

__device__ __forceinline__ half8_t lds_b_fragment_tr(const half_t* row0, int stride, int lane) {
  // Lane 16 t + 4 e + c: rows 8 t + e (first read) and 8 t + 4 + e (second).
  const int t = lane / 16, e = (lane % 16) / 4, c = lane % 4;
  const half_t* p0 = row0 + (size_t)(8 * t + e) * stride + 4 * c;
  const half4_t lo = __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_t*)p0));
  const half4_t hi =
      __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_t*)(p0 + 4 * stride)));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// LDS of one stage: As[SS][rp] (rounded up to whole 64-lane copies, plus 64
// bytes of slack for the column tail of the last row), Wg[SS + 8][4].
__host__ __device__ __forceinline__ size_t stage_a_bytes(int ss, int rp) {
  return (size_t)((ss * rp / 8 + kWave - 1) / kWave * kWave) * 16 + 64;
}
__host__ __device__ __forceinline__ size_t stage_bytes(int ss, int rp) {
  return stage_a_bytes(ss, rp) + (size_t)(ss + 8) * 8;
}

// DMA: A 16-byte aligned with rank % 4 == 0 (rows copied verbatim); else
// element-wise into the padded layout.
template <bool DMA>
__global__ void __launch_bounds__(kEcThreads) ec_project_kernel(EcKArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ uint32_t last_flag;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int c16 = lane % 16, t4 = lane / 16;
  const int m_tile = blockIdx.x, split = blockIdx.y;
  const int pblocks = (a.rank + 15) / 16;
  const int row0 = m_tile * kTileRows + w * 16;
  const int ss = a.ss, rp = a.rp;
  const size_t sb = stage_bytes(ss, rp);
  const int k_begin = split * a.k_slice;
  const int k_end = min(a.K, k_begin + a.k_slice);
  const int nsub = (k_end - k_begin + ss - 1) / ss;

  // X fragments through a buffer resource: rows >= M and k >= K read as zeros.
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, (uint32_t)((size_t)a.M * a.K * 2));
  const uint32_t xrow = row0 + c16 < a.M ? (uint32_t)(row0 + c16) * (uint32_t)a.K * 2u : kOutOfRange;

  auto stage_A = [&](int st) { return reinterpret_cast<half_t*>(lds + st * sb); };
  auto stage_W = [&](int st) { return reinterpret_cast<half_t*>(lds + st * sb + stage_a_bytes(ss, rp)); };
  // Copies of sub-slab s into stage st (k >= K: zero X meets clamped A).
  auto issue_A = [&](int s, int st) {
    const int k0 = k_begin + s * ss;
    const int kn = min(ss, k_end - k0);
    half_t* As = stage_A(st);
    if (DMA) {
      const int units = kn * a.rank / 8;          // k0 * rank * 2 is a multiple of 16
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.A + (size_t)k0 * a.rank);
      for (int base = w * kWave; base < (ss * rp / 8 + kWave - 1) / kWave * kWave; base += 4 * kWave)
        __builtin_amdgcn_global_load_lds((const void*)(src + min(base + lane, units - 1)),
                                         (lds_void_t*)(As + (size_t)base * 8), 16, 0, 0);
    } else {
      for (int idx = tid; idx < ss * rp; idx += kEcThreads) {
        const int kk = idx / rp, c = idx % rp;
        As[idx] = (kk < kn && c < a.rank) ? a.A[(size_t)(k0 + kk) * a.rank + c] : (half_t)0.0f;
      }
    }
    half_t* Wg = stage_W(st);
    for (int kk = tid; kk < ss + 8; kk += kEcThreads) {
      const half_t v = kk < kn ? a.w_g[k0 + kk] : (half_t)0.0f;
      half4_t q = {v, (half_t)0.0f, (half_t)0.0f, (half_t)0.0f};
      *reinterpret_cast<half4_t*>(Wg + (size_t)kk * 4) = q;
    }
  };
  constexpr int kMaxKb = 8;                     // ss / 32 <= 8
  auto load_x = [&](int s, half8_t* xf) {
    const int k0 = k_begin + s * ss;
#pragma unroll
    for (int i = 0; i < kMaxKb; ++i) {
      const int k = k0 + i * 32 + 8 * t4;
      xf[i] = buffer_load_half8(xr, (i * 32 < ss && k < k_end) ? xrow + (uint32_t)k * 2u : kOutOfRange);
    }
  };

  float4_t acc[kMaxBlocks];
#pragma unroll
  for (int j = 0; j < kMaxBlocks; ++j) acc[j] = zero_float4();
  half8_t xcur[kMaxKb], xnext[kMaxKb];
  issue_A(0, 0);
  load_x(0, xcur);
  for (int s = 0; s < nsub; ++s) {
    const int st = s & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();                            // stage st complete; stage st^1 free
    if (s + 1 < nsub) {
      issue_A(s + 1, st ^ 1);
      load_x(s + 1, xnext);
    }
    const half_t* As = stage_A(st);
    const half_t* Wg = stage_W(st);
#pragma unroll
    for (int i = 0; i < kMaxKb; ++i) {
      if (i * 32 < ss) {
#pragma unroll
        for (int j = 0; j < kMaxBlocks; ++j) {
          if (j < pblocks) {
            const half8_t bf = lds_b_fragment_tr(As + (size_t)i * 32 * rp + j * 16, rp, lane);
            acc[j] = mfma16x16x32(xcur[i], bf, acc[j]);
          }
        }
        // The gate logit (Wg column 0) accumulates in the last slot, which
        // the P blocks never reach (rank <= 256: at most 16 of them).
        const half8_t gf = lds_b_fragment_tr(Wg + (size_t)i * 32 * 4, 4, lane);
        acc[kMaxBlocks - 1] = mfma16x16x32(xcur[i], gf, acc[kMaxBlocks - 1]);
      }
    }
    if (s + 1 < nsub) {
#pragma unroll
      for (int i = 0; i < kMaxKb; ++i) xcur[i] = xnext[i];
    }
  }

  // Partial of this (row tile, slice): rows 4 t4 .. 4 t4 + 3 of column c16 per
  // block; layout [split][m_tile * 64 + row][cols], the gate logit in column
  // rank.
  const size_t part_row0 = ((size_t)split * a.m_tiles + m_tile) * kTileRows + w * 16;
#pragma unroll
  for (int j = 0; j < kMaxBlocks; ++j) {
    const bool gate = j == kMaxBlocks - 1;
    if (gate || j < pblocks) {
      const int col = gate ? a.rank : j * 16 + c16;
      if (gate ? c16 == 0 : col < a.rank) {
#pragma unroll
        for (int v = 0; v < 4; ++v) st_dev(&a.partials[(part_row0 + 4 * t4 + v) * a.cols + col], acc[j][v]);
      }
    }
  }
  drain_vm();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = add_dev_u32(&a.counters[m_tile], 1u);
    last_flag = (prev == (uint32_t)(a.splits - 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (!last_flag) return;

  // Last arriver: fixed-order sum over the slices (16-byte device-coherent
  // loads, eight slices per batch), gate, publish.
  const int rows_here = min(kTileRows, a.M - m_tile * kTileRows);
  const int u4 = a.cols / 4;
  const __amdgpu_buffer_rsrc_t pr =
      make_rsrc(a.partials, (uint32_t)((size_t)a.splits * a.m_tiles * kTileRows * a.cols * 4));
  for (int unit = tid; unit < rows_here * u4; unit += kEcThreads) {
    const int lr = unit / u4, c0 = (unit % u4) * 4;
    if (c0 > a.rank) continue;
    float4_t sum = zero_float4();
    for (int sp0 = 0; sp0 < a.splits; sp0 += 8) {
      float4_t v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int sp = min(sp0 + q, a.splits - 1);
        const size_t off = ((((size_t)sp * a.m_tiles + m_tile) * kTileRows + lr) * a.cols + c0) * 4;
        v[q] = buffer_load_f4_dev(pr, (uint32_t)off);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (sp0 + q < a.splits) sum += v[q];
    }
    const int row = m_tile * kTileRows + lr;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = c0 + e;
      const float s = sum[e];
      if (c < a.rank) {
        a.P_out[(size_t)row * a.p_out_stride + c] = s;
      } else if (c == a.rank) {
        float g = sigmoidf_(s + a.gate_bias);
        if (a.skip_tau > 0.0f && !(g >= a.skip_tau)) g = 0.0f;
        a.g_out[row] = g;
      }
    }
  }
  if (a.zero_pad) {
    const int padc = a.p_out_stride - a.rank;
    for (int idx = tid; idx < rows_here * padc; idx += kEcThreads) {
      const int lr = idx / padc, c = a.rank + idx % padc;
      a.P_out[(size_t)(m_tile * kTileRows + lr) * a.p_out_stride + c] = 0.0f;
    }
  }
  if (tid == 0) st_dev_u32(&a.counters[m_tile], 0u);
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
  a.rp = rank_pad(e.rank);
  a.cols = (int)ec_cols(e.rank);
  a.ss = sub_slab(e.rank);
  a.k_slice = L.k_slice; a.splits = L.splits; a.m_tiles = L.m_tiles;
  a.partials = (float*)(base + L.partials);
  a.counters = (uint32_t*)(base + L.counters);
  a.P_out = e.P_out ? (float*)e.P_out : (float*)(base + L.p);
  a.g_out = e.g_out ? (float*)e.g_out : (float*)(base + L.g);
  a.p_out_stride = e.P_out ? e.p_out_stride : (int)p_stride(e.rank);
  a.zero_pad = e.P_out ? 0 : 1;
  a.gate_bias = e.gate_bias; a.skip_tau = e.skip_tau;
  const size_t lds = 2 * stage_bytes(a.ss, a.rp);
  const dim3 grid(L.m_tiles, L.splits);
  const bool dma = e.rank % 4 == 0 && ((uintptr_t)e.A % 16) == 0;
  static const hipError_t attr_dma = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&ec_project_kernel<true>), hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
  static const hipError_t attr_el = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&ec_project_kernel<false>), hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
  if (attr_dma != hipSuccess) return attr_dma;
  if (attr_el != hipSuccess) return attr_el;
  if (dma)
    hipLaunchKernelGGL(ec_project_kernel<true>, grid, dim3(kEcThreads), lds, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(ec_project_kernel<false>, grid, dim3(kEcThreads), lds, (hipStream_t)stream, a);
  return hipGetLastError();
}

}  // namespace spear
