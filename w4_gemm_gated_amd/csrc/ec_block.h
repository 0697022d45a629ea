// One workgroup of the EC projection and per-token gate (SPEAR page,
// abstract: the small error compensators are scaled per token by a gate):
//
//   [P | z] = X . [A | w_g]      (fp32 accumulation on the matrix cores)
//   g'      = sigmoid(z + b_g), set to 0 when tau > 0 and g < tau
//
// Shared by the split variant's projection launch (ec_project.hip) and the
// fused tiled launch (gemm.hip), whose first workgroups run it.
//
// A workgroup owns one 64-row tile of X and one K slice; its four waves own
// 16 rows each.  The slice is walked in sub-slabs of SS k (two LDS stages):
// the A sub-slab [SS][rank] goes to LDS (row-major, row stride rank rounded up
// to 4), while each wave keeps its X fragments of the next sub-slab in
// registers.  B fragments of the row-major A come from two transposing LDS
// reads (ds_read_b64_tr_b16): within each 16-lane group, lane 4e + c supplies
// the address of A[k + e][j + 4c .. j + 4c + 3], and lane i then holds
// A[k .. k + 3][j + i].  The gate column needs no LDS: the B fragment of a
// 32-k block holds, in lane (column c, group t), B[8 t .. 8 t + 7][c]; giving
// every column the same w_g[8 t .. 8 t + 7] (one 16-byte load, the same for
// all 16 lanes of a group) makes every output column the gate logit, of
// which column 0 is kept.
//
// Each (row tile, K slice) partial goes to the workspace with device-coherent
// stores; the last workgroup of a row tile to arrive (device-scope counter)
// adds the slices in fixed order, so the result does not depend on
// scheduling, applies the gate, writes P and g' (device-coherent stores),
// resets the counter and, in the fused launch, raises the row tile's ready
// flag to the call's tag.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace spear {
namespace {

constexpr int kEcThreads = 256;
constexpr int kEcTileRows = 64;           // four waves x 16 rows
typedef __attribute__((address_space(3))) void ec_lds_void_t;
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4_t;

struct EcKArgs {
  const half_t* X;
  const half_t* A;
  const half_t* w_g;
  int M, K, rank, rp, cols, k_slice, splits, m_tiles, ss;
  float* partials;
  uint32_t* counters;
  float* P_out;
  int p_out_stride;
  int zero_pad;          // also write zeros in P_out columns [rank, p_out_stride)
  float* g_out;
  float gate_bias, skip_tau;
  uint32_t* ready;       // fused launch: [m_tiles] flags set to the call's tag; else null
  int partials_only;     // stop after the slice's partials (a second launch adds the slices)
};

inline int ec_rank_pad(int64_t rank) { return (int)round_up(rank, 4); }

inline EcKArgs make_ec_kargs(const EcArgs& e, const EcWorkspace& L) {
  char* base = (char*)e.workspace;
  EcKArgs a;
  a.X = (const half_t*)e.X;
  a.A = (const half_t*)e.A;
  a.w_g = (const half_t*)e.w_g;
  a.M = e.M; a.K = e.K; a.rank = e.rank;
  a.rp = ec_rank_pad(e.rank);
  a.cols = (int)ec_cols(e.rank);
  a.ss = L.ss;
  a.k_slice = L.k_slice; a.splits = L.splits; a.m_tiles = L.m_tiles;
  a.partials = (float*)(base + L.partials);
  a.counters = (uint32_t*)(base + L.counters);
  a.P_out = e.P_out ? (float*)e.P_out : (float*)(base + L.p);
  a.g_out = e.g_out ? (float*)e.g_out : (float*)(base + L.g);
  a.p_out_stride = e.P_out ? e.p_out_stride : (int)p_stride(e.rank);
  a.zero_pad = e.P_out ? 0 : 1;
  a.gate_bias = e.gate_bias; a.skip_tau = e.skip_tau;
  a.ready = nullptr;
  a.partials_only = 0;
  return a;
}

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
// bytes of slack for the column tail of the last row).
__host__ __device__ __forceinline__ size_t ec_stage_bytes(int ss, int rp) {
  return (size_t)((ss * rp / 8 + kWave - 1) / kWave * kWave) * 16 + 64;
}
__host__ __device__ __forceinline__ size_t ec_lds_bytes(int ss, int rp) { return 2 * ec_stage_bytes(ss, rp); }

// 32-k blocks per sub-slab for PB column blocks (SS = 256, 128, 64 for
// rank <= 64, 128, 256).
constexpr int ec_kb_for(int pb) { return pb <= 4 ? 8 : pb == 8 ? 4 : 2; }
// Column-block count a kernel is built for: a power of two >= ceil(rank/16).
inline int ec_pb_for(int rank) {
  const int pblocks = (rank + 15) / 16;
  return pblocks <= 1 ? 1 : pblocks <= 2 ? 2 : pblocks <= 4 ? 4 : pblocks <= 8 ? 8 : 16;
}

// Last arriver of a row tile: adds the slices' partials in fixed order,
// applies the gate and publishes P and g'.  Each thread takes up to U
// 16-byte units (row, 4 columns) per round and keeps U x SB device-coherent
// loads in flight (SB slices per batch): a batch costs one memory round trip.
template <int U, int SB>
__device__ void ec_reduce_publish(const EcKArgs& a, int m_tile, int rows_here) {
  const int tid = threadIdx.x;
  const int u4 = a.cols / 4;
  const int units = rows_here * u4;
  const __amdgpu_buffer_rsrc_t pr =
      make_rsrc(a.partials, (uint32_t)((size_t)a.splits * a.m_tiles * kEcTileRows * a.cols * 4));
  const uint32_t slice_bytes = (uint32_t)((size_t)a.m_tiles * kEcTileRows * a.cols * 4);
  for (int ubase = 0; ubase < units; ubase += kEcThreads * U) {
    float4_t sum[U];
    uint32_t off0[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      sum[u] = zero_float4();
      const int unit = ubase + u * kEcThreads + tid;
      const int lr = unit / u4, c0 = (unit % u4) * 4;
      off0[u] = (unit < units && c0 <= a.rank)
                    ? (uint32_t)((((size_t)m_tile * kEcTileRows + lr) * a.cols + c0) * 4)
                    : kOutOfRange;
    }
    for (int sp0 = 0; sp0 < a.splits; sp0 += SB) {
      float4_t v[U][SB];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < SB; ++q) {
          const uint32_t sp = (uint32_t)min(sp0 + q, a.splits - 1);
          v[u][q] = buffer_load_f4_dev(pr, off0[u] == kOutOfRange ? kOutOfRange : off0[u] + sp * slice_bytes);
        }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < SB; ++q)
          if (sp0 + q < a.splits) sum[u] += v[u][q];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int unit = ubase + u * kEcThreads + tid;
      if (off0[u] == kOutOfRange) continue;
      const int lr = unit / u4, c0 = (unit % u4) * 4;
      const int row = m_tile * kEcTileRows + lr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = c0 + e;
        const float sv = sum[u][e];
        if (c < a.rank) {
          st_dev(&a.P_out[(size_t)row * a.p_out_stride + c], sv);
        } else if (c == a.rank) {
          float g = sigmoidf_(sv + a.gate_bias);
          if (a.skip_tau > 0.0f && !(g >= a.skip_tau)) g = 0.0f;
          st_dev(&a.g_out[row], g);
        }
      }
    }
  }
}

// The workgroup of (m_tile, split).  DMA: A 16-byte aligned with
// rank % 4 == 0 (rows copied verbatim); else element-wise into the padded
// layout.  GVEC: w_g 16-byte aligned (one 16-byte load per gate fragment);
// else eight 2-byte loads.  PB: P column blocks computed, a power of two >=
// ceil(rank / 16) (blocks past the last read clamped columns and are never
// stored); it fixes the sub-slab too, so every loop of the matrix-instruction
// block has a compile-time trip count and the LDS fragment reads of a k block
// are issued together.  tag: the value the ready flag is raised to (fused
// launch).  Returns after the workgroup is done; the caller may follow it
// with a block-wide barrier.
template <bool DMA, bool GVEC, int PB>
__device__ __forceinline__ void ec_block(const EcKArgs& a, unsigned char* lds, int m_tile, int split,
                                         uint32_t tag) {
  constexpr int KB = ec_kb_for(PB);
  __shared__ uint32_t last_flag;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int c16 = lane % 16, t4 = lane / 16;
  const int pblocks = (a.rank + 15) / 16;
  const int row0 = m_tile * kEcTileRows + w * 16;
  const int ss = a.ss, rp = a.rp;
  const size_t sb = ec_stage_bytes(ss, rp);
  const int k_begin = split * a.k_slice;
  const int k_end = min(a.K, k_begin + a.k_slice);
  const int nsub = (k_end - k_begin + ss - 1) / ss;

  // X fragments through a buffer resource: rows >= M and k >= K read as zeros.
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, (uint32_t)((size_t)a.M * a.K * 2));
  const uint32_t xrow = row0 + c16 < a.M ? (uint32_t)(row0 + c16) * (uint32_t)a.K * 2u : kOutOfRange;

  auto stage_A = [&](int st) { return reinterpret_cast<half_t*>(lds + st * sb); };
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(a.A, (uint32_t)((size_t)a.K * a.rank * 2));
  // A sub-slab s.  DMA layout: the rows are copied verbatim, 16 bytes per
  // unit; a thread loads its units (at most kAUnits: SS * rank / 8 <= 2048)
  // into registers a sub-slab ahead and writes them to the stage the matrix
  // work no longer reads (units past the sub-slab read as zeros).  A copy
  // straight to LDS would make the compiler hold the transposing LDS reads of
  // the current stage until the copies of the next had landed.
  constexpr int kAUnits = 8;
  auto load_A = [&](int s, u32x4_t* regs) {
    const int k0 = k_begin + s * ss;
    const int units = min(ss, k_end - k0) * a.rank / 8;   // k0 * rank * 2 is a multiple of 16
    const uint32_t first = (uint32_t)k0 * (uint32_t)a.rank / 8u;
#pragma unroll
    for (int i = 0; i < kAUnits; ++i) {
      const int u = i * kEcThreads + tid;
      regs[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                ar, u < units ? (first + (uint32_t)u) * 16u : kOutOfRange, 0, 0));
    }
  };
  auto store_A = [&](int st, const u32x4_t* regs) {
    u32x4_t* As = reinterpret_cast<u32x4_t*>(stage_A(st));
#pragma unroll
    for (int i = 0; i < kAUnits; ++i) {
      const int u = i * kEcThreads + tid;
      if (u < ss * rp / 8) As[u] = regs[i];
    }
  };
  auto fill_A = [&](int s, int st) {
    const int k0 = k_begin + s * ss;
    const int kn = min(ss, k_end - k0);
    half_t* As = stage_A(st);
    for (int idx = tid; idx < ss * rp; idx += kEcThreads) {
      const int kk = idx / rp, c = idx % rp;
      As[idx] = (kk < kn && c < a.rank) ? a.A[(size_t)(k0 + kk) * a.rank + c] : (half_t)0.0f;
    }
  };
  // X fragments and the gate fragments (w_g; zeros past the slice) of
  // sub-slab s.
  const __amdgpu_buffer_rsrc_t gr = make_rsrc(a.w_g, (uint32_t)a.K * 2u);
  auto load_g = [&](uint32_t off) -> half8_t {
    if (GVEC) return buffer_load_half8(gr, off);
    half8_t v;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v[e] = __builtin_bit_cast(half_t, __builtin_amdgcn_raw_buffer_load_b16(
                                            gr, off == kOutOfRange ? kOutOfRange : off + 2u * e, 0, 0));
    return v;
  };
  auto load_x = [&](int s, half8_t* xf, half8_t* gf) {
    const int k0 = k_begin + s * ss;
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int k = k0 + i * 32 + 8 * t4;
      const bool in = k < k_end;
      xf[i] = buffer_load_half8(xr, in ? xrow + (uint32_t)k * 2u : kOutOfRange);
      gf[i] = load_g(in ? (uint32_t)k * 2u : kOutOfRange);
    }
  };

  float4_t acc[PB + 1];                        // the gate logit in acc[PB]
#pragma unroll
  for (int j = 0; j <= PB; ++j) acc[j] = zero_float4();
  // Loads run one sub-slab ahead of the matrix work and are issued before
  // anything waits: the first two sub-slabs' A, X and gate loads go out
  // together (one memory round trip), and sub-slab s + 2's when s + 1's A
  // reaches the LDS.
  half8_t xcur[KB], xnext[KB], gcur[KB], gnext[KB];
  u32x4_t a0[kAUnits], a1[kAUnits];
  if (DMA) load_A(0, a0);
  else fill_A(0, 0);
  load_x(0, xcur, gcur);
  if (nsub > 1) {
    if (DMA) load_A(1, a1);
    load_x(1, xnext, gnext);
  }
  if (DMA) store_A(0, a0);
  for (int s = 0; s < nsub; ++s) {
    const int st = s & 1;
    __syncthreads();                            // stage st complete; stage st^1 free
    if (!DMA && s + 1 < nsub) fill_A(s + 1, st ^ 1);
    const half_t* As = stage_A(st);
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      half8_t bf[PB];
#pragma unroll
      for (int j = 0; j < PB; ++j)
        bf[j] = lds_b_fragment_tr(As + (size_t)i * 32 * rp + min(j, pblocks - 1) * 16, rp, lane);
#pragma unroll
      for (int j = 0; j < PB; ++j) acc[j] = mfma16x16x32(xcur[i], bf[j], acc[j]);
      acc[PB] = mfma16x16x32(xcur[i], gcur[i], acc[PB]);
    }
    if (s + 1 < nsub) {
      if (DMA) store_A(st ^ 1, a1);
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        xcur[i] = xnext[i];
        gcur[i] = gnext[i];
      }
      if (s + 2 < nsub) {
        if (DMA) load_A(s + 2, a1);
        load_x(s + 2, xnext, gnext);
      }
    }
  }

  // Partial of this (row tile, slice): rows 4 t4 .. 4 t4 + 3 of column c16 per
  // block; layout [split][m_tile * 64 + row][cols], the gate logit in column
  // rank.
  const size_t part_row0 = ((size_t)split * a.m_tiles + m_tile) * kEcTileRows + w * 16;
#pragma unroll
  for (int j = 0; j <= PB; ++j) {
    const bool gate = j == PB;
    if (gate || j < pblocks) {
      const int col = gate ? a.rank : j * 16 + c16;
      if (gate ? c16 == 0 : col < a.rank) {
#pragma unroll
        for (int v = 0; v < 4; ++v) st_dev(&a.partials[(part_row0 + 4 * t4 + v) * a.cols + col], acc[j][v]);
      }
    }
  }
  if (a.partials_only) return;                // ec_slices_kernel adds the slices
  drain_vm();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = add_dev_u32(&a.counters[m_tile], 1u);
    last_flag = (prev == (uint32_t)(a.splits - 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (!last_flag) return;

  // Last arriver: fixed-order sum over the slices, gate, publish (in the
  // batch shape that needs fewer memory round trips).
  const int rows_here = min(kEcTileRows, a.M - m_tile * kEcTileRows);
  const int units = rows_here * (a.cols / 4);
  const int trips_a = (units + kEcThreads * 5 - 1) / (kEcThreads * 5) * ((a.splits + 7) / 8);
  const int trips_b = (units + kEcThreads * 2 - 1) / (kEcThreads * 2) * ((a.splits + 15) / 16);
  if (trips_a <= trips_b) ec_reduce_publish<5, 8>(a, m_tile, rows_here);
  else ec_reduce_publish<2, 16>(a, m_tile, rows_here);
  if (a.zero_pad) {
    const int padc = a.p_out_stride - a.rank;
    for (int idx = tid; idx < rows_here * padc; idx += kEcThreads) {
      const int lr = idx / padc, c = a.rank + idx % padc;
      st_dev(&a.P_out[(size_t)(m_tile * kEcTileRows + lr) * a.p_out_stride + c], 0.0f);
    }
  }
  if (a.ready) {
    // Every thread's P and g' stores have completed before the flag rises.
    drain_vm();
    __syncthreads();
    if (tid == 0) st_dev_u32(&a.ready[m_tile], tag);
  }
  if (tid == 0) st_dev_u32(&a.counters[m_tile], 0u);
}

}  // namespace
}  // namespace spear
