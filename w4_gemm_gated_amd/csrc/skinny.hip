// Skinny (decode, M <= 16 rows) W4 GEMM with the gated EC fused in: one launch
// computes the EC projection and gate, the W4 product and the gated EC
// epilogue (SPEAR abstract: ECs modulated by per-token gates, the post-EC
// computation fused into the low-bit GEMM).
//
// At decode the layer is bound by reading the packed weight (K N / 2 bytes)
// from HBM, so the kernel puts the whole weight in flight at once:
//   * grid = P EC-producer workgroups, then T column tiles x S K-splits;
//   * a GEMM workgroup owns NBW 16-column panels and one K range; each of its
//     four waves issues every 16-byte weight and X load of its part before
//     its first matrix instruction (no loop-carried latency); the waves add
//     their sums through LDS;
//   * when the tiles alone do not fill the GPU, K is split over S workgroups
//     and the last to arrive (device-scope counter) adds the S partial sums in
//     fixed order, so results do not depend on timing;
//   * the P producers (lowest block indices: dispatched first, never waiting)
//     each compute [P | z] = X [A | w_g] over one K slab and publish it; every
//     tile finisher waits (bounded) until all P slabs are published, adds them
//     in fixed order (16-byte device-coherent loads), applies the gate and
//     runs the EC epilogue.
// Data crosses workgroups only through device-coherent stores and loads (see
// device_common.h), never through L2 write-backs.  Every call returns its
// counters to zero.
#include "device_common.h"
#include "internal.h"

namespace spear {

namespace {

constexpr int kThreads = 256;
typedef __attribute__((address_space(3))) void lds_void_t;

// Sync words, each hot one on its own 128-byte line (pollers and updaters of
// different words then never contend for one line).
constexpr int kSlabs = 0, kFinishers = 32, kError = 64, kTiles = 96;

struct SkinnyKArgs {
  const half_t* X;
  const u32x4_t* Wq;
  const half_t* scales;
  const half_t* A;
  const half_t* Bec;
  const half_t* w_g;
  half_t* Y;
  int M, K, N, rank, KC, NBLK;
  int T, S, CPS, P, ksp, R1p, ps;
  int ec_mode;            // 0: no EC; 1: fused producers; 2: P and g given (split variant)
  float gate_bias, skip_tau;
  uint32_t* sync;         // [kSlabs] slabs published, [kFinishers] finishers past the wait,
                          // [kError] error, [kTiles + t] split-K tile counters
  float* ec_part;         // [P][16][r1p4], r1p4 = rank + 1 rounded up to 4
  float* gemm_part;       // [T*S][NBW][64][4]
  const float* Pext;      // ec_mode 2: [M][ps]
  const float* gext;      // ec_mode 2: [M]
  uint32_t spin_limit;
};

// Direct global -> LDS copies (no VGPR result, so nothing waits on them until
// the LDS is read).  For 2-byte copies lane L writes one dword at dst + 4 L
// (the value zero-extended), for 16-byte copies 16 bytes at dst + 16 L.
__device__ __forceinline__ void copy_to_lds_u16(const half_t* src, void* dst_wave_base) {
  __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)dst_wave_base, 2, 0, 0);
}
__device__ __forceinline__ void copy_to_lds_16b(const void* src, void* dst_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst_wave_base, 16, 0, 0);
}
__device__ __forceinline__ half_t lds_half(const uint32_t* slot) {
  return __builtin_bit_cast(half_t, (uint16_t)*slot);
}

// ---------------------------------------------------------------- producer
//
// A producer owns the K slab [k0, k0 + ksp) (ksp a power of two).  LDS:
// As[ksp][rank] halves (the A slab, copied verbatim: it is contiguous in
// memory), Wh[ksp] halves (the w_g slab), then red[4][kPass][64] float4 for
// the sum over the four waves.  Copy regions are rounded up to whole 64-lane
// copies so no copy spills over.  X fragments come straight from memory
// through a buffer resource: rows >= M and k >= K read as zeros, so the
// clamped (finite) A and w_g values past K contribute nothing.

constexpr int kPass = 4;                 // column blocks per pass (16 columns each)
constexpr int kMaxKbPerWave = 8;         // ksp <= 1024

struct ProducerLds {
  half_t* As;
  half_t* Wh;
  float4_t* red;
};

__device__ __forceinline__ int prod_a_units(int ksp, int rank) { return (ksp * rank / 8 + kWave - 1) / kWave * kWave; }
__device__ __forceinline__ int prod_w_units(int ksp) { return (ksp / 8 + kWave - 1) / kWave * kWave; }

__device__ ProducerLds producer_lds(unsigned char* lds, int ksp, int rank) {
  ProducerLds L;
  size_t off = 0;
  L.As = reinterpret_cast<half_t*>(lds + off);  off += (size_t)prod_a_units(ksp, rank) * 16;
  L.Wh = reinterpret_cast<half_t*>(lds + off);  off += (size_t)prod_w_units(ksp) * 16;
  L.red = reinterpret_cast<float4_t*>(lds + off);
  return L;
}

__device__ void ec_producer(const SkinnyKArgs& a, unsigned char* lds, int p) {
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int c16 = lane % 16, t4 = lane / 16;
  const int ksp = a.ksp;
  const int k0 = p * ksp;
  const int kn = min(ksp, a.K - k0);          // multiple of 8
  const int pblocks = (a.rank + 15) / 16;
  const int r1 = a.rank + 1;
  const ProducerLds L = producer_lds(lds, ksp, a.rank);

  // A slab rows k0 .. k0+kn (kn*rank/8 16-byte units; A is 16-byte aligned
  // and k0*rank*2 is a multiple of 16) and the w_g slab (kn/8 units; w_g is
  // 16-byte aligned, k0*2 a multiple of 64).  Clamped units duplicate the
  // last real unit.
  {
    const int nvec = kn * a.rank / 8;
    const u32x4_t* asrc = reinterpret_cast<const u32x4_t*>(a.A + (size_t)k0 * a.rank);
    for (int base = wave * kWave; base < prod_a_units(ksp, a.rank); base += 4 * kWave)
      copy_to_lds_16b(asrc + min(base + lane, nvec - 1), L.As + (size_t)base * 8);
    const u32x4_t* wsrc = reinterpret_cast<const u32x4_t*>(a.w_g + k0);
    for (int base = wave * kWave; base < prod_w_units(ksp); base += 4 * kWave)
      copy_to_lds_16b(wsrc + min(base + lane, kn / 8 - 1), L.Wh + (size_t)base * 8);
  }
  // X fragments of this wave's k-blocks kb = wave, wave + 4, ...
  const int kblocks = ksp / 32;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, (uint32_t)((size_t)a.M * a.K * 2));
  half8_t xa[kMaxKbPerWave];
#pragma unroll
  for (int i = 0; i < kMaxKbPerWave; ++i) {
    const int kb = wave + 4 * i;
    const int k = k0 + kb * 32 + 8 * t4;
    const bool live = kb < kblocks && c16 < a.M && k < a.K;
    xa[i] = buffer_load_half8(xr, live ? (uint32_t)(c16 * a.K + k) * 2u : kOutOfRange);
  }
  drain_vm();
  __syncthreads();

  // Column blocks in passes of kPass: blocks 0 .. pblocks-1 hold P (columns
  // >= rank clamped, never published); in the first pass, an extra block
  // holds the gate logit in its column 0.  Each wave sums its k-blocks, then
  // the four waves add up through LDS and publish rows 4 t4 .. 4 t4 + 3 of
  // this slab's [P | z] (row stride r1p4 = rank + 1 rounded up to 4).
  const int r1p4 = (r1 + 3) & ~3;
  float* part = a.ec_part + (size_t)p * 16 * r1p4;
  for (int nb0 = 0; nb0 < pblocks; nb0 += kPass) {
    float4_t acc[kPass + 1];
#pragma unroll
    for (int i = 0; i <= kPass; ++i) acc[i] = zero_float4();
#pragma unroll
    for (int i = 0; i < kMaxKbPerWave; ++i) {
      const int kb = wave + 4 * i;
      if (kb < kblocks) {
        const int kk0 = kb * 32 + 8 * t4;
#pragma unroll
        for (int j = 0; j < kPass; ++j) {
          if (nb0 + j < pblocks) {
            const half_t* col = L.As + (size_t)kk0 * a.rank + min((nb0 + j) * 16 + c16, a.rank - 1);
            half8_t b;
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = col[e * a.rank];
            acc[j] = mfma16x16x32(xa[i], b, acc[j]);
          }
        }
        if (nb0 == 0) {
          const half8_t wv = *reinterpret_cast<const half8_t*>(&L.Wh[kk0]);
          acc[kPass] = mfma16x16x32(xa[i], c16 == 0 ? wv : zero_half8(), acc[kPass]);
        }
      }
    }
    __syncthreads();   // previous pass is done with red
#pragma unroll
    for (int j = 0; j <= kPass; ++j) L.red[(wave * (kPass + 1) + j) * kWave + lane] = acc[j];
    __syncthreads();
    for (int j = wave; j <= kPass; j += 4) {
      const bool gate = j == kPass;
      if (gate ? nb0 != 0 : nb0 + j >= pblocks) continue;
      float4_t sum = L.red[j * kWave + lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) sum += L.red[(w * (kPass + 1) + j) * kWave + lane];
      const int col = gate ? a.rank : (nb0 + j) * 16 + c16;
      if (gate ? c16 == 0 : col < a.rank) {
#pragma unroll
        for (int v = 0; v < 4; ++v) st_dev(&part[(4 * t4 + v) * r1p4 + col], sum[v]);
      }
    }
  }
  // Publish: drain the stores, then count this slab in.
  drain_vm();
  __syncthreads();
  if (tid == 0) add_dev_u32(&a.sync[kSlabs], 1u);
}

// ---------------------------------------------------------------- GEMM tile

// EXACT: every wave owns exactly CPW chunks (no validity test, so no load
// ends up under a branch).
template <int NBW, int CPW, bool EXACT>
__global__ void __launch_bounds__(kThreads) skinny_kernel(SkinnyKArgs a) {
  extern __shared__ __align__(16) unsigned char dyn_lds[];
  __shared__ float4_t red[3][kWave][NBW];
  if ((int)blockIdx.x < a.P) {
    ec_producer(a, dyn_lds, blockIdx.x);
    return;
  }
  constexpr int TN = NBW * 16;
  const int b = blockIdx.x - a.P;
  const int s = b / a.T, t = b % a.T;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int c16 = lane % 16, t4 = lane / 16;
  const int cbeg = s * a.CPS, cend = min(a.KC, cbeg + a.CPS);
  const int wbeg = cbeg + w * CPW;
  const int nb0 = t * NBW;
  const int n0 = nb0 * 16;
  const int jblocks = a.ec_mode ? a.ps / 32 : 0;
  const int r1 = a.rank + 1;
  // LDS of a GEMM workgroup: the EC factor tile Bs[jblocks*32][TN] (one dword
  // per value, fp16 in the low half), then Pc[16][rank + 1] floats (P and z).
  uint32_t* Bs = reinterpret_cast<uint32_t*>(dyn_lds);
  float* Pc = reinterpret_cast<float*>(Bs + jblocks * 32 * TN);

  // Scales of this lane's columns (columns >= N are clamped, never stored).
  half_t scr[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) scr[nb] = a.scales[min(n0 + nb * 16 + c16, a.N - 1)];

  // ---- issue every load of this wave's K range.  Chunk validity is uniform
  // over the wave; X rows >= M are clamped (their outputs are never stored).
  u32x4_t bw[CPW][NBW];
  half8_t xa[CPW][4];
  // X through a buffer resource: lanes of rows >= M read out of range, which
  // returns zeros and moves no data (their outputs are never stored).
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, (uint32_t)((size_t)a.M * a.K * 2));
  const uint32_t xrow_off = c16 < a.M ? (uint32_t)c16 * (uint32_t)a.K * 2u : kOutOfRange;
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int kc = wbeg + c;
    if (EXACT || kc < cend) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
        bw[c][nb] = a.Wq[((size_t)min(nb0 + nb, a.NBLK - 1) * a.KC + kc) * kWave + lane];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xa[c][j] = buffer_load_half8(xr, xrow_off + 2u * (uint32_t)min(kc * kKChunk + j * 32 + 8 * t4, a.K - 8));
    } else {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
        bw[c][nb] = (u32x4_t){kZeroCodeWord, kZeroCodeWord, kZeroCodeWord, kZeroCodeWord};
#pragma unroll
      for (int j = 0; j < 4; ++j) xa[c][j] = zero_half8();
    }
  }
  // Keep every stream load above this point (no load may sink into the
  // matrix-instruction block and pay a second round trip).
  __builtin_amdgcn_sched_barrier(0);

  // ---- matrix instructions
  float4_t acc[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) acc[nb] = zero_float4();
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) acc[nb] = mfma16x16x32(xa[c][j], decode_w4(bw[c][nb][j]), acc[nb]);

  // EC factor tile B[0 .. jblocks*32) x [n0, n0 + TN) -> Bs, straight to LDS.
  // Rows >= rank are clamped (they meet zero P columns).  Issued after the
  // main matrix instructions: a direct-to-LDS copy among the stream loads
  // would make every wait a full drain, and its latency hides behind the EC
  // wait anyway.
  if (jblocks > 0) {
    constexpr int kRowsPerCopy = kWave / TN;          // 1, 2 or 4
    const int rows = jblocks * 32;
    for (int r0 = w * kRowsPerCopy; r0 < rows; r0 += 4 * kRowsPerCopy) {
      const int row = min(r0 + lane / TN, a.rank - 1);
      const int col = min(n0 + lane % TN, a.N - 1);
      copy_to_lds_u16(a.Bec + (size_t)row * a.N + col, Bs + r0 * TN);
    }
  }

  // ---- four waves -> wave 0 (the drain and barrier also publish the Bs copies)
  if (w > 0) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) red[w - 1][lane][nb] = acc[nb];
  }
  drain_vm();
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) acc[nb] += red[i][lane][nb];
  }

  // ---- S splits -> the last to arrive (wave 0 exchanges, the block follows)
  if (a.S > 1) {
    __shared__ uint32_t last_s;
    if (w == 0) {
      float* slot = a.gemm_part + ((size_t)(t * a.S + s) * NBW) * kWave * 4;
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int v = 0; v < 4; ++v) st_dev(&slot[(nb * kWave + lane) * 4 + v], acc[nb][v]);
      drain_vm();
      if (lane == 0) last_s = (add_dev_u32(&a.sync[kTiles + t], 1u) == (uint32_t)(a.S - 1)) ? 1u : 0u;
    }
    __syncthreads();
    if (!last_s) return;
    if (w == 0) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) acc[nb] = zero_float4();
      for (int ss = 0; ss < a.S; ++ss) {
        const float* sl = a.gemm_part + ((size_t)(t * a.S + ss) * NBW) * kWave * 4;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[nb][v] += ld_dev(&sl[(nb * kWave + lane) * 4 + v]);
      }
      if (lane == 0) st_dev_u32(&a.sync[kTiles + t], 0u);
    }
  }

  // ---- EC projection of the 16 rows -> Pc (all four waves): wait until the
  // P slabs are published, then add them in fixed order.  The finisher count
  // is bumped right after the wait; its result (last finisher resets the
  // counters) is needed only at the very end.
  uint32_t finishers_before = 0;
  if (a.ec_mode == 1) {
    if (tid == 0) {
      uint32_t n = 0;
      while (ld_dev_u32(&a.sync[kSlabs]) < (uint32_t)a.P) {
        if (++n > a.spin_limit) { st_dev_u32(&a.sync[kError], 1u); break; }
        __builtin_amdgcn_s_sleep(8);
      }
      finishers_before = add_dev_u32(&a.sync[kFinishers], 1u);
    }
    __syncthreads();
    const int r1p4 = (r1 + 3) & ~3, u4 = r1p4 / 4;
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.ec_part, (uint32_t)((size_t)a.P * 16 * r1p4 * 4));
    for (int unit = tid; unit < 16 * u4; unit += kThreads) {
      float4_t sum = zero_float4();
      for (int p0 = 0; p0 < a.P; p0 += 8) {
        float4_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          v[q] = buffer_load_f4_dev(pr, (uint32_t)((min(p0 + q, a.P - 1) * 16 * u4 + unit) * 16));
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (p0 + q < a.P) sum += v[q];
      }
      const int row = unit / u4, c0 = (unit % u4) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c0 + e < r1) Pc[row * r1 + c0 + e] = sum[e];
    }
    __syncthreads();
  } else if (a.ec_mode == 2) {
    for (int idx = tid; idx < 16 * r1; idx += kThreads) {
      const int row = min(idx / r1, a.M - 1), col = idx % r1;
      Pc[idx] = col < a.rank ? a.Pext[(size_t)row * a.ps + col] : a.gext[row];
    }
    __syncthreads();
  }
  if (w > 0) return;

  // ---- gated EC epilogue (wave 0)
  float4_t ec[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) ec[nb] = zero_float4();
  if (a.ec_mode) {
    float gv = 0.0f;
    if (c16 < a.M) {
      if (a.ec_mode == 1) {
        gv = sigmoidf_(Pc[c16 * r1 + a.rank] + a.gate_bias);
        if (a.skip_tau > 0.0f && !(gv >= a.skip_tau)) gv = 0.0f;
      } else {
        gv = Pc[c16 * r1 + a.rank];          // the split variant's gate, already final
      }
    }
    if (__any(gv != 0.0f)) {
      for (int jb = 0; jb < jblocks; ++jb) {
        half8_t pa;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int col = jb * 32 + 8 * t4 + e;
          pa[e] = col < a.rank ? (half_t)(gv * Pc[c16 * r1 + col]) : (half_t)0.0f;
        }
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          half8_t bb;
#pragma unroll
          for (int e = 0; e < 8; ++e) bb[e] = lds_half(&Bs[(jb * 32 + 8 * t4 + e) * TN + nb * 16 + c16]);
          ec[nb] = mfma16x16x32(pa, bb, ec[nb]);
        }
      }
    }
  }

  // ---- Y = fp16(s acc + EC)
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int col = n0 + nb * 16 + c16;
    const float sc = (float)scr[nb];
    if (col < a.N) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 4 * t4 + v;
        if (row < a.M) a.Y[(size_t)row * a.N + col] = (half_t)fmaf(sc, acc[nb][v], ec[nb][v]);
      }
    }
  }

  // The last finisher past the wait resets the counters for the next call
  // (every finisher has seen all slabs by then).
  if (a.ec_mode == 1 && lane == 0 && finishers_before == (uint32_t)(a.T - 1)) {
    st_dev_u32(&a.sync[kSlabs], 0u);
    st_dev_u32(&a.sync[kFinishers], 0u);
  }
}

template <int NBW, int CPW>
hipError_t launch_nbw_cpw(const SkinnyKArgs& k, bool exact, size_t lds, void* stream) {
  if (exact)
    hipLaunchKernelGGL((skinny_kernel<NBW, CPW, true>), dim3(k.P + k.T * k.S), dim3(kThreads), lds,
                       (hipStream_t)stream, k);
  else
    hipLaunchKernelGGL((skinny_kernel<NBW, CPW, false>), dim3(k.P + k.T * k.S), dim3(kThreads), lds,
                       (hipStream_t)stream, k);
  return hipGetLastError();
}

constexpr int kMaxCpw = 8;   // chunks per wave kept in flight (NBW <= 2)

template <int NBW>
hipError_t launch_nbw(const SkinnyKArgs& k, int cpw, bool exact, size_t lds, void* stream) {
  if (cpw <= 1) return launch_nbw_cpw<NBW, 1>(k, exact, lds, stream);
  if (cpw <= 2) return launch_nbw_cpw<NBW, 2>(k, exact, lds, stream);
  if constexpr (NBW == 4) {
    return launch_nbw_cpw<NBW, 4>(k, exact, lds, stream);
  } else {
    if (cpw <= 4) return launch_nbw_cpw<NBW, 4>(k, exact, lds, stream);
    return launch_nbw_cpw<NBW, 8>(k, exact, lds, stream);
  }
}

}  // namespace

SkinnyShape skinny_shape(int64_t M, int64_t K, int64_t N, int64_t rank, bool fused, int cus,
                         size_t scratch_base) {
  SkinnyShape sh;
  const int64_t KC = k_pad(K) / kKChunk, NBLK = n_pad(N) / kNBlock;
  // Candidates (panels per workgroup, K splits).  Preferred: a grid of at
  // least one workgroup per CU; then "exact" ranges (every wave owns CPW =
  // CPS / 4 chunks); then the fewest splits (each split adds a round trip of
  // partial sums); then the widest tiles (least re-reading of X).
  int64_t best_score = -1;
  for (int nbw : {4, 2, 1}) {
    const int64_t T = ceil_div(NBLK, nbw);
    const int64_t max_cpw = nbw == 4 ? 4 : kMaxCpw;
    for (int64_t S = 1; S <= KC && S <= 64; ++S) {
      const int64_t CPS = ceil_div(KC, S);
      if (ceil_div(KC, CPS) != S) continue;             // no empty split
      const int64_t CPW = ceil_div(CPS, 4);
      if (CPW > max_cpw) continue;
      const bool exact = CPS == 4 * CPW && CPS * S == KC && (CPW == 1 || CPW == 2 || CPW == 4 || CPW == 8);
      const int64_t wgs = T * S;
      const bool fills = wgs >= cus;
      const int64_t score = (fills ? 1LL << 40 : wgs << 20) + (exact ? 1LL << 30 : 0) +
                            ((64 - S) << 8) + nbw;
      if (score > best_score) {
        best_score = score;
        sh.nbw = nbw; sh.S = (int)S; sh.T = (int)T; sh.CPS = (int)CPS; sh.CPW = (int)CPW;
      }
    }
  }
  // Round CPW up to an instantiated value.
  sh.CPW = sh.CPW <= 1 ? 1 : sh.CPW <= 2 ? 2 : sh.CPW <= 4 ? 4 : 8;
  if (fused && rank > 0) {
    // Producer slabs: a power of two near K / 4 (32 .. 1024), halved until one
    // slab's LDS (A slab, w_g slab, four-wave sums) fits 64 KiB, and doubled
    // (up to 1024) while there would be more than 64 slabs.
    int64_t ksp = 32;
    while (ksp < 1024 && ksp * 4 < K) ksp *= 2;
    auto lds_of = [&](int64_t k) {
      return round_up(k * rank / 8, kWave) * 16 + round_up(k / 8, kWave) * 16 + 4 * 5 * kWave * 16;
    };
    while (ksp > 32 && lds_of(ksp) > 64 * 1024) ksp /= 2;
    while (ksp < 1024 && ceil_div(K, ksp) > 64) ksp *= 2;
    sh.ksp = (int)ksp;
    sh.P = (int)ceil_div(K, ksp);
    sh.lds = (size_t)lds_of(ksp);
  }
  if (rank > 0) {
    // EC factor tile and the 16 projected rows of a GEMM workgroup.
    sh.lds_gemm = (size_t)(p_stride(rank) * sh.nbw * 16 * 4 + 16 * (rank + 1) * 4);
  }
  // Workspace: sync words [4 + T] in the counter header; EC partials and the
  // GEMM slots as scratch from scratch_base on.
  size_t off = scratch_base;
  auto take = [&](size_t bytes) { size_t o = off; off = (size_t)round_up((int64_t)(off + bytes), 256); return o; };
  sh.ws_sync = kGemmSyncOffset;
  if (sh.P > 0) sh.ws_ec_part = take(sizeof(float) * (size_t)sh.P * 16 * (size_t)round_up(rank + 1, 4));
  if (sh.S > 1) sh.ws_gemm_part = take(sizeof(float) * 4 * kWave * (size_t)sh.nbw * sh.T * sh.S);
  sh.ws_bytes = (sh.S > 1 || sh.P > 0) ? off : 0;
  sh.sync_ok = kTiles + sh.T <= kMaxSyncWords;
  (void)M;
  return sh;
}

hipError_t launch_skinny(const SkinnyLaunch& L, void* stream) {
  const SkinnyShape& sh = L.shape;
  SkinnyKArgs k;
  k.X = (const half_t*)L.X;
  k.Wq = (const u32x4_t*)L.Wq;
  k.scales = (const half_t*)L.scales;
  k.A = (const half_t*)L.A;
  k.Bec = (const half_t*)L.B;
  k.w_g = (const half_t*)L.w_g;
  k.Y = (half_t*)L.Y;
  k.M = L.M; k.K = L.K; k.N = L.N; k.rank = L.rank;
  k.KC = (int)(k_pad(L.K) / kKChunk);
  k.NBLK = (int)(n_pad(L.N) / kNBlock);
  k.T = sh.T; k.S = sh.S; k.CPS = sh.CPS;
  k.P = L.ec_mode == 1 ? sh.P : 0;
  k.ksp = sh.ksp;
  k.R1p = L.rank > 0 ? (int)ec_cols(L.rank) : 0;
  k.ps = L.ec_mode ? (int)p_stride(L.rank) : 0;
  k.ec_mode = L.ec_mode;
  k.gate_bias = L.gate_bias; k.skip_tau = L.skip_tau;
  char* ws = (char*)L.workspace;
  k.sync = (uint32_t*)(ws + sh.ws_sync);   // absolute offsets from the workspace base
  k.ec_part = (float*)(ws + sh.ws_ec_part);
  k.gemm_part = (float*)(ws + sh.ws_gemm_part);
  k.Pext = L.Pext;
  k.gext = L.gext;
  k.spin_limit = 1u << 20;   // ~0.5 s of polling: far beyond any healthy wait
  size_t lds = k.P > 0 ? sh.lds : 0;
  if (L.ec_mode && sh.lds_gemm > lds) lds = sh.lds_gemm;
  const bool exact = sh.CPS == 4 * sh.CPW && (int64_t)sh.CPS * sh.S == k.KC;
  if (sh.nbw == 4) return launch_nbw<4>(k, sh.CPW, exact, lds, stream);
  if (sh.nbw == 2) return launch_nbw<2>(k, sh.CPW, exact, lds, stream);
  return launch_nbw<1>(k, sh.CPW, exact, lds, stream);
}

}  // namespace spear
