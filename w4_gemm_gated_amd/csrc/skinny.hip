// Skinny (decode, M <= 16 rows) W4 GEMM with the gated EC fused in: one launch
// computes the EC projection and gate, the W4 product and the gated EC
// epilogue (SPEAR page, abstract: per-token gated error compensators, their
// second half computed inside the low-bit GEMM).
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
//     each compute [P | z] = X [A | w_g] over one K slab for the M rows and
//     publish it in the hand-off table, each value tagged with the call's
//     epoch;
//   * every GEMM workgroup requests the hand-off table once its matrix
//     instructions are done, by which time the producers (on CUs with no
//     weight stream, and a head start) have normally published it; the tags
//     tell whether they had, and a bounded wait covers the entries they had
//     not.  The workgroup adds the slabs in fixed order and applies the gate
//     itself.
// Data crosses workgroups only through device-coherent stores and loads (see
// device_common.h), never through L2 write-backs.  Every call returns its
// counters to zero and advances the epoch; the last of its workgroups
// (producers included) to finish does both, when every producer has read the
// call's tag and every reader is done.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace spear {

namespace {

constexpr int kThreads = 256;          // four waves
// Fused: the GEMM workgroups' delay before their weight stream (the
// producers' head start), in s_sleep 1 units (64 clocks).  Measured on
// 4096 x 4096, rank 32, two panels and two K splits per workgroup (M = 1 /
// 16, us): 0: 8.5 / 10.4; 8: 8.7 / 9.8; 16: 8.9 / 9.9; 32: 9.4 / 10.3.
// Up to four rows take none (M = 2: 8.7 vs 8.9 us; M = 4: equal; M = 8:
// 9.7 vs 9.4 with the delay).
constexpr uint32_t kStreamDelay = 8;
typedef __attribute__((address_space(3))) void lds_void_t;

// Sync words of the GEMM half of the counter header, each hot one on its own
// 128-byte line (pollers and updaters of different words never share one).
constexpr int kError = kSyncError, kTiles = kSyncTiles;

struct SkinnyKArgs {
  const half_t* X;
  const u32x4_t* Wq;
  const half_t* scales;
  const half_t* A;
  const half_t* Bec;
  const half_t* w_g;
  half_t* Y;
  int M, K, N, rank, KC, NBLK;
  int T, S, CPS, P, ksp, ps, r1p;
  int ec_mode;            // 0: no EC; 1: fused producers; 2: P and g given (split variant)
  float gate_bias, skip_tau;
  uint32_t* sync;         // [kFinishers] workgroups done, [kError] sticky error bits, [kEpoch]
                          // call epoch, [kTiles + t] split-K tile counters
  uint64_t* handoff;      // ec_mode 1: [P][M][r1p] slab sums of [P | z], each
                          // (epoch + 1) << 32 | float bits
  float* gemm_part;       // [T*S][NBW][64][4]
  const float* Pext;      // ec_mode 2: [M][ps]
  const float* gext;      // ec_mode 2: [M]
  uint32_t spin_limit;
  uint32_t wait_xor;      // the consumers wait for tag ^ wait_xor (0, or a test hook's value)
  uint32_t stream_delay;  // ec_mode 1: s_sleep units before the weight stream (producers' head start)
};

// Direct global -> LDS copy of 16 bytes per lane (lane L writes
// dst + 16 L); no VGPR result, so nothing waits on it until the LDS is read.
__device__ __forceinline__ void copy_to_lds_16b(const void* src, void* dst_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst_wave_base, 16, 0, 0);
}
__device__ __forceinline__ uint64_t ld_dev_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- producer
//
// Producer p owns the K slab [k0, k0 + ksp).  LDS: the A slab As[ksp][rank]
// copied verbatim, the w_g slab Wh[ksp], one word that carries the call's
// tag, and the X slab Xs[16][ksp] whose 16-byte units are XOR-swizzled by
// row (unit u of row r in slot u ^ (r % 16)), so the 16 rows of one fragment
// read hit 16 different bank groups.  B fragments of the row-major A slab
// come from two transposing LDS reads (ds_read_b64_tr_b16): within each
// 16-lane group, lane 4e + c supplies the address of
// A[k + e][j + 4c .. j + 4c + 3], and lane i then holds A[k .. k + 3][j + i].
// The gate logit is one more matrix product whose B fragment is a plain
// 16-byte read of Wh: every lane gets w_g at its own k, so all 16 columns of
// that product hold the logit and only column 0 is published.

constexpr int kPass = 4;                 // P column blocks per pass (the last pass adds the gate)
constexpr int kCopyWaves = 3;            // waves that copy the slabs; the fourth warms the code
constexpr int kRedSlots = kPass + 1;
constexpr int kRedBytes = 4 * kRedSlots * kWave * 16;   // the four waves' sums of one pass
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4_t;

// Copy regions are rounded up to whole 64-lane copies so no copy spills over;
// the A slab has 64 bytes of slack for the column tail of its last row.
__host__ __device__ __forceinline__ int prod_a_units(int ksp, int rank) { return (ksp * rank / 8 + kWave - 1) / kWave * kWave; }
__host__ __device__ __forceinline__ int prod_w_units(int ksp) { return (ksp / 8 + kWave - 1) / kWave * kWave; }
// The four waves' sums of a pass (red) overlay the X slab when there is one
// pass only (the slab is no longer read then), else follow it.
__host__ __device__ __forceinline__ bool producer_red_own(int rank) { return (rank + 15) / 16 > kPass; }
__host__ __device__ __forceinline__ size_t producer_xs_bytes(int ksp, int rank) {
  const size_t xs = (size_t)16 * ksp * 2;
  if (producer_red_own(rank)) return xs + kRedBytes;
  return xs > (size_t)kRedBytes ? xs : (size_t)kRedBytes;
}
__host__ __device__ __forceinline__ size_t producer_lds_bytes(int ksp, int rank) {
  return (size_t)prod_a_units(ksp, rank) * 16 + 64 + (size_t)prod_w_units(ksp) * 16 + 16 +
         producer_xs_bytes(ksp, rank);
}

struct ProducerLds {
  half_t* As;
  half_t* Wh;
  uint32_t* tag;
  half_t* Xs;
};

__device__ ProducerLds producer_lds(unsigned char* base, int ksp, int rank) {
  ProducerLds L;
  size_t off = 0;
  L.As = reinterpret_cast<half_t*>(base + off);  off += (size_t)prod_a_units(ksp, rank) * 16 + 64;
  L.Wh = reinterpret_cast<half_t*>(base + off);  off += (size_t)prod_w_units(ksp) * 16;
  L.tag = reinterpret_cast<uint32_t*>(base + off);  off += 16;
  L.Xs = reinterpret_cast<half_t*>(base + off);
  return L;
}

__device__ __forceinline__ half8_t lds_b_fragment_tr(const half_t* row0, int rank, int lane) {
  // Lane 16 t + 4 e + c: rows 8 t + e (first read) and 8 t + 4 + e (second).
  const int t = lane / 16, e = (lane % 16) / 4, c = lane % 4;
  const half_t* p0 = row0 + (size_t)(8 * t + e) * rank + 4 * c;
  const half4_t lo = __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_t*)p0));
  const half4_t hi =
      __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_t*)(p0 + 4 * rank)));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---- wave w takes the 32-k blocks kb = w, w + 4, ... of the slab (KBW
// of them) for every P column block, kPass blocks a pass, and for the gate in
// the last pass; the four waves' sums meet in LDS (red), and wave j stores
// slot j (j + 4) of the pass.  Rows 4 t4 .. 4 t4 + 3 (< M) are published,
// columns >= rank of a P block are not.  Nothing waits for the stores: the
// tags tell the readers when they landed.
//
// The wave that copies nothing starts one pass early (nb0 = -kPass): it
// reads the LDS while the copies are still landing and drops the sums.  Its
// only purpose is to fetch the pass's instructions into the instruction
// cache while the copies are in flight.  It has no loads of its own in
// flight, so its LDS reads are not held back by the copies.
template <int KBW>
__device__ void producer_passes(const SkinnyKArgs& a, const ProducerLds& L, int p, int w, uint32_t tag) {
  const int lane = threadIdx.x % kWave;
  const int c16 = lane % 16, t4 = lane / 16;
  const int ksp = a.ksp;
  const int pblocks = (a.rank + 15) / 16;
  uint64_t* slab = a.handoff + (size_t)p * a.M * a.r1p;
  const half_t* xrow = L.Xs + (size_t)c16 * ksp;
  float4_t* red = reinterpret_cast<float4_t*>(L.Xs + (producer_red_own(a.rank) ? (size_t)16 * ksp : 0));
                                               // [4 waves][kRedSlots][64 lanes]
#pragma clang loop unroll(disable)
  for (int nb0 = w < kCopyWaves ? 0 : -kPass; nb0 < pblocks; nb0 += kPass) {
    if (nb0 == 0) {
      drain_vm();
      if (w == 0 && lane == 0) *L.tag = tag;
      __syncthreads();
      tag = __builtin_amdgcn_readfirstlane(*L.tag);
    }
    const int nbp = max(nb0, 0);
    const int np = min(kPass, pblocks - nbp);  // P blocks of this pass
    const bool last = nbp + kPass >= pblocks;  // the gate rides on the last pass
    float4_t acc[kPass], accg = zero_float4();
#pragma unroll
    for (int j = 0; j < kPass; ++j) acc[j] = zero_float4();
    // The k-blocks go in groups of up to four: every LDS fragment read of a
    // group is issued before its first matrix instruction.  P blocks past np
    // are neither read nor multiplied.
    constexpr int kGroup = KBW < 4 ? KBW : 4;
#pragma unroll
    for (int i0 = 0; i0 < KBW; i0 += kGroup) {
      half8_t xf[kGroup], gf[kGroup], bf[kGroup][kPass];
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        const int kb = w + 4 * (i0 + i);
        xf[i] = *reinterpret_cast<const half8_t*>(xrow + (size_t)(((kb * 4 + t4) ^ c16) * 8));
        gf[i] = *reinterpret_cast<const half8_t*>(L.Wh + (size_t)kb * 32 + 8 * t4);
#pragma unroll
        for (int j = 0; j < kPass; ++j)
          if (j < np)
            bf[i][j] = lds_b_fragment_tr(L.As + (size_t)(nbp + j) * 16 + (size_t)kb * 32 * a.rank, a.rank, lane);
      }
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
#pragma unroll
        for (int j = 0; j < kPass; ++j)
          if (j < np) acc[j] = mfma16x16x32(xf[i], bf[i][j], acc[j]);
        accg = mfma16x16x32(xf[i], gf[i], accg);
      }
    }
    if (nb0 < 0) continue;
    __syncthreads();                           // every wave is done with the X slab / last pass
#pragma unroll
    for (int j = 0; j < kPass; ++j) red[(w * kRedSlots + j) * kWave + lane] = acc[j];
    red[(w * kRedSlots + kPass) * kWave + lane] = accg;
    __syncthreads();
    const int nslots = np + (last ? 1 : 0);
    for (int sl = w; sl < nslots; sl += 4) {
      const bool gate = sl == np;
      const int rs = gate ? kPass : sl;
      float4_t sum = red[(0 * kRedSlots + rs) * kWave + lane];
#pragma unroll
      for (int q = 1; q < 4; ++q) sum += red[(q * kRedSlots + rs) * kWave + lane];
      const int col = gate ? a.rank : (nbp + sl) * 16 + c16;
      if (gate ? c16 == 0 : col < a.rank) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (4 * t4 + v < a.M)
            st_dev_u64(&slab[(size_t)(4 * t4 + v) * a.r1p + col], ((uint64_t)tag << 32) | float_bits(sum[v]));
      }
    }
  }
}

__device__ void ec_producer(const SkinnyKArgs& a, unsigned char* lds, int p) {
  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int ksp = a.ksp;                      // 128, 256, 512 or 1024
  const int k0 = p * ksp;
  const int kn = min(ksp, a.K - k0);          // multiple of 8
  const ProducerLds L = producer_lds(lds, ksp, a.rank);
  uint32_t tag = 0;                           // needed only at the end

  // ---- slab copies, split over waves 0 .. kCopyWaves-1.  A slab rows
  // k0 .. k0+kn (kn*rank/8 16-byte units; A is 16-byte aligned and
  // k0*rank*2 is a multiple of 16) and the w_g slab; clamped units duplicate
  // the last real unit.  X rows >= M and k >= K read as zeros.
  if (w < kCopyWaves) {
    if (w == 0) tag = call_tag(a.sync);
    const int nvec = kn * a.rank / 8;
    const u32x4_t* asrc = reinterpret_cast<const u32x4_t*>(a.A + (size_t)k0 * a.rank);
    for (int base = w * kWave; base < prod_a_units(ksp, a.rank); base += kCopyWaves * kWave)
      copy_to_lds_16b(asrc + min(base + lane, nvec - 1), L.As + (size_t)base * 8);
    const u32x4_t* wsrc = reinterpret_cast<const u32x4_t*>(a.w_g + k0);
    for (int base = w * kWave; base < prod_w_units(ksp); base += kCopyWaves * kWave)
      copy_to_lds_16b(wsrc + min(base + lane, kn / 8 - 1), L.Wh + (size_t)base * 8);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, (uint32_t)((size_t)a.M * a.K * 2));
    const int units = ksp / 8;                 // per row, >= 16
    for (int idx = w * kWave; idx < 16 * units; idx += kCopyWaves * kWave) {
      const int row = (idx + lane) / units, slot = (idx + lane) % units;
      const int unit = slot ^ (row % 16);
      const int k = k0 + unit * 8;
      const uint32_t voff = (row < a.M && k < a.K) ? ((uint32_t)row * (uint32_t)a.K + (uint32_t)k) * 2u : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t*)(L.Xs + (size_t)idx * 8), 16, voff, 0, 0, 0);
    }
  }

  const int kbw = ksp / 32 / 4;                // 32-k blocks per wave: 1, 2, 4 or 8
  if (kbw == 1) producer_passes<1>(a, L, p, w, tag);
  else if (kbw == 2) producer_passes<2>(a, L, p, w, tag);
  else if (kbw == 4) producer_passes<4>(a, L, p, w, tag);
  else producer_passes<8>(a, L, p, w, tag);
  // Wave 0 read the tag; the epoch may move on only after every producer
  // has (a later read would tag this call's slabs with the next call's tag).
  if (w == 0) count_out(a.sync, (uint32_t)(a.T * a.S + a.P), tag);
}

// ---------------------------------------------------------------- local EC
//
// ec_mode 3: every GEMM workgroup computes the whole [P | z] = X [A | w_g]
// itself, with four more waves (the local waves) that run while its four
// weight waves stream W; no other workgroup is involved and nothing crosses
// workgroups.  A is read by every workgroup, so it is served from L2 after
// the first touch on each XCD; the planner takes this mode only for small A.
// Local wave lw takes a contiguous range of chunks of A (8 KiB each: 128
// rows up to rank 32, 64 rows up to rank 64).  A chunk's
// rows (16-byte units, as they are in memory) go through registers into the
// wave's own LDS buffer and come back as B fragments from transposing reads;
// the X fragments and the gate fragments (plain 16-byte reads of w_g, as in
// the producer) come straight from memory.  The next chunk's loads are in
// flight while a chunk is multiplied.  The four waves' sums go to LDS (part)
// for wave 0, which adds them in fixed order after the block's barrier.

constexpr int kLocalWaves = 4;
constexpr int kLocalSlots = 5;       // P column blocks (up to four), then the gate
// A read by every workgroup (from L2).  Measured against the hand-off (two
// panels and two K splits, 16-byte partials; us, M = 1 / 16, local vs
// hand-off): 64 KiB of A, local always (1024 x 4096 r 32: 5.0 / 6.2, about
// 2.5 ahead); 128 KiB, local only for rank <= 32 and few rows (2048 x 4096
// r 32: 7.0 / 8.9 vs 7.5 / 8.2; 2048 x 8192: 8.4 / 9.9 vs 9.0 / 9.9;
// 1024 x 14336 r 64: 12.6 / 14.2 vs 11.2 / 13.1); 256 KiB, hand-off (by
// 2.6-3.2).
constexpr size_t kLocalMaxABytes = 128 * 1024;
constexpr size_t kLocalAnyABytes = 64 * 1024;
constexpr int64_t kLocalMaxRows = 4;            // rows up to which 128 KiB stays local
constexpr size_t kLocalBufBytes = 8 * 1024;      // one chunk: 8 units of 16 bytes per lane
__host__ __device__ __forceinline__ int local_pb(int rank) { return rank <= 32 ? 2 : 4; }
__host__ __device__ __forceinline__ size_t local_buf_bytes(int) { return kLocalBufBytes; }
__host__ __device__ __forceinline__ size_t local_lds_bytes(int rank) {
  return kLocalWaves * local_buf_bytes(rank) + (size_t)kLocalWaves * kLocalSlots * kWave * 16;
}

// PB column blocks (rank <= 16 PB); a chunk holds KB = 8 / PB 32-row blocks.
template <int PB>
struct LocalChunk {
  static constexpr int KB = 8 / PB;
  u32x4_t a[8];        // A units i * 64 + lane of the chunk
  half8_t x[KB];       // X fragments of the chunk's 32-k blocks
  half8_t g[KB];       // gate fragments (w_g) of the same blocks
};

template <int PB>
__device__ void ec_local_pass(const SkinnyKArgs& a, unsigned char* base, int lw) {
  const int lane = threadIdx.x % kWave, c16 = lane % 16, t4 = lane / 16;
  half_t* buf = reinterpret_cast<half_t*>(base + (size_t)lw * local_buf_bytes(a.rank));
  float4_t* part = reinterpret_cast<float4_t*>(base + kLocalWaves * local_buf_bytes(a.rank));
  constexpr int KB = LocalChunk<PB>::KB, kRows = 32 * KB;
  const int pblocks = (a.rank + 15) / 16;
  const int nch = (a.K + kRows - 1) / kRows;
  const int ch0 = lw * nch / kLocalWaves, ch1 = (lw + 1) * nch / kLocalWaves;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, (uint32_t)((size_t)a.M * a.K * 2));
  const __amdgpu_buffer_rsrc_t gr = make_rsrc(a.w_g, (uint32_t)a.K * 2u);
  const uint32_t xrow_off = c16 < a.M ? (uint32_t)c16 * (uint32_t)a.K * 2u : kOutOfRange;
  const u32x4_t* A16 = reinterpret_cast<const u32x4_t*>(a.A);
  // Rows past K: units clamped to the chunk's last real unit (finite), and
  // their X and w_g read as zeros.
  auto load = [&](LocalChunk<PB>& c, int ch) {
    const int r0 = ch * kRows;
    const int nvalid = min(kRows, a.K - r0) * a.rank / 8;   // rank % 4 == 0, K % 8 == 0
    const size_t u0 = (size_t)r0 * a.rank / 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) c.a[i] = A16[u0 + min(i * kWave + lane, nvalid - 1)];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int k = r0 + 32 * j + 8 * t4;
      c.x[j] = buffer_load_half8(xr, k < a.K ? xrow_off + 2u * (uint32_t)k : kOutOfRange);
      c.g[j] = buffer_load_half8(gr, k < a.K ? 2u * (uint32_t)k : kOutOfRange);
    }
  };
  float4_t acc[PB], accg = zero_float4();
#pragma unroll
  for (int p = 0; p < PB; ++p) acc[p] = zero_float4();
  auto process = [&](const LocalChunk<PB>& c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4_t*>(buf + (size_t)(i * kWave + lane) * 8) = c.a[i];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
#pragma unroll
      for (int p = 0; p < PB; ++p)
        if (p < pblocks)
          acc[p] = mfma16x16x32(c.x[j], lds_b_fragment_tr(buf + (size_t)j * 32 * a.rank + p * 16, a.rank, lane), acc[p]);
      accg = mfma16x16x32(c.x[j], c.g[j], accg);
    }
  };
  // Two chunks in registers: the steady-state loop issues every load
  // unconditionally, so the compiler's wait before a chunk's LDS writes
  // leaves the next chunk's loads in flight.
  LocalChunk<PB> c0, c1;
  if (ch0 < ch1) {
    load(c0, ch0);
    int ch = ch0;
    for (; ch + 2 < ch1; ch += 2) {
      load(c1, ch + 1);
      process(c0);
      load(c0, ch + 2);
      process(c1);
    }
    if (ch + 1 < ch1) {
      load(c1, ch + 1);
      process(c0);
      process(c1);
    } else {
      process(c0);
    }
  }
#pragma unroll
  for (int p = 0; p < PB; ++p) part[(lw * kLocalSlots + p) * kWave + lane] = acc[p];
  part[(lw * kLocalSlots + kLocalSlots - 1) * kWave + lane] = accg;
}

// ---------------------------------------------------------------- GEMM tile

// Static LDS of a GEMM workgroup: the sums of waves 1..3, then flags and the
// block-wide vote's word (512 bytes of room).
constexpr size_t static_lds_bytes(int nbw) { return (size_t)3 * kWave * nbw * 16 + 512; }

// Dynamic LDS of a GEMM workgroup with the EC on: the EC factor tile
// Bs[jblocks*32][TN] (fp16); Pc[16][pcs] floats (P in columns < rank, the
// final gate g' in column rank; pcs keeps every row 16-byte aligned and at
// least ps wide, so a row's P fragment is two 16-byte reads); then, split
// variant, Pt[16][ps] floats and gt[16].
//
// The EC operands that are ready at the start (the B tile, the split
// variant's P and g) are loaded into registers ahead of the weight stream, a
// fixed number per thread, with straight-line code.  (With a loop, or with a
// direct-to-LDS copy, among these loads the compiler can no longer count the
// loads in flight, and it waits for all of them before the first matrix
// instruction.)  Whatever these do not cover, and the fused variant's
// hand-off slabs, are loaded after the matrix instructions.
constexpr int kBLoads = 4;    // B tile halves per thread
constexpr int kPLoads = 1;    // split: 16-byte units of P per thread
__host__ __device__ __forceinline__ size_t gemm_bs_bytes(int ps, int tn) {
  return ((size_t)ps * tn * 2 + 15) & ~(size_t)15;
}
__host__ __device__ __forceinline__ int gemm_pc_stride(int rank, int ps) {
  const int w = rank + 1 > ps ? rank + 1 : ps;
  return (w + 3) & ~3;
}
__host__ __device__ __forceinline__ size_t gemm_pc_bytes(int rank, int ps) { return (size_t)16 * gemm_pc_stride(rank, ps) * 4; }
__host__ __device__ __forceinline__ size_t gemm_table_bytes(int ec_mode, int ps, int r1p, int P, int M) {
  if (ec_mode == 1) return 0;   // the fused hand-off is summed in registers
  return (size_t)16 * ps * 4 + 16 * 4;
}

// Fused consumer: the final [P | g'] of this call from the producers' slabs.
// Thread t takes 16-byte units q = t, t + 256, ... of a slab (two entries of
// row q / (r1p / 2)) and loads that unit of every slab, Q units x PB slabs
// in flight at once (one memory round trip per batch).  While any lane of the
// wave holds a unit whose tag is not yet this call's, the wave requests the
// whole batch again (bounded wait).  No per-unit branches: offsets of absent
// units are out of range (they read as zeros) and the tag test is plain
// arithmetic.  The slabs are added in fixed order and the gate applied to
// column rank; the result goes to Pc[row][col] (row stride pcs).
template <int Q, int PB>
struct HandoffBatch {
  u32x4_t v[Q][PB];
  uint32_t off[Q];   // byte offset of the unit in a slab (out of range: no unit)
  bool two[Q];       // entry 1 of the unit is a real column
  int row[Q], c0[Q];
};

template <int Q, int PB>
__device__ __forceinline__ void handoff_units(const SkinnyKArgs& a, int q0, HandoffBatch<Q, PB>& h) {
  const int pairs = a.M * a.r1p / 2;                     // 16-byte units per slab
#pragma unroll
  for (int i = 0; i < Q; ++i) {
    const int q = q0 + i * kThreads + (int)threadIdx.x;
    h.off[i] = q < pairs ? (uint32_t)q * 16u : kOutOfRange;
    h.row[i] = (2 * q) / a.r1p;
    h.c0[i] = (2 * q) % a.r1p;
    h.two[i] = h.c0[i] + 1 < a.rank + 1;
  }
}

template <int Q, int PB>
__device__ __forceinline__ void handoff_load(const SkinnyKArgs& a, __amdgpu_buffer_rsrc_t hr, int p0,
                                             HandoffBatch<Q, PB>& h) {
  const uint32_t slab_bytes = (uint32_t)a.M * (uint32_t)a.r1p * 8u;
#pragma unroll
  for (int i = 0; i < Q; ++i)
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      // off + slab offset stays out of range when off is (no wrap).
      const uint32_t o = p0 + j < a.P ? h.off[i] + (uint32_t)(p0 + j) * slab_bytes : kOutOfRange;
      h.v[i][j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(hr, o, 0, kCachePolicySc1));
    }
}

template <int Q, int PB>
__device__ __forceinline__ void handoff_wait(const SkinnyKArgs& a, __amdgpu_buffer_rsrc_t hr, uint32_t tag, int p0,
                                             HandoffBatch<Q, PB>& h) {
  for (uint32_t n = 0;; ++n) {
    bool stale = false;
#pragma unroll
    for (int i = 0; i < Q; ++i)
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const bool ready = (h.v[i][j][1] == tag) & (!h.two[i] | (h.v[i][j][3] == tag));
        stale |= (p0 + j < a.P) & (h.off[i] != kOutOfRange) & !ready;
      }
    if (!__any(stale)) break;
    if (n >= a.spin_limit) {
      if (threadIdx.x % kWave == 0) or_dev_u32(&a.sync[kError], kErrHandoffWait);
      break;
    }
    __builtin_amdgcn_s_sleep(4);
    handoff_load(a, hr, p0, h);
  }
}

template <int Q, int PB>
__device__ __forceinline__ void handoff_add(const SkinnyKArgs& a, int p0, const HandoffBatch<Q, PB>& h, float* s0,
                                            float* s1) {
#pragma unroll
  for (int i = 0; i < Q; ++i)
#pragma unroll
    for (int j = 0; j < PB; ++j)
      if (p0 + j < a.P) {
        s0[i] += bits_float(h.v[i][j][0]);
        s1[i] += bits_float(h.v[i][j][2]);
      }
}

template <int Q, int PB>
__device__ __forceinline__ void handoff_store(const SkinnyKArgs& a, const HandoffBatch<Q, PB>& h, const float* s0,
                                              const float* s1, float* Pc, int pcs) {
#pragma unroll
  for (int i = 0; i < Q; ++i) {
    if (h.off[i] == kOutOfRange) continue;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int col = h.c0[i] + e;
      if (col > a.rank) continue;
      float v = e == 0 ? s0[i] : s1[i];
      if (col == a.rank) {
        v = sigmoidf_(v + a.gate_bias);
        if (a.skip_tau > 0.0f && !(v >= a.skip_tau)) v = 0.0f;
      }
      Pc[h.row[i] * pcs + col] = v;
    }
  }
}

template <int Q, int PB>
__device__ void gather_handoff(const SkinnyKArgs& a, __amdgpu_buffer_rsrc_t hr, uint32_t tag, float* Pc, int pcs) {
  const int pairs = a.M * a.r1p / 2;
  for (int q0 = 0; q0 < pairs; q0 += Q * kThreads) {
    HandoffBatch<Q, PB> h;
    handoff_units(a, q0, h);
    float s0[Q], s1[Q];
#pragma unroll
    for (int i = 0; i < Q; ++i) s0[i] = s1[i] = 0.0f;
    for (int p0 = 0; p0 < a.P; p0 += PB) {
      handoff_load(a, hr, p0, h);
      handoff_wait(a, hr, tag, p0, h);
      handoff_add(a, p0, h, s0, s1);
    }
    handoff_store(a, h, s0, s1, Pc, pcs);
  }
}

// EXACT: every wave owns exactly CPW chunks (no validity test, so no load
// ends up under a branch).  ECM: the EC mode (0 none, 1 fused, 2 split), fixed
// at compile time so the loads of each mode are straight-line code.  G: group
// scales (one per 128-k chunk and column): each chunk's products are summed
// apart and scaled into the accumulator in fp32; the epilogue applies none.
template <int NBW, int CPW, bool EXACT, int ECM, bool G>
__global__ void __launch_bounds__(ECM == 3 ? kThreads + kLocalWaves * kWave : kThreads) skinny_kernel(SkinnyKArgs a) {
  extern __shared__ __align__(16) unsigned char dyn_lds[];
  __shared__ float4_t red[3][kWave][NBW];
  __shared__ uint32_t flags[2];        // [1] last split
  if (ECM == 1 && (int)blockIdx.x < a.P) {
    ec_producer(a, dyn_lds, blockIdx.x);
    return;
  }
  constexpr int TN = NBW * 16;
  // Local EC (waves 4..7): the projection, then the one barrier the weight
  // waves reach before wave 0 reads the sums (a split-K launch never takes
  // this mode).
  unsigned char* local_lds = dyn_lds + gemm_bs_bytes(a.ps, TN) + gemm_pc_bytes(a.rank, a.ps);
  if (ECM == 3 && threadIdx.x >= kThreads) {
    const int lw = __builtin_amdgcn_readfirstlane((int)(threadIdx.x - kThreads) / kWave);
    if (local_pb(a.rank) == 2) ec_local_pass<2>(a, local_lds, lw);
    else ec_local_pass<4>(a, local_lds, lw);
    __syncthreads();
    return;
  }
  const int b = blockIdx.x - a.P;
  const int s = b / a.T, t = b % a.T;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int c16 = lane % 16, t4 = lane / 16;
  const int cbeg = s * a.CPS, cend = min(a.KC, cbeg + a.CPS);
  const int wbeg = cbeg + w * CPW;
  const int nb0 = t * NBW;
  const int n0 = nb0 * 16;
  const int jblocks = ECM ? a.ps / 32 : 0;
  half_t* Bs = reinterpret_cast<half_t*>(dyn_lds);
  float* Pc = reinterpret_cast<float*>(dyn_lds + gemm_bs_bytes(a.ps, TN));
  unsigned char* table = dyn_lds + gemm_bs_bytes(a.ps, TN) + gemm_pc_bytes(a.rank, a.ps);
  const int pcs = gemm_pc_stride(a.rank, a.ps);
  // The epoch is read before the weight stream is requested, so it returns
  // ahead of it.
  const uint32_t tag = ECM == 1 ? call_tag(a.sync) : 0u;

  // ---- EC operands that are ready now, ahead of the weight stream: the B
  // tile (element q = row * TN + column; rows >= rank and columns >= N
  // clamped: they meet zero P columns or are never stored) and, split
  // variant, the given P (16-byte units of the [M][ps] table) and g.
  const int brows = jblocks * 32;
  half_t breg[kBLoads];
  if (ECM) {
#pragma unroll
    for (int i = 0; i < kBLoads; ++i) {
      const int q = i * kThreads + tid;
      const int row = min(q / TN, a.rank - 1), col = min(n0 + q % TN, a.N - 1);
      breg[i] = a.Bec[(size_t)row * a.N + col];
    }
  }
  float4_t preg[kPLoads];
  float greg = 0.0f;
  const int p_units = ECM == 2 ? a.M * a.ps / 4 : 0;
  if (ECM == 2) {
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.Pext, (uint32_t)((size_t)a.M * a.ps * 4));
#pragma unroll
    for (int i = 0; i < kPLoads; ++i) {
      const int u = i * kThreads + tid;
      preg[i] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                  pr, u < p_units ? (uint32_t)u * 16u : kOutOfRange, 0, 0));
    }
    greg = a.gext[min(tid, a.M - 1)];
  }

  // Fused: the producers' loads go first (their CUs carry no weight stream,
  // but the memory channels are shared).
  if (ECM == 1) {
    for (uint32_t i = 0; i < a.stream_delay; ++i) __builtin_amdgcn_s_sleep(1);
  }

  // Scales of this lane's columns (columns >= N are clamped, never stored);
  // group scales: those of each of the wave's chunks.
  half_t scr[NBW];
  half_t sg[G ? CPW : 1][NBW];
  if (!G) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) scr[nb] = a.scales[min(n0 + nb * 16 + c16, a.N - 1)];
  } else {
#pragma unroll
    for (int c = 0; c < (G ? CPW : 1); ++c) {
      const int kc = min(wbeg + c, a.KC - 1);   // chunks past the range meet zero X
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
        sg[c][nb] = a.scales[(size_t)kc * a.NBLK * 16 + min(n0 + nb * 16 + c16, a.N - 1)];
    }
  }

  // ---- issue every load of this wave's K range.  Chunk validity is uniform
  // over the wave.
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
  // Keep every load above this point (no load may sink into the
  // matrix-instruction block and pay a second round trip).
  __builtin_amdgcn_sched_barrier(0);

  // ---- matrix instructions
  float4_t acc[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) acc[nb] = zero_float4();
  if (!G) {
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[nb] = mfma16x16x32(xa[c][j], decode_w4(bw[c][nb][j]), acc[nb]);
  } else {
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      float4_t part[NBW];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) part[nb] = zero_float4();
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) part[nb] = mfma16x16x32(xa[c][j], decode_w4(bw[c][nb][j]), part[nb]);
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) acc[nb] += part[nb] * (float)sg[G ? c : 0][nb];
    }
  }

  // ---- EC operands -> LDS (then what the registers did not cover)
  if (ECM) {
#pragma unroll
    for (int i = 0; i < kBLoads; ++i) {
      const int q = i * kThreads + tid;
      if (q < brows * TN) Bs[q] = breg[i];
    }
    for (int q = kBLoads * kThreads + tid; q < brows * TN; q += kThreads) {
      const int row = min(q / TN, a.rank - 1), col = min(n0 + q % TN, a.N - 1);
      Bs[q] = a.Bec[(size_t)row * a.N + col];
    }
  }
  if (ECM == 2) {
    float4_t* Pt4 = reinterpret_cast<float4_t*>(table);
#pragma unroll
    for (int i = 0; i < kPLoads; ++i) {
      const int u = i * kThreads + tid;
      if (u < p_units) Pt4[u] = preg[i];
    }
    for (int u = kPLoads * kThreads + tid; u < p_units; u += kThreads)
      Pt4[u] = reinterpret_cast<const float4_t*>(a.Pext)[u];
    if (tid < a.M) reinterpret_cast<float*>(table + (size_t)16 * a.ps * 4)[tid] = greg;
  }

  // ---- four waves -> wave 0
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
  // Local EC: the four local waves' sums, in fixed order, into Pc (lane
  // (t4, c16) holds rows 4 t4 .. 4 t4 + 3 of column c16 of each block).
  if (ECM == 3 && w == 0) {
    const float4_t* part = reinterpret_cast<const float4_t*>(local_lds + kLocalWaves * local_buf_bytes(a.rank));
    const int pblocks = (a.rank + 15) / 16;
    for (int pb = 0; pb < pblocks; ++pb) {
      float4_t sum = part[pb * kWave + lane];
#pragma unroll
      for (int q = 1; q < kLocalWaves; ++q) sum += part[(q * kLocalSlots + pb) * kWave + lane];
      const int col = pb * 16 + c16;
      if (col < a.rank) {
#pragma unroll
        for (int v = 0; v < 4; ++v) Pc[(4 * t4 + v) * pcs + col] = sum[v];
      }
    }
    float4_t z = part[(kLocalSlots - 1) * kWave + lane];
#pragma unroll
    for (int q = 1; q < kLocalWaves; ++q) z += part[(q * kLocalSlots + kLocalSlots - 1) * kWave + lane];
    if (c16 == 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float g = sigmoidf_(z[v] + a.gate_bias);
        if (a.skip_tau > 0.0f && !(g >= a.skip_tau)) g = 0.0f;
        Pc[(4 * t4 + v) * pcs + a.rank] = g;
      }
    }
  }

  // ---- S splits -> the last to arrive (wave 0 exchanges, the block follows).
  // Workgroups that are not last count themselves out and leave.
  if (a.S > 1) {
    // One 16-byte device-coherent store / load per lane and panel.
    const __amdgpu_buffer_rsrc_t gpr = make_rsrc(a.gemm_part, (uint32_t)((size_t)a.T * a.S * NBW * kWave * 16));
    if (w == 0) {
      const uint32_t slot = (uint32_t)((t * a.S + s) * NBW) * kWave * 16u;
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[nb]), gpr,
                                               slot + (uint32_t)(nb * kWave + lane) * 16u, 0, kCachePolicySc1);
      drain_vm();
      if (lane == 0) flags[1] = (add_dev_u32(&a.sync[kTiles + t], 1u) == (uint32_t)(a.S - 1)) ? 1u : 0u;
    }
    __syncthreads();
    if (!flags[1]) {
      if (ECM == 1 && w == 0) count_out(a.sync, (uint32_t)(a.T * a.S + a.P), tag);
      return;
    }
    if (w == 0) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) acc[nb] = zero_float4();
      for (int ss = 0; ss < a.S; ++ss) {
        const uint32_t sl = (uint32_t)((t * a.S + ss) * NBW) * kWave * 16u;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[nb] += buffer_load_f4_dev(gpr, sl + (uint32_t)(nb * kWave + lane) * 16u);
      }
      if (lane == 0) st_dev_u32(&a.sync[kTiles + t], 0u);
    }
  }

  // ---- fused: gather the producers' slabs, check their tags (units not yet
  // published are reloaded, bounded wait), add them and apply the gate.
  if (ECM == 1) {
    // The whole table after the matrix instructions.  (Requested any
    // earlier, the loads would queue behind the weight stream and be served
    // about when it is, normally just before the producers publish, which
    // costs a second round trip.)  Sixteen loads in flight per thread.
    const __amdgpu_buffer_rsrc_t hr = make_rsrc(a.handoff, (uint32_t)((size_t)a.P * a.M * a.r1p * 8));
    if (a.P <= 8) gather_handoff<2, 8>(a, hr, tag ^ a.wait_xor, Pc, pcs);
    else gather_handoff<1, 16>(a, hr, tag ^ a.wait_xor, Pc, pcs);
    __syncthreads();
    // Count this workgroup out (wave 1, off wave 0's path): the last of the
    // call's workgroups returns the counters to zero and advances the epoch.
    if (w == 1) count_out(a.sync, (uint32_t)(a.T * a.S + a.P), tag);
  }
  if (w > 0) return;

  // ---- gated EC epilogue (wave 0).  Lane (t4, c16): P row c16, columns
  // 8 t4 .. 8 t4 + 7 of each 32-column block (two 16-byte reads of a
  // 16-byte aligned row), times the row's gate, as the A fragment; the B
  // fragment of Bs from two transposing reads.
  const float* prow = ECM != 2 ? Pc + (size_t)c16 * pcs : reinterpret_cast<const float*>(table) + (size_t)c16 * a.ps;
  float4_t ec[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) ec[nb] = zero_float4();
  if (ECM) {
    const float gv = c16 < a.M ? (ECM != 2 ? prow[a.rank] : reinterpret_cast<const float*>(table + (size_t)16 * a.ps * 4)[c16])
                               : 0.0f;                   // the final gate g'
    if (__any(gv != 0.0f)) {
      for (int jb = 0; jb < jblocks; ++jb) {
        const int k0 = jb * 32 + 8 * t4;
        const float4_t lo = *reinterpret_cast<const float4_t*>(prow + k0);
        const float4_t hi = *reinterpret_cast<const float4_t*>(prow + k0 + 4);
        half8_t pa;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = e < 4 ? lo[e] : hi[e - 4];
          pa[e] = (k0 + e < a.rank && gv != 0.0f) ? (half_t)(gv * pv) : (half_t)0.0f;
        }
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
          ec[nb] = mfma16x16x32(pa, lds_b_fragment_tr(Bs + (size_t)jb * 32 * TN + nb * 16, TN, lane), ec[nb]);
      }
    }
  }

  // ---- Y = fp16(s acc + EC)
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int col = n0 + nb * 16 + c16;
    const float sc = G ? 1.0f : (float)scr[nb];
    if (col < a.N) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 4 * t4 + v;
        if (row < a.M) a.Y[(size_t)row * a.N + col] = (half_t)fmaf(sc, acc[nb][v], ec[nb][v]);
      }
    }
  }
}

// Let a kernel use all of a workgroup's LDS beside its static LDS (once per
// instantiation and device).
template <auto Kernel, int NBW>
hipError_t allow_full_lds() {
  return set_max_dynamic_lds(reinterpret_cast<const void*>(Kernel), (int)(kMaxLdsBytes - static_lds_bytes(NBW)));
}

template <int NBW, int CPW, bool EXACT, bool G>
hipError_t launch_exact(const SkinnyKArgs& k, size_t lds, void* stream) {
  const dim3 grid(k.P + k.T * k.S), block(kThreads);
  hipError_t e = hipSuccess;
  if (k.ec_mode == 3) {
    e = allow_full_lds<&skinny_kernel<NBW, CPW, EXACT, 3, G>, NBW>();
    if (e == hipSuccess)
      hipLaunchKernelGGL((skinny_kernel<NBW, CPW, EXACT, 3, G>), grid, dim3(kThreads + kLocalWaves * kWave), lds,
                         (hipStream_t)stream, k);
  } else if (k.ec_mode == 1) {
    e = allow_full_lds<&skinny_kernel<NBW, CPW, EXACT, 1, G>, NBW>();
    if (e == hipSuccess) hipLaunchKernelGGL((skinny_kernel<NBW, CPW, EXACT, 1, G>), grid, block, lds, (hipStream_t)stream, k);
  } else if (k.ec_mode == 2) {
    e = allow_full_lds<&skinny_kernel<NBW, CPW, EXACT, 2, G>, NBW>();
    if (e == hipSuccess) hipLaunchKernelGGL((skinny_kernel<NBW, CPW, EXACT, 2, G>), grid, block, lds, (hipStream_t)stream, k);
  } else {
    e = allow_full_lds<&skinny_kernel<NBW, CPW, EXACT, 0, G>, NBW>();
    if (e == hipSuccess) hipLaunchKernelGGL((skinny_kernel<NBW, CPW, EXACT, 0, G>), grid, block, lds, (hipStream_t)stream, k);
  }
  return e != hipSuccess ? e : hipGetLastError();
}

template <int NBW, int CPW, bool G>
hipError_t launch_nbw_cpw(const SkinnyKArgs& k, bool exact, size_t lds, void* stream) {
  return exact ? launch_exact<NBW, CPW, true, G>(k, lds, stream) : launch_exact<NBW, CPW, false, G>(k, lds, stream);
}

constexpr int kMaxCpw = 8;   // chunks per wave kept in flight (NBW <= 2)

template <int NBW, bool G>
hipError_t launch_nbw(const SkinnyKArgs& k, int cpw, bool exact, size_t lds, void* stream) {
  if (cpw <= 1) return launch_nbw_cpw<NBW, 1, G>(k, exact, lds, stream);
  if (cpw <= 2) return launch_nbw_cpw<NBW, 2, G>(k, exact, lds, stream);
  if constexpr (NBW == 4) {
    return launch_nbw_cpw<NBW, 4, G>(k, exact, lds, stream);
  } else {
    if (cpw <= 4) return launch_nbw_cpw<NBW, 4, G>(k, exact, lds, stream);
    return launch_nbw_cpw<NBW, 8, G>(k, exact, lds, stream);
  }
}

template <bool G>
hipError_t launch_g(const SkinnyKArgs& k, int nbw, int cpw, bool exact, size_t lds, void* stream) {
  if (nbw == 4) return launch_nbw<4, G>(k, cpw, exact, lds, stream);
  if (nbw == 2) return launch_nbw<2, G>(k, cpw, exact, lds, stream);
  return launch_nbw<1, G>(k, cpw, exact, lds, stream);
}

}  // namespace

SkinnyShape skinny_shape(int64_t M, int64_t K, int64_t N, int64_t rank, bool fused, int cus,
                         size_t scratch_base) {
  SkinnyShape sh;
  const int64_t KC = k_pad(K) / kKChunk, NBLK = n_pad(N) / kNBlock;
  // Candidates (panels per workgroup, K splits).  Preferred: the most
  // workgroups up to one per CU; then "exact" ranges (every wave owns CPW =
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
      const int64_t score = (std::min<int64_t>(wgs, cus) << 32) + (exact ? 1LL << 30 : 0) +
                            ((64 - S) << 8) + nbw;
      if (score > best_score) {
        best_score = score;
        sh.nbw = nbw; sh.S = (int)S; sh.T = (int)T; sh.CPS = (int)CPS; sh.CPW = (int)CPW;
      }
    }
  }
  // Local EC (every GEMM workgroup computes the projection itself): no K
  // split of the weight GEMM, rank % 4 == 0 (transposing LDS reads), rank <=
  // 64, and an A small enough that every workgroup reading it from L2 costs
  // less than the producers' hand-off.
  auto local_ok = [&]() {
    const size_t a_bytes = (size_t)K * rank * 2;
    return fused && rank > 0 && sh.S == 1 && rank % 4 == 0 && rank <= 64 &&
           (a_bytes <= kLocalAnyABytes || (a_bytes <= kLocalMaxABytes && rank <= 32 && M <= kLocalMaxRows));
  };
  // Fused with the hand-off, where the search gives one 16-column panel and
  // no K split per workgroup: two panels and two K splits keep the workgroup
  // count and halve the X each workgroup reads and the hand-off gathers (only
  // the last split of a tile runs the epilogue).  Measured on 4096 x 4096,
  // rank 32: M = 16 11.35 -> 10.27 us, M = 1 9.48 -> 9.34 us.  Where the
  // search already splits K, doubling the split was slower (2048 x 2048,
  // 8192 x 2048, 14336 x 4096).
  if (fused && rank > 0 && !local_ok() && sh.nbw == 1 && sh.S == 1 && KC % 2 == 0 && KC / 2 <= 4 * kMaxCpw) {
    sh.nbw = 2;
    sh.S = 2;
    sh.T = (int)ceil_div(NBLK, 2);
    sh.CPS = (int)(KC / 2);
    sh.CPW = (int)ceil_div(sh.CPS, 4);
  }
  // Round CPW up to an instantiated value.
  sh.CPW = sh.CPW <= 1 ? 1 : sh.CPW <= 2 ? 2 : sh.CPW <= 4 ? 4 : 8;
  const int ps = rank > 0 ? (int)p_stride(rank) : 0;
  const int r1p = (int)round_up(rank + 1, 2);
  if (local_ok()) sh.local_ec = true;
  if (fused && rank > 0 && !sh.local_ec) {
    // Producer slabs: a power of two near K / 8 (128 .. 1024), or near K / 16
    // for calls of up to four rows, halved until one slab's LDS (A slab, w_g
    // slab and column, X slab) fits 64 KiB, so two workgroups fit a CU (every
    // workgroup of the launch gets this LDS).  Few slabs keep the hand-off
    // that every GEMM workgroup reads small; with few rows that hand-off is
    // small anyway and smaller slabs arrive sooner (4096 x 4096, rank 32:
    // 16 producers 8.54 / 8.70 us at M = 1 / 4 against 8.90 / 8.94 with 8; at
    // M = 16, 10.66 against 10.02).
    int64_t ksp = 128;
    const int64_t slabs = M <= 4 ? 16 : 8;
    while (ksp < 1024 && ksp * slabs < K) ksp *= 2;
    while (ksp > 128 && producer_lds_bytes((int)ksp, (int)rank) > 64 * 1024) ksp /= 2;
    sh.ksp = (int)ksp;
    sh.P = (int)ceil_div(K, ksp);
    sh.lds = producer_lds_bytes((int)ksp, (int)rank);
  }
  if (rank > 0)
    sh.lds_gemm = gemm_bs_bytes(ps, sh.nbw * 16) + gemm_pc_bytes((int)rank, ps) +
                  gemm_table_bytes(fused ? 1 : 2, ps, r1p, sh.P, (int)M) +
                  (sh.local_ec ? local_lds_bytes((int)rank) : 0);
  // Workspace: sync words in the counter header and the hand-off slabs in the
  // header's hand-off region; the split-K slots as scratch from scratch_base
  // on.
  size_t off = scratch_base;
  auto take = [&](size_t bytes) { size_t o = off; off = (size_t)round_up((int64_t)(off + bytes), 256); return o; };
  sh.ws_sync = kGemmSyncOffset;
  sh.ws_handoff = kHandoffOffset;
  if (sh.S > 1) sh.ws_gemm_part = take(sizeof(float) * 4 * kWave * (size_t)sh.nbw * sh.T * sh.S);
  sh.ws_bytes = (sh.S > 1 || sh.P > 0) ? (off > kSyncHeaderBytes ? off : kSyncHeaderBytes) : 0;
  const size_t lds_room = kMaxLdsBytes - static_lds_bytes(sh.nbw);
  // best_score < 0: no split of K fits the kernel's chunks per wave (K above
  // 64 splits x 32 chunks of 128).
  sh.fits = best_score >= 0 && kTiles + sh.T <= kMaxSyncWords && sh.lds <= lds_room && sh.lds_gemm <= lds_room &&
            (size_t)sh.P * M * r1p * 8 <= kHandoffBytes;
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
  const int ec_mode = L.ec_mode == 1 && sh.local_ec ? 3 : L.ec_mode;
  k.P = ec_mode == 1 ? sh.P : 0;
  k.ksp = sh.ksp;
  k.ps = L.ec_mode ? (int)p_stride(L.rank) : 0;
  k.r1p = (int)round_up(L.rank + 1, 2);
  k.ec_mode = ec_mode;
  k.gate_bias = L.gate_bias; k.skip_tau = L.skip_tau;
  char* ws = (char*)L.workspace;
  k.sync = (uint32_t*)(ws + sh.ws_sync);   // absolute offsets from the workspace base
  k.handoff = (uint64_t*)(ws + sh.ws_handoff);
  k.gemm_part = (float*)(ws + sh.ws_gemm_part);
  k.Pext = L.Pext;
  k.gext = L.gext;
  k.spin_limit = L.spin_limit;
  k.wait_xor = L.wait_xor;
  k.stream_delay = ec_mode == 1 && L.M > 4 ? kStreamDelay : 0;
  size_t lds = k.P > 0 ? sh.lds : 0;
  if (L.ec_mode && sh.lds_gemm > lds) lds = sh.lds_gemm;
  const bool exact = sh.CPS == 4 * sh.CPW && (int64_t)sh.CPS * sh.S == k.KC;
  if (L.grouped) return launch_g<true>(k, sh.nbw, sh.CPW, exact, lds, stream);
  return launch_g<false>(k, sh.nbw, sh.CPW, exact, lds, stream);
}

}  // namespace spear
