// Tiled (prefill, M > 16) W4 GEMM with the gated EC term in its epilogue
// (SPEAR page, abstract: the work after the EC projection runs inside the
// low-bit GEMM):
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
//
// Data flow per 128-k step (one packed chunk per 16-column panel):
//   * X tile [TM x 128] fp16 -> LDS by direct 16-byte copies (no VGPRs), two
//     stages; units of 16 bytes are XOR-swizzled by row so the fragment reads
//     of 16 rows hit 16 different bank groups;
//   * packed int4 weights -> VGPRs, one step ahead (16 bytes per lane = the B
//     operand of four 32-k blocks);
//   * one barrier per step: after it, stage s is complete and every wave is
//     done with stage s-1, whose buffer the copies for step s+1 then refill.
// Tiles are ordered so that the workgroups of one row of tiles run on one XCD
// (blocks are dealt round-robin to the 8 XCDs), keeping that X row in one L2.
//
// When the tiles alone do not fill the GPU (mid-size M), K is split over S
// workgroups per tile: each stores its fp32 partial tile (device-coherent
// 16-byte stores) and takes a ticket; the last to arrive adds the S partials
// in fixed order, so results do not depend on timing, and runs the epilogue.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "ec_block.h"
#include "internal.h"

namespace spear {

namespace {

constexpr int kGemmThreads = 256;
constexpr int kKt = 128;                 // k per step (one packed chunk)
constexpr int kUnitsPerRow = kKt / 8;    // 16-byte units per X row per step
constexpr int kEcChunk = 64;             // rank columns per epilogue pass
typedef __attribute__((address_space(3))) void lds_void_t;

struct GemmKArgs {
  const half_t* X;
  const u32x4_t* Wq;
  const half_t* scales;
  const half_t* B;
  const float* P;
  const float* g;
  half_t* Y;
  int M, K, N, rank, KC, NBLK, ps, ec;
  int MT, NT;             // row and column tiles
  int S, CPS;             // K splits, 128-k chunks per split
  float* part;            // [tile][S][MBW * NBW][256 threads] float4 partials
  uint32_t* tickets;      // [tile] split counters (back to zero after each call)
  // Fused launch only: P and g are produced by the launch's EC workgroups.
  const uint32_t* ready;  // [ec row tiles of 64] flags, raised to the call's tag
  int ec_tiles;           // EC row tiles
  uint32_t* error;        // sticky error word: kErrReadyWait when a wait for a ready flag gives up
  uint32_t spin_limit;
  uint32_t wait_xor;      // the tiles wait for tag ^ wait_xor (0, or a test hook's value)
};

// The fused launch: E EC workgroups (the first blocks), then the GEMM tiles.
struct FusedKArgs {
  GemmKArgs g;
  EcKArgs e;
  int E;                  // leading blocks that are EC workgroups (a multiple of 8)
  int ec_blocks;          // of which the real ones (m_tiles x splits)
  uint32_t* sync;         // GEMM sync words (finishers, epoch)
};

// ---- gated EC epilogue pieces shared by the tile kernels.  The LDS (free
// once every wave is done with the X stages) holds, per 64-column chunk of
// the rank, the B rows bs[64][TN] fp16 (rows >= rank clamped: they meet zero
// P columns; columns >= N clamped: never stored) and pg[TM][64] = fp16(g' P)
// of the tile's rows (rows >= M clamped: never stored), after gs[TM], the
// tile's gates.
template <int TN>
__device__ __forceinline__ size_t ec_pg_offset() { return (size_t)kEcChunk * TN * 2; }
template <int TM, int TN>
__device__ __forceinline__ size_t ec_gs_offset() { return (size_t)kEcChunk * TN * 2 + (size_t)TM * kEcChunk * 2; }

// Fused launch: the ready flags of the EC row tiles under rows
// [m0, m0 + TM), read by thread 0 when the workgroup starts (TM / 64 <= 4
// of them; those already raised then need no second look).
template <int TM, bool FUSED>
__device__ __forceinline__ void ec_flags_early(const GemmKArgs& a, int m0, uint32_t (&early)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) early[i] = 0;
  if (FUSED && a.ec && threadIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < (TM + 63) / 64; ++i)
      if (m0 / 64 + i < a.ec_tiles) early[i] = ld_dev_u32(&a.ready[m0 / 64 + i]);
  }
}

// Fused launch: wait until the EC row tiles under rows [m0, m0 + TM) are
// published (one thread polls the flags not seen raised early).  Then (every
// launch) gs[TM] = g' of the tile's rows, 0 past M.  Starts and ends with a
// block-wide barrier.
template <int TM, bool FUSED>
__device__ __forceinline__ void ec_prepare(const GemmKArgs& a, int m0, uint32_t tag, float* gs,
                                           const uint32_t (&early)[4], bool gs_ready = false) {
  const int tid = threadIdx.x;
  if (FUSED && tid == 0) {
    const int t_end = min(a.ec_tiles, (m0 + TM + 63) / 64);
#pragma unroll
    for (int i = 0; i < (TM + 63) / 64; ++i) {
      const int t = m0 / 64 + i;
      if (t >= t_end || early[i] == (tag ^ a.wait_xor)) continue;
      uint32_t n = 0;
      while (ld_dev_u32(&a.ready[t]) != (tag ^ a.wait_xor)) {
        __builtin_amdgcn_s_sleep(2);
        if (++n > a.spin_limit) {
          or_dev_u32(a.error, kErrReadyWait);
          break;
        }
      }
    }
  }
  if (gs_ready) wait_vm_all();                 // this wave's copies into gs (copy_ec_rows) have landed
  __syncthreads();                             // also: every wave is done with the X stages
  if (!gs_ready && tid < TM) gs[tid] = m0 + tid < a.M ? (FUSED ? ld_dev(&a.g[m0 + tid]) : a.g[m0 + tid]) : 0.0f;
  __syncthreads();
}

// Stage rank columns [j0, j0 + 64) of the EC operands: bs (16-byte loads
// when B rows are 16-byte aligned, else element-wise; b_ready: already
// copied there by copy_b_chunk) and pg (p_lds: the chunk's P units already
// copied into LDS by copy_ec_rows, unit u at p_lds + 16 u); every load of the
// chunk is issued before the first is used (one memory round trip), P's
// device-coherent when the same launch produced it.  Ends with a block-wide
// barrier.
template <int TM, int TN, bool FUSED, int THREADS>
__device__ __forceinline__ void ec_stage_chunk(const GemmKArgs& a, int j0, int m0, int n0, unsigned char* lds,
                                               __amdgpu_buffer_rsrc_t pr, bool b_ready = false,
                                               const unsigned char* p_lds = nullptr) {
  constexpr int kPUnits = TM * (kEcChunk / 4) / THREADS;   // 16-byte P units per thread
  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  constexpr int kBUnits = kEcChunk * TN / 8 / THREADS;   // 16-byte B units per thread
  static_assert(kEcChunk * TN / 8 % THREADS == 0, "whole B units per thread");
  static_assert(TM * (kEcChunk / 4) % THREADS == 0, "whole P units per thread");
  half_t* bs = reinterpret_cast<half_t*>(lds);
  half_t* pg = reinterpret_cast<half_t*>(lds + ec_pg_offset<TN>());
  const float* gs = reinterpret_cast<const float*>(lds + ec_gs_offset<TM, TN>());
  (void)w; (void)lane;
  __syncthreads();
  const bool bvec = a.N % 8 == 0 && (reinterpret_cast<uintptr_t>(a.B) & 15) == 0;
  u32x4_t bv[kBUnits];
  if (b_ready) {
  } else if (bvec) {
#pragma unroll
    for (int i = 0; i < kBUnits; ++i) {
      const int idx = i * THREADS + tid, r = idx / (TN / 8), c8 = idx % (TN / 8);
      bv[i] = *reinterpret_cast<const u32x4_t*>(a.B + (size_t)min(j0 + r, a.rank - 1) * a.N +
                                                 min(n0 + c8 * 8, a.N - 8));
    }
  } else {
    for (int idx = tid; idx < kEcChunk * TN; idx += THREADS) {
      const int r = idx / TN, c = idx % TN;
      bs[idx] = a.B[(size_t)min(j0 + r, a.rank - 1) * a.N + min(n0 + c, a.N - 1)];
    }
  }
  float4_t pv[kPUnits];
#pragma unroll
  for (int i = 0; i < kPUnits; ++i) {
    const int idx = i * THREADS + tid, r = idx / (kEcChunk / 4), c4 = idx % (kEcChunk / 4);
    const int row = min(m0 + r, a.M - 1), col = j0 + c4 * 4;
    const uint32_t off = col < a.ps ? (uint32_t)(((size_t)row * a.ps + col) * 4) : kOutOfRange;
    pv[i] = p_lds ? *reinterpret_cast<const float4_t*>(p_lds + (size_t)idx * 16)
          : FUSED ? buffer_load_f4_dev(pr, off)
                  : __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(pr, off, 0, 0));
  }
  if (bvec && !b_ready) {
#pragma unroll
    for (int i = 0; i < kBUnits; ++i) reinterpret_cast<u32x4_t*>(bs)[i * THREADS + tid] = bv[i];
  }
#pragma unroll
  for (int i = 0; i < kPUnits; ++i) {
    const int idx = i * THREADS + tid, r = idx / (kEcChunk / 4), c4 = idx % (kEcChunk / 4);
    const float gv = gs[r];
    half_t* dst = pg + (size_t)r * kEcChunk + c4 * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = (half_t)(gv * pv[i][e]);
  }
  wait_vm_all();
  __syncthreads();
}

// B rows [j0, j0 + 64) of the tile's columns straight into bs[64][TN] by
// direct 16-byte buffer-to-LDS copies (B rows 16-byte aligned, N % 8 == 0):
// copy i of wave w fills the 64 units (i NW + w) 64 .. + 63 of bs, unit u
// holding B[min(j0 + u / (TN / 8), rank - 1)][n0 + 8 (u % (TN / 8))]
// (columns past N read as zeros and are never stored).  Nothing waits for
// the copies here; ec_stage_chunk's final wait and barrier do.
template <int TN, int THREADS>
__device__ __forceinline__ void copy_b_chunk(const GemmKArgs& a, int j0, int n0, unsigned char* bs_lds) {
  constexpr int NW = THREADS / kWave;
  constexpr int kUnits = kEcChunk * TN / 8;
  static_assert(kUnits % THREADS == 0, "whole copies per wave");
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(a.B, (uint32_t)((size_t)a.rank * a.N * 2));
#pragma unroll
  for (int i = 0; i < kUnits / THREADS; ++i) {
    const int u0 = (i * NW + w) * kWave, u = u0 + lane;
    const int r = u / (TN / 8), c = n0 + (u % (TN / 8)) * 8;
    const uint32_t voff = c < a.N ? (uint32_t)(((size_t)min(j0 + r, a.rank - 1) * a.N + c) * 2) : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_void_t*)(bs_lds + (size_t)u0 * 16), 16, voff, 0, 0, 0);
  }
}

// P rank columns [0, 64) of the tile's rows and their gates, from an earlier
// launch (the split variant), straight into LDS: unit u = 16 r + c4 of P (row
// m0 + r clamped to M - 1, columns 4 c4 .. + 3; columns past the stride read
// as zeros) at p_lds + 16 u, the unit layout ec_stage_chunk reads, and
// g'[m0 + r] at gs + 4 r (rows past M read as zeros) by the first TM / 64
// waves.  Nothing waits for the copies here.
template <int TM, int THREADS>
__device__ __forceinline__ void copy_ec_rows(const GemmKArgs& a, int m0, unsigned char* p_lds, float* gs) {
  constexpr int NW = THREADS / kWave;
  constexpr int kUnits = TM * (kEcChunk / 4);
  static_assert(kUnits % THREADS == 0 && TM % kWave == 0 && TM / kWave <= NW, "whole copies per wave");
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.P, (uint32_t)((size_t)a.M * a.ps * 4));
#pragma unroll
  for (int i = 0; i < kUnits / THREADS; ++i) {
    const int u0 = (i * NW + w) * kWave, u = u0 + lane;
    const int r = u / (kEcChunk / 4), col = (u % (kEcChunk / 4)) * 4;
    const uint32_t voff = col < a.ps ? (uint32_t)(((size_t)min(m0 + r, a.M - 1) * a.ps + col) * 4) : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(pr, (lds_void_t*)(p_lds + (size_t)u0 * 16), 16, voff, 0, 0, 0);
  }
  if (w < TM / kWave) {
    const __amdgpu_buffer_rsrc_t gr = make_rsrc(a.g, (uint32_t)a.M * 4u);
    const int row = m0 + w * kWave + lane;
    const uint32_t voff = row < a.M ? (uint32_t)row * 4u : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(gr, (lds_void_t*)(gs + w * kWave), 4, voff, 0, 0, 0);
  }
}

// X stages of a tile kernel: three (loads two steps ahead) for the 64-row
// tiles of small M, where the steps are short; two otherwise.
constexpr int stages_for(int tm, bool split) { return split && tm == 64 ? 3 : 2; }
// Epilogue LDS after the X stages (the first B chunk copied in during the
// last k-step): 128-row tiles without a K split, where both fit.
constexpr bool epilogue_after_stages(int tm, bool split) { return tm == 128 && !split; }

// Waves side by side with uneven column panels (TP > 0): eight waves, each
// 128 rows of a 128 x 448 tile; waves 0-3 own four 16-column panels each
// (panels 0-15), waves 4-7 three (panels 16-27).  Waves are dealt to the
// four SIMDs of a CU round-robin, so each SIMD runs one wave of four panels
// and one of three: seven panels of matrix work per SIMD, two waves to issue
// it.
__device__ __forceinline__ int uneven_first_panel(int w) { return w < 4 ? 4 * w : 16 + 3 * (w - 4); }

// One GEMM workgroup (tile block `block`).  Wave tile MBW x NBW blocks of
// 16 x 16; workgroup WM x WN waves (four, or eight with TP = 28 panels per
// tile dealt unevenly: see uneven_first_panel).  SPLIT: K split over a.S
// workgroups per tile.  FUSED: P and g come from EC workgroups of the same
// launch; the epilogue waits for their ready flags (raised to `tag`) and
// reads P and g with device-coherent loads.
template <int MBW, int NBW, int WM, int WN, bool SPLIT, bool FUSED, bool G, int TP = 0>
__device__ __forceinline__ void gemm_block(const GemmKArgs& a, int block, unsigned char* lds, uint32_t tag) {
  constexpr int NW = WM * WN;
  constexpr int THREADS = NW * kWave;
  constexpr bool UNEVEN = TP != 0;
  static_assert(!UNEVEN ? NW == 4 : (WM == 1 && WN == 8 && NBW == 4 && TP == 28 && !SPLIT && !FUSED),
                "four waves, or eight with uneven panels");
  constexpr int TPANELS = UNEVEN ? TP : NBW * WN;           // 16-column panels per tile
  constexpr int TM = 16 * MBW * WM;
  constexpr int TN = 16 * TPANELS;
  constexpr int kStageHalves = TM * kKt;                    // one X stage
  constexpr int kCopiesPerWave = TM * kUnitsPerRow / kWave / NW;
  constexpr int NSTAGE = stages_for(TM, SPLIT);             // X stages in LDS
  half_t* xs = reinterpret_cast<half_t*>(lds);                // [NSTAGE][TM][kKt], swizzled units
  // 128-row tiles without a K split keep the epilogue's LDS past the X
  // stages, so the first B chunk can be copied in during the last k-step.
  constexpr bool PREF = epilogue_after_stages(TM, SPLIT);
  unsigned char* epi = lds + (PREF ? (size_t)NSTAGE * kStageHalves * 2 : 0);

  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int c16 = lane % 16, t4 = lane / 16;
  const int wm = w % WM, wn = w / WM;

  // Tile order: with a multiple of 8 row tiles, XCD x (block % 8) takes row
  // tiles x, x + 8, ... and walks the column tiles of each; with a multiple
  // of 16 it takes them in pairs (x + 16 i, x + 16 i + 8) whose two tiles of
  // one column run side by side, so each packed-weight tile the XCD fetches
  // serves two workgroups from its L2 (prefill 2048 x 4096 x 14336, A/B on
  // one box each: EC off 186-189 -> 182-184 us and 197-199 -> 195-198 us;
  // g128 unchanged).
  int m_tile, n_tile;
  const int tiles = a.MT * a.NT;
  const int split = block / tiles;
  {
    const int bid = block % tiles;
    if (a.MT % 16 == 0) {
      const int xcd = bid % 8, j = bid / 8;
      const int pair = j / (2 * a.NT), r = j % (2 * a.NT);
      m_tile = xcd + 8 * (2 * pair + r % 2);
      n_tile = r / 2;
    } else if (a.MT % 8 == 0) {
      const int xcd = bid % 8, j = bid / 8;
      m_tile = xcd + 8 * (j / a.NT);
      n_tile = j % a.NT;
    } else {
      m_tile = bid / a.NT;
      n_tile = bid % a.NT;
    }
  }
  // The wave's panels within the tile: [pan0, pan0 + NBW), or with uneven
  // panels [pan0, pan0 + 4) for waves 0-3 and [pan0, pan0 + 3) for 4-7;
  // has(nb): the wave owns its nb-th panel (wave-uniform).
  const int pan0 = UNEVEN ? uneven_first_panel(w) : wn * NBW;
  const bool four = !UNEVEN || w < 4;
  auto has = [&](int nb) { return !UNEVEN || nb < 3 || four; };
  const int m0 = m_tile * TM, nb_base = n_tile * TPANELS + pan0;
  uint32_t early[4];
  ec_flags_early<TM, FUSED>(a, m0, early);

  // ---- X tile copies for step kc into stage st, through a buffer resource
  // over X: rows >= M fall outside it and units at k >= K are sent outside
  // it, so both read as zeros.  Copy i of wave w fills rows (w * kCopiesPerWave + i) * 4
  // .. + 3; lane L writes slot L % 16 of row L / 16, holding the source unit
  // (slot ^ (row % 16)).
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, (uint32_t)((size_t)a.M * a.K * 2));
  const uint32_t row_bytes = (uint32_t)a.K * 2u;
  // A step whose 128 k lie inside K takes the unit's offset at k = 0, the
  // same every step, and adds the step's k as the scalar offset; only a last
  // step past K computes per-unit offsets (units at k >= K sent outside).
  uint32_t xoff[kCopiesPerWave];
#pragma unroll
  for (int i = 0; i < kCopiesPerWave; ++i) {
    const int row = (w * kCopiesPerWave + i) * 4 + lane / 16;
    xoff[i] = (uint32_t)(m0 + row) * row_bytes + (uint32_t)((lane % 16) ^ (row % 16)) * 16u;
  }
  const uint32_t* xo = xoff;
  auto issue_x = [&](int kc, int st) {
    if ((kc + 1) * kKt <= a.K) {
#pragma unroll
      for (int i = 0; i < kCopiesPerWave; ++i) {
        const int row = (w * kCopiesPerWave + i) * 4;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xr, (lds_void_t*)(xs + (size_t)st * kStageHalves + (size_t)row * kKt), 16, xo[i],
            (uint32_t)kc * (kKt * 2u), 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kCopiesPerWave; ++i) {
        const int row = (w * kCopiesPerWave + i) * 4 + lane / 16;
        const int unit = (lane % 16) ^ (row % 16);
        const int k = kc * kKt + unit * 8;
        const uint32_t voff = k < a.K ? (uint32_t)(m0 + row) * row_bytes + (uint32_t)k * 2u : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xr, (lds_void_t*)(xs + (size_t)st * kStageHalves + (size_t)(row - lane / 16) * kKt), 16, voff, 0, 0, 0);
      }
    }
  };
  // Packed weights through a buffer resource (panels >= NBLK clamped: their
  // columns are never stored).
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.Wq, (uint32_t)((size_t)a.NBLK * a.KC * 1024));
  auto load_w = [&](int kc, u32x4_t* dst) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      if (!has(nb)) continue;
      const uint32_t voff = ((uint32_t)min(nb_base + nb, a.NBLK - 1) * (uint32_t)a.KC * 64u + (uint32_t)lane) * 16u;
      dst[nb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wr, voff, kc * 1024, 0));
    }
  };

  // Group scales (G): s[kc][column] of the lane's column in each of its NBW
  // panels (columns >= N clamped: never stored).
  const int ncol0 = nb_base * 16 + c16;
  auto load_s = [&](int kc, half_t* dst) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
      if (has(nb)) dst[nb] = a.scales[(size_t)kc * a.NBLK * 16 + min(ncol0 + nb * 16, a.N - 1)];
  };

  float4_t acc[MBW][NBW];
#pragma unroll
  for (int i = 0; i < MBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[i][j] = zero_float4();

  const int kc_begin = split * a.CPS, kc_end = min(a.KC, kc_begin + a.CPS);
  // The matrix instructions of one 128-k step from X stage `st` and the
  // packed words w (G: each decoded fragment times its group scale, sg).
  auto compute = [&](int st, const u32x4_t* w_, const half_t* sg) {
    const half_t* xst = xs + (size_t)st * kStageHalves;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half8_t af[MBW];
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) {
        const int row = wm * MBW * 16 + mb * 16 + c16;
        const int slot = (j * 4 + t4) ^ (row % 16);
        af[mb] = *reinterpret_cast<const half8_t*>(xst + (size_t)row * kKt + slot * 8);
      }
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        if (!has(nb)) continue;
        const half8_t bf = G ? decode_w4(w_[nb][j]) * sg[nb] : decode_w4(w_[nb][j]);
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) acc[mb][nb] = mfma16x16x32(af[mb], bf, acc[mb][nb]);
      }
    }
  };
  const bool b_pref = PREF && a.ec && a.N % 8 == 0 && (reinterpret_cast<uintptr_t>(a.B) & 15) == 0;
  float* gs_pre = reinterpret_cast<float*>(epi + ec_gs_offset<TM, TN>());
  int p_stage = 0;                             // the X stage that holds the copied P (b_pref, split variant)
  if (NSTAGE == 2) {
    // Two stages, loads one step ahead (the 256-row tiles: two X stages fill
    // the LDS).
    u32x4_t wcur[NBW], wnext[NBW];
    half_t scur[NBW], snext[NBW];
    issue_x(kc_begin, 0);
    load_w(kc_begin, wcur);
    if (G) load_s(kc_begin, scur);
    for (int kc = kc_begin; kc < kc_end; ++kc) {
      const int st = (kc - kc_begin) & 1;
      wait_vm_all();
      __syncthreads();
      if (kc + 1 < kc_end) {
        issue_x(kc + 1, st ^ 1);
        load_w(kc + 1, wnext);
        if (G) load_s(kc + 1, snext);
      } else if (b_pref) {
        p_stage = st ^ 1;
        copy_b_chunk<TN, THREADS>(a, 0, n_tile * TN, epi);
        // The split variant's P and g' (an earlier launch): P into the X
        // stage this step does not read, g' into gs.
        if (!FUSED) copy_ec_rows<TM, THREADS>(a, m0, lds + (size_t)(st ^ 1) * kStageHalves * 2, gs_pre);
      }
      compute(st, wcur, scur);
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        wcur[nb] = wnext[nb];
        if (G) scur[nb] = snext[nb];
      }
    }
  } else {
    // Three stages, loads two steps ahead; the packed weights go through LDS
    // too (ws[stage][panel][64 lanes][16 bytes], after the X stages), so no
    // register holds a load in flight and the only waits are the explicit
    // ones.  Each step issues L copies per wave; at the top of step i those
    // of step i + 1 may still be in flight, those of step i must have landed.
    // Past the last step the copies repeat the last chunk into a stage
    // nothing reads again, so every step issues the same L copies.
    constexpr int kPanels = NBW * WN;                       // per workgroup
    constexpr int kWCopies = (kPanels + NW - 1) / NW;       // per wave
    // G: one 4-byte copy per lane (lanes 0..31: the wave's 64 group scales,
    // its NBW panels, from the row of chunk kc, N padded to 16) into its own
    // 256-byte slot per stage, ssm[stage][wave][128 halves].
    static_assert(!G || NSTAGE != 3 || NBW * 16 == kWave, "one scale copy per wave");
    constexpr int L = kCopiesPerWave + kWCopies + (G ? 1 : 0);
    unsigned char* wsm = lds + (size_t)NSTAGE * kStageHalves * 2;
    half_t* ssm = reinterpret_cast<half_t*>(wsm + (size_t)NSTAGE * ((kPanels + 3) / 4 * 4) * 1024);
    const int pan0 = n_tile * kPanels;
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.scales, (uint32_t)((size_t)a.KC * a.NBLK * 32));
    auto issue_s = [&](int kc, int st) {
      if (G) {
        const uint32_t voff = lane < kWave / 2 ? (uint32_t)nb_base * 32u + (uint32_t)lane * 4u : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_void_t*)(ssm + ((size_t)st * (WM * WN) + w) * 2 * kWave), 4,
                                                 voff, kc * a.NBLK * 32, 0, 0);
      }
    };
    auto issue_w = [&](int kc, int st) {
#pragma unroll
      for (int c = 0; c < kWCopies; ++c) {
        const int pl = min(w * kWCopies + c, kPanels - 1);   // extra copies repeat the last panel
        const uint32_t voff = ((uint32_t)min(pan0 + pl, a.NBLK - 1) * (uint32_t)a.KC * 64u + (uint32_t)lane) * 16u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wr, (lds_void_t*)(wsm + ((size_t)st * kPanels + pl) * 1024), 16, voff, kc * 1024, 0, 0);
      }
    };
    const int nsteps = kc_end - kc_begin;
    issue_x(kc_begin, 0);
    issue_w(kc_begin, 0);
    issue_s(kc_begin, 0);
    {
      const int k1 = min(kc_begin + 1, kc_end - 1);
      issue_x(k1, 1);
      issue_w(k1, 1);
      issue_s(k1, 1);
    }
    for (int i = 0; i < nsteps; ++i) {
      const int st = i % 3;
      // This wave's copies of step i have landed; after the barrier every
      // wave's have.  A plain barrier: the release fence of __syncthreads
      // would also wait for step i + 1's copies.  The stage refilled below
      // was last read in step i - 1, whose reads every wave has completed
      // (their results fed its matrix instructions) before arriving here.
      wait_vm_le<L>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const int kn = min(kc_begin + i + 2, kc_end - 1);
      issue_x(kn, (i + 2) % 3);
      issue_w(kn, (i + 2) % 3);
      issue_s(kn, (i + 2) % 3);
      u32x4_t wv[NBW];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
        wv[nb] = *reinterpret_cast<const u32x4_t*>(wsm + (((size_t)st * kPanels + wn * NBW + nb) * 64 + lane) * 16);
      half_t sv[NBW];
      if (G) {
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) sv[nb] = ssm[((size_t)st * (WM * WN) + w) * 2 * kWave + nb * 16 + c16];
      }
      compute(st, wv, sv);
    }
    wait_vm_all();   // the repeated copies land before the LDS is reused
  }

  // ---------------------------------------------------------------- split K
  if (SPLIT && a.S > 1) {
    __shared__ uint32_t ticket;
    const int tile = m_tile * a.NT + n_tile;
    const uint32_t slice = (uint32_t)MBW * NBW * THREADS * 16;   // bytes of one partial
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.part, (uint32_t)((size_t)tiles * a.S * slice));
    const uint32_t own = (uint32_t)(tile * a.S + split) * slice;
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[mb][nb]), pr,
                                               own + (uint32_t)((mb * NBW + nb) * THREADS + tid) * 16u, 0,
                                               kCachePolicySc1);
    drain_vm();
    __syncthreads();
    if (tid == 0) ticket = add_dev_u32(&a.tickets[tile], 1u);
    __syncthreads();
    if (ticket != (uint32_t)(a.S - 1)) return;
    if (tid == 0) st_dev_u32(&a.tickets[tile], 0u);
    // Fixed order: every partial, this workgroup's own included, from memory.
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = zero_float4();
    // SB splits per batch, all their loads in flight together (about 32 per
    // thread): one memory round trip per batch.
    constexpr int SB = MBW * NBW >= 32 ? 1 : 32 / (MBW * NBW);
    for (int sp0 = 0; sp0 < a.S; sp0 += SB) {
      float4_t v[SB][MBW][NBW];
#pragma unroll
      for (int q = 0; q < SB; ++q) {
        const bool in = sp0 + q < a.S;
        const uint32_t base = (uint32_t)(tile * a.S + sp0 + q) * slice;
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb)
            v[q][mb][nb] = buffer_load_f4_dev(
                pr, in ? base + (uint32_t)((mb * NBW + nb) * THREADS + tid) * 16u : kOutOfRange);
      }
#pragma unroll
      for (int q = 0; q < SB; ++q)
        if (sp0 + q < a.S) {
#pragma unroll
          for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] += v[q][mb][nb];
        }
    }
  }

  // ---------------------------------------------------------------- epilogue
  // acc <- s acc, then the EC term accumulates onto it on the matrix cores,
  // 64 rank columns at a time.  For each chunk the LDS (free once every wave
  // is done with the X stages) holds the B rows bs[64][TN] (dword slots, fp16
  // in the low half; rows >= rank clamped: they meet zero P columns) and
  // pg[TM][64] = fp16(g' P) of the tile's rows (rows >= M clamped: never
  // stored), after gs[TM], the tile's gates.
  if (!G) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      if (!has(nb)) continue;
      const float s = (float)a.scales[min((nb_base + nb) * 16 + c16, a.N - 1)];
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) acc[mb][nb] *= s;
    }
  }
  const int jblocks = a.ec ? a.ps / 32 : 0;
  const half_t* bs = reinterpret_cast<const half_t*>(epi);
  const half_t* pg = reinterpret_cast<const half_t*>(epi + ec_pg_offset<TN>());
  float* gs = reinterpret_cast<float*>(epi + ec_gs_offset<TM, TN>());
  bool any_gate = false;
  if (jblocks > 0) {
    ec_prepare<TM, FUSED>(a, m0, tag, gs, early, b_pref && !FUSED);
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) any_gate |= gs[wm * MBW * 16 + mb * 16 + c16] != 0.0f;
    any_gate = __any(any_gate);
  }
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.P, (uint32_t)((size_t)a.M * a.ps * 4));
  const int n0 = n_tile * TN;
  for (int j0 = 0; j0 < jblocks * 32; j0 += kEcChunk) {
    ec_stage_chunk<TM, TN, FUSED, THREADS>(a, j0, m0, n0, epi, pr, b_pref && j0 == 0,
                                           b_pref && !FUSED && j0 == 0 ? lds + (size_t)p_stage * kStageHalves * 2
                                                                       : nullptr);
    if (any_gate) {
      const int jbn = min(kEcChunk, jblocks * 32 - j0) / 32;
      for (int jb = 0; jb < jbn; ++jb) {
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          if (!has(nb)) continue;
          // B operand rows jb*32 + 8 t4 .. + 7 of column (pan0 + nb) 16 + c16.
          const half8_t bb = lds_b_fragment_tr(bs + (size_t)jb * 32 * TN + (pan0 + nb) * 16, TN, lane);
#pragma unroll
          for (int mb = 0; mb < MBW; ++mb) {
            const int r = wm * MBW * 16 + mb * 16 + c16;
            const half8_t pa = *reinterpret_cast<const half8_t*>(pg + (size_t)r * kEcChunk + jb * 32 + t4 * 8);
            acc[mb][nb] = mfma16x16x32(pa, bb, acc[mb][nb]);
          }
        }
      }
    }
  }

  // ---- Y through LDS: each wave writes its fp16 results into ys[TM][YS],
  // then the workgroup stores whole rows, 16 bytes per thread and store when
  // Y rows are 16-byte aligned (N % 8 == 0), else element by element along
  // the rows.
  constexpr int YS = TN + 8;                   // row stride (halves), off the bank period
  half_t* ys = reinterpret_cast<half_t*>(lds);
  __syncthreads();                             // every wave is done with the epilogue LDS
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    if (!has(nb)) continue;
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        ys[(wm * MBW * 16 + mb * 16 + 4 * t4 + v) * YS + (pan0 + nb) * 16 + c16] = (half_t)acc[mb][nb][v];
  }
  __syncthreads();
  const int rows = min(TM, a.M - m0);
  if (a.N % 8 == 0 && (reinterpret_cast<uintptr_t>(a.Y) & 15) == 0) {
    const int cols8 = min(TN, a.N - n0) / 8;
    for (int idx = tid; idx < rows * (TN / 8); idx += THREADS) {
      const int r = idx / (TN / 8), c8 = idx % (TN / 8);
      if (c8 < cols8)
        *reinterpret_cast<u32x4_t*>(a.Y + (size_t)(m0 + r) * a.N + n0 + c8 * 8) =
            *reinterpret_cast<const u32x4_t*>(ys + r * YS + c8 * 8);
    }
  } else {
    const int cols = min(TN, a.N - n0);
    for (int idx = tid; idx < rows * TN; idx += THREADS) {
      const int r = idx / TN, c = idx % TN;
      if (c < cols) a.Y[(size_t)(m0 + r) * a.N + n0 + c] = ys[r * YS + c];
    }
  }
}

template <int TM, int TN, bool SPLIT>
constexpr size_t lds_bytes_for() {
  // X stages, and with three stages the packed-weight stages (TN / 16 panels
  // of 1 KiB each, one copy per wave at least); the epilogue's B chunk, g' P
  // and gates overlay them, or follow them (epilogue_after_stages).
  constexpr int NS = stages_for(TM, SPLIT);
  constexpr size_t w_stages = NS == 3 ? (size_t)3 * ((TN / 16 + 3) / 4 * 4) * 1024 + (size_t)3 * 4 * kWave * 4 : 0;
  constexpr size_t stages = (size_t)NS * TM * kKt * 2 + w_stages;
  constexpr size_t epilogue =
      epilogue_after_stages(TM, SPLIT)
          ? stages + (size_t)kEcChunk * TN * 2 + (size_t)TM * kEcChunk * 2 + (size_t)TM * 4
          : (size_t)kEcChunk * TN * 2 + (size_t)TM * kEcChunk * 2 + (size_t)TM * 4;
  constexpr size_t y_tile = (size_t)TM * (TN + 8) * 2;
  constexpr size_t m = stages > epilogue ? stages : epilogue;
  return m > y_tile ? m : y_tile;
}

// Waves per SIMD a kernel is built for: two for the 128-row mid-size tiles
// (128 x 256 with a K split), so that two workgroups share a CU (256
// registers per wave, under 80 KiB of LDS each) and, in the fused launch, the
// leading EC workgroups do not keep GEMM workgroups off the CUs they hold
// (mixed-gate down_proj M = 512, K = 14336, N = 4096, fused: 84-88 -> 71-78
// us; M = 1024, K = N = 4096: 50-55 -> 45 us; EC off unchanged).
constexpr int waves_per_simd(int tm, bool split) { return split && tm == 128 ? 2 : 1; }

template <int MBW, int NBW, int WM, int WN, bool SPLIT, bool G, int TP>
__global__ void __launch_bounds__(WM * WN * kWave, waves_per_simd(16 * MBW * WM, SPLIT))
    w4_gemm_tiled_kernel(GemmKArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  gemm_block<MBW, NBW, WM, WN, SPLIT, false, G, TP>(a, blockIdx.x, lds, 0u);
}

// Fused tiled launch: blocks [0, E) are EC workgroups (the first ec_blocks
// of them real, the rest padding so that the GEMM blocks keep their XCD
// order), the others GEMM tiles.  EC workgroups have the lowest block
// indices, so they are dispatched before any GEMM workgroup and never wait
// for one; a GEMM workgroup waits only in its epilogue, for ready flags that
// the EC workgroups raise.  Every block reads the call epoch first and counts
// itself out last (count_out: the last to finish returns the finisher count
// to zero and advances the epoch; every block has read it by then).
template <int MBW, int NBW, int WM, int WN, bool SPLIT, int PB, bool G>
__global__ void __launch_bounds__(kGemmThreads, waves_per_simd(16 * MBW * WM, SPLIT))
    w4_gemm_fused_kernel(FusedKArgs f) {
  extern __shared__ __align__(16) unsigned char lds[];
  const uint32_t tag = call_tag(f.sync);
  const int b = blockIdx.x;
  if (b < f.E) {
    if (b < f.ec_blocks) ec_block<true, true, PB>(f.e, lds, b % f.e.m_tiles, b / f.e.m_tiles, tag);
  } else {
    gemm_block<MBW, NBW, WM, WN, SPLIT, true, G>(f.g, b - f.E, lds, tag);
  }
  __syncthreads();
  if (threadIdx.x < kWave) count_out(f.sync, gridDim.x, tag);
}

template <int MBW, int NBW, int WM, int WN, bool SPLIT, bool G, int TP = 0>
hipError_t launch_cfg(const GemmKArgs& k, void* stream) {
  constexpr size_t lds =
      lds_bytes_for<16 * MBW * WM, 16 * (TP ? TP : NBW * WN), SPLIT>();
  const hipError_t attr = set_max_dynamic_lds(
      reinterpret_cast<const void*>(&w4_gemm_tiled_kernel<MBW, NBW, WM, WN, SPLIT, G, TP>), (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((w4_gemm_tiled_kernel<MBW, NBW, WM, WN, SPLIT, G, TP>), dim3((unsigned)(k.MT * k.NT * k.S)),
                     dim3(WM * WN * kWave), lds, (hipStream_t)stream, k);
  return hipGetLastError();
}

template <int MBW, int NBW, int WM, int WN, bool SPLIT, int PB, bool G>
hipError_t launch_fused_pb(const FusedKArgs& f, void* stream) {
  const size_t tile = lds_bytes_for<16 * MBW * WM, 16 * NBW * WN, SPLIT>();
  const size_t ec = ec_lds_bytes(f.e.ss, f.e.rp);
  const size_t lds = tile > ec ? tile : ec;
  if (ec_kb_for(PB) * 32 != f.e.ss || lds > kMaxLdsBytes - 1024) return hipErrorInvalidValue;
  const hipError_t attr = set_max_dynamic_lds(
      reinterpret_cast<const void*>(&w4_gemm_fused_kernel<MBW, NBW, WM, WN, SPLIT, PB, G>), (int)(kMaxLdsBytes - 1024));
  if (attr != hipSuccess) return attr;
  const unsigned grid = (unsigned)(f.E + f.g.MT * f.g.NT * f.g.S);
  hipLaunchKernelGGL((w4_gemm_fused_kernel<MBW, NBW, WM, WN, SPLIT, PB, G>), dim3(grid), dim3(kGemmThreads), lds,
                     (hipStream_t)stream, f);
  return hipGetLastError();
}

template <int MBW, int NBW, int WM, int WN, bool SPLIT, bool G>
hipError_t launch_fused(const FusedKArgs& f, void* stream) {
  switch (ec_pb_for(f.e.rank)) {
    case 1: return launch_fused_pb<MBW, NBW, WM, WN, SPLIT, 1, G>(f, stream);
    case 2: return launch_fused_pb<MBW, NBW, WM, WN, SPLIT, 2, G>(f, stream);
    case 4: return launch_fused_pb<MBW, NBW, WM, WN, SPLIT, 4, G>(f, stream);
    case 8: return launch_fused_pb<MBW, NBW, WM, WN, SPLIT, 8, G>(f, stream);
    default: return launch_fused_pb<MBW, NBW, WM, WN, SPLIT, 16, G>(f, stream);
  }
}

template <bool G>
hipError_t launch_tiles(const GemmKArgs& k, const FusedKArgs* f, const TiledShape& t, void* stream) {
  if (f) {
    if (t.tn == 448) return launch_fused<8, 7, 1, 4, false, G>(*f, stream);
    if (t.tm == 256 && t.tn == 224) return launch_fused<8, 7, 2, 2, false, G>(*f, stream);
    if (t.tm == 256) return launch_fused<8, 8, 2, 2, false, G>(*f, stream);
    if (t.tm == 128) return launch_fused<8, 4, 1, 4, true, G>(*f, stream);
    return launch_fused<2, 4, 2, 2, true, G>(*f, stream);
  }
  // The large tiles never split; the mid-size tiles are built with the split
  // path, which they skip when S is 1.
  if (t.tn == 448) return launch_cfg<8, 4, 1, 8, false, G, 28>(k, stream);
  if (t.tm == 256 && t.tn == 224) return launch_cfg<8, 7, 2, 2, false, G>(k, stream);
  if (t.tm == 256) return launch_cfg<8, 8, 2, 2, false, G>(k, stream);
  if (t.tm == 128) return launch_cfg<8, 4, 1, 4, true, G>(k, stream);
  return launch_cfg<2, 4, 2, 2, true, G>(k, stream);
}

}  // namespace

TiledShape tiled_shape(int64_t M, int64_t K, int64_t N, int cus, size_t scratch_base) {
  // Large M: 128 x 448 tiles (four waves side by side, each 128 x 112) when
  // N fills whole 448-column tiles, else 256-row tiles (224 columns when that
  // gives whole waves of 256 tiles), no split.  The 128 x 448 tile has the
  // same wave tile as the 256 x 224 one but copies half the X bytes per step
  // and decodes each packed word once per workgroup instead of twice
  // (prefill 2048 x 4096 x 14336, EC off: 186-188 us vs 204-205 us).
  // Mid-size M, where those tiles would not fill the GPU:
  // 128 x 256 tiles (M > 256; four waves of 128 x 64 side by side) or
  // 64 x 128 tiles, with K split so that about one workgroup per CU runs,
  // each split at least four 128-k chunks.  (At M = 256 the 64-row tiles need
  // no K split where 128-row ones need two: measured 12-22 % faster there,
  // 25 % slower at M = 512 with K = 14336.  The 128 x 256 tiles replaced
  // 2 x 2 waves of 64 x 64 on 128 x 128: EC off 71-73 -> 60-61 us at M = 512,
  // K = 14336, N = 4096, fused 92-99 -> 83-84; 64 x 256 tiles for M <= 256
  // measured slower than 64 x 128, 15.0 -> 17.6 us at 256 x 2048 x 2048.)
  TiledShape t;
  const int64_t nblk = n_pad(N) / 16, KC = k_pad(K) / kKChunk;
  if (nblk % 28 == 0) {
    t.tm = 128;
    t.tn = 448;
  } else {
    t.tm = 256;
    t.tn = (nblk % 14 == 0 && nblk >= 14) ? 224 : 256;
  }
  int64_t tiles = ceil_div(M, t.tm) * ceil_div(nblk, t.tn / 16);
  if (tiles < (int64_t)cus * 3 / 4) {
    t.tm = M > 256 ? 128 : 64;
    t.tn = t.tm == 128 ? 256 : 128;
    tiles = ceil_div(M, t.tm) * ceil_div(nblk, t.tn / 16);
    int64_t S = cus / tiles;
    const int64_t max_s = std::max<int64_t>(1, std::min<int64_t>(KC / 4, t.tm == 64 ? 16 : 8));
    S = std::max<int64_t>(1, std::min(S, max_s));
    t.cps = (int)ceil_div(KC, S);
    t.split = (int)ceil_div(KC, t.cps);
  } else {
    t.split = 1;
    t.cps = (int)KC;
  }
  // One launch's workgroup count (and the planner's sums over it) stays
  // within 2^30.
  if (ceil_div(M, t.tm) * ceil_div(nblk, t.tn / 16) * t.split > (int64_t)1 << 30) {
    t.fits = false;
    return t;
  }
  t.mt = (int)ceil_div(M, t.tm);
  t.nt = (int)ceil_div(nblk, t.tn / 16);
  t.grid = t.mt * t.nt * t.split;
  if (t.split > 1) {
    t.ws_part = (size_t)round_up((int64_t)scratch_base, 256);
    t.ws_bytes = t.ws_part + (size_t)t.mt * t.nt * t.split * t.tm * t.tn * 4;
    t.fits = (int64_t)t.mt * t.nt <= kMaxSyncWords - 128;
  }
  return t;
}

TiledShape fused_tiled_shape(int64_t M, int64_t K, int64_t N, int cus, int ec_blocks, size_t scratch_base) {
  const int left = cus - ec_blocks > cus / 2 ? cus - ec_blocks : cus / 2;
  const TiledShape t = tiled_shape(M, K, N, left, scratch_base);
  if ((int64_t)t.grid * 3 >= (int64_t)cus * 2) return t;
  return tiled_shape(M, K, N, cus, scratch_base);
}

hipError_t launch_gemm(const GemmArgs& a, const spear_plan_t& plan, void* stream) {
  const EcWorkspace ecl = a.fused ? ec_workspace_layout(a.M, a.K, a.rank, kEcBlocksFused) : EcWorkspace{};
  const int ec_blocks = a.fused ? (int)round_up(ecl.m_tiles * ecl.splits, 8) : 0;
  const TiledShape t = a.fused ? fused_tiled_shape(a.M, a.K, a.N, plan.cus, ec_blocks, a.scratch_base)
                               : tiled_shape(a.M, a.K, a.N, plan.cus, a.scratch_base);
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
  k.MT = t.mt; k.NT = t.nt;
  k.S = t.split; k.CPS = t.cps;
  k.part = t.split > 1 ? (float*)((char*)a.workspace + t.ws_part) : nullptr;
  uint32_t* sync = (uint32_t*)((char*)a.workspace + kGemmSyncOffset);
  k.tickets = t.split > 1 ? sync + kSyncTiles : nullptr;
  k.ready = nullptr;
  k.ec_tiles = 0;
  k.error = sync + kSyncError;
  k.spin_limit = a.spin_limit;
  k.wait_xor = a.wait_xor;
  if (a.fused) {
    // EC workgroups first (P and g into the EC workspace, ready flags in the
    // EC counter region), then the GEMM tiles.
    const EcWorkspace& L = ecl;
    FusedKArgs f;
    f.e = make_ec_kargs(a.ecargs, L);
    f.e.ready = (uint32_t*)a.workspace + kEcReadyWord;
    f.ec_blocks = L.m_tiles * L.splits;
    f.E = (int)round_up(f.ec_blocks, 8);
    f.sync = sync;
    k.P = f.e.P_out;
    k.g = f.e.g_out;
    k.ready = f.e.ready;
    k.ec_tiles = L.m_tiles;
    f.g = k;
    return a.grouped ? launch_tiles<true>(k, &f, t, stream) : launch_tiles<false>(k, &f, t, stream);
  }
  return a.grouped ? launch_tiles<true>(k, nullptr, t, stream) : launch_tiles<false>(k, nullptr, t, stream);
}

}  // namespace spear
