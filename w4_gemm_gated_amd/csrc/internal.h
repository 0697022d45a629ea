// Internal interfaces between the C ABI (api.cpp), the host planner
// (plan.cpp) and the kernel launchers (*.hip).  Not installed; not part of
// the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "../../include/spear_w4ec.h"

namespace spear {

// ----------------------------------------------------------------- geometry

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

inline int64_t k_pad(int64_t K) { return round_up(K, 128); }
inline int64_t n_pad(int64_t N) { return round_up(N, 16); }

// Columns of the EC projection output: rank columns of P, one of the gate
// logit, padded to the 16-column granule of the matrix instruction.
inline int64_t ec_cols(int64_t rank) { return round_up(rank + 1, 16); }
// Row stride (floats) of the stored P: rank padded to the 32-k granule.
inline int64_t p_stride(int64_t rank) { return round_up(rank, 32); }

// Every workspace starts with a fixed 256 KiB header: cross-workgroup
// counters of the EC projection in [0, 32 KiB) and of the GEMM kernels in
// [32 KiB, 64 KiB), which every call returns to zero (except the GEMM call
// epoch, which every fused call advances), and the fused variant's hand-off
// slabs in [64 KiB, 1 MiB), whose entries carry the epoch of the call that
// wrote them (room for the producers' entries of rank 64 up to K = 16384 at
// 16 rows).  All scratch lies after the header, so a zero-filled workspace
// serves calls of any plan (each plan's counters and hand-off sit in the
// header, never in another plan's scratch).
constexpr size_t kSyncHeaderBytes = 1024 * 1024;
constexpr size_t kGemmSyncOffset = 32 * 1024;
constexpr size_t kHandoffOffset = 64 * 1024;
constexpr size_t kHandoffBytes = 960 * 1024;
constexpr int64_t kMaxSyncWords = 8192;   // per counter region
// Words of the GEMM counter region ([32 KiB, 64 KiB)), each hot one on its own
// 128-byte line: fused finisher count, error flag, call epoch (advanced by
// every fused call), then split-K tile counters.
constexpr int kSyncFinishers = 32, kSyncError = 64, kSyncEpoch = 96, kSyncTiles = 128;
// Bits of the sticky error word (kSyncError): a bounded wait gave up, so the
// call that set it wrote a wrong Y.  spear_take_error reads and clears it.
constexpr uint32_t kErrHandoffWait = 1u;   // fused decode: the producers' hand-off
constexpr uint32_t kErrReadyWait = 2u;     // fused tiled: an EC row tile's ready flag
// Default bound of every cross-workgroup wait, in polls (about half a second:
// far beyond any healthy wait).
constexpr uint32_t kDefaultSpinLimit = 1u << 20;
// EC counter region ([0, 32 KiB)): row-tile counters in words [0, 4096), the
// fused tiled launch's ready flags (raised to the call's epoch + 1) in words
// [4096, 8192).
constexpr int kEcReadyWord = 4096;
constexpr int64_t kMaxEcTiles = 4096;

// Workspace layout of the EC projection (offsets in bytes, 256-aligned).
struct EcWorkspace {
  int32_t m_tiles = 0;   // row tiles of the projection
  int32_t tile_rows = 0; // rows per tile (16 or 64)
  int32_t splits = 0;    // K slices
  int32_t k_slice = 0;   // k per slice (multiple of the sub-slab)
  int32_t ss = 0;        // k per sub-slab (256, 128 or 64 by rank)
  size_t counters = 0;   // uint32 [m_tiles]
  size_t partials = 0;   // float [splits][m_tiles * tile_rows][ec_cols]
  size_t p = 0;          // float [M][p_stride]
  size_t g = 0;          // float [M]
  size_t bytes = 0;
};
// target_blocks: about how many workgroups the K slices should give (the
// split variant's own launch spreads the read of X over the GPU; the fused
// tiled launch, whose EC workgroups each hold a CU the GEMM tiles wait for,
// takes fewer: 128 shorter ones delay the tiles less than 64 longer ones,
// measured 240 -> 230 us at M = 2048, K = 4096, N = 14336, rank 64; 256 gave
// 235 us).
constexpr int kEcBlocksSplit = 256, kEcBlocksFused = 128;
EcWorkspace ec_workspace_layout(int64_t M, int64_t K, int64_t rank, int target_blocks = kEcBlocksSplit);

// Host planner (pure host code; no HIP calls).
spear_status_t make_plan(const spear_linear_desc_t& d, int cus, spear_plan_t* plan);
spear_status_t check_desc(const spear_linear_desc_t& d);
// The plan a call runs: `plan` checked against the descriptor (re-planned
// and compared), or planned here when it is NULL.  No device work.
spear_status_t resolve_plan(const spear_linear_desc_t& desc, const spear_plan_t* plan, spear_plan_t* out);

// Shapes of the main kernel families.
constexpr int kSkinnyMaxM = 16;   // rows handled by the skinny kernel
constexpr size_t kMaxLdsBytes = 160 * 1024;   // LDS of one gfx950 workgroup

// ----------------------------------------------------------------- launchers

struct EcArgs {
  const void* X;      // fp16 [M, K]
  const void* A;      // fp16 [K, rank]
  const void* w_g;    // fp16 [K]
  int32_t M, K, rank;
  float gate_bias, skip_tau;
  void* workspace;    // base; layout from ec_workspace_layout
  void* P_out;        // float [M][p_stride] (may alias workspace P)
  void* g_out;        // float [M]
  int32_t p_out_stride;  // floats per row of P_out
};

struct GemmArgs {
  const void* X;       // fp16 [M, K]
  const void* Wq;      // packed, layout id 2
  const void* scales;  // fp16 [N]
  const void* B;       // fp16 [rank, N] (EC) or null
  const float* P;      // float [M][p_stride] or null
  const float* g;      // float [M] or null
  void* Y;             // fp16 [M, N]
  int32_t M, K, N, rank;
  int32_t ec;          // apply the gated EC term
  void* workspace;     // base (split partials and tile counters), may be null without splits
  size_t scratch_base; // first workspace byte the GEMM may use as scratch
  int32_t fused;       // P and g computed by EC workgroups of the same launch
  EcArgs ecargs;       // fused: the projection's arguments (P and g in the EC workspace)
  uint32_t spin_limit; // polls before a cross-workgroup wait gives up
  uint32_t wait_xor;   // 0; nonzero (test hook) makes every wait look for a tag nobody writes
  int32_t grouped;     // scales fp16 [KC][N], one per 128-k chunk and column (else [N])
};

// Skinny (M <= 16) kernel: tile shape, producers and workspace layout.
struct SkinnyShape {
  int nbw = 1;      // 16-column panels per workgroup
  int S = 1;        // K splits across workgroups
  int T = 0;        // column tiles
  int CPS = 0;      // 128-k chunks per split
  int CPW = 1;      // chunks per wave (<= 4)
  bool local_ec = false;  // fused: every GEMM workgroup computes the projection itself
  int P = 0;        // EC producer workgroups (fused variant, hand-off)
  int ksp = 0;      // k per producer slab
  size_t lds = 0;   // dynamic LDS of a producer
  size_t lds_gemm = 0;  // dynamic LDS of a GEMM workgroup (EC factor tile)
  size_t ws_sync = 0, ws_handoff = 0, ws_gemm_part = 0;
  size_t ws_bytes = 0;   // total workspace (0: none needed)
  bool fits = true;      // counters and hand-off fit the header, LDS fits
};
// scratch_base: first byte of the workspace this kernel may use as scratch.
SkinnyShape skinny_shape(int64_t M, int64_t K, int64_t N, int64_t rank, bool fused, int cus,
                         size_t scratch_base);

struct SkinnyLaunch {
  SkinnyShape shape;
  const void* X;
  const void* Wq;
  const void* scales;
  const void* A;
  const void* B;
  const void* w_g;
  void* Y;
  int32_t M, K, N, rank;
  int32_t ec_mode;          // 0 none, 1 fused (hand-off or local, per shape), 2 P/g given
  float gate_bias, skip_tau;
  void* workspace;          // skinny workspace (layout in shape)
  const float* Pext;        // ec_mode 2
  const float* gext;
  uint32_t spin_limit;      // polls before a cross-workgroup wait gives up
  uint32_t wait_xor;        // 0; nonzero (test hook) makes every wait look for a tag nobody writes
  int32_t grouped;          // scales fp16 [KC][N], one per 128-k chunk and column (else [N])
};
hipError_t launch_skinny(const SkinnyLaunch& L, void* stream);

// Tiled (M > 16) kernel: tile shape and grid.
struct TiledShape {
  int tm = 256, tn = 256;   // tile rows and columns
  int mt = 0, nt = 0;       // row and column tiles
  int split = 1;            // K splits (partial sums added by the last to arrive)
  int cps = 0;              // 128-k chunks per split
  int grid = 0;
  size_t ws_part = 0;       // split partials (bytes from the workspace base)
  size_t ws_bytes = 0;      // workspace this kernel needs (0: none)
  bool fits = true;         // tile counters fit the counter header
};
// scratch_base: first byte of the workspace this kernel may use as scratch.
TiledShape tiled_shape(int64_t M, int64_t K, int64_t N, int cus, size_t scratch_base);
// The tiles of a fused tiled launch, whose ec_blocks EC workgroups lead the
// grid and hold their CUs: the K split is planned for the CUs they leave free
// (else a second wave of tiles waits for a free CU), unless the tiles would
// then cover less than two thirds of the GPU.
TiledShape fused_tiled_shape(int64_t M, int64_t K, int64_t N, int cus, int ec_blocks, size_t scratch_base);

// The allocation-free entry point's workspace: a file-scope device array of
// this size (noalloc.hip), one per GPU; static_scratch returns the current
// device's address, setting it up on first use (its header zeroed on `stream`).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
hipError_t static_scratch(void** out, void* stream);

// Raise a kernel's dynamic-LDS limit on the current device (once per kernel
// and device; later calls return at once).
hipError_t set_max_dynamic_lds(const void* kernel, int bytes);
hipError_t launch_take_error(void* workspace, void* out, void* stream);
hipError_t launch_stream_read(const void* src, size_t bytes, int grid, void* sink, void* stream);
hipError_t launch_mfma_rate(int shape, int waves_per_simd, int iterations, int grid, void* sink, void* stream);
// Data-free EC initialisation (ec_init.hip): workspace layout (byte offsets)
// and launch arguments.
struct EcInitLayout {
  int l = 0;            // columns of the subspace iteration (rank + 16, even, <= 128)
  size_t E = 0, Y = 0, Y2 = 0, V = 0, part = 0, G = 0, T = 0, T2 = 0, evals = 0, A32 = 0, Bt32 = 0, sign = 0;
  size_t bytes = 0;
  bool fits = false;    // rank within what the eigen-solver's LDS holds
};
EcInitLayout ec_init_layout(int64_t K, int64_t N, int64_t rank);
struct EcInitArgs {
  const void* W;        // fp16 [K, N]
  const void* Wq;       // packed codes (layout id 2)
  const void* scales;   // per channel [N] or group [KC][N_pad]
  int32_t K, N, rank, grouped, iterations;
  void* A;              // fp16 [K, rank]
  void* B;              // fp16 [rank, N]
  void* workspace;
  EcInitLayout layout;
};
hipError_t launch_ec_init(const EcInitArgs& a, void* stream);

hipError_t launch_pack_w4(const void* W, int32_t K, int32_t N, void* Wq, void* scales, void* stream);
hipError_t launch_pack_w4_grouped(const void* W, int32_t K, int32_t N, void* Wq, void* scales, void* stream);
hipError_t launch_unpack_w4(const void* Wq, int32_t K, int32_t N, void* q_out, void* stream);
hipError_t launch_ec_project(const EcArgs& a, void* stream);
hipError_t launch_gemm(const GemmArgs& a, const spear_plan_t& plan, void* stream);

}  // namespace spear
