// Host planner: the per-call choice of fusion variant (SPEAR page, abstract),
// reduced to what one GPU needs.  Pure host arithmetic on the descriptor; the
// device is touched only by the caller (api.cpp) to read the CU count.
//
// Decisions:
//   * no EC (rank 0) or variant NO_EC            -> NO_EC: the W4 GEMM alone;
//   * AUTO and rank % 4 == 0                     -> FUSED: one launch (EC
//     workgroups first, then the W4 GEMM with the gated epilogue, which
//     waits for the EC results it needs; at M <= 16 the EC computed by every
//     GEMM workgroup itself when A is small), except on the 128 x 448 tiles,
//     where the measured crossover favours SPLIT;
//   * AUTO otherwise (rank % 4 != 0)             -> SPLIT (EC projection
//     launch, then the W4 GEMM with the gated epilogue);
//   * the per-token gate-value decision (skip the EC term where every gate of
//     a wave's rows is below tau) is taken on the device in the epilogue.
//   * main kernel family by M: skinny (M <= 16 rows) or tiled (128 x 448 or
//     256-row tiles; 128 x 256 or 64 x 128 tiles with K split where those
//     would not fill the GPU).
#include <algorithm>
#include <cmath>
#include <cstring>

#include "internal.h"

namespace spear {

spear_status_t check_desc(const spear_linear_desc_t& d) {
  if (d.M < 0 || d.K < 8 || d.K % 8 != 0 || d.N < 1) return SPEAR_ERR_INVALID_SHAPE;
  if (d.rank < 0 || d.rank > SPEAR_MAX_RANK) return SPEAR_ERR_INVALID_SHAPE;
  if (d.variant < SPEAR_VARIANT_AUTO || d.variant > SPEAR_VARIANT_NO_EC) return SPEAR_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(d.gate_bias) || !std::isfinite(d.skip_tau)) return SPEAR_ERR_INVALID_ARGUMENT;
  if (d.skip_tau < 0.0f || d.skip_tau > 1.0f) return SPEAR_ERR_INVALID_ARGUMENT;
  if (d.device_cus < 0) return SPEAR_ERR_INVALID_ARGUMENT;
  if (d.group_size != 0 && d.group_size != SPEAR_GROUP_SIZE) return SPEAR_ERR_UNSUPPORTED;
  // Index arithmetic inside the kernels uses 32-bit row and column counts.
  if ((int64_t)d.K * 8 > INT32_MAX || (int64_t)d.N * 16 > INT32_MAX) return SPEAR_ERR_UNSUPPORTED;
  return SPEAR_OK;
}

// ------------------------------------------------------------ cost model
// Predicted time of a call (microseconds) from its plan: a roofline with
// constants fitted to this library's kernels measured on MI355X (graph replay,
// cold weights):
//   t = launch + max(bytes / stream rate, main flops / matrix rate of the
//       kernel family) + split-K exchange + the variant's EC cost,
// and for the decode kernel also the X rows every column tile re-reads from
// L2 (column tiles x M x K x 2 bytes).
// Tiled kernels: a plain read of B bytes in one launch takes 1.65 us + B / 7.2
// TB/s (8 MiB .. 256 MiB); matrix rates: the 128 x 448 tiles reach 1.28 PF/s on
// the prefill shape, the 256-row tiles 1.13, the 128 x 256 and 64-row tiles
// 1.0 and 0.55 (mid-size M, K split); EC cost of the fused tiles 4 us plus the EC workgroups' read of X
// (1.3 TB/s, partly under the GEMM), of the split variant one more launch plus
// its read of X and its flops.
// Decode kernel (fitted to 120 calls: ten layer shapes, M = 1, 4, 8, 16, the
// three variants; median error 4.5 %, largest 17 %): 2.46 us + bytes / 4.06
// TB/s + X re-reads / 18.95 TB/s, 1.91 us for a K split; hand-off EC 2.04 us +
// 0.063 per producer + 0.131 per thousand entries gathered (producers x rows
// x (rank + 1)) + 0.018 per row; local EC 1.83 us plus every workgroup's read
// of A from L2 (16.8 TB/s); split variant 7.11 us + 4.60 per MiB of A + 0.029
// per row (its projection launch reads A with few workgroups).
namespace {

struct CostConstants {
  double stream_bytes_per_us = 7.2e6, skinny_stream_bytes_per_us = 4.06e6, skinny_x_l2_bytes_per_us = 18.95e6;
  double launch_skinny_us = 2.46, launch_tiled_us = 3.0;
  double mma_skinny = 0.26e9, mma_64 = 0.55e9, mma_128 = 1.0e9, mma_256 = 1.13e9, mma_448 = 1.28e9;   // flop per us
  double split_skinny_us = 1.91, split_tiled_us = 3.0;
  double ec_handoff_us = 2.04, ec_handoff_per_producer_us = 0.063, ec_handoff_per_kentry_us = 0.131,
         ec_handoff_per_row_us = 0.018;
  double ec_local_us = 1.83, l2_bytes_per_us = 16.8e6;
  double ec_fused_tiled_us = 4.0, ec_fused_x_bytes_per_us = 1.3e6;
  double ec_split_launch_us = 3.0, ec_split_x_bytes_per_us = 2.0e6, ec_split_flops_per_us = 0.5e9;
  double ec_split_skinny_us = 7.11, ec_split_skinny_per_a_mib_us = 4.60, ec_split_skinny_per_row_us = 0.029;
};

double predict_call_us(const spear_plan_t& p) {
  const CostConstants c;
  const double M = p.M, K = p.K, N = p.N, r = p.rank;
  const bool ec = p.variant != SPEAR_VARIANT_NO_EC && p.rank > 0;
  const bool skinny = p.kernel == 0;
  const double scale_bytes = p.group_size ? (double)(k_pad(p.K) / 128) * (double)n_pad(p.N) * 2.0 : 2.0 * N;
  double bytes = K * N / 2.0 + scale_bytes + 2.0 * M * K + 2.0 * M * N;
  if (ec) bytes += 2.0 * r * (K + N) + 2.0 * K;
  const double mma_rate = skinny               ? c.mma_skinny
                          : p.tile_n == 448    ? c.mma_448
                          : p.tile_m >= 256    ? c.mma_256
                          : p.tile_m >= 128    ? c.mma_128
                                               : c.mma_64;
  double t = (skinny ? c.launch_skinny_us : c.launch_tiled_us) +
             std::max(bytes / (skinny ? c.skinny_stream_bytes_per_us : c.stream_bytes_per_us),
                      2.0 * M * K * N / mma_rate);
  // Decode: every column tile reads the X rows of its K range, all of X over
  // the tile's splits.
  if (skinny) t += std::ceil((double)n_pad(p.N) / p.tile_n) * M * K * 2.0 / c.skinny_x_l2_bytes_per_us;
  if (p.split_k > 1) t += skinny ? c.split_skinny_us : c.split_tiled_us;
  if (ec) {
    const double ec_flops = 2.0 * M * (K * (r + 1) + r * N);
    if (p.variant == SPEAR_VARIANT_SPLIT && skinny) {
      t += c.ec_split_skinny_us + c.ec_split_skinny_per_a_mib_us * (2.0 * K * r / 1048576.0) +
           c.ec_split_skinny_per_row_us * M;
    } else if (p.variant == SPEAR_VARIANT_SPLIT) {
      t += c.ec_split_launch_us + 2.0 * M * K / c.ec_split_x_bytes_per_us + ec_flops / c.ec_split_flops_per_us;
    } else if (skinny && p.ec_local) {
      t += c.ec_local_us + 2.0 * K * r * (double)p.grid / c.l2_bytes_per_us;
    } else if (skinny) {
      // The producers' chain: their count, the entries every consumer gathers
      // and the rows they carry.
      const double entries = (double)p.producers * M * (double)round_up(p.rank + 1, 2);
      t += c.ec_handoff_us + c.ec_handoff_per_producer_us * p.producers + c.ec_handoff_per_kentry_us * entries / 1000.0 +
           c.ec_handoff_per_row_us * M;
    } else {
      t += c.ec_fused_tiled_us + 2.0 * M * K / c.ec_fused_x_bytes_per_us;
    }
  }
  return t;
}

}  // namespace

spear_status_t make_plan(const spear_linear_desc_t& d, int cus, spear_plan_t* plan) {
  const spear_status_t st = check_desc(d);
  if (st != SPEAR_OK) return st;
  spear_plan_t p;
  std::memset(&p, 0, sizeof(p));
  p.abi_version = SPEAR_ABI_VERSION;
  p.layout_id = SPEAR_LAYOUT_ID;
  p.M = d.M; p.K = d.K; p.N = d.N; p.rank = d.rank;
  p.cus = cus;
  p.group_size = d.group_size;
  const bool skinny = d.M <= kSkinnyMaxM;
  const bool ec = d.rank > 0 && d.variant != SPEAR_VARIANT_NO_EC;
  // The fused EC workgroups copy A rows verbatim (16-byte units) and read it
  // with 8-byte transposing LDS reads: rank % 4 == 0.
  auto fused_ok = [&]() {
    if (d.rank % 4 != 0) return false;
    if (skinny) return skinny_shape(d.M, d.K, d.N, d.rank, true, cus, kSyncHeaderBytes).fits;
    const EcWorkspace L = ec_workspace_layout(d.M, d.K, d.rank, kEcBlocksFused);
    return L.m_tiles <= kMaxEcTiles;
  };
  // Measured crossover (cold weights, 128 EC workgroups): on 128 x 256
  // tiles (M of about 257 to 1024) the fused variant is faster (M = 512,
  // K = 4096, N = 14336: 65 vs 71 us; M = 512, K = 14336, N = 4096: 83-84 vs
  // 85; M = 1024, K = N = 4096: 51 vs 55), as with 64-row (M <= 256) and
  // 256-row tiles.  On 128 x 448 tiles the split variant runs the eight-wave
  // tile kernel, which only the split and EC-off launches have (M = 2048,
  // K = 4096, N = 14336: split 200-213 us vs fused 211-220 over four boxes).
  auto split_wins = [&]() {
    if (skinny) return false;
    const EcWorkspace L = ec_workspace_layout(d.M, d.K, d.rank, kEcBlocksFused);
    const int eb = (int)round_up(L.m_tiles * L.splits, 8);
    const TiledShape t = fused_tiled_shape(d.M, d.K, d.N, cus, eb, kSyncHeaderBytes);
    return t.tn == 448;
  };
  if (!ec) {
    p.variant = SPEAR_VARIANT_NO_EC;
  } else if (d.variant == SPEAR_VARIANT_AUTO) {
    p.variant = fused_ok() && !split_wins() ? SPEAR_VARIANT_FUSED : SPEAR_VARIANT_SPLIT;
  } else {
    p.variant = d.variant;
  }
  if (p.variant == SPEAR_VARIANT_FUSED && !fused_ok()) return SPEAR_ERR_UNSUPPORTED;
  size_t ws = 0;
  size_t scratch_base = kSyncHeaderBytes;
  // The EC projection's workspace: the split variant's first launch, or the
  // fused tiled launch's EC workgroups.
  const bool ec_ws = p.variant == SPEAR_VARIANT_SPLIT || (p.variant == SPEAR_VARIANT_FUSED && !skinny);
  int ec_blocks = 0;
  if (ec_ws) {
    const EcWorkspace L = ec_workspace_layout(d.M, d.K, d.rank,
                                              p.variant == SPEAR_VARIANT_FUSED ? kEcBlocksFused : kEcBlocksSplit);
    if (L.m_tiles > kMaxEcTiles) return SPEAR_ERR_UNSUPPORTED;
    ws = L.bytes;
    scratch_base = L.bytes;
    p.ec_split = L.splits;
    p.producers = L.m_tiles * L.splits;
    ec_blocks = (int)round_up(p.producers, 8);
  }
  if (skinny) {
    const SkinnyShape sh = skinny_shape(d.M, d.K, d.N, d.rank, p.variant == SPEAR_VARIANT_FUSED, cus,
                                        scratch_base);
    if (!sh.fits) return SPEAR_ERR_UNSUPPORTED;
    p.kernel = 0;
    p.tile_m = 16;
    p.tile_n = sh.nbw * 16;
    p.split_k = sh.S;
    p.grid = sh.T * sh.S + (p.variant == SPEAR_VARIANT_FUSED ? sh.P : 0);
    if (p.variant == SPEAR_VARIANT_FUSED) {
      p.producers = sh.P;
      p.ec_split = sh.P;
      p.ec_local = sh.local_ec ? 1 : 0;
    }
    if (sh.ws_bytes > ws) ws = sh.ws_bytes;
  } else {
    // X and the packed weight are addressed with 32-bit buffer offsets.
    if ((int64_t)d.M * d.K * 2 > INT32_MAX || n_pad(d.N) * k_pad(d.K) / 2 > INT32_MAX)
      return SPEAR_ERR_UNSUPPORTED;
    // Group scales are addressed the same way (2 bytes per 128 k and column).
    if (d.group_size != 0 && n_pad(d.N) * (k_pad(d.K) / 128) * 2 > INT32_MAX) return SPEAR_ERR_UNSUPPORTED;
    const TiledShape t = p.variant == SPEAR_VARIANT_FUSED ? fused_tiled_shape(d.M, d.K, d.N, cus, ec_blocks, scratch_base)
                                                          : tiled_shape(d.M, d.K, d.N, cus, scratch_base);
    if (!t.fits) return SPEAR_ERR_UNSUPPORTED;
    p.kernel = 1;
    p.tile_m = t.tm; p.tile_n = t.tn;
    p.split_k = t.split;
    // Fused: the EC workgroups (padded to a multiple of 8) lead the grid.
    p.grid = t.grid + (p.variant == SPEAR_VARIANT_FUSED ? ec_blocks : 0);
    if (t.ws_bytes > ws) ws = t.ws_bytes;
  }
  p.workspace_bytes = d.M > 0 ? ws : 0;
  p.predicted_us = (float)predict_call_us(p);
  p.predicted_no_ec_us = p.predicted_us;
  if (p.variant != SPEAR_VARIANT_NO_EC) {
    spear_linear_desc_t off = d;
    off.rank = 0;
    off.variant = SPEAR_VARIANT_NO_EC;
    spear_plan_t po;
    if (make_plan(off, cus, &po) == SPEAR_OK) p.predicted_no_ec_us = po.predicted_us;
  }
  *plan = p;
  return SPEAR_OK;
}

}  // namespace spear
