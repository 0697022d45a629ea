// Host planner: the per-call choice of fusion variant (SPEAR page, abstract),
// reduced to what one GPU needs.  Pure host arithmetic on the descriptor; the
// device is touched only by the caller (api.cpp) to read the CU count.
//
// Decisions:
//   * no EC (rank 0) or variant NO_EC            -> NO_EC: the W4 GEMM alone;
//   * AUTO and rank % 4 == 0                     -> FUSED: one launch (EC
//     workgroups first, then the W4 GEMM with the gated epilogue, which
//     waits for the EC results it needs; at M <= 16 the EC computed by every
//     GEMM workgroup itself when A is small), except 128-row tiles whose
//     fused launch would exceed the CUs (M of about 257 to 1024), where the
//     measured crossover favours SPLIT;
//   * AUTO otherwise (rank % 4 != 0)             -> SPLIT (EC projection
//     launch, then the W4 GEMM with the gated epilogue);
//   * the per-token gate-value decision (skip the EC term where every gate of
//     a wave's rows is below tau) is taken on the device in the epilogue.
//   * main kernel family by M: skinny (M <= 16 rows) or tiled (256-row tiles;
//     128- or 64-row tiles with K split where those would not fill the GPU).
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
  // Measured crossover (mid M, hot weights, 128 EC workgroups): with
  // 128-row tiles that alone exceed the CUs the split variant is faster
  // (M = 512, K = 4096, N = 14336: 87 vs 94 us); where the tiles fit, the
  // fused one is, also when its EC workgroups overflow the CUs (M = 512,
  // K = 14336, N = 4096: 98 vs 104 us; M = 768: 153 vs 161; M = 1024: 163 vs
  // 172; M = 1024, K = N = 4096: 57 vs 61; M = 512, K = 2048, N = 8192: a
  // tie), as with 64-row (M <= 256) and 256-row tiles.
  auto split_wins = [&]() {
    if (skinny) return false;
    const EcWorkspace L = ec_workspace_layout(d.M, d.K, d.rank, kEcBlocksFused);
    const int eb = (int)round_up(L.m_tiles * L.splits, 8);
    const TiledShape t = fused_tiled_shape(d.M, d.K, d.N, cus, eb, kSyncHeaderBytes);
    return t.tm == 128 && t.grid > cus;
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
  *plan = p;
  return SPEAR_OK;
}

}  // namespace spear
