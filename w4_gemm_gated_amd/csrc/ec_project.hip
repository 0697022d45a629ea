// EC projection and per-token gate, the first launch of the split variant
// (the workgroup's work is in ec_block.h).  It is bound by reading X once
// (M K 2 bytes); [A | w_g] is small and stays in L2.
//
// Grid: 64-row tiles x K slices.
#include "ec_block.h"

namespace spear {

namespace {

// Sub-slab k: A sub-slab of at most 32 KiB.
inline int sub_slab(int64_t rank) {
  const int rp = ec_rank_pad(rank);
  return rp <= 64 ? 256 : rp <= 128 ? 128 : 64;
}

}  // namespace

EcWorkspace ec_workspace_layout(int64_t M, int64_t K, int64_t rank, int target_blocks) {
  EcWorkspace w;
  if (rank <= 0 || M <= 0) return w;
  w.tile_rows = kEcTileRows;
  w.m_tiles = (int32_t)ceil_div(M, kEcTileRows);
  // K slices: about target_blocks workgroups, at most 16 slices (the last
  // arriver of a row tile adds them all).
  const int ss = sub_slab(rank);
  w.ss = ss;
  const int64_t max_splits = ceil_div(K, ss);
  int64_t splits = ceil_div(target_blocks, w.m_tiles);
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

template <bool DMA, bool GVEC, int PB>
__global__ void __launch_bounds__(kEcThreads) ec_project_kernel(EcKArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  ec_block<DMA, GVEC, PB>(a, lds, blockIdx.x, blockIdx.y, 0u);
}

template <bool DMA, bool GVEC, int PB>
hipError_t launch_ec_pb(const EcKArgs& a, dim3 grid, size_t lds, void* stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&ec_project_kernel<DMA, GVEC, PB>), hipFuncAttributeMaxDynamicSharedMemorySize,
      96 * 1024);
  if (attr != hipSuccess) return attr;
  if (ec_kb_for(PB) * 32 != a.ss) return hipErrorInvalidValue;   // sub-slab and block count disagree
  hipLaunchKernelGGL((ec_project_kernel<DMA, GVEC, PB>), grid, dim3(kEcThreads), lds, (hipStream_t)stream, a);
  return hipGetLastError();
}

template <bool DMA, bool GVEC>
hipError_t launch_ec(const EcKArgs& a, dim3 grid, size_t lds, void* stream) {
  switch (ec_pb_for(a.rank)) {
    case 1: return launch_ec_pb<DMA, GVEC, 1>(a, grid, lds, stream);
    case 2: return launch_ec_pb<DMA, GVEC, 2>(a, grid, lds, stream);
    case 4: return launch_ec_pb<DMA, GVEC, 4>(a, grid, lds, stream);
    case 8: return launch_ec_pb<DMA, GVEC, 8>(a, grid, lds, stream);
    default: return launch_ec_pb<DMA, GVEC, 16>(a, grid, lds, stream);
  }
}

}  // namespace

hipError_t launch_ec_project(const EcArgs& e, void* stream) {
  const EcWorkspace L = ec_workspace_layout(e.M, e.K, e.rank);
  const EcKArgs a = make_ec_kargs(e, L);
  const size_t lds = ec_lds_bytes(a.ss, a.rp);
  const dim3 grid(L.m_tiles, L.splits);
  const bool dma = e.rank % 4 == 0 && ((uintptr_t)e.A % 16) == 0;
  const bool gvec = ((uintptr_t)e.w_g % 16) == 0;
  if (dma && gvec) return launch_ec<true, true>(a, grid, lds, stream);
  if (dma) return launch_ec<true, false>(a, grid, lds, stream);
  if (gvec) return launch_ec<false, true>(a, grid, lds, stream);
  return launch_ec<false, false>(a, grid, lds, stream);
}

}  // namespace spear
