// C ABI entry points (declared in include/spear_w4ec.h): argument checks,
// planning, and launches.  Nothing here allocates device memory or
// synchronizes; every check runs before anything is enqueued.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <set>
#include <utility>

#include "internal.h"

using namespace spear;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_cache[kMaxDevices];
// Polls before a cross-workgroup wait gives up (spear_debug_set_spin_limit).
std::atomic<uint32_t> g_spin_limit{kDefaultSpinLimit};
// Test hook (spear_debug_fail_waits): the fused waits look for tag ^ this.
std::atomic<uint32_t> g_wait_xor{0};

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

spear_status_t device_cus(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SPEAR_ERR_HIP;
  if (dev >= 0 && dev < kMaxDevices) {
    const int cached = g_cu_cache[dev].load(std::memory_order_relaxed);
    if (cached > 0) { *out = cached; return SPEAR_OK; }
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return SPEAR_ERR_HIP;
  if (dev >= 0 && dev < kMaxDevices) g_cu_cache[dev].store(cus, std::memory_order_relaxed);
  *out = cus;
  return SPEAR_OK;
}

spear_status_t plan_for(const spear_linear_desc_t& d, spear_plan_t* out) {
  spear_status_t st = check_desc(d);
  if (st != SPEAR_OK) return st;
  int cus = d.device_cus;
  if (cus == 0) {
    st = device_cus(&cus);
    if (st != SPEAR_OK) return st;
  }
  return make_plan(d, cus, out);
}

bool same_plan(const spear_plan_t& a, const spear_plan_t& b) {
  return a.abi_version == b.abi_version && a.layout_id == b.layout_id && a.variant == b.variant &&
         a.kernel == b.kernel && a.M == b.M && a.K == b.K && a.N == b.N && a.rank == b.rank &&
         a.tile_m == b.tile_m && a.tile_n == b.tile_n && a.split_k == b.split_k &&
         a.grid == b.grid && a.producers == b.producers && a.ec_split == b.ec_split &&
         a.cus == b.cus && a.group_size == b.group_size && a.workspace_bytes == b.workspace_bytes &&
         a.predicted_us == b.predicted_us && a.predicted_no_ec_us == b.predicted_no_ec_us;
}

spear_status_t hip_status(hipError_t e) { return e == hipSuccess ? SPEAR_OK : SPEAR_ERR_HIP; }

}  // namespace

namespace spear {

spear_status_t resolve_plan(const spear_linear_desc_t& desc, const spear_plan_t* plan, spear_plan_t* out) {
  spear_status_t st = check_desc(desc);
  if (st != SPEAR_OK) return st;
  if (!plan) return plan_for(desc, out);
  if (plan->abi_version != SPEAR_ABI_VERSION || plan->layout_id != SPEAR_LAYOUT_ID) return SPEAR_ERR_INVALID_PLAN;
  if (plan->variant < SPEAR_VARIANT_FUSED || plan->variant > SPEAR_VARIANT_NO_EC || plan->cus <= 0)
    return SPEAR_ERR_INVALID_PLAN;
  spear_linear_desc_t d2 = desc;
  d2.variant = plan->variant;
  d2.device_cus = plan->cus;
  spear_plan_t again;
  st = make_plan(d2, plan->cus, &again);
  if (st != SPEAR_OK || !same_plan(again, *plan)) return SPEAR_ERR_INVALID_PLAN;
  *out = *plan;
  return SPEAR_OK;
}

// hipFuncSetAttribute applies to the current device: remember, per (kernel,
// device), that it was set, so each device gets it once.
hipError_t set_max_dynamic_lds(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({kernel, dev})) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert({kernel, dev});
  return e;
}

}  // namespace spear

extern "C" {

const char* spear_status_str(spear_status_t status) {
  // A C caller may pass any int; read it as one (an out-of-range value held
  // in the C++ enum type would be undefined behaviour).
  int32_t s;
  static_assert(sizeof s == sizeof status, "spear_status_t is an int");
  std::memcpy(&s, &status, sizeof s);
  switch (s) {
    case SPEAR_OK: return "SPEAR_OK";
    case SPEAR_ERR_NULL_POINTER: return "SPEAR_ERR_NULL_POINTER: a required pointer is NULL";
    case SPEAR_ERR_INVALID_SHAPE: return "SPEAR_ERR_INVALID_SHAPE: need M >= 0, K >= 8, K % 8 == 0, N >= 1, 0 <= rank <= 256";
    case SPEAR_ERR_UNSUPPORTED: return "SPEAR_ERR_UNSUPPORTED: request outside what the kernels implement";
    case SPEAR_ERR_MISALIGNED: return "SPEAR_ERR_MISALIGNED: X, Wq and workspace need 16-byte, fp16 tensors 2-byte alignment";
    case SPEAR_ERR_WORKSPACE_TOO_SMALL: return "SPEAR_ERR_WORKSPACE_TOO_SMALL: workspace_bytes < plan.workspace_bytes (spear_w4ec_linear_noalloc: the plan needs more than its 64 MiB)";
    case SPEAR_ERR_INVALID_PLAN: return "SPEAR_ERR_INVALID_PLAN: plan does not match the descriptor or this library";
    case SPEAR_ERR_HIP: return "SPEAR_ERR_HIP: the HIP runtime reported an error";
    case SPEAR_ERR_INVALID_ARGUMENT: return "SPEAR_ERR_INVALID_ARGUMENT: non-finite bias, tau outside [0, 1] or unknown variant";
  }
  return "SPEAR_ERR_UNKNOWN";
}

uint32_t spear_abi_version(void) { return SPEAR_ABI_VERSION; }

spear_status_t spear_packed_bytes(int32_t K, int32_t N, size_t* bytes) {
  if (!bytes) return SPEAR_ERR_NULL_POINTER;
  if (K < 8 || K % 8 != 0 || N < 1) return SPEAR_ERR_INVALID_SHAPE;
  *bytes = (size_t)(k_pad(K) * n_pad(N) / 2);
  return SPEAR_OK;
}

spear_status_t spear_pack_w4(const void* W, int32_t K, int32_t N, void* Wq, void* scales, void* stream) {
  if (!W || !Wq || !scales) return SPEAR_ERR_NULL_POINTER;
  if (K < 8 || K % 8 != 0 || N < 1) return SPEAR_ERR_INVALID_SHAPE;
  if ((int64_t)K * 8 > INT32_MAX || (int64_t)N * 16 > INT32_MAX) return SPEAR_ERR_UNSUPPORTED;
  if (!aligned(W, 2) || !aligned(Wq, 16) || !aligned(scales, 2)) return SPEAR_ERR_MISALIGNED;
  return hip_status(launch_pack_w4(W, K, N, Wq, scales, stream));
}

spear_status_t spear_pack_w4_grouped(const void* W, int32_t K, int32_t N, int32_t group_size, void* Wq,
                                     void* scales, void* stream) {
  if (!W || !Wq || !scales) return SPEAR_ERR_NULL_POINTER;
  if (K < 8 || K % 8 != 0 || N < 1) return SPEAR_ERR_INVALID_SHAPE;
  if (group_size != SPEAR_GROUP_SIZE) return SPEAR_ERR_UNSUPPORTED;
  if ((int64_t)K * 8 > INT32_MAX || (int64_t)N * 16 > INT32_MAX) return SPEAR_ERR_UNSUPPORTED;
  if (!aligned(W, 2) || !aligned(Wq, 16) || !aligned(scales, 16)) return SPEAR_ERR_MISALIGNED;
  return hip_status(launch_pack_w4_grouped(W, K, N, Wq, scales, stream));
}

spear_status_t spear_ec_init_workspace_bytes(int32_t K, int32_t N, int32_t rank, size_t* bytes) {
  if (!bytes) return SPEAR_ERR_NULL_POINTER;
  if (K < 8 || K % 8 != 0 || N < 1 || rank < 1 || rank > SPEAR_MAX_RANK) return SPEAR_ERR_INVALID_SHAPE;
  if ((int64_t)K * 8 > INT32_MAX || (int64_t)N * 16 > INT32_MAX) return SPEAR_ERR_UNSUPPORTED;
  const EcInitLayout L = ec_init_layout(K, N, rank);
  if (!L.fits) return SPEAR_ERR_UNSUPPORTED;
  *bytes = L.bytes;
  return SPEAR_OK;
}

spear_status_t spear_ec_init(const void* W, const void* Wq, const void* scales, int32_t K, int32_t N,
                             int32_t group_size, int32_t rank, int32_t iterations, void* A, void* B,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!W || !Wq || !scales || !A || !B || !workspace) return SPEAR_ERR_NULL_POINTER;
  if (K < 8 || K % 8 != 0 || N < 1 || rank < 1 || rank > SPEAR_MAX_RANK) return SPEAR_ERR_INVALID_SHAPE;
  if (iterations < 0 || iterations > 64) return SPEAR_ERR_INVALID_ARGUMENT;
  if (group_size != 0 && group_size != SPEAR_GROUP_SIZE) return SPEAR_ERR_UNSUPPORTED;
  if ((int64_t)K * 8 > INT32_MAX || (int64_t)N * 16 > INT32_MAX) return SPEAR_ERR_UNSUPPORTED;
  const EcInitLayout L = ec_init_layout(K, N, rank);
  if (!L.fits) return SPEAR_ERR_UNSUPPORTED;
  if (workspace_bytes < L.bytes) return SPEAR_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned(W, 2) || !aligned(Wq, 16) || !aligned(scales, 2) || !aligned(A, 2) || !aligned(B, 2) ||
      !aligned(workspace, 16))
    return SPEAR_ERR_MISALIGNED;
  EcInitArgs a;
  a.W = W; a.Wq = Wq; a.scales = scales;
  a.K = K; a.N = N; a.rank = rank; a.grouped = group_size != 0 ? 1 : 0;
  a.iterations = iterations == 0 ? 10 : iterations;
  a.A = A; a.B = B; a.workspace = workspace; a.layout = L;
  return hip_status(launch_ec_init(a, stream));
}

spear_status_t spear_debug_unpack_w4(const void* Wq, int32_t K, int32_t N, void* q_out, void* stream) {
  if (!Wq || !q_out) return SPEAR_ERR_NULL_POINTER;
  if (K < 8 || K % 8 != 0 || N < 1) return SPEAR_ERR_INVALID_SHAPE;
  if (!aligned(Wq, 16)) return SPEAR_ERR_MISALIGNED;
  return hip_status(launch_unpack_w4(Wq, K, N, q_out, stream));
}

spear_status_t spear_dispatch_plan(const spear_linear_desc_t* desc, spear_plan_t* plan) {
  if (!desc || !plan) return SPEAR_ERR_NULL_POINTER;
  return plan_for(*desc, plan);
}

spear_status_t spear_ec_workspace_bytes(int32_t M, int32_t K, int32_t rank, size_t* bytes) {
  if (!bytes) return SPEAR_ERR_NULL_POINTER;
  if (M < 0 || K < 8 || K % 8 != 0 || rank < 1 || rank > SPEAR_MAX_RANK) return SPEAR_ERR_INVALID_SHAPE;
  *bytes = ec_workspace_layout(M, K, rank).bytes;
  return SPEAR_OK;
}

spear_status_t spear_ec_project(int32_t M, int32_t K, int32_t rank, const void* X, const void* A,
                                const void* w_g, float gate_bias, float skip_tau, void* P, void* g,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || K < 8 || K % 8 != 0 || rank < 1 || rank > SPEAR_MAX_RANK) return SPEAR_ERR_INVALID_SHAPE;
  if (!std::isfinite(gate_bias) || !std::isfinite(skip_tau) || skip_tau < 0.0f || skip_tau > 1.0f)
    return SPEAR_ERR_INVALID_ARGUMENT;
  if (M == 0) return SPEAR_OK;
  if (!X || !A || !w_g || !P || !g) return SPEAR_ERR_NULL_POINTER;
  const EcWorkspace L = ec_workspace_layout(M, K, rank);
  if (!workspace) return SPEAR_ERR_NULL_POINTER;
  if (workspace_bytes < L.bytes) return SPEAR_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned(X, 16) || !aligned(workspace, 16) || !aligned(A, 2) || !aligned(w_g, 2) ||
      !aligned(P, 4) || !aligned(g, 4))
    return SPEAR_ERR_MISALIGNED;
  EcArgs e;
  e.X = X; e.A = A; e.w_g = w_g;
  e.M = M; e.K = K; e.rank = rank;
  e.gate_bias = gate_bias; e.skip_tau = skip_tau;
  e.workspace = workspace;
  e.P_out = P; e.g_out = g; e.p_out_stride = rank;
  return hip_status(launch_ec_project(e, stream));
}

spear_status_t spear_w4ec_linear(const spear_linear_desc_t* desc, const spear_plan_t* plan,
                                 const void* X, const void* Wq, const void* scales, const void* A,
                                 const void* B, const void* w_g, void* Y, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!desc) return SPEAR_ERR_NULL_POINTER;
  spear_plan_t p;
  spear_status_t st = resolve_plan(*desc, plan, &p);
  if (st != SPEAR_OK) return st;
  if (desc->M == 0) return SPEAR_OK;
  const bool ec = p.variant != SPEAR_VARIANT_NO_EC;
  if (!X || !Wq || !scales || !Y) return SPEAR_ERR_NULL_POINTER;
  if (ec && (!A || !B || !w_g)) return SPEAR_ERR_NULL_POINTER;
  if (p.workspace_bytes > 0 && !workspace) return SPEAR_ERR_NULL_POINTER;
  if (workspace_bytes < p.workspace_bytes) return SPEAR_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned(X, 16) || !aligned(Wq, 16) || !aligned(scales, 2) || !aligned(Y, 2))
    return SPEAR_ERR_MISALIGNED;
  if (workspace && !aligned(workspace, 16)) return SPEAR_ERR_MISALIGNED;
  if (ec && (!aligned(A, 2) || !aligned(B, 2) || !aligned(w_g, 2))) return SPEAR_ERR_MISALIGNED;
  if (desc->group_size != 0 && !aligned(scales, 16)) return SPEAR_ERR_MISALIGNED;
  if (p.variant == SPEAR_VARIANT_FUSED && (!aligned(A, 16) || !aligned(w_g, 16))) return SPEAR_ERR_MISALIGNED;

  const bool skinny = p.kernel == 0;
  const bool fused_tiled = p.variant == SPEAR_VARIANT_FUSED && !skinny;
  size_t ec_bytes = 0;
  EcWorkspace L;
  EcArgs e;
  std::memset(&e, 0, sizeof(e));
  if (p.variant == SPEAR_VARIANT_SPLIT || fused_tiled) {
    L = ec_workspace_layout(desc->M, desc->K, desc->rank, fused_tiled ? kEcBlocksFused : kEcBlocksSplit);
    ec_bytes = L.bytes;
    e.X = X; e.A = A; e.w_g = w_g;
    e.M = desc->M; e.K = desc->K; e.rank = desc->rank;
    e.gate_bias = desc->gate_bias; e.skip_tau = desc->skip_tau;
    e.workspace = workspace;
    e.P_out = nullptr; e.g_out = nullptr; e.p_out_stride = 0;
  }
  if (p.variant == SPEAR_VARIANT_SPLIT) {
    st = hip_status(launch_ec_project(e, stream));
    if (st != SPEAR_OK) return st;
  }
  if (skinny) {
    SkinnyLaunch s;
    s.shape = skinny_shape(desc->M, desc->K, desc->N, desc->rank, p.variant == SPEAR_VARIANT_FUSED, p.cus,
                           ec_bytes ? ec_bytes : kSyncHeaderBytes);
    s.X = X; s.Wq = Wq; s.scales = scales; s.A = A; s.B = B; s.w_g = w_g; s.Y = Y;
    s.M = desc->M; s.K = desc->K; s.N = desc->N; s.rank = ec ? desc->rank : 0;
    s.ec_mode = p.variant == SPEAR_VARIANT_FUSED ? 1 : (p.variant == SPEAR_VARIANT_SPLIT ? 2 : 0);
    s.gate_bias = desc->gate_bias; s.skip_tau = desc->skip_tau;
    s.workspace = workspace;
    s.Pext = ec_bytes ? (const float*)((const char*)workspace + L.p) : nullptr;
    s.gext = ec_bytes ? (const float*)((const char*)workspace + L.g) : nullptr;
    s.grouped = desc->group_size != 0 ? 1 : 0;
    s.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    s.wait_xor = g_wait_xor.load(std::memory_order_relaxed);
    return hip_status(launch_skinny(s, stream));
  }
  GemmArgs ga;
  std::memset(&ga, 0, sizeof(ga));
  ga.X = X; ga.Wq = Wq; ga.scales = scales; ga.Y = Y;
  ga.workspace = workspace;
  ga.scratch_base = ec_bytes ? ec_bytes : kSyncHeaderBytes;
  ga.M = desc->M; ga.K = desc->K; ga.N = desc->N; ga.rank = desc->rank;
  if (ec) {
    ga.B = B;
    ga.P = (const float*)((const char*)workspace + L.p);
    ga.g = (const float*)((const char*)workspace + L.g);
    ga.ec = 1;
  }
  ga.fused = fused_tiled ? 1 : 0;
  ga.ecargs = e;
  ga.grouped = desc->group_size != 0 ? 1 : 0;
  ga.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  ga.wait_xor = g_wait_xor.load(std::memory_order_relaxed);
  return hip_status(launch_gemm(ga, p, stream));
}

spear_status_t spear_take_error(void* workspace, size_t workspace_bytes, void* code_out, void* stream) {
  if (!code_out) return SPEAR_ERR_NULL_POINTER;
  if (!workspace && workspace_bytes == 0) {
    // The allocation-free entry point's workspace on the current device.
    if (static_scratch(&workspace, stream) != hipSuccess) return SPEAR_ERR_HIP;
    workspace_bytes = kStaticScratchBytes;
  }
  if (!workspace) return SPEAR_ERR_NULL_POINTER;
  if (workspace_bytes < kSyncHeaderBytes) return SPEAR_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned(workspace, 16) || !aligned(code_out, 4)) return SPEAR_ERR_MISALIGNED;
  return hip_status(launch_take_error(workspace, code_out, stream));
}

void spear_debug_set_spin_limit(int64_t polls) {
  const uint32_t v = polls < 0 ? kDefaultSpinLimit : polls > (int64_t)UINT32_MAX ? UINT32_MAX : (uint32_t)polls;
  g_spin_limit.store(v, std::memory_order_relaxed);
}

void spear_debug_fail_waits(int32_t on) { g_wait_xor.store(on ? 0x40000000u : 0u, std::memory_order_relaxed); }

spear_status_t spear_debug_stream_read(const void* src, size_t bytes, int32_t grid, void* sink, void* stream) {
  if (!src || !sink) return SPEAR_ERR_NULL_POINTER;
  if (bytes == 0 || bytes % 16 != 0 || grid < 1) return SPEAR_ERR_INVALID_SHAPE;
  if (!aligned(src, 16) || !aligned(sink, 4)) return SPEAR_ERR_MISALIGNED;
  return hip_status(launch_stream_read(src, bytes, grid, sink, stream));
}

spear_status_t spear_debug_mfma_rate(int32_t shape, int32_t waves_per_simd, int32_t iterations, void* sink,
                                    void* stream, double* flops) {
  if (!sink || !flops) return SPEAR_ERR_NULL_POINTER;
  if ((shape != 0 && shape != 1) || (waves_per_simd != 1 && waves_per_simd != 2 && waves_per_simd != 4) ||
      iterations < 1 || iterations > (1 << 20))
    return SPEAR_ERR_INVALID_ARGUMENT;
  if (!aligned(sink, 4)) return SPEAR_ERR_MISALIGNED;
  int cus = 0;
  const spear_status_t st = device_cus(&cus);
  if (st != SPEAR_OK) return st;
  // 16 x 16 x 32 and 32 x 32 x 16: 8192 and 16384 multiply-adds per
  // instruction; 8 and 4 accumulators per wave and round.
  const double per_round = shape == 0 ? 8.0 * 8192 * 2 : 4.0 * 16384 * 2;
  *flops = per_round * iterations * 4.0 * waves_per_simd * cus;
  return hip_status(launch_mfma_rate(shape, waves_per_simd, iterations, cus, sink, stream));
}

}  // extern "C"
