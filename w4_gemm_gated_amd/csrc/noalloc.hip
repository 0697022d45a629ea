// Allocation-free form of the layer call, for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops that forbid
// it): the call's workspace is the library's own file-scope device array
// `scratch`, one copy per GPU, held until the process ends.
//
// Host code never passes `scratch` itself to a kernel (on the host that name
// is a stand-in, not a device address): at set-up, once per device with that
// device current, hipGetSymbolAddress gives this device's address, which is
// kept and used for every kernel argument.  Set-up also zeroes the array's
// workspace header with a fill kernel on the caller's stream, ordered before
// the first call; every call returns the header's counters to zero, so later
// calls need no clearing.  Set-up refuses a stream under graph capture: the
// fill would be recorded into the graph instead of run.  Every call on one GPU shares its array: calls that
// overlap on one GPU race (they must be ordered, e.g. on one stream).
#include <atomic>
#include <mutex>

#include "device_common.h"
#include "internal.h"

namespace spear {

namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_setup_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

__global__ void zero_header_kernel(u32x4_t* p, int units) {
  const u32x4_t z = {0u, 0u, 0u, 0u};
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < units; i += gridDim.x * blockDim.x) p[i] = z;
}

}  // namespace

hipError_t static_scratch(void** out, void* stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) {
    *out = p;
    return hipSuccess;
  }
  std::lock_guard<std::mutex> lock(g_setup_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing((hipStream_t)stream, &capture);
    if (e != hipSuccess) return e;
    if (capture != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    const int units = (int)(kSyncHeaderBytes / 16);
    hipLaunchKernelGGL(zero_header_kernel, dim3(64), dim3(256), 0, (hipStream_t)stream, (u32x4_t*)p, units);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace spear

using namespace spear;

extern "C" spear_status_t spear_w4ec_linear_noalloc(const spear_linear_desc_t* desc, const spear_plan_t* plan,
                                                    const void* X, const void* Wq, const void* scales,
                                                    const void* A, const void* B, const void* w_g, void* Y,
                                                    void* stream) {
  if (!desc) return SPEAR_ERR_NULL_POINTER;
  spear_plan_t p;
  const spear_status_t st = resolve_plan(*desc, plan, &p);
  if (st != SPEAR_OK) return st;
  if (p.workspace_bytes > kStaticScratchBytes) return SPEAR_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (p.workspace_bytes > 0 && desc->M > 0) {
    if (static_scratch(&ws, stream) != hipSuccess) return SPEAR_ERR_HIP;
  }
  return spear_w4ec_linear(desc, &p, X, Wq, scales, A, B, w_g, Y, ws, ws ? kStaticScratchBytes : 0, stream);
}
