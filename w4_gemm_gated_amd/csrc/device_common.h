// Device helpers shared by the gfx950 kernels of the W4+EC linear layer.
//
// Matrix instruction: v_mfma_f32_16x16x32_f16 (64 lanes).  For lane L,
// t = L / 16 and c = L % 16:
//   A operand (16 x 32): row c, k = 8t .. 8t+7 (8 halves, 16 bytes)
//   B operand (32 x 16): column c, k = 8t .. 8t+7
//   C/D (16 x 16 fp32): column c, rows 4t .. 4t+3
// The packed weight (layout id 2) stores, in the 16 bytes of lane slot L of
// every 1 KiB tile, the B operand of that lane for four consecutive 32-k
// blocks, so one 16-byte load per lane feeds four instructions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace spear {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kKChunk = 128;   // k extent of one packed tile
constexpr int kNBlock = 16;    // columns of one packed panel
constexpr uint32_t kZeroCodeWord = 0x88888888u;  // eight codes u = 8 (q = 0)

__device__ __forceinline__ float4_t mfma16x16x32(const half8_t& a, const half8_t& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Decode one packed word (eight 4-bit codes u, fields in k order
// 0,2,4,6,1,3,5,7) into the eight fp16 values q = u - 8 in k order.
// OR-ing 0x6400 into a 16-bit half holding u (< 16) in its low mantissa bits
// gives exactly the fp16 value 1024 + u; subtracting 1032 leaves u - 8.  A
// code in mantissa bits 4..7 gives 1024 + 16 u instead, and one fused
// multiply-add (x / 16 - 72) leaves u - 8, exactly (64 + u is an fp16
// integer).  So the word and one copy shifted by 8 cover all eight codes:
// one shift, four AND-ORs, two packed subtractions and two packed FMAs.
// (x & m) | e in one instruction (the compiler emits an AND and an OR).
// One scalar operand at most (one constant-bus read per instruction).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t e) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(x), "s"(m), "v"(e));
  return d;
}
__device__ __forceinline__ half8_t decode_w4(uint32_t w) {
  const uint32_t lo = 0x000F000Fu, hi = 0x00F000F0u, e = 0x64006400u;
  const uint32_t w8 = w >> 8;
  const uint32_t d0 = and_or(w, lo, e);     // fields 0, 4 -> 1024 + u
  const uint32_t d1 = and_or(w, hi, e);     // fields 1, 5 -> 1024 + 16 u
  const uint32_t d2 = and_or(w8, lo, e);    // fields 2, 6 -> 1024 + u
  const uint32_t d3 = and_or(w8, hi, e);    // fields 3, 7 -> 1024 + 16 u
  const half2_t bias = {(half_t)1032.0f, (half_t)1032.0f};
  const half2_t sixteenth = {(half_t)0.0625f, (half_t)0.0625f};
  const half2_t bias16 = {(half_t)-72.0f, (half_t)-72.0f};
  const half2_t h0 = __builtin_bit_cast(half2_t, d0) - bias;
  const half2_t h1 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, d1), sixteenth, bias16);
  const half2_t h2 = __builtin_bit_cast(half2_t, d2) - bias;
  const half2_t h3 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, d3), sixteenth, bias16);
  half8_t r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

__device__ __forceinline__ half8_t zero_half8() {
  half8_t z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (half_t)0.0f;
  return z;
}

__device__ __forceinline__ float4_t zero_float4() {
  float4_t z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// 16-byte load of 8 halves; the caller guarantees 16-byte alignment.
__device__ __forceinline__ half8_t load_half8(const half_t* p) {
  return *reinterpret_cast<const half8_t*>(p);
}

// Bit casts through a by-value parameter.  (This compiler miscompiles
// __builtin_bit_cast applied directly to a vector element, v[i]: it reads
// element 0 for every i.  A scalar parameter avoids that form.)
__device__ __forceinline__ uint32_t float_bits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bits_float(uint32_t x) { return __builtin_bit_cast(float, x); }

// 1 / (1 + e^-z) from the hardware base-2 exponential and reciprocal (a few
// ulp; the gate feeds an fp16 product).  z = -inf-like values give 0, large
// z give 1.
__device__ __forceinline__ float sigmoidf_(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.44269504088896341f));
}

// Buffer resource over [base, base + bytes): raw buffer loads at an offset
// outside it return zeros without touching memory, which masks lanes without
// a branch (a branch around a load makes the compiler wait for it early).
constexpr uint32_t kBufferRsrcWord3 = 0x00020000u;   // gfx9 family: 32-bit data format
constexpr uint32_t kOutOfRange = 0x80000000u;         // offset beyond any resource here
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kBufferRsrcWord3);
}
__device__ __forceinline__ half8_t buffer_load_half8(__amdgpu_buffer_rsrc_t r, uint32_t byte_offset) {
  return __builtin_bit_cast(half8_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 0));
}
// 16-byte device-coherent load (cache policy sc1, as a device-scope atomic
// load uses), for data other workgroups published with device-coherent stores.
constexpr int kCachePolicySc1 = 16;
__device__ __forceinline__ float4_t buffer_load_f4_dev(__amdgpu_buffer_rsrc_t r, uint32_t byte_offset) {
  return __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, kCachePolicySc1));
}

// ---------------------------------------------------------------------------
// Cross-workgroup exchange without L2 write-backs.  Workgroups on different
// XCDs do not share an L2, and a release/acquire fence at device scope
// writes back / invalidates the whole L2 of the issuing XCD.  Data exchanged
// between workgroups is instead stored and loaded with device-scope relaxed
// atomics, which the compiler emits as sc1 (device-coherent) stores and
// loads; the writer drains its stores (s_waitcnt vmcnt(0)) before it bumps
// the device-scope counter that publishes them, and the reader loads the data
// only after it has seen the counter (or flag).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev_u32(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory instruction this wave issued has completed.
__device__ __forceinline__ void drain_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// The same wait in a form the compiler sees (s_waitcnt with vmcnt = 0 and
// the other counters at their maximum, gfx9 encoding).  A wait written in
// inline asm is opaque to the compiler's own wait insertion, which then adds
// a second vmcnt(0) at the first use of a loaded register, possibly after
// loads issued meanwhile; this form lets it know those registers are ready.
// The empty asm statements keep memory accesses from moving across it.
__device__ __forceinline__ void wait_vm_all() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}
// Wait until at most N of this wave's memory instructions are in flight
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vm_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x0F70 | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t or_dev_u32(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Call epochs of the fused variants.  Every block of a fused call reads the
// epoch word of the workspace header when it starts; the call's tag is
// epoch + 1, the value that its ready flags and hand-off entries carry.  The
// epoch stays in [0, 2^32 - 2], so a tag is never 0 (the value of a zero-filled
// header).  Each block counts itself out once it no longer needs the tag
// (count_out, run by one whole wave); the last of the call's blocks returns
// the finisher count to zero and advances the epoch to the tag.  When the tag
// is the largest value, that block instead clears every tagged word of the
// header (the ready flags and the hand-off slabs) and restarts the epoch at 0,
// so no word written before the wrap can match a later tag.
// ---------------------------------------------------------------------------
constexpr uint32_t kLastTag = 0xFFFFFFFFu;

__device__ __forceinline__ uint32_t call_tag(const uint32_t* sync) {
  return ld_dev_u32(&sync[kSyncEpoch]) + 1u;
}

__device__ __noinline__ void count_out(uint32_t* sync, uint32_t total, uint32_t tag) {
  const int lane = threadIdx.x % kWave;
  uint32_t before = 0;
  if (lane == 0) before = add_dev_u32(&sync[kSyncFinishers], 1u);
  before = __builtin_amdgcn_readfirstlane(before);
  if (before != total - 1) return;
  if (tag == kLastTag) {
    unsigned char* base = reinterpret_cast<unsigned char*>(sync) - kGemmSyncOffset;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base, (uint32_t)kSyncHeaderBytes);
    const u32x4_t z = {0u, 0u, 0u, 0u};
    // ready flags: words [kEcReadyWord, 8192) of the EC counter region
    for (uint32_t off = kEcReadyWord * 4u + 16u * lane; off < 8192u * 4u; off += 16u * kWave)
      __builtin_amdgcn_raw_buffer_store_b128(z, r, off, 0, kCachePolicySc1);
    for (uint32_t off = (uint32_t)kHandoffOffset + 16u * lane; off < (uint32_t)(kHandoffOffset + kHandoffBytes);
         off += 16u * kWave)
      __builtin_amdgcn_raw_buffer_store_b128(z, r, off, 0, kCachePolicySc1);
    drain_vm();
  }
  if (lane == 0) {
    st_dev_u32(&sync[kSyncFinishers], 0u);
    st_dev_u32(&sync[kSyncEpoch], tag == kLastTag ? 0u : tag);
  }
}

}  // namespace spear
