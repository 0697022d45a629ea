/*
 * spear_w4ec.h -- C ABI of the MI355X (gfx950) W4 linear layer with a
 * per-token-gated low-rank Error Compensator (EC).
 *
 * Method: "SPEAR: A System for Post-Quantization Error-Adaptive Recovery
 * Enabling Efficient Low-Bit LLM Serving" (arXiv 2606.11244), abstract: weights
 * in 4 bits with one scale per output channel, small error-compensating
 * branches whose output each token's gate scales, the second half of that
 * branch computed inside the low-bit GEMM, and a per-call choice of how much
 * to fuse.  The page gives no formulas; this library computes
 *
 *     Y = X . dequant(Wq, s) + g' (.) ((X . A) . B)
 *     g = sigmoid(X . w_g + b_g),  g' = g, or g . [g >= tau] when tau > 0
 *
 * with a symmetric int4 per-output-channel quantizer s = fp16(max|w| / 7),
 * q = clamp(rint(w / s), -7, 7).
 *
 * Conventions for every entry point
 *   - Tensors are device pointers owned by the caller and borrowed until the
 *     work enqueued on `stream` completes.  The library allocates, frees and
 *     synchronizes nothing.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - All work is enqueued asynchronously on `stream`; argument checks happen
 *     before anything is enqueued and return a status without side effects.
 *     Faults inside kernels surface at the caller's next synchronization.
 *   - Row-major layouts; "fp16" is IEEE binary16.
 *   - No C++ exception crosses this interface.  Functions are reentrant; the
 *     only global state is a per-device cache of the compute-unit count.
 */
#ifndef SPEAR_W4EC_H
#define SPEAR_W4EC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEAR_ABI_VERSION 1u
#define SPEAR_LAYOUT_ID 2u
#define SPEAR_MAX_RANK 256

typedef enum spear_status {
  SPEAR_OK = 0,
  SPEAR_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
  SPEAR_ERR_INVALID_SHAPE = 2,       /* M < 0, K < 8, K % 8 != 0, N < 1, rank outside [0, 256] */
  SPEAR_ERR_UNSUPPORTED = 3,         /* a request outside what the kernels implement */
  SPEAR_ERR_MISALIGNED = 4,          /* a pointer misses its required alignment */
  SPEAR_ERR_WORKSPACE_TOO_SMALL = 5, /* workspace_bytes < plan.workspace_bytes */
  SPEAR_ERR_INVALID_PLAN = 6,        /* plan does not match the descriptor or this library */
  SPEAR_ERR_HIP = 7,                 /* the HIP runtime reported an error (device query or launch) */
  SPEAR_ERR_INVALID_ARGUMENT = 8     /* a non-finite bias/threshold or an unknown variant */
} spear_status_t;

/* Kernel-fusion variants (SPEAR page, abstract: the fusion is chosen per call). */
typedef enum spear_variant {
  SPEAR_VARIANT_AUTO = 0,  /* let spear_dispatch_plan choose */
  SPEAR_VARIANT_FUSED = 1, /* one launch: EC projection and gate, W4 GEMM, gated EC epilogue */
  SPEAR_VARIANT_SPLIT = 2, /* EC projection and gate launch, then the W4 GEMM with the gated EC epilogue */
  SPEAR_VARIANT_NO_EC = 3  /* skip-EC: the W4 GEMM alone (rank 0, or the EC switched off) */
} spear_variant_t;

/* One call of the layer. */
typedef struct spear_linear_desc {
  int32_t M;          /* tokens (rows of X and Y); 0 is a no-op */
  int32_t K;          /* input features; multiple of 8 */
  int32_t N;          /* output features; >= 1 */
  int32_t rank;       /* EC rank r in [0, 256]; 0 = no EC */
  float gate_bias;    /* b_g */
  float skip_tau;     /* tau in [0, 1]; 0 keeps every gate (the exact definition) */
  int32_t variant;    /* spear_variant_t */
  int32_t device_cus; /* 0: query the current device; > 0: plan for that many CUs, no device access */
} spear_linear_desc_t;

/* A resolved launch plan (plain data; may be cached and reused for the same
 * descriptor shape).  Produced by spear_dispatch_plan only. */
typedef struct spear_plan {
  uint32_t abi_version; /* SPEAR_ABI_VERSION */
  uint32_t layout_id;   /* SPEAR_LAYOUT_ID */
  int32_t variant;      /* resolved variant: FUSED, SPLIT or NO_EC */
  int32_t kernel;       /* main kernel family: 0 = skinny (small M), 1 = tiled (large M) */
  int32_t M, K, N, rank;
  int32_t tile_m, tile_n; /* output tile of one workgroup */
  int32_t split_k;        /* K slices of the main GEMM reduced across workgroups (1 = none) */
  int32_t grid;           /* workgroups of the main launch */
  int32_t producers;      /* workgroups that compute the EC projection */
  int32_t ec_split;       /* K slices of the EC projection */
  int32_t cus;            /* compute units planned for */
  int32_t ec_local;       /* 1: every workgroup of the main launch computes the EC projection itself */
  size_t workspace_bytes; /* device workspace the call needs (0 = none) */
} spear_plan_t;

/* Human-readable name of a status code (static storage; never NULL). */
const char* spear_status_str(spear_status_t status);

/* SPEAR_ABI_VERSION of the loaded library. */
uint32_t spear_abi_version(void);

/* Size in bytes of the packed weight for a K x N matrix: K and N are padded
 * to multiples of 128 and 16, four bits per weight.
 * Errors: NULL_POINTER (bytes), INVALID_SHAPE. */
spear_status_t spear_packed_bytes(int32_t K, int32_t N, size_t* bytes);

/*
 * spear_pack_w4 -- quantize and pack a weight (SPEAR page, abstract: 4-bit weights,
 * one scale per output channel).
 *   W      fp16 [K, N] row-major (input dimension first; an nn.Linear weight
 *          is W = weight^T), 2-byte aligned.
 *   Wq     output, spear_packed_bytes(K, N) bytes, 16-byte aligned.
 *   scales output, fp16 [N], 2-byte aligned.
 * s[n] = fp16(max_k |W[k,n]| / 7) (float32 division, round to nearest even);
 * q = clamp(rint(W / s), -7, 7) (float32 division, ties to even), q = 0 where
 * s = 0; u = q + 8.  Layout id 2: the u of k-octet (k8, n) form one uint32
 * whose bit field i (bits 4i..4i+3) holds k-offset (0,2,4,6,1,3,5,7)[i];
 * with nb = n/16, c = n%16, kc = k8/16, j = (k8%16)/4, t = k8%4 the word sits
 * at index ((nb*(K_pad/128) + kc)*64 + t*16 + c)*4 + j.  Padding words hold
 * u = 8 (q = 0).  Inputs must be finite.
 * Errors: NULL_POINTER, INVALID_SHAPE (K % 8, K < 8, N < 1), MISALIGNED, HIP.
 */
spear_status_t spear_pack_w4(const void* W, int32_t K, int32_t N, void* Wq, void* scales,
                             void* stream);

/*
 * spear_dispatch_plan -- choose the kernel-fusion variant and the launch
 * shape for a call (SPEAR page, abstract: the fusion variant adapts to the call).
 * Host only; touches the device only to read its CU count when
 * desc->device_cus == 0 (cached per device).
 * Rules: rank 0 or variant NO_EC -> NO_EC; AUTO -> FUSED when rank % 4 == 0
 * (any M: the skinny kernel up to 16 rows, the tiled kernel above, both with
 * the EC projection in the same launch), except where the tiled kernel uses
 * 128-row tiles (M of about 257 to 1024) that alone exceed the GPU's CUs
 * (measured: SPLIT faster there); else SPLIT.  Skinny FUSED takes
 * one of two forms, reported by plan.ec_local: when the weight GEMM needs no
 * K split, rank <= 64 and A is at most 64 KiB (128 KiB with rank <= 32 and
 * M <= 4), every GEMM workgroup
 * computes the whole projection itself with four extra waves (ec_local = 1,
 * producers = 0, no workspace); otherwise producer workgroups lead the grid
 * and hand P and the gate over through the workspace (ec_local = 0).  FUSED with
 * rank % 4 != 0 (or with more than 4096 row tiles of 64 in the tiled case),
 * and the tiled kernel (M > 16) with X or the packed weight above
 * 2^31 - 1 bytes (32-bit buffer offsets), are UNSUPPORTED.  The per-token gate-value
 * decision (skip the EC term of a tile whose gates are all below tau) is
 * taken on the device inside the epilogue, so no gate value ever crosses to
 * the host.
 * Errors: NULL_POINTER, INVALID_SHAPE, INVALID_ARGUMENT, UNSUPPORTED, HIP.
 */
spear_status_t spear_dispatch_plan(const spear_linear_desc_t* desc, spear_plan_t* plan);

/*
 * spear_w4ec_linear -- Y = X . dequant(Wq, s) + g' (.) ((X . A) . B).
 *   desc     the call; plan may be NULL (planned internally) or the result of
 *            spear_dispatch_plan for the same M, K, N, rank and variant.
 *   X        fp16 [M, K], 16-byte aligned.
 *   Wq, scales  from spear_pack_w4 (16- and 2-byte aligned).
 *   A        fp16 [K, rank], B fp16 [rank, N], w_g fp16 [K] (2-byte aligned;
 *            A and w_g 16-byte aligned for the fused variant); may be NULL when
 *            rank == 0 or the resolved variant is NO_EC.  Inputs must be finite.
 *   Y        output fp16 [M, N] (2-byte aligned), fully overwritten,
 *            fp16(s[n] acc[m,n] + g'[m] sum_j P[m,j] B[j,n]) with fp32
 *            accumulation; must not alias any input.
 *   workspace  device memory of at least plan.workspace_bytes (16-byte
 *            aligned; may be NULL when that is 0).  It must be zero-filled
 *            before its first use.  Its first 256 KiB are a header owned by
 *            the library: cross-workgroup counters, which every call returns
 *            to zero, a call epoch, which every fused call advances by one,
 *            and the fused variants' ready flags and hand-off slabs, which
 *            carry the epoch of the call that wrote them.  The rest is
 *            scratch.  So a
 *            zero-filled workspace can be reused, without clearing, by later
 *            calls of any plan that fit in it; the caller must not write to
 *            it between calls.  Calls that run concurrently must not share a
 *            workspace.
 * Errors: NULL_POINTER, INVALID_SHAPE, INVALID_ARGUMENT, MISALIGNED,
 *         WORKSPACE_TOO_SMALL, INVALID_PLAN, UNSUPPORTED, HIP.
 */
spear_status_t spear_w4ec_linear(const spear_linear_desc_t* desc, const spear_plan_t* plan,
                                 const void* X, const void* Wq, const void* scales,
                                 const void* A, const void* B, const void* w_g, void* Y,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * spear_ec_project -- the EC projection and gate alone, in one pass over X
 * (the first half of the split variant):
 *   P[m, j] = sum_k X[m,k] A[k,j]   (fp32 [M, rank])
 *   g[m]    = g'(sigmoid(sum_k X[m,k] w_g[k] + b_g))   (fp32 [M], after tau)
 * X fp16 [M, K] 16-byte aligned; A fp16 [K, rank]; w_g fp16 [K]; rank >= 1.
 * workspace as for spear_w4ec_linear, size from spear_ec_workspace_bytes.
 * Errors: NULL_POINTER, INVALID_SHAPE, INVALID_ARGUMENT, MISALIGNED,
 *         WORKSPACE_TOO_SMALL, HIP.
 */
spear_status_t spear_ec_workspace_bytes(int32_t M, int32_t K, int32_t rank, size_t* bytes);
spear_status_t spear_ec_project(int32_t M, int32_t K, int32_t rank, const void* X, const void* A,
                                const void* w_g, float gate_bias, float skip_tau, void* P,
                                void* g, void* workspace, size_t workspace_bytes, void* stream);

/*
 * spear_debug_unpack_w4 -- decode a packed weight back to int8 codes
 * q [K, N] (row-major, values in [-8, 7]) with the same in-register decode
 * the GEMM kernels use.  For bit-exactness tests.
 * Errors: NULL_POINTER, INVALID_SHAPE, MISALIGNED, HIP.
 */
spear_status_t spear_debug_unpack_w4(const void* Wq, int32_t K, int32_t N, void* q_out,
                                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEAR_W4EC_H */
