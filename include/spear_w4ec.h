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
 *     global state is a per-device cache of the compute-unit count, a record
 *     of which kernels had their LDS limit raised on which device, and the
 *     debug bound of cross-workgroup waits (spear_debug_set_spin_limit).
 */
#ifndef SPEAR_W4EC_H
#define SPEAR_W4EC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEAR_ABI_VERSION 3u
#define SPEAR_LAYOUT_ID 2u
#define SPEAR_MAX_RANK 256
#define SPEAR_GROUP_SIZE 128   /* the one group size of group-wise scales */

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
  int32_t group_size; /* 0: one scale per output channel, scales fp16 [N] (spear_pack_w4);
                         SPEAR_GROUP_SIZE: one scale per 128 input rows and output channel,
                         scales fp16 [ceil(K / 128), N rounded up to 16] (spear_pack_w4_grouped) */
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
  int32_t group_size;     /* as in the descriptor */
  float predicted_us;       /* cost model: predicted time of this call (microseconds, MI355X) */
  float predicted_no_ec_us; /* cost model: the same call with the EC switched off */
  size_t workspace_bytes; /* device workspace the call needs (0 = none) */
} spear_plan_t;

/* One linear layer of a batch, as the EC scheduler sees it. */
typedef struct spear_sched_layer {
  int32_t K, N, rank;   /* rank 0: the layer has no EC */
  int32_t group_size;   /* 0 or SPEAR_GROUP_SIZE, as in spear_linear_desc_t */
  float weight;         /* value of keeping this layer's EC on (>= 0), e.g. its share of the
                           error the ECs remove; layers of equal weight are equally worth it */
} spear_sched_layer_t;

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
 * spear_pack_w4_grouped -- quantize and pack a weight with group-wise scales
 * (SPEAR page, abstract: per-channel quantization is named the challenging
 * setting; this is its usual counterpart, one scale per group of input rows).
 *   W, Wq as for spear_pack_w4 (the same packed layout of the codes).
 *   group_size  SPEAR_GROUP_SIZE (other sizes: UNSUPPORTED).
 *   scales  output, fp16 [ceil(K / 128), N_pad] row-major, N_pad = N rounded up
 *           to 16 (columns >= N hold 0), 16-byte aligned:
 *           s[g, n] = fp16(max over k in [128 g, 128 g + 128) of |W[k, n]| / 7)
 *           (the last group may be shorter); q = clamp(rint(W[k, n] / s[g, n]),
 *           -7, 7) with g = k / 128 and the per-channel rules otherwise.
 * Errors: NULL_POINTER, INVALID_SHAPE, UNSUPPORTED, MISALIGNED, HIP.
 */
spear_status_t spear_pack_w4_grouped(const void* W, int32_t K, int32_t N, int32_t group_size, void* Wq,
                                     void* scales, void* stream);

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
 * the skinny kernel (M <= 16) with K above 262144 (64 K splits of 32 chunks of
 * 128), and the tiled kernel (M > 16) with X or the packed weight above
 * 2^31 - 1 bytes (32-bit buffer offsets), are UNSUPPORTED.  The per-token gate-value
 * decision (skip the EC term of a tile whose gates are all below tau) is
 * taken on the device inside the epilogue, so no gate value ever crosses to
 * the host.  The plan also carries the cost model's predicted time of the
 * call and of the same call with the EC off (a roofline with constants fitted
 * to this library's measured kernels on MI355X: launch, HBM stream, matrix
 * rate of the tile family, split-K exchange, and the variant's EC cost).
 * Errors: NULL_POINTER, INVALID_SHAPE, INVALID_ARGUMENT, UNSUPPORTED, HIP.
 */
spear_status_t spear_dispatch_plan(const spear_linear_desc_t* desc, spear_plan_t* plan);

/*
 * spear_schedule_ec -- the SLO-constrained, EC-aware choice for one batch
 * (SPEAR page, abstract: a scheduler that decides under a latency objective
 * where the error compensators run).  For M tokens through the n_layers
 * linears, choose which layers keep their EC so that the predicted latency of
 * the batch (the sum over layers of spear_dispatch_plan's predicted_us with
 * the EC on, predicted_no_ec_us with it off) stays within slo_us, and the
 * total weight of the ECs kept on is the largest possible.  Exact 0/1
 * knapsack over the layers' extra time (EC on minus off), each rounded up to
 * a grid of the slack (as spear_schedule_ec_costs: rounding never breaks the
 * objective); among optimal sets the one that adds the least time.
 *   layers   host array [n_layers]; ec_on  host output [n_layers] (1: keep the
 *            EC; always 0 for rank 0); predicted_us host output (may be NULL):
 *            the batch's predicted latency under the choice.
 *   device_cus  as in spear_linear_desc_t (0: query the current device).
 * When even every EC off exceeds slo_us, all are off and predicted_us says by
 * how much (status SPEAR_OK).  Host only; nothing is enqueued.
 * Errors: NULL_POINTER, INVALID_SHAPE (a layer, M < 1, n_layers < 0),
 *         INVALID_ARGUMENT (slo_us or a weight not finite, weight < 0),
 *         UNSUPPORTED, HIP.
 */
spear_status_t spear_schedule_ec(const spear_sched_layer_t* layers, int32_t n_layers, int32_t M, double slo_us,
                                 int32_t device_cus, uint8_t* ec_on, double* predicted_us);

/*
 * spear_schedule_ec_costs -- the selection step of spear_schedule_ec on costs
 * the caller gives: among the layers i with extra_us[i] >= 0 (a negative extra
 * marks a layer without an EC) and weight[i] > 0, the set of largest total
 * weight whose extra times, each rounded up to the grid unit
 * u = max(slack_us / G, 1e-9), sum to at most min(G, floor(slack_us / u))
 * units, with G = 65536 grid steps for up to 256 layers and
 * max(256, floor(65536 x 256 / n)) beyond (so a call does about 2^24 cell
 * updates and holds one bit per cell); ties go to the set of fewer units.  Weights are summed in layer order.
 * slack_us < 0: nothing is chosen.  ec_on host output [n]; added_us (may be
 * NULL): the chosen extra time.  Host only.
 * Errors: NULL_POINTER, INVALID_SHAPE (n outside [0, 4096]),
 *         INVALID_ARGUMENT (a value not finite, a weight < 0).
 */
spear_status_t spear_schedule_ec_costs(const double* extra_us, const float* weight, int32_t n, double slack_us,
                                       uint8_t* ec_on, double* added_us);

/*
 * spear_w4ec_linear -- Y = X . dequant(Wq, s) + g' (.) ((X . A) . B).
 * SPEAR page, abstract: the low-bit GEMM of a layer whose quantization error
 * is compensated by a small branch that a per-token gate scales, with the
 * work after the branch's projection fused into that GEMM.
 *   desc     the call; plan may be NULL (planned internally) or the result of
 *            spear_dispatch_plan for the same M, K, N, rank and variant.
 *   X        fp16 [M, K], 16-byte aligned.
 *   Wq, scales  from spear_pack_w4 (desc->group_size 0) or spear_pack_w4_grouped
 *            (desc->group_size SPEAR_GROUP_SIZE) (16- and 2-byte aligned).  With group
 *            scales the dequantized weight is q[k, n] s[k / 128, n]: the decode
 *            kernel (M <= 16) sums each 128-k group in fp32 and scales it there,
 *            the tile kernels scale the decoded fp16 weights (fp16(q s)) before
 *            the matrix instructions.
 *   A        fp16 [K, rank], B fp16 [rank, N], w_g fp16 [K] (2-byte aligned;
 *            A and w_g 16-byte aligned for the fused variant); may be NULL when
 *            rank == 0 or the resolved variant is NO_EC.  Inputs must be finite.
 *   Y        output fp16 [M, N] (2-byte aligned), fully overwritten,
 *            fp16(s[n] acc[m,n] + g'[m] sum_j P[m,j] B[j,n]) with fp32
 *            accumulation; must not alias any input.
 *   workspace  device memory of at least plan.workspace_bytes (16-byte
 *            aligned; may be NULL when that is 0).  It must be zero-filled
 *            before its first use.  Its first 1 MiB is a header owned by
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
 * Device-side failure: the fused variants wait, inside the launch, for the
 * EC projection that other workgroups of the same launch publish.  Every such
 * wait is bounded; one that gives up (it never should: the bound is about
 * half a second of polling) lets the call finish with a wrong Y and sets a
 * bit of a sticky error word in the workspace header, which only
 * spear_take_error reads and clears.
 */
spear_status_t spear_w4ec_linear(const spear_linear_desc_t* desc, const spear_plan_t* plan,
                                 const void* X, const void* Wq, const void* scales,
                                 const void* A, const void* B, const void* w_g, void* Y,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * spear_w4ec_linear_noalloc -- spear_w4ec_linear without a caller workspace,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that forbid allocation).  Same arguments and result
 * as spear_w4ec_linear minus workspace and workspace_bytes; it allocates
 * nothing (no hipMalloc, no allocating library call).  Its workspace is the
 * library's own device array of SPEAR_NOALLOC_WORKSPACE_BYTES (64 MiB) per GPU,
 * kept until the process ends; its address is looked up on the first call on
 * each device, which also enqueues on `stream` a small kernel that zeroes the
 * array's 1 MiB header before the call.  That first call must not be made
 * while `stream` is being captured into a graph (it returns SPEAR_ERR_HIP,
 * with nothing enqueued); later calls may be captured.  Every call on one GPU shares that
 * array: calls that overlap in time on one GPU race and must not be issued
 * (order them, e.g. on one stream).  Its sticky error word is read with
 * spear_take_error(NULL, 0, code_out, stream).
 * Errors: as spear_w4ec_linear; WORKSPACE_TOO_SMALL when the plan needs more
 * than SPEAR_NOALLOC_WORKSPACE_BYTES (nothing is enqueued then).
 */
#define SPEAR_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
spear_status_t spear_w4ec_linear_noalloc(const spear_linear_desc_t* desc, const spear_plan_t* plan,
                                         const void* X, const void* Wq, const void* scales,
                                         const void* A, const void* B, const void* w_g, void* Y,
                                         void* stream);

/*
 * spear_ec_project -- the EC projection and gate alone, in one pass over X
 * (the first half of the split variant).  SPEAR page, abstract: the error
 * compensators are lightweight branches whose output a per-token gate
 * scales; the branch's first factor and the gate read the same input.
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
 * spear_take_error -- read and clear the sticky error word of a workspace.
 * Enqueues on `stream` a kernel that writes the word to *code_out (device
 * memory, uint32, 4-byte aligned) and sets it to zero, so the caller reads it
 * after synchronizing the stream.  0: no wait gave up since the word was last
 * cleared.  Bit 0 (1): a fused decode call's wait for the EC producers' hand-off
 * gave up; bit 1 (2): a fused tiled call's wait for an EC row tile's ready
 * flag gave up.  Each set bit means at least one call on this workspace wrote
 * a wrong Y.  Ordered on `stream` like the calls it reports on.
 * workspace and workspace_bytes as passed to spear_w4ec_linear (at least the
 * 1 MiB header); workspace NULL with workspace_bytes 0 reads the word of
 * spear_w4ec_linear_noalloc's workspace on the current device.
 * Errors: NULL_POINTER, WORKSPACE_TOO_SMALL, MISALIGNED, HIP.
 */
spear_status_t spear_take_error(void* workspace, size_t workspace_bytes, void* code_out, void* stream);

/*
 * spear_debug_set_spin_limit -- bound of every cross-workgroup wait of later
 * calls, in polls (process-wide; negative restores the default of 2^20).
 * 0 makes a wait give up at its first unsuccessful poll: a test hook that
 * lets the failure path run with every kernel still ending normally.
 */
void spear_debug_set_spin_limit(int64_t polls);

/*
 * spear_debug_fail_waits -- test hook (process-wide): while `on` is nonzero,
 * every cross-workgroup wait of later fused calls looks for a tag that no
 * workgroup writes, so it runs to its bound (spear_debug_set_spin_limit) and
 * gives up; the kernels still end normally, Y is wrong and the sticky error
 * word is set.  0 restores normal calls.
 */
void spear_debug_fail_waits(int32_t on);

/*
 * spear_debug_stream_read -- a plain streaming read of `bytes` bytes at src
 * (16-byte loads, `grid` workgroups of 256 threads, each reading one
 * contiguous share), with nothing computed but a fold of the loaded words; a
 * measurement aid: the read rate one launch of a given size gets from the
 * memory system, the practical ceiling of the weight stream of a decode call.
 * src 16-byte aligned, bytes a multiple of 16; sink: device memory of `grid`
 * uint32 (written only in the practically impossible case that a fold equals
 * a magic value).
 * Errors: NULL_POINTER, INVALID_SHAPE, MISALIGNED, HIP.
 */
spear_status_t spear_debug_stream_read(const void* src, size_t bytes, int32_t grid, void* sink, void* stream);

/*
 * spear_debug_mfma_rate -- the matrix cores' practical ceiling: one workgroup
 * per CU of the current device, 4 x waves_per_simd waves each, every wave
 * issuing `iterations` rounds of independent fp16 matrix instructions on
 * register operands (shape 0: 8 accumulators of v_mfma_f32_16x16x32_f16, the
 * instruction of this library's tile kernels; shape 1: 4 accumulators of
 * v_mfma_f32_32x32x16_f16).  *flops (host) receives the launch's floating-point
 * operations, so the caller's timing of it gives the rate.  sink: device
 * memory of one float per CU (written only in a practically impossible case).
 * A measurement aid, not part of the layer call.
 * Errors: NULL_POINTER, INVALID_ARGUMENT (shape not 0/1, waves_per_simd not
 *         1/2/4, iterations outside [1, 2^20]), MISALIGNED, HIP.
 */
spear_status_t spear_debug_mfma_rate(int32_t shape, int32_t waves_per_simd, int32_t iterations, void* sink,
                                    void* stream, double* flops);

/*
 * spear_ec_init -- data-free initialisation of the EC factors: A B = the
 * rank-r truncated SVD of the quantization residual E = W - dequant(Wq, s)
 * (SPEAR page, abstract: lightweight compensators of the quantization error;
 * SERQ page, "Saliency-Aware Low-Rank Error Reconstruction for LLM
 * Quantization", Figure 1 and Table 8: a low-rank reconstruction of that error
 * from its singular value decomposition).  The singular values are split
 * evenly, A = U_r diag(sqrt(s)), B = diag(sqrt(s)) V_r^T, and each pair's sign
 * makes the largest-magnitude entry of A's column positive.  Computed by
 * randomized subspace iteration (rank + 16 columns, `iterations` rounds, 0 =
 * 10) in fp32, each block orthonormalized by Cholesky QR applied twice, and a
 * final Rayleigh-Ritz step whose small eigen-problem is solved on the device.
 *   W        fp16 [K, N] (the weight that was packed), 2-byte aligned.
 *   Wq, scales  its packed form (spear_pack_w4: group_size 0; spear_pack_w4_grouped:
 *            group_size SPEAR_GROUP_SIZE).
 *   A        output fp16 [K, rank]; B output fp16 [rank, N] (2-byte aligned).
 *   workspace  device memory of spear_ec_init_workspace_bytes (no clearing
 *            needed; holds E in fp32, K N 4 bytes, and the iteration's blocks).
 * rank <= 112 (the small solvers keep rank + 16 columns in LDS): larger ranks,
 * and K above 2^28 - 1 or N above 2^27 - 1, are UNSUPPORTED (also by
 * spear_ec_init_workspace_bytes).  A weight-preparation step, not part of the layer call.
 * Errors: NULL_POINTER, INVALID_SHAPE, INVALID_ARGUMENT (iterations outside
 *         [0, 64]), UNSUPPORTED, WORKSPACE_TOO_SMALL, MISALIGNED, HIP.
 */
spear_status_t spear_ec_init_workspace_bytes(int32_t K, int32_t N, int32_t rank, size_t* bytes);
spear_status_t spear_ec_init(const void* W, const void* Wq, const void* scales, int32_t K, int32_t N,
                             int32_t group_size, int32_t rank, int32_t iterations, void* A, void* B,
                             void* workspace, size_t workspace_bytes, void* stream);

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
