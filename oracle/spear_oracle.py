"""Plain CPU definition of the SPEAR W4+EC linear layer (test infrastructure only).

Method source: "SPEAR: A System for Post-Quantization Error-Adaptive Recovery
Enabling Efficient Low-Bit LLM Serving" (arXiv 2606.11244), Abstract: W4
per-channel weight quantization, lightweight Error Compensators (ECs)
modulated by per-token gates, post-EC computation fused into the low-bit
GEMM.  The abstract fixes no formula, no quantizer detail and no bit layout;
the readings taken here are stated at each function.

Shapes: X [M, K] fp16, W [K, N] fp16 (input dimension first), A [K, r] fp16,
B [r, N] fp16, w_g [K] fp16, b_g a float32 scalar, Y [M, N].

Nothing here is blocked, fused or reordered beyond the definition; library
primitives used as steps: numpy matmul/dot (float64), numpy exp.
"""

import numpy as np

# Packed-weight layout produced by spear_pack_w4 (layout id 2, "panel tiled").
LAYOUT_ID = 2
K_CHUNK = 128   # k extent of one 1 KiB tile
N_BLOCK = 16    # column extent of one panel
_QMAX = 7       # symmetric int4: codes -7..7 (SPEAR page, abstract: 4-bit, per channel)


def padded_dims(K, N):
    """(K_pad, N_pad): K rounded up to 128, N rounded up to 16."""
    return -(-K // K_CHUNK) * K_CHUNK, -(-N // N_BLOCK) * N_BLOCK


def packed_words(K, N):
    """Number of uint32 words the packed weight occupies."""
    kp, np_ = padded_dims(K, N)
    return kp * np_ // 8


# --------------------------------------------------------------------------
# Quantizer.  Abstract: "per-channel quantization settings", "W4".
# Reading: symmetric int4 with one scale per output channel n,
# s[n] = fp16(max_k |W[k, n]| / 7), q = clamp(rint(W / s), -7, 7), q = 0 where
# s = 0.  The two rounding decisions (scale to fp16, ratio to an integer) are
# taken in float32 with correctly rounded division, the precision the kernel
# uses; the tests show exhaustively that float64 gives the same decisions.
# --------------------------------------------------------------------------

def channel_scales(W):
    """fp16 per-output-channel scales of W [K, N] fp16."""
    W = np.asarray(W, dtype=np.float16)
    colmax = np.max(np.abs(W.astype(np.float32)), axis=0)        # exact
    ratio = colmax / np.float32(_QMAX)                           # fp32, RNE
    return ratio.astype(np.float16)                              # fp32 -> fp16 RNE


def quantize(W, s):
    """int8 codes q [K, N] in [-7, 7] of W [K, N] fp16 under scales s [N] fp16."""
    W = np.asarray(W, dtype=np.float16).astype(np.float32)
    s32 = np.asarray(s, dtype=np.float16).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = W / s32[None, :]                                 # fp32 division
    q = np.rint(ratio)                                           # half to even
    q = np.clip(q, -_QMAX, _QMAX)
    q = np.where(s32[None, :] == 0, 0.0, q)
    return q.astype(np.int8)


# --------------------------------------------------------------------------
# Bit packing.  Reading (the pages are silent): offset binary u = q + 8 in
# [0, 15]; eight consecutive k of one column in one uint32, k ascending from
# bit 0 ("canonical" word (k8, n)).  Code 0 (q = -8) is decodable though the
# quantizer never produces it.
# --------------------------------------------------------------------------

def pack_canonical(q):
    """q [K, N] ints in [-8, 7], K % 8 == 0 -> words [K/8, N] uint32."""
    q = np.asarray(q, dtype=np.int64)
    K, N = q.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    u = (q + 8).astype(np.uint32)
    if np.any(u > 15):
        raise ValueError("code out of range")
    words = np.zeros((K // 8, N), dtype=np.uint32)
    for i in range(8):
        words |= u[i::8, :] << np.uint32(4 * i)
    return words


def unpack_canonical(words):
    """words [K/8, N] uint32 -> q [K, N] int8."""
    words = np.asarray(words, dtype=np.uint32)
    K8, N = words.shape
    q = np.empty((K8 * 8, N), dtype=np.int8)
    for i in range(8):
        q[i::8, :] = ((words >> np.uint32(4 * i)) & np.uint32(0xF)).astype(np.int8) - 8
    return q


# --------------------------------------------------------------------------
# Tiled layout (layout id 2).  Two steps on the canonical words:
# (1) nibble interleave inside each word: bit field i (bits 4i..4i+3) holds
#     k-offset NIBBLE_K[i] = (0, 2, 4, 6, 1, 3, 5, 7)[i], so that the 16-bit
#     halves of (word >> 4j) & 0x000F000F are the codes of k-offsets 2j and
#     2j+1, in that order;
# (2) placement: K is padded to K_pad (multiple of 128) and N to N_pad
#     (multiple of 16) with code 8 (q = 0), and word (k8, n) goes to
#         nb = n // 16, c = n % 16, kc = k8 // 16, j = (k8 % 16) // 4, t = k8 % 4
#         index = ((nb * (K_pad/128) + kc) * 64 + (t * 16 + c)) * 4 + j
#     so each 16-column panel is contiguous over K, and in every 1 KiB tile
#     (16 columns x 128 k) the 16 bytes at slot L = t*16 + c hold, for the four
#     32-k blocks j, the k-octet t of column c: the B operand a 64-lane
#     16x16x32 matrix instruction takes from lane L.
# --------------------------------------------------------------------------

NIBBLE_K = (0, 2, 4, 6, 1, 3, 5, 7)


def interleave_nibbles(words):
    """Canonical words (k-offset i in field i) -> interleaved (NIBBLE_K order)."""
    words = np.asarray(words, dtype=np.uint32)
    out = np.zeros_like(words)
    for field, koff in enumerate(NIBBLE_K):
        out |= ((words >> np.uint32(4 * koff)) & np.uint32(0xF)) << np.uint32(4 * field)
    return out


def deinterleave_nibbles(words):
    """Inverse of interleave_nibbles."""
    words = np.asarray(words, dtype=np.uint32)
    out = np.zeros_like(words)
    for field, koff in enumerate(NIBBLE_K):
        out |= ((words >> np.uint32(4 * field)) & np.uint32(0xF)) << np.uint32(4 * koff)
    return out


def place_words(words_c, K, N):
    """Words [K/8, N] -> flat array in the tiled placement (padded with code 8)."""
    kp, np_ = padded_dims(K, N)
    full = np.full((kp // 8, np_), 0x88888888, dtype=np.uint32)
    full[: K // 8, :N] = words_c
    kc_n, nb_n = kp // K_CHUNK, np_ // N_BLOCK
    t5 = full.reshape(kc_n, 4, 4, nb_n, 16)          # [kc, j, t, nb, c]
    return np.ascontiguousarray(t5.transpose(3, 0, 2, 4, 1)).reshape(-1)  # [nb, kc, t, c, j]


def unplace_words(flat, K, N):
    """Inverse of place_words (padding dropped)."""
    kp, np_ = padded_dims(K, N)
    kc_n, nb_n = kp // K_CHUNK, np_ // N_BLOCK
    flat = np.asarray(flat, dtype=np.uint32)
    if flat.size != kp * np_ // 8:
        raise ValueError("packed size mismatch")
    t5 = flat.reshape(nb_n, kc_n, 4, 16, 4)           # [nb, kc, t, c, j]
    full = t5.transpose(1, 4, 2, 0, 3).reshape(kp // 8, np_)
    return np.ascontiguousarray(full[: K // 8, :N])


def tile_words(words_c, K, N):
    """Canonical words [K/8, N] -> flat layout-2 array (interleave, then place)."""
    return place_words(interleave_nibbles(words_c), K, N)


def untile_words(flat, K, N):
    """Flat layout-2 array -> canonical words [K/8, N]."""
    return deinterleave_nibbles(unplace_words(flat, K, N))


def pack_w4(W):
    """W [K, N] fp16 -> (Wq flat uint32 in layout 2, s [N] fp16)."""
    W = np.asarray(W, dtype=np.float16)
    K, N = W.shape
    s = channel_scales(W)
    q = quantize(W, s)
    return tile_words(pack_canonical(q), K, N), s


def unpack_w4(Wq, K, N):
    """Layout-2 words -> q [K, N] int8."""
    return unpack_canonical(untile_words(Wq, K, N))


def dequant(Wq, s, K, N):
    """dequant(Wq, s) [K, N] float64 = q * s, exact (never rounded to fp16)."""
    q = unpack_w4(Wq, K, N).astype(np.float64)
    return q * np.asarray(s, dtype=np.float16).astype(np.float64)[None, :]


# --------------------------------------------------------------------------
# Group-wise quantizer (the W4 variant next to per-channel scales).  The
# abstract calls per-channel quantization the challenging setting, which
# places it against the usual alternative, one scale per group of input rows
# of each column.  Reading: groups of `group` consecutive k (128 here, the
# common choice, and the k extent of one packed tile), the last group possibly
# shorter; s[g, n] = fp16(max_{k in group g} |W[k, n]| / 7) and
# q[k, n] = clamp(rint(W[k, n] / s[k // group, n]), -7, 7), q = 0 where the
# group's s = 0; the same fp32 decisions as the per-channel quantizer, one
# group at a time.  The codes are packed exactly as in layout 2; only the
# scales change shape, to [ceil(K / group), N].
# --------------------------------------------------------------------------

def group_scales(W, group):
    """fp16 scales s [ceil(K / group), N] of W [K, N] fp16, one per group of
    `group` consecutive rows and column."""
    W = np.asarray(W, dtype=np.float16)
    K, N = W.shape
    G = -(-K // group)
    out = np.empty((G, N), dtype=np.float16)
    for g in range(G):
        out[g] = channel_scales(W[g * group: (g + 1) * group])
    return out


def quantize_grouped(W, s, group):
    """int8 codes q [K, N] of W [K, N] under group scales s [ceil(K/group), N]."""
    W = np.asarray(W, dtype=np.float16)
    K, N = W.shape
    q = np.empty((K, N), dtype=np.int8)
    for g in range(np.asarray(s).shape[0]):
        q[g * group: (g + 1) * group] = quantize(W[g * group: (g + 1) * group], np.asarray(s)[g])
    return q


def pack_w4_grouped(W, group=128):
    """W [K, N] fp16 -> (Wq flat uint32 in layout 2, s [ceil(K/group), N] fp16)."""
    W = np.asarray(W, dtype=np.float16)
    K, N = W.shape
    s = group_scales(W, group)
    q = quantize_grouped(W, s, group)
    return tile_words(pack_canonical(q), K, N), s


def dequant_grouped(Wq, s, K, N, group):
    """q * s[k // group, n] [K, N] float64, exact."""
    q = unpack_w4(Wq, K, N).astype(np.float64)
    s64 = np.asarray(s, dtype=np.float16).astype(np.float64)
    rows = np.arange(K) // group
    return q * s64[rows, :]


# --------------------------------------------------------------------------
# Gate.  Abstract: ECs "modulated by per-token gates".  Reading: one scalar
# per token, g = sigmoid(X . w_g + b_g), from the layer's own fp16 input.
# Optional skip threshold tau: g' = g if g >= tau else 0 (tau = 0: g' = g).
# The skip decision is compared through the float32 gate, the kernel's
# precision; tokens whose logit lies within `band` of logit(tau) are reported
# as ambiguous (both decisions are correct up to accumulation order).
# --------------------------------------------------------------------------

def gate_logits(X, w_g, b_g):
    """z [M] float64 = X . w_g + b_g."""
    X64 = np.asarray(X, dtype=np.float16).astype(np.float64)
    w64 = np.asarray(w_g, dtype=np.float16).astype(np.float64)
    return X64 @ w64 + float(np.float32(b_g))


def gate(z, tau=0.0, band=1e-3):
    """Returns (g, g_eff, ambiguous): g = 1/(1+exp(-z)) in float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        g = 1.0 / (1.0 + np.exp(-z))
    tau = float(np.float32(tau))
    if tau <= 0.0:
        return g, g.copy(), np.zeros(z.shape, dtype=bool)
    with np.errstate(over="ignore"):
        g32 = (np.float32(1.0) / (np.float32(1.0) + np.exp(-z.astype(np.float32)))).astype(np.float32)
    keep = g32 >= np.float32(tau)
    g_eff = np.where(keep, g, 0.0)
    if tau >= 1.0:
        ambiguous = np.zeros(z.shape, dtype=bool)
    else:
        ambiguous = np.abs(z - np.log(tau / (1.0 - tau))) <= band
    return g, g_eff, ambiguous


def ec_project(X, A, w_g, b_g):
    """EC projection and gate logit in one pass over X: (P [M, r], z [M])."""
    X64 = np.asarray(X, dtype=np.float16).astype(np.float64)
    P = X64 @ np.asarray(A, dtype=np.float16).astype(np.float64)
    return P, gate_logits(X, w_g, b_g)


def w4ec_linear(X, Wq, s, A, B, w_g, b_g, tau=0.0, K=None, N=None, gate_override=None, W_deq=None,
                group=None):
    """Y [M, N] float64 (unrounded) of the gated W4+EC linear layer.

    Y = X dequant(Wq, s) + diag(g') (X A) B, where dequant is q diag(s) for
    per-channel scales s [N] (group None) and q * s[k // group, n] for group
    scales s [ceil(K/group), N].  With rank 0 (A or B None or r = 0) the EC
    term is absent.  `gate_override` replaces g' (tests only).  `W_deq`, if
    given, must be that dequantized weight computed beforehand (the weight
    preparation done once per weight); it is used as the product.
    Returns (Y, info) with info = {"z", "g", "g_eff", "ambiguous", "P"}.
    """
    X = np.asarray(X, dtype=np.float16)
    M, Kx = X.shape
    K = Kx if K is None else K
    if N is None:
        N = np.asarray(s).shape[-1]
    X64 = X.astype(np.float64)
    if W_deq is None:
        W_deq = dequant(Wq, s, K, N) if group is None else dequant_grouped(Wq, s, K, N, group)
    Y = X64 @ W_deq
    info = {"z": None, "g": None, "g_eff": None, "ambiguous": np.zeros(M, bool), "P": None}
    r = 0 if (A is None or B is None) else np.asarray(A).shape[1]
    if r > 0:
        P, z = ec_project(X, A, w_g, b_g)
        g, g_eff, amb = gate(z, tau)
        if gate_override is not None:
            g_eff = np.asarray(gate_override, dtype=np.float64)
        Y = Y + g_eff[:, None] * (P @ np.asarray(B, dtype=np.float16).astype(np.float64))
        info.update(z=z, g=g, g_eff=g_eff, ambiguous=amb, P=P)
    return Y, info


# --------------------------------------------------------------------------
# Comparison metrics (tolerance: relative L2 <= 1e-3, max-abs <= 1e-2 rms(Y)).
# --------------------------------------------------------------------------

def rel_l2(Y_test, Y_ref):
    Y_test = np.asarray(Y_test, dtype=np.float64)
    Y_ref = np.asarray(Y_ref, dtype=np.float64)
    den = np.linalg.norm(Y_ref)
    num = np.linalg.norm(Y_test - Y_ref)
    return num / den if den > 0 else num


def max_abs_over_rms(Y_test, Y_ref):
    Y_test = np.asarray(Y_test, dtype=np.float64)
    Y_ref = np.asarray(Y_ref, dtype=np.float64)
    rms = np.sqrt(np.mean(Y_ref ** 2)) if Y_ref.size else 0.0
    err = np.max(np.abs(Y_test - Y_ref)) if Y_ref.size else 0.0
    return err / rms if rms > 0 else err
