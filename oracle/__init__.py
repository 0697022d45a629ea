"""Oracle for the SPEAR W4 linear layer with a per-token-gated Error Compensator.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
CPU implementation (NumPy, float64 unless a step fixes another precision) of
what the HIP path computes.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The HIP library
and its Python binding never import it, and it imports nothing from them.

Source of the method: "SPEAR: A System for Post-Quantization Error-Adaptive
Recovery Enabling Efficient Low-Bit LLM Serving" (arXiv 2606.11244),
abstract.  The page describes 4-bit weights with one scale per output channel,
small error-compensating branches (ECs) whose output a per-token gate scales,
and the second half of that branch computed inside the low-bit GEMM.  It gives
no formulas; the layer computed here is

    Y = X . dequant(Wq, s) + g (.) ((X . A) . B),   g = sigmoid(X . w_g + b_g)

with a symmetric int4 per-output-channel quantizer (s = max|w| / 7) and
rank-r fp16 factors A [K, r], B [r, N].  Every reading of a step the abstract
leaves open is listed in the module that implements it.

Pins (tests marked ``not gpu``):
  * pack/unpack: exhaustive round trip over all 16 codes at all 8 nibble
    positions; hand-written golden words; the tiled layout is a bijection and
    each lane slot holds the k-octet the matrix instruction reads.
  * scale/quantize: exhaustive fp16 check that the fp32 decisions equal the
    fp64 ones; |w - q s| <= s/2; grid weights w = s q quantize back to q;
    zero and subnormal-scale columns.
  * group-wise scales (g128): one group spanning K reproduces the per-channel
    quantizer bit for bit; a brute-force per-element loop; the s/2 bound and
    grid weights per group; a group of zeros; the layer at g = 0 against the
    textbook matmul with the group-dequantized weight.
  * gate: closed forms (g(0) = 1/2, g(-z) = 1 - g(z)), saturation at +-1e4,
    agreement with scipy.special.expit.
  * layer: g = 0 reduces to the textbook W4 GEMM; g = 1 reduces to a static
    dense correction X (q s + A B); brute-force scalar loops on tiny shapes;
    exactly rounded sums (math.fsum) at sampled outputs; linearity in g.

The scheduler's selection step (``oracle.spear_sched``, a submodule): every
subset of the candidate layers enumerated under the documented grid rule;
pinned by hand-worked instances, special cases, monotonicity in the slack and
scipy's MILP solver on the same integer knapsack.

The data-free EC initialisation (``oracle.spear_ec_init``): the rank-r
truncated SVD of the quantization residual; pinned by the Eckart-Young error,
the eigenvectors of E^T E (an independent algorithm), a residual of known
singular structure, the balanced split, an exactly zero residual on a grid
weight, and the falling gate-1 error as the rank grows.

Parity unpinned: none of the functions here.  The quality claim of the
abstract (perplexity-gap recovery) is outside this oracle.
"""

from .spear_oracle import (  # noqa: F401
    LAYOUT_ID,
    K_CHUNK,
    N_BLOCK,
    padded_dims,
    packed_words,
    channel_scales,
    quantize,
    pack_canonical,
    unpack_canonical,
    NIBBLE_K,
    interleave_nibbles,
    deinterleave_nibbles,
    place_words,
    unplace_words,
    tile_words,
    untile_words,
    pack_w4,
    unpack_w4,
    dequant,
    group_scales,
    quantize_grouped,
    pack_w4_grouped,
    dequant_grouped,
    gate_logits,
    gate,
    ec_project,
    w4ec_linear,
    rel_l2,
    max_abs_over_rms,
)
