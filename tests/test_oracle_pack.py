"""Pins of the oracle's quantizer and bit packing (CPU only).

The quantizer follows the SPEAR page's 4-bit, one-scale-per-output-channel
setting (abstract) with the symmetric reading s = fp16(max|w| / 7),
q = clamp(rint(w / s), -7, 7).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_words.json")


def all_fp16_positive_finite():
    bits = np.arange(1, 0x7C00, dtype=np.uint16)          # +subnormals and normals
    return bits.view(np.float16)


# ---------------------------------------------------------------- packing

def test_canonical_round_trip_every_code_every_position():
    for pos in range(8):
        for code in range(16):
            q = np.zeros((8, 1), dtype=np.int64)
            q[pos, 0] = code - 8
            w = oracle.pack_canonical(q)
            assert int(w[0, 0]) == (code << (4 * pos)) | (0x88888888 & ~(0xF << (4 * pos)))
            back = oracle.unpack_canonical(w)
            assert back[pos, 0] == code - 8
            assert np.all(np.delete(back[:, 0], pos) == 0)


def test_canonical_random_words_round_trip():
    rng = np.random.default_rng(7)
    words = rng.integers(0, 2 ** 32, size=(1000, 1000), dtype=np.uint64).astype(np.uint32)
    q = oracle.unpack_canonical(words)
    assert q.min() >= -8 and q.max() <= 7
    assert np.array_equal(oracle.pack_canonical(q), words)


def test_golden_canonical_words():
    with open(GOLDEN) as f:
        g = json.load(f)
    for ex in g["canonical_examples"]:
        q = np.array(ex["q"], dtype=np.int64).reshape(8, 1)
        assert int(oracle.pack_canonical(q)[0, 0]) == int(ex["word"], 16), ex


def test_golden_interleaved_words():
    with open(GOLDEN) as f:
        g = json.load(f)
    for ex in g["interleave_examples"]:
        c = np.array([int(ex["canonical"], 16)], dtype=np.uint32)
        i = oracle.interleave_nibbles(c)
        assert int(i[0]) == int(ex["interleaved"], 16), ex
        assert int(oracle.deinterleave_nibbles(i)[0]) == int(c[0])


def test_interleave_gives_fp16_pairs_in_k_order():
    """(word >> 4j) & 0x000F000F must hold k-offset 2j in the low half and
    2j+1 in the high half: OR-ing 0x6400 makes each half the fp16 1024 + u."""
    rng = np.random.default_rng(12)
    for _ in range(200):
        u = rng.integers(0, 16, size=8)
        canon = np.array([sum(int(u[k]) << (4 * k) for k in range(8))], dtype=np.uint32)
        w = int(oracle.interleave_nibbles(canon)[0])
        for j in range(4):
            pair = ((w >> (4 * j)) & 0x000F000F) | 0x64006400
            lo = np.array([pair & 0xFFFF], dtype=np.uint16).view(np.float16)[0]
            hi = np.array([pair >> 16], dtype=np.uint16).view(np.float16)[0]
            assert float(lo) - 1032 == u[2 * j] - 8 and float(hi) - 1032 == u[2 * j + 1] - 8


def test_golden_tiled_indexes():
    with open(GOLDEN) as f:
        g = json.load(f)
    for ex in g["tiled_examples"]:
        K, N = ex["K"], ex["N"]
        words = np.zeros((K // 8, N), dtype=np.uint32)
        words[ex["k8"], ex["n"]] = 0xDEADBEEF
        flat = oracle.place_words(words, K, N)
        assert flat.size == ex["total_words"] == oracle.packed_words(K, N)
        hits = np.nonzero(flat == 0xDEADBEEF)[0]
        assert list(hits) == [ex["index"]], ex


@pytest.mark.parametrize("K,N", [(8, 1), (128, 16), (136, 20), (512, 48), (4096, 16)])
def test_tiling_is_bijection_and_pads_with_zero_code(K, N):
    rng = np.random.default_rng(K * 1000 + N)
    words = rng.integers(0, 2 ** 32, size=(K // 8, N), dtype=np.uint64).astype(np.uint32)
    flat = oracle.tile_words(words, K, N)
    assert np.array_equal(oracle.untile_words(flat, K, N), words)
    assert np.array_equal(oracle.unplace_words(oracle.place_words(words, K, N), K, N), words)
    kp, npad = oracle.padded_dims(K, N)
    assert flat.size == kp * npad // 8
    # positions that hold real words: where a permutation of 1..n lands
    ident = np.arange(1, words.size + 1, dtype=np.uint32).reshape(words.shape)
    landed = oracle.place_words(ident, K, N)
    real = landed != 0x88888888
    assert real.sum() == words.size
    assert np.array_equal(np.sort(landed[real]), np.arange(1, words.size + 1))
    # every padding word decodes to q = 0 in all 8 nibbles
    assert np.all(flat[~real] == 0x88888888)


def test_tile_slot_holds_matrix_instruction_b_operand():
    """Lane L of a 16x16x32 fp16 matrix instruction reads, as its B operand, 8
    consecutive k (8*(L//16) .. +7 inside the 32-k block) of column L%16; the
    16-byte slot L of each 1 KiB tile must hold those octets for the 4 blocks."""
    K, N = 384, 48
    rng = np.random.default_rng(3)
    q = rng.integers(-8, 8, size=(K, N))
    flat = oracle.tile_words(oracle.pack_canonical(q), K, N).reshape(N // 16, K // 128, 64, 4)
    for nb in range(N // 16):
        for kc in range(K // 128):
            for lane in range(64):
                for j in range(4):
                    word = int(flat[nb, kc, lane, j])
                    kb = kc * 4 + j
                    col = nb * 16 + lane % 16
                    for e in range(8):
                        k = kb * 32 + 8 * (lane // 16) + e
                        field = e // 2 if e % 2 == 0 else 4 + e // 2
                        assert ((word >> (4 * field)) & 0xF) - 8 == q[k, col]


# ---------------------------------------------------------------- scales

def test_scale_fp32_division_equals_fp64_for_every_fp16():
    m = all_fp16_positive_finite()
    s32 = (m.astype(np.float32) / np.float32(7)).astype(np.float16)
    s64 = (m.astype(np.float64) / 7.0).astype(np.float16)
    assert np.array_equal(s32.view(np.uint16), s64.view(np.uint16))


def test_channel_scales_match_column_max():
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((64, 24)) * 0.02).astype(np.float16)
    s = oracle.channel_scales(W)
    expect = (np.abs(W.astype(np.float64)).max(axis=0) / 7.0).astype(np.float16)
    assert np.array_equal(s.view(np.uint16), expect.view(np.uint16))


# ---------------------------------------------------------------- quantizer

def _decisions(w, s):
    r32 = np.rint(w.astype(np.float32) / s.astype(np.float32))
    r64 = np.rint(w.astype(np.float64) / s.astype(np.float64))
    return r32.astype(np.float64), r64


def test_ratio_rounding_fp32_equals_fp64_exhaustive_by_binade():
    """The exact ratio w/s depends only on the mantissas and the exponent gap, so
    s over the binade [1, 2) with every fp16 w in [0, 7.6 s], plus every
    subnormal s with every w in [0, 10.5 s], covers every pair that can occur."""
    allpos = np.concatenate([[np.float16(0)], all_fp16_positive_finite()])
    bad = 0
    s_binade = (np.arange(0x3C00, 0x4000, dtype=np.uint16)).view(np.float16)
    for s in s_binade:
        w = allpos[allpos.astype(np.float64) <= 7.6 * float(s)]
        a, b = _decisions(w, np.full(w.shape, s))
        bad += int(np.count_nonzero(a != b))
    s_sub = np.arange(1, 0x0400, dtype=np.uint16).view(np.float16)
    for s in s_sub:
        w = allpos[allpos.astype(np.float64) <= 10.5 * float(s)]
        a, b = _decisions(w, np.full(w.shape, s))
        bad += int(np.count_nonzero(a != b))
    assert bad == 0


def test_ties_round_half_even():
    s = np.array([1.0], dtype=np.float16)
    W = np.array([[0.5], [1.5], [2.5], [-0.5], [-1.5], [-2.5], [3.5], [6.5]], dtype=np.float16)
    q = oracle.quantize(W, s)
    assert list(q[:, 0]) == [0, 2, 2, 0, -2, -2, 4, 6]


def test_quantization_error_at_most_half_step():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((256, 64)) * 0.02).astype(np.float16)
    s = oracle.channel_scales(W)
    q = oracle.quantize(W, s)
    err = np.abs(W.astype(np.float64) - q * s.astype(np.float64)[None, :])
    assert np.all(err <= s.astype(np.float64)[None, :] / 2 * (1 + 1e-12))
    # the column maximum maps to +-7
    idx = np.argmax(np.abs(W.astype(np.float64)), axis=0)
    assert np.all(np.abs(q[idx, np.arange(64)]) == 7)


def test_grid_weights_quantize_back_exactly():
    """W = s q with s a power of two and max |q| = 7 per column: the quantizer
    must return that s and that q, so a wrong divisor, offset or sign fails."""
    rng = np.random.default_rng(9)
    K, N = 96, 40
    q = rng.integers(-7, 8, size=(K, N))
    q[rng.integers(0, K, N), np.arange(N)] = rng.choice([-7, 7], N)
    e = rng.integers(-10, -3, size=N)
    s_true = np.ldexp(1.0, e)
    W = (q * s_true[None, :]).astype(np.float16)
    assert np.array_equal(W.astype(np.float64), q * s_true[None, :])
    Wq, s = oracle.pack_w4(W)
    assert np.array_equal(s.astype(np.float64), s_true)
    assert np.array_equal(oracle.unpack_w4(Wq, K, N), q)
    assert np.array_equal(oracle.dequant(Wq, s, K, N), W.astype(np.float64))


def test_zero_column_and_subnormal_scale_clamp():
    W = np.zeros((8, 3), dtype=np.float16)
    # column 1: max |w| = 17 * 2^-24 -> s = fp16(17 * 2^-24 / 7) = 2 * 2^-24 ->
    # 17 / 2 = 8.5 -> rint 8 -> clamped to 7; 5 * 2^-24 / (2 * 2^-24) = 2.5 -> 2
    tiny = np.float16(2.0 ** -24)
    W[0, 1] = tiny * 17
    W[1, 1] = -tiny * 17
    W[2, 1] = tiny * 5
    W[3, 2] = np.float16(0.25)
    s = oracle.channel_scales(W)
    assert float(s[0]) == 0.0
    assert float(s[1]) == float(tiny * 2)
    q = oracle.quantize(W, s)
    assert list(q[:, 0]) == [0] * 8
    assert list(q[:4, 1]) == [7, -7, 2, 0]
    assert q[3, 2] == 7
