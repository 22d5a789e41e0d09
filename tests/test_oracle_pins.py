"""The CPU oracle against facts fixed outside it (see tests/oracle_pins.py)."""
import numpy as np
import pytest

import synth
from oracle import act_ref, sherry_ref, tern2_ref, tern3_ref
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", [
    P.pin_bijection, P.pin_code_table, P.pin_packed_groups, P.pin_row_layout, P.pin_straddles, P.pin_size,
    P.pin_ramp_dot, P.pin_closed_forms, P.pin_brute_force, P.pin_packer, P.pin_epilogue,
    P.pin_bf16_path, P.pin_bf16_wide_range, P.pin_gemm_bf16,
], ids=lambda f: f.__name__)
def test_pin(pin):
    pin(sherry_ref)


def test_vectorised_matches_scalar_routines():
    g = synth.rng(3)
    n, k = 11, 640
    words = synth.random_words(n * (k // 128) * 5, g)
    codes = sherry_ref.unpack_codes(words, n, k)
    d = sherry_ref.group_words(words, n, k)
    G = k // 128
    for r in range(n):
        for grp in range(G):
            w5 = [words[5 * G * r + 4 * grp + i] for i in range(4)] + [words[5 * G * r + 4 * G + grp]]
            assert d[r, grp].tolist() == [int(v) for v in w5]
            assert sherry_ref.unpack_group(w5) == codes[r, grp * 32:(grp + 1) * 32].tolist()
    assert np.array_equal(sherry_ref.pack_codes(codes), words)
    dense = sherry_ref.dense_from_codes(codes)
    for r in range(0, n, 3):
        for j in range(0, k // 4, 7):
            assert tuple(dense[r, 4 * j:4 * j + 4]) == sherry_ref.decode_block(int(codes[r, j]))
    assert np.array_equal(sherry_ref.codes_from_dense(dense), codes)


def test_quantize_matches_scalar_block_rule():
    g = synth.rng(5)
    w = g.standard_normal((4, 256)).astype(np.float32)
    w[0, :8] = [0.5, -0.5, 0.5, 0.5, -0.0, 0.0, 1.0, -1.0]
    codes, _ = sherry_ref.quantize(w)
    for r in range(4):
        for j in range(64):
            assert int(codes[r, j]) == sherry_ref.quantize_block(w[r, 4 * j:4 * j + 4])


def test_errors():
    with pytest.raises(ValueError):
        sherry_ref.check_shape(4, 100)
    with pytest.raises(ValueError):
        sherry_ref.decode_block(32)
    with pytest.raises(ValueError):
        sherry_ref.encode_block((1, 1, 1, 1))
    with pytest.raises(ValueError):
        sherry_ref.codes_from_dense(np.zeros((1, 128), np.int8))
    with pytest.raises(ValueError):
        sherry_ref.quantize(np.full((1, 128), np.nan))
    with pytest.raises(ValueError):
        tern2_ref.decode_word(0b10)


def test_tern2_hand_words():
    # R8 by hand: weight 0 at bits 0-1, weight 1 at bits 8-9, weight 4 at bits 2-3,
    # weight 15 (q=3, p=3) at bits 30-31.
    # (+1, -1, 0, ...) -> 01 | 11 << 8 = 0x301
    assert tern2_ref.encode_word([1, -1] + [0] * 14) == 0x301
    assert tern2_ref.encode_word([0] * 4 + [-1] + [0] * 11) == 0xC
    assert tern2_ref.encode_word([0] * 15 + [1]) == 0x40000000
    # a shift by 2q and mask 0x03030303 yields weights 4q..4q+3, one per byte
    t16 = [1, -1, 0, 1, 0, 0, -1, 1, -1, -1, 1, 0, 1, 1, 1, -1]
    w = tern2_ref.encode_word(t16)
    for q in range(4):
        sel = (w >> (2 * q)) & 0x03030303
        got = [{0: 0, 1: 1, 3: -1}[(sel >> (8 * p)) & 3] for p in range(4)]
        assert got == t16[4 * q:4 * q + 4]
    assert tern2_ref.encode_word([-1] * 16) == 0xFFFFFFFF
    assert tern2_ref.encode_word([1] * 16) == 0x55555555
    assert tern2_ref.decode_word(0x55555555) == [1] * 16
    g = synth.rng(9)
    t = synth.ternary_dense(5, 256, g)
    words = tern2_ref.pack(t)
    assert words.nbytes == tern2_ref.packed_bytes(5, 256) == 5 * 256 // 4
    assert np.array_equal(tern2_ref.unpack(words, 5, 256), t)
    for r in range(5):
        for i in range(16):
            assert tern2_ref.decode_word(words[r * 16 + i]) == t[r, 16 * i:16 * i + 16].tolist()


def test_tern2_pack_weights():
    """Reading R8b: the 2-bit packer keeps the 3:4 quantizer's decisions and
    scales.  Hand row: block 0 = (0.5, -0.1, 2.0, -3.0) -> zero at slot 1,
    (+1, 0, +1, -1); every other block is all zeros -> zero at slot 0 (lowest
    slot on ties), (0, +1, +1, +1).  Word 0 holds blocks 0-3, block q's weight
    p at bits 8p + 2q: 0x03010001 | 0x04040400 | 0x10101000 | 0x40404000;
    words of four zero blocks: 0x01010100 | 0x04040400 | 0x10101000 |
    0x40404000.  Scale: kept magnitudes 0.5 + 2 + 3 over 3 * 128 / 4 = 96."""
    w = np.zeros((1, 128), np.float32)
    w[0, :4] = [0.5, -0.1, 2.0, -3.0]
    words, s = tern2_ref.pack_weights(w, np.float32)
    assert int(words[0]) == 0x57555401
    assert all(int(v) == 0x55555500 for v in words[1:])
    assert s[0] == np.float32(5.5 / 96)
    # W = s T with T 3:4 ternary: the words of T and the scale s exactly
    g = synth.rng(31)
    t = synth.ternary_34(6, 256, g)
    sc = synth.row_scales(6, g, np.float32)
    words, s2 = tern2_ref.pack_weights(t.astype(np.float32) * sc[:, None], np.float32)
    assert np.array_equal(words, tern2_ref.pack(t)) and np.array_equal(s2, sc)


def test_sherry_and_tern2_agree_on_the_same_matrix():
    """Two encodings of one ternary matrix give one product, bit for bit."""
    g = synth.rng(13)
    n, k, m = 48, 512, 3
    t = synth.ternary_34(n, k, g)
    sw = synth.row_scales(n, g, np.float16)
    xq, sx, _ = synth.act_absmax_int8(m, k, g)
    w5 = sherry_ref.pack_codes(sherry_ref.codes_from_dense(t))
    w2 = tern2_ref.pack(t)
    a5, y5 = sherry_ref.gemm_i8(w5, sw, n, k, xq, sx)
    a2, y2 = tern2_ref.gemm_i8(w2, sw, n, k, xq, sx)
    assert np.array_equal(a5, a2) and np.array_equal(y5.view(np.uint16), y2.view(np.uint16))
    b5, z5 = sherry_ref.gemv_i8(w5, sw, n, k, xq[0], sx[0])
    b2, z2 = tern2_ref.gemv_i8(w2, sw, n, k, xq[0], sx[0])
    assert np.array_equal(b5, b2) and np.array_equal(z5.view(np.uint16), z2.view(np.uint16))
    assert np.array_equal(b5, a5[0])


def test_accumulator_bound_at_largest_shape():
    """The largest reduction (k = 8192) with x = +-127 stays far inside int32
    and inside fp32's exact-integer range (2^24)."""
    k = 8192
    assert 127 * 3 * k // 4 < 2 ** 24
    t = np.zeros((1, k), np.int8)
    t[0] = np.tile([0, 1, 1, 1], k // 4)
    words = sherry_ref.pack_codes(sherry_ref.codes_from_dense(t))
    acc, _ = sherry_ref.gemv_i8(words, np.ones(1, np.float32), 1, k, np.full(k, 127, np.int8), None, np.float32)
    assert int(acc[0]) == 127 * 3 * k // 4


@pytest.mark.parametrize("pin", P.ACT_PINS, ids=lambda f: f.__name__)
def test_act_pin(pin):
    pin(act_ref)


@pytest.mark.parametrize("pin", P.T3_PINS, ids=lambda f: f.__name__)
def test_t3_pin(pin):
    pin(tern3_ref)
