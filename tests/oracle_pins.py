"""Pins for the CPU oracle: checks against facts fixed outside the oracle.

Each ``pin_*`` function takes the oracle module (``oracle.sherry_ref`` or a copy
with a planted mistake) and raises AssertionError when the module disagrees
with a fact that does not come from the oracle itself:
  * the counting argument of the format (4 zero slots x 8 sign patterns = 32
    codes; Sherry paper, Abstract: four weights in five bits);
  * the code table and packed words derived by hand from the layout readings
    R2/R3 (derivations written next to each literal);
  * closed forms (all-ones x, one-hot x, sign flip, linearity);
  * brute-force loops over the generator's dense ternary matrix, which never
    passes through the oracle's decoder;
  * brute-force optimality of the packer over all 32 codes;
  * exact rational arithmetic for the fp32 / fp16 epilogue rounding.
"""
from __future__ import annotations

import itertools
import math
import os
from fractions import Fraction

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "sherry_format_hand.txt")


def _load_hand_fixture(path=GOLDEN):
    """Parse tests/golden/sherry_format_hand.txt (hand-derived, see its header)."""
    sec, table, groups, dots, straddle = None, {}, {}, {}, ()
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("["):
                sec = line.strip("[]")
                continue
            tok = line.split()
            if sec == "table":
                table[int(tok[0])] = (tuple(int(v) for v in tok[1:5]), int(tok[5], 16))
            elif sec == "groups":
                kind = tok[1]
                codes = {"ramp": list(range(32)), "ramp_down": [31 - j for j in range(32)],
                         "const0": [0] * 32, "const31": [31] * 32}[kind]
                groups[tok[0]] = (codes, [int(v, 16) for v in tok[2:7]])
            elif sec == "dot":
                dots[tok[0]] = int(tok[1])
            elif sec == "straddle":
                straddle = tuple(int(v) for v in tok)
    assert sorted(table) == list(range(32)) and len(groups) == 4
    for c, (blk, dw) in table.items():  # the two columns of a row agree
        assert sum((v & 0xFF) << (8 * i) for i, v in enumerate(blk)) == dw, c
    return table, groups, dots, straddle


_TABLE, HAND_GROUPS, _DOTS, STRADDLING_CODES = _load_hand_fixture()
HAND_BLOCKS = {c: b for c, (b, _) in _TABLE.items()}
HAND_DWORDS = [_TABLE[c][1] for c in range(32)]
RAMP_DOT = _DOTS["ramp"]


def dword_of(block) -> int:
    return sum((int(v) & 0xFF) << (8 * i) for i, v in enumerate(block))


def all_blocks():
    """The 32 valid blocks, enumerated without the oracle: zero slot x signs."""
    out = []
    for z in range(4):
        for signs in itertools.product((1, -1), repeat=3):
            b = list(signs)
            b.insert(z, 0)
            out.append(tuple(b))
    return out


# ----------------------------------------------------------------- format ---

def pin_bijection(ref):
    decoded = [tuple(ref.decode_block(c)) for c in range(32)]
    assert len(set(decoded)) == 32, "decode is not injective"
    assert set(decoded) == set(all_blocks()), "decoded set != the 32 valid 3:4 blocks"
    for b in decoded:
        assert b.count(0) == 1 and all(v in (-1, 0, 1) for v in b)
    for b in all_blocks():
        c = ref.encode_block(b)
        assert 0 <= c < 32 and tuple(ref.decode_block(c)) == b


def pin_code_table(ref):
    for c, b in HAND_BLOCKS.items():
        assert tuple(ref.decode_block(c)) == b, f"code {c}"
    for c in range(32):
        assert dword_of(ref.decode_block(c)) == HAND_DWORDS[c], f"code {c}"
    # vectorised decoder agrees with the hand table
    codes = np.arange(32, dtype=np.uint8)[None, :]
    dense = ref.dense_from_codes(codes).reshape(32, 4)
    for c in range(32):
        assert dword_of(dense[c]) == HAND_DWORDS[c], f"vectorised code {c}"


def pin_packed_groups(ref):
    for name, (codes, words) in HAND_GROUPS.items():
        assert list(ref.pack_group(codes)) == words, name
        assert list(ref.unpack_group(words)) == codes, name
        v = ref.pack_codes(np.array(codes, dtype=np.uint8)[None, :])
        assert [int(w) for w in v] == words, f"vectorised pack {name}"
        u = ref.unpack_codes(np.array(words, dtype=np.uint32), 1, 128)
        assert [int(c) for c in u[0]] == codes, f"vectorised unpack {name}"


def pin_row_layout(ref):
    """R4 by hand: a row of two groups, "ramp" then "ramp_down", is the four
    leading words of each group followed by the fifth word of each group."""
    ramp, down = HAND_GROUPS["ramp"], HAND_GROUPS["ramp_down"]
    want = ramp[1][:4] + down[1][:4] + [ramp[1][4], down[1][4]]
    codes = np.array([ramp[0] + down[0]], dtype=np.uint8)
    assert [int(w) for w in ref.pack_codes(codes)] == want
    assert ref.unpack_codes(np.array(want, np.uint32), 1, 256).tolist() == codes.tolist()
    # two rows: each row is contiguous, the second starts after 10 words
    two = ref.pack_codes(np.vstack([codes, codes[:, ::-1]]))
    assert [int(w) for w in two[:10]] == want
    assert ref.unpack_codes(two, 2, 256)[1].tolist() == codes[0, ::-1].tolist()


def pin_straddles(ref):
    """A code straddles two words iff flipping it changes two words."""
    found = []
    for j in range(32):
        codes = [0] * 32
        codes[j] = 31
        words = ref.pack_group(codes)
        if sum(1 for w in words if w) == 2:
            found.append(j)
    assert tuple(found) == STRADDLING_CODES


def pin_size(ref):
    for n, k in [(1, 128), (3, 256), (256, 1024), (2048, 8192)]:
        assert ref.packed_bytes(n, k) * 8 == n * k * 5 // 4  # 1.25 bits per weight
    g = synth.rng(7)
    t = synth.ternary_34(5, 384, g)
    words = ref.pack_codes(ref.codes_from_dense(t))
    assert words.dtype == np.uint32 and words.nbytes == 5 * 384 * 5 // 32


def pin_ramp_dot(ref):
    x = np.array([(k % 127) - 63 for k in range(128)], dtype=np.int8)
    words = np.array(HAND_GROUPS["ramp"][1], dtype=np.uint32)
    acc, _ = ref.gemv_i8(words, np.ones(1, np.float32), 1, 128, x, None, np.float32)
    assert int(acc[0]) == RAMP_DOT


# ---------------------------------------------------------- closed forms ---

def pin_closed_forms(ref):
    g = synth.rng(11)
    n, k = 37, 384
    words = synth.random_words(n * (k // 128) * 5, g)
    codes = ref.unpack_codes(words, n, k)
    sw = np.ones(n, np.float32)
    # x = 1: each block adds (#plus - #minus) = 3 - 2 * popcount(sign bits)
    acc1, _ = ref.gemv_i8(words, sw, n, k, np.ones(k, np.int8), None, np.float32)
    pop = np.array([[bin(int(c) >> 2).count("1") for c in row] for row in codes])
    assert np.array_equal(acc1, (3 - 2 * pop).sum(axis=1))
    # x = e_k picks column k of the matrix: bitstream slice + hand table
    for col in (0, 1, 2, 3, 127, 128, 255, 383):
        e = np.zeros(k, np.int8)
        e[col] = 1
        acc, _ = ref.gemv_i8(words, sw, n, k, e, None, np.float32)
        for r in range(n):
            G, gi = k // 128, col // 128  # R4: d0-d3 at 5Gr + 4g + i, d4 at 5Gr + 4G + g
            grp = [int(words[5 * G * r + 4 * gi + i]) for i in range(4)] + [int(words[5 * G * r + 4 * G + gi])]
            v = 0
            for i, w in enumerate(grp):
                v |= w << (32 * i)
            c = (v >> (5 * ((col % 128) // 4))) & 31
            byte = (HAND_DWORDS[c] >> (8 * (col % 4))) & 0xFF  # hand table, not the decoder
            want = byte - 256 if byte > 127 else byte
            assert int(acc[r]) == want, (r, col)
    # flipping every sign bit negates the product
    x = synth.x_int8_uniform(k, g)
    flipped = ref.pack_codes(codes ^ np.uint8(0b11100))
    a, _ = ref.gemv_i8(words, sw, n, k, x, None, np.float32)
    b, _ = ref.gemv_i8(flipped, sw, n, k, x, None, np.float32)
    assert np.array_equal(a, -b)
    # linearity in x (values kept inside int8)
    x1 = (x // 2).astype(np.int8)
    x2 = (x - x1).astype(np.int8)
    a1, _ = ref.gemv_i8(words, sw, n, k, x1, None, np.float32)
    a2, _ = ref.gemv_i8(words, sw, n, k, x2, None, np.float32)
    assert np.array_equal(a, a1 + a2)


# ------------------------------------------------------------ brute force ---

def naive_gemm(t, x):
    """Triple loop: acc[m][r] = sum_k x[m][k] * t[r][k] (pure Python ints)."""
    m, n, k = len(x), len(t), len(t[0])
    return [[sum(int(x[i][c]) * int(t[r][c]) for c in range(k)) for r in range(n)] for i in range(m)]


def pin_brute_force(ref):
    g = synth.rng(23)
    for n, k, m in [(1, 128, 1), (3, 128, 2), (7, 256, 5), (64, 128, 1)]:
        t = synth.ternary_34(n, k, g)  # generator's dense T, never decoded by the oracle
        words = ref.pack_codes(ref.codes_from_dense(t))
        x = synth.x_int8_uniform((m, k), g)
        want = naive_gemm(t.tolist(), x.tolist())
        sw = np.ones(n, np.float32)
        acc, _ = ref.gemm_i8(words, sw, n, k, x, np.ones(m, np.float32), np.float32)
        assert acc.shape == (m, n)
        assert acc.tolist() == want, (n, k, m)
        a1, _ = ref.gemv_i8(words, sw, n, k, x[0], None, np.float32)
        assert a1.tolist() == want[0]


def pin_packer(ref):
    g = synth.rng(31)
    # brute force: the packed code minimises ||w - a * dec(c)||^2 over all 32 codes
    for _ in range(300):
        w4 = g.standard_normal(4)
        a = float(g.uniform(0.05, 2.0))
        c = ref.quantize_block(w4)
        cost = [sum((w4[i] - a * v) ** 2 for i, v in enumerate(b)) for b in (ref.decode_block(cc) for cc in range(32))]
        assert cost[c] <= min(cost) + 1e-12
    # ties go to the lowest slot; -0.0 counts as positive
    assert ref.decode_block(ref.quantize_block([0.5, -0.5, 0.5, 0.5])) == (0, -1, 1, 1)
    assert ref.decode_block(ref.quantize_block([1.0, 0.25, -0.25, 2.0])) == (1, 0, -1, 1)
    assert ref.decode_block(ref.quantize_block([-0.0, 0.0, 1.0, -1.0])) == (0, 1, 1, -1)
    # the row scale is the least-squares scale: perturbing it raises the error
    n, k = 6, 256
    w = g.standard_normal((n, k))
    codes, alpha = ref.quantize(w)
    t = np.array([[v for c in row for v in ref.decode_block(int(c))] for row in codes], dtype=np.float64)
    for r in range(n):
        err = lambda s: float(np.sum((w[r] - s * t[r]) ** 2))  # noqa: E731
        assert err(alpha[r]) < err(alpha[r] * (1 + 1e-3)) and err(alpha[r]) < err(alpha[r] * (1 - 1e-3))
        assert math.isclose(alpha[r], float(np.sum(np.abs(w[r]) * (t[r] != 0))) / (3 * k // 4), rel_tol=1e-14)
    # fp16 scales below 2^-14 round to subnormals, ties to even: W = s T with s
    # halfway between two subnormals (multiples of 2^-24), the smallest
    # subnormal, and values that round to zero or up to 2^-24
    t8 = synth.ternary_34(8, 128, g)
    for r, s16 in enumerate([(2 * mm + 1) * 2.0 ** -25 for mm in (0, 1, 2, 500)] +
                            [2.0 ** -24, 2.0 ** -26, 3 * 2.0 ** -26, 0.3e-6]):
        _, sc = ref.pack((t8[r:r + 1] * s16).astype(np.float32), np.float16)
        exact = Fraction(float(np.float32(s16)))
        assert Fraction(float(sc[0])) == f16_exact(exact), (r, s16)
    # pack(s * T) recovers T and s exactly (fp32 s; fp64 sums of equal values are exact)
    t34 = synth.ternary_34(9, 512, g)
    s = synth.row_scales(9, g, np.float32)
    words, scales = ref.pack((t34 * s[:, None]).astype(np.float32), np.float32)
    assert np.array_equal(ref.unpack(words, 9, 512), t34)
    assert np.array_equal(scales, s)


# -------------------------------------------------------- exact rounding ---

def round_to_float(q: Fraction, mant_bits: int, emin: int, emax: int) -> Fraction:
    """Round a rational to the nearest binary float with ``mant_bits``
    significant bits (ties to even), normal exponent range [emin, emax];
    subnormals below emin.  Overflow returns +-inf as a float."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - mant_bits + 1)
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r >= Fraction(2) ** (emax + 1):
        return float("inf") * sign
    return sign * r


def f32_exact(q):
    return round_to_float(Fraction(q), 24, -126, 127)


def f16_exact(q):
    return round_to_float(Fraction(q), 11, -14, 15)


def pin_epilogue(ref):
    g = synth.rng(41)
    acc = g.integers(-780288, 780289, size=400).astype(np.int32)
    acc[:4] = [0, 1, -1, 780288]
    sw = synth.row_scales(400, g, np.float16)
    sx = np.float32(g.uniform(0.005, 0.05))
    y = ref.epilogue(acc, sw, sx, np.float16)
    for i in range(400):
        t = f32_exact(Fraction(int(acc[i])) * Fraction(float(sw[i])))
        t = f32_exact(t * Fraction(float(sx)))
        assert Fraction(float(y[i])) == f16_exact(t), i
    # inputs where rounding after every product differs from rounding once
    # (found with numpy, confirmed with exact rationals before use)
    cand_acc = g.integers(-780288, 780289, size=200000)
    cand_sw = synth.row_scales(200000, g, np.float16)
    cand_sx = g.uniform(0.005, 0.05, size=200000).astype(np.float32)
    chain = ((cand_acc.astype(np.float32) * cand_sw.astype(np.float32)) * cand_sx).astype(np.float16)
    once = (cand_acc.astype(np.float64) * cand_sw.astype(np.float64) * cand_sx.astype(np.float64)).astype(np.float16)
    picked = np.nonzero(chain != once)[0][:40]
    assert picked.size >= 5
    for i in picked:
        a, s1, s2 = int(cand_acc[i]), Fraction(float(cand_sw[i])), Fraction(float(cand_sx[i]))
        want = f16_exact(f32_exact(f32_exact(Fraction(a) * s1) * s2))
        assert want != f16_exact(Fraction(a) * s1 * s2)
        got = ref.epilogue(np.array([a], np.int32), cand_sw[i:i + 1], cand_sx[i], np.float16)
        assert Fraction(float(got[0])) == want, i
    y32 = ref.epilogue(acc, sw.astype(np.float32), None, np.float32)
    for i in range(400):
        assert Fraction(float(y32[i])) == f32_exact(Fraction(int(acc[i])) * Fraction(float(sw[i]))), i


def pin_bf16_path(ref):
    g = synth.rng(43)
    n, k = 9, 384
    t = synth.ternary_34(n, k, g)
    words = ref.pack_codes(ref.codes_from_dense(t))
    xb = synth.x_bf16_normal(k, g)
    sw = synth.row_scales(n, g, np.float32)
    y = ref.gemv_bf16(words, sw, n, k, xb)
    # bf16 -> value by the definition sign * (1 + m/128) * 2^(e - 127)
    xv = []
    for b in xb.tolist():
        sgn = -1 if b >> 15 else 1
        e = (b >> 7) & 0xFF
        m = b & 0x7F
        xv.append(Fraction(0) if e == 0 and m == 0 else sgn * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127))
    for r in range(n):
        exact = sum(int(t[r, c]) * xv[c] for c in range(k))
        # one rounding of the exact sum to fp64, one for the scale product
        assert y[r] == float(exact) * float(sw[r]), r


def _bf16_value(b: int) -> Fraction:
    """bf16 bit pattern -> exact value by the definition
    sign * (1 + m / 128) * 2^(e - 127) (normal numbers and zero only)."""
    sgn = -1 if b >> 15 else 1
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    if e == 0 and m == 0:
        return Fraction(0)
    assert 0 < e < 255, "normal bf16 only"
    return sgn * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def pin_bf16_wide_range(ref):
    """bf16 x whose exponents span far more than fp64's 53 bits, so that no
    fp64 summation order is exact: every block is (a, a, 0, b) against x =
    (B, -B, u, s) with B huge (2^60 .. 2^120) and s tiny (2^-120 .. 2^-60).
    The huge terms cancel exactly inside each block, so the exact row sum is
    sum_j b_j s_j, which any fp64 running sum that meets a huge partial sum
    loses.  Each row must equal that exact sum rounded once to fp64, times
    the row scale."""
    g = synth.rng(44)
    n, k = 5, 256
    nb = k // 4
    a = g.choice([-1, 1], size=(n, nb))
    b = g.choice([-1, 1], size=(n, nb))
    t = np.zeros((n, nb, 4), np.int8)
    t[:, :, 0] = a
    t[:, :, 1] = a
    t[:, :, 3] = b
    t = t.reshape(n, k)
    bits = np.zeros(k, np.int64)
    for j in range(nb):
        big = (int(g.integers(127 + 60, 127 + 121)) << 7) | int(g.integers(0, 128))
        tiny = (int(g.integers(127 - 120, 127 - 59)) << 7) | int(g.integers(0, 128))
        mid = (int(g.integers(127 - 20, 127 + 21)) << 7) | int(g.integers(0, 128))
        bits[4 * j:4 * j + 4] = [big, big | 0x8000, mid | (int(g.integers(0, 2)) << 15),
                                 tiny | (int(g.integers(0, 2)) << 15)]
    xb = bits.astype(np.uint16)
    words = ref.pack_codes(ref.codes_from_dense(t))
    sw = synth.row_scales(n, g, np.float32)
    y = ref.gemv_bf16(words, sw, n, k, xb)
    xv = [_bf16_value(int(v)) for v in xb.tolist()]
    for r in range(n):
        exact = sum(int(t[r, c]) * xv[c] for c in range(k))
        assert exact != 0 and abs(exact) < Fraction(2) ** -50, r  # only the tiny terms survive
        assert y[r] == float(exact) * float(sw[r]), r


def pin_gemm_bf16(ref):
    """M tokens of bf16 x against exact rationals, on the generator's dense
    matrix (never decoded by the oracle): one token of N(0, 1) values, one
    spanning 2^-120 .. 2^120 (the exact-sum fallback), one of zeros, and
    ragged sizes.  Each Y[m, r] is the exact sum rounded once to fp64, times
    the row scale."""
    g = synth.rng(45)
    for n, k, m in [(3, 128, 3), (7, 256, 2)]:
        t = synth.ternary_34(n, k, g)
        words = ref.pack_codes(ref.codes_from_dense(t))
        xb = np.zeros((m, k), np.uint16)
        xb[0] = synth.x_bf16_normal(k, g)
        if m > 2:
            e = g.integers(127 - 120, 127 + 121, size=k)
            xb[1] = ((g.integers(0, 2, size=k) << 15) | (e << 7) | g.integers(0, 128, size=k)).astype(np.uint16)
        sw = synth.row_scales(n, g, np.float32)
        y = ref.gemm_bf16(words, sw, n, k, xb)
        assert y.shape == (m, n)
        for i in range(m):
            xv = [_bf16_value(int(v)) for v in xb[i].tolist()]
            for r in range(n):
                exact = sum(int(t[r, c]) * xv[c] for c in range(k))
                assert y[i, r] == float(exact) * float(sw[r]), (n, k, i, r)


# ------------------------------------------- activation quantization ---
# Pins for oracle.act_ref (per-token absmax int8, readings A1-A3): hand
# values, exact rational arithmetic, invariants, and the generator's own
# independent quantizer.

def _rint_half_even(q: Fraction) -> int:
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def pin_act_hand(act):
    # s = 127 / 127 = 1 exactly; quotients are the values: ties go to even
    q, s = act.quantize(np.array([[127.0, 63.5, -62.5, 0.5, -1.5, 2.5, -126.5]], np.float32))
    assert s.tolist() == [1.0]
    assert q.tolist() == [[127, 64, -62, 0, -2, 2, -126]]
    # amax 190.5 -> s = 190.5 / 127 = 1.5 exactly; 0.75 / 1.5 = 0.5,
    # 3.75 / 1.5 = 2.5, -6.75 / 1.5 = -4.5, 2.25 / 1.5 = 1.5 exactly (ties);
    # a product with fp32(1 / 1.5) would push 0.75 over 0.5
    q, s = act.quantize(np.array([[190.5, 0.75, 3.75, -6.75, 2.25]], np.float32))
    assert s.tolist() == [1.5]
    assert q.tolist() == [[127, 0, 2, -4, 2]]
    # amax 222.25 -> s = 1.75 exactly; 11.375 / 1.75 = 6.5 exactly, a tie
    # that goes to 6, while 11.375 * fp32(1 / 1.75) rounds to 6.5000005
    q, s = act.quantize(np.array([[222.25, 11.375, -11.375, 4.375]], np.float32))
    assert s.tolist() == [1.75]
    assert q.tolist() == [[127, 6, -6, 2]]


def pin_act_zero_and_signs(act):
    q, s = act.quantize(np.zeros((2, 64), np.float32))
    assert s.tolist() == [1.0, 1.0] and not q.any()
    g = synth.rng(51)
    x = g.standard_normal((5, 256)).astype(np.float32)
    q, s = act.quantize(x)
    qn, sn = act.quantize(-x)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)  # round-half-even is odd-symmetric
    am = np.argmax(np.abs(x), axis=1)
    for t in range(5):
        assert q[t, am[t]] == (127 if x[t, am[t]] > 0 else -127)
    assert np.abs(q.astype(np.int32)).max() <= 127
    # power-of-two scaling is exact in fp32: same codes, scale times 2^e
    for e in (-7, 5):
        q2, s2 = act.quantize(x * np.float32(2.0 ** e))
        assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(2.0 ** e))
    # error bound: |q s - x| <= s / 2 up to the quotient's rounding
    err = np.abs(q.astype(np.float64) * s[:, None].astype(np.float64) - x.astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 2.0 ** -16))


def pin_act_exact(act):
    """Every element against exact rationals: s = RN32(amax / 127), then
    rint_even(RN32(x / s)) clipped."""
    g = synth.rng(52)
    x = (g.standard_normal((4, 96)) * np.array([[1.0], [1e-3], [37.0], [0.25]])).astype(np.float32)
    x[3, :8] = [0.0, -0.0, 1.0, -1.0, 0.5, 0.25, -0.125, 0.0]
    q, s = act.quantize(x)
    for t in range(x.shape[0]):
        amax = max(abs(Fraction(float(v))) for v in x[t])
        st = f32_exact(amax / 127)
        assert Fraction(float(s[t])) == st, t
        for j in range(x.shape[1]):
            want = max(-127, min(127, _rint_half_even(f32_exact(Fraction(float(x[t, j])) / st))))
            assert int(q[t, j]) == want, (t, j)


def pin_act_generator(act):
    """The input generator quantizes by the same rule with its own code."""
    g = synth.rng(53)
    xq, sx, x = synth.act_absmax_int8(7, 640, g)
    q, s = act.quantize(x)
    assert np.array_equal(q, xq) and np.array_equal(s, sx)


def pin_act_dtypes(act):
    """fp16 and bf16 inputs quantize as their (exact) fp32 values."""
    g = synth.rng(54)
    x = g.standard_normal((3, 128)).astype(np.float32)
    h = x.astype(np.float16)
    assert all(np.array_equal(a, b) for a, b in zip(act.quantize(h, "f16"), act.quantize(h.astype(np.float32))))
    bits = synth.f32_to_bf16_bits(x)
    # bf16 value by the definition sign * (1 + m / 128) * 2^(e - 127)
    vals = np.array([[(-1.0 if b >> 15 else 1.0) * (1 + (b & 0x7F) / 128.0) * 2.0 ** (((b >> 7) & 0xFF) - 127)
                      for b in row] for row in bits.tolist()], np.float32)
    assert all(np.array_equal(a, b) for a, b in zip(act.quantize(bits, "bf16"), act.quantize(vals)))


ACT_PINS = [pin_act_hand, pin_act_zero_and_signs, pin_act_exact, pin_act_generator, pin_act_dtypes]


# ------------------------------------------------ 1.67-bit comparator ---
# Pins for oracle.tern3_ref (three ternary weights in five bits, readings
# F1-F4): base-3 digits written out by hand, the all-zero row from the bit
# pattern of its code, one changed weight located by hand, sizes, and
# brute-force products over the generator's dense matrix.

def pin_t3_codes(t3):
    # c = (t0 + 1) + 3 (t1 + 1) + 9 (t2 + 1), digits written out by hand
    hand = {0: (-1, -1, -1), 13: (0, 0, 0), 26: (1, 1, 1), 5: (1, 0, -1), 21: (-1, 0, 1), 1: (0, -1, -1),
            9: (-1, -1, 0), 14: (1, 0, 0)}
    for c, blk in hand.items():
        assert t3.decode_block(c) == blk, c
        assert t3.encode_block(blk) == c, c
    seen = {t3.encode_block(b) for b in itertools.product((-1, 0, 1), repeat=3)}
    assert seen == set(range(27))
    for c in range(27, 32):
        try:
            t3.decode_block(c)
        except ValueError:
            continue
        raise AssertionError(f"code {c} is not a block")


def pin_t3_layout(t3):
    assert t3.packed_words(1, 128) == 10 and t3.packed_words(1, 2048) == 110 and t3.packed_words(3, 8192) == 3 * 430
    # an all-zero row: every code is 13 = 0b01101, so stream bit b is set iff
    # b mod 5 is 0, 2 or 3; the words are the stream's 32-bit slices
    k, G = 2048, 22
    bits = [1 if b % 5 in (0, 2, 3) else 0 for b in range(160)]
    slices = [sum(bits[32 * i + j] << j for j in range(32)) for i in range(5)]
    w = t3.pack(np.zeros((1, k), np.int8))
    for g in range(G):
        assert [int(v) for v in w[4 * g:4 * g + 4]] == slices[:4], g
        assert int(w[4 * G + g]) == slices[4], g
    # weight 189 = 96 + 3 * 31 is t0 of code 31 of group 1 (stream bits
    # 155..159, word 4 of the group, bits 27..31, stored at word 4 G + 1);
    # setting it to +1 turns that code from 13 into 14 (0b01110)
    t = np.zeros((1, k), np.int8)
    t[0, 189] = 1
    w2 = t3.pack(t)
    diff = np.nonzero(w2 != w)[0].tolist()
    assert diff == [4 * G + 1]
    assert int(w2[4 * G + 1]) ^ int(w[4 * G + 1]) == (13 ^ 14) << 27
    # weight 20 is t2 of code 6 of group 0, which straddles words 0 and 1
    # (stream bits 30..34): 13 -> 22, 13 ^ 22 = 0b11011, so word 0 flips its
    # bits 30, 31 and word 1 its bits 1, 2
    t = np.zeros((1, k), np.int8)
    t[0, 20] = 1
    w3 = t3.pack(t)
    assert np.nonzero(w3 != w)[0].tolist() == [0, 1]
    assert int(w3[0]) ^ int(w[0]) == 3 << 30 and int(w3[1]) ^ int(w[1]) == 6
    # K = 128: two groups, weights 128..191 padding (zeros, code 13); weight
    # 127 is t1 of code 10 of group 1 (stream bits 50..54: word 1 of the group,
    # stored at 4 + 1, bits 18..22), 13 -> 16
    t = np.zeros((1, 128), np.int8)
    w0 = t3.pack(t)
    assert len(w0) == 10 and int(w0[8]) == int(w0[9]) == slices[4]
    t[0, 127] = 1
    w4 = t3.pack(t)
    assert np.nonzero(w4 != w0)[0].tolist() == [5]
    assert int(w4[5]) ^ int(w0[5]) == (13 ^ 16) << 18


def pin_t3_products(t3):
    g = synth.rng(57)
    n, k = 5, 256
    t = synth.ternary_dense(n, k, g)
    words = t3.pack(t)
    assert np.array_equal(t3.unpack(words, n, k), t)
    codes_ok = True
    G = t3.groups(k)
    for r in range(n):
        for grp in range(G):
            parts = [int(words[5 * G * r + 4 * grp + i]) for i in range(4)] + [int(words[5 * G * r + 4 * G + grp])]
            stream = sum(p << (32 * i) for i, p in enumerate(parts))
            codes_ok &= all(((stream >> (5 * j)) & 31) < 27 for j in range(32))
    assert codes_ok
    x = synth.x_int8_uniform(k, g)
    sw = synth.row_scales(n, g, np.float32)
    acc, y = t3.gemv_i8(words, sw, n, k, x, None, np.float32)
    for r in range(n):  # brute force over the generator's dense matrix
        want = 0
        for c in range(k):
            want += int(t[r, c]) * int(x[c])
        assert int(acc[r]) == want, r
        assert Fraction(float(y[r])) == f32_exact(Fraction(want) * Fraction(float(sw[r]))), r
    # with a token scale and fp16 output: ((acc * s_w) * s_x) rounded to fp32
    # after each product, then once to fp16, against exact rationals
    sx = np.float32(g.uniform(0.005, 0.05))
    sw16 = synth.row_scales(n, g, np.float16)
    acc2, y2 = t3.gemv_i8(words, sw16, n, k, x, sx, np.float16)
    assert np.array_equal(acc2, acc)
    for r in range(n):
        t1 = f32_exact(Fraction(int(acc[r])) * Fraction(float(sw16[r])))
        want = f16_exact(f32_exact(t1 * Fraction(float(sx))))
        assert Fraction(float(y2[r])) == want, r


T3_PINS = [pin_t3_codes, pin_t3_layout, pin_t3_products]
