"""Planted mistakes in a private copy of the oracle must trip at least one pin.

Each case loads a fresh copy of oracle/sherry_ref.py, replaces one routine with
a plausibly wrong variant (a dropped term, a wrong sign or bit order, a
transposed operand, a different tie rule), and checks that the pins reject it.
The real oracle module is never modified."""
import importlib.util
import types
import os

import numpy as np
import pytest

from tests import oracle_pins as P

PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "sherry_ref.py")
ALL_PINS = [P.pin_bijection, P.pin_code_table, P.pin_packed_groups, P.pin_row_layout, P.pin_straddles, P.pin_size,
            P.pin_ramp_dot, P.pin_closed_forms, P.pin_brute_force, P.pin_packer, P.pin_epilogue,
            P.pin_bf16_path, P.pin_bf16_wide_range, P.pin_gemm_bf16]


def fresh():
    spec = importlib.util.spec_from_file_location("sherry_ref_planted", PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def m_sign_order_reversed(ref):
    orig = ref.dense_from_codes

    def bad(codes):
        c = np.asarray(codes).astype(np.int64)
        s = c >> 2
        rev = ((s & 1) << 2) | (s & 2) | ((s >> 2) & 1)
        return orig(((c & 3) | (rev << 2)).astype(np.uint8))
    ref.dense_from_codes = bad
    d = ref.decode_block
    ref.decode_block = lambda c: d((c & 3) | ((((c >> 2) & 1) << 2 | ((c >> 2) & 2) | ((c >> 4) & 1)) << 2))


def m_sign_meaning_flipped(ref):
    orig = ref.dense_from_codes
    ref.dense_from_codes = lambda codes: (-orig(codes)).astype(np.int8)
    d = ref.decode_block
    ref.decode_block = lambda c: tuple(-v for v in d(c))


def m_zero_field_high(ref):
    """zero slot taken from the top two bits instead of the bottom two"""
    orig = ref.dense_from_codes

    def bad(codes):
        c = np.asarray(codes).astype(np.int64)
        return orig((((c >> 3) & 3) | ((c & 7) << 2)).astype(np.uint8))
    ref.dense_from_codes = bad
    d = ref.decode_block
    ref.decode_block = lambda c: d(((c >> 3) & 3) | ((c & 7) << 2))


def m_msb_first_stream(ref):
    orig_pack, orig_unpack = ref.pack_codes, ref.unpack_codes

    def rev5(c):
        c = np.asarray(c).astype(np.uint8)
        out = np.zeros_like(c)
        for b in range(5):
            out |= ((c >> b) & 1) << (4 - b)
        return out
    ref.pack_codes = lambda codes: orig_pack(rev5(codes))
    ref.unpack_codes = lambda words, n, k: rev5(orig_unpack(words, n, k))
    pg, ug = ref.pack_group, ref.unpack_group
    ref.pack_group = lambda codes: pg([int(rev5(np.uint8(c))) for c in codes])
    ref.unpack_group = lambda words: [int(rev5(np.uint8(c))) for c in ug(words)]


def m_word_order_swapped(ref):
    orig_unpack = ref.unpack_codes

    def bad(words, n, k):
        w = np.asarray(words, np.uint32).reshape(-1, 5)[:, ::-1].reshape(-1)
        return orig_unpack(np.ascontiguousarray(w), n, k)
    ref.unpack_codes = bad


def m_layout_groups_contiguous(ref):
    """Checks that the row layout R4 is pinned: the five words of every group
    stored together (another plausible layout, not the one this oracle takes)
    must be told apart from R4 by the pins."""
    def pack(codes):
        c = np.asarray(codes).astype(np.uint8)
        n, nb = c.shape
        out = []
        for r in range(n):
            for gi in range(nb // 32):
                out += ref.pack_group(c[r, 32 * gi:32 * gi + 32])
        return np.array(out, dtype=np.uint32)
    ref.pack_codes = pack


def m_transposed_operand(ref):
    def bad(words, s_w, n, k, x, s_x, y_dtype=np.float16):
        t = ref.unpack(words, n, k)
        tt = t.reshape(k, n) if t.size == n * k else t  # wrong orientation
        acc = ref._exact_int_matmul(np.asarray(x).astype(np.int64), tt.astype(np.int64)).astype(np.int32)
        return acc, ref.epilogue(acc, s_w, s_x, y_dtype)
    ref.gemm_i8 = bad


def m_dropped_token_scale(ref):
    orig = ref.epilogue
    ref.epilogue = lambda acc, s_w, s_x=None, y_dtype=np.float16: orig(acc, s_w, None, y_dtype)


def m_fp64_epilogue(ref):
    def bad(acc, s_w, s_x=None, y_dtype=np.float16):
        t = np.asarray(acc).astype(np.float64) * np.asarray(s_w).astype(np.float64)
        if s_x is not None:
            sx = np.asarray(s_x, dtype=np.float64)
            t = t * (sx[:, None] if sx.ndim == 1 and t.ndim == 2 else sx)
        return t.astype(y_dtype)
    ref.epilogue = bad


def m_tie_to_highest(ref):
    orig = ref.quantize_block

    def bad(w4):
        w = [float(v) for v in w4]
        z = max(range(4), key=lambda s: (-abs(w[s]), s))
        t = [0 if s == z else (-1 if w[s] < 0 else 1) for s in range(4)]
        return ref.encode_block(t)
    ref.quantize_block = bad
    del orig


def m_absmean_scale(ref):
    orig = ref.quantize

    def bad(w):
        codes, _ = orig(w)
        return codes, np.mean(np.abs(np.asarray(w, np.float64)), axis=1)
    ref.quantize = bad


def m_bf16_scale_dropped(ref):
    def bad(words, s_w, n, k, x_bits):
        t = ref.unpack(words, n, k)
        return ref._exact_rows_dot(t, ref.bf16_bits_to_f64(x_bits))
    ref.gemv_bf16 = bad


def m_gemm_bf16_token_order(ref):
    """tokens taken in reverse order"""
    orig = ref.gemm_bf16
    ref.gemm_bf16 = lambda words, s_w, n, k, x_bits: orig(words, s_w, n, k, np.asarray(x_bits)[::-1])


def m_gemm_bf16_scale_per_token(ref):
    """the row scales applied along the token axis"""
    def bad(words, s_w, n, k, x_bits):
        t = ref.unpack(words, n, k)
        xb = np.asarray(x_bits)
        sw = np.asarray(s_w).astype(np.float64)
        return np.stack([ref._exact_rows_dot(t, ref.bf16_bits_to_f64(xb[i])) * sw[i % len(sw)]
                         for i in range(xb.shape[0])])
    ref.gemm_bf16 = bad


def m_gemm_bf16_fp32_sum(ref):
    """the sums accumulated in fp32"""
    def bad(words, s_w, n, k, x_bits):
        t = ref.unpack(words, n, k).astype(np.float32)
        x = np.stack([ref.bf16_bits_to_f64(r) for r in np.asarray(x_bits)]).astype(np.float32)
        return (x @ t.T).astype(np.float64) * np.asarray(s_w).astype(np.float64)
    ref.gemm_bf16 = bad


MUTANTS = [m_sign_order_reversed, m_sign_meaning_flipped, m_zero_field_high, m_msb_first_stream,
           m_word_order_swapped, m_layout_groups_contiguous, m_transposed_operand, m_dropped_token_scale, m_fp64_epilogue,
           m_tie_to_highest, m_absmean_scale, m_bf16_scale_dropped, m_gemm_bf16_token_order,
           m_gemm_bf16_scale_per_token, m_gemm_bf16_fp32_sum]


# Planted in the source text of a private copy of oracle/sherry_ref.py: the
# exact-sum fallback of the bf16 product, taken when x spans too many binades
# for an exact fp64 BLAS sum.
SHERRY_SRC_MUTANTS = {
    "fsum_fallback_doubled": ("return np.array([math.fsum((t[r] * x64).tolist()) for r in range(t.shape[0])])",
                              "return 2 * np.array([math.fsum((t[r] * x64).tolist()) for r in range(t.shape[0])])"),
    "fsum_fallback_never_taken": ("if bound * 2.0 ** (-e_min) < 2.0 ** 52:", "if True:"),
}


@pytest.mark.parametrize("name", sorted(SHERRY_SRC_MUTANTS))
def test_sherry_source_planted_mistake_is_caught(name):
    ref = fresh_module(PATH, "sherry_ref_src_planted", SHERRY_SRC_MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(ref)
        except (AssertionError, ValueError, OverflowError):
            caught.append(pin.__name__)
    assert caught, f"{name} passed every pin"


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_planted_mistake_is_caught(mutant):
    ref = fresh()
    for pin in ALL_PINS:  # the unmodified copy passes every pin
        pin(ref)
    mutant(ref)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(ref)
        except (AssertionError, ValueError, OverflowError):
            caught.append(pin.__name__)
    assert caught, f"{mutant.__name__} passed every pin"


# ------------------------------------------- activation quantization ---
# Planted in the source text of a private copy of oracle/act_ref.py.
ACT_PATH = os.path.join(os.path.dirname(PATH), "act_ref.py")
ACT_MUTANTS = {
    "reciprocal_product": ("quot = (row / st).astype(np.float32)",
                           "quot = (row * np.float32(np.float32(1) / st)).astype(np.float32)"),
    "half_away_from_zero": ("np.rint(quot)", "np.trunc(quot + np.copysign(np.float32(0.5), quot))"),
    "divide_by_128": ("amax / np.float32(127)", "amax / np.float32(128)"),
    "zero_token_scale_0": ("continue  # s = 1, x_q = 0", "s[t] = 0\n            continue"),
    "mean_not_max": ("np.max(np.abs(row))", "np.mean(np.abs(row))"),
}


def fresh_act(patch=None):
    src = open(ACT_PATH).read()
    if patch:
        assert patch[0] in src, patch[0]
        src = src.replace(patch[0], patch[1])
    mod = types.ModuleType("act_ref_planted")
    exec(compile(src, ACT_PATH, "exec"), mod.__dict__)
    return mod


def test_act_copy_passes_every_pin():
    act = fresh_act()
    for pin in P.ACT_PINS:
        pin(act)


@pytest.mark.parametrize("name", sorted(ACT_MUTANTS))
def test_act_planted_mistake_is_caught(name):
    act = fresh_act(ACT_MUTANTS[name])
    caught = []
    for pin in P.ACT_PINS:
        try:
            pin(act)
        except (AssertionError, ValueError, OverflowError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"{name} passed every pin"


# ------------------------------------------------ 1.67-bit comparator ---
T3_PATH = os.path.join(os.path.dirname(PATH), "tern3_ref.py")
T3_MUTANTS = {
    "digit_order_reversed": ("return (t0 + 1) + 3 * (t1 + 1) + 9 * (t2 + 1)",
                             "return (t2 + 1) + 3 * (t1 + 1) + 9 * (t0 + 1)"),
    "signs_swapped": ("return (c % 3 - 1, (c // 3) % 3 - 1, c // 9 - 1)",
                      "return (1 - c % 3, 1 - (c // 3) % 3, 1 - c // 9)"),
    "groups_contiguous": ("out[r, 4 * g + i if i < 4 else 4 * G + g] = word", "out[r, 5 * g + i] = word"),
    "msb_first_stream": ("stream |= encode_block(padded[r, w0:w0 + 3]) << (5 * j)",
                         "stream |= encode_block(padded[r, w0:w0 + 3]) << (5 * (31 - j))"),
    "token_scale_divides": ("a = a * np.float32(s_x)", "a = a / np.float32(s_x)"),
    "token_scale_dropped": ("a = a * np.float32(s_x)", "a = a * np.float32(1)"),
}


def fresh_module(path, name, patch=None):
    src = open(path).read()
    if patch:
        assert patch[0] in src, patch[0]
        src = src.replace(patch[0], patch[1])
    mod = types.ModuleType(name)
    exec(compile(src, path, "exec"), mod.__dict__)
    return mod


def test_t3_copy_passes_every_pin():
    t3 = fresh_module(T3_PATH, "tern3_ref_copy")
    for pin in P.T3_PINS:
        pin(t3)


@pytest.mark.parametrize("name", sorted(T3_MUTANTS))
def test_t3_planted_mistake_is_caught(name):
    t3 = fresh_module(T3_PATH, "tern3_ref_planted", T3_MUTANTS[name])
    caught = []
    for pin in P.T3_PINS:
        try:
            pin(t3)
        except (AssertionError, ValueError, OverflowError):
            caught.append(pin.__name__)
    assert caught, f"{name} passed every pin"
