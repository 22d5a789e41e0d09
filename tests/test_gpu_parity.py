"""HIP path (libsherry.so via the C ABI) against the CPU oracle, element by element.

Integer results (codes, int32 sums) must match bit for bit; fp16/fp32 outputs of
the int8 paths too (the epilogue is the same chain of IEEE fp32 products).  The
bf16 path accumulates in fp32 in a different order from the exact reference,
so it is held to max|d| <= 1e-3 * max|y_ref| and relative L2 <= 1e-4.
"""
import os

import numpy as np
import pytest
import torch

import synth
from oracle import act_ref, sherry_ref, tern2_ref, tern3_ref

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def words_dev(w):
    return dev(np.asarray(w, dtype=np.uint32).view(np.int32))


def host_words(t):
    return t.cpu().numpy().view(np.uint32)


def say(*a):
    print(*a, flush=True)


# ----------------------------------------------------------------- runtime ---

def test_single_hip_runtime_in_process(gpu_lib):
    x = torch.zeros(4, device=DEV)
    gpu_lib.gemv(words_dev(np.zeros(20, np.uint32)), dev(np.ones(1, np.float16)), dev(np.zeros(128, np.int8)))
    torch.cuda.synchronize()
    maps = open("/proc/self/maps").read().splitlines()
    libs = {ln.split()[-1] for ln in maps if "libamdhip64" in ln}
    assert len(libs) == 1, libs
    assert x.sum().item() == 0


# -------------------------------------------------------------------- pack ---

PACK_SHAPES = [(1, 128), (3, 256), (37, 640), (256, 1024), (64, 2048), (5, 3072), (9, 8192)]


@pytest.mark.parametrize("n,k", PACK_SHAPES)
@pytest.mark.parametrize("w_dtype", [np.float32, np.float16, "bf16"])
@pytest.mark.parametrize("s_dtype", [np.float32, np.float16])
def test_pack_matches_oracle(gpu_lib, n, k, w_dtype, s_dtype):
    say(f"pack n={n} k={k} w={w_dtype} s={s_dtype}")
    g = synth.rng(1000 + n + k)
    w32 = g.standard_normal((n, k)).astype(np.float32)
    w32[0, :12] = [0.5, -0.5, 0.5, 0.5, -0.0, 0.0, 1.0, -1.0, 0.25, 0.25, 0.25, 0.25]  # ties, signed zero
    if w_dtype == "bf16":
        bits = synth.f32_to_bf16_bits(w32)
        w_host = (bits.astype(np.uint32) << 16).view(np.float32)  # exact values the GPU sees
        w_t = dev(bits.view(np.int16)).view(torch.bfloat16)
    else:
        w_host = w32.astype(w_dtype)
        w_t = dev(w_host)
    ref_words, ref_scales = sherry_ref.pack(w_host, s_dtype)
    codes, scales = gpu_lib.pack(w_t, torch.float32 if s_dtype == np.float32 else torch.float16)
    torch.cuda.synchronize()
    assert np.array_equal(host_words(codes), ref_words)
    got = scales.cpu().numpy()
    assert np.array_equal(got.view(np.uint32 if s_dtype == np.float32 else np.uint16),
                          ref_scales.view(np.uint32 if s_dtype == np.float32 else np.uint16))


@pytest.mark.parametrize("n,k", [(1, 128), (37, 640), (256, 2048)])
@pytest.mark.parametrize("w_dtype", [np.float32, np.float16, "bf16"])
def test_tern2_pack_matches_oracle(gpu_lib, n, k, w_dtype):
    """The 2-bit packer keeps the 3:4 decisions and scales (reading R8b):
    words and scales equal the oracle's, and equal tern2_encode of the 3:4
    packer's decoded matrix."""
    say(f"tern2_pack n={n} k={k} {w_dtype}")
    g = synth.rng(11 * n + k)
    w32 = (g.standard_normal((n, k)) * 0.05).astype(np.float32)
    w32[0, :12] = [0.5, -0.5, 0.5, 0.5, -0.0, 0.0, 1.0, -1.0, 0.25, 0.25, 0.25, 0.25]  # ties, signed zero
    if w_dtype == "bf16":
        bits = synth.f32_to_bf16_bits(w32)
        w_ref = (bits.astype(np.uint32) << 16).view(np.float32)
        w_dev = dev(bits.view(np.int16)).view(torch.bfloat16)
    else:
        w_ref = w32.astype(w_dtype)
        w_dev = dev(w_ref)
    words, sc = gpu_lib.tern2_pack(w_dev, torch.float16)
    c5, s5 = gpu_lib.pack(w_dev, torch.float16)
    via = gpu_lib.tern2_encode(gpu_lib.decode(c5, n, k))
    torch.cuda.synchronize()
    ref_words, ref_s = tern2_ref.pack_weights(w_ref, np.float16)
    assert np.array_equal(host_words(words), ref_words)
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), ref_s.view(np.uint16))
    assert torch.equal(words, via) and torch.equal(sc.view(torch.int16), s5.view(torch.int16))


@pytest.mark.parametrize("w_dtype", [np.float32, "bf16"])
def test_pack_subnormal_fp16_scales(gpu_lib, w_dtype):
    """Row scales in fp16's subnormal range (below 2^-14): weights of about
    1e-6, rows whose exact scale lies halfway between two subnormals (ties go
    to the even one), the smallest subnormal 2^-24, and a scale that rounds
    to zero (2^-26).  Codes and fp16 scale bits against the oracle."""
    say(f"pack subnormal fp16 scales w={w_dtype}")
    g = synth.rng(4711)
    n, k = 16, 256
    w32 = (g.standard_normal((n, k)) * 1e-6).astype(np.float32)
    t = synth.ternary_34(8, k, g)
    halves = [(2 * mm + 1) * 2.0 ** -25 for mm in (0, 1, 2, 3, 500)] + [2.0 ** -24, 2.0 ** -26, 3 * 2.0 ** -26]
    for r, s in enumerate(halves):  # W = s T: the exact scale is s
        w32[8 + r] = (t[r] * s).astype(np.float32)
    if w_dtype == "bf16":
        bits = synth.f32_to_bf16_bits(w32)
        w_host = (bits.astype(np.uint32) << 16).view(np.float32)
        w_t = dev(bits.view(np.int16)).view(torch.bfloat16)
    else:
        w_host = w32
        w_t = dev(w32)
    ref_words, ref_scales = sherry_ref.pack(w_host, np.float16)
    assert np.all(np.abs(ref_scales.astype(np.float32)) < 2.0 ** -14)  # every scale subnormal (or zero)
    codes, scales = gpu_lib.pack(w_t, torch.float16)
    torch.cuda.synchronize()
    assert np.array_equal(host_words(codes), ref_words)
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), ref_scales.view(np.uint16))


def test_pack_exact_ternary_and_row_stride(gpu_lib):
    g = synth.rng(77)
    n, k, ld = 50, 1024, 1024 + 64
    t = synth.ternary_34(n, k, g)
    s = synth.row_scales(n, g, np.float32)
    full = np.zeros((n, ld), np.float32)
    full[:, :k] = t * s[:, None]
    full[:, k:] = 1e6  # padding past k must be ignored
    wt = dev(full)[:, :k]
    codes, scales = gpu_lib.pack(wt, torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(sherry_ref.unpack(host_words(codes), n, k), t)
    assert np.array_equal(scales.cpu().numpy(), s)


@pytest.mark.parametrize("n,k", [(1, 128), (37, 640), (256, 1024), (9, 8192)])
def test_decode_matches_oracle(gpu_lib, n, k):
    g = synth.rng(n * 13 + k)
    words = synth.random_words(n * (k // 128) * 5, g)
    t = gpu_lib.decode(words_dev(words), n, k)
    torch.cuda.synchronize()
    assert np.array_equal(t.cpu().numpy(), sherry_ref.unpack(words, n, k))


# -------------------------------------------------------------- int8 GEMV ---

GEMV_K = [128, 256, 384, 640, 1024, 2048, 3072, 4096, 8192]
GEMV_N = [1, 7, 64, 257, 1000]


@pytest.mark.parametrize("k", GEMV_K)
@pytest.mark.parametrize("n", GEMV_N)
def test_gemv_i8_matches_oracle(gpu_lib, n, k):
    say(f"gemv_i8 n={n} k={k}")
    g = synth.rng(n * 31 + k)
    words = synth.random_words(n * (k // 128) * 5, g)
    s16 = synth.row_scales(n, g, np.float16)
    x = synth.x_int8_uniform(k, g)
    x[:3] = [-128, 127, -127]
    sx = np.float32(g.uniform(0.005, 0.05))
    ref_acc, ref_y = sherry_ref.gemv_i8(words, s16, n, k, x, sx, np.float16)
    acc, y = gpu_lib.gemv(words_dev(words), dev(s16), dev(x), dev(np.array([sx], np.float32)), torch.float16,
                          want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), ref_acc)
    assert np.array_equal(y.cpu().numpy().view(np.uint16), ref_y.view(np.uint16))


@pytest.mark.parametrize("k", [1024, 2048, 8192])
def test_gemv_i8_fp32_scales_and_outputs(gpu_lib, k):
    g = synth.rng(5 + k)
    n = 256
    words = synth.random_words(n * (k // 128) * 5, g)
    s32 = synth.row_scales(n, g, np.float32)
    x = synth.x_int8_uniform(k, g)
    ref_acc, ref_y = sherry_ref.gemv_i8(words, s32, n, k, x, None, np.float32)
    _, y = gpu_lib.gemv(words_dev(words), dev(s32), dev(x), None, torch.float32)
    acc, y2 = gpu_lib.gemv(words_dev(words), dev(s32), dev(x), None, None, want_acc=True)
    torch.cuda.synchronize()
    assert y2 is None
    assert np.array_equal(acc.cpu().numpy(), ref_acc)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), ref_y.view(np.uint32))


def test_gemv_i8_extreme_accumulators(gpu_lib):
    """All weights of a row +1 where x = 127 (max positive sum) and a flipped
    row (max negative sum), at the largest k."""
    k, n = 8192, 2
    t = np.zeros((n, k), np.int8)
    t[0] = np.tile([0, 1, 1, 1], k // 4)
    t[1] = -t[0]
    t[1, ::4] = 0
    words = sherry_ref.pack_codes(sherry_ref.codes_from_dense(t))
    x = np.full(k, 127, np.int8)
    acc, _ = gpu_lib.gemv(words_dev(words), dev(np.ones(n, np.float32)), dev(x), None, None, want_acc=True)
    torch.cuda.synchronize()
    assert acc.cpu().numpy().tolist() == [127 * 3 * k // 4, -127 * 3 * k // 4]


# -------------------------------------------------------------- bf16 GEMV ---

def check_fp_tolerance(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.max(np.abs(ref))
    assert np.max(np.abs(got - ref)) <= 1e-3 * scale, np.max(np.abs(got - ref)) / scale
    assert np.linalg.norm(got - ref) <= 1e-4 * np.linalg.norm(ref), np.linalg.norm(got - ref) / np.linalg.norm(ref)


@pytest.mark.parametrize("k", [128, 640, 1024, 1152, 2048, 3072, 4096, 8192, 16384])
@pytest.mark.parametrize("n", [1, 33, 512])
def test_gemv_bf16_within_tolerance(gpu_lib, n, k):
    """Every k class and the generic walk (k = 640, 1152, 16384); a second
    call gives the same bits."""
    say(f"gemv_bf16 n={n} k={k}")
    g = synth.rng(n * 7 + k)
    words = synth.random_words(n * (k // 128) * 5, g)
    sw = synth.row_scales(n, g, np.float16)
    xb = synth.x_bf16_normal(k, g)
    ref = sherry_ref.gemv_bf16(words, sw, n, k, xb)
    x_t = dev(xb.view(np.int16)).view(torch.bfloat16)
    _, y = gpu_lib.gemv(words_dev(words), dev(sw), x_t, None, torch.float32)
    _, y2 = gpu_lib.gemv(words_dev(words), dev(sw), x_t, None, torch.float32)
    torch.cuda.synchronize()
    check_fp_tolerance(y.cpu().numpy(), ref)
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))


# ------------------------------------------------ bf16 GEMM (few tokens) ---

def bf16_dev(xb):
    return dev(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("m", [2, 3, 4, 8, 16])
@pytest.mark.parametrize("n,k", [(1, 128), (37, 384), (100, 1024), (513, 2048), (3072, 3072), (64, 8192),
                                 (300, 4096), (1024, 3072)])
def test_gemm_bf16_within_tolerance(gpu_lib, m, n, k):
    """bf16 X for a few tokens on the matrix cores: every k slice count
    (1 .. 16 slices of 512), ragged rows and tokens; each token's outputs
    within the bf16 tolerance of the exact reference, and a second call
    gives the same bits."""
    say(f"gemm_bf16 m={m} n={n} k={k}")
    g = synth.rng(m * 1000 + n * 7 + k)
    words = synth.random_words(n * (k // 128) * 5, g)
    sw = synth.row_scales(n, g, np.float16 if n % 2 else np.float32)
    xb = synth.x_bf16_normal((m, k), g)
    ref = sherry_ref.gemm_bf16(words, sw, n, k, xb)
    _, y = gpu_lib.gemm(words_dev(words), dev(sw), bf16_dev(xb))
    _, y2 = gpu_lib.gemm(words_dev(words), dev(sw), bf16_dev(xb))
    torch.cuda.synchronize()
    assert y.dtype == torch.float32 and tuple(y.shape) == (m, n)
    got = y.cpu().numpy()
    for t in range(m):
        check_fp_tolerance(got[t], ref[t])
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))


def test_gemm_bf16_strided_x_and_y(gpu_lib):
    """X rows ldx > k elements apart, Y rows ldy > n apart."""
    say("gemm_bf16 strided")
    g = synth.rng(515)
    m, n, k = 5, 700, 3072
    words = synth.random_words(n * (k // 128) * 5, g)
    sw = synth.row_scales(n, g, np.float16)
    big = synth.x_bf16_normal((m, k + 64), g)
    ref = sherry_ref.gemm_bf16(words, sw, n, k, big[:, :k])
    ybig = torch.full((m, n + 40), -7.0, dtype=torch.float32, device=DEV)
    gpu_lib.gemm(words_dev(words), dev(sw), bf16_dev(big)[:, :k], out=ybig[:, :n])
    torch.cuda.synchronize()
    got = ybig.cpu().numpy()
    for t in range(m):
        check_fp_tolerance(got[t, :n], ref[t])
    assert np.all(got[:, n:] == -7.0)


@pytest.mark.parametrize("m", [2, 16])
def test_grouped_gemm_bf16_3b_layer(gpu_lib, m):
    """The seven matrices of a LLaMA-3.2-3B decoder layer at full size with
    bf16 X for m tokens, one grouped launch; every output of every token
    within the bf16 tolerance, and a second launch repeats the bits."""
    say(f"grouped gemm_bf16 3B layer m={m}")
    g = synth.rng(300 + m)
    probs, refs = [], []
    xs = {k: synth.x_bf16_normal((m, k), g) for k in (3072, 8192)}
    for name, n, k in synth.LLAMA32_3B_LAYER:
        words = synth.random_words(n * (k // 128) * 5, g)
        sw = synth.row_scales(n, g, np.float16)
        refs.append(sherry_ref.gemm_bf16(words, sw, n, k, xs[k]))
        probs.append(dict(codes=words_dev(words), scales=dev(sw), x=bf16_dev(xs[k]),
                          y=torch.empty(m, n, dtype=torch.float32, device=DEV)))
    grouped = gpu_lib.GroupedGemm(probs)
    grouped()
    torch.cuda.synchronize()
    first = [p["y"].clone() for p in probs]
    for p, r, (name, n, k) in zip(probs, refs, synth.LLAMA32_3B_LAYER):
        got = p["y"].cpu().numpy()
        for t in range(m):
            check_fp_tolerance(got[t], r[t])
    grouped()
    torch.cuda.synchronize()
    for p, y0 in zip(probs, first):
        assert torch.equal(p["y"].view(torch.int32), y0.view(torch.int32))


# -------------------------------------------------------------------- GEMM ---

@pytest.mark.parametrize("m", [1, 2, 3, 4, 8, 15, 16, 17, 33])
@pytest.mark.parametrize("n,k", [(1, 128), (16, 384), (100, 1024), (513, 2048), (64, 8192), (40, 3072)])
def test_gemm_matches_oracle(gpu_lib, m, n, k):
    say(f"gemm m={m} n={n} k={k}")
    g = synth.rng(m * 1000 + n * 3 + k)
    words = synth.random_words(n * (k // 128) * 5, g)
    sw = synth.row_scales(n, g, np.float16)
    xq, sx, _ = synth.act_absmax_int8(m, k, g)
    ref_acc, ref_y = sherry_ref.gemm_i8(words, sw, n, k, xq, sx, np.float16)
    acc, y = gpu_lib.gemm(words_dev(words), dev(sw), dev(xq), dev(sx), torch.float16, want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), ref_acc)
    assert np.array_equal(y.cpu().numpy().view(np.uint16), ref_y.view(np.uint16))


def test_gemm_strided_x_and_fp32_out(gpu_lib):
    g = synth.rng(99)
    m, n, k, ldx = 5, 96, 1024, 1024 + 32
    words = synth.random_words(n * (k // 128) * 5, g)
    sw = synth.row_scales(n, g, np.float32)
    big = synth.x_int8_uniform((m, ldx), g)
    ref_acc, ref_y = sherry_ref.gemm_i8(words, sw, n, k, big[:, :k], None, np.float32)
    acc, y = gpu_lib.gemm(words_dev(words), dev(sw), dev(big)[:, :k], None, torch.float32, want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), ref_acc)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), ref_y.view(np.uint32))


@pytest.mark.parametrize("m", [1, 2])
@pytest.mark.parametrize("k", [1024, 2048, 3072, 4096, 8192])
def test_gemm_two_tokens_strided(gpu_lib, m, k):
    """m <= 2 with a register-class k (the two-token walk): strided x, no
    token scales, fp32 scales and outputs, ragged rows."""
    say(f"gemm two tokens m={m} k={k}")
    g = synth.rng(4100 + 7 * m + k)
    n, ldx = 1029, k + 32
    words = synth.random_words(n * (k // 128) * 5, g)
    sw = synth.row_scales(n, g, np.float32)
    big = synth.x_int8_uniform((m, ldx), g)
    ref_acc, ref_y = sherry_ref.gemm_i8(words, sw, n, k, big[:, :k], None, np.float32)
    acc, y = gpu_lib.gemm(words_dev(words), dev(sw), dev(big)[:, :k], None, torch.float32, want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), ref_acc)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), ref_y.view(np.uint32))


@pytest.mark.parametrize("m", [64, 100, 128, 200, 300])
@pytest.mark.parametrize("n,k", [(1, 128), (130, 640), (100, 1024), (513, 2048), (64, 8192), (40, 3072)])
def test_gemm_tiled_matches_oracle(gpu_lib, m, n, k):
    """Token counts that take the tiled (prefill) kernel: ragged in tokens and rows."""
    say(f"gemm tiled m={m} n={n} k={k}")
    g = synth.rng(m * 7919 + n * 3 + k)
    words = synth.random_words(n * (k // 128) * 5, g)
    sw = synth.row_scales(n, g, np.float16)
    xq, sx, _ = synth.act_absmax_int8(m, k, g)
    ref_acc, ref_y = sherry_ref.gemm_i8(words, sw, n, k, xq, sx, np.float16)
    acc, y = gpu_lib.gemm(words_dev(words), dev(sw), dev(xq), dev(sx), torch.float16, want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), ref_acc)
    assert np.array_equal(y.cpu().numpy().view(np.uint16), ref_y.view(np.uint16))


def test_gemm_tiled_strided_x_fp32_scales_and_out(gpu_lib):
    say("gemm tiled strided")
    g = synth.rng(1999)
    m, n, k, ldx = 150, 200, 1024, 1024 + 48
    words = synth.random_words(n * (k // 128) * 5, g)
    sw = synth.row_scales(n, g, np.float32)
    big = synth.x_int8_uniform((m, ldx), g)
    ref_acc, ref_y = sherry_ref.gemm_i8(words, sw, n, k, big[:, :k], None, np.float32)
    acc, y = gpu_lib.gemm(words_dev(words), dev(sw), dev(big)[:, :k], None, torch.float32, want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), ref_acc)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), ref_y.view(np.uint32))


def test_gemm_tiled_extreme_accumulators(gpu_lib):
    """All weights +1 or all -1 against x = -128 / 127: the largest sums the
    int32 accumulator sees at K = 8192."""
    say("gemm tiled extremes")
    n, k, m = 4, 8192, 64
    t = np.zeros((n, k), np.int8)
    t[0] = 1
    t[1] = -1
    t[2] = np.where(np.arange(k) % 2 == 0, 1, -1)
    t[3] = np.where(np.arange(k) % 3 == 0, -1, 1)
    t[:, 3::4] = 0  # keep every block 3:4
    words, _ = sherry_ref.pack(t.astype(np.float64))
    sw = np.ones(n, np.float32)
    x = np.full((m, k), 127, np.int8)
    x[1::2] = -128
    ref_acc, _ = sherry_ref.gemm_i8(words, sw, n, k, x, None, np.float32)
    acc, _ = gpu_lib.gemm(words_dev(words), dev(sw), dev(x), None, torch.float32, want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), ref_acc)


@pytest.fixture(params=["tiled", "decode_once", "tiled32"])
def prefill_kernel(request, gpu_lib):
    """Each prefill test runs with every kernel of the large tiles; the
    default is restored afterwards."""
    kind = {"tiled": gpu_lib.PREFILL_TILED, "decode_once": gpu_lib.PREFILL_DECODE_ONCE,
            "tiled32": gpu_lib.PREFILL_TILED32}[request.param]
    gpu_lib.set_prefill_kernel(kind)
    yield request.param
    gpu_lib.set_prefill_kernel(gpu_lib.PREFILL_TILED)


@pytest.mark.parametrize("n,m,k", [(4133, 2930, 1024), (4101, 2900, 2048), (3100, 4000, 3072), (2900, 4100, 8192),
                                   (8193, 1537, 384), (4000, 3100, 1152)])
def test_gemm_large_tiles_every_output(gpu_lib, prefill_kernel, n, m, k):
    """Shapes that take the large (256 x 128) tiles, every output against the
    oracle, with each kernel: ragged rows and tokens; k a multiple of 1024
    (the decode-once kernel takes these: one, two, three and eight runs of
    eight groups) and other k (always the general tiled kernel; odd group
    counts: unaligned row starts)."""
    say(f"gemm large tiles {prefill_kernel} n={n} m={m} k={k}")
    g = synth.rng(n + 3 * m + 7 * k)
    words = synth.random_words(n * (k // 128) * 5, g)
    sw = synth.row_scales(n, g, np.float16)
    xq, sx, _ = synth.act_absmax_int8(m, k, g)
    ref_acc, ref_y = sherry_ref.gemm_i8(words, sw, n, k, xq, sx, np.float16)
    acc, y = gpu_lib.gemm(words_dev(words), dev(sw), dev(xq), dev(sx), torch.float16, want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), ref_acc)
    assert np.array_equal(y.cpu().numpy().view(np.uint16), ref_y.view(np.uint16))


@pytest.mark.parametrize("ks", [(1024, 2048, 1024), (640, 256, 1408)])
def test_grouped_gemm_large_tiles_every_output(gpu_lib, prefill_kernel, ks):
    """A grouped launch with large tiles over three ragged problems (fp32
    scales and outputs, rows of x with a stride): every output.  Group
    counts all multiples of eight (the decode-once kernel) or not (the
    general tiled kernel)."""
    say(f"grouped gemm large tiles {prefill_kernel} k={ks}")
    g = synth.rng(4242 + ks[0])
    m = 1300
    probs, refs = [], []
    for n, k, pad in zip((3000, 5001, 1030), ks, (0, 48, 16)):
        words = synth.random_words(n * (k // 128) * 5, g)
        sw = synth.row_scales(n, g, np.float32)
        big = synth.x_int8_uniform((m, k + pad), g)
        sx = (g.uniform(0.5, 2.0, m)).astype(np.float32)
        refs.append(sherry_ref.gemm_i8(words, sw, n, k, big[:, :k], sx, np.float32))
        probs.append(dict(codes=words_dev(words), scales=dev(sw), x=dev(big)[:, :k], x_scales=dev(sx),
                          acc=torch.empty(m, n, dtype=torch.int32, device=DEV),
                          y=torch.empty(m, n, dtype=torch.float32, device=DEV)))
    grouped = gpu_lib.GroupedGemm(probs)
    grouped()
    torch.cuda.synchronize()
    for p, (ra, ry) in zip(probs, refs):
        assert np.array_equal(p["acc"].cpu().numpy(), ra)
        assert np.array_equal(p["y"].cpu().numpy().view(np.uint32), ry.view(np.uint32))


@pytest.mark.parametrize("name,n,k", [("q", 2048, 2048), ("up", 8192, 2048), ("down", 2048, 8192)])
def test_gemm_prefill_full_size_sampled(gpu_lib, prefill_kernel, name, n, k):
    """LLaMA-3.2-1B prefill at 2048 tokens, the launch the benchmark times;
    64 sampled weight rows checked against every token."""
    say(f"gemm prefill {prefill_kernel} {name} {n}x{k} m=2048")
    g = synth.rng({"q": 77, "up": 78, "down": 79}[name])
    m = 2048
    words = synth.random_words(n * (k // 128) * 5, g)
    sw = synth.row_scales(n, g, np.float16)
    xq, sx, _ = synth.act_absmax_int8(m, k, g)
    acc, y = gpu_lib.gemm(words_dev(words), dev(sw), dev(xq), dev(sx), torch.float16, want_acc=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, n - 1], g.integers(0, n, 62)]))
    sub = sherry_ref.row_words(words, n, k, rows)
    ra, ry = sherry_ref.gemm_i8(sub, sw[rows], len(rows), k, xq, sx, np.float16)
    assert np.array_equal(acc.cpu().numpy()[:, rows], ra)
    assert np.array_equal(y.cpu().numpy()[:, rows].view(np.uint16), ry.view(np.uint16))


@pytest.mark.parametrize("m", [64, 130])
@pytest.mark.parametrize("n,k", [(37, 640), (256, 2048)])
def test_tern2_gemm_tiled(gpu_lib, m, n, k):
    say(f"tern2 gemm tiled m={m} n={n} k={k}")
    g = synth.rng(m + 5 * n + k)
    t = synth.ternary_dense(n, k, g)
    words = tern2_ref.pack(t)
    sw = synth.row_scales(n, g, np.float16)
    xq, sx, _ = synth.act_absmax_int8(m, k, g)
    ref_acc, ref_y = tern2_ref.gemm_i8(words, sw, n, k, xq, sx, np.float16)
    acc, y = gpu_lib.tern2_gemm(words_dev(words), dev(sw), dev(xq), dev(sx), torch.float16, want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), ref_acc)
    assert np.array_equal(y.cpu().numpy().view(np.uint16), ref_y.view(np.uint16))


@pytest.mark.parametrize("tern2", [False, True])
def test_grouped_gemm_small_tiling(gpu_lib, tern2):
    """Several ragged products in one launch (128 x 128 tiles)."""
    say(f"grouped gemm small tern2={tern2}")
    g = synth.rng(515 + tern2)
    shapes = [(300, 1024, 200), (64, 128, 64), (130, 640, 100), (17, 384, 300)]
    probs, refs = [], []
    for n, k, m in shapes:
        sw = synth.row_scales(n, g, np.float16)
        xq, sx, _ = synth.act_absmax_int8(m, k, g)
        if tern2:
            words = tern2_ref.pack(synth.ternary_dense(n, k, g))
            refs.append(tern2_ref.gemm_i8(words, sw, n, k, xq, sx, np.float16))
        else:
            words = synth.random_words(n * (k // 128) * 5, g)
            refs.append(sherry_ref.gemm_i8(words, sw, n, k, xq, sx, np.float16))
        probs.append(dict(codes=words_dev(words), scales=dev(sw), x=dev(xq), x_scales=dev(sx),
                          acc=torch.empty(m, n, dtype=torch.int32, device=DEV),
                          y=torch.empty(m, n, dtype=torch.float16, device=DEV)))
    grouped = gpu_lib.GroupedGemm(probs, tern2=tern2)
    assert grouped.n_tiles == 3 * 2 + 1 + 2 * 1 + 1 * 3
    grouped()
    torch.cuda.synchronize()
    for p, (ra, ry) in zip(probs, refs):
        assert np.array_equal(p["acc"].cpu().numpy(), ra)
        assert np.array_equal(p["y"].cpu().numpy().view(np.uint16), ry.view(np.uint16))


def run_grouped_gemm(gpu_lib, tern2, shapes, seed, n_tiles):
    g = synth.rng(seed)
    probs, refs = [], []
    for n, k, m in shapes:
        sw = synth.row_scales(n, g, np.float16)
        xq, sx, _ = synth.act_absmax_int8(m, k, g)
        if tern2:
            words = tern2_ref.pack(synth.ternary_dense(n, k, g))
            refs.append(tern2_ref.gemm_i8(words, sw, n, k, xq, sx, np.float16))
        else:
            words = synth.random_words(n * (k // 128) * 5, g)
            refs.append(sherry_ref.gemm_i8(words, sw, n, k, xq, sx, np.float16))
        probs.append(dict(codes=words_dev(words), scales=dev(sw), x=dev(xq), x_scales=dev(sx),
                          acc=torch.empty(m, n, dtype=torch.int32, device=DEV),
                          y=torch.empty(m, n, dtype=torch.float16, device=DEV)))
    grouped = gpu_lib.GroupedGemm(probs, tern2=tern2)
    assert grouped.n_tiles == n_tiles
    grouped()
    torch.cuda.synchronize()
    for p, (ra, ry) in zip(probs, refs):
        assert np.array_equal(p["acc"].cpu().numpy(), ra)
        assert np.array_equal(p["y"].cpu().numpy().view(np.uint16), ry.view(np.uint16))


@pytest.mark.parametrize("tern2", [False, True])
def test_grouped_gemm_few_tokens(gpu_lib, tern2):
    """Problems with m <= 16 and k <= 8192 in one launch (few-token kernel):
    ragged rows, m from 1 to 16, and every k-slice class (k / 512 rounded up
    to 1, 2, 4, 8, 16).  Row tiles of 512 rows."""
    say(f"grouped gemm few tokens tern2={tern2}")
    shapes = [(300, 1024, 1), (64, 128, 16), (513, 2048, 7), (17, 8192, 3), (1000, 640, 12), (2048, 3072, 16)]
    run_grouped_gemm(gpu_lib, tern2, shapes, 717 + tern2, 1 + 1 + 2 + 1 + 2 + 4)


@pytest.mark.parametrize("tern2", [False, True])
def test_grouped_gemm_two_tokens(gpu_lib, tern2):
    """Every problem with m <= 2 and a register-class k in one launch (the
    two-token walk): m = 1 and 2, ragged rows, every class.  Row tiles as in
    the grouped GEMV: 1024 rows at k = 1024, 512 at 2048, 256 at 3072 and
    4096, 128 at 8192."""
    say(f"grouped gemm two tokens tern2={tern2}")
    shapes = [(300, 1024, 1), (513, 2048, 2), (17, 8192, 2), (1000, 4096, 1), (257, 3072, 2)]
    run_grouped_gemm(gpu_lib, tern2, shapes, 727 + tern2, 1 + 2 + 1 + 4 + 2)


@pytest.mark.parametrize("tern2", [False, True])
def test_grouped_gemm_few_tokens_long_rows(gpu_lib, tern2):
    """m <= 16 with a k above 8192: the 256 x 16 tiles of the tiled kernel."""
    say(f"grouped gemm few tokens, k > 8192, tern2={tern2}")
    shapes = [(300, 9216, 5), (40, 256, 16)]
    run_grouped_gemm(gpu_lib, tern2, shapes, 718 + tern2, 2 + 1)


@pytest.mark.parametrize("m", [16, 2])
def test_grouped_gemm_few_tokens_layer(gpu_lib, m):
    """The seven LLaMA-3.2-1B matrices at m tokens in one launch (the
    benchmark's small-batch launch), every output checked."""
    say(f"grouped gemm few tokens 1B layer m={m}")
    g = synth.rng(919 + m)
    xs = {}
    probs, refs = [], []
    for name, n, k in synth.LLAMA32_1B_LAYER:
        if k not in xs:
            xq, sx, _ = synth.act_absmax_int8(m, k, g)
            xs[k] = (xq, sx, dev(xq), dev(sx))
        sw = synth.row_scales(n, g, np.float16)
        words = synth.random_words(n * (k // 128) * 5, g)
        refs.append(sherry_ref.gemm_i8(words, sw, n, k, xs[k][0], xs[k][1], np.float16))
        probs.append(dict(codes=words_dev(words), scales=dev(sw), x=xs[k][2], x_scales=xs[k][3],
                          acc=torch.empty(m, n, dtype=torch.int32, device=DEV),
                          y=torch.empty(m, n, dtype=torch.float16, device=DEV)))
    grouped = gpu_lib.GroupedGemm(probs)
    grouped()
    torch.cuda.synchronize()
    for p, (ra, ry), (name, _, _) in zip(probs, refs, synth.LLAMA32_1B_LAYER):
        assert np.array_equal(p["acc"].cpu().numpy(), ra), name
        assert np.array_equal(p["y"].cpu().numpy().view(np.uint16), ry.view(np.uint16)), name


@pytest.mark.parametrize("tern2", [False, True])
def test_grouped_gemm_fp16_outputs_every_output(gpu_lib, prefill_kernel, tern2):
    """fp16 outputs without raw sums (the benchmark's form) on the large
    tiles, more tiles than CUs: every output of four ragged problems with row
    strides that are multiples of 4 (four rows per store; odd row counts end
    with single stores) or odd (single stores), k from 384 to 2048, launched
    twice."""
    say(f"grouped gemm fp16 outputs {prefill_kernel} tern2={tern2}")
    g = synth.rng(808 + tern2)
    m = 1500
    shapes = [(3001, 1024, 3), (2050, 384, 2), (1027, 2048, 0), (4096, 640, 0)]
    probs, refs = [], []
    for n, k, ypad in shapes:
        sw = synth.row_scales(n, g, np.float16)
        if tern2:
            t = synth.ternary_dense(n, k, g)
            words = tern2_ref.pack(t)
        else:
            words = synth.random_words(n * (k // 128) * 5, g)
        xq, sx, _ = synth.act_absmax_int8(m, k, g)
        ref = (tern2_ref if tern2 else sherry_ref).gemm_i8(words, sw, n, k, xq, sx, np.float16)[1]
        ybig = torch.full((m, n + ypad), float("nan"), dtype=torch.float16, device=DEV)
        probs.append(dict(codes=words_dev(words), scales=dev(sw), x=dev(xq), x_scales=dev(sx), y=ybig[:, :n]))
        refs.append((ref, ybig, n))
    grouped = gpu_lib.GroupedGemm(probs, tern2=tern2)
    assert grouped.n_tiles > 256
    for rep in range(2):  # the plan runs twice: no state carried between launches
        grouped()
        torch.cuda.synchronize()
        for ref, ybig, n in refs:
            got = ybig.cpu().numpy()
            assert np.array_equal(got[:, :n].view(np.uint16), ref.view(np.uint16)), (n, rep)
            assert np.isnan(got[:, n:]).all()  # nothing written past the row end
            ybig[:, :n] = float("nan")


@pytest.mark.parametrize("tern2", [False, True])
def test_grouped_gemm_prefill_layer_sampled(gpu_lib, prefill_kernel, tern2):
    """The seven matrices of a LLaMA-3.2-1B layer at 2048 tokens in one launch
    (256 x 192 tiles, the benchmark's launch); 48 sampled rows of every
    matrix checked against every token."""
    say(f"grouped gemm prefill layer {prefill_kernel} tern2={tern2}")
    g = synth.rng(616 + tern2)
    m = 2048
    xs = {}
    probs, keep = [], []
    for name, n, k in synth.LLAMA32_1B_LAYER:
        if k not in xs:
            xq, sx, _ = synth.act_absmax_int8(m, k, g)
            xs[k] = (xq, sx, dev(xq), dev(sx))
        sw = synth.row_scales(n, g, np.float16)
        if tern2:
            t = synth.ternary_dense(n, k, g)
            words = tern2_ref.pack(t)
        else:
            t = None
            words = synth.random_words(n * (k // 128) * 5, g)
        probs.append(dict(codes=words_dev(words), scales=dev(sw), x=xs[k][2], x_scales=xs[k][3],
                          acc=torch.empty(m, n, dtype=torch.int32, device=DEV),
                          y=torch.empty(m, n, dtype=torch.float16, device=DEV)))
        keep.append((name, n, k, words, t, sw))
    grouped = gpu_lib.GroupedGemm(probs, tern2=tern2)
    grouped()
    torch.cuda.synchronize()
    for p, (name, n, k, words, t, sw) in zip(probs, keep):
        rows = np.unique(np.concatenate([[0, n - 1], g.integers(0, n, 46)]))
        xq, sx = xs[k][0], xs[k][1]
        if tern2:
            ra, ry = tern2_ref.gemm_i8(tern2_ref.pack(t[rows]), sw[rows], len(rows), k, xq, sx, np.float16)
        else:
            ra, ry = sherry_ref.gemm_i8(sherry_ref.row_words(words, n, k, rows), sw[rows], len(rows), k, xq, sx,
                                        np.float16)
        assert np.array_equal(p["acc"].cpu().numpy()[:, rows], ra), name
        assert np.array_equal(p["y"].cpu().numpy()[:, rows].view(np.uint16), ry.view(np.uint16)), name


# ------------------------------------------------------ 2-bit comparator ---

@pytest.mark.parametrize("n,k", [(1, 128), (37, 640), (256, 2048), (64, 8192)])
def test_tern2_encode_and_products(gpu_lib, n, k):
    say(f"tern2 n={n} k={k}")
    g = synth.rng(n + 3 * k)
    t = synth.ternary_dense(n, k, g)
    codes = gpu_lib.tern2_encode(dev(t))
    torch.cuda.synchronize()
    ref_words = tern2_ref.pack(t)
    assert np.array_equal(host_words(codes), ref_words)
    sw = synth.row_scales(n, g, np.float16)
    xq, sx, _ = synth.act_absmax_int8(3, k, g)
    ref_acc, ref_y = tern2_ref.gemv_i8(ref_words, sw, n, k, xq[0], sx[0], np.float16)
    acc, y = gpu_lib.tern2_gemv(codes, dev(sw), dev(xq[0]), dev(sx[:1]), torch.float16, want_acc=True)
    ref_acc2, ref_y2 = tern2_ref.gemm_i8(ref_words, sw, n, k, xq, sx, np.float16)
    acc2, y2 = gpu_lib.tern2_gemm(codes, dev(sw), dev(xq), dev(sx), torch.float16, want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), ref_acc)
    assert np.array_equal(y.cpu().numpy().view(np.uint16), ref_y.view(np.uint16))
    assert np.array_equal(acc2.cpu().numpy(), ref_acc2)
    assert np.array_equal(y2.cpu().numpy().view(np.uint16), ref_y2.view(np.uint16))


def test_sherry_and_tern2_agree_on_gpu(gpu_lib):
    """Same 3:4 ternary matrix in both encodings: identical sums and outputs."""
    g = synth.rng(4242)
    n, k = 512, 2048
    t = synth.ternary_34(n, k, g)
    s = synth.row_scales(n, g, np.float32)
    codes5, scales = gpu_lib.pack(dev((t * s[:, None]).astype(np.float32)), torch.float16)
    codes2 = gpu_lib.tern2_encode(dev(t))
    xq, sx, _ = synth.act_absmax_int8(4, k, g)
    a5, y5 = gpu_lib.gemv(codes5, scales, dev(xq[0]), dev(sx[:1]), torch.float16, want_acc=True)
    a2, y2 = gpu_lib.tern2_gemv(codes2, scales, dev(xq[0]), dev(sx[:1]), torch.float16, want_acc=True)
    b5, z5 = gpu_lib.gemm(codes5, scales, dev(xq), dev(sx), torch.float16, want_acc=True)
    b2, z2 = gpu_lib.tern2_gemm(codes2, scales, dev(xq), dev(sx), torch.float16, want_acc=True)
    torch.cuda.synchronize()
    assert torch.equal(a5, a2) and torch.equal(y5, y2)
    assert torch.equal(b5, b2) and torch.equal(z5, z2)
    assert torch.equal(b5[0], a5)


# ----------------------------------------------------------------- grouped ---

def test_grouped_gemv_matches_single_calls_and_oracle(gpu_lib):
    g = synth.rng(31337)
    shapes = [(2048, 2048), (512, 2048), (700, 8192), (256, 1024), (300, 384), (65, 3072), (17, 4096)]
    probs, refs = [], []
    for n, k in shapes:
        words = synth.random_words(n * (k // 128) * 5, g)
        sw = synth.row_scales(n, g, np.float16)
        x = synth.x_int8_uniform(k, g)
        sx = np.array([g.uniform(0.01, 0.03)], np.float32)
        refs.append(sherry_ref.gemv_i8(words, sw, n, k, x, sx[0], np.float16))
        probs.append(dict(codes=words_dev(words), scales=dev(sw), x=dev(x), x_scale=dev(sx),
                          acc=torch.empty(n, dtype=torch.int32, device=DEV),
                          y=torch.empty(n, dtype=torch.float16, device=DEV)))
    grouped = gpu_lib.GroupedGemv(probs)
    grouped()
    torch.cuda.synchronize()
    for p, (ra, ry), (n, k) in zip(probs, refs, shapes):
        assert np.array_equal(p["acc"].cpu().numpy(), ra), (n, k)
        assert np.array_equal(p["y"].cpu().numpy().view(np.uint16), ry.view(np.uint16)), (n, k)
    for p in probs:  # run twice: the plan is reusable
        p["y"].zero_()
    grouped()
    torch.cuda.synchronize()
    for p, (ra, ry) in zip(probs, refs):
        assert np.array_equal(p["y"].cpu().numpy().view(np.uint16), ry.view(np.uint16))


@pytest.mark.parametrize("generic", [False, True])
def test_grouped_gemv_many_problems_every_output(gpu_lib, generic):
    """A plan of 800 problems (more than a benchmark launch over 112 layers
    holds) with ragged row counts over every register class, optionally one
    problem of a generic k; every output of every problem against the
    oracle."""
    say(f"800-problem plan generic={generic}")
    g = synth.rng(800 + generic)
    ks = [1024, 2048, 3072, 4096, 8192]
    shapes = [(int(g.integers(1, 160)), ks[i % 5]) for i in range(800)]
    if generic:
        shapes[17] = (333, 640)
    probs, refs = [], []
    for n, k in shapes:
        words = synth.random_words(n * (k // 128) * 5, g)
        sw = synth.row_scales(n, g, np.float16)
        xq, sx, _ = synth.act_absmax_int8(1, k, g)
        refs.append(sherry_ref.gemv_i8(words, sw, n, k, xq[0], sx[0], np.float16))
        probs.append(dict(codes=words_dev(words), scales=dev(sw), x=dev(xq[0]), x_scale=dev(sx),
                          acc=torch.empty(n, dtype=torch.int32, device=DEV),
                          y=torch.empty(n, dtype=torch.float16, device=DEV)))
    grouped = gpu_lib.GroupedGemv(probs)
    grouped()
    torch.cuda.synchronize()
    for i, (p, (ra, ry)) in enumerate(zip(probs, refs)):
        assert np.array_equal(p["acc"].cpu().numpy(), ra), (i, shapes[i])
        assert np.array_equal(p["y"].cpu().numpy().view(np.uint16), ry.view(np.uint16)), (i, shapes[i])


@pytest.mark.parametrize("shapes,mfma", [
    ([(1024, 3072), (300, 8192), (64, 2048), (1500, 1024), (77, 640), (520, 4096)], False),
    ([(1024, 3072), (200, 16384), (64, 2048)], False),
    ([(1024, 3072), (300, 8192), (64, 2048), (1500, 1024), (77, 640), (520, 4096), (33, 128), (300, 1152)], True),
])
def test_grouped_bf16(gpu_lib, shapes, mfma):
    """VALU kernels (with and without the k = 3072 family) and the
    matrix-core plan: one 16-row column per group of 4 lanes, P = ceil(G / 4)
    columns per row (k = 640, 1152, 128: groups past k; 1500 and 520 rows:
    partial tiles).  The matrix-core results repeat bit for bit."""
    say(f"grouped bf16 mfma={mfma} {shapes}")
    g = synth.rng(2718 + len(shapes))
    probs, refs = [], []
    for n, k in shapes:
        words = synth.random_words(n * (k // 128) * 5, g)
        sw = synth.row_scales(n, g, np.float16)
        xb = synth.x_bf16_normal(k, g)
        refs.append(sherry_ref.gemv_bf16(words, sw, n, k, xb))
        probs.append(dict(codes=words_dev(words), scales=dev(sw), x=dev(xb.view(np.int16)).view(torch.bfloat16),
                          y=torch.empty(n, dtype=torch.float32, device=DEV)))
    grouped = gpu_lib.GroupedGemv(probs, mfma=mfma)
    grouped()
    torch.cuda.synchronize()
    first = [p["y"].clone() for p in probs]
    for p, r in zip(probs, refs):
        check_fp_tolerance(p["y"].cpu().numpy(), r)
    if mfma:
        grouped()
        torch.cuda.synchronize()
        for p, y0 in zip(probs, first):
            assert torch.equal(p["y"].view(torch.int32), y0.view(torch.int32))


def test_grouped_tern2(gpu_lib):
    g = synth.rng(2718)
    probs2, refs2 = [], []
    for n, k in [(512, 2048), (128, 8192)]:
        t = synth.ternary_dense(n, k, g)
        sw = synth.row_scales(n, g, np.float16)
        x = synth.x_int8_uniform(k, g)
        refs2.append(tern2_ref.gemv_i8(tern2_ref.pack(t), sw, n, k, x, None, np.float16))
        probs2.append(dict(codes=gpu_lib.tern2_encode(dev(t)), scales=dev(sw), x=dev(x),
                           acc=torch.empty(n, dtype=torch.int32, device=DEV),
                           y=torch.empty(n, dtype=torch.float16, device=DEV)))
    gpu_lib.GroupedGemv(probs2, tern2=True)()
    torch.cuda.synchronize()
    for p, (ra, ry) in zip(probs2, refs2):
        assert np.array_equal(p["acc"].cpu().numpy(), ra)
        assert np.array_equal(p["y"].cpu().numpy().view(np.uint16), ry.view(np.uint16))


# ------------------------------------------------ full-size LLaMA shapes ---

@pytest.mark.parametrize("layer", ["1b", "3b"])
def test_full_layer_sampled_rows(gpu_lib, layer):
    """Every matrix of a LLaMA-3.2 decoder layer at full size, through the
    grouped launch the benchmark times; 64 sampled rows per matrix checked."""
    g = synth.rng(11 if layer == "1b" else 12)
    shapes = synth.LLAMA32_1B_LAYER if layer == "1b" else synth.LLAMA32_3B_LAYER
    probs, keep = [], []
    for name, n, k in shapes:
        say(f"full {layer} {name} {n}x{k}")
        words = synth.random_words(n * (k // 128) * 5, g)
        sw = synth.row_scales(n, g, np.float16)
        if layer == "1b":
            xq, sx, _ = synth.act_absmax_int8(1, k, g)
            x_t, xs_t = dev(xq[0]), dev(sx)
            y = torch.empty(n, dtype=torch.float16, device=DEV)
            acc = torch.empty(n, dtype=torch.int32, device=DEV)
        else:
            xb = synth.x_bf16_normal(k, g)
            x_t, xs_t = dev(xb.view(np.int16)).view(torch.bfloat16), None
            y = torch.empty(n, dtype=torch.float32, device=DEV)
            acc = None
        probs.append(dict(codes=words_dev(words), scales=dev(sw), x=x_t, x_scale=xs_t, acc=acc, y=y))
        keep.append((words, sw, xq[0] if layer == "1b" else xb, sx if layer == "1b" else None, n, k))
    gpu_lib.GroupedGemv(probs)()
    torch.cuda.synchronize()
    for p, (words, sw, x, sx, n, k) in zip(probs, keep):
        rows = np.unique(np.concatenate([[0, n - 1], g.integers(0, n, 62)]))
        sub = sherry_ref.row_words(words, n, k, rows)
        if layer == "1b":
            ra, ry = sherry_ref.gemv_i8(sub, sw[rows], len(rows), k, x, sx[0], np.float16)
            assert np.array_equal(p["acc"].cpu().numpy()[rows], ra)
            assert np.array_equal(p["y"].cpu().numpy()[rows].view(np.uint16), ry.view(np.uint16))
        else:
            ref = sherry_ref.gemv_bf16(sub, sw[rows], len(rows), k, x)
            check_fp_tolerance(p["y"].cpu().numpy()[rows], ref)


# ------------------------------------------- activation quantization ---

@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("m,k", [(1, 2048), (5, 8192), (3, 100), (2048, 2048), (2, 10000)])
def test_act_quant(gpu_lib, dt, m, k):
    """Per-token absmax int8 on the GPU equals the oracle bit for bit (codes
    and scales); rows include an all-zero token and exact ties."""
    say(f"act quant {dt} m={m} k={k}")
    g = synth.rng(61 + m + k)
    x = g.standard_normal((m, k)).astype(np.float32) * np.float32(g.uniform(0.01, 30.0))
    if m >= 3:
        x[1] = 0.0
        x[2, :5] = [222.25, 11.375, -11.375, 4.375, 0.0]  # s = 1.75, exact ties
        x[2, 5:] = np.clip(x[2, 5:], -200.0, 200.0)
    if dt == "f32":
        host, tx = x, torch.from_numpy(x)
    elif dt == "f16":
        host = x.astype(np.float16)
        tx = torch.from_numpy(host)
    else:
        host = synth.f32_to_bf16_bits(x)
        tx = torch.from_numpy(host.view(np.int16)).view(torch.bfloat16)
    q, s = gpu_lib.act_quant(tx.to(DEV))
    torch.cuda.synchronize()
    rq, rs = act_ref.quantize(host, dt)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), rq)


def test_act_quant_strided_rows(gpu_lib):
    """Rows of a wider buffer (ldx > k) and a 1-D token."""
    g = synth.rng(66)
    full = torch.from_numpy(g.standard_normal((4, 3072)).astype(np.float32)).to(DEV)
    q, s = gpu_lib.act_quant(full[:, :2048])
    q1, s1 = gpu_lib.act_quant(full[2, 1024:3072])
    torch.cuda.synchronize()
    host = full.cpu().numpy()
    rq, rs = act_ref.quantize(host[:, :2048])
    assert np.array_equal(q.cpu().numpy(), rq) and np.array_equal(s.cpu().numpy(), rs)
    rq1, rs1 = act_ref.quantize(host[2:3, 1024:3072])
    assert np.array_equal(q1.cpu().numpy(), rq1[0]) and np.array_equal(s1.cpu().numpy(), rs1)


@pytest.mark.parametrize("m", [1, 16])
def test_quantized_fused_projections(gpu_lib, m):
    """bf16 activations -> int8 on the GPU -> one product over the
    concatenated q | k | v rows (3072 x 2048, shared x) and one over gate | up
    (16384 x 2048), as a decode step runs them; every output checked against
    the oracle chain (quantization, then the int8 product)."""
    say(f"fused qkv / gate-up after activation quant m={m}")
    g = synth.rng(67 + m)
    xb = synth.x_bf16_normal((m, 2048), g)
    xq, sx = gpu_lib.act_quant(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(DEV))
    rq, rs = act_ref.quantize(xb, "bf16")
    for n in (2048 + 512 + 512, 8192 + 8192):
        words = synth.random_words(n * 16 * 5, g)
        sw = synth.row_scales(n, g, np.float16)
        if m == 1:
            acc, y = gpu_lib.gemv(words_dev(words), dev(sw), xq[0], sx, torch.float16, want_acc=True)
            ra, ry = sherry_ref.gemv_i8(words, sw, n, 2048, rq[0], rs[0], np.float16)
        else:
            acc, y = gpu_lib.gemm(words_dev(words), dev(sw), xq, sx, torch.float16, want_acc=True)
            ra, ry = sherry_ref.gemm_i8(words, sw, n, 2048, rq, rs, np.float16)
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy(), ra)
        assert np.array_equal(y.cpu().numpy().view(np.uint16), ry.view(np.uint16))


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n,k", [(256, 1024), (3072, 2048), (300, 384), (2048, 8192), (8192, 2048), (40, 3072)])
def test_gemv_quant(gpu_lib, dt, n, k):
    """fp x quantized inside the GEMV: sums, outputs and the scale equal the
    oracle chain (quantize, then the int8 product) bit for bit."""
    say(f"gemv with in-kernel x quantization {dt} n={n} k={k}")
    g = synth.rng(71 + n + k)
    x = (g.standard_normal(k) * g.uniform(0.01, 20.0)).astype(np.float32)
    x[:5] = [0.0, 222.25 / 8, 11.375 / 8, -11.375 / 8, 4.375 / 8]  # exact ties when 222.25 / 8 is the max
    if dt == "f32":
        host, tx = x, torch.from_numpy(x)
    elif dt == "f16":
        host = x.astype(np.float16)
        tx = torch.from_numpy(host)
    else:
        host = synth.f32_to_bf16_bits(x)
        tx = torch.from_numpy(host.view(np.int16)).view(torch.bfloat16)
    words = synth.random_words(n * (k // 128) * 5, g)
    sw = synth.row_scales(n, g, np.float16)
    acc, y, sx = gpu_lib.gemv_quant(words_dev(words), dev(sw), tx.to(DEV), torch.float16, want_acc=True,
                                    want_scale=True)
    torch.cuda.synchronize()
    rq, rs = act_ref.quantize(host.reshape(1, k), dt)
    ra, ry = sherry_ref.gemv_i8(words, sw, n, k, rq[0], rs[0], np.float16)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(acc.cpu().numpy(), ra)
    assert np.array_equal(y.cpu().numpy().view(np.uint16), ry.view(np.uint16))


def test_prepared_gemv_quant_follows_x(gpu_lib):
    """The prepared call reads x's current contents on every call: two calls
    with x rewritten between them (bf16, the 2048 class, then the 8192 class
    with fp32 x) each equal the oracle chain bit for bit."""
    for n, k, tdt, dt in ((3072, 2048, torch.bfloat16, "bf16"), (512, 8192, torch.float32, "f32")):
        say(f"prepared gemv_quant n={n} k={k} {dt}")
        g = synth.rng(73 + k)
        words = synth.random_words(n * (k // 128) * 5, g)
        sw = synth.row_scales(n, g, np.float16)
        x = torch.empty(k, dtype=tdt, device=DEV)
        call = gpu_lib.PreparedGemvQuant(words_dev(words), dev(sw), x, torch.float16, want_acc=True, want_scale=True)
        for rep in range(2):
            xs = (g.standard_normal(k) * (1.0 + 4.0 * rep)).astype(np.float32)
            if dt == "f32":
                host = xs
                x.copy_(torch.from_numpy(xs))
            else:
                host = synth.f32_to_bf16_bits(xs)
                x.copy_(torch.from_numpy(host.view(np.int16)).view(torch.bfloat16))
            y = call()
            torch.cuda.synchronize()
            rq, rs = act_ref.quantize(host.reshape(1, k), dt)
            ra, ry = sherry_ref.gemv_i8(words, sw, n, k, rq[0], rs[0], np.float16)
            assert np.array_equal(call.scale.cpu().numpy().view(np.uint32), rs.view(np.uint32))
            assert np.array_equal(call.acc.cpu().numpy(), ra)
            assert np.array_equal(y.cpu().numpy().view(np.uint16), ry.view(np.uint16))


def test_gemv_quant_zero_token(gpu_lib):
    """An all-zero x: scale 1, every sum 0."""
    g = synth.rng(72)
    n, k = 130, 2048
    words = synth.random_words(n * (k // 128) * 5, g)
    sw = synth.row_scales(n, g, np.float16)
    acc, y, sx = gpu_lib.gemv_quant(words_dev(words), dev(sw), torch.zeros(k, dtype=torch.bfloat16, device=DEV),
                                    torch.float32, want_acc=True, want_scale=True)
    torch.cuda.synchronize()
    assert sx.item() == 1.0 and not acc.any().item() and not y.any().item()


# --------------------------------------------------- 1.67-bit comparator ---

@pytest.mark.parametrize("n,k", [(1, 128), (37, 640), (256, 2048), (64, 8192), (40, 3072), (300, 2048)])
def test_tern3_encode_and_gemv(gpu_lib, n, k):
    """GPU encode equals the oracle's words; the batch-1 product equals the
    oracle's sums and outputs bit for bit (22- and 86-group classes and the
    generic walk)."""
    say(f"tern3 n={n} k={k}")
    g = synth.rng(5 * n + k)
    t = synth.ternary_dense(n, k, g)
    codes = gpu_lib.tern3_encode(dev(t))
    torch.cuda.synchronize()
    ref_words = tern3_ref.pack(t)
    assert np.array_equal(host_words(codes), ref_words)
    sw = synth.row_scales(n, g, np.float16)
    xq, sx, _ = synth.act_absmax_int8(1, k, g)
    acc, y = gpu_lib.tern3_gemv(codes, dev(sw), dev(xq[0]), dev(sx), torch.float16, want_acc=True)
    torch.cuda.synchronize()
    ra, ry = tern3_ref.gemv_i8(ref_words, sw, n, k, xq[0], sx[0], np.float16)
    assert np.array_equal(acc.cpu().numpy(), ra)
    assert np.array_equal(y.cpu().numpy().view(np.uint16), ry.view(np.uint16))


def test_tern3_grouped(gpu_lib):
    """Grouped 1.67-bit products over ragged problems of every class (22 and
    86 groups, generic), every output checked against the oracle."""
    say("tern3 grouped")
    g = synth.rng(7373)
    shapes = [(2048, 2048), (512, 2048), (300, 8192), (65, 1024), (17, 2048)]
    probs, refs = [], []
    for n, k in shapes:
        t = synth.ternary_dense(n, k, g)
        sw = synth.row_scales(n, g, np.float16)
        xq, sx, _ = synth.act_absmax_int8(1, k, g)
        words = tern3_ref.pack(t)
        refs.append(tern3_ref.gemv_i8(words, sw, n, k, xq[0], sx[0], np.float16))
        probs.append(dict(codes=words_dev(words), scales=dev(sw), x=dev(xq[0]), x_scale=dev(sx),
                          acc=torch.empty(n, dtype=torch.int32, device=DEV),
                          y=torch.empty(n, dtype=torch.float16, device=DEV)))
    grouped = gpu_lib.GroupedGemv(probs, tern3=True)
    assert grouped.n_tiles == 8 + 2 + 3 + 1 + 1
    grouped()
    torch.cuda.synchronize()
    for p, (ra, ry) in zip(probs, refs):
        assert np.array_equal(p["acc"].cpu().numpy(), ra)
        assert np.array_equal(p["y"].cpu().numpy().view(np.uint16), ry.view(np.uint16))


# ------------------------------------------------------------------ probes ---

def test_probes_and_bench_line(gpu_lib):
    """The ceiling probes run and give rates below the published peaks (a
    figure above them would mean cache hits or dropped work), and the
    benchmark's JSON line holds the fields its contract names."""
    import json
    import subprocess
    import sys
    say("probes")
    sink = torch.zeros(256, dtype=torch.int32, device=DEV)
    buf = torch.ones(1 << 26, dtype=torch.int32, device=DEV)
    gpu_lib.probe_read(buf, sink)
    for mode in range(7):
        gpu_lib.probe_rates(mode, 64, 256, sink)
    torch.cuda.synchronize()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--probes"], capture_output=True, text=True,
                       timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    pk = json.loads(r.stdout.strip().splitlines()[-1])
    assert 0.5 < pk["read_1GiB_TBps"] < 8.0
    assert 10 < pk["mfma_i8_TOPS"] < 5000 and 10 < pk["mfma32_i8_TOPS"] < 5000
    assert 1 < pk["dot4_i8_TOPS"] < 2 * 314.6  # 314.6: 1024 SIMDs x 64 lanes x 8 ops / 4 cycles x 2.4 GHz
    say("bench line")
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--steps", "5", "--warmup", "2", "--replicas",
                        "8", "--no-extras", "--no-cpu-baseline"], capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 5 and line["value"] > 0
    assert "workload" in line["config"]
    rf = line["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and 0 < rf["frac"] < 1 and rf["peak"] == 8000.0
