"""libsherry.so on the host: it loads, exports every function the headers in
include/ declare, and rejects invalid arguments before any HIP call (no GPU
needed)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sherry.h")
# SHERRY_TEST_LIB selects another build of the library (the sanitized one of
# tests/test_abi_sanitized.py); default: the in-tree library
LIB = os.environ.get("SHERRY_TEST_LIB") or os.path.join(ROOT, "ultra_bit_weight_amd", "lib", "libsherry.so")

OK, EINVAL, ESHAPE, EDTYPE, EALIGN, EDEVICE, ESCRATCH = 0, 1, 2, 3, 4, 5, 7
I8, I32, F16, BF16, F32 = 0, 1, 2, 3, 4
A = 0x10000  # a fake, well-aligned non-null "device" address: never dereferenced


def declared_functions(paths=None):
    names = set()
    for path in paths or sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names.update(re.findall(r"\b(\w+)\s*\([^;{]*\)\s*;", text))
    return sorted(n for n in names if n.startswith(("sherry_", "tern2_", "tern3_")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} missing: build with __graft_entry__.build()")
    from ultra_bit_weight_amd import sherry

    return sherry.load(LIB)


def test_header_declares_the_api():
    names = declared_functions([HEADER])
    for required in ("sherry_pack", "sherry_gemv", "sherry_gemm", "sherry_gemv_grouped", "tern2_gemv"):
        assert required in names
    assert len(names) >= 14


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(raw, name), f"{name} declared in include/ but not exported"


def test_version_and_status_strings(lib):
    assert lib.sherry_version().decode().count(".") == 2
    for s in range(8):
        assert lib.sherry_status_str(s).decode().startswith("SHERRY_")
    assert lib.sherry_status_str(99).decode() == "SHERRY_UNKNOWN_STATUS"


def test_set_prefill_kernel(lib):
    """The one process-wide setting: the three kinds accepted (and left at
    the default), anything else EINVAL; no device needed."""
    assert lib.sherry_set_prefill_kernel(1) == 0
    assert lib.sherry_set_prefill_kernel(2) == 0
    assert lib.sherry_set_prefill_kernel(0) == 0
    for bad in (3, -1, 99):
        assert lib.sherry_set_prefill_kernel(bad) == 1


def test_packed_bytes(lib):
    assert lib.sherry_packed_bytes(256, 1024) == 256 * 1024 * 5 // 32
    assert lib.sherry_packed_bytes(2048, 8192) == 2048 * 8192 * 5 // 32
    assert lib.sherry_packed_bytes(1, 128) == 20
    for n, k in [(0, 128), (4, 0), (4, 100), (-1, 128), (4, 129)]:
        assert lib.sherry_packed_bytes(n, k) == 0
    assert lib.tern2_packed_bytes(256, 1024) == 256 * 1024 // 4
    assert lib.tern2_packed_bytes(3, 100) == 0


def gemv(lib, codes=A, sw=A, s_dt=F16, n=64, k=1024, x=A, x_dt=I8, xs=None, acc=A, y=A, y_dt=F16, fn="sherry_gemv"):
    return getattr(lib, fn)(codes, sw, s_dt, n, k, x, x_dt, xs, acc, y, y_dt, None)


@pytest.mark.parametrize("fn", ["sherry_gemv", "tern2_gemv"])
def test_gemv_validation(lib, fn):
    assert gemv(lib, codes=None, fn=fn) == EINVAL
    assert gemv(lib, sw=None, fn=fn) == EINVAL
    assert gemv(lib, x=None, fn=fn) == EINVAL
    assert gemv(lib, acc=None, y=None, fn=fn) == EINVAL
    assert gemv(lib, n=0, fn=fn) == EINVAL
    assert gemv(lib, k=-128, fn=fn) == EINVAL
    assert gemv(lib, k=1000, fn=fn) == ESHAPE
    assert gemv(lib, n=2 ** 31, fn=fn) == ESHAPE
    assert gemv(lib, s_dt=BF16, fn=fn) == EDTYPE
    assert gemv(lib, x_dt=F32, fn=fn) == EDTYPE
    assert gemv(lib, y_dt=I8, fn=fn) == EDTYPE
    assert gemv(lib, codes=A + 2, fn=fn) == EALIGN
    assert gemv(lib, x=A + 4, fn=fn) == EALIGN
    assert gemv(lib, sw=A + 1, fn=fn) == EALIGN
    assert gemv(lib, y=A + 1, fn=fn) == EALIGN
    assert gemv(lib, acc=A + 2, fn=fn) == EALIGN
    # valid arguments: the first HIP call finds no gfx950 device here
    assert gemv(lib, fn=fn) == EDEVICE


@pytest.mark.parametrize("fn, row_bytes", [("sherry_gemv", 64 * 20), ("tern2_gemv", 64 * 32),
                                           ("tern3_gemv", 86 * 20), ("sherry_gemm", 64 * 20),
                                           ("tern2_gemm", 64 * 32)])
def test_codes_below_4gib(lib, fn, row_bytes):
    """The kernels address one matrix's codes with 32-bit byte offsets: the
    largest accepted n at k = 8192 is the last whose codes fit 2^32 - 1 bytes
    in that format (5 words per 128 weights, 8 for the 2-bit codes, 5 per 96
    weights for the 1.67-bit codes)."""
    n_max = (2 ** 32 - 1) // row_bytes
    call = gemm if fn.endswith("gemm") else gemv
    extra = {"ldx": 8192, "ldy": n_max + 1} if fn.endswith("gemm") else {}
    assert call(lib, n=n_max, k=8192, fn=fn, **extra) == EDEVICE
    assert call(lib, n=n_max + 1, k=8192, fn=fn, **extra) == ESHAPE


def test_gemm_x_below_4gib(lib):
    m_max = (2 ** 32 - 1) // 8192
    assert gemm(lib, m=m_max, k=8192, ldx=8192) == EDEVICE
    assert gemm(lib, m=m_max + 1, k=8192, ldx=8192) == ESHAPE


def test_gemv_bf16_rules(lib):
    assert gemv(lib, x_dt=BF16, acc=None, y_dt=F32) == EDEVICE  # valid
    assert gemv(lib, x_dt=BF16, acc=A, y_dt=F32) == EDTYPE       # no int32 sums for bf16
    assert gemv(lib, x_dt=BF16, acc=None, y_dt=F16) == EDTYPE
    assert gemv(lib, x_dt=BF16, acc=None, y_dt=F32, xs=A) == EDTYPE
    assert gemv(lib, x_dt=BF16, acc=None, y=None) == EINVAL
    assert gemv(lib, x_dt=BF16, acc=None, y_dt=F32, fn="tern2_gemv") == EDTYPE


@pytest.mark.parametrize("fn", ["sherry_pack", "tern2_pack"])
def test_pack_validation(lib, fn):
    f = getattr(lib, fn)
    assert f(None, F32, 8, 128, 128, A, A, F16, None) == EINVAL
    assert f(A, F32, 8, 128, 128, None, A, F16, None) == EINVAL
    assert f(A, F32, 8, 100, 100, A, A, F16, None) == ESHAPE
    assert f(A, F32, 8, 128, 64, A, A, F16, None) == ESHAPE
    assert f(A, I8, 8, 128, 128, A, A, F16, None) == EDTYPE
    assert f(A, F32, 8, 128, 128, A, A, BF16, None) == EDTYPE
    assert f(A + 4, F32, 8, 128, 128, A, A, F16, None) == EALIGN
    assert f(A, F32, 8, 128, 130, A, A, F16, None) == EALIGN
    assert f(A, F32, 8, 128, 128, A, A, F16, None) == EDEVICE


def gemm(lib, codes=A, sw=A, s_dt=F16, n=64, k=1024, x=A, x_dt=I8, m=4, ldx=1024, xs=A, acc=A, y=A, y_dt=F16,
         ldy=64, fn="sherry_gemm"):
    return getattr(lib, fn)(codes, sw, s_dt, n, k, x, x_dt, m, ldx, xs, acc, y, y_dt, ldy, None)


@pytest.mark.parametrize("fn", ["sherry_gemm", "tern2_gemm"])
def test_gemm_validation(lib, fn):
    assert gemm(lib, x=None, fn=fn) == EINVAL
    assert gemm(lib, m=0, fn=fn) == EINVAL
    assert gemm(lib, acc=None, y=None, fn=fn) == EINVAL
    assert gemm(lib, k=1000, ldx=1008, fn=fn) == ESHAPE
    assert gemm(lib, ldx=1000, fn=fn) == ESHAPE
    assert gemm(lib, ldx=1032, fn=fn) == ESHAPE
    assert gemm(lib, ldy=32, fn=fn) == ESHAPE
    assert gemm(lib, x_dt=BF16, fn=fn) == EDTYPE
    assert gemm(lib, y_dt=I32, fn=fn) == EDTYPE
    assert gemm(lib, x=A + 8, fn=fn) == EALIGN
    assert gemm(lib, xs=A + 2, fn=fn) == EALIGN
    assert gemm(lib, fn=fn) == EDEVICE
    assert gemm(lib, xs=None, acc=None, fn=fn) == EDEVICE


def test_gemm_bf16_validation(lib):
    """bf16 X: 3:4 codes only, m <= 16, k <= 8192, fp32 Y, no token scales
    and no int32 sums; ldx counts elements (a multiple of 8: 16-byte rows)."""
    ok = dict(x_dt=BF16, xs=None, acc=None, y_dt=F32)
    assert gemm(lib, **ok) == EDEVICE
    assert gemm(lib, **dict(ok, ldx=1032)) == EDEVICE        # 8-element multiple
    assert gemm(lib, **dict(ok, ldx=1028)) == ESHAPE
    assert gemm(lib, **dict(ok, m=16)) == EDEVICE
    assert gemm(lib, **dict(ok, m=17)) == ESHAPE
    assert gemm(lib, **dict(ok, k=8192, ldx=8192)) == EDEVICE
    assert gemm(lib, **dict(ok, k=8320, ldx=8320)) == ESHAPE
    assert gemm(lib, **dict(ok, y_dt=F16)) == EDTYPE
    assert gemm(lib, **dict(ok, xs=A)) == EDTYPE
    assert gemm(lib, **dict(ok, acc=A)) == EDTYPE
    assert gemm(lib, **dict(ok, y=None)) == EINVAL          # neither acc nor y
    assert gemm(lib, **dict(ok, fn="tern2_gemm")) == EDTYPE


def test_act_quant_validation(lib):
    f = lib.sherry_act_quant
    assert f(None, F32, 2, 128, 128, A, 128, A, None) == EINVAL
    assert f(A, F32, 2, 128, 128, None, 128, A, None) == EINVAL
    assert f(A, F32, 2, 128, 128, A, 128, None, None) == EINVAL
    assert f(A, F32, 0, 128, 128, A, 128, A, None) == EINVAL
    assert f(A, F32, 2, 0, 128, A, 128, A, None) == EINVAL
    assert f(A, I8, 2, 128, 128, A, 128, A, None) == EDTYPE
    assert f(A, I32, 2, 128, 128, A, 128, A, None) == EDTYPE
    assert f(A, F32, 2, 128, 100, A, 128, A, None) == ESHAPE
    assert f(A, F32, 2, 128, 128, A, 127, A, None) == ESHAPE
    assert f(A, F32, 2 ** 31, 128, 128, A, 128, A, None) == ESHAPE
    assert f(A + 2, F32, 2, 128, 128, A, 128, A, None) == EALIGN
    assert f(A + 1, BF16, 2, 128, 128, A, 128, A, None) == EALIGN
    assert f(A, F32, 2, 128, 128, A, 128, A + 2, None) == EALIGN
    assert f(A + 2, F16, 2, 100, 100, A + 1, 100, A, None) == EDEVICE  # valid: odd k, ld, 2-byte x
    assert f(A, BF16, 1, 8192, 8192, A, 8192, A, None) == EDEVICE


def test_gemv_quant_validation(lib):
    def call(codes=A, sw=A, s_dt=F16, n=64, k=1024, x=A, x_dt=BF16, xs=None, acc=A, y=A, y_dt=F16):
        return lib.sherry_gemv_quant(codes, sw, s_dt, n, k, x, x_dt, xs, acc, y, y_dt, None)
    assert call(codes=None) == EINVAL
    assert call(x=None) == EINVAL
    assert call(acc=None, y=None) == EINVAL
    assert call(k=1000) == ESHAPE
    assert call(k=8192 + 128) == ESHAPE
    assert call(x_dt=I8) == EDTYPE
    assert call(s_dt=BF16) == EDTYPE
    assert call(y_dt=I8) == EDTYPE
    assert call(x=A + 1) == EALIGN
    assert call(x=A + 2, x_dt=F32) == EALIGN
    assert call(xs=A + 2) == EALIGN
    assert call(x=A + 2, x_dt=F16, xs=A) == EDEVICE  # valid
    assert call(k=8192, x_dt=F32, acc=None) == EDEVICE


def test_tern3_sizes_and_validation(lib):
    assert lib.tern3_packed_bytes(1, 2048) == 22 * 20
    assert lib.tern3_packed_bytes(3, 8192) == 3 * 86 * 20
    assert lib.tern3_packed_bytes(2, 128) == 2 * 2 * 20
    assert lib.tern3_packed_bytes(2, 100) == 0
    f = lib.tern3_encode
    assert f(None, 4, 128, 128, A, None) == EINVAL
    assert f(A, 4, 96, 96, A, None) == ESHAPE
    assert f(A, 4, 128, 120, A, None) == ESHAPE
    assert f(A + 8, 4, 128, 128, A, None) == EALIGN
    assert f(A, 4, 128, 128, A, None) == EDEVICE
    assert gemv(lib, fn="tern3_gemv", x_dt=BF16, acc=None, y_dt=F32) == EDTYPE
    assert gemv(lib, fn="tern3_gemv") == EDEVICE
    from ultra_bit_weight_amd.sherry import GemvProblem
    arr = (GemvProblem * 2)()
    arr[0] = GemvProblem(A, A, 1024, 2048, A, None, None, A)  # 22 groups: 32 lanes, 8 rows per iteration
    arr[1] = GemvProblem(A, A, 300, 8192, A, None, None, A)   # 86 groups: 64 lanes, 4 rows per iteration
    nbytes = lib.tern3_gemv_plan_bytes(arr, 2)
    assert nbytes == 64 + 64 * 2 + 8 * (4 + 3)
    buf = ctypes.create_string_buffer(nbytes + 8)
    base = (ctypes.addressof(buf) + 7) // 8 * 8
    assert lib.tern3_gemv_plan(arr, 2, F16, I8, F16, base, nbytes) == OK
    assert int.from_bytes(ctypes.string_at(base + 12, 4), "little") == 7


def test_decode_validation(lib):
    f = lib.sherry_decode
    assert f(None, 4, 128, A, 128, None) == EINVAL
    assert f(A, 4, 100, A, 112, None) == ESHAPE
    assert f(A, 4, 128, A, 112, None) == ESHAPE
    assert f(A, 4, 128, A + 8, 128, None) == EALIGN
    assert f(A, 4, 128, A, 136, None) == EALIGN
    assert f(A, 4, 128, A, 128, None) == EDEVICE


def test_tern2_encode_validation(lib):
    f = lib.tern2_encode
    assert f(None, 4, 128, 128, A, None) == EINVAL
    assert f(A, 4, 96, 96, A, None) == ESHAPE
    assert f(A, 4, 128, 120, A, None) == ESHAPE
    assert f(A, 4, 128, 136, A, None) == EALIGN
    assert f(A + 8, 4, 128, 128, A, None) == EALIGN
    assert f(A, 4, 128, 128, A, None) == EDEVICE


def test_grouped_plan_on_host(lib):
    from ultra_bit_weight_amd.sherry import GemvProblem

    shapes = [(2048, 2048), (512, 2048), (2048, 8192), (256, 1024), (300, 384)]
    arr = (GemvProblem * len(shapes))()
    for i, (n, k) in enumerate(shapes):
        arr[i] = GemvProblem(A, A, n, k, A, None, None, A)
    nbytes = lib.sherry_gemv_plan_bytes(arr, len(shapes))
    # 64-byte header + 64 bytes per problem + 8 bytes per tile; tile rows are
    # 32 iterations x rows per iteration (4 waves x 64 / lanes per row):
    # k=2048 -> 16 lanes -> 512 rows, k=8192 -> 64 lanes -> 128 rows,
    # k=1024 -> 8 lanes -> 1024 rows, other k -> 64 lanes -> 128 rows
    tiles = 4 + 1 + 16 + 1 + 3
    assert nbytes == 64 + 64 * len(shapes) + 8 * tiles
    buf = ctypes.create_string_buffer(nbytes + 8)
    base = (ctypes.addressof(buf) + 7) // 8 * 8
    assert lib.sherry_gemv_plan(arr, len(shapes), F16, I8, F16, base, nbytes) == OK
    hdr = ctypes.string_at(base, 16)
    assert int.from_bytes(hdr[8:12], "little") == len(shapes)
    assert int.from_bytes(hdr[12:16], "little") == tiles
    # tiles of the longest rows come first (k = 8192, then 2048, 1024, 384)
    raw = ctypes.string_at(base + 64 + 64 * len(shapes), 8 * tiles)
    order = [(int.from_bytes(raw[8 * t:8 * t + 4], "little"), int.from_bytes(raw[8 * t + 4:8 * t + 8], "little"))
             for t in range(tiles)]
    assert order == ([(2, 128 * j) for j in range(16)] + [(0, 0), (0, 512), (0, 1024), (0, 1536), (1, 0)] +
                     [(3, 0)] + [(4, 0), (4, 128), (4, 256)])
    assert lib.sherry_gemv_plan(arr, len(shapes), F16, I8, F16, base, nbytes - 8) == EINVAL
    assert lib.sherry_gemv_plan(arr, len(shapes), F16, F32, F16, base, nbytes) == EDTYPE
    assert lib.sherry_gemv_plan(arr, len(shapes), F16, I8, F16, base + 4, nbytes) == EALIGN
    arr[1].k = 100
    assert lib.sherry_gemv_plan_bytes(arr, len(shapes)) == 0
    assert lib.sherry_gemv_plan(arr, len(shapes), F16, I8, F16, base, nbytes) == ESHAPE
    # a malformed host plan is rejected before any device call
    bad = ctypes.create_string_buffer(64)
    assert lib.sherry_gemv_grouped(ctypes.addressof(bad), A, None) == EINVAL
    assert lib.sherry_gemv_grouped(None, A, None) == EINVAL


def test_grouped_noalloc_validation(lib):
    """sherry_gemv_grouped_noalloc checks the host plan before any device
    call: a null or misaligned plan, a malformed header or a byte count short
    of the records is rejected, a plan above the 1 MiB static plan memory is
    ESCRATCH, and the largest plan that fits reaches the device check (no
    gfx950 device here).  Problems of 256 x 1024 take one tile each, so a plan
    of c problems is 64 + 72 c bytes."""
    from ultra_bit_weight_amd.sherry import GemvProblem

    def plan(count):
        arr = (GemvProblem * count)()
        for i in range(count):
            arr[i] = GemvProblem(A, A, 256, 1024, A, None, None, A)
        nbytes = lib.sherry_gemv_plan_bytes(arr, count)
        assert nbytes == 64 + 72 * count
        buf = ctypes.create_string_buffer(nbytes + 8)
        base = (ctypes.addressof(buf) + 7) // 8 * 8
        assert lib.sherry_gemv_plan(arr, count, F16, I8, F16, base, nbytes) == OK
        return buf, base, nbytes

    buf, base, nbytes = plan(3)
    assert lib.sherry_gemv_grouped_noalloc(base, None) == EDEVICE
    assert lib.sherry_gemv_grouped_noalloc(None, None) == EINVAL
    assert lib.sherry_gemv_grouped_noalloc(base + 4, None) == EALIGN
    ctypes.memmove(base + 32, (nbytes - 8).to_bytes(8, "little"), 8)  # byte count short of the last tile
    assert lib.sherry_gemv_grouped_noalloc(base, None) == EINVAL
    ctypes.memmove(base + 32, nbytes.to_bytes(8, "little"), 8)
    ctypes.memmove(base, b"\0\0\0\0", 4)  # magic
    assert lib.sherry_gemv_grouped_noalloc(base, None) == EINVAL
    fit = (2 ** 20 - 64) // 72
    buf, base, nbytes = plan(fit)
    assert nbytes <= 2 ** 20 and lib.sherry_gemv_grouped_noalloc(base, None) == EDEVICE
    buf, base, nbytes = plan(fit + 1)
    assert nbytes > 2 ** 20 and lib.sherry_gemv_grouped_noalloc(base, None) == ESCRATCH
    assert "static plan memory" in lib.sherry_status_str(ESCRATCH).decode()


def test_grouped_plan_tiles_by_x_type(lib):
    """int8 x at k = 3072 puts one group in each of 24 of 32 lanes (8 rows per
    iteration, 256-row tiles; k = 2048: 512-row tiles); bf16 x keeps 3 groups
    in each of 8 lanes at k = 3072 (1024-row tiles, reserved[0] set).  The
    matrix-core plan (bf16 x, every k <= 8192) takes tiles of max(256, the
    int8 tile) rows and sets reserved[1].  The plan size covers the int8
    tiling, the largest."""
    from ultra_bit_weight_amd.sherry import GemvProblem

    def header(arr, count, x_dt, y_dt, fn=lib.sherry_gemv_plan):
        nbytes = lib.sherry_gemv_plan_bytes(arr, count)
        buf = ctypes.create_string_buffer(nbytes + 8)
        base = (ctypes.addressof(buf) + 7) // 8 * 8
        st = fn(arr, count, F16, x_dt, y_dt, base, nbytes)
        if st != OK:
            return st
        hdr = ctypes.string_at(base, 64)
        return (int.from_bytes(hdr[12:16], "little"), int.from_bytes(hdr[40:48], "little"),
                int.from_bytes(hdr[48:56], "little"))

    arr = (GemvProblem * 3)()
    arr[0] = GemvProblem(A, A, 1024, 3072, A, None, None, A)
    arr[1] = GemvProblem(A, A, 300, 2048, A, None, None, A)
    arr[2] = GemvProblem(A, A, 300, 16384, A, None, None, A)
    assert lib.sherry_gemv_plan_bytes(arr, 2) == 64 + 64 * 2 + 8 * (4 + 1)
    assert header(arr, 2, I8, F16) == (5, 0, 0)
    assert header(arr, 2, I8, F16, lib.sherry_gemv_plan_mfma) == EDTYPE
    for a in arr:
        a.x_scale = None
        a.acc = None
    assert header(arr, 2, BF16, F32) == (1 + 1, 1, 0)
    assert header(arr, 2, BF16, F32, lib.sherry_gemv_plan_mfma) == (4 + 1, 1, 1)
    # k = 16384 (generic class, 128-row tiles): beyond the matrix-core kernel
    assert header(arr, 3, BF16, F32) == (1 + 1 + 3, 1, 0)
    assert header(arr, 3, BF16, F32, lib.sherry_gemv_plan_mfma) == ESHAPE


def test_grouped_gemm_plan_on_host(lib):
    from ultra_bit_weight_amd.sherry import GemmProblem

    def problems(shapes):
        arr = (GemmProblem * len(shapes))()
        for i, (n, k, m) in enumerate(shapes):
            arr[i] = GemmProblem(A, A, n, k, A, m, k, None, None, A, n)
        return arr

    def tiles_of(base, count, n_tiles):
        raw = ctypes.string_at(base + 64 + 80 * count, 16 * n_tiles)
        return [tuple(int.from_bytes(raw[16 * t + 4 * f:16 * t + 4 * f + 4], "little") for f in range(3))
                for t in range(n_tiles)]

    # a prefill layer (LLaMA-3.2-1B, 2000 tokens): 256 x 128 tiles (16 token
    # tiles, the last one ragged), longest rows first
    layer = [(2048, 2048, 2000), (512, 2048, 2000), (512, 2048, 2000), (2048, 2048, 2000), (8192, 2048, 2000),
             (8192, 2048, 2000), (2048, 8192, 2000)]
    arr = problems(layer)
    TT = 16  # token tiles of 128
    n_tiles = (8 + 2 + 2 + 8 + 32 + 32 + 8) * TT
    nbytes = lib.sherry_gemm_plan_bytes(arr, len(layer))
    assert nbytes == 64 + 80 * len(layer) + 16 * n_tiles
    buf = ctypes.create_string_buffer(nbytes + 8)
    base = (ctypes.addressof(buf) + 7) // 8 * 8
    assert lib.sherry_gemm_plan(arr, len(layer), F16, I8, F16, base, nbytes) == OK
    hdr = ctypes.string_at(base, 64)
    assert int.from_bytes(hdr[8:12], "little") == len(layer)
    assert int.from_bytes(hdr[12:16], "little") == n_tiles
    assert int.from_bytes(hdr[40:48], "little") == 1  # 256 x 128 tiling
    t = tiles_of(base, len(layer), n_tiles)
    # eight interleaved lists, one per XCD (workgroup w runs on XCD w % 8):
    # XCD c takes share c of every problem's tiles (listed token tile by token
    # tile), problems with the longest rows (down, k = 8192) first; shares of
    # equal count, the remainders dealt to the XCDs in turn
    assert sorted(t) == sorted((i, a, b) for i, (n, _, _) in enumerate(layer) for a in range(n // 256)
                               for b in range(TT)) and len(set(t)) == n_tiles
    lists = [t[c::8] for c in range(8)]
    assert [len(x) for x in lists] == [184] * 8  # 1472 = 8 * 184
    nxt = 0
    for i in (6, 0, 1, 2, 3, 4, 5):
        tn = layer[i][0] // 256
        seq = [(i, u % tn, u // tn) for u in range(TT * tn)]
        q, r = divmod(len(seq), 8)
        u = 0
        for c in range(8):
            share = q + (1 if (c - nxt) % 8 < r else 0)
            assert [x for x in lists[c] if x[0] == i] == seq[u:u + share], (i, c)
            u += share
        nxt = (nxt + r) % 8
    # the XCD lists hold the problems in order: down first
    assert all([x[0] for x in lst] == sorted((x[0] for x in lst), key=(6, 0, 1, 2, 3, 4, 5).index)
               for lst in lists)
    assert t[0] == (6, 0, 0) and t[1] == (6, 0, 2) and t[-1][0] == 5
    assert lib.tern2_gemm_plan(arr, len(layer), F16, I8, F16, base, nbytes) == OK
    # a small set of problems: 128 x 128 tiles (ragged in rows and tokens)
    small = [(300, 1024, 200), (64, 128, 64)]
    arr2 = problems(small)
    n2 = 3 * 2 + 1 * 1
    nb2 = lib.sherry_gemm_plan_bytes(arr2, len(small))
    assert nb2 == 64 + 80 * 2 + 16 * n2
    assert lib.sherry_gemm_plan(arr2, 2, F16, I8, F16, base, nb2) == OK
    assert int.from_bytes(ctypes.string_at(base + 40, 8), "little") == 0
    # fewer tiles than one round of XCD runs: the logical order
    assert tiles_of(base, 2, n2) == [(0, a, b) for b in range(2) for a in range(3)] + [(1, 0, 0)]
    # validation: buffer too small, bad dtype, misaligned, bad shape, bad m
    assert lib.sherry_gemm_plan(arr2, 2, F16, I8, F16, base, nb2 - 8) == EINVAL
    assert lib.sherry_gemm_plan(arr2, 2, F16, BF16, F16, base, nb2) == EDTYPE
    assert lib.sherry_gemm_plan(arr2, 2, F16, BF16, F32, base, nb2) == ESHAPE  # bf16 x: at most 16 tokens
    assert lib.sherry_gemm_plan(arr2, 2, F16, I8, F16, base + 4, nb2) == EALIGN
    arr2[1].k = 100
    assert lib.sherry_gemm_plan_bytes(arr2, 2) == 0
    assert lib.sherry_gemm_plan(arr2, 2, F16, I8, F16, base, nb2) == ESHAPE
    arr2[1].k = 128
    arr2[1].m = 0
    assert lib.sherry_gemm_plan(arr2, 2, F16, I8, F16, base, nb2) == EINVAL
    # every problem with m <= 16 and k <= 8192: the few-token kernel, row
    # tiles of 512 rows for every k
    few = [(2048, 2048, 16), (300, 1024, 3), (300, 8192, 1)]
    arr3 = problems(few)
    n3 = 4 + 1 + 1
    nb3 = lib.sherry_gemm_plan_bytes(arr3, 3)
    # room for the bf16 tiling too (every m <= 16, k <= 8192): 1024-row tiles
    n3_bf16 = 2 + 1 + 1
    assert nb3 == 64 + 80 * 3 + 16 * max(n3, n3_bf16)
    assert lib.sherry_gemm_plan(arr3, 3, F16, I8, F16, base, nb3) == OK
    assert int.from_bytes(ctypes.string_at(base + 40, 8), "little") == 3
    assert tiles_of(base, 3, n3) == [(2, 0, 0)] + [(0, a, 0) for a in range(4)] + [(1, 0, 0)]
    # the same problems with bf16 x (fp32 y, no token scales): tiling 5,
    # 1024-row tiles, longest rows first
    assert lib.sherry_gemm_plan(arr3, 3, F16, BF16, F32, base, nb3) == OK
    hdr = ctypes.string_at(base, 64)
    assert int.from_bytes(hdr[12:16], "little") == n3_bf16 and int.from_bytes(hdr[40:48], "little") == 5
    assert tiles_of(base, 3, n3_bf16) == [(2, 0, 0), (0, 0, 0), (0, 1, 0), (1, 0, 0)]
    assert lib.sherry_gemm_plan(arr3, 3, F16, BF16, F16, base, nb3) == EDTYPE
    assert lib.tern2_gemm_plan(arr3, 3, F16, BF16, F32, base, nb3) == EDTYPE
    arr3[0].m = 17
    assert lib.sherry_gemm_plan(arr3, 3, F16, BF16, F32, base, nb3) == ESHAPE
    arr3[0].m = 16
    # every problem with m <= 2 and a register-class k: the two-token walk
    # (tiling 4), row tiles of the grouped GEMV: 512 rows at k = 2048, 1024 at
    # 1024, 256 at 3072, 128 at 8192; longest rows first
    two = [(2048, 2048, 2), (300, 1024, 1), (300, 8192, 2), (100, 3072, 1)]
    arr5 = problems(two)
    n5 = 4 + 1 + 3 + 1
    nb5 = lib.sherry_gemm_plan_bytes(arr5, 4)
    assert nb5 == 64 + 80 * 4 + 16 * max(n5, 2 + 1 + 1 + 1)  # room for the bf16 tiling too
    assert lib.sherry_gemm_plan(arr5, 4, F16, I8, F16, base, nb5) == OK
    assert int.from_bytes(ctypes.string_at(base + 40, 8), "little") == 4
    assert tiles_of(base, 4, n5) == ([(2, a, 0) for a in range(3)] + [(3, 0, 0)] + [(0, a, 0) for a in range(4)]
                                     + [(1, 0, 0)])
    # one problem outside the register classes (k = 640) keeps the few-token kernel
    arr5[3].k = 640
    assert lib.sherry_gemm_plan(arr5, 4, F16, I8, F16, base, lib.sherry_gemm_plan_bytes(arr5, 4)) == OK
    assert int.from_bytes(ctypes.string_at(base + 40, 8), "little") == 3
    # m <= 16 with a k above 8192: the 256 x 16 tiling
    skinny = [(2048, 2048, 16), (300, 9216, 3)]
    arr4 = problems(skinny)
    n4 = 8 + 2
    nb4 = lib.sherry_gemm_plan_bytes(arr4, 2)
    assert nb4 == 64 + 80 * 2 + 16 * n4
    assert lib.sherry_gemm_plan(arr4, 2, F16, I8, F16, base, nb4) == OK
    assert int.from_bytes(ctypes.string_at(base + 40, 8), "little") == 2
    assert tiles_of(base, 2, n4) == [(1, 0, 0), (1, 1, 0)] + [(0, a, 0) for a in range(8)]
    # a malformed or foreign host plan is rejected before any device call
    bad = ctypes.create_string_buffer(64)
    assert lib.sherry_gemm_grouped(ctypes.addressof(bad), A, None) == EINVAL
    assert lib.sherry_gemm_plan(arr, len(layer), F16, I8, F16, base, nbytes) == OK
    assert lib.sherry_gemv_grouped(base, A, None) == EINVAL  # a GEMM plan is not a GEMV plan


def test_probe_validation(lib):
    """Ceiling probes (include/sherry_probes.h): argument checks before any
    HIP call; EDEVICE without a GPU."""
    raw = ctypes.CDLL(LIB)
    rd, rt = raw.sherry_probe_read, raw.sherry_probe_rates
    rd.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    rt.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert rd(None, 1024, A, None) == EINVAL
    assert rd(A, 0, A, None) == EINVAL
    assert rd(A, 1000, A, None) == ESHAPE
    assert rd(A + 4, 1024, A, None) == EALIGN
    assert rd(A, 1024, A, None) == EDEVICE
    assert rt(7, 10, 10, A, None) == EINVAL
    assert rt(-1, 10, 10, A, None) == EINVAL
    assert rt(0, 0, 10, A, None) == EINVAL
    assert rt(0, 10, 0, A, None) == EINVAL
    assert rt(0, 10, 10, None, None) == EINVAL
    assert rt(0, 10, 10, A + 2, None) == EALIGN
    assert rt(0, 10, 10, A, None) == EDEVICE
    rc = raw.sherry_probe_clock
    rc.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert rc(0, 10, 10, A, None, None) == EINVAL
    assert rc(7, 10, 10, A, A, None) == EINVAL
    assert rc(0, 10, 10, A, A + 4, None) == EALIGN
    assert rc(0, 10, 10, A, A, None) == EDEVICE


# ------------------------------------------------- binding size checks ---
# The C ABI takes bare pointers, so the binding checks every tensor's size,
# type and device against the problem before it calls the library.  These
# checks read tensor metadata only, so CPU tensors exercise them here; a
# call that passes them still stops at the device check.

def _t(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def test_binding_rejects_mismatched_gemv_buffers(lib):
    import torch

    from ultra_bit_weight_amd import sherry

    n, k = 64, 1024
    words = n * (k // 128) * 5
    ok = dict(codes=_t(words, torch.int32), scales=_t(n, torch.float16), x=_t(k, torch.int8),
              x_scale=_t(1, torch.float32), acc_out=_t(n, torch.int32), out=_t(n, torch.float16))

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return sherry.gemv(a["codes"], a["scales"], a["x"], a["x_scale"], out=a["out"], acc_out=a["acc_out"])

    bad = [dict(codes=_t(words - 1, torch.int32)), dict(codes=_t(words // 2, torch.int8)),
           dict(scales=_t(n + 1, torch.float16)),  # codes now too short for n + 1 rows
           dict(x=_t((1, k), torch.int8)), dict(x=_t(k + 128, torch.int8)),
           dict(x_scale=_t(2, torch.float32)), dict(x_scale=_t(1, torch.float16)),
           dict(acc_out=_t(n - 1, torch.int32)), dict(acc_out=_t(n, torch.float32)),
           dict(out=_t(n + 1, torch.float16)), dict(out=_t(n, torch.int32)),
           dict(scales=_t(n, torch.int32))]
    for kw in bad:
        with pytest.raises(ValueError) as e:
            call(**kw)
        assert "GPU" not in str(e.value), (kw, str(e.value))  # caught by the size check, not the device check
    with pytest.raises(ValueError, match="GPU"):  # well-formed but on the CPU
        call()
    with pytest.raises(ValueError, match="GPU"):  # codes at the start of a larger buffer are accepted
        call(codes=_t(words + 5, torch.int32))
    with pytest.raises(ValueError):
        sherry.tern2_gemv(_t(words, torch.int32), ok["scales"], ok["x"], None, out=ok["out"])  # 2-bit: n k / 16 words
    with pytest.raises(ValueError):
        sherry.tern3_gemv(_t(words, torch.int32), ok["scales"], ok["x"], None, out=ok["out"])
    with pytest.raises(ValueError, match="elements|bytes"):
        sherry.gemv_quant(ok["codes"], ok["scales"], _t(k, torch.float32), out=_t(n - 1, torch.float16))
    with pytest.raises(ValueError, match="bytes"):
        sherry.decode(_t(words - 1, torch.int32), n, k)
    # the prepared call makes the same checks once, at construction
    with pytest.raises(ValueError, match="elements|bytes"):
        sherry.PreparedGemvQuant(ok["codes"], ok["scales"], _t(k, torch.bfloat16), out=_t(n + 1, torch.float16))
    with pytest.raises(ValueError, match="bytes"):
        sherry.PreparedGemvQuant(_t(words - 1, torch.int32), ok["scales"], _t(k, torch.bfloat16))
    with pytest.raises(ValueError, match="dtype"):
        sherry.PreparedGemvQuant(ok["codes"], ok["scales"], _t(k, torch.int8))
    with pytest.raises(ValueError, match="GPU"):
        sherry.PreparedGemvQuant(ok["codes"], ok["scales"], _t(k, torch.bfloat16), out=ok["out"])


def test_binding_rejects_mismatched_gemm_buffers(lib):
    import torch

    from ultra_bit_weight_amd import sherry

    n, k, m = 48, 640, 5
    words = n * (k // 128) * 5
    ok = dict(codes=_t(words, torch.int32), scales=_t(n, torch.float32), x=_t((m, k), torch.int8),
              x_scales=_t(m, torch.float32), acc_out=_t((m, n), torch.int32), out=_t((m, n), torch.float16))

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return sherry.gemm(a["codes"], a["scales"], a["x"], a["x_scales"], out=a["out"], acc_out=a["acc_out"])

    bad = [dict(codes=_t(words - 5, torch.int32)), dict(x=_t(m * k, torch.int8)),
           dict(x=_t((m, 2 * k), torch.int8)[:, ::2]), dict(x_scales=_t(m + 1, torch.float32)),
           dict(acc_out=_t((m, n - 1), torch.int32)), dict(out=_t((m + 1, n), torch.float16)),
           dict(out=_t((m, n + 1), torch.float16)), dict(out=_t((n, m), torch.float16).t())]
    for kw in bad:
        with pytest.raises(ValueError) as e:
            call(**kw)
        assert "GPU" not in str(e.value), (kw, str(e.value))
    with pytest.raises(ValueError, match="GPU"):
        call()
    # grouped launches validate each problem the same way
    p = dict(codes=ok["codes"], scales=ok["scales"], x=ok["x"], x_scales=ok["x_scales"], y=_t((m, n + 1), torch.float16))
    with pytest.raises(ValueError, match="y must be"):
        sherry.GroupedGemm([p])
    q = dict(codes=_t(words, torch.int32), scales=ok["scales"], x=_t(k, torch.int8), x_scale=None, acc=None,
             y=_t(n - 1, torch.float16))
    with pytest.raises(ValueError, match="elements"):
        sherry.GroupedGemv([q])
