"""Thin ctypes binding over libsherry.so (C ABI in include/sherry.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libsherry.so.  Tensors are torch tensors on the current HIP device;
the binding passes their data pointers and the current stream to the C ABI and
raises SherryError on any non-OK status.  If the library is missing the binding
raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SHERRY_LIB names another build of the library (for comparing build-time
# variants); by default the in-tree one
LIB_PATH = os.environ.get("SHERRY_LIB") or os.path.join(_HERE, "lib", "libsherry.so")

I8, I32, F16, BF16, F32 = 0, 1, 2, 3, 4
_DT = {torch.int8: I8, torch.int32: I32, torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}
STATUS = {0: "SHERRY_OK", 1: "SHERRY_EINVAL", 2: "SHERRY_ESHAPE", 3: "SHERRY_EDTYPE", 4: "SHERRY_EALIGN",
          5: "SHERRY_EDEVICE", 6: "SHERRY_ELAUNCH"}

EXPORTS = [
    "sherry_version", "sherry_status_str", "sherry_packed_bytes", "sherry_pack", "sherry_decode", "sherry_gemv",
    "sherry_act_quant", "sherry_gemv_quant",
    "sherry_gemv_plan_bytes", "sherry_gemv_plan", "sherry_gemv_plan_mfma", "sherry_gemv_grouped",
    "sherry_gemv_grouped_noalloc", "sherry_gemm",
    "sherry_gemm_plan_bytes", "sherry_gemm_plan", "sherry_gemm_grouped",
    "tern2_packed_bytes", "tern2_pack", "tern2_encode", "tern2_gemv", "tern2_gemv_plan", "tern2_gemm", "tern2_gemm_plan",
    "tern3_packed_bytes", "tern3_encode", "tern3_gemv", "tern3_gemv_plan_bytes", "tern3_gemv_plan",
    "sherry_probe_read", "sherry_probe_rates", "sherry_probe_clock", "sherry_set_prefill_kernel",
]


class SherryError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg}")
        self.status = status


class GemvProblem(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("w_scales", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("k", ctypes.c_int64), ("x", ctypes.c_void_p), ("x_scale", ctypes.c_void_p),
                ("acc", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class GemmProblem(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("w_scales", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("k", ctypes.c_int64), ("x", ctypes.c_void_p), ("m", ctypes.c_int64), ("ldx", ctypes.c_int64),
                ("x_scales", ctypes.c_void_p), ("acc", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("ldy", ctypes.c_int64)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsherry.so (after torch, so it binds to torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    vp, i64, i32, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    sz = ctypes.c_size_t
    lib.sherry_probe_read.restype = i
    lib.sherry_probe_read.argtypes = [vp, sz, vp, vp]
    lib.sherry_probe_rates.restype = i
    lib.sherry_probe_rates.argtypes = [i32, i32, i32, vp, vp]
    lib.sherry_probe_clock.restype = i
    lib.sherry_probe_clock.argtypes = [i32, i32, i32, vp, vp, vp]
    lib.sherry_version.restype = ctypes.c_char_p
    lib.sherry_status_str.restype = ctypes.c_char_p
    lib.sherry_status_str.argtypes = [i]
    lib.sherry_packed_bytes.restype = sz
    lib.sherry_packed_bytes.argtypes = [i64, i64]
    lib.tern2_packed_bytes.restype = sz
    lib.tern2_packed_bytes.argtypes = [i64, i64]
    lib.tern3_packed_bytes.restype = sz
    lib.tern3_packed_bytes.argtypes = [i64, i64]
    for f in (lib.sherry_pack, lib.tern2_pack):
        f.restype = i
        f.argtypes = [vp, i, i64, i64, i64, vp, vp, i, vp]
    lib.sherry_decode.restype = i
    lib.sherry_decode.argtypes = [vp, i64, i64, vp, i64, vp]
    lib.sherry_gemv_quant.restype = i
    lib.sherry_gemv_quant.argtypes = [vp, vp, i, i64, i64, vp, i, vp, vp, vp, i, vp]
    lib.sherry_act_quant.restype = i
    lib.sherry_act_quant.argtypes = [vp, i, i64, i64, i64, vp, i64, vp, vp]
    gemv_args = [vp, vp, i, i64, i64, vp, i, vp, vp, vp, i, vp]
    for f in (lib.sherry_gemv, lib.tern2_gemv, lib.tern3_gemv):
        f.restype = i
        f.argtypes = gemv_args
    lib.sherry_gemv_plan_bytes.restype = sz
    lib.sherry_gemv_plan_bytes.argtypes = [ctypes.POINTER(GemvProblem), i32]
    lib.tern3_gemv_plan_bytes.restype = sz
    lib.tern3_gemv_plan_bytes.argtypes = [ctypes.POINTER(GemvProblem), i32]
    for f in (lib.sherry_gemv_plan, lib.sherry_gemv_plan_mfma, lib.tern2_gemv_plan, lib.tern3_gemv_plan):
        f.restype = i
        f.argtypes = [ctypes.POINTER(GemvProblem), i32, i, i, i, vp, sz]
    lib.sherry_gemv_grouped.restype = i
    lib.sherry_gemv_grouped.argtypes = [vp, vp, vp]
    lib.sherry_gemv_grouped_noalloc.restype = i
    lib.sherry_gemv_grouped_noalloc.argtypes = [vp, vp]
    gemm_args = [vp, vp, i, i64, i64, vp, i, i64, i64, vp, vp, vp, i, i64, vp]
    for f in (lib.sherry_gemm, lib.tern2_gemm):
        f.restype = i
        f.argtypes = gemm_args
    lib.tern2_encode.restype = i
    lib.tern2_encode.argtypes = [vp, i64, i64, i64, vp, vp]
    lib.tern3_encode.restype = i
    lib.tern3_encode.argtypes = [vp, i64, i64, i64, vp, vp]
    lib.sherry_gemm_plan_bytes.restype = sz
    lib.sherry_gemm_plan_bytes.argtypes = [ctypes.POINTER(GemmProblem), i32]
    for f in (lib.sherry_gemm_plan, lib.tern2_gemm_plan):
        f.restype = i
        f.argtypes = [ctypes.POINTER(GemmProblem), i32, i, i, i, vp, sz]
    lib.sherry_gemm_grouped.restype = i
    lib.sherry_gemm_grouped.argtypes = [vp, vp, vp]
    lib.sherry_set_prefill_kernel.restype = i
    lib.sherry_set_prefill_kernel.argtypes = [i]
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise SherryError(fn, status, load().sherry_status_str(status).decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev(*ts):
    """Every given tensor contiguous, on the GPU, and all on one device."""
    devs = set()
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous and on the GPU")
        devs.add(t.device)
    if len(devs) > 1:
        raise ValueError(f"tensors are on different devices: {sorted(str(d) for d in devs)}")


def _need(t, name, numel=None, nbytes=None, dtypes=None, dim=None, min_nbytes=None):
    """Size and type checks the C ABI cannot make (it takes bare pointers):
    a wrong size here would let a kernel read or write past a buffer.  Runs on
    tensor metadata only, before any device check."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must be {dim}-D, got shape {tuple(t.shape)}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    if nbytes is not None and t.numel() * t.element_size() != nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, expected {nbytes}")
    if min_nbytes is not None and t.numel() * t.element_size() < min_nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs at least {min_nbytes}")


_SCALE_DT = (torch.float32, torch.float16)
_Y_DT = (torch.float32, torch.float16)


def _codes_bytes(fmt: str, n: int, k: int) -> int:
    nb = {"sherry": packed_bytes, "tern2": tern2_packed_bytes, "tern3": tern3_packed_bytes}[fmt](n, k)
    if nb == 0:
        raise ValueError(f"invalid shape n={n} k={k} (k must be a positive multiple of 128)")
    return nb


def _check_gemv_args(fmt, codes, scales, x, x_scale, acc, y):
    """Batch-1 product: n from the scales, k from x (1-D)."""
    _need(scales, "scales", dim=1, dtypes=_SCALE_DT)
    _need(x, "x", dim=1)
    n, k = scales.numel(), x.numel()
    _need(codes, "codes", min_nbytes=_codes_bytes(fmt, n, k))
    _need(x_scale, "x_scale", numel=1, dtypes=(torch.float32,))
    _need(acc, "acc", numel=n, dtypes=(torch.int32,))
    _need(y, "y", numel=n, dtypes=_Y_DT)
    _dev(codes, scales, x, x_scale, acc, y)
    return n, k


def _check_gemm_args(fmt, codes, scales, x, x_scales, acc, y):
    """M-token product: x [m, k] with unit column stride, y [m, n] likewise,
    acc [m, n] contiguous."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [m, k] with unit column stride")
    _need(x, "x", dtypes=(torch.int8, torch.bfloat16))
    _need(scales, "scales", dim=1, dtypes=_SCALE_DT)
    m, k = x.shape
    n = scales.numel()
    _need(codes, "codes", min_nbytes=_codes_bytes(fmt, n, k))
    _need(x_scales, "x_scales", numel=m, dtypes=(torch.float32,))
    _need(acc, "acc", numel=m * n, dtypes=(torch.int32,))
    if y is not None:
        if y.dim() != 2 or tuple(y.shape) != (m, n) or y.stride(1) != 1:
            raise ValueError(f"y must be [{m}, {n}] with unit column stride, got shape {tuple(y.shape)}")
        _need(y, "y", dtypes=_Y_DT)
    _dev(codes, scales, x_scales, acc)  # x and y may have a row stride
    for name, t in (("x", x), ("y", y)):
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
    if len({t.device for t in (codes, scales, x, x_scales, acc, y) if t is not None}) > 1:
        raise ValueError("tensors are on different devices")
    return m, n, k


PREFILL_TILED, PREFILL_DECODE_ONCE, PREFILL_TILED32 = 0, 1, 2


def set_prefill_kernel(kind: int) -> None:
    """Process-wide choice of the many-token kernel
    (sherry_set_prefill_kernel): PREFILL_TILED (default), PREFILL_DECODE_ONCE
    or PREFILL_TILED32."""
    _check("sherry_set_prefill_kernel", load().sherry_set_prefill_kernel(kind))


def packed_bytes(n: int, k: int) -> int:
    return load().sherry_packed_bytes(n, k)


def tern2_packed_bytes(n: int, k: int) -> int:
    return load().tern2_packed_bytes(n, k)


def version() -> str:
    return load().sherry_version().decode()


def empty_codes(n: int, k: int, device=None) -> torch.Tensor:
    """Uninitialised code buffer for an n x k matrix (int32 view of the words)."""
    words = packed_bytes(n, k) // 4
    if words == 0:
        raise ValueError(f"invalid shape n={n} k={k}")
    return torch.empty(words, dtype=torch.int32, device=device or "cuda")


def pack(w: torch.Tensor, scale_dtype=torch.float16):
    """Real weights [n, k] (fp32/fp16/bf16, row stride = w.stride(0)) ->
    (codes int32 [n*k*5/128], scales [n])."""
    if w.dim() != 2 or w.stride(1) != 1 or not w.is_cuda:
        raise ValueError("w must be a 2-D GPU tensor with unit column stride")
    n, k = w.shape
    codes = empty_codes(n, k, w.device)
    scales = torch.empty(n, dtype=scale_dtype, device=w.device)
    _check("sherry_pack", load().sherry_pack(w.data_ptr(), _DT[w.dtype], n, k, w.stride(0), codes.data_ptr(),
                                             scales.data_ptr(), _DT[scale_dtype], _stream()))
    return codes, scales


def tern2_pack(w: torch.Tensor, scale_dtype=torch.float16):
    """Real weights [n, k] -> (2-bit words int32 [n*k/16], scales [n]) with
    the decisions and scales of pack(): the same ternary matrix."""
    if w.dim() != 2 or w.stride(1) != 1 or not w.is_cuda:
        raise ValueError("w must be a 2-D GPU tensor with unit column stride")
    n, k = w.shape
    codes = torch.empty(max(tern2_packed_bytes(n, k) // 4, 1), dtype=torch.int32, device=w.device)
    scales = torch.empty(n, dtype=scale_dtype, device=w.device)
    _check("tern2_pack", load().tern2_pack(w.data_ptr(), _DT[w.dtype], n, k, w.stride(0), codes.data_ptr(),
                                           scales.data_ptr(), _DT[scale_dtype], _stream()))
    return codes, scales


PROBE_MFMA, PROBE_DOT4, PROBE_SAME_WAVE, PROBE_ALT_WAVES, PROBE_MFMA32, PROBE_ALU, PROBE_SAME_ALU = 0, 1, 2, 3, 4, 5, 6
# int8 ops per wave and iteration of the rate probe: 4 matrix-core products
# of 16 x 16 x 64, 16 v_dot4 over 64 lanes
PROBE_MFMA_OPS, PROBE_DOT4_OPS = 4 * 2 * 16 * 16 * 64, 16 * 2 * 4 * 64


def probe_read(buf: torch.Tensor, sink: torch.Tensor):
    """Read all of buf (GPU, bytes a multiple of 16) once (sherry_probe_read)."""
    _dev(buf, sink)
    _check("sherry_probe_read", load().sherry_probe_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                                         sink.data_ptr(), _stream()))


def probe_rates(mode: int, iters: int, blocks: int, sink: torch.Tensor):
    """Rate probe (sherry_probe_rates): `blocks` workgroups of 4 waves."""
    _dev(sink)
    _check("sherry_probe_rates", load().sherry_probe_rates(mode, iters, blocks, sink.data_ptr(), _stream()))


def probe_clock(mode: int, iters: int, blocks: int, sink: torch.Tensor, ticks: torch.Tensor):
    """Rate probe with the clock record (sherry_probe_clock); ticks: int64
    [blocks, 4] on the GPU."""
    _need(ticks, "ticks", numel=4 * blocks, dtypes=(torch.int64,))
    _dev(sink, ticks)
    _check("sherry_probe_clock", load().sherry_probe_clock(mode, iters, blocks, sink.data_ptr(), ticks.data_ptr(),
                                                           _stream()))


def decode(codes: torch.Tensor, n: int, k: int) -> torch.Tensor:
    """Packed codes -> dense int8 ternary matrix [n, k]."""
    _need(codes, "codes", min_nbytes=_codes_bytes("sherry", n, k))
    _dev(codes)
    t = torch.empty(n, k, dtype=torch.int8, device=codes.device)
    _check("sherry_decode", load().sherry_decode(codes.data_ptr(), n, k, t.data_ptr(), t.stride(0), _stream()))
    return t


def act_quant(x: torch.Tensor):
    """Per-token int8 quantization of activations x [m, k] (fp32, fp16 or
    bf16; a 1-D x is one token) -> (x_q int8 [m, k], scales fp32 [m])."""
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    if not x.is_cuda or x2.dim() != 2 or x2.stride(1) != 1:
        raise ValueError("x must be a GPU tensor [m, k] with unit stride along k")
    m, k = x2.shape
    q = torch.empty(m, k, dtype=torch.int8, device=x.device)
    s = torch.empty(m, dtype=torch.float32, device=x.device)
    _check("sherry_act_quant", load().sherry_act_quant(x2.data_ptr(), _DT.get(x2.dtype, -1), m, k, x2.stride(0),
                                                       q.data_ptr(), q.stride(0), s.data_ptr(), _stream()))
    if x.dim() == 1:
        return q[0], s
    return q, s


def gemv_quant(codes, scales, x, out_dtype=torch.float16, want_acc=False, want_scale=False, out=None):
    """y = diag(scales) T q(x) for fp x [k] (fp32, fp16 or bf16), x quantized
    per token inside the kernel.  Returns (acc or None, y or None, scale or
    None)."""
    _need(x, "x", dim=1, dtypes=(torch.float32, torch.float16, torch.bfloat16))
    n, k = _check_gemv_args("sherry", codes, scales, x, None, None, out)
    y = out if out is not None else (torch.empty(n, dtype=out_dtype, device=x.device) if out_dtype else None)
    acc = torch.empty(n, dtype=torch.int32, device=x.device) if want_acc else None
    sx = torch.empty(1, dtype=torch.float32, device=x.device) if want_scale else None
    _check("sherry_gemv_quant", load().sherry_gemv_quant(
        codes.data_ptr(), scales.data_ptr(), _DT[scales.dtype], n, k, x.data_ptr(), _DT.get(x.dtype, -1), _ptr(sx),
        _ptr(acc), _ptr(y), _DT[y.dtype] if y is not None else F32, _stream()))
    return acc, y, sx


class PreparedGemvQuant:
    """gemv_quant with its arguments checked and marshalled once, for loops
    that run the same product over and over (a decode step): each call is
    then one foreign call.  The tensors are held, and read at their current
    contents on every call; reallocating them (a new tensor under the same
    name) is not seen.  call(stream) launches on `stream` (a HIP stream
    handle) or, when None, on torch's current stream (which a graph capture
    replaces with its own)."""

    def __init__(self, codes, scales, x, out_dtype=torch.float16, want_acc=False, want_scale=False, out=None):
        _need(x, "x", dim=1, dtypes=(torch.float32, torch.float16, torch.bfloat16))
        n, k = _check_gemv_args("sherry", codes, scales, x, None, None, out)
        self.y = out if out is not None else (torch.empty(n, dtype=out_dtype, device=x.device) if out_dtype else None)
        self.acc = torch.empty(n, dtype=torch.int32, device=x.device) if want_acc else None
        self.scale = torch.empty(1, dtype=torch.float32, device=x.device) if want_scale else None
        if self.y is None and self.acc is None:
            raise ValueError("nothing to compute: neither y nor acc")
        self._keep = (codes, scales, x)
        self._f = load().sherry_gemv_quant
        self._args = (codes.data_ptr(), scales.data_ptr(), _DT[scales.dtype], n, k, x.data_ptr(), _DT[x.dtype],
                      _ptr(self.scale), _ptr(self.acc), _ptr(self.y),
                      _DT[self.y.dtype] if self.y is not None else F32)

    def __call__(self, stream=None):
        status = self._f(*self._args, _stream() if stream is None else stream)
        if status:
            _check("sherry_gemv_quant", status)
        return self.y


_FMT = {"sherry_gemv": "sherry", "tern2_gemv": "tern2", "tern3_gemv": "tern3", "sherry_gemm": "sherry",
        "tern2_gemm": "tern2"}


def _gemv(fn_name, codes, scales, x, x_scale, acc, y):
    n, k = _check_gemv_args(_FMT[fn_name], codes, scales, x, x_scale, acc, y)
    f = getattr(load(), fn_name)
    _check(fn_name, f(codes.data_ptr(), scales.data_ptr(), _DT[scales.dtype], n, k, x.data_ptr(), _DT[x.dtype],
                      _ptr(x_scale), _ptr(acc), _ptr(y), _DT[y.dtype] if y is not None else F32, _stream()))


def gemv(codes, scales, x, x_scale=None, out_dtype=torch.float16, want_acc=False, out=None, acc_out=None):
    """y = diag(scales) T x for int8 or bf16 x.  Returns (acc or None, y or None)."""
    n = scales.numel()
    y = out if out is not None else (torch.empty(n, dtype=out_dtype, device=x.device) if out_dtype else None)
    acc = acc_out if acc_out is not None else (torch.empty(n, dtype=torch.int32, device=x.device) if want_acc else None)
    _gemv("sherry_gemv", codes, scales, x, x_scale, acc, y)
    return acc, y


def tern2_gemv(codes, scales, x, x_scale=None, out_dtype=torch.float16, want_acc=False, out=None, acc_out=None):
    n = scales.numel()
    y = out if out is not None else (torch.empty(n, dtype=out_dtype, device=x.device) if out_dtype else None)
    acc = acc_out if acc_out is not None else (torch.empty(n, dtype=torch.int32, device=x.device) if want_acc else None)
    _gemv("tern2_gemv", codes, scales, x, x_scale, acc, y)
    return acc, y


def _gemm(fn_name, codes, scales, x, x_scales, out_dtype, want_acc, out=None, acc_out=None):
    m, n, k = _check_gemm_args(_FMT[fn_name], codes, scales, x, x_scales, acc_out, out)
    y = out if out is not None else (torch.empty(m, n, dtype=out_dtype, device=x.device) if out_dtype else None)
    acc = acc_out if acc_out is not None else (torch.empty(m, n, dtype=torch.int32, device=x.device) if want_acc
                                               else None)
    f = getattr(load(), fn_name)
    _check(fn_name, f(codes.data_ptr(), scales.data_ptr(), _DT[scales.dtype], n, k, x.data_ptr(), _DT[x.dtype], m,
                      x.stride(0), _ptr(x_scales), _ptr(acc), _ptr(y), _DT[y.dtype] if y is not None else F32,
                      y.stride(0) if y is not None else n, _stream()))
    return acc, y


def gemm(codes, scales, x, x_scales=None, out_dtype=torch.float16, want_acc=False, out=None, acc_out=None):
    """Y[m, r] = s_x[m] s_w[r] sum_k X[m, k] T[r, k] for int8 X [m, k]; for
    bf16 X (m <= 16, k <= 8192) Y[m, r] = s_w[r] sum_k X[m, k] T[r, k] in fp32
    (no token scales, no int32 sums, fp32 outputs)."""
    if x.dtype == torch.bfloat16 and out is None:
        out_dtype = torch.float32
    return _gemm("sherry_gemm", codes, scales, x, x_scales, out_dtype, want_acc, out, acc_out)


def tern2_gemm(codes, scales, x, x_scales=None, out_dtype=torch.float16, want_acc=False, out=None, acc_out=None):
    return _gemm("tern2_gemm", codes, scales, x, x_scales, out_dtype, want_acc, out, acc_out)


def tern3_packed_bytes(n: int, k: int) -> int:
    return load().tern3_packed_bytes(n, k)


def tern3_encode(t: torch.Tensor) -> torch.Tensor:
    """Dense int8 ternary [n, k] -> 1.67-bit words (int32 view)."""
    if t.dim() != 2 or t.stride(1) != 1 or not t.is_cuda or t.dtype != torch.int8:
        raise ValueError("t must be a 2-D int8 GPU tensor with unit column stride")
    n, k = t.shape
    words = tern3_packed_bytes(n, k) // 4
    if words == 0:
        raise ValueError(f"invalid shape n={n} k={k}")
    codes = torch.empty(words, dtype=torch.int32, device=t.device)
    _check("tern3_encode", load().tern3_encode(t.data_ptr(), n, k, t.stride(0), codes.data_ptr(), _stream()))
    return codes


def tern3_gemv(codes, scales, x, x_scale=None, out_dtype=torch.float16, want_acc=False, out=None, acc_out=None):
    n = scales.numel()
    y = out if out is not None else (torch.empty(n, dtype=out_dtype, device=x.device) if out_dtype else None)
    acc = acc_out if acc_out is not None else (torch.empty(n, dtype=torch.int32, device=x.device) if want_acc else None)
    _gemv("tern3_gemv", codes, scales, x, x_scale, acc, y)
    return acc, y


def tern2_encode(t: torch.Tensor) -> torch.Tensor:
    """Dense int8 ternary [n, k] -> 2-bit words (int32 view) [n * k / 16]."""
    if t.dim() != 2 or t.stride(1) != 1 or not t.is_cuda or t.dtype != torch.int8:
        raise ValueError("t must be a 2-D int8 GPU tensor with unit column stride")
    n, k = t.shape
    words = tern2_packed_bytes(n, k) // 4
    if words == 0:
        raise ValueError(f"invalid shape n={n} k={k}")
    codes = torch.empty(words, dtype=torch.int32, device=t.device)
    _check("tern2_encode", load().tern2_encode(t.data_ptr(), n, k, t.stride(0), codes.data_ptr(), _stream()))
    return codes


class GroupedGemv:
    """Many batch-1 products in one launch.  `problems` is a list of dicts with
    keys codes, scales, x, x_scale (or None), acc (or None), y (or None); all
    share the scale / x / y dtypes.  The plan is built once on the host and
    copied to the device; call() launches it on the current stream.  With
    mfma=True (bf16 x, k <= 8192) the plan runs on the matrix cores
    (sherry_gemv_plan_mfma)."""

    def __init__(self, problems, tern2: bool = False, tern3: bool = False, mfma: bool = False):
        lib = load()
        arr = (GemvProblem * len(problems))()
        self._keep = []
        fmt = "tern3" if tern3 else ("tern2" if tern2 else "sherry")
        for i, p in enumerate(problems):
            _check_gemv_args(fmt, p["codes"], p["scales"], p["x"], p.get("x_scale"), p.get("acc"), p.get("y"))
            arr[i] = GemvProblem(p["codes"].data_ptr(), p["scales"].data_ptr(), p["scales"].numel(), p["x"].numel(),
                                 p["x"].data_ptr(), _ptr(p.get("x_scale")), _ptr(p.get("acc")), _ptr(p.get("y")))
            self._keep.append(p)
        p0 = problems[0]
        s_dt = _DT[p0["scales"].dtype]
        x_dt = _DT[p0["x"].dtype]
        y_dt = _DT[p0["y"].dtype] if p0.get("y") is not None else F32
        nbytes = (lib.tern3_gemv_plan_bytes if tern3 else lib.sherry_gemv_plan_bytes)(arr, len(problems))
        if nbytes == 0:
            raise ValueError("invalid grouped GEMV problems")
        self.host = torch.empty(nbytes, dtype=torch.uint8)
        if mfma:
            fn = lib.sherry_gemv_plan_mfma
        else:
            fn = lib.tern3_gemv_plan if tern3 else (lib.tern2_gemv_plan if tern2 else lib.sherry_gemv_plan)
        _check("gemv_plan", fn(arr, len(problems), s_dt, x_dt, y_dt, self.host.data_ptr(), nbytes))
        self.dev = self.host.to(p0["x"].device, non_blocking=False)
        self.n_tiles = int.from_bytes(bytes(self.host[12:16].tolist()), "little", signed=True)
        self.count = len(problems)

    def __call__(self):
        _check("sherry_gemv_grouped", load().sherry_gemv_grouped(self.host.data_ptr(), self.dev.data_ptr(), _stream()))

    def call_noalloc(self):
        """Launch the same plan through sherry_gemv_grouped_noalloc: the host
        plan is copied into the library's static plan memory on the current
        stream (no device copy of the plan is used)."""
        _check("sherry_gemv_grouped_noalloc", load().sherry_gemv_grouped_noalloc(self.host.data_ptr(), _stream()))


class GroupedGemm:
    """Many products for M tokens in one launch.  `problems` is a list of dicts
    with keys codes, scales, x ([m, k] int8 or bf16, unit column stride; one
    type for all), x_scales (or
    None), acc (or None, [m, n] int32 contiguous), y (or None, [m, n] with unit
    column stride); all share the scale / y dtypes.  The plan is built once on
    the host and copied to the device; call() launches it on the current
    stream."""

    def __init__(self, problems, tern2: bool = False):
        lib = load()
        arr = (GemmProblem * len(problems))()
        self._keep = []
        for i, p in enumerate(problems):
            x, y, acc = p["x"], p.get("y"), p.get("acc")
            m, n, k = _check_gemm_args("tern2" if tern2 else "sherry", p["codes"], p["scales"], x, p.get("x_scales"),
                                       acc, y)
            arr[i] = GemmProblem(p["codes"].data_ptr(), p["scales"].data_ptr(), n, k, x.data_ptr(), m, x.stride(0),
                                 _ptr(p.get("x_scales")), _ptr(acc), _ptr(y), y.stride(0) if y is not None else n)
            self._keep.append(p)
        p0 = problems[0]
        s_dt = _DT[p0["scales"].dtype]
        x_dt = _DT[p0["x"].dtype]
        y_dt = _DT[p0["y"].dtype] if p0.get("y") is not None else F32
        nbytes = lib.sherry_gemm_plan_bytes(arr, len(problems))
        if nbytes == 0:
            raise ValueError("invalid grouped GEMM problems")
        self.host = torch.empty(nbytes, dtype=torch.uint8)
        fn = lib.tern2_gemm_plan if tern2 else lib.sherry_gemm_plan
        _check("gemm_plan", fn(arr, len(problems), s_dt, x_dt, y_dt, self.host.data_ptr(), nbytes))
        self.dev = self.host.to(p0["x"].device, non_blocking=False)
        self.n_tiles = int.from_bytes(bytes(self.host[12:16].tolist()), "little", signed=True)
        self.count = len(problems)

    def __call__(self):
        _check("sherry_gemm_grouped", load().sherry_gemm_grouped(self.host.data_ptr(), self.dev.data_ptr(), _stream()))
