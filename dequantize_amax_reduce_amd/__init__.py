"""FP8 scaled cast for AMD Instinct MI355X: Python binding of libfp8q.so.

Every step of quantize and dequantize runs in the HIP kernels of
``csrc/fp8q_kernels.hip`` behind the C ABI of ``include/fp8q.h``; this module
only marshals torch tensors (device memory) and the current HIP stream into
those calls.  There is no CPU or PyTorch fallback: importing the package fails
if the library is not built (``python dequantize_amax_reduce_amd/build.py``).

Two layers:

* ``fp8q_*`` -- one function per C entry point, same name, caller-allocated
  outputs, returns None or raises (TypeError for FP8Q_EDTYPE, ValueError for
  FP8Q_ESHAPE / FP8Q_EINVAL / FP8Q_EALIGN, RuntimeError for FP8Q_EHIP).
* page-level helpers that allocate outputs with torch, mirroring the
  functions the method is defined by: ``cast_to_fp8`` / ``cast_from_fp8``
  (ColossalAI fp8.py), ``per_token_cast_to_fp8`` / ``per_token_cast_back``
  (DeepEP "5 Utils") and ``weight_dequant`` (CSDN fp8_cast_bf16 notes).
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8q.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "fp8q.h")

E4M3FN, E5M2 = 0, 1
F32, BF16, F16 = 0, 1, 2
OK, EINVAL, EDTYPE, ESHAPE, EALIGN, EHIP = range(6)

_FMT = {"e4m3": E4M3FN, "e4m3fn": E4M3FN, "e5m2": E5M2, E4M3FN: E4M3FN, E5M2: E5M2,
        torch.float8_e4m3fn: E4M3FN, torch.float8_e5m2: E5M2}
_FP8_DTYPE = {E4M3FN: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


def _load(path: str = LIB_PATH):
    """ctypes handle of a build of the C ABI with every signature set."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python dequantize_amax_reduce_amd/build.py` "
                          "(the HIP library is required; there is no fallback)")
    L = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sigs = {
        "fp8q_abi_version": (I, []),
        "fp8q_status_str": (ctypes.c_char_p, [I]),
        "fp8q_per_tensor_workspace_bytes": (ctypes.c_size_t, []),
        "fp8q_amax": (I, [P, I, I64, P, P]),
        "fp8q_cast_per_tensor": (I, [P, I, I64, I, P, P, P, P]),
        "fp8q_cast_per_tensor_noalloc": (I, [P, I, I64, I, P, P, P]),
        "fp8q_cast_per_channel": (I, [P, I, I64, I64, I, P, P, P]),
        "fp8q_cast_per_group128": (I, [P, I, I64, I64, I, P, P, P]),
        "fp8q_cast_per_group128_wave64": (I, [P, I, I64, I64, I, P, P, P]),
        "fp8q_dequant_per_tensor": (I, [P, I, I64, P, P, I, P]),
        "fp8q_dequant_per_channel": (I, [P, I, I64, I64, P, P, I, P]),
        "fp8q_dequant_per_group128": (I, [P, I, I64, I64, P, P, I, P]),
        "fp8q_weight_dequant_block128": (I, [P, I, I64, I64, P, P, I, P]),
        "fp8q_amax_guarded": (I, [P, I, I64, P, P]),
        "fp8q_cast_with_amax": (I, [P, I, I64, I, P, P, P, P]),
        "fp8q_dequant_div_scale": (I, [P, I, I64, P, P, I, P]),
        "fp8q_cast_to_fp8_pipeline": (I, [P, I, I64, P, P, P, P, P]),
        "fp8q_cast_from_fp8_pipeline": (I, [P, P, I64, P, P, I, P]),
        "fp8q_cast_to_packed": (I, [P, I, I64, I, P, P, P]),
        "fp8q_dequant_packed": (I, [P, I, I64, I64, P, I, P]),
        "fp8q_dequant_sum": (I, [P, I, I64, I64, P, I, P, I, P]),
        "fp8q_dequant_sum_requant": (I, [P, I, I64, I64, P, I, P, I, P, P, P, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()
ABI_FUNCTIONS = ("fp8q_abi_version", "fp8q_status_str", "fp8q_per_tensor_workspace_bytes", "fp8q_amax",
                 "fp8q_cast_per_tensor", "fp8q_cast_per_channel", "fp8q_cast_per_group128",
                 "fp8q_cast_per_group128_wave64",
                 "fp8q_dequant_per_tensor", "fp8q_dequant_per_channel", "fp8q_dequant_per_group128",
                 "fp8q_weight_dequant_block128", "fp8q_dequant_sum", "fp8q_dequant_sum_requant",
                 "fp8q_amax_guarded", "fp8q_cast_with_amax", "fp8q_dequant_div_scale",
                 "fp8q_cast_to_fp8_pipeline", "fp8q_cast_from_fp8_pipeline", "fp8q_cast_to_packed",
                 "fp8q_dequant_packed", "fp8q_cast_per_tensor_noalloc")


def header_functions() -> list:
    """Names of the functions include/fp8q.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:fp8q_status_t|int|size_t|const char\*)\s+(fp8q_\w+)\s*\(",
                                 text, re.M)))


class Fp8qError(RuntimeError):
    pass


def _check(status: int, what: str):
    if status == OK:
        return
    msg = f"{what}: {lib.fp8q_status_str(status).decode()}"
    if status == EDTYPE:
        raise TypeError(msg)
    if status in (EINVAL, ESHAPE, EALIGN):
        raise ValueError(msg)
    raise Fp8qError(msg)


# ---------------------------------------------------------------------------
# marshalling
# ---------------------------------------------------------------------------

def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.numel() > 0:
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU (got {t.device})")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() if t.numel() > 0 else 0


def _stream(t: torch.Tensor, stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if t.device.type == "cuda":
        return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _hp_dtype(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"{name}: only float32, bfloat16 and float16 are supported (got {t.dtype})")
    return _DT[t.dtype]


def _fmt(fmt) -> int:
    if fmt not in _FMT:
        raise TypeError(f"unknown fp8 format {fmt!r} (use 'e4m3fn'/'e4m3' or 'e5m2')")
    return _FMT[fmt]


def _fp8(t: torch.Tensor, fmt, name: str) -> int:
    """fp8 tensors may be float8_e4m3fn / float8_e5m2 or uint8 codes."""
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        if fmt is not None and _fmt(fmt) != _FMT[t.dtype]:
            raise TypeError(f"{name} is {t.dtype} but fmt={fmt!r}")
        return _FMT[t.dtype]
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must be float8_e4m3fn, float8_e5m2 or uint8 codes (got {t.dtype})")
    return _fmt("e4m3fn" if fmt is None else fmt)


def _rows_cols(t: torch.Tensor):
    if t.dim() == 0:
        return 1, 1
    cols = t.shape[-1]
    rows = t.numel() // cols if cols else (t.numel() if t.dim() == 1 else int(torch.tensor(t.shape[:-1]).prod()))
    return rows, cols


# ---------------------------------------------------------------------------
# one function per C entry point
# ---------------------------------------------------------------------------

def fp8q_abi_version() -> int:
    return lib.fp8q_abi_version()


def fp8q_status_str(status: int) -> str:
    return lib.fp8q_status_str(status).decode()


def fp8q_per_tensor_workspace_bytes() -> int:
    return lib.fp8q_per_tensor_workspace_bytes()


def fp8q_amax(x: torch.Tensor, amax: torch.Tensor, stream=None) -> None:
    if amax.dtype != torch.float32 or amax.numel() < 1:
        raise TypeError("amax must be a float32 tensor with at least one element")
    _check(lib.fp8q_amax(_dev(x, "x"), _hp_dtype(x, "x"), x.numel(), _dev(amax, "amax"), _stream(x, stream)),
           "fp8q_amax")


def fp8q_cast_per_tensor(x, q, scale_inv, workspace, fmt="e4m3fn", stream=None) -> None:
    f = _fp8(q, fmt, "q")
    if q.numel() != x.numel() or scale_inv.dtype != torch.float32 or scale_inv.numel() < 1:
        raise ValueError("fp8q_cast_per_tensor: q must match x and scale_inv must be float32[1]")
    if workspace.numel() * workspace.element_size() < fp8q_per_tensor_workspace_bytes():
        raise ValueError("fp8q_cast_per_tensor: workspace too small")
    _check(lib.fp8q_cast_per_tensor(_dev(x, "x"), _hp_dtype(x, "x"), x.numel(), f, _dev(q, "q"),
                                    _dev(scale_inv, "scale_inv"), _dev(workspace, "workspace"),
                                    _stream(x, stream)), "fp8q_cast_per_tensor")


def fp8q_cast_per_tensor_noalloc(x, q, scale_inv, fmt="e4m3fn", stream=None) -> None:
    """fp8q_cast_per_tensor with the library's own device scratch instead of
    a caller workspace; it allocates nothing.  Calls that overlap in time on
    one GPU share that scratch and race."""
    f = _fp8(q, fmt, "q")
    if q.numel() != x.numel() or scale_inv.dtype != torch.float32 or scale_inv.numel() < 1:
        raise ValueError("fp8q_cast_per_tensor_noalloc: q must match x and scale_inv must be float32[1]")
    _check(lib.fp8q_cast_per_tensor_noalloc(_dev(x, "x"), _hp_dtype(x, "x"), x.numel(), f, _dev(q, "q"),
                                            _dev(scale_inv, "scale_inv"), _stream(x, stream)),
           "fp8q_cast_per_tensor_noalloc")


def fp8q_cast_per_channel(x, q, scale_inv, fmt="e4m3fn", stream=None) -> None:
    f = _fp8(q, fmt, "q")
    rows, cols = _rows_cols(x)
    if q.numel() != x.numel() or scale_inv.dtype != torch.float32 or scale_inv.numel() != rows:
        raise ValueError("fp8q_cast_per_channel: q must match x and scale_inv must be float32[rows]")
    _check(lib.fp8q_cast_per_channel(_dev(x, "x"), _hp_dtype(x, "x"), rows, cols, f, _dev(q, "q"),
                                     _dev(scale_inv, "scale_inv"), _stream(x, stream)), "fp8q_cast_per_channel")


def _group128_cast(name, x, q, scale_inv, fmt, stream) -> None:
    f = _fp8(q, fmt, "q")
    rows, cols = _rows_cols(x)
    if q.numel() != x.numel() or scale_inv.dtype != torch.float32 or \
            (cols % 128 == 0 and scale_inv.numel() != rows * (cols // 128)):
        raise ValueError(f"{name}: q must match x and scale_inv must be float32[rows, cols/128]")
    _check(getattr(lib, name)(_dev(x, "x"), _hp_dtype(x, "x"), rows, cols, f, _dev(q, "q"),
                              _dev(scale_inv, "scale_inv"), _stream(x, stream)), name)


def fp8q_cast_per_group128(x, q, scale_inv, fmt="e4m3fn", stream=None) -> None:
    _group128_cast("fp8q_cast_per_group128", x, q, scale_inv, fmt, stream)


def fp8q_cast_per_group128_wave64(x, q, scale_inv, fmt="e4m3fn", stream=None) -> None:
    """The same cast in the one-wavefront-per-group kernel shape (for
    measurement; x aligned to two elements, q to 2 bytes)."""
    _group128_cast("fp8q_cast_per_group128_wave64", x, q, scale_inv, fmt, stream)


def fp8q_dequant_per_tensor(q, scale_inv, y, fmt=None, stream=None) -> None:
    f = _fp8(q, fmt, "q")
    if y.numel() != q.numel() or scale_inv.dtype != torch.float32:
        raise ValueError("fp8q_dequant_per_tensor: y must match q and scale_inv must be float32[1]")
    _check(lib.fp8q_dequant_per_tensor(_dev(q, "q"), f, q.numel(), _dev(scale_inv, "scale_inv"), _dev(y, "y"),
                                       _hp_dtype(y, "y"), _stream(q, stream)), "fp8q_dequant_per_tensor")


def fp8q_dequant_per_channel(q, scale_inv, y, fmt=None, stream=None) -> None:
    f = _fp8(q, fmt, "q")
    rows, cols = _rows_cols(q)
    if y.numel() != q.numel() or scale_inv.dtype != torch.float32 or scale_inv.numel() != rows:
        raise ValueError("fp8q_dequant_per_channel: y must match q and scale_inv must be float32[rows]")
    _check(lib.fp8q_dequant_per_channel(_dev(q, "q"), f, rows, cols, _dev(scale_inv, "scale_inv"), _dev(y, "y"),
                                        _hp_dtype(y, "y"), _stream(q, stream)), "fp8q_dequant_per_channel")


def fp8q_dequant_per_group128(q, scale_inv, y, fmt=None, stream=None) -> None:
    f = _fp8(q, fmt, "q")
    rows, cols = _rows_cols(q)
    if y.numel() != q.numel() or scale_inv.dtype != torch.float32 or \
            (cols % 128 == 0 and scale_inv.numel() != rows * (cols // 128)):
        raise ValueError("fp8q_dequant_per_group128: y must match q and scale_inv must be float32[rows, cols/128]")
    _check(lib.fp8q_dequant_per_group128(_dev(q, "q"), f, rows, cols, _dev(scale_inv, "scale_inv"), _dev(y, "y"),
                                         _hp_dtype(y, "y"), _stream(q, stream)), "fp8q_dequant_per_group128")


def fp8q_weight_dequant_block128(q, scale_inv, y, fmt=None, stream=None) -> None:
    f = _fp8(q, fmt, "q")
    if q.dim() != 2 or scale_inv.dim() != 2:
        raise ValueError("fp8q_weight_dequant_block128: q and scale_inv must be 2-D")
    M, N = q.shape
    if tuple(scale_inv.shape) != ((M + 127) // 128, (N + 127) // 128) or scale_inv.dtype != torch.float32:
        raise ValueError("fp8q_weight_dequant_block128: scale_inv must be float32[ceil(M/128), ceil(N/128)]")
    if y.numel() != q.numel():
        raise ValueError("fp8q_weight_dequant_block128: y must match q")
    _check(lib.fp8q_weight_dequant_block128(_dev(q, "q"), f, M, N, _dev(scale_inv, "scale_inv"), _dev(y, "y"),
                                            _hp_dtype(y, "y"), _stream(q, stream)),
           "fp8q_weight_dequant_block128")


def fp8q_amax_guarded(x: torch.Tensor, amax: torch.Tensor, stream=None) -> None:
    if amax.dtype != torch.float32 or amax.numel() < 1:
        raise TypeError("amax must be a float32 tensor with at least one element")
    _check(lib.fp8q_amax_guarded(_dev(x, "x"), _hp_dtype(x, "x"), x.numel(), _dev(amax, "amax"),
                                 _stream(x, stream)), "fp8q_amax_guarded")


def fp8q_cast_with_amax(x, amax, q, scale_out, fmt="e5m2", stream=None) -> None:
    f = _fp8(q, fmt, "q")
    if q.numel() != x.numel() or amax.dtype != torch.float32 or scale_out.dtype != torch.float32:
        raise ValueError("fp8q_cast_with_amax: q must match x; amax and scale_out must be float32")
    _check(lib.fp8q_cast_with_amax(_dev(x, "x"), _hp_dtype(x, "x"), x.numel(), f, _dev(amax, "amax"), _dev(q, "q"),
                                   _dev(scale_out, "scale_out"), _stream(x, stream)), "fp8q_cast_with_amax")


def fp8q_dequant_div_scale(q, scale, y, fmt=None, stream=None) -> None:
    f = _fp8(q, fmt, "q")
    if y.numel() != q.numel() or scale.dtype != torch.float32:
        raise ValueError("fp8q_dequant_div_scale: y must match q and scale must be float32[1]")
    _check(lib.fp8q_dequant_div_scale(_dev(q, "q"), f, q.numel(), _dev(scale, "scale"), _dev(y, "y"),
                                      _hp_dtype(y, "y"), _stream(q, stream)), "fp8q_dequant_div_scale")


def _word(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.numel() < 1:
        raise TypeError(f"{name} must be an int32 tensor with at least one element")
    return _dev(t, name)


def fp8q_cast_to_fp8_pipeline(x, q, scale_inv, fmt_out, workspace, stream=None) -> None:
    """q: uint8 codes (the format is only known on the device); fmt_out:
    int32[1] on the device, 0 = e4m3fn, 1 = e5m2."""
    if q.dtype != torch.uint8 or q.numel() != x.numel():
        raise ValueError("fp8q_cast_to_fp8_pipeline: q must be uint8 codes matching x")
    if scale_inv.dtype != torch.float32 or scale_inv.numel() < 1:
        raise ValueError("fp8q_cast_to_fp8_pipeline: scale_inv must be float32[1]")
    if workspace.numel() * workspace.element_size() < fp8q_per_tensor_workspace_bytes():
        raise ValueError("fp8q_cast_to_fp8_pipeline: workspace too small")
    _check(lib.fp8q_cast_to_fp8_pipeline(_dev(x, "x"), _hp_dtype(x, "x"), x.numel(), _dev(q, "q"),
                                         _dev(scale_inv, "scale_inv"), _word(fmt_out, "fmt_out"),
                                         _dev(workspace, "workspace"), _stream(x, stream)),
           "fp8q_cast_to_fp8_pipeline")


def fp8q_cast_from_fp8_pipeline(q, fmt, scale_inv, y, stream=None) -> None:
    if q.dtype != torch.uint8 or y.numel() != q.numel() or scale_inv.dtype != torch.float32:
        raise ValueError("fp8q_cast_from_fp8_pipeline: q must be uint8 codes, y must match q and "
                         "scale_inv must be float32[1]")
    _check(lib.fp8q_cast_from_fp8_pipeline(_dev(q, "q"), _word(fmt, "fmt"), q.numel(), _dev(scale_inv, "scale_inv"),
                                           _dev(y, "y"), _hp_dtype(y, "y"), _stream(q, stream)),
           "fp8q_cast_from_fp8_pipeline")


def fp8q_cast_to_packed(x, slot, workspace, fmt="e5m2", stream=None) -> None:
    """slot: uint8 tensor of 4 + x.numel() bytes (4-byte aligned)."""
    if slot.dtype != torch.uint8 or slot.numel() != 4 + x.numel():
        raise ValueError("fp8q_cast_to_packed: slot must be uint8 with 4 + x.numel() bytes")
    if workspace.numel() * workspace.element_size() < fp8q_per_tensor_workspace_bytes():
        raise ValueError("fp8q_cast_to_packed: workspace too small")
    _check(lib.fp8q_cast_to_packed(_dev(x, "x"), _hp_dtype(x, "x"), x.numel(), _fmt(fmt), _dev(slot, "slot"),
                                   _dev(workspace, "workspace"), _stream(x, stream)), "fp8q_cast_to_packed")


def fp8q_dequant_packed(slots, W, n, y, fmt="e5m2", stream=None) -> None:
    """slots: uint8 tensor of W * (4 + n) bytes; y: W * n elements."""
    if slots.dtype != torch.uint8 or slots.numel() != W * (4 + n) or y.numel() != W * n:
        raise ValueError("fp8q_dequant_packed: slots must be uint8 with W * (4 + n) bytes and y W * n elements")
    _check(lib.fp8q_dequant_packed(_dev(slots, "slots"), _fmt(fmt), W, n, _dev(y, "y"), _hp_dtype(y, "y"),
                                   _stream(slots, stream)), "fp8q_dequant_packed")


def _sum_args(q, scale_inv, y, fmt):
    f = _fp8(q, fmt, "q")
    if q.dim() != 2:
        raise ValueError("q must be [W, n] (one received chunk per row)")
    W, n = q.shape
    if scale_inv.dtype != torch.float32 or scale_inv.numel() != W or y.numel() != n:
        raise ValueError("scale_inv must be float32[W] and y must have n elements")
    return f, W, n


def fp8q_dequant_sum(q, scale_inv, y, fmt=None, average=False, stream=None) -> None:
    f, W, n = _sum_args(q, scale_inv, y, fmt)
    _check(lib.fp8q_dequant_sum(_dev(q, "q"), f, W, n, _dev(scale_inv, "scale_inv"), int(bool(average)),
                                _dev(y, "y"), _hp_dtype(y, "y"), _stream(q, stream)), "fp8q_dequant_sum")


def fp8q_dequant_sum_requant(q, scale_inv, y, q_out, scale_inv_out, workspace, fmt=None, average=False,
                             stream=None) -> None:
    f, W, n = _sum_args(q, scale_inv, y, fmt)
    if q_out.numel() != n or scale_inv_out.dtype != torch.float32 or scale_inv_out.numel() < 1:
        raise ValueError("q_out must have n elements and scale_inv_out must be float32[1]")
    fo = _fp8(q_out, f, "q_out")
    if workspace.numel() * workspace.element_size() < fp8q_per_tensor_workspace_bytes():
        raise ValueError("workspace too small")
    _check(lib.fp8q_dequant_sum_requant(_dev(q, "q"), fo, W, n, _dev(scale_inv, "scale_inv"), int(bool(average)),
                                        _dev(y, "y"), _hp_dtype(y, "y"), _dev(q_out, "q_out"),
                                        _dev(scale_inv_out, "scale_inv_out"), _dev(workspace, "workspace"),
                                        _stream(q, stream)), "fp8q_dequant_sum_requant")


# ---------------------------------------------------------------------------
# page-level helpers (allocate outputs with torch; all compute in the kernels)
# ---------------------------------------------------------------------------

def cast_to_fp8(inp: torch.Tensor, fp8_format="e4m3", per_channel_scale=False, out=None):
    """(fp8 tensor, scale_inv) -- ColossalAI fp8.py cast_to_fp8.  scale_inv is
    float32[1] per-tensor or float32[rows] per-channel (row-indexed).  With
    `out` (an fp8 tensor of fp8_format, or uint8 codes, with inp's number of
    elements) the codes are written there and `out` is returned, as the page's
    torch.mul(scale, inp.float(), out=out) does."""
    f = _fmt(fp8_format)
    _hp_dtype(inp, "inp")
    if out is not None:
        _fp8(out, f, "out")
        if out.numel() != inp.numel():
            raise ValueError("cast_to_fp8: out must have as many elements as inp")
        q = out
    else:
        q = torch.empty(inp.shape, dtype=_FP8_DTYPE[f], device=inp.device)
    if per_channel_scale:
        rows, _ = _rows_cols(inp)
        sinv = torch.empty(rows, dtype=torch.float32, device=inp.device)
        fp8q_cast_per_channel(inp, q, sinv, f)
    else:
        sinv = torch.empty(1, dtype=torch.float32, device=inp.device)
        ws = torch.empty(fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device=inp.device)
        fp8q_cast_per_tensor(inp, q, sinv, ws, f)
    return q, sinv


def cast_from_fp8(inp: torch.Tensor, scale_inv: torch.Tensor, ret_type: torch.dtype, per_channel_scale=False,
                  out=None):
    """ColossalAI fp8.py cast_from_fp8: ret_type(fp32(inp) * scale_inv).  With
    `out`, the result is written there in out's own dtype and `out` is
    returned (the page's torch.mul(scale_inv, inp.float(), out=out))."""
    if inp.dtype not in (torch.float8_e4m3fn, torch.float8_e5m2):
        raise TypeError("Only float8_e4m3fn and float8_e5m2 are allowed.")
    if out is not None:
        if out.numel() != inp.numel():
            raise ValueError("cast_from_fp8: out must have as many elements as inp")
        y = out
    else:
        y = torch.empty(inp.shape, dtype=ret_type, device=inp.device)
    if per_channel_scale:
        fp8q_dequant_per_channel(inp, scale_inv.reshape(-1), y)
    else:
        fp8q_dequant_per_tensor(inp, scale_inv.reshape(-1), y)
    return y


def per_token_cast_to_fp8(x: torch.Tensor, fp8_format="e4m3fn"):
    """DeepEP per_token_cast_to_fp8: x [m, n], n % 128 == 0 ->
    (fp8 [m, n], scale_inv float32 [m, n/128])."""
    if x.dim() != 2 or x.size(1) % 128 != 0:
        raise ValueError("per_token_cast_to_fp8: x must be 2-D with x.size(1) % 128 == 0")
    f = _fmt(fp8_format)
    m, n = x.shape
    q = torch.empty((m, n), dtype=_FP8_DTYPE[f], device=x.device)
    sinv = torch.empty((m, n // 128), dtype=torch.float32, device=x.device)
    fp8q_cast_per_group128(x, q, sinv, f)
    return q, sinv


def per_token_cast_back(q: torch.Tensor, scale_inv: torch.Tensor, ret_type=torch.bfloat16):
    """Inverse of per_token_cast_to_fp8: ret_type(fp32(q) * scale_inv[r, c // 128])."""
    y = torch.empty(q.shape, dtype=ret_type, device=q.device)
    fp8q_dequant_per_group128(q, scale_inv, y)
    return y


def reduce_fp8_chunks(chunks: torch.Tensor, scales: torch.Tensor, input_type: torch.dtype, average=False,
                      requant=False, fp8_format=None):
    """The reduce step of the fp8-compressed collectives on one rank: chunks
    [W, n] fp8 received from W ranks with their scale_inv [W].  Returns the
    in-type sum (reduce-scatter), or (sum, fp8 re-cast, scale_inv) with
    requant=True (all-reduce)."""
    W, n = chunks.shape
    y = torch.empty(n, dtype=input_type, device=chunks.device)
    if not requant:
        fp8q_dequant_sum(chunks, scales, y, fp8_format, average)
        return y
    f = _fp8(chunks, fp8_format, "chunks")
    qo = torch.empty(n, dtype=_FP8_DTYPE[f], device=chunks.device)
    so = torch.empty(1, dtype=torch.float32, device=chunks.device)
    ws = torch.empty(fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device=chunks.device)
    fp8q_dequant_sum_requant(chunks, scales, y, qo, so, ws, fp8_format, average)
    return y, qo, so


def cast_to_fp8_pipeline(inp) -> None:
    """ColossalAI fp8.py cast_to_fp8_pipeline, in place on the dict: the
    "hidden_states" tensor becomes uint8 fp8 codes, "fp8_scale" its scale_inv
    (float32[1]), "fp8_format" the device int32 word naming the format the
    kernel chose (the page encodes it in the view dtype, which needs amax on
    the host), and "dtype" the original element type.  None and bare tensors
    are left alone, as on the page."""
    if inp is None or isinstance(inp, torch.Tensor):
        return
    x = inp["hidden_states"]
    dev = x.device
    q = torch.empty(x.shape, dtype=torch.uint8, device=dev)
    sinv = torch.empty(1, dtype=torch.float32, device=dev)
    word = torch.empty(1, dtype=torch.int32, device=dev)
    ws = torch.empty(fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device=dev)
    fp8q_cast_to_fp8_pipeline(x, q, sinv, word, ws)
    inp["hidden_states"] = q
    inp["fp8_scale"] = sinv
    inp["fp8_format"] = word
    inp["dtype"] = x.dtype


def cast_from_fp8_pipeline(inp, del_metadata=True) -> None:
    """ColossalAI fp8.py cast_from_fp8_pipeline: hidden_states back to the
    recorded dtype, the format taken from the device word."""
    if inp is None or isinstance(inp, torch.Tensor):
        return
    q = inp["hidden_states"]
    y = torch.empty(q.shape, dtype=inp["dtype"], device=q.device)
    fp8q_cast_from_fp8_pipeline(q, inp["fp8_format"], inp["fp8_scale"], y)
    inp["hidden_states"] = y
    if del_metadata:
        del inp["fp8_scale"], inp["fp8_format"], inp["dtype"]


def all_gather_pack(inp: torch.Tensor, combined: torch.Tensor, rank: int, world_size: int, fp8_format="e5m2"):
    """The send side of all_gather_fp8_lagacy / all_gather_fp8_ring: cast inp
    into rank's slot of the combined uint8 buffer (world_size * (4 + n)
    bytes)."""
    n = inp.numel()
    if combined.numel() != world_size * (4 + n) or not 0 <= rank < world_size:
        raise ValueError("all_gather_pack: combined must hold world_size * (4 + inp.numel()) bytes")
    ws = torch.empty(fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device=inp.device)
    fp8q_cast_to_packed(inp.reshape(-1), combined[rank * (4 + n):(rank + 1) * (4 + n)], ws, fp8_format)


def all_gather_unpack(combined: torch.Tensor, world_size: int, shape, input_type: torch.dtype, fp8_format="e5m2"):
    """The receive side: every slot of the combined buffer back to
    input_type, as one [world_size, *shape] tensor (output_list[w] = out[w])."""
    n = combined.numel() // world_size - 4
    out = torch.empty((world_size, *shape), dtype=input_type, device=combined.device)
    fp8q_dequant_packed(combined, world_size, n, out, fp8_format)
    return out


def weight_dequant(x: torch.Tensor, s: torch.Tensor, block_size: int = 128, ret_type=torch.bfloat16):
    """CSDN fp8_cast_bf16 notes, weight_dequant: x [M, N] fp8 with s
    [ceil(M/128), ceil(N/128)] -> ret_type (bf16, the page's default dtype)."""
    if block_size != 128:
        raise ValueError("weight_dequant: only block_size=128 is implemented")
    if x.dim() != 2 or s.dim() != 2:
        raise ValueError("Input tensors must have 2 dimensions")
    y = torch.empty(x.shape, dtype=ret_type, device=x.device)
    fp8q_weight_dequant_block128(x, s, y)
    return y
