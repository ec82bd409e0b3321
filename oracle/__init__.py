"""CPU oracle for the FP8 scaled-cast path (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library in
``dequantize_amax_reduce_amd``) never imports it and never falls back to it.

The arithmetic lives in ``fp8_oracle.c`` (plain C, binary32, no FMA
contraction, no flush-to-zero); this module only builds it with gcc and
marshals numpy arrays through ctypes.  Element types: ``"f32"`` (float32
arrays), ``"bf16"`` (uint16 arrays holding bfloat16 bits), ``"f16"`` (uint16
or float16 arrays holding binary16 bits).  fp8 codes are uint8 arrays.

``OracleLib(path)`` wraps any build of the C source (the tests also build
deliberately broken copies to show that the pins catch them); the module-level
functions use the default build ``oracle/libfp8_oracle.so``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "fp8_oracle.c")
LIB = os.path.join(_HERE, "libfp8_oracle.so")

DTYPES = {"f32": 0, "bf16": 1, "f16": 2}
FORMATS = {"e4m3fn": 0, "e5m2": 1}
FORMAT_NAMES = {v: k for k, v in FORMATS.items()}


def build(force: bool = True, src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle C source with gcc into a shared library."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fno-unsafe-math-optimizations", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-I", _HERE, "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(tmp, out)
    return out


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _in(a, dtype: str) -> np.ndarray:
    a = np.asarray(a)
    if dtype == "f16" and a.dtype == np.float16:
        a = a.view(np.uint16)
    want = np.float32 if dtype == "f32" else np.uint16
    if a.dtype != want:
        raise TypeError(f"oracle: {dtype} input must be a {np.dtype(want).name} array, got {a.dtype}")
    return np.ascontiguousarray(a)


def _out(shape, dtype: str) -> np.ndarray:
    return np.empty(shape, dtype=np.float32 if dtype == "f32" else np.uint16)


def _check(rc: int, what: str):
    if rc == -9:
        raise RuntimeError("oracle: FPU is in flush-to-zero / denormals-are-zero mode")
    if rc == -3:
        raise ValueError(f"{what}: cols must be a multiple of 128")
    if rc != 0:
        raise ValueError(f"{what}: invalid arguments (rc={rc})")


class OracleLib:
    """ctypes wrapper of one build of fp8_oracle.c."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        P, I64, I, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        sigs = {
            "oracle_fpu_check": (I, []),
            "oracle_fp8_decode": (F, [ctypes.c_uint8, I]),
            "oracle_fp8_encode": (ctypes.c_uint8, [F, I]),
            "oracle_fp8_max": (F, [I]),
            "oracle_fp8_encode_array": (None, [P, I64, I, P]),
            "oracle_fp8_decode_array": (None, [P, I64, I, P]),
            "oracle_bf16_from_f32_array": (None, [P, I64, P]),
            "oracle_f16_from_f32_array": (None, [P, I64, P]),
            "oracle_amax": (F, [P, I, I64]),
            "oracle_per_tensor_scale": (None, [F, I, P, P]),
            "oracle_scale_and_cast": (None, [P, I, I64, F, I, P]),
            "oracle_cast_per_tensor": (I, [P, I, I64, I, P, P]),
            "oracle_cast_per_channel": (I, [P, I, I64, I64, I, P, P]),
            "oracle_cast_per_group128": (I, [P, I, I64, I64, I, P, P]),
            "oracle_dequant_per_tensor": (I, [P, I, I64, P, P, I]),
            "oracle_dequant_per_channel": (I, [P, I, I64, I64, P, P, I]),
            "oracle_dequant_per_group128": (I, [P, I, I64, I64, P, P, I]),
            "oracle_weight_dequant_block128": (I, [P, I, I64, I64, P, P, I]),
            "oracle_dequant_sum": (I, [P, I, I64, I64, P, I, P, I]),
            "oracle_dequant_sum_requant": (I, [P, I, I64, I64, P, I, P, I, P, P]),
            "oracle_amax_guarded": (F, [P, I, I64]),
            "oracle_cast_with_amax": (I, [P, I, I64, I, F, P, P]),
            "oracle_dequant_div_scale": (I, [P, I, I64, F, P, I]),
            "oracle_cast_to_fp8_pipeline": (I, [P, I, I64, P, P, P]),
            "oracle_cast_from_fp8_pipeline": (I, [P, I, I64, F, P, I]),
            "oracle_cast_to_packed": (I, [P, I, I64, I, P]),
            "oracle_dequant_packed": (I, [P, I, I64, I64, P, I]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        self.L = L
        self.path = path

    # ---- element codecs -------------------------------------------------
    def fp8_encode(self, v, fmt: str) -> np.ndarray:
        v = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
        out = np.empty(v.shape, dtype=np.uint8)
        self.L.oracle_fp8_encode_array(_ptr(v), v.size, FORMATS[fmt], _ptr(out))
        return out

    def fp8_decode(self, c, fmt: str) -> np.ndarray:
        c = np.ascontiguousarray(np.asarray(c, dtype=np.uint8))
        out = np.empty(c.shape, dtype=np.float32)
        self.L.oracle_fp8_decode_array(_ptr(c), c.size, FORMATS[fmt], _ptr(out))
        return out

    def fp8_max(self, fmt: str) -> float:
        return float(self.L.oracle_fp8_max(FORMATS[fmt]))

    def bf16_from_f32(self, v) -> np.ndarray:
        v = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
        out = np.empty(v.shape, dtype=np.uint16)
        self.L.oracle_bf16_from_f32_array(_ptr(v), v.size, _ptr(out))
        return out

    def f16_from_f32(self, v) -> np.ndarray:
        v = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
        out = np.empty(v.shape, dtype=np.uint16)
        self.L.oracle_f16_from_f32_array(_ptr(v), v.size, _ptr(out))
        return out

    # ---- steps ----------------------------------------------------------
    def amax(self, x, dtype: str) -> np.float32:
        x = _in(x, dtype)
        return np.float32(self.L.oracle_amax(_ptr(x), DTYPES[dtype], x.size))

    def per_tensor_scale(self, amax_value, fmt: str):
        s, si = ctypes.c_float(), ctypes.c_float()
        self.L.oracle_per_tensor_scale(float(np.float32(amax_value)), FORMATS[fmt],
                                       ctypes.byref(s), ctypes.byref(si))
        return np.float32(s.value), np.float32(si.value)

    def scale_and_cast(self, x, dtype: str, scale, fmt: str) -> np.ndarray:
        x = _in(x, dtype)
        q = np.empty(x.shape, dtype=np.uint8)
        self.L.oracle_scale_and_cast(_ptr(x), DTYPES[dtype], x.size, float(np.float32(scale)),
                                     FORMATS[fmt], _ptr(q))
        return q

    # ---- whole operations -----------------------------------------------
    def cast_per_tensor(self, x, dtype: str, fmt: str):
        """-> (q uint8 with x's shape, scale_inv float32[1])"""
        x = _in(x, dtype)
        q = np.zeros(x.shape, dtype=np.uint8)
        si = np.zeros(1, dtype=np.float32)
        _check(self.L.oracle_cast_per_tensor(_ptr(x), DTYPES[dtype], x.size, FORMATS[fmt],
                                             _ptr(q), _ptr(si)), "cast_per_tensor")
        return q, si

    def cast_per_channel(self, x, dtype: str, fmt: str):
        """x [rows, cols] -> (q [rows, cols], scale_inv float32[rows])"""
        x = _in(x, dtype)
        rows, cols = x.shape
        q = np.zeros(x.shape, dtype=np.uint8)
        si = np.zeros(rows, dtype=np.float32)
        _check(self.L.oracle_cast_per_channel(_ptr(x), DTYPES[dtype], rows, cols, FORMATS[fmt],
                                              _ptr(q), _ptr(si)), "cast_per_channel")
        return q, si

    def cast_per_group128(self, x, dtype: str, fmt: str = "e4m3fn"):
        """x [rows, cols], cols % 128 == 0 -> (q [rows, cols], scale_inv float32[rows, cols/128])"""
        x = _in(x, dtype)
        rows, cols = x.shape
        q = np.zeros(x.shape, dtype=np.uint8)
        si = np.zeros((rows, cols // 128 if cols % 128 == 0 else 0), dtype=np.float32)
        _check(self.L.oracle_cast_per_group128(_ptr(x), DTYPES[dtype], rows, cols, FORMATS[fmt],
                                               _ptr(q), _ptr(si)), "cast_per_group128")
        return q, si

    def dequant_per_tensor(self, q, fmt: str, scale_inv, ydtype: str):
        q = np.ascontiguousarray(np.asarray(q, dtype=np.uint8))
        si = np.ascontiguousarray(np.asarray(scale_inv, dtype=np.float32).reshape(-1))
        y = _out(q.shape, ydtype)
        _check(self.L.oracle_dequant_per_tensor(_ptr(q), FORMATS[fmt], q.size, _ptr(si), _ptr(y),
                                                DTYPES[ydtype]), "dequant_per_tensor")
        return y

    def dequant_per_channel(self, q, fmt: str, scale_inv, ydtype: str):
        q = np.ascontiguousarray(np.asarray(q, dtype=np.uint8))
        si = np.ascontiguousarray(np.asarray(scale_inv, dtype=np.float32).reshape(-1))
        rows, cols = q.shape
        y = _out(q.shape, ydtype)
        _check(self.L.oracle_dequant_per_channel(_ptr(q), FORMATS[fmt], rows, cols, _ptr(si), _ptr(y),
                                                 DTYPES[ydtype]), "dequant_per_channel")
        return y

    def dequant_per_group128(self, q, fmt: str, scale_inv, ydtype: str):
        q = np.ascontiguousarray(np.asarray(q, dtype=np.uint8))
        si = np.ascontiguousarray(np.asarray(scale_inv, dtype=np.float32))
        rows, cols = q.shape
        y = _out(q.shape, ydtype)
        _check(self.L.oracle_dequant_per_group128(_ptr(q), FORMATS[fmt], rows, cols, _ptr(si), _ptr(y),
                                                  DTYPES[ydtype]), "dequant_per_group128")
        return y

    def weight_dequant_block128(self, q, fmt: str, scale_inv, ydtype: str = "bf16"):
        q = np.ascontiguousarray(np.asarray(q, dtype=np.uint8))
        si = np.ascontiguousarray(np.asarray(scale_inv, dtype=np.float32))
        M, N = q.shape
        if si.shape != ((M + 127) // 128, (N + 127) // 128):
            raise ValueError("weight_dequant_block128: scale_inv must be [ceil(M/128), ceil(N/128)]")
        y = _out(q.shape, ydtype)
        _check(self.L.oracle_weight_dequant_block128(_ptr(q), FORMATS[fmt], M, N, _ptr(si), _ptr(y),
                                                     DTYPES[ydtype]), "weight_dequant_block128")
        return y


    # ---- reduce step of the compressed collectives ----------------------
    def dequant_sum(self, q, fmt: str, scale_inv, ydtype: str, average: bool = False):
        """q [W, n] fp8 codes, scale_inv [W] -> the chunk-ordered sum [n] in ydtype"""
        q = np.ascontiguousarray(np.asarray(q, dtype=np.uint8))
        W, n = q.shape
        si = np.ascontiguousarray(np.asarray(scale_inv, dtype=np.float32).reshape(-1))
        if si.size != W:
            raise ValueError("dequant_sum: scale_inv must have W entries")
        y = _out(n, ydtype)
        _check(self.L.oracle_dequant_sum(_ptr(q), FORMATS[fmt], W, n, _ptr(si), int(average), _ptr(y),
                                         DTYPES[ydtype]), "dequant_sum")
        return y

    def dequant_sum_requant(self, q, fmt: str, scale_inv, ydtype: str, average: bool = False):
        """-> (summed [n] in ydtype, q_out [n], scale_inv_out [1])"""
        q = np.ascontiguousarray(np.asarray(q, dtype=np.uint8))
        W, n = q.shape
        si = np.ascontiguousarray(np.asarray(scale_inv, dtype=np.float32).reshape(-1))
        if si.size != W:
            raise ValueError("dequant_sum_requant: scale_inv must have W entries")
        y = _out(n, ydtype)
        qo = np.zeros(n, dtype=np.uint8)
        so = np.zeros(1, dtype=np.float32)
        _check(self.L.oracle_dequant_sum_requant(_ptr(q), FORMATS[fmt], W, n, _ptr(si), int(average), _ptr(y),
                                                 DTYPES[ydtype], _ptr(qo), _ptr(so)), "dequant_sum_requant")
        return y, qo, so


    # ---- FSDP parameter hook: cross-rank global amax -----------------------
    def amax_guarded(self, x, dtype: str) -> np.float32:
        x = _in(x, dtype)
        return np.float32(self.L.oracle_amax_guarded(_ptr(x), DTYPES[dtype], x.size))

    def cast_with_amax(self, x, dtype: str, fmt: str, amax):
        """-> (q with x's shape, scale float32[1])"""
        x = _in(x, dtype)
        q = np.zeros(x.shape, dtype=np.uint8)
        sc = np.zeros(1, dtype=np.float32)
        _check(self.L.oracle_cast_with_amax(_ptr(x), DTYPES[dtype], x.size, FORMATS[fmt], float(np.float32(amax)),
                                            _ptr(q), _ptr(sc)), "cast_with_amax")
        return q, sc

    def dequant_div_scale(self, q, fmt: str, scale, ydtype: str):
        q = np.ascontiguousarray(np.asarray(q, dtype=np.uint8))
        y = _out(q.shape, ydtype)
        _check(self.L.oracle_dequant_div_scale(_ptr(q), FORMATS[fmt], q.size, float(np.float32(scale)), _ptr(y),
                                               DTYPES[ydtype]), "dequant_div_scale")
        return y

    def cast_to_fp8_pipeline(self, x, dtype: str):
        """-> (q with x's shape, scale_inv float32[1], fmt name)"""
        x = _in(x, dtype)
        q = np.zeros(x.shape, dtype=np.uint8)
        si = np.zeros(1, dtype=np.float32)
        f = np.zeros(1, dtype=np.int32)
        _check(self.L.oracle_cast_to_fp8_pipeline(_ptr(x), DTYPES[dtype], x.size, _ptr(q), _ptr(si), _ptr(f)),
               "cast_to_fp8_pipeline")
        return q, si, FORMAT_NAMES[int(f[0])]

    def cast_from_fp8_pipeline(self, q, fmt: str, scale_inv, ydtype: str):
        q = np.ascontiguousarray(np.asarray(q, dtype=np.uint8))
        y = _out(q.shape, ydtype)
        _check(self.L.oracle_cast_from_fp8_pipeline(_ptr(q), FORMATS[fmt], q.size, float(np.float32(scale_inv)),
                                                    _ptr(y), DTYPES[ydtype]), "cast_from_fp8_pipeline")
        return y

    def cast_to_packed(self, x, dtype: str, fmt: str) -> np.ndarray:
        """-> uint8[4 + n]: binary32 scale_inv, then the n codes"""
        x = _in(x, dtype)
        slot = np.zeros(4 + x.size, dtype=np.uint8)
        _check(self.L.oracle_cast_to_packed(_ptr(x), DTYPES[dtype], x.size, FORMATS[fmt], _ptr(slot)),
               "cast_to_packed")
        return slot

    def dequant_packed(self, slots, fmt: str, W: int, n: int, ydtype: str):
        """slots: uint8[W * (4 + n)] -> y [W, n]"""
        slots = np.ascontiguousarray(np.asarray(slots, dtype=np.uint8).reshape(-1))
        if slots.size != W * (4 + n):
            raise ValueError("dequant_packed: slots must hold W * (4 + n) bytes")
        y = _out((W, n), ydtype)
        _check(self.L.oracle_dequant_packed(_ptr(slots), FORMATS[fmt], W, n, _ptr(y), DTYPES[ydtype]),
               "dequant_packed")
        return y


_default = None


def default() -> OracleLib:
    """The default build (compiled on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB):
            build()
        _default = OracleLib(LIB)
    return _default


def __getattr__(name):
    # module-level access to the default build's methods: oracle.cast_per_group128(...)
    if not name.startswith("_") and hasattr(OracleLib, name):
        return getattr(default(), name)
    raise AttributeError(name)
