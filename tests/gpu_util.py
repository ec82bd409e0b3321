"""Helpers for the GPU parity tests: host <-> device marshalling and
bit-exact comparisons with NaN compared by class (the exact NaN code the
hardware emits is not fixed by the pages)."""
from __future__ import annotations

import numpy as np
import torch

FP8_NAN_CLASS = {
    "e4m3fn": lambda c: (c & 0x7F) == 0x7F,
    "e5m2": lambda c: ((c & 0x7C) == 0x7C) & ((c & 0x03) != 0),
}
TORCH_HP = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def dev(a: np.ndarray, dtype: str = None) -> torch.Tensor:
    """numpy host array -> contiguous device tensor.  uint16 arrays are
    reinterpreted as bf16 or f16 by `dtype`."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype in ("bf16", "f16"):
        t = t.view(torch.int16).view(TORCH_HP[dtype])
    return t.to("cuda:0")


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().to("cpu")
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        return t.view(torch.uint8).numpy()
    return t.numpy()


def empty_hp(shape, dtype: str) -> torch.Tensor:
    return torch.empty(shape, dtype=TORCH_HP[dtype], device="cuda:0")


def assert_fp8_equal(got: np.ndarray, want: np.ndarray, fmt: str, what: str = ""):
    got = np.asarray(got, np.uint8).reshape(-1)
    want = np.asarray(want, np.uint8).reshape(-1)
    assert got.shape == want.shape, what
    nan_w = FP8_NAN_CLASS[fmt](want)
    nan_g = FP8_NAN_CLASS[fmt](got)
    bad = np.nonzero((got != want) & ~(nan_w & nan_g))[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {got.size} fp8 codes differ; first at {bad[:8]}: "
                           f"got {got[bad[:8]]} want {want[bad[:8]]}")


def assert_f32_equal(got: np.ndarray, want: np.ndarray, what: str = ""):
    got = np.asarray(got, np.float32).reshape(-1)
    want = np.asarray(want, np.float32).reshape(-1)
    assert got.shape == want.shape, what
    gb, wb = got.view(np.uint32), want.view(np.uint32)
    both_nan = np.isnan(got) & np.isnan(want)
    bad = np.nonzero((gb != wb) & ~both_nan)[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {got.size} fp32 values differ; first at {bad[:8]}: "
                           f"got {got[bad[:8]]} want {want[bad[:8]]}")


def assert_u16_equal(got: np.ndarray, want: np.ndarray, kind: str, what: str = ""):
    """bf16 or f16 bit patterns; NaN by class."""
    got = np.asarray(got, np.uint16).reshape(-1)
    want = np.asarray(want, np.uint16).reshape(-1)
    assert got.shape == want.shape, what
    if kind == "bf16":
        nan = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    else:
        nan = lambda b: ((b & 0x7C00) == 0x7C00) & ((b & 0x3FF) != 0)
    bad = np.nonzero((got != want) & ~(nan(got) & nan(want)))[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {got.size} {kind} values differ; first at {bad[:8]}: "
                           f"got {got[bad[:8]]} want {want[bad[:8]]}")


def assert_hp_equal(got: np.ndarray, want: np.ndarray, dtype: str, what: str = ""):
    if dtype == "f32":
        assert_f32_equal(got, want, what)
    else:
        assert_u16_equal(got, want, dtype, what)
