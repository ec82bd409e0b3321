"""Helpers for the GPU parity tests: host <-> device marshalling, guarded
device buffers, and bit-exact comparisons with NaN compared by class (the
exact NaN code the hardware emits is not fixed by the pages).

Guard canaries: ``G.empty`` / ``G.full`` / ``G.zeros`` / ``G.ones`` allocate
every device buffer of a test inside a larger one, with GUARD bytes of a fixed
pattern before and after it.  The conftest fixture calls ``G.check()`` after
every GPU test: a kernel store past either end of an output (a ragged tail, a
byte-store path, a grid-stride edge) changes a guard and fails the test, where
a plain exact-size allocation would hide it.  Buffers above GUARD_LIMIT bytes
(the beyond-2^32 tests) are allocated plainly so that they can be freed
mid-test.
"""
from __future__ import annotations

import math

import numpy as np
import torch

FP8_NAN_CLASS = {
    "e4m3fn": lambda c: (c & 0x7F) == 0x7F,
    "e5m2": lambda c: ((c & 0x7C) == 0x7C) & ((c & 0x03) != 0),
}
TORCH_HP = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


GUARD = 4096                    # bytes of canary on each side (keeps 4 KiB alignment)
GUARD_PATTERN = 0xA5
GUARD_LIMIT = 2 << 30           # larger buffers are not guarded (they are freed mid-test)


class GuardedAllocator:
    """Device buffers with canary regions on both sides (see the module
    docstring).  The signatures follow torch.empty / torch.full."""

    def __init__(self):
        self.live = []          # (backing uint8 buffer, payload bytes, shape, dtype)

    @staticmethod
    def _shape(size):
        if len(size) == 1 and isinstance(size[0], (tuple, list, torch.Size)):
            size = tuple(size[0])
        return tuple(int(d) for d in size)

    def empty(self, *size, dtype=torch.float32, device="cuda:0"):
        shape = self._shape(size)
        if torch.device(device).type != "cuda":
            return torch.empty(shape, dtype=dtype, device=device)
        nbytes = math.prod(shape) * torch.empty(0, dtype=dtype).element_size()
        if nbytes > GUARD_LIMIT:
            return torch.empty(shape, dtype=dtype, device=device)
        raw = torch.empty(nbytes + 2 * GUARD, dtype=torch.uint8, device=device)
        raw[:GUARD].fill_(GUARD_PATTERN)
        raw[GUARD + nbytes:].fill_(GUARD_PATTERN)
        self.live.append((raw, nbytes, shape, dtype))
        return raw[GUARD:GUARD + nbytes].view(dtype).view(shape)

    def full(self, size, fill_value, dtype=torch.float32, device="cuda:0"):
        t = self.empty(size, dtype=dtype, device=device)
        return t.fill_(fill_value) if t.numel() else t

    def zeros(self, *size, dtype=torch.float32, device="cuda:0"):
        return self.full(self._shape(size), 0, dtype=dtype, device=device)

    def ones(self, *size, dtype=torch.float32, device="cuda:0"):
        return self.full(self._shape(size), 1, dtype=dtype, device=device)

    def check(self):
        """Synchronize, assert every live buffer's canaries are intact, and
        release them."""
        live, self.live = self.live, []
        if not live:
            return
        torch.cuda.synchronize()
        bad = []
        for raw, nbytes, shape, dtype in live:
            for side, g in (("before", raw[:GUARD]), ("after", raw[GUARD + nbytes:])):
                h = g.cpu().numpy()
                off = np.nonzero(h != GUARD_PATTERN)[0]
                if off.size:
                    bad.append(f"{side} {tuple(shape)} {dtype}: {off.size} guard bytes changed, first at "
                               f"offset {int(off[0]) - (GUARD if side == 'before' else 0)} "
                               f"from the {'start' if side == 'before' else 'end'} (value {int(h[off[0]]):#04x})")
        assert not bad, "store outside an output buffer: " + "; ".join(bad)


G = GuardedAllocator()


def dev(a: np.ndarray, dtype: str = None) -> torch.Tensor:
    """numpy host array -> contiguous device tensor (guarded).  uint16 arrays
    are reinterpreted as bf16 or f16 by `dtype`."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype in ("bf16", "f16"):
        t = t.view(torch.int16).view(TORCH_HP[dtype])
    out = G.empty(t.shape, dtype=t.dtype)
    if out.numel():
        out.copy_(t)
    return out


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().to("cpu")
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        return t.view(torch.uint8).numpy()
    return t.numpy()


def empty_hp(shape, dtype: str) -> torch.Tensor:
    return G.empty(shape, dtype=TORCH_HP[dtype], device="cuda:0")


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
