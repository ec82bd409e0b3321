"""Seeded synthetic inputs for the FP8 scaled-cast workloads.

This module holds no arithmetic of the method (no amax, scale, cast or
dequant): it only draws numbers.  Both the HIP path's tests/benchmark and the
CPU oracle consume the same host arrays produced here.

Recipe (every workload): ``numpy.random.Generator(PCG64(seed))``, normals drawn
with ``standard_normal(dtype=float32)``, bfloat16 inputs made by rounding those
float32 values to nearest-even with torch's CPU conversion.  bf16 arrays are
returned as uint16 bit patterns, fp8 codes as uint8.

The workloads stand in for the pages' data (activations [tokens, hidden],
FP8 checkpoint weights with 128x128 block scales, DDP gradient buckets); none
of the pages measures on a public dataset.
"""
from __future__ import annotations

import numpy as np
import torch


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 array of bfloat16 bits (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def group_cast_small(rows: int = 128, cols: int = 512, seed: int = 1,
                     zero_rows: int = 3, outlier_every: int = 10, outlier: float = 200.0):
    """Per-128-group cast input, small: bf16 [rows, cols] from N(0,1); every
    `outlier_every`-th group (row-major group order) gets one seeded position
    set to +-outlier (seeded sign); then `zero_rows` seeded distinct rows are
    set to +0.0 (overriding outliers), so all-zero groups hit the 1e-4 clamp."""
    rng = _rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    groups = rows * (cols // 128)
    gsel = np.arange(0, groups, outlier_every)
    pos = rng.integers(0, 128, size=gsel.size)
    sign = np.where(rng.integers(0, 2, size=gsel.size) == 1, 1.0, -1.0).astype(np.float32)
    flat = x.reshape(-1)
    flat[gsel * 128 + pos] = sign * np.float32(outlier)
    zr = rng.choice(rows, size=min(zero_rows, rows), replace=False)
    x[zr, :] = 0.0
    return to_bf16_bits(x), np.sort(zr)


def tensor_rows_scaled(rows: int = 4096, cols: int = 4096, seed: int = 2, zero_frac: float = 0.01):
    """Per-tensor / per-channel input: row r = N(0,1) * s_r with
    s_r = 10**U(-3, 3); round(zero_frac * rows) seeded rows set to zero.
    Returns (float32 array, bf16-bit array of the same values, zeroed rows)."""
    rng = _rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    s = (10.0 ** rng.uniform(-3.0, 3.0, size=rows)).astype(np.float32)
    x *= s[:, None]
    nz = int(round(zero_frac * rows))
    zr = rng.choice(rows, size=nz, replace=False) if nz else np.zeros(0, dtype=np.int64)
    x[zr, :] = 0.0
    return x, to_bf16_bits(x), np.sort(zr)


def activation_outlier_channels(rows: int = 16384, cols: int = 7168, seed: int = 3,
                                outlier_frac: float = 0.001, outlier_scale: float = 50.0):
    """LLM activation for the per-128-group quantize: bf16 [tokens, hidden] from
    N(0,1), with round(outlier_frac * cols) seeded channels scaled by
    outlier_scale over all tokens.  Returns (bf16 bits, outlier channels)."""
    rng = _rng(seed)
    nch = max(1, int(round(outlier_frac * cols)))
    ch = np.sort(rng.choice(cols, size=nch, replace=False))
    x = np.empty((rows, cols), dtype=np.uint16)
    step = 1024
    for r0 in range(0, rows, step):          # chunked to bound host memory
        blk = rng.standard_normal((min(step, rows - r0), cols), dtype=np.float32)
        blk[:, ch] *= np.float32(outlier_scale)
        x[r0:r0 + blk.shape[0]] = to_bf16_bits(blk)
    return x, ch


def block_weight(M: int = 18432, N: int = 7168, seed: int = 4, lo: float = -4.0, hi: float = -1.0):
    """FP8 e4m3fn weight with 128x128 block scales: codes uniform over the 254
    non-NaN codes (0x7F and 0xFF excluded); scale_inv [ceil(M/128), ceil(N/128)]
    float32 = 10**U(lo, hi).  Returns (uint8 codes [M, N], float32 scales)."""
    rng = _rng(seed)
    c = rng.integers(0, 254, size=(M, N), dtype=np.uint8)
    c = c + (c >= 0x7F).astype(np.uint8)          # skip 0x7F; 253 -> 0xFE, so 0xFF never occurs
    s = (10.0 ** rng.uniform(lo, hi, size=((M + 127) // 128, (N + 127) // 128))).astype(np.float32)
    return c, s


def gradient_payload(n: int = 1 << 28, seed: int = 5, sigma: float = 1e-3):
    """Gradient-like 1-D payload: bf16 [n] from N(0, sigma^2)."""
    rng = _rng(seed)
    out = np.empty(n, dtype=np.uint16)
    step = 1 << 24
    for i0 in range(0, n, step):
        blk = rng.standard_normal(min(step, n - i0), dtype=np.float32) * np.float32(sigma)
        out[i0:i0 + blk.size] = to_bf16_bits(blk)
    return out


def fp8_codes_finite(shape, fmt: str, seed: int):
    """Uniformly random fp8 codes excluding NaN (and inf for e5m2)."""
    rng = _rng(seed)
    if fmt == "e4m3fn":
        bad = {0x7F, 0xFF}
    else:
        bad = {0x7C, 0x7D, 0x7E, 0x7F, 0xFC, 0xFD, 0xFE, 0xFF}
    table = np.array([c for c in range(256) if c not in bad], dtype=np.uint8)
    return table[rng.integers(0, table.size, size=shape)]


def received_chunks(W: int, n: int, fmt: str = "e5m2", seed: int = 6, lo: float = -6.0, hi: float = -2.0):
    """What one rank holds at the reduce step of an fp8-compressed collective:
    W chunks of n fp8 codes (uniform over the finite codes) received from W
    ranks, each with its own per-tensor scale_inv = 10**U(lo, hi).
    Returns (uint8 codes [W, n], float32 scale_inv [W])."""
    rng = _rng(seed)
    codes = fp8_codes_finite((W, n), fmt, seed=seed + 1000)
    s = (10.0 ** rng.uniform(lo, hi, size=W)).astype(np.float32)
    return codes, s
