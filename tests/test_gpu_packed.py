"""GPU parity: the packed [scale_inv | payload] slots of the fp8 all-gather --
every simulated rank casts into its own slot of one combined buffer
(fp8q_cast_to_packed), then all slots are read back in one launch
(fp8q_dequant_packed) or one at a time (the ring's per-step cast) --
bit-exact against the CPU oracle, bytes of the combined buffer included."""
import numpy as np
import pytest
import torch

import dequantize_amax_reduce_amd as fq
import oracle
from dequantize_amax_reduce_amd import workloads as W
from gpu_util import G, assert_hp_equal, dev, empty_hp, host

pytestmark = pytest.mark.gpu


def _ws():
    return G.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device="cuda:0")


def _inputs(Wn, n, dtype, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    xs = []
    for r in range(Wn):
        x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 3)).astype(np.float32)
        if r == 1:
            x[:] = 0.0
        xs.append(W.to_bf16_bits(x) if dtype == "bf16" else (x.astype(np.float16).view(np.uint16) if dtype == "f16"
                                                              else x))
    return xs


def _round_trip(xs, dtype, fmt, ydtypes, base_offset=0, what=""):
    Wn, n = len(xs), xs[0].size
    print(f"[case] packed {what} W={Wn} n={n} {dtype}->{fmt} offset={base_offset}", flush=True)
    ws = _ws()
    big = G.full((base_offset + Wn * (4 + n),), 0xA5, dtype=torch.uint8, device="cuda:0")
    combined = big[base_offset:]
    for r, x in enumerate(xs):
        fq.fp8q_cast_to_packed(dev(x, dtype), combined[r * (4 + n):(r + 1) * (4 + n)], ws, fmt)
    torch.cuda.synchronize()
    want = np.concatenate([oracle.cast_to_packed(x, dtype, fmt) for x in xs])
    got = host(combined)
    assert np.array_equal(got, want), f"{what}: combined buffer differs at {np.nonzero(got != want)[0][:8]}"
    for ydt in ydtypes:
        y = empty_hp((Wn, n), ydt)
        fq.fp8q_dequant_packed(combined, Wn, n, y, fmt)
        torch.cuda.synchronize()
        wy = oracle.dequant_packed(want, fmt, Wn, n, ydt)
        assert_hp_equal(host(y), wy, ydt, f"{what} -> {ydt}")
        # the ring: one slot per step, each into its own output
        y1 = empty_hp((Wn, n), ydt)
        for r in range(Wn):
            fq.fp8q_dequant_packed(combined[r * (4 + n):(r + 1) * (4 + n)], 1, n, y1[r], fmt)
        torch.cuda.synchronize()
        assert_hp_equal(host(y1), wy, ydt, f"{what} ring -> {ydt}")


@pytest.mark.parametrize("fmt", ["e5m2", "e4m3fn"])
@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_packed_shapes(fmt, dtype):
    # n * 2 % 16 == 0 (vector path), n % 4 == 0 only (element-wise rows), and one rank
    for Wn, n in ((2, 4096), (3, 1004), (8, 5000), (1, 37), (1, 1), (4, 8)):
        _round_trip(_inputs(Wn, n, dtype, seed=Wn * 7 + n), dtype, fmt, ("bf16", "f32", "f16"), what="shape")


def test_packed_fat_chunks():
    """Slot casts whose amax and cast passes take 4 or 8 sub-steps per chunk."""
    _round_trip(_inputs(2, 9_000_004, "bf16", seed=31), "bf16", "e5m2", ("bf16",), what="fat K=4")
    _round_trip(_inputs(1, 30_000_000, "bf16", seed=32), "bf16", "e4m3fn", ("f32",), what="fat K=8")
    _round_trip(_inputs(2, 12_000_000, "f32", seed=33), "f32", "e5m2", ("bf16",), what="fat f32 K=8")


def test_packed_base_offsets():
    """The combined buffer at 4, 8 and 12 bytes past a 16-B boundary."""
    for off in (4, 8, 12):
        _round_trip(_inputs(4, 2048, "bf16", seed=off), "bf16", "e5m2", ("bf16",), base_offset=off, what="offset")


def test_packed_empty_and_errors():
    slot = G.full((4,), 0xEE, dtype=torch.uint8, device="cuda:0")
    fq.fp8q_cast_to_packed(G.empty(0, dtype=torch.bfloat16, device="cuda:0"), slot, _ws(), "e5m2")
    torch.cuda.synchronize()
    assert list(host(slot)) == [0x00, 0x00, 0x80, 0x3F]
    y = empty_hp((3, 0), "bf16")
    fq.fp8q_dequant_packed(G.zeros(12, dtype=torch.uint8, device="cuda:0"), 3, 0, y, "e5m2")
    buf = G.zeros(2 * (4 + 6), dtype=torch.uint8, device="cuda:0")
    with pytest.raises(Exception):          # n % 4 != 0 with W > 1: rejected on the host
        fq.fp8q_dequant_packed(buf, 2, 6, empty_hp((2, 6), "bf16"), "e5m2")
    misaligned = G.zeros(3 + 4 + 8, dtype=torch.uint8, device="cuda:0")[3:]
    with pytest.raises(Exception):          # slot not 4-byte aligned
        fq.fp8q_cast_to_packed(dev(np.ones(8, np.float32)), misaligned[:12], _ws(), "e5m2")
    torch.cuda.synchronize()


def test_packed_helpers():
    xs = _inputs(4, 3 * 512, "bf16", seed=71)
    combined = G.empty(4 * (4 + xs[0].size), dtype=torch.uint8, device="cuda:0")
    for r, x in enumerate(xs):
        fq.all_gather_pack(dev(x, "bf16").reshape(3, 512), combined, r, 4, "e5m2")
    out = fq.all_gather_unpack(combined, 4, (3, 512), torch.bfloat16, "e5m2")
    torch.cuda.synchronize()
    want = np.concatenate([oracle.cast_to_packed(x, "bf16", "e5m2") for x in xs])
    assert out.shape == (4, 3, 512)
    assert_hp_equal(host(out), oracle.dequant_packed(want, "e5m2", 4, xs[0].size, "bf16"), "bf16")


def test_packed_full_size():
    """8 ranks, each with a 2^25-element bf16 share of the 2^28-element
    gradient-like payload, e5m2 slots, back to bf16."""
    x = W.gradient_payload()
    n = x.size // 8
    _round_trip([x[r * n:(r + 1) * n] for r in range(8)], "bf16", "e5m2", ("bf16",), what="full 8x2^25")
