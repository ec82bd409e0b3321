"""CPU tests of the C ABI boundary: the HIP library loads without a GPU,
exports every function include/fp8q.h declares, and every argument error is
reported before any HIP call (these calls enqueue nothing, so they need no
GPU).  Fake device addresses are never dereferenced on these paths."""
import ctypes
import os
import re
import subprocess

import pytest

import dequantize_amax_reduce_amd as fq

# test_sanitizers.py reruns this file against the ABI layer built with
# -fsanitize=address,undefined over host-only launcher stubs
# (tests/sanitize/fp8q_launch_stubs.cpp); FP8Q_ABI_LIB names that build.
LIB_PATH = os.environ.get("FP8Q_ABI_LIB") or fq.LIB_PATH
L = fq._load(LIB_PATH) if LIB_PATH != fq.LIB_PATH else fq.lib
STUBS = hasattr(L, "fp8q_stub_count")
P = lambda a: ctypes.c_void_p(a)          # a fake, never-dereferenced address
A = 0x7F0000000000                          # 256-B aligned fake base
E4, E5, F32, BF16, F16 = 0, 1, 0, 1, 2


def test_exports_match_header():
    declared = fq.header_functions()
    assert set(declared) == set(fq.ABI_FUNCTIONS)
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (fp8q_\w+)$", out, re.M))
    assert set(declared) <= exported, set(declared) - exported


def test_version_and_strings():
    assert L.fp8q_abi_version() == 1
    for st in range(7):
        assert L.fp8q_status_str(st)
    assert L.fp8q_per_tensor_workspace_bytes() >= 4
    assert L.fp8q_per_tensor_workspace_bytes() % 16 == 0


def test_group128_errors():
    f = L.fp8q_cast_per_group128
    assert f(P(A), BF16, 4, 100, E4, P(A + 4096), P(A + 8192), None) == fq.ESHAPE
    assert f(P(A), 7, 4, 128, E4, P(A + 4096), P(A + 8192), None) == fq.EDTYPE
    assert f(P(A), BF16, 4, 128, 9, P(A + 4096), P(A + 8192), None) == fq.EDTYPE
    assert f(P(A), BF16, -1, 128, E4, P(A + 4096), P(A + 8192), None) == fq.EINVAL
    assert f(None, BF16, 4, 128, E4, P(A + 4096), P(A + 8192), None) == fq.EINVAL
    assert f(P(A), BF16, 4, 128, E4, None, P(A + 8192), None) == fq.EINVAL
    assert f(P(A), BF16, 4, 128, E4, P(A + 4096), None, None) == fq.EINVAL
    assert f(P(A + 1), BF16, 4, 128, E4, P(A + 4096), P(A + 8192), None) == fq.EALIGN
    assert f(P(A), F32, 4, 128, E4, P(A + 4096), P(A + 8194), None) == fq.EALIGN
    assert f(P(A), BF16, 4, 128, E4, P(A + 512), P(A + 8192), None) == fq.EINVAL      # x/q overlap
    assert f(P(A), BF16, 4, 128, E4, P(A + 4096), P(A + 4096 + 500), None) == fq.EINVAL  # q/s overlap
    assert f(P(A), BF16, 2 ** 62, 2 ** 10, E4, P(A + 4096), P(A + 8192), None) == fq.EINVAL  # overflow
    # empty shapes are valid no-ops that never touch the pointers
    assert f(None, BF16, 0, 128, E4, None, None, None) == fq.OK
    assert f(None, BF16, 5, 0, E4, None, None, None) == fq.OK


def test_group128_wave64_errors():
    """The one-wavefront-per-group variant validates like the group cast and
    also needs x aligned to two elements and q to 2 bytes."""
    f = L.fp8q_cast_per_group128_wave64
    assert f(P(A), BF16, 4, 100, E4, P(A + 4096), P(A + 8192), None) == fq.ESHAPE
    assert f(P(A), 7, 4, 128, E4, P(A + 4096), P(A + 8192), None) == fq.EDTYPE
    assert f(None, BF16, 4, 128, E4, P(A + 4096), P(A + 8192), None) == fq.EINVAL
    assert f(P(A + 2), BF16, 4, 128, E4, P(A + 4096), P(A + 8192), None) == fq.EALIGN   # one bf16 in
    assert f(P(A + 4), F32, 4, 128, E4, P(A + 4096), P(A + 8192), None) == fq.EALIGN    # one fp32 in
    assert f(P(A), BF16, 4, 128, E4, P(A + 4097), P(A + 8192), None) == fq.EALIGN       # q odd
    assert f(None, BF16, 0, 128, E4, None, None, None) == fq.OK
    assert f(P(A + 1), BF16, 0, 128, E4, P(A + 4097), P(A + 8192), None) == fq.EALIGN


def test_tensor_and_channel_errors():
    t = L.fp8q_cast_per_tensor
    assert t(P(A), BF16, 16, E4, P(A + 4096), P(A + 8192), None, None) == fq.EINVAL       # no workspace
    assert t(P(A), BF16, 16, E4, P(A + 4096), P(A + 8192), P(A + 8194), None) == fq.EALIGN
    assert t(P(A), BF16, 16, E4, P(A + 4096), P(A + 8192), P(A + 8192), None) == fq.EINVAL  # ws = scale_inv
    assert t(P(A), 3, 16, E4, P(A + 4096), P(A + 8192), P(A + 9000), None) == fq.EDTYPE
    assert t(P(A), BF16, -5, E4, P(A + 4096), P(A + 8192), P(A + 9000), None) == fq.EINVAL
    t = L.fp8q_cast_per_tensor_noalloc
    assert t(P(A), BF16, -5, E4, P(A + 4096), P(A + 8192), None) == fq.EINVAL
    assert t(P(A), 3, 16, E4, P(A + 4096), P(A + 8192), None) == fq.EDTYPE
    assert t(P(A), BF16, 16, 7, P(A + 4096), P(A + 8192), None) == fq.EDTYPE
    assert t(P(A), BF16, 16, E4, None, P(A + 8192), None) == fq.EINVAL
    assert t(P(A), BF16, 16, E4, P(A + 4096), None, None) == fq.EINVAL
    assert t(P(A + 1), BF16, 16, E4, P(A + 4096), P(A + 8192), None) == fq.EALIGN
    assert t(P(A), BF16, 16, E4, P(A + 4096), P(A + 8194), None) == fq.EALIGN
    assert t(P(A), BF16, 16, E4, P(A + 8), P(A + 8192), None) == fq.EINVAL                 # x/q overlap
    assert t(P(A), BF16, 16, E4, P(A + 4096), P(A + 4100), None) == fq.EINVAL              # q/scale overlap
    c = L.fp8q_cast_per_channel
    assert c(P(A), F32, 4, 16, E5, P(A + 4096), None, None) == fq.EINVAL
    assert c(P(A + 2), F32, 4, 16, E5, P(A + 4096), P(A + 8192), None) == fq.EALIGN
    assert c(P(A), F32, 4, -16, E5, P(A + 4096), P(A + 8192), None) == fq.EINVAL
    assert c(None, F32, 0, 16, E5, None, None, None) == fq.OK
    a = L.fp8q_amax
    assert a(P(A), F32, 10, None, None) == fq.EINVAL
    assert a(P(A), F32, 10, P(A + 2), None) == fq.EALIGN
    assert a(P(A), F32, 10, P(A + 4), None) == fq.EINVAL                                   # overlap
    assert a(P(A), 5, 10, P(A + 4096), None) == fq.EDTYPE


def test_dequant_errors():
    d = L.fp8q_dequant_per_tensor
    assert d(P(A), E4, 16, None, P(A + 4096), BF16, None) == fq.EINVAL
    assert d(P(A), E4, 16, P(A + 8192), P(A + 4097), BF16, None) == fq.EALIGN
    assert d(P(A), E4, 16, P(A + 8192), P(A + 8), BF16, None) == fq.EINVAL                 # q/y overlap
    assert d(P(A), 2, 16, P(A + 8192), P(A + 4096), BF16, None) == fq.EDTYPE
    assert d(None, E4, 0, None, None, BF16, None) == fq.OK
    g = L.fp8q_dequant_per_group128
    assert g(P(A), E4, 4, 130, P(A + 8192), P(A + 4096 * 4), F32, None) == fq.ESHAPE
    assert g(P(A), E4, 4, 128, P(A + 8193), P(A + 4096 * 4), F32, None) == fq.EALIGN
    r = L.fp8q_dequant_per_channel
    assert r(P(A), E4, 4, 16, P(A + 8192), P(A + 4096), 9, None) == fq.EDTYPE
    b = L.fp8q_weight_dequant_block128
    assert b(P(A), E4, -1, 16, P(A + 8192), P(A + 4096), BF16, None) == fq.EINVAL
    assert b(P(A), E4, 2 ** 62, 2 ** 62, P(A + 8192), P(A + 4096), BF16, None) == fq.EINVAL
    assert b(P(A), E4, 16, 16, None, P(A + 4096), BF16, None) == fq.EINVAL
    assert b(None, E4, 0, 16, None, None, BF16, None) == fq.OK


def test_fsdp_hook_errors():
    g = L.fp8q_amax_guarded
    assert g(P(A), BF16, 10, None, None) == fq.EINVAL
    assert g(P(A), 7, 10, P(A + 4096), None) == fq.EDTYPE
    assert g(P(A), F32, 10, P(A + 4), None) == fq.EINVAL                                   # overlap
    c = L.fp8q_cast_with_amax
    assert c(P(A), BF16, -1, E5, P(A + 9000), P(A + 4096), P(A + 8192), None) == fq.EINVAL
    assert c(P(A), BF16, 16, E5, None, P(A + 4096), P(A + 8192), None) == fq.EINVAL         # no amax
    assert c(P(A), BF16, 16, E5, P(A + 9001), P(A + 4096), P(A + 8192), None) == fq.EALIGN
    assert c(P(A), BF16, 16, E5, P(A + 8), P(A + 4096), P(A + 8192), None) == fq.EINVAL     # amax in x
    assert c(P(A), BF16, 16, E5, P(A + 8192), P(A + 4096), P(A + 8192), None) == fq.EINVAL  # amax = scale
    assert c(P(A), BF16, 16, 3, P(A + 9000), P(A + 4096), P(A + 8192), None) == fq.EDTYPE
    assert c(P(A), BF16, 16, E5, P(A + 9000), P(A + 4096), None, None) == fq.EINVAL         # no scale out
    d = L.fp8q_dequant_div_scale
    assert d(P(A), E5, 16, None, P(A + 4096), BF16, None) == fq.EINVAL
    assert d(P(A), E5, 16, P(A + 8192), P(A + 4097), BF16, None) == fq.EALIGN
    assert d(P(A), E5, 16, P(A + 8192), P(A + 8), F32, None) == fq.EINVAL                  # q/y overlap
    assert d(P(A), E5, -3, P(A + 8192), P(A + 4096), F32, None) == fq.EINVAL
    assert d(None, E5, 0, None, None, F32, None) == fq.OK


def test_pipeline_errors():
    c = L.fp8q_cast_to_fp8_pipeline
    ws, fw = P(A + 16384), P(A + 12288)
    assert c(P(A), BF16, -1, P(A + 4096), P(A + 8192), fw, ws, None) == fq.EINVAL
    assert c(P(A), 5, 16, P(A + 4096), P(A + 8192), fw, ws, None) == fq.EDTYPE
    assert c(P(A), BF16, 16, P(A + 4096), P(A + 8192), None, ws, None) == fq.EINVAL          # no format word
    assert c(P(A), BF16, 16, P(A + 4096), P(A + 8192), fw, None, None) == fq.EINVAL          # no workspace
    assert c(P(A), BF16, 16, P(A + 4096), P(A + 8192), P(A + 12290), ws, None) == fq.EALIGN
    assert c(P(A), BF16, 16, P(A + 4096), P(A + 8192), P(A + 8192), ws, None) == fq.EINVAL   # word = scale_inv
    assert c(P(A), BF16, 16, P(A + 4096), P(A + 8192), P(A + 16400), ws, None) == fq.EINVAL  # word in workspace
    assert c(P(A), BF16, 16, P(A + 4096), P(A + 8192), P(A + 8), ws, None) == fq.EINVAL      # word in x
    d = L.fp8q_cast_from_fp8_pipeline
    assert d(P(A), None, 16, P(A + 8192), P(A + 4096), BF16, None) == fq.EINVAL
    assert d(P(A), P(A + 12290), 16, P(A + 8192), P(A + 4096), BF16, None) == fq.EALIGN
    assert d(P(A), P(A + 4100), 16, P(A + 8192), P(A + 4096), BF16, None) == fq.EINVAL      # word in y
    assert d(P(A), fw, 16, None, P(A + 4096), BF16, None) == fq.EINVAL
    assert d(P(A), fw, 16, P(A + 8192), P(A + 4096), 7, None) == fq.EDTYPE
    assert d(P(A), fw, -2, P(A + 8192), P(A + 4096), F32, None) == fq.EINVAL
    assert d(None, None, 0, None, None, F32, None) == fq.OK


def test_packed_errors():
    c = L.fp8q_cast_to_packed
    ws = P(A + 65536)
    assert c(P(A), BF16, -1, E5, P(A + 4096), ws, None) == fq.EINVAL
    assert c(P(A), BF16, 2 ** 63 - 2, E5, P(A + 4096), ws, None) == fq.EINVAL           # 4 + n overflows
    assert c(P(A), 9, 16, E5, P(A + 4096), ws, None) == fq.EDTYPE
    assert c(P(A), BF16, 16, 2, P(A + 4096), ws, None) == fq.EDTYPE
    assert c(P(A), BF16, 16, E5, None, ws, None) == fq.EINVAL
    assert c(P(A), BF16, 16, E5, P(A + 4096), None, None) == fq.EINVAL
    assert c(None, BF16, 16, E5, P(A + 4096), ws, None) == fq.EINVAL
    assert c(P(A), BF16, 16, E5, P(A + 4098), ws, None) == fq.EALIGN                    # slot not 4-aligned
    assert c(P(A), BF16, 16, E5, P(A + 16), ws, None) == fq.EINVAL                      # slot overlaps x
    assert c(P(A), BF16, 16, E5, P(A + 4096), P(A + 4100), None) == fq.EINVAL           # workspace in slot
    d = L.fp8q_dequant_packed
    assert d(P(A), E5, -1, 16, P(A + 8192), BF16, None) == fq.EINVAL
    assert d(P(A), E5, 2, -16, P(A + 8192), BF16, None) == fq.EINVAL
    assert d(P(A), E5, 2 ** 62, 2 ** 62, P(A + 8192), BF16, None) == fq.EINVAL          # overflow
    assert d(P(A), 3, 2, 16, P(A + 8192), BF16, None) == fq.EDTYPE
    assert d(P(A), E5, 2, 16, P(A + 8192), 4, None) == fq.EDTYPE
    assert d(P(A), E5, 2, 6, P(A + 8192), BF16, None) == fq.EALIGN                      # n % 4 with W > 1
    assert d(P(A + 2), E5, 1, 16, P(A + 8192), BF16, None) == fq.EALIGN
    assert d(P(A), E5, 1, 16, P(A + 8193), BF16, None) == fq.EALIGN
    assert d(None, E5, 2, 16, P(A + 8192), BF16, None) == fq.EINVAL
    assert d(P(A), E5, 2, 16, P(A + 20), BF16, None) == fq.EINVAL                       # y overlaps the slots
    assert d(None, E5, 0, 16, None, BF16, None) == fq.OK
    assert d(None, E5, 3, 0, None, BF16, None) == fq.OK


def test_reduce_step_errors():
    d = L.fp8q_dequant_sum
    #        q      fmt W  n   scale_inv       avg  y              ydt
    assert d(P(A), E5, 0, 16, P(A + 8192), 0, P(A + 4096), BF16, None) == fq.EINVAL      # W < 1
    assert d(P(A), E5, 2, -1, P(A + 8192), 0, P(A + 4096), BF16, None) == fq.EINVAL
    assert d(P(A), E5, 2 ** 62, 0, P(A + 8192), 0, P(A + 4096), BF16, None) == fq.EINVAL  # W * 4 overflows
    assert d(P(A), E5, 2 ** 40, 2 ** 40, P(A + 8192), 0, P(A + 4096), BF16, None) == fq.EINVAL
    assert d(P(A), 2, 2, 16, P(A + 8192), 0, P(A + 4096), BF16, None) == fq.EDTYPE
    assert d(P(A), E5, 2, 16, P(A + 8192), 0, P(A + 4096), 5, None) == fq.EDTYPE
    assert d(P(A), E5, 2, 16, None, 0, P(A + 4096), BF16, None) == fq.EINVAL
    assert d(P(A), E5, 2, 16, P(A + 8194), 0, P(A + 4096), BF16, None) == fq.EALIGN
    assert d(P(A), E5, 2, 16, P(A + 8192), 0, P(A + 4097), BF16, None) == fq.EALIGN
    assert d(P(A), E5, 2, 16, P(A + 8192), 0, P(A + 16), BF16, None) == fq.EINVAL        # y overlaps q
    assert d(P(A), E5, 2, 16, P(A + 4100), 0, P(A + 4096), BF16, None) == fq.EINVAL      # scale_inv in y
    assert d(None, E5, 3, 0, P(A + 8192), 0, None, BF16, None) == fq.OK
    r = L.fp8q_dequant_sum_requant
    ws = P(A + 65536)
    #        q      fmt W  n   scale_inv       avg  y              ydt   q_out           sinv_out        ws
    assert r(P(A), E5, 2, 16, P(A + 8192), 1, P(A + 4096), BF16, P(A + 12288), P(A + 16384), None, None) == fq.EINVAL
    assert r(P(A), E5, 2, 16, P(A + 8192), 1, P(A + 4096), BF16, P(A + 12288), None, ws, None) == fq.EINVAL
    assert r(P(A), E5, 2, 16, P(A + 8192), 1, P(A + 4096), BF16, None, P(A + 16384), ws, None) == fq.EINVAL
    assert r(P(A), E5, 2, 16, P(A + 8192), 1, P(A + 4096), BF16, P(A + 12288), P(A + 16386), ws, None) == fq.EALIGN
    assert r(P(A), E5, 2, 16, P(A + 8192), 1, P(A + 4096), BF16, P(A + 12288), P(A + 16384), P(A + 65537),
             None) == fq.EALIGN
    assert r(P(A), E5, 2, 16, P(A + 8192), 1, P(A + 4096), BF16, P(A + 12288), P(A + 16384), P(A + 4096),
             None) == fq.EINVAL                                                                   # workspace = y
    assert r(P(A), E5, 2, 16, P(A + 8192), 1, P(A + 4096), BF16, P(A + 4100), P(A + 16384), ws, None) == fq.EINVAL


def test_python_binding_rejects_host_tensors():
    import torch
    x = torch.zeros((2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fq.fp8q_cast_per_group128(x, torch.empty((2, 128), dtype=torch.uint8), torch.empty((2, 1)))
    with pytest.raises(TypeError):
        fq.cast_from_fp8(torch.zeros(4), torch.ones(1), torch.float32)


@pytest.mark.skipif(not STUBS, reason="needs the launcher-stub build of the ABI layer (run by test_sanitizers.py)")
def test_valid_calls_reach_the_launchers():
    """Valid arguments get past validation and reach exactly the launchers
    each entry point is documented to use; the no-op shapes reach none."""
    L.fp8q_stub_count.restype = ctypes.c_long
    L.fp8q_stub_count.argtypes = [ctypes.c_char_p]

    def calls(fn, *args):
        L.fp8q_stub_reset()
        assert fn(*args) == fq.OK, fn.__name__
        names = ("fill_f32", "amax", "amax_partials", "guard_amax", "cast_given_amax", "dequant_packed",
                 "pipeline_cast", "dequant_pipeline", "tensor_cast", "channel_cast", "group128_cast",
                 "dequant_flat", "dequant_rows", "block128", "dequant_sum", "scratch_words",
                 "group128_cast_wave64")
        return {k: L.fp8q_stub_count(k.encode()) for k in names if L.fp8q_stub_count(k.encode())}

    x, q, s, y, ws, w = P(A), P(A + (1 << 20)), P(A + (2 << 20)), P(A + (3 << 20)), P(A + (4 << 20)), P(A + (5 << 20))
    assert calls(L.fp8q_cast_per_group128, x, BF16, 4, 256, E4, q, s, None) == {"group128_cast": 1}
    assert calls(L.fp8q_cast_per_group128, None, BF16, 0, 256, E4, None, None, None) == {}
    assert calls(L.fp8q_cast_per_group128_wave64, P(A + 4), BF16, 4, 256, E4, P(A + (1 << 20) + 2), s, None) == \
        {"group128_cast_wave64": 1}
    assert calls(L.fp8q_cast_per_group128_wave64, None, BF16, 0, 256, E4, None, None, None) == {}
    assert calls(L.fp8q_cast_per_tensor, x, F32, 16, E5, q, s, ws, None) == {"amax_partials": 1, "tensor_cast": 1}
    assert calls(L.fp8q_cast_per_tensor, None, F32, 0, E5, None, s, ws, None) == {"fill_f32": 1}
    assert calls(L.fp8q_cast_per_tensor_noalloc, x, BF16, 16, E4, q, s, None) == \
        {"scratch_words": 1, "amax_partials": 1, "tensor_cast": 1}
    assert calls(L.fp8q_cast_per_tensor_noalloc, None, BF16, 0, E4, None, s, None) == {"fill_f32": 1}
    assert calls(L.fp8q_cast_per_channel, x, F16, 4, 16, E4, q, s, None) == {"channel_cast": 1}
    assert calls(L.fp8q_cast_per_channel, None, F16, 4, 0, E4, None, s, None) == {"fill_f32": 1}
    assert calls(L.fp8q_dequant_per_tensor, q, E4, 16, s, y, BF16, None) == {"dequant_flat": 1}
    assert calls(L.fp8q_dequant_per_channel, q, E4, 4, 16, s, y, F32, None) == {"dequant_rows": 1}
    assert calls(L.fp8q_dequant_per_group128, q, E5, 2, 256, s, y, F16, None) == {"dequant_flat": 1}
    assert calls(L.fp8q_weight_dequant_block128, q, E4, 300, 272, s, y, BF16, None) == {"block128": 1}
    assert calls(L.fp8q_weight_dequant_block128, None, E4, 0, 272, None, None, BF16, None) == {}
    assert calls(L.fp8q_amax, x, BF16, 0, s, None) == {"amax": 1}
    assert calls(L.fp8q_amax_guarded, x, BF16, 10, s, None) == {"amax": 1, "guard_amax": 1}
    assert calls(L.fp8q_cast_with_amax, None, BF16, 0, E5, w, None, s, None) == {"cast_given_amax": 1}
    assert calls(L.fp8q_dequant_div_scale, q, E5, 16, s, y, BF16, None) == {"dequant_flat": 1}
    assert calls(L.fp8q_cast_to_fp8_pipeline, None, BF16, 0, None, s, w, ws, None) == \
        {"amax_partials": 1, "pipeline_cast": 1}
    assert calls(L.fp8q_cast_from_fp8_pipeline, q, w, 16, s, y, F32, None) == {"dequant_pipeline": 1}
    assert calls(L.fp8q_cast_to_packed, x, BF16, 16, E5, q, ws, None) == {"amax_partials": 1, "tensor_cast": 1}
    assert calls(L.fp8q_cast_to_packed, None, BF16, 0, E5, q, ws, None) == {"fill_f32": 1}
    assert calls(L.fp8q_dequant_packed, q, E5, 3, 16, y, BF16, None) == {"dequant_packed": 1}
    assert calls(L.fp8q_dequant_sum, q, E5, 4, 64, s, 1, y, BF16, None) == {"dequant_sum": 1}
    assert calls(L.fp8q_dequant_sum_requant, q, E5, 4, 64, s, 1, y, BF16, w, P(A + (6 << 20)), ws, None) == \
        {"dequant_sum": 1, "tensor_cast": 1}
    assert calls(L.fp8q_dequant_sum_requant, None, E5, 4, 0, s, 1, None, BF16, None, w, ws, None) == \
        {"fill_f32": 1}


@pytest.mark.skipif(not STUBS, reason="needs the launcher-stub build of the ABI layer (run by test_sanitizers.py)")
def test_fuzz_validation():
    """Random calls of every entry point with sizes at and beyond the int64
    limits, NULL, odd and far-apart fake pointers, and out-of-range enum values.
    Every call must return one of the documented status codes; under the
    sanitizer build any undefined behaviour in the validation arithmetic aborts
    the process, and a call that reaches a launcher with a broken precondition
    aborts in the stub."""
    import numpy as np
    rng = np.random.Generator(np.random.PCG64(77))
    sizes = [0, 1, 2, 3, 7, 8, 127, 128, 129, 4096, 2 ** 31 - 1, 2 ** 31, 2 ** 32 + 1, 2 ** 40, 2 ** 62,
             2 ** 63 - 1, -1, -2, -(2 ** 63)]
    ptrs = [None, A, A + 1, A + 2, A + 4, A + 8, A + 16, A + 4096, A + (1 << 20), A + (1 << 40),
            2 ** 64 - 4096, 4]
    enums = [0, 1, 2, 3, -1, 7, 2 ** 31 - 1, -(2 ** 31)]
    codes = {fq.OK, fq.EINVAL, fq.EDTYPE, fq.ESHAPE, fq.EALIGN, fq.EHIP}
    for name in fq.ABI_FUNCTIONS:
        fn = getattr(L, name)
        if name in ("fp8q_abi_version", "fp8q_status_str", "fp8q_per_tensor_workspace_bytes"):
            continue
        for _ in range(1000):
            args = []
            for t in fn.argtypes:
                if t is ctypes.c_void_p:
                    p = ptrs[int(rng.integers(0, len(ptrs)))]
                    args.append(None if p is None else P(p))
                elif t is ctypes.c_int64:
                    args.append(sizes[int(rng.integers(0, len(sizes)))] if rng.random() < 0.8
                                else int(rng.integers(0, 1 << 20)))
                else:
                    args.append(enums[int(rng.integers(0, len(enums)))] if rng.random() < 0.5
                                else int(rng.integers(0, 3)))
            args[-1] = None                                  # the stream
            assert fn(*args) in codes, (name, args)
