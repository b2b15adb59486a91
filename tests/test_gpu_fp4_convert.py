"""The gfx950 pair converts fp32 -> FP4 (E2M1) and FP4 -> fp32, which the
streaming quantizer uses for the element rounding, against the library's
arithmetic rounding (half-to-even onto {0, 0.5, ..., 6}, saturating at 6,
the sign kept on zero), on every non-NaN fp32 bit pattern.  That arithmetic
rounding is itself pinned to the oracle by every parity test."""
import ctypes
import os

import pytest
import torch

from gpu_helpers import DEV, note

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "microscaling_fp4_block_fp4q_amd", "libfp4q_probe.so")


def test_hardware_fp4_convert_matches_on_every_pattern():
    lib = ctypes.CDLL(PROBE)
    lib.fp4q_probe_fp4_convert.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.fp4q_probe_fp4_convert.restype = ctypes.c_int
    counts = torch.zeros(3, dtype=torch.int64, device=DEV)
    note("hardware FP4 convert, 2^32 patterns")
    assert lib.fp4q_probe_fp4_convert(ctypes.c_void_p(counts.data_ptr()),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    bad_code, bad_value, checked = counts.tolist()
    assert checked == (1 << 32) - 2 * ((1 << 23) - 1)          # every pattern but the NaNs
    assert bad_code == 0, f"{bad_code} nibbles differ"
    assert bad_value == 0, f"{bad_value} decoded values differ"


def test_scaled_fp4_converts_with_power_of_two_scales_are_exact():
    """The scaled FP4 -> bf16 / fp16 converts the NVFP4 GEMM dequantizes its
    operands with: every byte at every position of its dword, times the
    power-of-two part of every E4M3 block scale, equals the exact product
    (the values; fp16 zeros may carry either sign).
    Given a scale that is not a power of two they apply only its exponent
    (so the GEMM multiplies the scale's mantissa in afterwards); that case
    is counted and must differ for most scales."""
    lib = ctypes.CDLL(PROBE)
    lib.fp4q_probe_fp4_scaled_convert.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.fp4q_probe_fp4_scaled_convert.restype = ctypes.c_int
    counts = torch.zeros(8, dtype=torch.int64, device=DEV)
    note("scaled FP4 -> bf16 / fp16 converts, 127 scales x 256 bytes x 4 positions")
    assert lib.fp4q_probe_fp4_scaled_convert(ctypes.c_void_p(counts.data_ptr()),
                                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    c = counts.tolist()
    assert c[4] == 127 * 256 * 4 * 2
    assert c[0] == 0 and c[2] == 0, f"value mismatches bf16 {c[0]} f16 {c[2]}"
    # bf16 keeps the sign of zero; fp16 may not (the GEMM adds zeros to a +0
    # accumulator, where that sign is lost anyway)
    assert c[1] == 0, f"bf16 bit mismatches {c[1]}"
    assert c[5] > c[4] // 2, "a full E4M3 scale value was applied as a product"
