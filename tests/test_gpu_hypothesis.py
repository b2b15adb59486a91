"""Property-based GPU parity (hypothesis): tiny tensors of one to a few
blocks per row, drawn as mixtures of the values that decide the encoding —
zeros of both signs, subnormals, NaN, infinities, exact E2M1 grid points
times powers of two, values next to the rounding boundaries, huge values and
plain random floats — under drawn configurations (scale format, block,
strategy, per-tensor scale mode, rotation, input type, caller-given scales).
Every draw is compared with the oracle element by element (codes, scales, g,
dequantized values, block MSE).  Generation is derandomised, so a run is
reproducible and each case prints its configuration before touching the
GPU."""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from microscaling_fp4_block_fp4q_amd import fp4q as F
from microscaling_fp4_block_fp4q_amd import synth as S

from gpu_helpers import assert_same, gpu_quantize, note, oracle_quantize

pytestmark = pytest.mark.gpu

GRID = [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
BOUNDS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


def _value():
    pw = st.integers(-30, 30).map(lambda k: 2.0 ** k)
    return st.one_of(
        st.sampled_from([0.0, -0.0, float("nan"), float("inf"), -float("inf"), 1e-40, -1e-42, 3.0e38]),
        st.tuples(st.sampled_from(GRID), pw, st.sampled_from([1.0, -1.0])).map(lambda t: t[0] * t[1] * t[2]),
        st.tuples(st.sampled_from(BOUNDS), pw, st.integers(-2, 2)).map(
            lambda t: t[0] * t[1] * (1.0 + t[2] * 2.0 ** -23)),
        st.floats(min_value=-1e6, max_value=1e6, allow_nan=False, width=32),
        st.floats(allow_nan=True, allow_infinity=True, width=32),
    )


@st.composite
def _case(draw):
    fmt = draw(st.sampled_from([F.E8M0, F.E4M3, F.UE5M3]))
    B = draw(st.sampled_from([4, 8, 16, 32]))
    H = draw(st.sampled_from([0, 16, 32]))
    dt = draw(st.sampled_from([S.F32, S.BF16, S.F16]))
    strategies = [F.ABSMAX, F.PREVENT_ZERO, F.BRUTE_FORCE, F.GIVEN] + ([F.FOUR_OVER_SIX] if fmt != F.E8M0 else [])
    strategy = draw(st.sampled_from(strategies))
    if fmt == F.E8M0:
        modes = [F.GLOBAL_NONE]
    elif fmt == F.UE5M3:
        modes = [F.GLOBAL_NONE, F.GLOBAL_USER]
    else:
        modes = [F.GLOBAL_NONE, F.GLOBAL_TENSOR_AMAX, F.GLOBAL_USER]
        if strategy != F.GIVEN:
            modes.append(F.GLOBAL_SEARCH)
    gm = draw(st.sampled_from(modes))
    user_g = draw(st.sampled_from([2.0 ** -20, 0.3, 1.0, 37.5]))
    rows = draw(st.integers(1, 3))
    unit = max(B, H, 8)                    # whole blocks and segments, 16-byte rows for every input type
    cols = unit * draw(st.integers(1, 3))
    vals = draw(st.lists(_value(), min_size=rows * cols, max_size=rows * cols))
    scales = draw(st.lists(st.integers(0, 255), min_size=rows * cols // B, max_size=rows * cols // B))
    return fmt, B, H, dt, strategy, gm, user_g, rows, cols, vals, scales


@settings(max_examples=400, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(_case())
def test_tiny_tensors_match_oracle(O_lib, case):
    fmt, B, H, dt, strategy, gm, user_g, rows, cols, vals, scales = case
    cfg = F.config(fmt, B, strategy, gm, global_scale=user_g, hadamard=H)
    x64 = np.array(vals, dtype=np.float64).reshape(rows, cols)
    with np.errstate(over="ignore", invalid="ignore"):
        x = S.cast(x64, dt)
    sc = np.array(scales, dtype=np.uint8).reshape(rows, cols // B) if strategy == F.GIVEN else None
    note(f"hypothesis fmt={fmt} B={B} H={H} dt={dt} strategy={strategy} gm={gm} g={user_g} {rows}x{cols}")
    gpu = gpu_quantize(x, dt, cfg, scales_in=sc)
    ref = oracle_quantize(x, dt, cfg, scales_in=sc)
    assert_same(gpu["g"], ref["g"], "g")
    for k in ("codes", "scales", "dequant", "mse"):
        assert_same(gpu[k], ref[k], k)
