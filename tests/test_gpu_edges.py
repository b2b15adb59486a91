"""GPU edge cases against the oracle: empty tensors, ragged tails, row
strides, special values (NaN, inf, signed zero, subnormals, values near the
fp32 maximum, exactly representable blocks), fp16 input, determinism."""
import numpy as np
import pytest
import torch

from microscaling_fp4_block_fp4q_amd import fp4q as F
from microscaling_fp4_block_fp4q_amd import synth as S
from oracle import oracle as O

from gpu_helpers import DEV, TORCH_DT, assert_same, compare_quant, gpu_quantize, note, oracle_quantize

pytestmark = pytest.mark.gpu

E8M0, E4M3 = F.E8M0, F.E4M3
ALL_CFGS = [
    ("e4m3-absmax-none", F.config(E4M3, 16, F.ABSMAX)),
    ("e4m3-pz-none", F.config(E4M3, 8, F.PREVENT_ZERO)),
    ("e4m3-4o6-amax", F.config(E4M3, 16, F.FOUR_OVER_SIX, F.GLOBAL_TENSOR_AMAX)),
    ("e4m3-bf-none", F.config(E4M3, 4, F.BRUTE_FORCE)),
    ("e4m3-bf-user", F.config(E4M3, 32, F.BRUTE_FORCE, F.GLOBAL_USER, 3.0e-3)),
    ("e8m0-absmax", F.config(E8M0, 32, F.ABSMAX)),
    ("e8m0-bf", F.config(E8M0, 16, F.BRUTE_FORCE)),
]


def special_tensor(with_nonfinite=True):
    rng = np.random.default_rng(99)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    x[0, :32] = 0.0
    x[0, 5] = -0.0
    x[1, :32] = rng.standard_normal(32).astype(np.float32) * np.float32(1e-40)   # subnormals
    x[2, :32] = np.float32(3.0e38) * np.sign(rng.standard_normal(32)).astype(np.float32)
    x[2, 40] = np.float32(3.4028235e38)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    x[3, :32] = grid[rng.integers(0, 8, 32)] * np.float32(0.0546875)          # exact grid * E4M3 value
    x[3, 0] = np.float32(6 * 0.0546875)
    x[4, :] = np.float32(1e-4) * x[4, :]
    x[5, :16] = np.float32(2.0 ** -20) * np.arange(16, dtype=np.float32)
    if with_nonfinite:
        x[6, 3] = np.nan
        x[6, 37] = np.inf
        x[7, 70] = -np.inf
    return x


@pytest.mark.parametrize("name,cfg", ALL_CFGS)
@pytest.mark.parametrize("nonfinite", [False, True])
def test_special_values(O_lib, name, cfg, nonfinite):
    x = special_tensor(nonfinite)
    note(f"special values {name} nonfinite={nonfinite}")
    gpu = gpu_quantize(x, S.F32, cfg)
    ref = oracle_quantize(x, S.F32, cfg)
    assert gpu["g"].view(np.uint32) == ref["g"].view(np.uint32)
    compare_quant(gpu, ref)


@pytest.mark.parametrize("name,cfg", ALL_CFGS[:3] + ALL_CFGS[5:6])
def test_given_scales_with_nonfinite_elements(O_lib, name, cfg):
    x = special_tensor(True)
    scales = np.random.default_rng(1).integers(0, 0x80, (8, 128 // cfg.block)).astype(np.uint8)
    scales[0, 0] = 0x7F if cfg.scale_fmt == E4M3 else 0xFF
    given = F.config(cfg.scale_fmt, cfg.block, F.GIVEN, F.GLOBAL_NONE)
    note(f"given scales with non-finite elements {name}")
    gpu = gpu_quantize(x, S.F32, given, scales_in=scales)
    ref = oracle_quantize(x, S.F32, given, scales_in=scales)
    compare_quant(gpu, ref)


@pytest.mark.parametrize("rows,cols", [(0, 64), (5, 0)])
def test_empty_tensors(O_lib, rows, cols):
    note(f"empty {rows}x{cols}")
    x = torch.zeros((rows, cols), dtype=torch.float32, device=DEV)
    r = F.quantize(x, F.nvfp4(), dequant_dtype=torch.float32)
    torch.cuda.synchronize()
    assert r["codes"].numel() == 0 and r["g"].item() == 1.0
    r = F.quantize(x, F.nvfp4(global_mode=F.GLOBAL_USER, global_scale=0.5))
    torch.cuda.synchronize()
    assert r["g"].item() == 0.5


@pytest.mark.parametrize("rows,cols,B,dt", [(1, 16, 16, S.F32), (3, 32, 32, S.BF16), (257, 48, 16, S.F32),
                                            (2, 8, 4, S.BF16), (513, 8, 8, S.F16), (1, 4, 4, S.F32)])
def test_tiny_and_ragged(O_lib, rows, cols, B, dt):
    x = S.laplace(rows, cols, rows + cols, dt)
    for st in (F.ABSMAX, F.FOUR_OVER_SIX, F.BRUTE_FORCE):
        cfg = F.config(E4M3, B, st, F.GLOBAL_TENSOR_AMAX)
        note(f"tiny {rows}x{cols} B={B} dt={dt} st={st}")
        gpu = gpu_quantize(x, dt, cfg, dq_dt=dt)
        ref = oracle_quantize(x, dt, cfg, dq_dt=dt)
        assert gpu["g"].view(np.uint32) == ref["g"].view(np.uint32)
        compare_quant(gpu, ref)


def test_row_stride(O_lib):
    """x and dequant as column slices of wider tensors (ld > cols)."""
    big = S.laplace(50, 1024 + 64, 31)
    x = big[:, :1024]
    cfg = F.nvfp4(F.FOUR_OVER_SIX, hadamard=32)
    note("row stride")
    xt = S.to_torch(big, S.F32, DEV)[:, :1024]
    codes = torch.empty((50, 512), dtype=torch.uint8, device=DEV)
    scales = torch.empty((50, 64), dtype=torch.uint8, device=DEV)
    g = torch.empty(1, dtype=torch.float32, device=DEV)
    dq_big = torch.zeros((50, 1024 + 128), dtype=torch.bfloat16, device=DEV)
    dq = dq_big[:, :1024]
    mse = torch.empty((50, 64), dtype=torch.float32, device=DEV)
    ws = torch.empty(F.workspace_bytes(cfg, 50, 1024), dtype=torch.uint8, device=DEV)
    F.fp4q_quantize(cfg, xt, codes, scales, g, dq, mse, ws)
    torch.cuda.synchronize()
    ref = oracle_quantize(np.ascontiguousarray(x), S.F32, cfg, dq_dt=S.BF16)
    assert_same(S.from_torch(codes), ref["codes"], "codes")
    assert_same(S.from_torch(scales), ref["scales"], "scales")
    assert_same(S.from_torch(dq), ref["dequant"], "dequant")
    assert_same(S.from_torch(mse), ref["mse"], "mse")
    assert torch.all(dq_big[:, 1024:] == 0)           # nothing written past cols


@pytest.mark.parametrize("out_dt", [S.F32, S.F16])
def test_fp16_input(O_lib, out_dt):
    x = S.activations(40, 2048, 12, S.F16)
    for cfg in (F.nvfp4(F.FOUR_OVER_SIX, hadamard=16), F.mxfp4(), F.config(E4M3, 8, F.BRUTE_FORCE)):
        note(f"fp16 input fmt={cfg.scale_fmt} st={cfg.strategy} out={out_dt}")
        gpu = gpu_quantize(x, S.F16, cfg, dq_dt=out_dt)
        ref = oracle_quantize(x, S.F16, cfg, dq_dt=out_dt)
        compare_quant(gpu, ref)


def test_deterministic_across_runs(O_lib):
    x = S.laplace(300, 4096, 41)
    for cfg in (F.nvfp4(F.FOUR_OVER_SIX), F.config(E4M3, 8, F.BRUTE_FORCE, F.GLOBAL_TENSOR_AMAX)):
        note(f"determinism st={cfg.strategy}")
        a = gpu_quantize(x, S.F32, cfg)
        b = gpu_quantize(x, S.F32, cfg)
        for k in ("codes", "scales", "dequant", "mse"):
            assert_same(a[k], b[k], k)


def boundary_tensor(g):
    """Row c holds, for E4M3 code c (S = fl(dec(c) g)), the elements
    fl(m S) and its two fp32 neighbours for every E2M1 rounding boundary m
    (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5), then m = 6 (the largest grid value),
    with alternating signs; 24 values, padded with zeros to 32."""
    dec = np.array([O.e4m3_decode(c) for c in range(127)], np.float64)
    bounds = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    x = np.zeros((127, 32), np.float32)
    for c in range(1, 127):
        S = np.float32(np.float32(dec[c]) * np.float32(g))
        vals = []
        for m in bounds[:7]:
            v = np.float32(m * S)
            vals += [np.nextafter(v, np.float32(0)), v, np.nextafter(v, np.float32(np.inf))]
        vals += [np.float32(6 * S), np.nextafter(np.float32(6 * S), np.float32(np.inf)), np.float32(0)]
        row = np.array(vals, np.float32)
        row[1::2] *= -1
        x[c, :24] = row
    return x


@pytest.mark.parametrize("g", [1.0, 0.3, 2.0 ** -20])
@pytest.mark.parametrize("B", [8, 16, 32])
def test_quotients_on_rounding_boundaries(O_lib, g, B):
    """Caller-given scales: row c is encoded at code c, so every quotient lies
    on, or one ulp off, an E2M1 rounding boundary (ties and their neighbours)."""
    x = boundary_tensor(g)
    scales = np.repeat(np.arange(127, dtype=np.uint8)[:, None], 32 // B, axis=1)
    cfg = F.config(E4M3, B, F.GIVEN, F.GLOBAL_USER, g)
    note(f"rounding-boundary quotients g={g} B={B}")
    gpu = gpu_quantize(x, S.F32, cfg, scales_in=scales)
    ref = oracle_quantize(x, S.F32, cfg, scales_in=scales)
    compare_quant(gpu, ref)


@pytest.mark.parametrize("strategy", [F.ABSMAX, F.PREVENT_ZERO, F.FOUR_OVER_SIX, F.BRUTE_FORCE])
def test_boundary_blocks_every_strategy(O_lib, strategy):
    """The same boundary rows with the scale chosen by each strategy."""
    x = boundary_tensor(0.3)
    cfg = F.config(E4M3, 8, strategy, F.GLOBAL_TENSOR_AMAX)
    note(f"rounding-boundary blocks strategy={strategy}")
    gpu = gpu_quantize(x, S.F32, cfg)
    ref = oracle_quantize(x, S.F32, cfg)
    assert gpu["g"].view(np.uint32) == ref["g"].view(np.uint32)
    compare_quant(gpu, ref)


@pytest.mark.parametrize("g,xs", [(2.0 ** -110, 50.0 * 2.0 ** -110), (2.0 ** -120, 50.0 * 2.0 ** -120),
                                  (1.0e33, 5.0e34), (2.0 ** -95, 2.0 ** -22)])
@pytest.mark.parametrize("B", [4, 16])
def test_brute_force_extreme_global_scale(O_lib, g, xs, B):
    """User scales that put block scales outside the division-free range
    (below 2^-100, fp32 subnormals at 2^-120, or above 2^100): brute force
    takes the IEEE division for every candidate.  In fp32 such scales leave
    every code with the same SSE: with values near the scales the squared
    errors underflow to 0 or overflow to inf, and values of 2^-22 against
    g = 2^-95 saturate at a dequantized value below half an ulp of the
    value, which the difference absorbs.  The smallest code wins; the test
    checks that the division path reaches the oracle's ties and outputs."""
    x = (S.laplace(9, 512, 31) * np.float32(xs)).astype(np.float32)
    cfg = F.config(E4M3, B, F.BRUTE_FORCE, F.GLOBAL_USER, g)
    note(f"brute force with g={g} x scale={xs} B={B}")
    gpu = gpu_quantize(x, S.F32, cfg)
    ref = oracle_quantize(x, S.F32, cfg)
    compare_quant(gpu, ref)


@pytest.mark.parametrize("g,xs", [(2.0 ** -110, 2.0 ** -104), (2.0 ** -63, 2.0 ** -57), (2.0 ** -62, 2.0 ** -56),
                                  (2.0 ** 57, 2.0 ** 63), (2.0 ** 59, 2.0 ** 65), (1.0e33, 5.0e34)])
@pytest.mark.parametrize("strategy", [F.ABSMAX, F.PREVENT_ZERO, F.FOUR_OVER_SIX])
@pytest.mark.parametrize("B", [4, 16, 32])
def test_streaming_extreme_global_scale(O_lib, g, xs, strategy, B):
    """User scales on both sides of the range that the branch-free trips
    need (fl(6 g) and fl(4 g) in [2^-60, 2^60], every table scale
    fl(dec(c) g) in [2^-100, 2^100]): g = 2^-62 and 2^57 take the
    branch-free trips, 2^-63, 2^59, 2^-110 and 1e33 the chunk-by-chunk path
    (with the IEEE division where a quotient leaves its range).  Values near
    g times mid-range codes, with a NaN, infinities and a zero block in whole
    trips (64 rows of 512 values)."""
    x = (S.laplace(64, 512, 41) * np.float32(xs)).astype(np.float32)
    x[3, 17] = np.nan
    x[40, 200] = np.inf
    x[63, 511] = -np.inf
    x[10, :16] = 0.0
    cfg = F.config(E4M3, B, strategy, F.GLOBAL_USER, g)
    note(f"streaming strategy={strategy} B={B} g={g} x scale={xs}")
    gpu = gpu_quantize(x, S.F32, cfg)
    ref = oracle_quantize(x, S.F32, cfg)
    compare_quant(gpu, ref)
