"""GPU parity of the UE5M3 block scale (reading: 5 exponent bits, bias 15,
3 mantissa bits, 0xFF NaN) against the oracle, bit for bit: every strategy
and block size with no and with a caller's per-tensor scale, quotients on
every rounding boundary at every code, special values, caller-given codes,
bf16 with rotation, stand-alone dequantize / block MSE, FOCUS forward and
backward, and the full 4096 x 4096 workload on sampled rows."""
import functools

import numpy as np
import pytest
import torch

from microscaling_fp4_block_fp4q_amd import fp4q as F
from microscaling_fp4_block_fp4q_amd import synth as S
from oracle import oracle as O

from gpu_helpers import DEV, TORCH_DT, assert_same, compare_quant, gpu_quantize, note, oracle_quantize, sample_rows

pytestmark = pytest.mark.gpu

UE = F.UE5M3
NAMES = {F.ABSMAX: "absmax", F.PREVENT_ZERO: "prevent-zero", F.FOUR_OVER_SIX: "4-over-6",
         F.BRUTE_FORCE: "brute-force"}


def small(kind, rows, cols=4000):
    base = S.normal(rows, cols, 1) if kind.startswith("normal") else S.laplace(rows, cols, 2)
    return S.scaled_fp32(base, 1e-4) if kind.endswith("1e-4") else base


@pytest.mark.parametrize("kind", ["normal", "laplace", "normal_1e-4", "laplace_1e-4"])
@pytest.mark.parametrize("B", [4, 8, 16, 32])
@pytest.mark.parametrize("strategy", [F.ABSMAX, F.PREVENT_ZERO, F.FOUR_OVER_SIX, F.BRUTE_FORCE])
@pytest.mark.parametrize("gm,g", [(F.GLOBAL_NONE, 1.0), (F.GLOBAL_USER, 0.37)])
def test_ue5m3_sweep(O_lib, kind, B, strategy, gm, g):
    x = small(kind, 9 if strategy == F.BRUTE_FORCE else 37)
    cfg = F.config(UE, B, strategy, gm, g)
    note(f"ue5m3 {kind} B={B} {NAMES[strategy]} gm={gm}")
    gpu = gpu_quantize(x, S.F32, cfg)
    ref = oracle_quantize(x, S.F32, cfg)
    compare_quant(gpu, ref)


def boundary_rows():
    """Row c: fl(m S_c) and its fp32 neighbours for every E2M1 rounding
    boundary m, then 6 S_c and its upper neighbour, for UE5M3 code c."""
    bounds = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    x = np.zeros((255, 32), np.float32)
    for c in range(1, 255):
        Sc = np.float32(O.ue5m3_decode(c))
        vals = []
        for m in bounds:
            v = np.float32(m * Sc)
            vals += [np.nextafter(v, np.float32(0)), v, np.nextafter(v, np.float32(np.inf))]
        six = np.float32(6 * Sc)
        vals += [six, np.nextafter(six, np.float32(np.inf)), np.float32(0)]
        row = np.array(vals, np.float32)
        row[1::2] *= -1
        x[c, :24] = row
    return x


@pytest.mark.parametrize("B", [8, 32])
def test_quotients_on_rounding_boundaries(O_lib, B):
    x = boundary_rows()
    scales = np.repeat(np.arange(255, dtype=np.uint8)[:, None], 32 // B, axis=1)
    cfg = F.config(UE, B, F.GIVEN)
    note(f"ue5m3 rounding-boundary quotients B={B}")
    gpu = gpu_quantize(x, S.F32, cfg, scales_in=scales)
    ref = oracle_quantize(x, S.F32, cfg, scales_in=scales)
    compare_quant(gpu, ref)
    for st in (F.ABSMAX, F.FOUR_OVER_SIX, F.BRUTE_FORCE):
        cfg = F.config(UE, B, st)
        note(f"ue5m3 rounding-boundary rows {NAMES[st]} B={B}")
        compare_quant(gpu_quantize(x, S.F32, cfg), oracle_quantize(x, S.F32, cfg))


def special_tensor():
    rng = np.random.default_rng(17)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    x[0, :32] = 0.0
    x[0, 5] = -0.0
    x[1, :32] = rng.standard_normal(32).astype(np.float32) * np.float32(1e-40)
    x[2, :32] = np.float32(3.0e38) * np.sign(rng.standard_normal(32)).astype(np.float32)
    x[3, :16] = np.float32(2.0 ** -20) * np.arange(16, dtype=np.float32)
    x[4, :] *= np.float32(1e5)                                   # past the largest scale 114688 * 6
    x[6, 3] = np.nan
    x[6, 37] = np.inf
    x[7, 70] = -np.inf
    return x


@pytest.mark.parametrize("strategy", [F.ABSMAX, F.FOUR_OVER_SIX, F.BRUTE_FORCE])
def test_special_values(O_lib, strategy):
    x = special_tensor()
    cfg = F.config(UE, 16, strategy)
    note(f"ue5m3 special values {NAMES[strategy]}")
    compare_quant(gpu_quantize(x, S.F32, cfg), oracle_quantize(x, S.F32, cfg))


def test_given_codes_full_byte(O_lib):
    x = special_tensor()
    scales = np.random.default_rng(3).integers(0, 256, (8, 128 // 16)).astype(np.uint8)
    scales[0, 0] = 0xFF
    scales[1, 1] = 0x80
    cfg = F.config(UE, 16, F.GIVEN, F.GLOBAL_USER, 0.5)
    note("ue5m3 given codes")
    compare_quant(gpu_quantize(x, S.F32, cfg, scales_in=scales), oracle_quantize(x, S.F32, cfg, scales_in=scales))


@pytest.mark.parametrize("H", [16, 32])
def test_bf16_rotated(O_lib, H):
    x = S.cast(S.laplace(40, 2048, 5), S.BF16)
    cfg = F.config(UE, 16, F.FOUR_OVER_SIX, F.GLOBAL_NONE, 1.0, H)
    note(f"ue5m3 bf16 H={H}")
    compare_quant(gpu_quantize(x, S.BF16, cfg, dq_dt=S.BF16), oracle_quantize(x, S.BF16, cfg, dq_dt=S.BF16))


@pytest.mark.parametrize("out_dt", [S.F32, S.BF16])
def test_dequantize_and_block_mse(O_lib, out_dt):
    x = S.laplace(45, 1024, 9)
    g = np.float32(0.75)
    ref = O.quantize(x, fmt=UE, block=16, strategy=F.FOUR_OVER_SIX, global_mode=F.GLOBAL_USER, user_g=g,
                     dq_dt=out_dt)
    cfg = F.config(UE, 16, F.ABSMAX, F.GLOBAL_USER, float(g))
    note(f"ue5m3 dequantize/block_mse out={out_dt}")
    codes = torch.from_numpy(ref["codes"]).to(DEV)
    scales = torch.from_numpy(ref["scales"]).to(DEV)
    gt = torch.tensor([g], dtype=torch.float32, device=DEV)
    dq = F.dequantize(codes, scales, cfg, g=gt, out_dtype=TORCH_DT[out_dt])
    mse = F.block_mse(S.to_torch(x, S.F32, DEV), codes, scales, cfg, g=gt)
    torch.cuda.synchronize()
    assert_same(S.from_torch(dq), ref["dequant"], "dequant")
    assert_same(S.from_torch(mse), ref["mse"], "mse")


@pytest.mark.parametrize("K", [4, 8])
def test_focus(O_lib, K):
    w, c, grad = S.focus_inputs(33, 1024, K, seeds=(6, 7, 8))
    cfg = F.config(UE, 16, F.ABSMAX)
    q = O.quantize(w, x_dt=S.BF16, fmt=UE, block=16, strategy=F.ABSMAX, dq_dt=None)
    note(f"ue5m3 focus K={K}")
    wt, ct, gt = S.to_torch(w, S.BF16, DEV), S.to_torch(c, S.F16, DEV), S.to_torch(grad, S.BF16, DEV)
    st = torch.from_numpy(q["scales"]).to(DEV)
    wh, codes = F.relaxed_fakequant_fwd(wt, st, ct, cfg, sub_block=K, want_codes=True)
    gc = F.relaxed_fakequant_bwd(wt, st, ct, gt, cfg, sub_block=K)
    torch.cuda.synchronize()
    rw, rc = O.relaxed_fwd(w, q["scales"], 1.0, c, fmt=UE, block=16, sub_block=K, w_dt=S.BF16)
    rg = O.relaxed_bwd(w, q["scales"], 1.0, c, grad, fmt=UE, block=16, sub_block=K, w_dt=S.BF16, g_dt=S.BF16)
    assert_same(S.from_torch(wh), rw, "w_hat")
    assert_same(S.from_torch(codes), rc, "codes")
    assert_same(S.from_torch(gc), rg, "grad_c")


@functools.lru_cache(maxsize=1)
def full_c2():
    return S.config2()


@pytest.mark.parametrize("strategy", [F.ABSMAX, F.FOUR_OVER_SIX, F.BRUTE_FORCE])
def test_full_size_sampled(O_lib, strategy):
    full = full_c2()["normal"]
    rows = sample_rows(full.shape[0], seed=11)
    for B in (16, 4):
        cfg = F.config(UE, B, strategy)
        note(f"ue5m3 full 4096x4096 B={B} {NAMES[strategy]}")
        gpu = gpu_quantize(full, S.F32, cfg)
        compare_quant(gpu, oracle_quantize(full[rows], S.F32, cfg), rows)
