"""GPU parity: the HIP library (through its C ABI) against the CPU oracle,
element by element, on seeded synthetic inputs shaped like the pages'
workloads.  Codes, scales, g, dequantized values, block MSE and FOCUS
gradients must be bit-identical (the spec fixes the fp32 operation order).

Sizes: reduced tensors with the workloads' recipes that the oracle finishes
in seconds (several tiles of 256 lanes plus a ragged tail), and the full
workload sizes with the oracle evaluated on a sample of rows (the global
scale of the full tensor comes from the oracle too).
"""
import functools

import numpy as np
import pytest
import torch

from microscaling_fp4_block_fp4q_amd import fp4q as F
from microscaling_fp4_block_fp4q_amd import synth as S
from oracle import oracle as O

from gpu_helpers import (DEV, TORCH_DT, assert_same, compare_quant, gpu_quantize, note, oracle_quantize,
                         sample_rows)

pytestmark = pytest.mark.gpu

E8M0, E4M3 = F.E8M0, F.E4M3
ABSMAX, PZ, FOS, BF, GIVEN = F.ABSMAX, F.PREVENT_ZERO, F.FOUR_OVER_SIX, F.BRUTE_FORCE, F.GIVEN
NONE, TAMAX, USER = F.GLOBAL_NONE, F.GLOBAL_TENSOR_AMAX, F.GLOBAL_USER
STRAT_NAMES = {ABSMAX: "absmax", PZ: "prevent-zero", FOS: "4-over-6", BF: "brute-force"}


# --------------------------------------------------------------------------
# fp32 1024 x 1024 N(0,1): MXFP4 and NVFP4 abs-max, every output, full size
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name,cfg", [("mxfp4", F.mxfp4()), ("nvfp4", F.nvfp4())])
def test_fp32_1024_full(O_lib, name, cfg):
    note(f"fp32 1024x1024 {name}")
    x = S.config1()
    gpu = gpu_quantize(x, S.F32, cfg)
    ref = oracle_quantize(x, S.F32, cfg)
    assert gpu["g"].view(np.uint32) == ref["g"].view(np.uint32)
    compare_quant(gpu, ref)


# --------------------------------------------------------------------------
# block-size sweep with every strategy, hierarchical on and off, reduced size
# (37 x 4000: 4000 is a multiple of 32, rows * units is not a multiple of 256)
# --------------------------------------------------------------------------

KINDS = ["normal", "laplace", "normal_1e-4", "laplace_1e-4"]


@functools.lru_cache(maxsize=1)
def full_c2():
    return S.config2()


@functools.lru_cache(maxsize=1)
def full_c3():
    return S.config3()


def small_c2(kind, rows=37, cols=4000):
    base = S.normal(rows, cols, 1) if kind.startswith("normal") else S.laplace(rows, cols, 2)
    return S.scaled_fp32(base, 1e-4) if kind.endswith("1e-4") else base


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("B", [4, 8, 16, 32])
@pytest.mark.parametrize("strategy", [ABSMAX, PZ, FOS, BF])
@pytest.mark.parametrize("gm", [TAMAX, NONE])
def test_block_sweep_small(O_lib, kind, B, strategy, gm):
    rows = 9 if strategy == BF else 37
    x = small_c2(kind, rows)
    cfg = F.config(E4M3, B, strategy, gm)
    note(f"sweep {kind} B={B} {STRAT_NAMES[strategy]} gm={gm} shape={x.shape}")
    gpu = gpu_quantize(x, S.F32, cfg)
    ref = oracle_quantize(x, S.F32, cfg)
    assert gpu["g"].view(np.uint32) == ref["g"].view(np.uint32)
    compare_quant(gpu, ref)


@pytest.mark.parametrize("strategy", [ABSMAX, BF])
@pytest.mark.parametrize("B", [4, 8, 16, 32])
def test_e8m0_block_sizes(O_lib, strategy, B):
    x = small_c2("laplace", 9 if strategy == BF else 37)
    cfg = F.config(E8M0, B, strategy)
    note(f"e8m0 B={B} {STRAT_NAMES[strategy]}")
    compare_quant(gpu_quantize(x, S.F32, cfg), oracle_quantize(x, S.F32, cfg))


@pytest.mark.parametrize("fmt,B,gm", [(E4M3, 4, NONE), (E4M3, 4, TAMAX), (E4M3, 8, NONE), (E4M3, 8, TAMAX),
                                      (E4M3, 16, NONE), (E4M3, 16, TAMAX), (E4M3, 32, NONE), (E4M3, 32, TAMAX),
                                      (E8M0, 16, NONE), (E8M0, 32, NONE), (F.UE5M3, 16, NONE)])
@pytest.mark.parametrize("kind", ["normal", "laplace"])
def test_brute_force_many_blocks(O_lib, fmt, B, gm, kind):
    """Brute force on 64 x 4096 values (8192 to 65536 blocks per case), every
    block against the oracle's exhaustive search: the branch-and-bound
    windows must never cut off the argmin."""
    x = S.normal(64, 4096, 21) if kind == "normal" else S.laplace(64, 4096, 22)
    cfg = F.config(fmt, B, BF, gm)
    note(f"brute force many blocks fmt={fmt} B={B} gm={gm} {kind}")
    gpu = gpu_quantize(x, S.F32, cfg, dq_dt=None)
    ref = oracle_quantize(x, S.F32, cfg, dq_dt=None)
    assert gpu["g"].view(np.uint32) == ref["g"].view(np.uint32)
    compare_quant(gpu, ref, keys=("scales", "codes", "mse"))


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("strategy", [ABSMAX, PZ, FOS, BF])
def test_block_sweep_full_size_sampled(O_lib, kind, strategy):
    """fp32 4096 x 4096 at B = 16 and 4: full-size launch, oracle on sampled rows."""
    full = full_c2()[kind]
    rows = sample_rows(full.shape[0], seed=len(kind))
    for B in (16, 4):
        for gm in (TAMAX, NONE):
            cfg = F.config(E4M3, B, strategy, gm)
            note(f"sweep full {kind} B={B} {STRAT_NAMES[strategy]} gm={gm}")
            gpu = gpu_quantize(full, S.F32, cfg)
            g = O.tensor_global_scale(full) if gm == TAMAX else None
            if g is not None:
                assert gpu["g"].view(np.uint32) == g.view(np.uint32)
            ref = oracle_quantize(full[rows], S.F32, cfg, user_g=g)
            compare_quant(gpu, ref, rows)


# --------------------------------------------------------------------------
# Llama-3.1-8B-shaped bf16 MLP weights
# --------------------------------------------------------------------------

@pytest.mark.parametrize("which", ["w_down", "w_up"])
@pytest.mark.parametrize("name,cfg", [("nvfp4-4over6", F.nvfp4(FOS)), ("mxfp4-absmax", F.mxfp4())])
@pytest.mark.parametrize("full_outputs", [False, True])
def test_llama_mlp_weights(O_lib, which, name, cfg, full_outputs):
    w = full_c3()[which]
    note(f"llama {which} {w.shape} {name} full_outputs={full_outputs}")
    gpu = gpu_quantize(w, S.BF16, cfg, dq_dt=S.BF16 if full_outputs else None, want_mse=full_outputs)
    g = O.tensor_global_scale(w, x_dt=S.BF16) if cfg.global_mode == TAMAX else None
    if g is not None:
        assert gpu["g"].view(np.uint32) == g.view(np.uint32)
    rows = sample_rows(w.shape[0], seed=3)
    ref = oracle_quantize(w[rows], S.BF16, cfg, dq_dt=S.BF16, user_g=g)
    compare_quant(gpu, ref, rows)


# --------------------------------------------------------------------------
# dynamic activations with the block Hadamard fused before quantization
# --------------------------------------------------------------------------

ACT_CFGS = [
    ("mxfp4", lambda H: F.mxfp4(hadamard=H)),
    ("nvfp4-amax", lambda H: F.nvfp4(hadamard=H)),
    ("nvfp4-user", lambda H: F.nvfp4(global_mode=USER, global_scale=0.015625, hadamard=H)),
    ("nvfp4-4over6", lambda H: F.nvfp4(FOS, hadamard=H)),
]


@pytest.mark.parametrize("H", [0, 16, 32])
@pytest.mark.parametrize("name,mk", ACT_CFGS)
def test_activations_rotation_small(O_lib, H, name, mk):
    a = S.activations(67, 4096, 5)
    cfg = mk(H)
    note(f"activations small H={H} {name}")
    gpu = gpu_quantize(a, S.BF16, cfg, dq_dt=S.BF16)
    ref = oracle_quantize(a, S.BF16, cfg, dq_dt=S.BF16)
    assert gpu["g"].view(np.uint32) == ref["g"].view(np.uint32)
    compare_quant(gpu, ref)


@pytest.mark.parametrize("H", [16, 32])
@pytest.mark.parametrize("name,mk", ACT_CFGS[:3])
def test_activations_rotation_full_size_sampled(O_lib, H, name, mk):
    a = S.config4()
    cfg = mk(H)
    note(f"activations full {a.shape} H={H} {name}")
    gpu = gpu_quantize(a, S.BF16, cfg, dq_dt=None, want_mse=False)
    g = O.tensor_global_scale(a, hadamard=H, x_dt=S.BF16) if cfg.global_mode == TAMAX else None
    if g is not None:
        assert gpu["g"].view(np.uint32) == g.view(np.uint32)
    rows = sample_rows(a.shape[0], seed=H)
    ref = oracle_quantize(a[rows], S.BF16, cfg, user_g=g)
    compare_quant(gpu, ref, rows, keys=("codes", "scales"))


# --------------------------------------------------------------------------
# FOCUS relaxed fake-quant forward / STE backward
# --------------------------------------------------------------------------

def focus_case(fmt, rows, cols, K, seeds=(6, 7, 8)):
    w, c, g = S.focus_inputs(rows, cols, K, seeds=seeds)
    cfg = F.mxfp4() if fmt == E8M0 else F.nvfp4()
    q = O.quantize(w, x_dt=S.BF16, fmt=cfg.scale_fmt, block=cfg.block, strategy=ABSMAX,
                   global_mode=cfg.global_mode, dq_dt=None)
    return w, c, g, cfg, q


def gpu_focus(w, c, grad, cfg, scales, gval, K):
    wt = S.to_torch(w, S.BF16, DEV)
    ct = S.to_torch(c, S.F16, DEV)
    gt = S.to_torch(grad, S.BF16, DEV)
    st = torch.from_numpy(scales).to(DEV)
    gd = None if cfg.scale_fmt == E8M0 else torch.tensor([gval], dtype=torch.float32, device=DEV)
    wh, codes = F.relaxed_fakequant_fwd(wt, st, ct, cfg, sub_block=K, g=gd, want_codes=True)
    gc = F.relaxed_fakequant_bwd(wt, st, ct, gt, cfg, sub_block=K, g=gd)
    torch.cuda.synchronize()
    return S.from_torch(wh), S.from_torch(codes), S.from_torch(gc)


@pytest.mark.parametrize("fmt", [E8M0, E4M3])
@pytest.mark.parametrize("K", [4, 8, 16])
def test_focus_small(O_lib, fmt, K):
    w, c, grad, cfg, q = focus_case(fmt, 33, 1024, K)
    note(f"focus small fmt={fmt} K={K}")
    wh, codes, gc = gpu_focus(w, c, grad, cfg, q["scales"], q["g"], K)
    rw, rc = O.relaxed_fwd(w, q["scales"], q["g"], c, fmt=cfg.scale_fmt, block=cfg.block, sub_block=K, w_dt=S.BF16)
    rg = O.relaxed_bwd(w, q["scales"], q["g"], c, grad, fmt=cfg.scale_fmt, block=cfg.block, sub_block=K,
                       w_dt=S.BF16, g_dt=S.BF16)
    assert_same(wh, rw, "w_hat")
    assert_same(codes, rc, "codes")
    assert_same(gc, rg, "grad_c")


@pytest.mark.parametrize("fmt", [E8M0, E4M3])
def test_focus_full_size_sampled(O_lib, fmt):
    K = 8
    w, c, grad = S.config5(K)
    cfg = F.mxfp4() if fmt == E8M0 else F.nvfp4()
    note(f"focus full {w.shape} fmt={fmt}")
    # the dequantization scales: abs-max of the whole tensor, from the oracle
    gval = O.tensor_global_scale(w, x_dt=S.BF16) if fmt == E4M3 else np.float32(1)
    rows = sample_rows(w.shape[0], seed=5)
    full_scales = np.zeros((w.shape[0], w.shape[1] // cfg.block), np.uint8)
    qs = O.quantize(w[rows], x_dt=S.BF16, fmt=cfg.scale_fmt, block=cfg.block, strategy=ABSMAX,
                    global_mode=USER if fmt == E4M3 else NONE, user_g=gval, dq_dt=None)
    full_scales[rows] = qs["scales"]
    # rows outside the sample get arbitrary valid scales (their outputs are not compared)
    wh, codes, gc = gpu_focus(w, c, grad, cfg, full_scales, gval, K)
    rw, rc = O.relaxed_fwd(w[rows], qs["scales"], gval, c[rows], fmt=cfg.scale_fmt, block=cfg.block,
                           sub_block=K, w_dt=S.BF16)
    rg = O.relaxed_bwd(w[rows], qs["scales"], gval, c[rows], grad[rows], fmt=cfg.scale_fmt, block=cfg.block,
                       sub_block=K, w_dt=S.BF16, g_dt=S.BF16)
    assert_same(wh[rows], rw, "w_hat")
    assert_same(codes[rows], rc, "codes")
    assert_same(gc[rows], rg, "grad_c")


# --------------------------------------------------------------------------
# stand-alone dequantize / block MSE / scale search
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,B,gm,H", [(E4M3, 16, TAMAX, 0), (E8M0, 32, NONE, 0), (E4M3, 4, NONE, 0),
                                        (E4M3, 16, TAMAX, 32), (E8M0, 32, NONE, 16)])
@pytest.mark.parametrize("out_dt", [S.F32, S.BF16, S.F16])
def test_dequantize_and_block_mse(O_lib, fmt, B, gm, H, out_dt):
    x = S.laplace(45, 1024, 9)
    ref = O.quantize(x, fmt=fmt, block=B, strategy=FOS if fmt == E4M3 else ABSMAX, global_mode=gm,
                     hadamard=H, dq_dt=out_dt)
    cfg = F.config(fmt, B, ABSMAX, gm, hadamard=H)
    note(f"dequantize/block_mse fmt={fmt} B={B} H={H} out={out_dt}")
    codes = torch.from_numpy(ref["codes"]).to(DEV)
    scales = torch.from_numpy(ref["scales"]).to(DEV)
    g = None if fmt == E8M0 else torch.tensor([ref["g"]], dtype=torch.float32, device=DEV)
    dq = F.dequantize(codes, scales, cfg, g=g, out_dtype=TORCH_DT[out_dt])
    mse = F.block_mse(S.to_torch(x, S.F32, DEV), codes, scales, cfg, g=g)
    torch.cuda.synchronize()
    assert_same(S.from_torch(dq), ref["dequant"], "dequant")
    assert_same(S.from_torch(mse), ref["mse"], "mse")


@pytest.mark.parametrize("strategy", [ABSMAX, PZ, FOS, BF])
def test_scale_search(O_lib, strategy):
    x = small_c2("laplace_1e-4", 11, 2048)
    cfg = F.config(E4M3, 8, strategy, NONE)
    note(f"scale_search {STRAT_NAMES[strategy]}")
    r = F.scale_search(S.to_torch(x, S.F32, DEV), cfg)
    torch.cuda.synchronize()
    ref = oracle_quantize(x, S.F32, cfg)
    assert_same(S.from_torch(r["scales"]), ref["scales"], "scales")
    assert_same(S.from_torch(r["sse"]), ref["sse"], "sse")


def test_given_scales(O_lib):
    x = S.normal(40, 512, 17)
    ref0 = O.quantize(x, fmt=E4M3, block=16, strategy=BF, global_mode=USER, user_g=0.25)
    cfg = F.config(E4M3, 16, GIVEN, USER, 0.25)
    note("given scales")
    gpu = gpu_quantize(x, S.F32, cfg, scales_in=ref0["scales"])
    ref = oracle_quantize(x, S.F32, cfg, scales_in=ref0["scales"])
    compare_quant(gpu, ref)
