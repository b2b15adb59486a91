"""GPU parity at the full workload sizes, every row: each call the benchmark
times is run here through the C ABI on the same seeded input, and every
output (codes, scales, g, dequantized values, block MSE, FOCUS W_hat and
grad_c) is compared bit for bit with the oracle run on all rows.

The oracle is single-threaded; it runs here on row chunks spread over the
host's cores (rows are independent once the per-tensor scale is known; that
scale comes from the oracle's own whole-tensor abs-max and is passed to the
chunks as the user scale, and the GPU's g is checked against it).  The
brute-force cases include the launches that run the quantize kernels
residency-capped, where every lane prefetches a real next tile: block 32 on
4096 x 4096 fp32, E8M0 block 32 on 16.8 M values, and the 32-wide rotation
on the 8192 x 4096 bf16 activations.
"""
import functools

import numpy as np
import pytest
import torch

from microscaling_fp4_block_fp4q_amd import fp4q as F
from microscaling_fp4_block_fp4q_amd import synth as S
from oracle import oracle as O

from gpu_helpers import DEV, TORCH_DT, assert_same, compare_quant, gpu_quantize, note, oracle_rows

pytestmark = pytest.mark.gpu

E8M0, E4M3 = F.E8M0, F.E4M3
ABSMAX, PZ, FOS, BF = F.ABSMAX, F.PREVENT_ZERO, F.FOUR_OVER_SIX, F.BRUTE_FORCE
NONE, TAMAX, USER = F.GLOBAL_NONE, F.GLOBAL_TENSOR_AMAX, F.GLOBAL_USER
STRAT = {ABSMAX: "absmax", PZ: "prevent-zero", FOS: "4-over-6", BF: "brute-force"}
KINDS = ["normal", "laplace", "normal_1e-4", "laplace_1e-4"]


@functools.lru_cache(maxsize=1)
def c2():
    return S.config2()


@functools.lru_cache(maxsize=1)
def c3():
    return S.config3()


@functools.lru_cache(maxsize=1)
def c4():
    return S.config4()


def oracle_full(x, x_dt, cfg, dq_dt=S.F32):
    """The oracle's quantization of every row of x under cfg, with the
    whole tensor's per-tensor scale for TENSOR_AMAX."""
    gm, g = cfg.global_mode, cfg.global_scale
    if gm == TAMAX:
        g = O.tensor_global_scale(x, hadamard=cfg.hadamard, x_dt=x_dt)
        gm = USER
    ref = oracle_rows(O.quantize, [x], fmt=cfg.scale_fmt, block=cfg.block, strategy=cfg.strategy,
                      global_mode=gm, user_g=g, hadamard=cfg.hadamard, x_dt=x_dt, dq_dt=dq_dt)
    if cfg.global_mode == TAMAX:
        ref["g"] = np.float32(g)
    return ref


def check_all_rows(x, x_dt, cfg, dq_dt=S.F32, want_mse=True):
    gpu = gpu_quantize(x, x_dt, cfg, dq_dt=dq_dt, want_mse=want_mse)
    ref = oracle_full(x, x_dt, cfg, dq_dt=dq_dt if dq_dt is not None else S.F32)
    if cfg.global_mode != NONE:
        assert gpu["g"].view(np.uint32) == np.float32(ref["g"]).view(np.uint32), (gpu["g"], ref["g"])
    keys = ("codes", "scales") + (("dequant",) if dq_dt is not None else ()) + (("mse",) if want_mse else ())
    compare_quant(gpu, ref, keys=keys)
    return gpu, ref


# --------------------------------------------------------------------------
# the step: fp32 4096 x 4096, block sweep x strategy x per-tensor scale
# --------------------------------------------------------------------------

@pytest.mark.parametrize("gm", [TAMAX, NONE])
@pytest.mark.parametrize("strategy", [ABSMAX, PZ, FOS, BF])
@pytest.mark.parametrize("B", [4, 8, 16, 32])
@pytest.mark.parametrize("kind", KINDS)
def test_step_quantize_every_row(O_lib, kind, B, strategy, gm):
    x = c2()[kind]
    cfg = F.config(E4M3, B, strategy, gm)
    note(f"full 4096x4096 {kind} B={B} {STRAT[strategy]} gm={gm}")
    check_all_rows(x, S.F32, cfg)


@pytest.mark.parametrize("H,cfg", [(16, F.nvfp4(hadamard=16)), (32, F.mxfp4(hadamard=32))])
def test_step_rotation_every_row(O_lib, H, cfg):
    x = c2()["normal"]
    note(f"full 4096x4096 normal H={H}")
    check_all_rows(x, S.F32, cfg)


def test_step_dequantize_and_block_mse_every_row(O_lib):
    x = c2()["normal"]
    cfg = F.nvfp4(hadamard=16)
    note("full 4096x4096 dequantize + block MSE of the rotated NVFP4 result")
    ref = oracle_full(x, S.F32, cfg)
    codes = torch.from_numpy(ref["codes"]).to(DEV)
    scales = torch.from_numpy(ref["scales"]).to(DEV)
    g = torch.tensor([ref["g"]], dtype=torch.float32, device=DEV)
    dq = F.dequantize(codes, scales, cfg, g=g, out_dtype=torch.float32)
    mse = F.block_mse(S.to_torch(x, S.F32, DEV), codes, scales, cfg, g=g)
    torch.cuda.synchronize()
    assert_same(S.from_torch(dq), ref["dequant"], "dequant")
    assert_same(S.from_torch(mse), ref["mse"], "mse")


def focus_every_row(w, w_dt, c, grad, g_dt, cfg, gq_user, out_dt, K=8):
    """FOCUS forward (+ codes) and backward on every row, S_dq from the
    oracle's abs-max quantization of w under cfg (per-tensor scale: the
    tensor's own for TENSOR_AMAX, else cfg's)."""
    ref_q = oracle_full(w, w_dt, cfg, dq_dt=None) if gq_user is None else \
        oracle_rows(O.quantize, [w], fmt=cfg.scale_fmt, block=cfg.block, strategy=ABSMAX, global_mode=USER,
                    user_g=gq_user, x_dt=w_dt, dq_dt=None)
    gval = np.float32(1.0) if cfg.scale_fmt == E8M0 else np.float32(ref_q["g"] if gq_user is None else gq_user)
    wt, ct = S.to_torch(w, w_dt, DEV), S.to_torch(c, S.F16, DEV)
    gt = S.to_torch(grad, g_dt, DEV)
    st = torch.from_numpy(ref_q["scales"]).to(DEV)
    gd = None if cfg.scale_fmt == E8M0 else torch.tensor([gval], dtype=torch.float32, device=DEV)
    wh, codes = F.relaxed_fakequant_fwd(wt, st, ct, cfg, sub_block=K, g=gd, out_dtype=TORCH_DT[out_dt],
                                        want_codes=True)
    gc = F.relaxed_fakequant_bwd(wt, st, ct, gt, cfg, sub_block=K, g=gd)
    torch.cuda.synchronize()
    rw, rc = oracle_rows(_relaxed_fwd_rows, [w, ref_q["scales"], c], g=gval, fmt=cfg.scale_fmt, block=cfg.block,
                         sub_block=K, w_dt=w_dt, out_dt=out_dt)
    rg = oracle_rows(_relaxed_bwd_rows, [w, ref_q["scales"], c, grad], g=gval, fmt=cfg.scale_fmt, block=cfg.block,
                     sub_block=K, w_dt=w_dt, g_dt=g_dt)
    assert_same(S.from_torch(wh), rw, "w_hat")
    assert_same(S.from_torch(codes), rc, "codes")
    assert_same(S.from_torch(gc), rg, "grad_c")


def _relaxed_fwd_rows(w, scales, c, g, **kw):
    return O.relaxed_fwd(w, scales, g, c, **kw)


def _relaxed_bwd_rows(w, scales, c, grad, g, **kw):
    return O.relaxed_bwd(w, scales, g, c, grad, **kw)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4-user"])
def test_step_focus_every_row(O_lib, fmt):
    x = c2()["normal"]
    R, C = x.shape
    K = 8
    c16 = S.cast(np.random.default_rng(7).uniform(0.8, 1.25, (R, C // K)), S.F16)
    grad = S.normal(R, C, 8, S.F32)
    cfg = F.mxfp4() if fmt == "mxfp4" else F.nvfp4(0, USER, 2.0 ** -12)
    note(f"full 4096x4096 FOCUS fp32 {fmt}")
    focus_every_row(x, S.F32, c16, grad, S.F32, cfg, None if fmt == "mxfp4" else np.float32(2.0 ** -12), S.F32)


# --------------------------------------------------------------------------
# brute force where the kernels run residency-capped (prefetching lanes)
# --------------------------------------------------------------------------

def test_e8m0_block32_brute_force_every_row(O_lib):
    x = c2()["laplace"]
    note("full 4096x4096 laplace E8M0 B=32 brute force")
    check_all_rows(x, S.F32, F.config(E8M0, 32, BF))


@pytest.mark.parametrize("name,cfg", [("e4m3-b16-amax", F.config(E4M3, 16, BF, TAMAX, hadamard=32)),
                                      ("e8m0-b32", F.config(E8M0, 32, BF, hadamard=32))])
def test_activations_rotation32_brute_force_every_row(O_lib, name, cfg):
    a = c4()
    note(f"full 8192x4096 bf16 activations H=32 brute force {name}")
    check_all_rows(a, S.BF16, cfg, dq_dt=S.BF16)


# --------------------------------------------------------------------------
# the other workloads the benchmark times
# --------------------------------------------------------------------------

@pytest.mark.parametrize("full", [False, True])
@pytest.mark.parametrize("name,cfg", [("nvfp4-4over6", F.nvfp4(FOS)), ("mxfp4-absmax", F.mxfp4())])
@pytest.mark.parametrize("which", ["w_down", "w_up"])
def test_llama_weights_every_row(O_lib, which, name, cfg, full):
    w = c3()[which]
    note(f"llama {which} {w.shape} {name} full={full}")
    check_all_rows(w, S.BF16, cfg, dq_dt=S.BF16 if full else None, want_mse=full)


ACT = [("mxfp4", lambda H: F.mxfp4(hadamard=H)),
       ("nvfp4-amax", lambda H: F.nvfp4(hadamard=H)),
       ("nvfp4-user", lambda H: F.nvfp4(global_mode=USER, global_scale=0.015625, hadamard=H)),
       ("nvfp4-4over6", lambda H: F.nvfp4(FOS, hadamard=H))]


@pytest.mark.parametrize("full", [False, True])
@pytest.mark.parametrize("name,mk", ACT)
@pytest.mark.parametrize("H", [0, 16, 32])
def test_activations_every_row(O_lib, H, name, mk, full):
    a = c4()
    note(f"activations {a.shape} H={H} {name} full={full}")
    check_all_rows(a, S.BF16, mk(H), dq_dt=S.BF16 if full else None, want_mse=full)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_focus_bf16_every_row(O_lib, fmt):
    K = 8
    w, c, g = S.config5(K)
    cfg = F.mxfp4() if fmt == "mxfp4" else F.nvfp4()
    note(f"FOCUS bf16 {w.shape} {fmt} every row")
    focus_every_row(w, S.BF16, c, g, S.BF16, cfg, None, S.BF16)
