"""fp4q_quantize_noalloc (the quantize entry point whose workspace is the
library's static device scratch) against fp4q_quantize with a caller
workspace: every output bit for bit, on two calls in a row, the second on a
smaller input (the scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

from microscaling_fp4_block_fp4q_amd import fp4q as F
from microscaling_fp4_block_fp4q_amd import synth as S

from gpu_helpers import DEV, TORCH_DT, assert_same, note

pytestmark = pytest.mark.gpu

CASES = [
    ("nvfp4-4over6-amax fp32", F.nvfp4(F.FOUR_OVER_SIX), S.F32, (512, 4096), (96, 1024)),
    ("e4m3-b16-search fp32", F.config(F.E4M3, 16, F.ABSMAX, F.GLOBAL_SEARCH), S.F32, (256, 2048), (40, 512)),
    ("e4m3-b8-bruteforce-search fp32", F.config(F.E4M3, 8, F.BRUTE_FORCE, F.GLOBAL_SEARCH), S.F32,
     (64, 1024), (9, 256)),
    ("nvfp4-amax-rot16 bf16", F.nvfp4(hadamard=16), S.BF16, (384, 4096), (33, 256)),
    ("mxfp4 bf16", F.mxfp4(), S.BF16, (128, 1024), (16, 256)),
]


def outputs(cfg, x, dq_dtype):
    rows, cols = x.shape
    return dict(codes=torch.full((rows, cols // 2), 0xAB, dtype=torch.uint8, device=DEV),
                scales=torch.full((rows, cols // cfg.block), 0xCD, dtype=torch.uint8, device=DEV),
                g=torch.full((1,), -1.0, dtype=torch.float32, device=DEV),
                dequant=torch.full((rows, cols), 7.0, dtype=dq_dtype, device=DEV),
                mse=torch.full((rows, cols // cfg.block), -1.0, dtype=torch.float32, device=DEV))


@pytest.mark.parametrize("name,cfg,x_dt,big,small", CASES)
def test_noalloc_matches_quantize_twice(O_lib, name, cfg, x_dt, big, small):
    dq_dtype = TORCH_DT[x_dt]
    for k, shape in enumerate((big, small)):
        x = S.laplace(*shape, 50 + k, x_dt) if x_dt == S.F32 else S.activations(*shape, 50 + k, x_dt)
        xt = S.to_torch(x, x_dt, DEV)
        note(f"noalloc {name} call {k} shape={shape}")
        a = outputs(cfg, xt, dq_dtype)
        F.fp4q_quantize_noalloc(cfg, xt, a["codes"], a["scales"], a["g"], a["dequant"], a["mse"])
        b = outputs(cfg, xt, dq_dtype)
        ws = torch.empty(max(F.workspace_bytes(cfg, *shape), 16), dtype=torch.uint8, device=DEV)
        F.fp4q_quantize(cfg, xt, b["codes"], b["scales"], b["g"], b["dequant"], b["mse"], ws)
        torch.cuda.synchronize()
        for key in ("codes", "scales", "g", "dequant", "mse"):
            assert_same(S.from_torch(a[key]), S.from_torch(b[key]), f"{key} (call {k})")
