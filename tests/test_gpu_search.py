"""GPU parity of the MSE-searched per-tensor scale (global mode SEARCH)
against the oracle: the chosen g bit for bit and every output at it, on
reduced tensors with ragged tiles, bf16 input, rotation, row strides, the
scale-search entry point, special tensors, and the full 4096 x 4096 fp32
workload (g from the oracle's search over the whole tensor, outputs on
sampled rows)."""
import functools
import json
import os

import numpy as np
import pytest
import torch

from microscaling_fp4_block_fp4q_amd import fp4q as F
from microscaling_fp4_block_fp4q_amd import synth as S
from oracle import oracle as O

from gpu_helpers import DEV, assert_same, compare_quant, gpu_quantize, note, oracle_quantize, sample_rows

pytestmark = pytest.mark.gpu

E4M3 = F.E4M3
SEARCH = F.GLOBAL_SEARCH
NAMES = {F.ABSMAX: "absmax", F.PREVENT_ZERO: "prevent-zero", F.FOUR_OVER_SIX: "4-over-6", F.BRUTE_FORCE: "brute-force"}


def small(kind, rows=37, cols=4000):
    if kind == "normal":
        return S.normal(rows, cols, 1)
    if kind == "laplace":
        return S.laplace(rows, cols, 2)
    if kind == "normal_1e-4":
        return S.scaled_fp32(S.normal(rows, cols, 1), 1e-4)
    x = S.normal(rows, cols, 3)                    # a few outliers: shrinking g clips their blocks
    x[::7, 11] *= np.float32(30.0)
    return x


@pytest.mark.parametrize("kind", ["normal", "laplace", "normal_1e-4", "outliers"])
@pytest.mark.parametrize("B", [4, 8, 16, 32])
@pytest.mark.parametrize("strategy", [F.ABSMAX, F.PREVENT_ZERO, F.FOUR_OVER_SIX, F.BRUTE_FORCE])
def test_search_small(O_lib, kind, B, strategy):
    # brute force inside: 32 exhaustive searches in the oracle, so fewer rows
    x = small(kind, 5 if strategy == F.BRUTE_FORCE else 37)
    cfg = F.config(E4M3, B, strategy, SEARCH)
    note(f"search {kind} B={B} {NAMES[strategy]} shape={x.shape}")
    gpu = gpu_quantize(x, S.F32, cfg)
    ref = oracle_quantize(x, S.F32, cfg)
    assert gpu["g"].view(np.uint32) == ref["g"].view(np.uint32), (gpu["g"], ref["g"])
    compare_quant(gpu, ref)


@pytest.mark.parametrize("strategy", [F.ABSMAX, F.BRUTE_FORCE])
@pytest.mark.parametrize("H", [16, 32])
def test_search_bf16_rotated(O_lib, H, strategy):
    x = S.cast(S.laplace(8 if strategy == F.BRUTE_FORCE else 40, 2048, 5), S.BF16)
    cfg = F.config(E4M3, 16, strategy, SEARCH, 1.0, H)
    note(f"search bf16 H={H} {NAMES[strategy]}")
    gpu = gpu_quantize(x, S.BF16, cfg, dq_dt=S.BF16)
    ref = oracle_quantize(x, S.BF16, cfg, dq_dt=S.BF16)
    assert gpu["g"].view(np.uint32) == ref["g"].view(np.uint32)
    compare_quant(gpu, ref)


def test_search_row_stride(O_lib):
    full = S.normal(24, 640, 9)
    x = full[:, :512]                              # a strided view: ld 640, cols 512
    cfg = F.config(E4M3, 16, F.FOUR_OVER_SIX, SEARCH)
    note("search row stride 640")
    xt = S.to_torch(full, S.F32, DEV)[:, :512]
    r = F.quantize(xt, cfg, dequant_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle_quantize(np.ascontiguousarray(x), S.F32, cfg)
    assert S.from_torch(r["g"])[0].view(np.uint32) == ref["g"].view(np.uint32)
    for k in ("codes", "scales", "dequant", "mse"):
        assert_same(S.from_torch(r[k]), ref[k], k)


@pytest.mark.parametrize("strategy", [F.FOUR_OVER_SIX, F.BRUTE_FORCE])
def test_scale_search_entry(O_lib, strategy):
    x = small("laplace", 21, 1024)
    cfg = F.config(E4M3, 16, strategy, SEARCH)
    note(f"scale_search entry with SEARCH {NAMES[strategy]}")
    r = F.scale_search(S.to_torch(x, S.F32, DEV), cfg)
    torch.cuda.synchronize()
    ref = oracle_quantize(x, S.F32, cfg)
    assert S.from_torch(r["g"])[0].view(np.uint32) == ref["g"].view(np.uint32)
    assert_same(S.from_torch(r["scales"]), ref["scales"], "scales")
    assert_same(S.from_torch(r["sse"]), ref["sse"], "best_sse")


def test_search_special_tensors(O_lib):
    cfg = F.config(E4M3, 16, F.ABSMAX, SEARCH)
    z = np.zeros((4, 64), np.float32)
    note("search zero tensor")
    gpu = gpu_quantize(z, S.F32, cfg)
    ref = oracle_quantize(z, S.F32, cfg)
    assert gpu["g"] == np.float32(1.0) and ref["g"] == np.float32(1.0)
    compare_quant(gpu, ref)
    x = small("normal", 5, 256)
    x[2, 17] = np.nan
    note("search tensor with NaN")
    gpu = gpu_quantize(x, S.F32, cfg)
    ref = oracle_quantize(x, S.F32, cfg)
    assert gpu["g"].view(np.uint32) == ref["g"].view(np.uint32)
    compare_quant(gpu, ref)
    note("search empty tensor")
    e = F.quantize(torch.zeros((0, 64), dtype=torch.float32, device=DEV), cfg)
    torch.cuda.synchronize()
    assert float(e["g"][0]) == 1.0


@functools.lru_cache(maxsize=1)
def full_normal():
    return S.config2()["normal"]


def test_search_quarter_size_live(O_lib):
    """1024 x 4096 fp32 N(0,1), B = 16 abs-max: the oracle searches the
    whole tensor live (4096 tiles: a reduction level past the tiles)."""
    x = np.ascontiguousarray(full_normal()[:1024])
    cfg = F.config(E4M3, 16, F.ABSMAX, SEARCH)
    note("search 1024x4096 absmax")
    gpu = gpu_quantize(x, S.F32, cfg)
    g, totals = O.global_scale_search(x, block=16, strategy=F.ABSMAX)
    assert gpu["g"].view(np.uint32) == g.view(np.uint32), (gpu["g"], g, int(np.argmin(totals)))
    rows = sample_rows(x.shape[0], seed=3)
    ref = oracle_quantize(x[rows], S.F32, F.config(E4M3, 16, F.ABSMAX, F.GLOBAL_USER, float(g)), user_g=g)
    compare_quant(gpu, ref, rows)


@pytest.mark.parametrize("strategy", [F.ABSMAX, F.FOUR_OVER_SIX, F.BRUTE_FORCE])
def test_search_full_size_sampled(O_lib, strategy):
    """4096 x 4096 fp32 at B = 16 (two reduction levels past the tiles): the
    oracle's search over the whole tensor is stored in
    tests/golden/search_full_4096.json by make_search_golden.py (it takes the
    oracle minutes, half an hour with brute force inside); outputs are
    compared on sampled rows at that g."""
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "search_full_4096.json")))
    want = gold["cases"][NAMES[strategy]]
    g = np.uint32(want["g_bits"]).view(np.float32)
    full = full_normal()
    cfg = F.config(E4M3, 16, strategy, SEARCH)
    note(f"search full 4096x4096 {NAMES[strategy]}")
    gpu = gpu_quantize(full, S.F32, cfg)
    assert gpu["g"].view(np.uint32) == np.uint32(want["g_bits"]), (gpu["g"], g, want["j"])
    rows = sample_rows(full.shape[0], seed=strategy)
    ref = oracle_quantize(full[rows], S.F32, F.config(E4M3, 16, strategy, F.GLOBAL_USER, float(g)), user_g=g)
    compare_quant(gpu, ref, rows)
