"""The hand-derived worked examples of tests/golden/ through the HIP path.

The same fixtures pin the oracle (tests/test_oracle_golden.py); here the
GPU library is checked against the fixtures' own expected values, which
were derived by hand from the definitions each file cites.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden")
ST = {"ABSMAX": 0, "PREVENT_ZERO": 1, "FOUR_OVER_SIX": 2, "BRUTE_FORCE": 3}


def load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def f32bits(a):
    return np.asarray(a, np.float32).reshape(-1).view(np.uint32)


def run_quant(F, torch, x, fmt, block, strategy, hadamard=0):
    from gpu_helpers import note
    cfg = F.config(F.E8M0 if fmt == "E8M0" else F.E4M3, block, ST[strategy], F.GLOBAL_NONE, 1.0, hadamard)
    note(f"golden quantize fmt={fmt} B={block} {strategy} H={hadamard} shape={x.shape}")
    r = F.quantize(torch.from_numpy(x).cuda(), cfg, dequant_dtype=torch.float32, want_mse=True)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in r.items() if v is not None}


@pytest.fixture(scope="module")
def lib_torch():
    import torch
    from microscaling_fp4_block_fp4q_amd import fp4q as F
    F.lib()
    return F, torch


def test_mxfp4_absmax_block(lib_torch):
    F, torch = lib_torch
    d = load("mxfp4_absmax_block.json")
    x = np.asarray(d["x"], np.float32).reshape(1, -1)
    r = run_quant(F, torch, x, d["fmt"], d["block"], d["strategy"])
    assert r["scales"].reshape(-1).tolist() == d["scales"]
    assert r["codes"].reshape(-1).tolist() == d["codes"]
    assert np.array_equal(f32bits(r["dequant"]), f32bits(d["dequant"]))
    assert np.array_equal(f32bits(r["mse"]), f32bits(d["mse"]))


@pytest.mark.parametrize("name", ["nvfp4_absmax_vs_4over6.json", "prevent_zero_block.json"])
def test_e4m3_strategy_cases(lib_torch, name):
    F, torch = lib_torch
    d = load(name)
    x = np.asarray(d["x"], np.float32).reshape(1, -1)
    for st, want in d["cases"].items():
        r = run_quant(F, torch, x, d["fmt"], d["block"], st)
        assert r["scales"].reshape(-1).tolist() == want["scales"], st
        assert r["codes"].reshape(-1).tolist() == want["codes"], st
        assert np.array_equal(f32bits(r["dequant"]), f32bits(want["dequant"])), st
        assert np.array_equal(f32bits(r["mse"]), f32bits(want["mse"])), st


def test_hadamard16_unit_vectors(lib_torch):
    F, torch = lib_torch
    d = load("hadamard16_unit_vectors.json")
    x = np.asarray(d["x"], np.float32)
    r = run_quant(F, torch, x, d["fmt"], d["block"], d["strategy"], hadamard=d["hadamard"])
    assert r["scales"].tolist() == d["scales"]
    assert r["codes"].tolist() == d["codes"]
    assert np.array_equal(f32bits(r["mse"]), f32bits(d["mse"]))


def test_focus_relaxed_block(lib_torch):
    from gpu_helpers import note
    F, torch = lib_torch
    d = load("focus_relaxed_block.json")
    w = torch.from_numpy(np.asarray(d["w"], np.float32).reshape(1, -1)).cuda()
    c = torch.from_numpy(np.asarray(d["c"], np.float16).reshape(1, -1)).cuda()
    scales = torch.from_numpy(np.asarray(d["scales"], np.uint8).reshape(1, -1)).cuda()
    cfg = F.mxfp4()
    note("golden focus fwd/bwd MXFP4 1x32 K=8")
    w_hat, codes = F.relaxed_fakequant_fwd(w, scales, c, cfg, sub_block=d["sub_block"], out_dtype=torch.float32,
                                           want_codes=True)
    grad_c = F.relaxed_fakequant_bwd(w, scales, c, torch.ones_like(w), cfg, sub_block=d["sub_block"])
    torch.cuda.synchronize()
    assert np.array_equal(f32bits(w_hat.cpu().numpy()), f32bits(d["w_hat"]))
    assert codes.cpu().numpy().reshape(-1).tolist() == d["codes"]
    want = [np.float32(float(Fraction(s))) for s in d["grad_c"]]
    assert np.array_equal(f32bits(grad_c.cpu().numpy()), f32bits(want))
