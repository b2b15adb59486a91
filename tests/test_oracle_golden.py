"""Hand-derived worked examples (tests/golden/*.json) against the oracle.

The pages print no quantized values, so each fixture is derived by hand
from the definitions it cites (its "derivation" field), with dyadic inputs
so every expected value is exact.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")
FMT = {"E8M0": 0, "E4M3": 1}
ST = {"ABSMAX": 0, "PREVENT_ZERO": 1, "FOUR_OVER_SIX": 2, "BRUTE_FORCE": 3}


def load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def f32(a):
    return np.asarray(a, np.float32)


def same_bits(a, b):
    return np.array_equal(f32(a).view(np.uint32), f32(b).view(np.uint32))


def test_mxfp4_absmax_block(O):
    d = load("mxfp4_absmax_block.json")
    x = f32(d["x"]).reshape(1, -1)
    r = O.quantize(x, fmt=FMT[d["fmt"]], block=d["block"], strategy=ST[d["strategy"]])
    assert list(r["scales"].reshape(-1)) == d["scales"]
    assert list(r["codes"].reshape(-1)) == d["codes"]
    assert same_bits(r["dequant"].reshape(-1), d["dequant"])
    assert same_bits(r["mse"].reshape(-1), d["mse"])


@pytest.mark.parametrize("name", ["nvfp4_absmax_vs_4over6.json", "prevent_zero_block.json"])
def test_e4m3_strategy_cases(O, name):
    d = load(name)
    x = f32(d["x"]).reshape(1, -1)
    for st, want in d["cases"].items():
        r = O.quantize(x, fmt=FMT[d["fmt"]], block=d["block"], strategy=ST[st])
        assert list(r["scales"].reshape(-1)) == want["scales"], st
        assert list(r["codes"].reshape(-1)) == want["codes"], st
        assert same_bits(r["dequant"].reshape(-1), want["dequant"]), st
        assert same_bits(r["mse"].reshape(-1), want["mse"]), st


def test_hadamard16_unit_vectors(O):
    d = load("hadamard16_unit_vectors.json")
    x = f32(d["x"])
    r = O.quantize(x, fmt=FMT[d["fmt"]], block=d["block"], strategy=ST[d["strategy"]], hadamard=d["hadamard"])
    assert r["scales"].tolist() == d["scales"]
    assert r["codes"].tolist() == d["codes"]
    assert same_bits(r["mse"], d["mse"])


def test_focus_relaxed_block(O):
    d = load("focus_relaxed_block.json")
    w = f32(d["w"]).reshape(1, -1)
    c = np.asarray(d["c"], np.float16).view(np.uint16).reshape(1, -1)
    scales = np.asarray(d["scales"], np.uint8).reshape(1, -1)
    wh, codes = O.relaxed_fwd(w, scales, 1.0, c, fmt=FMT[d["fmt"]], block=d["block"], sub_block=d["sub_block"])
    assert same_bits(wh.reshape(-1), d["w_hat"])
    assert list(codes.reshape(-1)) == d["codes"]
    G = np.ones_like(w)
    gc = O.relaxed_bwd(w, scales, 1.0, c, G, fmt=FMT[d["fmt"]], block=d["block"], sub_block=d["sub_block"])
    want = [np.float32(float(Fraction(s))) for s in d["grad_c"]]
    assert same_bits(gc.reshape(-1), want)
