"""Pins of the oracle's MSE-searched per-tensor scale (global mode SEARCH).

The MR-GPTQ page (technical summary, section 2.2) chooses scale grids per
tensor and group for minimum MSE; the Finer-is-Better page (method part 2)
leaves the per-tensor scale of hierarchical scaling at abs-max / (6 * 448).
The search scores the candidates g_j = fl(g0 * (1 - j/64)), j = 0..31, by
the tensor's total squared error under the block strategy and keeps the
smallest, ties to the smallest j.  Here each candidate's total is recomputed
in exact rationals from scale codes restated with numpy fp32 and torch's
e4m3 cast, and the oracle's totals and choice are checked against it.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import exact_ref as X

E4M3 = 1
ABSMAX, PZ, FOS, BF = 0, 1, 2, 3
TAMAX, SEARCH = 1, 3
J = 32


def torch_e4m3(v):
    t = torch.tensor(np.asarray(v, dtype=np.float32)).reshape(-1)
    return t.clamp(max=448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def tensor(seed, rows, cols, kind):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal((rows, cols)).astype(np.float32)
    if kind == "laplace":
        return rng.laplace(0, 1, (rows, cols)).astype(np.float32)
    if kind == "outlier":                       # one large value: shrinking g clips one block
        x = rng.standard_normal((rows, cols)).astype(np.float32)
        x[0, 3] = np.float32(40.0)
        return x
    raise ValueError(kind)


def exact_totals(x, B, strategy):
    """Exact total SSE of every candidate, and the candidates' g."""
    g0 = np.float32(np.abs(x).max() / np.float32(2688.0))
    blocks = x.reshape(-1, B)
    a = np.abs(blocks).max(axis=1).astype(np.float32)
    totals, gs = [], []
    for j in range(J):
        g = np.float32(g0 * np.float32(1.0 - j / 64.0))
        gs.append(g)
        s6 = torch_e4m3((a / (np.float32(6.0) * g)).astype(np.float32))
        s4 = torch_e4m3((a / (np.float32(4.0) * g)).astype(np.float32))
        tot = Fraction(0)
        for b in range(blocks.shape[0]):
            def sse_at(code):
                S = Fraction(float(np.float32(np.float32(float(X.E4M3[code]) if code else 0.0) * g)))
                return X.block_sse_exact(blocks[b], S)
            if strategy == ABSMAX:
                tot += sse_at(int(s6[b]))
            elif strategy == PZ:
                tot += sse_at(max(int(s6[b]), 1))
            else:
                tot += min(sse_at(int(s6[b])), sse_at(int(s4[b])))
        totals.append(tot)
    return totals, gs


@pytest.mark.parametrize("kind", ["normal", "laplace", "outlier"])
@pytest.mark.parametrize("strategy", [ABSMAX, PZ, FOS])
@pytest.mark.parametrize("B", [4, 16])
def test_search_matches_exact_totals(O, kind, strategy, B):
    x = tensor(11 + B, 4, 64, kind)
    g, totals = O.global_scale_search(x, block=B, strategy=strategy)
    want, gs = exact_totals(x, B, strategy)
    for j in range(J):
        w = float(want[j])
        assert abs(totals[j] - w) <= 1e-6 * w + 1e-30, (j, totals[j], w)
    order = sorted(range(J), key=lambda j: (want[j], j))
    best = order[0]
    gap = float(want[order[1]] - want[best]) / max(float(want[best]), 1e-30)
    if gap > 1e-5:                         # away from near-ties the choice is the exact argmin
        assert g == gs[best], (g, gs[best], best)
    assert g in gs
    # the quantize call uses the searched scale
    r = O.quantize(x, fmt=E4M3, block=B, strategy=strategy, global_mode=SEARCH)
    assert r["g"] == g


def test_search_never_worse_than_abs_max_scale(O):
    for kind in ("normal", "laplace", "outlier"):
        x = tensor(5, 16, 128, kind)
        for st in (ABSMAX, FOS):
            rs = O.quantize(x, fmt=E4M3, block=16, strategy=st, global_mode=SEARCH)
            ra = O.quantize(x, fmt=E4M3, block=16, strategy=st, global_mode=TAMAX)
            assert rs["sse"].astype(np.float64).sum() <= ra["sse"].astype(np.float64).sum() * (1 + 1e-6)
            assert rs["g"] <= ra["g"]


def test_exactly_representable_tensor_keeps_g0(O):
    """A tensor that quantizes without error at g0 scores 0 there; ties go to
    the least shrink, so g0 is kept."""
    rng = np.random.default_rng(3)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    g0 = np.float32(2.0 ** -8)
    codes = rng.integers(40, 0x7E, 32)                # E4M3 block scale codes
    codes[0] = 0x7E                                   # block 0 holds the tensor maximum 6 * 448 * g0
    S = np.array([float(X.E4M3[int(c)]) for c in codes], np.float32) * g0
    q = grid[rng.integers(0, 8, (32, 16))]
    q[:, 0] = 6.0
    x = (q * S[:, None]).astype(np.float32).reshape(8, 64)
    assert np.float32(np.abs(x).max() / np.float32(2688.0)) == g0
    g, totals = O.global_scale_search(x, block=16, strategy=ABSMAX)
    assert totals[0] == 0.0 and g == g0


def test_search_special_tensors(O):
    z = np.zeros((2, 32), np.float32)
    g, totals = O.global_scale_search(z, block=16)
    assert g == 1.0 and np.all(totals == 0.0)
    x = tensor(1, 2, 32, "normal")
    x[1, 5] = np.nan
    g, _ = O.global_scale_search(x, block=16)
    assert np.isnan(g)
    r = O.quantize(x, fmt=E4M3, block=16, strategy=ABSMAX, global_mode=SEARCH)
    assert np.all(r["scales"] == 0x7F)


def test_brute_force_search_never_above_prevent_zero(O):
    """With brute force inside, each candidate's total is at most the
    prevent-zero total at the same candidate: per block the exhaustive
    minimum runs over codes 1..126, which include prevent-zero's code, and
    the fp64 tree sum is monotone in its terms."""
    for kind in ("normal", "laplace", "outlier"):
        for B in (4, 16):
            x = tensor(21 + B, 8, 128, kind)
            gb, tb = O.global_scale_search(x, block=B, strategy=BF)
            gp, tp = O.global_scale_search(x, block=B, strategy=PZ)
            assert np.all(tb <= tp), (kind, B, np.argmax(tb - tp))
            assert gb == np.float32(np.float32(np.abs(x).max() / np.float32(2688.0)) *
                                    np.float32(1.0 - int(np.argmin(tb)) / 64.0))
            assert np.all(tb[np.argmin(tb)] < tb[:np.argmin(tb)])   # ties go to the least shrink


def test_brute_force_search_matches_exact_totals(O):
    """Brute force inside the search on 8 blocks of 4: every candidate's
    total against exact rationals (each block at its exact-minimum code over
    1..126, S = fl(dec(code) g) as the format defines it)."""
    x = tensor(7, 1, 32, "laplace")
    B = 4
    g, totals = O.global_scale_search(x, block=B, strategy=BF)
    g0 = np.float32(np.abs(x).max() / np.float32(2688.0))
    blocks = x.reshape(-1, B)
    for j in range(J):
        gj = np.float32(g0 * np.float32(1.0 - j / 64.0))
        tot = Fraction(0)
        for blk in blocks:
            tot += min(X.block_sse_exact(blk, Fraction(float(np.float32(np.float32(float(X.E4M3[c])) * gj))))
                       for c in range(1, 0x7F))
        w = float(tot)
        assert abs(totals[j] - w) <= 1e-6 * w + 1e-30, (j, totals[j], w)
