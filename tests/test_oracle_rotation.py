"""Pins of the oracle's block-wise Walsh-Hadamard rotation (MR-GPTQ page,
technical summary sections 2.1-2.3: a block Hadamard transform mixes each
block before quantization; weights and activations look Laplace before the
rotation and Gaussian after it).

Checked against scipy.linalg.hadamard (Sylvester order), exact integer
orthogonality, exact rational bounds on fl(1/sqrt(n)), and fp64 products.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

E4M3, E8M0 = 1, 0


@pytest.mark.parametrize("n", [16, 32])
def test_fwht_matrix_is_sylvester_hadamard(O, n):
    c = float(O.hadamard_coef(n))
    cols = O.fwht(np.eye(n, dtype=np.float32))      # row j = transform of e_j
    H = np.rint(cols.astype(np.float64) / c).astype(np.int64)
    assert np.array_equal(cols.astype(np.float64), H * c)    # entries are exactly +-c
    assert np.array_equal(H.T, scipy.linalg.hadamard(n))
    assert np.array_equal(H @ H.T, n * np.eye(n, dtype=np.int64))


@pytest.mark.parametrize("n", [16, 32])
def test_normalisation_is_rounded_inverse_sqrt(O, n):
    c = O.hadamard_coef(n)
    cf = Fraction(float(c))
    ulp = Fraction(float(np.spacing(c)))
    lo, hi = cf - ulp / 2, cf + ulp / 2
    # 1/sqrt(n) lies within half an ulp of c  <=>  lo^2 <= 1/n <= hi^2
    assert lo * lo <= Fraction(1, n) <= hi * hi
    if n == 16:
        assert c == np.float32(0.25)


@pytest.mark.parametrize("n", [16, 32])
def test_fwht_vs_fp64_product(O, n):
    rng = np.random.default_rng(n)
    x = rng.laplace(0, 1, (64, n)).astype(np.float32)
    got = O.fwht(x).astype(np.float64)
    want = x.astype(np.float64) @ scipy.linalg.hadamard(n).T / math.sqrt(n)
    err = np.linalg.norm(got - want, axis=1) / np.linalg.norm(want, axis=1)
    assert np.all(err <= 1e-6)
    # orthonormal: norms preserved, applying twice returns x
    nx = np.linalg.norm(x.astype(np.float64), axis=1)
    assert np.all(np.abs(np.linalg.norm(got, axis=1) - nx) <= 1e-6 * nx)
    twice = O.fwht(O.fwht(x)).astype(np.float64)
    assert np.all(np.linalg.norm(twice - x, axis=1) <= 1e-6 * nx)


@pytest.mark.parametrize("H,B,fmt", [(16, 16, E4M3), (32, 16, E4M3), (16, 32, E8M0), (32, 32, E8M0)])
def test_quantize_rotates_aligned_segments(O, H, B, fmt):
    rng = np.random.default_rng(H + B)
    x = rng.laplace(0, 1, (6, 128)).astype(np.float32)
    rot = O.fwht(x.reshape(-1, H)).reshape(x.shape)
    gm = 1 if fmt == E4M3 else 0
    a = O.quantize(x, fmt=fmt, block=B, strategy=0, global_mode=gm, hadamard=H)
    b = O.quantize(rot, fmt=fmt, block=B, strategy=0, global_mode=gm, hadamard=0)
    for k in ("codes", "scales", "dequant", "mse"):
        assert np.array_equal(a[k], b[k]), k
    assert a["g"] == b["g"]
    if fmt == E4M3:
        assert a["g"] == O.global_scale(rot)           # the tensor scale sees rotated values
    m = O.block_mse(x, a["codes"], a["scales"], a["g"], fmt=fmt, block=B, hadamard=H)
    assert np.array_equal(m, a["mse"])


def test_rotation_gaussianises_laplace_blocks(O):
    """Soft check of the distribution model (Laplace before, near-Gaussian
    after the block Hadamard): excess kurtosis drops toward 0."""
    rng = np.random.default_rng(0)
    x = rng.laplace(0, 1, (512, 256)).astype(np.float32)
    r = O.fwht(x.reshape(-1, 32)).reshape(x.shape).astype(np.float64)

    def kurt(v):
        v = v - v.mean()
        return (v ** 4).mean() / (v ** 2).mean() ** 2 - 3.0

    k0, k1 = kurt(x.astype(np.float64)), kurt(r)
    assert k0 > 2.5 and abs(k1) < 0.5
