"""Pins of the oracle's MXFP4 GEMM (the MR-GPTQ page, section 2.3: FP4
matrix products on the packed codes and block scales).  Checked against
numpy's fp64 matmul of the oracle's own dequantized operands (a library
primitive on an independently pinned decode), a hand-built product, and
exact integer arithmetic where all values are small integers."""
import numpy as np

E8M0 = 0


def operands(seed, M, N, K, spread=3):
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    b = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sa = (127 + rng.integers(-spread, spread + 1, (M, K // 32))).astype(np.uint8)
    sb = (127 + rng.integers(-spread, spread + 1, (N, K // 32))).astype(np.uint8)
    return a, sa, b, sb


def test_against_matmul_of_dequantized(O):
    a, sa, b, sb = operands(1, 24, 40, 256)
    A = O.dequantize(a, sa, 1.0, fmt=E8M0, block=32, rows=24, cols=256).astype(np.float64)
    B = O.dequantize(b, sb, 1.0, fmt=E8M0, block=32, rows=40, cols=256).astype(np.float64)
    C = O.mxfp4_gemm(a, sa, b, sb)
    # both are fp64 sums of the same exact products; they differ only by summation order
    bound = 256 * 2.0 ** -52 * (np.abs(A) @ np.abs(B).T)
    assert np.all(np.abs(C - A @ B.T) <= bound)


def test_small_integers_exact(O):
    """Codes with magnitudes 1..4 (grid values 0.5..2) at scale 2^1 are small
    integers; the fp64 sum of their products is exact."""
    rng = np.random.default_rng(2)
    M, N, K = 8, 8, 64
    mags = rng.integers(1, 5, (M, K))
    signs = rng.integers(0, 2, (M, K))
    q = (mags | (signs << 3)).astype(np.uint8)
    a = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    sa = np.full((M, K // 32), 128, np.uint8)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    vals = grid[mags] * np.where(signs == 1, -1, 1) * 2
    C = O.mxfp4_gemm(a, sa, a, sa)
    assert np.array_equal(C, (vals.astype(np.int64) @ vals.T.astype(np.int64)).astype(np.float64))


def test_one_hot_positions(O):
    """A single 1.0 at (m, k) in A and at (n, k) in B gives C[m][n] = 1 and
    zeros elsewhere; a different k gives all zeros (nibble order, block
    scale index and transposition)."""
    M, N, K = 4, 5, 128
    for (m, n, k, kb) in ((1, 3, 37, 37), (0, 4, 64, 65), (3, 0, 127, 127)):
        a = np.zeros((M, K // 2), np.uint8)
        b = np.zeros((N, K // 2), np.uint8)
        a[m, k // 2] = 2 << (4 * (k & 1))
        b[n, kb // 2] = 2 << (4 * (kb & 1))
        sa = np.full((M, K // 32), 127, np.uint8)
        sb = np.full((N, K // 32), 127, np.uint8)
        sa[m, k // 32] = 129                                   # 4x on A's block
        C = O.mxfp4_gemm(a, sa, b, sb)
        want = np.zeros((M, N))
        if k == kb:
            want[m, n] = 4.0
        assert np.array_equal(C, want), (m, n, k, kb)


def test_nan_scale(O):
    a, sa, b, sb = operands(3, 4, 4, 64)
    sa[2, 1] = 0xFF
    C = O.mxfp4_gemm(a, sa, b, sb)
    assert np.all(np.isnan(C[2])) and not np.any(np.isnan(np.delete(C, 2, axis=0)))


# ---------------------------------------------------------------------------
# NVFP4 operands: E4M3 scales per 16 values and a per-tensor g per operand
# ---------------------------------------------------------------------------

E4M3 = 1


def nv_operands(seed, M, N, K):
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    b = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sa = rng.integers(0, 127, (M, K // 16)).astype(np.uint8)     # every finite E4M3 code, subnormals included
    sb = rng.integers(0, 127, (N, K // 16)).astype(np.uint8)
    return a, sa, b, sb


def test_nvfp4_against_matmul_of_dequantized(O):
    a, sa, b, sb = nv_operands(4, 24, 40, 256)
    ga, gb = 0.0078125 * 1.3, 0.02
    A = O.dequantize(a, sa, ga, fmt=E4M3, block=16, rows=24, cols=256).astype(np.float64)
    B = O.dequantize(b, sb, gb, fmt=E4M3, block=16, rows=40, cols=256).astype(np.float64)
    C = O.nvfp4_gemm(a, sa, ga, b, sb, gb)
    bound = 256 * 2.0 ** -52 * (np.abs(A) @ np.abs(B).T)
    assert np.all(np.abs(C - A @ B.T) <= bound)


def test_nvfp4_small_integers_exact(O):
    """Magnitudes 1..4 (grid 0.5..2) at the E4M3 scale 2 (code 0x40) with
    g = 1 are small integers; the sum of their products is exact."""
    rng = np.random.default_rng(5)
    M, K = 8, 64
    mags = rng.integers(1, 5, (M, K))
    signs = rng.integers(0, 2, (M, K))
    q = (mags | (signs << 3)).astype(np.uint8)
    a = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    sa = np.full((M, K // 16), 0x40, np.uint8)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    vals = (grid[mags] * np.where(signs == 1, -1, 1) * 2).astype(np.int64)
    C = O.nvfp4_gemm(a, sa, 1.0, a, sa, 1.0)
    assert np.array_equal(C, (vals @ vals.T).astype(np.float64))


def test_nvfp4_one_hot_positions(O):
    """A single grid value 1 at (m, k) of A and at (n, kb) of B, the block of
    k scaled by 1.5 (code 0x3C) and g_a = 0.25: C[m][n] = 0.375 when k = kb,
    zeros otherwise (nibble order, 16-element block index, transposition)."""
    M, N, K = 4, 5, 64
    for (m, n, k, kb) in ((1, 3, 15, 15), (0, 4, 16, 16), (2, 1, 15, 16), (3, 0, 63, 63)):
        a = np.zeros((M, K // 2), np.uint8)
        b = np.zeros((N, K // 2), np.uint8)
        a[m, k // 2] = 2 << (4 * (k & 1))
        b[n, kb // 2] = 2 << (4 * (kb & 1))
        sa = np.full((M, K // 16), 0x38, np.uint8)             # 1.0
        sb = np.full((N, K // 16), 0x38, np.uint8)
        sa[m, k // 16] = 0x3C                                  # 1.5 on A's block
        C = O.nvfp4_gemm(a, sa, 0.25, b, sb, 1.0)
        want = np.zeros((M, N))
        if k == kb:
            want[m, n] = 0.375
        assert np.array_equal(C, want), (m, n, k, kb)


def test_nvfp4_equals_mxfp4_on_power_of_two_scales(O):
    """With E4M3 scales 2^j (code (j + 7) << 3) shared by both 16-blocks of
    each 32-block and g = 1, NVFP4 operands are MXFP4 operands with E8M0
    scale 127 + j: the two GEMMs (separate decodes) must agree exactly."""
    rng = np.random.default_rng(6)
    M, N, K = 12, 9, 128
    a = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    b = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    ja = rng.integers(-5, 6, (M, K // 32))
    jb = rng.integers(-5, 6, (N, K // 32))
    C_nv = O.nvfp4_gemm(a, np.repeat((ja + 7) << 3, 2, axis=1).astype(np.uint8), 1.0,
                        b, np.repeat((jb + 7) << 3, 2, axis=1).astype(np.uint8), 1.0)
    C_mx = O.mxfp4_gemm(a, (127 + ja).astype(np.uint8), b, (127 + jb).astype(np.uint8))
    assert np.array_equal(C_nv, C_mx)


def test_nvfp4_nan_scale(O):
    a, sa, b, sb = nv_operands(7, 4, 4, 64)
    sb[1, 2] = 0x7F
    C = O.nvfp4_gemm(a, sa, 1.0, b, sb, 1.0)
    assert np.all(np.isnan(C[:, 1])) and not np.any(np.isnan(np.delete(C, 1, axis=1)))
