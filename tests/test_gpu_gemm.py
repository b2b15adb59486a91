"""GPU parity of the MXFP4 GEMM (block-scaled matrix cores) against the
oracle's fp64 product C = dq(A) dq(B)^T.

Tolerance, from the arithmetic: every product of two decoded MXFP4 values
is exact in fp32 (at most 2 x 2 significant bits times a power of two);
one matrix-core instruction adds the 64 products of a 64-wide K substep to
the running fp32 sum.  Allowing for an internal pairwise sum rounded at
every level (depth 7 with the running sum) plus one rounding of the running
sum per substep: |C_gpu - C| <= (K/64 + 8) * 2^-24 * sum_k |a_k b_k|; the
test allows twice that.  bf16 output adds the final rounding (2^-8
relative)."""
import numpy as np
import pytest
import torch

from microscaling_fp4_block_fp4q_amd import fp4q as F
from microscaling_fp4_block_fp4q_amd import synth as S
from oracle import oracle as O

from gpu_helpers import DEV, note

pytestmark = pytest.mark.gpu


def operands(seed, M, N, K, spread=4):
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    b = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sa = (127 + rng.integers(-spread, spread + 1, (M, K // 32))).astype(np.uint8)
    sb = (127 + rng.integers(-spread, spread + 1, (N, K // 32))).astype(np.uint8)
    return a, sa, b, sb


def abs_product(a, sa, b, sb):
    K = a.shape[1] * 2
    A = O.dequantize(a, sa, 1.0, fmt=0, block=32, rows=a.shape[0], cols=K).astype(np.float64)
    B = O.dequantize(b, sb, 1.0, fmt=0, block=32, rows=b.shape[0], cols=K).astype(np.float64)
    return np.abs(A) @ np.abs(B).T


def run_gpu(a, sa, b, sb, out=torch.float32):
    t = [torch.from_numpy(v).to(DEV) for v in (a, sa, b, sb)]
    c = F.mxfp4_gemm(*t, out_dtype=out)
    torch.cuda.synchronize()
    return c.float().cpu().numpy().astype(np.float64)


def check(got, want, bound_abs, K, bf16=False):
    tol = 2 * (K / 64 + 8) * 2.0 ** -24 * bound_abs
    if bf16:
        tol = tol + 2.0 ** -8 * np.abs(want)
    bad = np.abs(got - want) > tol
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:3].tolist())


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (256, 256, 1024), (512, 768, 512), (96, 200, 256),
                                   (16, 16, 256), (300, 1000, 768), (256, 256, 1280), (128, 512, 1792),
                                   (520, 264, 2048), (640, 1000, 256), (2700, 600, 256), (2304, 2304, 256),
                                   (1, 1, 256), (1, 300, 512), (257, 1, 768),
                                   # K not a multiple of 256: operands padded to the K-step in the workspace
                                   (64, 96, 32), (100, 200, 96), (257, 130, 288), (300, 1000, 800),
                                   (128, 128, 4128), (1, 1, 32)])
def test_random_codes(O_lib, M, N, K):
    a, sa, b, sb = operands(M + N + K, M, N, K)
    note(f"gemm random {M}x{N}x{K}")
    got = run_gpu(a, sa, b, sb)
    want = O.mxfp4_gemm(a, sa, b, sb)
    check(got, want, abs_product(a, sa, b, sb), K)


def test_bf16_output(O_lib):
    a, sa, b, sb = operands(5, 256, 512, 256)
    note("gemm bf16 output")
    got = run_gpu(a, sa, b, sb, torch.bfloat16)
    want = O.mxfp4_gemm(a, sa, b, sb)
    check(got, want, abs_product(a, sa, b, sb), 256, bf16=True)


def test_quantized_llm_shapes(O_lib):
    """Activations [tokens, hidden] times an MLP weight [out, in], both
    quantized to MXFP4 by the library; the oracle's product on sampled rows."""
    x = S.laplace(512, 4096, 5)
    w = S.normal(1024, 4096, 6) * np.float32(0.02)
    note("gemm of library-quantized 512x4096 and 1024x4096")
    qa = F.quantize(S.to_torch(x, S.F32, DEV), F.mxfp4(), want_mse=False)
    qb = F.quantize(S.to_torch(w.astype(np.float32), S.F32, DEV), F.mxfp4(), want_mse=False)
    c = F.mxfp4_gemm(qa["codes"], qa["scales"], qb["codes"], qb["scales"])
    torch.cuda.synchronize()
    a, sa = qa["codes"].cpu().numpy(), qa["scales"].cpu().numpy()
    b, sb = qb["codes"].cpu().numpy(), qb["scales"].cpu().numpy()
    rows = np.array([0, 1, 255, 511])
    want = O.mxfp4_gemm(a[rows], sa[rows], b, sb)
    check(c.cpu().numpy().astype(np.float64)[rows], want, abs_product(a[rows], sa[rows], b, sb), 4096)


def test_wide_scale_range(O_lib):
    a, sa, b, sb = operands(9, 256, 256, 512, spread=40)
    note("gemm wide scale range")
    check(run_gpu(a, sa, b, sb), O.mxfp4_gemm(a, sa, b, sb), abs_product(a, sa, b, sb), 512)


def test_ragged_n_padded_ldc(O_lib):
    """N = 77 (not a whole 16-byte chunk of either output type) through a
    padded C [M, 80]: the edge chunks are stored element by element and the
    padding columns are left alone."""
    M, N, K = 70, 77, 512
    a, sa, b, sb = operands(21, M, N, K)
    t = [torch.from_numpy(v).to(DEV) for v in (a, sa, b, sb)]
    want = O.mxfp4_gemm(a, sa, b, sb)
    bound = abs_product(a, sa, b, sb)
    for dt in (torch.float32, torch.bfloat16):
        note(f"gemm ragged N=77 ldc=80 {dt}")
        full = torch.full((M, 80), 7.0, dtype=dt, device=DEV)
        F.fp4q_mxfp4_gemm(*t, full[:, :N], F.gemm_workspace(M, N, K, DEV))
        torch.cuda.synchronize()
        got = full.float().cpu().numpy().astype(np.float64)
        check(got[:, :N], want, bound, K, bf16=dt == torch.bfloat16)
        assert np.all(got[:, N:] == 7.0)


def test_full_size_sampled(O_lib):
    """8192 x 8192 x 8192 with bf16 output, the shape the throughput is
    measured on: sampled rows and columns against the oracle."""
    M = N = K = 8192
    gen = torch.Generator(device=DEV).manual_seed(5)
    a = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device=DEV, generator=gen)
    b = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=DEV, generator=gen)
    sa = torch.randint(123, 132, (M, K // 32), dtype=torch.uint8, device=DEV, generator=gen)
    sb = torch.randint(123, 132, (N, K // 32), dtype=torch.uint8, device=DEV, generator=gen)
    note("gemm 8192^3 bf16")
    c = F.mxfp4_gemm(a, sa, b, sb, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 2047, 4100, 8191])
    cols = np.array([0, 255, 256, 5000, 8191])
    an, san, bn, sbn = (v.cpu().numpy() for v in (a, sa, b, sb))
    got = c.float().cpu().numpy().astype(np.float64)
    want_r = O.mxfp4_gemm(an[rows], san[rows], bn, sbn)
    check(got[rows], want_r, abs_product(an[rows], san[rows], bn, sbn), K, bf16=True)
    want_c = O.mxfp4_gemm(an, san, bn[cols], sbn[cols])
    check(got[:, cols], want_c, abs_product(an, san, bn[cols], sbn[cols]), K, bf16=True)


def test_empty_and_validation(O_lib):
    L = F.lib()
    z = torch.zeros(64, dtype=torch.uint8, device=DEV)
    c = torch.zeros((4, 4), dtype=torch.float32, device=DEV)
    ws = F.gemm_workspace(4, 4, 256, DEV)
    p = lambda t: t.data_ptr()
    assert L.fp4q_mxfp4_gemm(p(z), p(z), p(z), p(z), 0, 4, 256, p(c), F.F32, 4, p(ws), None) == F.OK
    assert L.fp4q_mxfp4_gemm(p(z), p(z), p(z), p(z), 4, 4, 48, p(c), F.F32, 4, p(ws), None) == F.ERR_SHAPE
    assert L.fp4q_mxfp4_gemm(p(z), p(z), p(z), p(z), 4, 4, 0, p(c), F.F32, 4, p(ws), None) == F.ERR_SHAPE
    assert L.fp4q_mxfp4_gemm(p(z), p(z), p(z), p(z), 4, 4, 256, p(c), F.F16, 4, p(ws), None) == F.ERR_INVALID_ARG
    assert L.fp4q_mxfp4_gemm(p(z), p(z), p(z), p(z), 4, 4, 256, p(c), F.F32, 4, None, None) == F.ERR_INVALID_ARG
    assert L.fp4q_mxfp4_gemm(p(z), p(z), p(z), p(z), 4, 4, 256, p(c), F.F32, 4, p(ws) + 16, None) == \
        F.ERR_ALIGNMENT
    assert L.fp4q_mxfp4_gemm(p(z), p(z), p(z), p(z), 4, 4, 256, p(c), F.F32, 3, p(ws), None) == F.ERR_SHAPE


def test_operand_at_the_size_limit(O_lib):
    """A's codes one row short of 2^32 bytes (M = 2^20 - 1 at K = 8192; one
    more row is refused): the direct loads' 32-bit buffer offsets reach their
    top and the last tile of rows is ragged.  A's codes are 256 copies of a
    seeded 4096-row block, built on the device; its scales are drawn for
    every row.  Sampled rows of C are compared with the oracle."""
    M, N, K = (1 << 20) - 1, 256, 8192
    assert M * (K // 2) < 2 ** 32 <= (M + 1) * (K // 2)
    rng = np.random.default_rng(81)
    base = rng.integers(0, 256, (4096, K // 2), dtype=np.uint8)
    sa = rng.integers(127 - 4, 127 + 5, (M, K // 32), dtype=np.uint8)
    _, _, b, sb = operands(82, 1, N, K)
    note(f"gemm at the operand size limit {M}x{N}x{K}")
    a_dev = torch.from_numpy(base).to(DEV).repeat(256, 1)[:M]
    t = [a_dev] + [torch.from_numpy(v).to(DEV) for v in (sa, b, sb)]
    c = F.mxfp4_gemm(*t, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = [0, 1, 4095, 4096, 1 << 19, M - 256, M - 255, M - 2, M - 1]
    got = c[rows].cpu().numpy().astype(np.float64)
    del a_dev, t, c
    torch.cuda.empty_cache()
    a_rows = base[[r % 4096 for r in rows]]
    want = O.mxfp4_gemm(a_rows, sa[rows], b, sb)
    check(got, want, abs_product(a_rows, sa[rows], b, sb), K)
