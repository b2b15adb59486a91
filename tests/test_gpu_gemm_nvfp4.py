"""GPU parity of the NVFP4 GEMM (operands decoded to fp16 on the way to the
fp16 matrix cores) against the oracle's fp64 product C = dq(A) dq(B)^T,
dq the NVFP4 decode fp4q_dequantize applies (E2M1 value times fl(dec(s) g)).

Tolerance, from the arithmetic: the kernel's operand values grid * dec(s)
are exact in fp16 and their products exact in fp32; one matrix-core
instruction adds the 16 products of a 16-wide K substep to the running fp32
sum (a pairwise sum of depth 4, then the running sum: K/16 + 5 roundings of
at most 2^-24 relative to the sum of |products|, doubled as margin).  The
definition's values carry the roundings of fl(dec g) and fl(grid S) (four
per product) and the kernel multiplies the sum by fl(g_a g_b) once (two
more): |C_gpu - C| <= (2 (K/16 + 5) + 6) 2^-24 sum_k |a_k b_k|, for scaled
values in fp32's normal range.  bf16 output adds 2^-8 relative."""
import numpy as np
import pytest
import torch

from microscaling_fp4_block_fp4q_amd import fp4q as F
from microscaling_fp4_block_fp4q_amd import synth as S
from oracle import oracle as O

from gpu_helpers import DEV, note

pytestmark = pytest.mark.gpu

E4M3 = 1


def operands(seed, M, N, K, lo=0x10, hi=0x60):
    """Random codes; E4M3 scale codes in [lo, hi) (subnormal codes below 8)."""
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    b = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sa = rng.integers(lo, hi, (M, K // 16)).astype(np.uint8)
    sb = rng.integers(lo, hi, (N, K // 16)).astype(np.uint8)
    return a, sa, b, sb


def abs_product(a, sa, ga, b, sb, gb):
    K = a.shape[1] * 2
    A = O.dequantize(a, sa, ga, fmt=E4M3, block=16, rows=a.shape[0], cols=K).astype(np.float64)
    B = O.dequantize(b, sb, gb, fmt=E4M3, block=16, rows=b.shape[0], cols=K).astype(np.float64)
    return np.abs(A) @ np.abs(B).T


def g_tensor(g):
    return None if g is None else torch.tensor([g], dtype=torch.float32, device=DEV)


def run_gpu(a, sa, ga, b, sb, gb, out=torch.float32):
    ta, tsa, tb, tsb = (torch.from_numpy(v).to(DEV) for v in (a, sa, b, sb))
    c = F.nvfp4_gemm(ta, tsa, g_tensor(ga), tb, tsb, g_tensor(gb), out_dtype=out)
    torch.cuda.synchronize()
    return c.float().cpu().numpy().astype(np.float64)


def check(got, want, bound_abs, K, bf16=False):
    tol = (2 * (K / 16 + 5) + 6) * 2.0 ** -24 * bound_abs
    if bf16:
        tol = tol + 2.0 ** -8 * np.abs(want)
    bad = ~(np.abs(got - want) <= tol)
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:3].tolist())


def oracle(a, sa, ga, b, sb, gb):
    return O.nvfp4_gemm(a, sa, 1.0 if ga is None else ga, b, sb, 1.0 if gb is None else gb)


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (256, 256, 1024), (512, 768, 512), (96, 200, 256),
                                   (16, 16, 256), (300, 1000, 768), (256, 256, 1280), (520, 264, 2048),
                                   (2304, 2304, 256), (1, 1, 256), (1, 300, 512), (257, 1, 768),
                                   # K not a multiple of 256: operands padded to the K-step in the workspace
                                   (64, 96, 16), (100, 200, 48), (257, 130, 272), (300, 1000, 800),
                                   (128, 128, 4112), (1, 1, 16)])
def test_random_codes(O_lib, M, N, K):
    a, sa, b, sb = operands(M + N + K, M, N, K)
    ga, gb = 0.0123, 0.0371
    note(f"nvfp4 gemm random {M}x{N}x{K}")
    got = run_gpu(a, sa, ga, b, sb, gb)
    check(got, oracle(a, sa, ga, b, sb, gb), abs_product(a, sa, ga, b, sb, gb), K)


def test_every_scale_code_and_no_g(O_lib):
    """Scale codes over the whole finite E4M3 range (subnormals 1..7 and 0
    included) with g = 1 (no per-tensor scale: NULL pointers)."""
    a, sa, b, sb = operands(31, 256, 256, 512, lo=0, hi=127)
    note("nvfp4 gemm every scale code, g null")
    got = run_gpu(a, sa, None, b, sb, None)
    check(got, oracle(a, sa, None, b, sb, None), abs_product(a, sa, 1.0, b, sb, 1.0), 512)


def test_bf16_output(O_lib):
    a, sa, b, sb = operands(5, 256, 512, 256)
    note("nvfp4 gemm bf16 output")
    got = run_gpu(a, sa, 0.5, b, sb, 3.0, torch.bfloat16)
    check(got, oracle(a, sa, 0.5, b, sb, 3.0), abs_product(a, sa, 0.5, b, sb, 3.0), 256, bf16=True)


def test_nan_scale(O_lib):
    """Scale code 0x7F (NaN) in one block of A's row 3 and of B's row 10:
    that row and that column of C are NaN, the rest finite."""
    a, sa, b, sb = operands(41, 64, 64, 256)
    sa[3, 5] = 0x7F
    sb[10, 0] = 0xFF                               # the sign bit of a scale byte is ignored
    note("nvfp4 gemm NaN scales")
    got = run_gpu(a, sa, 0.25, b, sb, 0.25)
    want = oracle(a, sa, 0.25, b, sb, 0.25)
    assert np.all(np.isnan(got[3])) and np.all(np.isnan(got[:, 10]))
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    check(got[ok], want[ok], abs_product(a, np.where(sa == 0x7F, 0x38, sa), 0.25,
                                         b, np.where(sb == 0xFF, 0x38, sb), 0.25)[ok], 256)


def test_quantized_llm_shapes(O_lib):
    """Activations [tokens, hidden] times an MLP weight [out, in], both
    quantized to NVFP4 (tensor-amax g, 4-over-6 for the weight) by the
    library; the oracle's product on sampled rows, with the g's the
    quantizer wrote."""
    x = S.laplace(512, 4096, 15)
    w = S.normal(1024, 4096, 16) * np.float32(0.02)
    note("nvfp4 gemm of library-quantized 512x4096 and 1024x4096")
    qa = F.quantize(S.to_torch(x, S.F32, DEV), F.nvfp4(), want_mse=False)
    qb = F.quantize(S.to_torch(w.astype(np.float32), S.F32, DEV), F.nvfp4(F.FOUR_OVER_SIX), want_mse=False)
    c = F.nvfp4_gemm(qa["codes"], qa["scales"], qa["g"], qb["codes"], qb["scales"], qb["g"])
    torch.cuda.synchronize()
    a, sa = qa["codes"].cpu().numpy(), qa["scales"].cpu().numpy()
    b, sb = qb["codes"].cpu().numpy(), qb["scales"].cpu().numpy()
    ga, gb = float(qa["g"].item()), float(qb["g"].item())
    rows = np.array([0, 1, 255, 511])
    want = O.nvfp4_gemm(a[rows], sa[rows], ga, b, sb, gb)
    check(c.cpu().numpy().astype(np.float64)[rows], want, abs_product(a[rows], sa[rows], ga, b, sb, gb), 4096)


def test_ragged_n_padded_ldc(O_lib):
    M, N, K = 70, 77, 512
    a, sa, b, sb = operands(21, M, N, K)
    t = [torch.from_numpy(v).to(DEV) for v in (a, sa, b, sb)]
    want = oracle(a, sa, 2.0, b, sb, 0.125)
    bound = abs_product(a, sa, 2.0, b, sb, 0.125)
    for dt in (torch.float32, torch.bfloat16):
        note(f"nvfp4 gemm ragged N=77 ldc=80 {dt}")
        full = torch.full((M, 80), 7.0, dtype=dt, device=DEV)
        ws = torch.empty(F.nvfp4_gemm_workspace_bytes(M, N, K), dtype=torch.uint8, device=DEV)
        F.fp4q_nvfp4_gemm(t[0], t[1], g_tensor(2.0), t[2], t[3], g_tensor(0.125), full[:, :N], ws)
        torch.cuda.synchronize()
        got = full.float().cpu().numpy().astype(np.float64)
        check(got[:, :N], want, bound, K, bf16=dt == torch.bfloat16)
        assert np.all(got[:, N:] == 7.0)


def test_full_size_sampled(O_lib):
    """8192 x 8192 x 8192 with bf16 output, the shape the throughput is
    measured on: sampled rows and columns against the oracle."""
    M = N = K = 8192
    gen = torch.Generator(device=DEV).manual_seed(6)
    a = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device=DEV, generator=gen)
    b = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=DEV, generator=gen)
    sa = torch.randint(0x20, 0x48, (M, K // 16), dtype=torch.uint8, device=DEV, generator=gen)
    sb = torch.randint(0x20, 0x48, (N, K // 16), dtype=torch.uint8, device=DEV, generator=gen)
    ga, gb = 0.0071, 0.0133
    note("nvfp4 gemm 8192^3 bf16")
    c = F.nvfp4_gemm(a, sa, g_tensor(ga), b, sb, g_tensor(gb), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 2047, 4100, 8191])
    cols = np.array([0, 255, 256, 5000, 8191])
    an, san, bn, sbn = (v.cpu().numpy() for v in (a, sa, b, sb))
    got = c.float().cpu().numpy().astype(np.float64)
    check(got[rows], O.nvfp4_gemm(an[rows], san[rows], ga, bn, sbn, gb),
          abs_product(an[rows], san[rows], ga, bn, sbn, gb), K, bf16=True)
    check(got[:, cols], O.nvfp4_gemm(an, san, ga, bn[cols], sbn[cols], gb),
          abs_product(an, san, ga, bn[cols], sbn[cols], gb), K, bf16=True)


def test_empty_and_validation(O_lib):
    L = F.lib()
    z = torch.zeros(64, dtype=torch.uint8, device=DEV)
    g = torch.ones(2, dtype=torch.float32, device=DEV)
    c = torch.zeros((4, 4), dtype=torch.float32, device=DEV)
    ws = torch.empty(F.nvfp4_gemm_workspace_bytes(4, 4, 256), dtype=torch.uint8, device=DEV)
    p = lambda t: t.data_ptr()
    gp = p(g)
    call = lambda M, K, dt, ldc, w, ga=gp: L.fp4q_nvfp4_gemm(p(z), p(z), ga, p(z), p(z), gp, M, 4, K, p(c), dt, ldc,
                                                              w, None)
    assert call(0, 256, F.F32, 4, p(ws)) == F.OK
    assert call(4, 40, F.F32, 4, p(ws)) == F.ERR_SHAPE
    assert call(4, 0, F.F32, 4, p(ws)) == F.ERR_SHAPE
    assert call(4, 256, F.F16, 4, p(ws)) == F.ERR_INVALID_ARG
    assert call(4, 256, F.F32, 4, None) == F.ERR_INVALID_ARG
    assert call(4, 256, F.F32, 4, p(ws) + 16) == F.ERR_ALIGNMENT
    assert call(4, 256, F.F32, 3, p(ws)) == F.ERR_SHAPE
    assert call(4, 256, F.F32, 4, p(ws), ga=gp + 2) == F.ERR_ALIGNMENT
    assert F.nvfp4_gemm_workspace_bytes(4, 4, 40) == 0
