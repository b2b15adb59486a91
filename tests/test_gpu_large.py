"""A tensor past 2^31 elements: bf16 [81920, 32768] (2.68 G values, 5.4 GB),
so element offsets of the input and of the dequantized output pass 2^31 and
their byte offsets pass 2^32 from row 65536 on.

The tensor is 20 copies of a seeded 4096-row block, copy k scaled by
2^-(k mod 4) (exact in bf16), built on the device with torch.  A row of it
is therefore known on the host without holding the whole tensor, and its
abs-max equals the block's (copies 0, 4, 8, ... are unscaled), so the
oracle's per-tensor scale of the block is the full tensor's.  Sampled rows
around the 2^31 boundary and at both ends are compared with the oracle.
"""
import numpy as np
import pytest
import torch

from microscaling_fp4_block_fp4q_amd import fp4q as F
from microscaling_fp4_block_fp4q_amd import synth as S
from oracle import oracle as O

from gpu_helpers import DEV, assert_same, note

pytestmark = pytest.mark.gpu

BASE_ROWS, COPIES, COLS = 4096, 20, 32768
ROWS = BASE_ROWS * COPIES
SAMPLE = [0, 1, 4095, 4096, 65535, 65536, 65537, 70001, ROWS - 1]


def copy_factor(r):
    return 2.0 ** -((r // BASE_ROWS) % 4)


def host_rows(base_bits, rows):
    """Rows of the large tensor as bf16 bit patterns, from the base block."""
    f = (base_bits[[r % BASE_ROWS for r in rows]].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return S.cast(f * np.array([copy_factor(r) for r in rows])[:, None], S.BF16)


def build_large(base):
    """The [ROWS, COLS] device tensor whose copy k is base * copy_factor."""
    base_dev = S.to_torch(base, S.BF16, DEV)
    x = torch.empty((ROWS, COLS), dtype=torch.bfloat16, device=DEV)
    for k in range(COPIES):
        torch.mul(base_dev, copy_factor(k * BASE_ROWS), out=x[k * BASE_ROWS:(k + 1) * BASE_ROWS])
    return x


def test_tensor_past_2_31_elements(O_lib):
    assert ROWS * COLS > 2 ** 31 and SAMPLE[5] * COLS == 2 ** 31
    base = S.normal(BASE_ROWS, COLS, 71, S.BF16)
    note(f"large tensor bf16 [{ROWS}, {COLS}]: build on the device")
    x = build_large(base)

    nv = F.nvfp4(F.FOUR_OVER_SIX)
    bf = F.config(F.E4M3, 16, F.BRUTE_FORCE, F.GLOBAL_NONE)
    note("large tensor: NVFP4 4-over-6 with the pre-pass, every output")
    c1 = torch.empty((ROWS, COLS // 2), dtype=torch.uint8, device=DEV)
    s1 = torch.empty((ROWS, COLS // 16), dtype=torch.uint8, device=DEV)
    g1 = torch.empty(1, dtype=torch.float32, device=DEV)
    dq1 = torch.empty((ROWS, COLS), dtype=torch.bfloat16, device=DEV)
    m1 = torch.empty((ROWS, COLS // 16), dtype=torch.float32, device=DEV)
    ws = torch.empty(F.workspace_bytes(nv, ROWS, COLS), dtype=torch.uint8, device=DEV)
    F.fp4q_quantize(nv, x, c1, s1, g1, dq1, m1, ws)
    torch.cuda.synchronize()
    note("large tensor: E4M3 block 16 brute force, codes and scales")
    c2 = torch.empty((ROWS, COLS // 2), dtype=torch.uint8, device=DEV)
    s2 = torch.empty((ROWS, COLS // 16), dtype=torch.uint8, device=DEV)
    F.fp4q_quantize(bf, x, c2, s2)
    torch.cuda.synchronize()
    note("large tensor: block MSE of the NVFP4 result")
    m3 = torch.empty_like(m1)
    F.fp4q_block_mse(nv, x, c1, s1, m3, g1)
    torch.cuda.synchronize()
    assert torch.equal(m3.view(torch.int32), m1.view(torch.int32)), "block MSE differs from the quantizer's"
    del m3
    note("large tensor: dequantize of the NVFP4 result")
    dq4 = torch.empty_like(dq1)
    F.fp4q_dequantize(nv, c1, s1, dq4, g1)
    torch.cuda.synchronize()
    assert torch.equal(dq4.view(torch.int16), dq1.view(torch.int16)), "dequantize differs from the quantizer's"
    del dq4, x

    got = {name: S.from_torch(t[SAMPLE]) for name, t in
           (("c1", c1), ("s1", s1), ("dq1", dq1), ("m1", m1), ("c2", c2), ("s2", s2))}
    g_full = O.tensor_global_scale(base, x_dt=S.BF16)
    assert S.from_torch(g1)[0].view(np.uint32) == np.float32(g_full).view(np.uint32), "per-tensor scale"
    xr = host_rows(base, SAMPLE)
    r1 = O.quantize(xr, x_dt=S.BF16, fmt=F.E4M3, block=16, strategy=F.FOUR_OVER_SIX, global_mode=F.GLOBAL_USER,
                    user_g=g_full, dq_dt=S.BF16)
    r2 = O.quantize(xr, x_dt=S.BF16, fmt=F.E4M3, block=16, strategy=F.BRUTE_FORCE, global_mode=F.GLOBAL_NONE,
                    dq_dt=None)
    assert_same(got["c1"], r1["codes"], "nvfp4 codes")
    assert_same(got["s1"], r1["scales"], "nvfp4 scales")
    assert_same(got["dq1"], r1["dequant"], "nvfp4 dequant")
    assert_same(got["m1"], r1["mse"], "nvfp4 mse")
    assert_same(got["c2"], r2["codes"], "brute-force codes")
    assert_same(got["s2"], r2["scales"], "brute-force scales")
    del c1, s1, dq1, m1, c2, s2, ws
    torch.cuda.empty_cache()


def test_focus_past_2_31_elements(O_lib):
    """FOCUS forward and backward (MXFP4, sub-blocks of 8) on the same kind
    of tensor, used both as W and as the upstream gradient G.  The block
    scales are seeded E8M0 codes drawn on the host for every block (the
    relaxed quantizer takes them as an input); c repeats a seeded block."""
    K = 8
    cfg = F.mxfp4()
    base = S.normal(BASE_ROWS, COLS, 72, S.BF16, sigma=0.02)
    rng = np.random.default_rng(73)
    scales = rng.integers(118, 124, (ROWS, COLS // 32), dtype=np.uint8)
    _, c_base, _ = S.focus_inputs(BASE_ROWS, 64, K, seeds=(74, 75, 76))     # c_base [4096, 8] fp16 bits
    c_base = np.tile(c_base, (1, COLS // 64))                                 # [4096, COLS / 8]
    note(f"large FOCUS bf16 [{ROWS}, {COLS}] K={K}: build on the device")
    w = build_large(base)
    c = S.to_torch(c_base, S.F16, DEV).repeat(COPIES, 1)
    st = torch.from_numpy(scales).to(DEV)
    w_hat = torch.empty_like(w)
    codes = torch.empty((ROWS, COLS // 2), dtype=torch.uint8, device=DEV)
    grad_c = torch.empty((ROWS, COLS // K), dtype=torch.float32, device=DEV)
    note("large FOCUS: forward")
    F.fp4q_relaxed_fakequant_fwd(cfg, w, st, c, K, w_hat, None, codes)
    torch.cuda.synchronize()
    note("large FOCUS: backward")
    F.fp4q_relaxed_fakequant_bwd(cfg, w, st, c, K, w, grad_c, None)
    torch.cuda.synchronize()
    got = {n: S.from_torch(t[SAMPLE]) for n, t in (("w_hat", w_hat), ("codes", codes), ("grad_c", grad_c))}
    del w, c, st, w_hat, codes, grad_c
    torch.cuda.empty_cache()
    wr = host_rows(base, SAMPLE)
    cr = c_base[[r % BASE_ROWS for r in SAMPLE]]
    rw, rc = O.relaxed_fwd(wr, scales[SAMPLE], 1.0, cr, fmt=F.E8M0, block=32, sub_block=K, w_dt=S.BF16)
    rg = O.relaxed_bwd(wr, scales[SAMPLE], 1.0, cr, wr, fmt=F.E8M0, block=32, sub_block=K, w_dt=S.BF16,
                       g_dt=S.BF16)
    assert_same(got["w_hat"], rw, "w_hat")
    assert_same(got["codes"], rc, "codes")
    assert_same(got["grad_c"], rg, "grad_c")
