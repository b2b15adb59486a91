"""The C ABI of libfp4q.so without a GPU: it loads, exports every function
include/fp4q.h declares, and rejects bad arguments synchronously with the
documented status codes before anything is launched.

The pointers passed here are fake host addresses; every call below must be
rejected by host-side validation, so no kernel ever sees them.  To keep it
that way on a machine with a GPU, the validation cases only run where no
GPU device node exists.
"""
import ctypes
import os
import re

import pytest

from microscaling_fp4_block_fp4q_amd import fp4q as F

HAVE_LIB = os.path.exists(F.LIB_PATH)
NO_GPU = not os.path.exists("/dev/kfd")
needs_lib = pytest.mark.skipif(not HAVE_LIB, reason="libfp4q.so not built")
cpu_only = pytest.mark.skipif(not NO_GPU, reason="fake-pointer validation runs only without a GPU")

P = ctypes.c_void_p
A = 0x10000          # a 16-byte-aligned fake address, never dereferenced


@needs_lib
def test_library_exports_every_declared_symbol():
    L = F.lib()
    names = F.declared_entry_points()
    assert set(names) >= {"fp4q_quantize", "fp4q_dequantize", "fp4q_block_mse", "fp4q_scale_search",
                          "fp4q_relaxed_fakequant_fwd", "fp4q_relaxed_fakequant_bwd",
                          "fp4q_abi_version", "fp4q_status_string", "fp4q_workspace_bytes"}
    for n in names:
        assert hasattr(L, n), n


@needs_lib
def test_version_strings_workspace():
    hdr = open(F.HEADER).read()
    declared = int(re.search(r"#define FP4Q_ABI_VERSION (\d+)", hdr).group(1))
    assert F.abi_version() == declared == F.ABI_VERSION
    for s in range(7):
        assert F.status_string(s) and F.status_string(s) != "unknown status"
    assert F.status_string(99) == "unknown status"
    assert F.workspace_bytes(F.nvfp4(), 4096, 4096) >= 4
    assert F.workspace_bytes(F.mxfp4(), 4096, 4096) == 0
    # search: abs-max partials + 32 fp64 sums per tile of 64 units (fp32: 4 elements per unit at
    # block 4) + one reduction level
    tiles = 4096 * 4096 // 4 // 64
    want = 4096 + 32 * 8 * (tiles + (tiles + 511) // 512)
    assert F.workspace_bytes(F.config(F.E4M3, 4, F.ABSMAX, F.GLOBAL_SEARCH), 4096, 4096) == want
    assert F.workspace_bytes(F.config(F.E4M3, 16, F.ABSMAX, F.GLOBAL_SEARCH), 0, 64) == 4096
    assert F.lib().fp4q_workspace_bytes(None, 1, 1) == 0


def quant(cfg, x=A, x_dt=F.F32, rows=16, cols=64, ld=64, codes=A, scales=A, g=A, dq=None, dq_dt=F.F32,
          ld_dq=64, mse=None, ws=A):
    return F.lib().fp4q_quantize(ctypes.byref(cfg) if cfg is not None else None, P(x), x_dt, rows, cols, ld,
                                 P(codes), P(scales), P(g), P(dq), dq_dt, ld_dq, P(mse), P(ws), None)


@needs_lib
@cpu_only
def test_quantize_validation():
    nv = F.nvfp4()
    assert quant(None) == F.ERR_INVALID_ARG
    bad = F.nvfp4()
    bad.struct_size = 4
    assert quant(bad) == F.ERR_INVALID_ARG
    assert quant(F.config(1, 12)) == F.ERR_SHAPE                       # block 12
    assert quant(F.config(1, 16, 7)) == F.ERR_INVALID_ARG                        # strategy
    assert quant(F.config(5, 16)) == F.ERR_INVALID_ARG                           # scale format
    assert quant(F.config(1, 16, 0, 9)) == F.ERR_INVALID_ARG                     # global mode
    assert quant(F.config(1, 16, hadamard=-16)) == F.ERR_INVALID_ARG
    assert quant(F.config(1, 16, hadamard=64)) == F.ERR_UNSUPPORTED
    assert quant(F.config(1, 16, hadamard=8)) == F.ERR_UNSUPPORTED
    assert quant(F.config(0, 32, 0, F.GLOBAL_TENSOR_AMAX)) == F.ERR_UNSUPPORTED  # E8M0 + g
    assert quant(F.config(0, 32, F.FOUR_OVER_SIX)) == F.ERR_UNSUPPORTED          # E8M0 + 4/6
    assert quant(F.config(0, 32, 0, F.GLOBAL_SEARCH)) == F.ERR_UNSUPPORTED       # E8M0 + search
    assert quant(F.config(F.UE5M3, 16, 0, F.GLOBAL_TENSOR_AMAX)) == F.ERR_UNSUPPORTED
    assert quant(F.config(F.UE5M3, 16, 0, F.GLOBAL_SEARCH)) == F.ERR_UNSUPPORTED
    assert quant(F.config(1, 16, F.GIVEN, F.GLOBAL_SEARCH)) == F.ERR_UNSUPPORTED
    assert quant(F.config(1, 16, 0, F.GLOBAL_SEARCH), g=0) == F.ERR_INVALID_ARG  # writes g
    assert quant(F.config(1, 16, 0, F.GLOBAL_SEARCH), ws=0) == F.ERR_INVALID_ARG # needs workspace
    for gs in (0.0, -1.0, float("inf"), float("nan"), 1e-39, 1e36):
        assert quant(F.config(1, 16, 0, F.GLOBAL_USER, gs)) == F.ERR_INVALID_ARG, gs
    assert quant(nv, x=0) == F.ERR_INVALID_ARG
    assert quant(nv, codes=0) == F.ERR_INVALID_ARG
    assert quant(nv, scales=0) == F.ERR_INVALID_ARG
    assert quant(nv, g=0) == F.ERR_INVALID_ARG                                   # TENSOR_AMAX writes g
    assert quant(nv, ws=0) == F.ERR_INVALID_ARG                                  # needs workspace
    assert quant(nv, x_dt=7) == F.ERR_INVALID_ARG
    assert quant(nv, rows=-1) == F.ERR_INVALID_ARG
    assert quant(nv, cols=40, ld=40) == F.ERR_SHAPE                              # 40 % 16
    assert quant(F.config(1, 16, hadamard=32), cols=48, ld=48) == F.ERR_SHAPE     # 48 % 32
    assert quant(nv, ld=32) == F.ERR_SHAPE                                       # ld < cols
    assert quant(nv, x=A + 4) == F.ERR_ALIGNMENT
    assert quant(nv, codes=A + 8) == F.ERR_ALIGNMENT
    assert quant(nv, ld=66) == F.ERR_ALIGNMENT                                   # 66 * 4 % 16
    assert quant(F.config(1, 4), x_dt=F.BF16, cols=4, ld=8) == F.ERR_ALIGNMENT    # 4 bf16 = 8 bytes
    assert quant(nv, dq=A, dq_dt=9) == F.ERR_INVALID_ARG
    assert quant(nv, dq=A, ld_dq=8) == F.ERR_SHAPE
    assert quant(nv, dq=A + 2) == F.ERR_ALIGNMENT
    assert quant(nv, mse=A + 4) == F.ERR_ALIGNMENT


@needs_lib
@cpu_only
def test_histogram_validation():
    L = F.lib()
    assert L.fp4q_code_histogram(P(A), 4, 64, None, None) == F.ERR_INVALID_ARG
    assert L.fp4q_code_histogram(None, 4, 64, P(A), None) == F.ERR_INVALID_ARG
    assert L.fp4q_code_histogram(P(A), -1, 64, P(A), None) == F.ERR_INVALID_ARG
    assert L.fp4q_code_histogram(P(A), 4, 63, P(A), None) == F.ERR_SHAPE
    assert L.fp4q_code_histogram(P(A + 4), 4, 64, P(A), None) == F.ERR_ALIGNMENT
    assert L.fp4q_code_histogram(P(A), 4, 64, P(A + 4), None) == F.ERR_ALIGNMENT


def quant_hist(cfg, counts=A, x=A, rows=16, cols=64, ld=64, codes=A, scales=A, g=A, ws=A):
    return F.lib().fp4q_quantize_histogram(ctypes.byref(cfg) if cfg is not None else None, P(x), F.F32, rows,
                                           cols, ld, P(codes), P(scales), P(g), None, F.F32, cols, None,
                                           P(counts), P(ws), None)


@needs_lib
@cpu_only
def test_quantize_histogram_validation():
    """The quantize call with fused code counts: counts is required and
    8-byte aligned; the rest is checked as for fp4q_quantize."""
    nv = F.nvfp4()
    assert quant_hist(None) == F.ERR_INVALID_ARG
    assert quant_hist(nv, counts=0) == F.ERR_INVALID_ARG
    assert quant_hist(nv, counts=A + 4) == F.ERR_ALIGNMENT
    assert quant_hist(nv, codes=0) == F.ERR_INVALID_ARG
    assert quant_hist(F.config(1, 12)) == F.ERR_SHAPE
    assert quant_hist(nv, x=A + 4) == F.ERR_ALIGNMENT
    assert quant_hist(nv, ws=0) == F.ERR_INVALID_ARG                 # TENSOR_AMAX needs the workspace


@needs_lib
@cpu_only
def test_gemm_validation_and_workspace():
    L = F.lib()
    W = F.mxfp4_gemm_workspace_bytes
    # per operand: ceil(rows / 32) fragments x K / 256 steps x 64 lanes x 4 bytes, each part 256-byte aligned
    assert W(8192, 8192, 8192) == 2 * (8192 // 32) * 32 * 256
    assert W(33, 1, 256) == 2 * 256 + 256
    assert W(4, 4, 48) == 0 and W(0, 4, 256) == 0 and W(4, 4, 0) == 0
    # K not a multiple of 256: rearranged scales for K rounded up to 512, then the padded copies of
    # codes (rows x 256 bytes) and scales (rows x 16 bytes), every part 256-byte aligned
    assert W(33, 1, 288) == (1024 + 512) + (8448 + 256) + (768 + 256)

    def g(M=4, N=4, K=256, a=A, sa=A, b=A, sb=A, c=A, dt=F.F32, ldc=4, ws=A):
        return L.fp4q_mxfp4_gemm(P(a), P(sa), P(b), P(sb), M, N, K, P(c), dt, ldc, P(ws), None)
    assert g(M=0) == F.OK and g(N=0) == F.OK                                     # empty: nothing to do
    assert g(M=-1) == F.ERR_INVALID_ARG
    assert g(dt=F.F16) == F.ERR_INVALID_ARG
    assert g(K=48) == F.ERR_SHAPE and g(K=16) == F.ERR_SHAPE and g(K=0) == F.ERR_SHAPE
    assert g(ldc=3) == F.ERR_SHAPE
    assert g(M=1 << 24, K=1 << 9) == F.ERR_SHAPE                                 # M * K / 2 = 2^32 bytes
    assert g(M=1 << 24, K=480) == F.ERR_SHAPE                                    # K runs padded to 512
    assert g(ws=0) == F.ERR_INVALID_ARG and g(a=0) == F.ERR_INVALID_ARG and g(sb=0) == F.ERR_INVALID_ARG
    assert g(ws=A + 16) == F.ERR_ALIGNMENT
    assert g(a=A + 8) == F.ERR_ALIGNMENT and g(sa=A + 2) == F.ERR_ALIGNMENT
    assert g(c=A + 4) == F.ERR_ALIGNMENT
    assert g(ldc=6) == F.ERR_ALIGNMENT                                           # 6 * 4 % 16
    assert g(dt=F.BF16, ldc=4) == F.ERR_ALIGNMENT                                # 4 * 2 % 16


@needs_lib
@cpu_only
def test_nvfp4_gemm_validation_and_workspace():
    L = F.lib()
    W = F.nvfp4_gemm_workspace_bytes
    # per operand: ceil(rows / 32) fragments x K / 256 steps x 64 lanes x 8 bytes, each part 256-byte aligned
    assert W(8192, 8192, 8192) == 2 * (8192 // 32) * 32 * 512
    assert W(33, 1, 256) == 2 * 512 + 512
    assert W(4, 4, 40) == 0 and W(0, 4, 256) == 0 and W(4, 4, 0) == 0
    # K = 272: rearranged scales for K rounded up to 512, then the padded copies of codes (rows x 256
    # bytes) and scales (rows x 32 bytes), every part 256-byte aligned
    assert W(33, 1, 272) == (2048 + 1024) + (8448 + 256) + (1280 + 256)

    def g(M=4, N=4, K=256, a=A, sa=A, ga=A, b=A, sb=A, gb=A, c=A, dt=F.F32, ldc=4, ws=A):
        return L.fp4q_nvfp4_gemm(P(a), P(sa), P(ga), P(b), P(sb), P(gb), M, N, K, P(c), dt, ldc, P(ws), None)
    assert g(M=0) == F.OK and g(N=0) == F.OK
    assert g(M=-1) == F.ERR_INVALID_ARG
    assert g(dt=F.F16) == F.ERR_INVALID_ARG
    assert g(K=40) == F.ERR_SHAPE and g(K=8) == F.ERR_SHAPE and g(K=0) == F.ERR_SHAPE
    assert g(ldc=3) == F.ERR_SHAPE
    assert g(M=1 << 24, K=1 << 9) == F.ERR_SHAPE
    assert g(M=1 << 24, K=496) == F.ERR_SHAPE                                    # K runs padded to 512
    assert g(ws=0) == F.ERR_INVALID_ARG and g(a=0) == F.ERR_INVALID_ARG and g(sb=0) == F.ERR_INVALID_ARG
    assert g(ws=A + 16) == F.ERR_ALIGNMENT
    assert g(a=A + 8) == F.ERR_ALIGNMENT and g(sa=A + 2) == F.ERR_ALIGNMENT and g(gb=A + 2) == F.ERR_ALIGNMENT
    assert g(c=A + 4) == F.ERR_ALIGNMENT
    assert g(ldc=6) == F.ERR_ALIGNMENT


@needs_lib
@cpu_only
def test_other_entry_points_validation():
    L = F.lib()
    nv, mx = F.nvfp4(), F.mxfp4()
    r = ctypes.byref
    # scale search rejects GIVEN
    assert L.fp4q_scale_search(r(F.nvfp4(F.GIVEN)), P(A), 0, 16, 64, 64, P(A), P(A), None, P(A), None) == F.ERR_INVALID_ARG
    # dequantize
    assert L.fp4q_dequantize(r(nv), None, P(A), None, 16, 64, P(A), 0, 64, None) == F.ERR_INVALID_ARG
    assert L.fp4q_dequantize(r(mx), P(A), P(A), P(A), 16, 64, P(A), 0, 64, None) == F.ERR_UNSUPPORTED   # g with E8M0
    assert L.fp4q_dequantize(r(nv), P(A), P(A), None, 16, 72, P(A), 0, 72, None) == F.ERR_SHAPE
    assert L.fp4q_dequantize(r(nv), P(A), P(A), None, 16, 64, P(A + 4), 0, 64, None) == F.ERR_ALIGNMENT
    # block mse
    assert L.fp4q_block_mse(r(nv), P(A), 0, 16, 64, 64, P(A), P(A), None, None, None) == F.ERR_INVALID_ARG
    # relaxed fwd / bwd
    fwd, bwd = L.fp4q_relaxed_fakequant_fwd, L.fp4q_relaxed_fakequant_bwd
    assert fwd(r(F.mxfp4(hadamard=32)), P(A), 0, 16, 64, 64, P(A), None, P(A), 8, P(A), 0, 64, None, None) == F.ERR_UNSUPPORTED
    assert fwd(r(mx), P(A), 0, 16, 64, 64, P(A), None, P(A), 6, P(A), 0, 64, None, None) == F.ERR_SHAPE
    assert fwd(r(nv), P(A), 0, 16, 64, 64, P(A), None, P(A), 32, P(A), 0, 64, None, None) == F.ERR_SHAPE  # 16 % 32
    assert fwd(r(mx), P(A), 0, 16, 64, 64, P(A), None, None, 8, P(A), 0, 64, None, None) == F.ERR_INVALID_ARG
    assert fwd(r(mx), P(A), 0, 16, 64, 64, P(A), None, P(A), 8, None, 0, 64, None, None) == F.ERR_INVALID_ARG
    assert bwd(r(mx), P(A), 0, 16, 64, 64, P(A), None, P(A), 8, P(A), 0, 64, None, None) == F.ERR_INVALID_ARG
    assert bwd(r(mx), P(A), 0, 16, 64, 64, P(A), None, P(A), 8, None, 0, 64, P(A), None) == F.ERR_INVALID_ARG


def test_binding_refuses_to_run_without_library(monkeypatch, tmp_path):
    """The product path has no fallback: a missing library is an error."""
    monkeypatch.setattr(F, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(F, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        F.lib()


def quant_noalloc(cfg, x=A, x_dt=F.F32, rows=16, cols=64, ld=64, codes=A, scales=A, g=A, dq=None, dq_dt=F.F32,
                  ld_dq=64, mse=None):
    return F.lib().fp4q_quantize_noalloc(ctypes.byref(cfg) if cfg is not None else None, P(x), x_dt, rows, cols,
                                         ld, P(codes), P(scales), P(g), P(dq), dq_dt, ld_dq, P(mse), None)


@needs_lib
@cpu_only
def test_quantize_noalloc_validation():
    """The allocation-free quantize: the same argument checks, and a
    workspace beyond the static scratch (16 MiB) is refused before any
    device call."""
    assert quant_noalloc(None) == F.ERR_INVALID_ARG
    assert quant_noalloc(F.config(1, 12)) == F.ERR_SHAPE
    assert quant_noalloc(F.nvfp4(), codes=0) == F.ERR_INVALID_ARG
    assert quant_noalloc(F.nvfp4(), x=A + 4) == F.ERR_ALIGNMENT
    search = F.config(F.E4M3, 4, F.ABSMAX, F.GLOBAL_SEARCH)
    assert F.workspace_bytes(search, 8192, 8192) > 16 << 20
    assert quant_noalloc(search, rows=8192, cols=8192, ld=8192) == F.ERR_TOO_LARGE
    assert F.status_string(F.ERR_TOO_LARGE) != "unknown status"
