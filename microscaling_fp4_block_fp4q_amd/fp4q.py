"""Thin ctypes binding of libfp4q.so (include/fp4q.h).

Argument marshalling only: torch tensors become device pointers, element
types and row strides; the current torch stream becomes the hipStream_t.
Every step of the quantize-dequantize path runs in the library's HIP
kernels.  There is no CPU fallback: a missing library raises.

The raw entry points keep the C names (``fp4q_quantize`` ...); the short
names (``quantize`` ...) also allocate the outputs with torch.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfp4q.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "fp4q.h")

# FP4Q_ABI_VERSION and the enums (include/fp4q.h)
ABI_VERSION = 8
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_SHAPE, ERR_ALIGNMENT, ERR_DEVICE, ERR_TOO_LARGE = range(7)
F32, BF16, F16 = 0, 1, 2
E8M0, E4M3, UE5M3 = 0, 1, 2
ABSMAX, PREVENT_ZERO, FOUR_OVER_SIX, BRUTE_FORCE, GIVEN = range(5)
GLOBAL_NONE, GLOBAL_TENSOR_AMAX, GLOBAL_USER, GLOBAL_SEARCH = range(4)
COUNT_REPLICAS = 64          # FP4Q_COUNT_REPLICAS: rows of the fused code counts


class Config(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("scale_fmt", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("strategy", ctypes.c_int32),
        ("global_mode", ctypes.c_int32),
        ("global_scale", ctypes.c_float),
        ("hadamard", ctypes.c_int32),
    ]


def config(scale_fmt=E4M3, block=16, strategy=ABSMAX, global_mode=GLOBAL_NONE, global_scale=1.0,
           hadamard=0) -> Config:
    return Config(ctypes.sizeof(Config), scale_fmt, block, strategy, global_mode, global_scale, hadamard)


def mxfp4(strategy=ABSMAX, hadamard=0) -> Config:
    """E2M1 in blocks of 32 with a power-of-two E8M0 scale."""
    return config(E8M0, 32, strategy, GLOBAL_NONE, 1.0, hadamard)


def nvfp4(strategy=ABSMAX, global_mode=GLOBAL_TENSOR_AMAX, global_scale=1.0, hadamard=0) -> Config:
    """E2M1 in blocks of 16 with an E4M3 scale under a per-tensor fp32 scale."""
    return config(E4M3, 16, strategy, global_mode, global_scale, hadamard)


class Fp4qError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfp4q.so (built by microscaling_fp4_block_fp4q_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m microscaling_fp4_block_fp4q_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, p, cp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(Config)
        L.fp4q_abi_version.restype = ctypes.c_int
        L.fp4q_abi_version.argtypes = []
        L.fp4q_status_string.restype = ctypes.c_char_p
        L.fp4q_status_string.argtypes = [ctypes.c_int]
        L.fp4q_workspace_bytes.restype = ctypes.c_size_t
        L.fp4q_workspace_bytes.argtypes = [cp, i64, i64]
        L.fp4q_quantize.restype = ctypes.c_int
        L.fp4q_quantize.argtypes = [cp, p, ctypes.c_int, i64, i64, i64, p, p, p, p, ctypes.c_int, i64, p, p, p]
        L.fp4q_quantize_histogram.restype = ctypes.c_int
        L.fp4q_quantize_histogram.argtypes = [cp, p, ctypes.c_int, i64, i64, i64, p, p, p, p, ctypes.c_int, i64, p,
                                              p, p, p]
        L.fp4q_quantize_noalloc.restype = ctypes.c_int
        L.fp4q_quantize_noalloc.argtypes = [cp, p, ctypes.c_int, i64, i64, i64, p, p, p, p, ctypes.c_int, i64, p, p]
        L.fp4q_dequantize.restype = ctypes.c_int
        L.fp4q_dequantize.argtypes = [cp, p, p, p, i64, i64, p, ctypes.c_int, i64, p]
        L.fp4q_block_mse.restype = ctypes.c_int
        L.fp4q_block_mse.argtypes = [cp, p, ctypes.c_int, i64, i64, i64, p, p, p, p, p]
        L.fp4q_scale_search.restype = ctypes.c_int
        L.fp4q_scale_search.argtypes = [cp, p, ctypes.c_int, i64, i64, i64, p, p, p, p, p]
        L.fp4q_relaxed_fakequant_fwd.restype = ctypes.c_int
        L.fp4q_relaxed_fakequant_fwd.argtypes = [cp, p, ctypes.c_int, i64, i64, i64, p, p, p, i32, p,
                                                 ctypes.c_int, i64, p, p]
        L.fp4q_relaxed_fakequant_bwd.restype = ctypes.c_int
        L.fp4q_relaxed_fakequant_bwd.argtypes = [cp, p, ctypes.c_int, i64, i64, i64, p, p, p, i32, p,
                                                 ctypes.c_int, i64, p, p]
        L.fp4q_code_histogram.restype = ctypes.c_int
        L.fp4q_code_histogram.argtypes = [p, i64, i64, p, p]
        L.fp4q_mxfp4_gemm.restype = ctypes.c_int
        L.fp4q_mxfp4_gemm.argtypes = [p, p, p, p, i64, i64, i64, p, ctypes.c_int, i64, p, p]
        L.fp4q_mxfp4_gemm_workspace_bytes.restype = ctypes.c_size_t
        L.fp4q_mxfp4_gemm_workspace_bytes.argtypes = [i64, i64, i64]
        L.fp4q_nvfp4_gemm.restype = ctypes.c_int
        L.fp4q_nvfp4_gemm.argtypes = [p, p, p, p, p, p, i64, i64, i64, p, ctypes.c_int, i64, p, p]
        L.fp4q_nvfp4_gemm_workspace_bytes.restype = ctypes.c_size_t
        L.fp4q_nvfp4_gemm_workspace_bytes.argtypes = [i64, i64, i64]
        _lib = L
    return _lib


def declared_entry_points() -> list[str]:
    """Function names include/fp4q.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(fp4q_\w+)\s*\(", text, re.M)))


def status_string(status: int) -> str:
    return lib().fp4q_status_string(status).decode()


def abi_version() -> int:
    return lib().fp4q_abi_version()


def workspace_bytes(cfg: Config, rows: int, cols: int) -> int:
    return lib().fp4q_workspace_bytes(ctypes.byref(cfg), rows, cols)


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


def dtype_code(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported element type {t.dtype}") from None


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _rows_cols_ld(t: torch.Tensor):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.shape[0], t.shape[1], t.stride(0)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Make the launch stream current while outputs and workspace are
    allocated, so that the caching allocator orders their reuse after the
    launches on that stream."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _dense(t, dtype, shape, what):
    """A buffer the C ABI addresses as dense memory: device tensor of the
    given element type and shape, contiguous (None passes)."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{what}: expected a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{what}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous tensor")


def _scalar_g(g, what="g"):
    if g is None:
        return
    if not isinstance(g, torch.Tensor) or g.device.type != "cuda" or g.dtype != torch.float32 or g.numel() < 1:
        raise ValueError(f"{what}: expected a device float32 tensor of at least one element")


def _workspace_ok(ws, cfg, rows, cols):
    need = workspace_bytes(cfg, rows, cols)
    if ws is None:
        return
    if not isinstance(ws, torch.Tensor) or ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("workspace: expected a contiguous device tensor")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace: {need} bytes needed, {ws.numel() * ws.element_size()} given")


def _out_2d(t, rows, cols, what):
    """A [rows, cols] row-strided output or input (unit column stride)."""
    r, c, ld = _rows_cols_ld(t)
    if (r, c) != (rows, cols):
        raise ValueError(f"{what}: expected shape {(rows, cols)}, got {(r, c)}")
    dtype_code(t)
    return ld


def _check(status: int, what: str):
    if status != OK:
        raise Fp4qError(status, what)


# --------------------------------------------------------------------------
# raw entry points (caller allocates every buffer)
# --------------------------------------------------------------------------

def fp4q_quantize(cfg, x, codes, scales, g=None, dequant=None, block_mse=None, workspace=None, stream=None):
    rows, cols, ld = _rows_cols_ld(x)
    nb = cols // cfg.block
    _dense(codes, torch.uint8, (rows, cols // 2), "codes")
    _dense(scales, torch.uint8, (rows, nb), "scales")
    _dense(block_mse, torch.float32, (rows, nb), "block_mse")
    _scalar_g(g)
    _workspace_ok(workspace, cfg, rows, cols)
    dq_dt, ld_dq = F32, cols
    if dequant is not None:
        ld_dq = _out_2d(dequant, rows, cols, "dequant")
        dq_dt = dtype_code(dequant)
    st = lib().fp4q_quantize(ctypes.byref(cfg), _ptr(x), dtype_code(x), rows, cols, ld, _ptr(codes),
                             _ptr(scales), _ptr(g), _ptr(dequant), dq_dt, ld_dq, _ptr(block_mse),
                             _ptr(workspace), _stream(stream))
    _check(st, "fp4q_quantize")


def fp4q_quantize_histogram(cfg, x, codes, scales, counts, g=None, dequant=None, block_mse=None, workspace=None,
                            stream=None):
    """fp4q_quantize that also adds the written codes' occupancy to counts
    (int64 [COUNT_REPLICAS, 16]; the occupancy is counts.sum(0))."""
    rows, cols, ld = _rows_cols_ld(x)
    nb = cols // cfg.block
    _dense(codes, torch.uint8, (rows, cols // 2), "codes")
    _dense(scales, torch.uint8, (rows, nb), "scales")
    _dense(block_mse, torch.float32, (rows, nb), "block_mse")
    _dense(counts, torch.int64, (COUNT_REPLICAS, 16), "counts")
    _scalar_g(g)
    _workspace_ok(workspace, cfg, rows, cols)
    dq_dt, ld_dq = F32, cols
    if dequant is not None:
        ld_dq = _out_2d(dequant, rows, cols, "dequant")
        dq_dt = dtype_code(dequant)
    st = lib().fp4q_quantize_histogram(ctypes.byref(cfg), _ptr(x), dtype_code(x), rows, cols, ld, _ptr(codes),
                                       _ptr(scales), _ptr(g), _ptr(dequant), dq_dt, ld_dq, _ptr(block_mse),
                                       _ptr(counts), _ptr(workspace), _stream(stream))
    _check(st, "fp4q_quantize_histogram")


def fp4q_quantize_noalloc(cfg, x, codes, scales, g=None, dequant=None, block_mse=None, stream=None):
    """fp4q_quantize with the workspace in the library's static device scratch."""
    rows, cols, ld = _rows_cols_ld(x)
    nb = cols // cfg.block
    _dense(codes, torch.uint8, (rows, cols // 2), "codes")
    _dense(scales, torch.uint8, (rows, nb), "scales")
    _dense(block_mse, torch.float32, (rows, nb), "block_mse")
    _scalar_g(g)
    dq_dt, ld_dq = F32, cols
    if dequant is not None:
        ld_dq = _out_2d(dequant, rows, cols, "dequant")
        dq_dt = dtype_code(dequant)
    st = lib().fp4q_quantize_noalloc(ctypes.byref(cfg), _ptr(x), dtype_code(x), rows, cols, ld, _ptr(codes),
                                     _ptr(scales), _ptr(g), _ptr(dequant), dq_dt, ld_dq, _ptr(block_mse),
                                     _stream(stream))
    _check(st, "fp4q_quantize_noalloc")


def fp4q_scale_search(cfg, x, scales, g=None, best_sse=None, workspace=None, stream=None):
    rows, cols, ld = _rows_cols_ld(x)
    nb = cols // cfg.block
    _dense(scales, torch.uint8, (rows, nb), "scales")
    _dense(best_sse, torch.float32, (rows, nb), "best_sse")
    _scalar_g(g)
    _workspace_ok(workspace, cfg, rows, cols)
    st = lib().fp4q_scale_search(ctypes.byref(cfg), _ptr(x), dtype_code(x), rows, cols, ld, _ptr(scales),
                                 _ptr(g), _ptr(best_sse), _ptr(workspace), _stream(stream))
    _check(st, "fp4q_scale_search")


def fp4q_dequantize(cfg, codes, scales, out, g=None, stream=None):
    rows, cols, ld = _rows_cols_ld(out)
    _dense(codes, torch.uint8, (rows, cols // 2), "codes")
    _dense(scales, torch.uint8, (rows, cols // cfg.block), "scales")
    _scalar_g(g)
    st = lib().fp4q_dequantize(ctypes.byref(cfg), _ptr(codes), _ptr(scales), _ptr(g), rows, cols, _ptr(out),
                               dtype_code(out), ld, _stream(stream))
    _check(st, "fp4q_dequantize")


def fp4q_block_mse(cfg, x, codes, scales, block_mse, g=None, stream=None):
    rows, cols, ld = _rows_cols_ld(x)
    nb = cols // cfg.block
    _dense(codes, torch.uint8, (rows, cols // 2), "codes")
    _dense(scales, torch.uint8, (rows, nb), "scales")
    _dense(block_mse, torch.float32, (rows, nb), "block_mse")
    _scalar_g(g)
    st = lib().fp4q_block_mse(ctypes.byref(cfg), _ptr(x), dtype_code(x), rows, cols, ld, _ptr(codes),
                              _ptr(scales), _ptr(g), _ptr(block_mse), _stream(stream))
    _check(st, "fp4q_block_mse")


def fp4q_relaxed_fakequant_fwd(cfg, w, scales, c, sub_block, w_hat, g=None, codes=None, stream=None):
    rows, cols, ld = _rows_cols_ld(w)
    _dense(scales, torch.uint8, (rows, cols // cfg.block), "scales")
    _dense(c, torch.float16, (rows, cols // sub_block), "c")
    _dense(codes, torch.uint8, (rows, cols // 2), "codes")
    _scalar_g(g)
    ld_out = _out_2d(w_hat, rows, cols, "w_hat")
    st = lib().fp4q_relaxed_fakequant_fwd(ctypes.byref(cfg), _ptr(w), dtype_code(w), rows, cols, ld,
                                          _ptr(scales), _ptr(g), _ptr(c), sub_block, _ptr(w_hat),
                                          dtype_code(w_hat), ld_out, _ptr(codes), _stream(stream))
    _check(st, "fp4q_relaxed_fakequant_fwd")


def fp4q_relaxed_fakequant_bwd(cfg, w, scales, c, sub_block, grad_out, grad_c, g=None, stream=None):
    rows, cols, ld = _rows_cols_ld(w)
    _dense(scales, torch.uint8, (rows, cols // cfg.block), "scales")
    _dense(c, torch.float16, (rows, cols // sub_block), "c")
    _dense(grad_c, torch.float32, (rows, cols // sub_block), "grad_c")
    _scalar_g(g)
    ld_g = _out_2d(grad_out, rows, cols, "grad_out")
    st = lib().fp4q_relaxed_fakequant_bwd(ctypes.byref(cfg), _ptr(w), dtype_code(w), rows, cols, ld,
                                          _ptr(scales), _ptr(g), _ptr(c), sub_block, _ptr(grad_out),
                                          dtype_code(grad_out), ld_g, _ptr(grad_c), _stream(stream))
    _check(st, "fp4q_relaxed_fakequant_bwd")


def fp4q_code_histogram(codes, counts, stream=None):
    if codes.dim() != 2:
        raise ValueError("codes: expected a 2-D tensor [rows, cols/2]")
    rows, half = codes.shape
    _dense(codes, torch.uint8, (rows, half), "codes")
    _dense(counts, torch.int64, (16,), "counts")
    st = lib().fp4q_code_histogram(_ptr(codes), rows, 2 * half, _ptr(counts), _stream(stream))
    _check(st, "fp4q_code_histogram")


def mxfp4_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return lib().fp4q_mxfp4_gemm_workspace_bytes(M, N, K)


def fp4q_mxfp4_gemm(a_codes, a_scales, b_codes, b_scales, c, workspace, stream=None):
    if a_codes.dim() != 2 or b_codes.dim() != 2:
        raise ValueError("codes: expected 2-D tensors [rows, K/2]")
    M, N = a_codes.shape[0], b_codes.shape[0]
    K = 2 * a_codes.shape[1]
    _dense(a_codes, torch.uint8, (M, K // 2), "a_codes")
    _dense(b_codes, torch.uint8, (N, K // 2), "b_codes")
    _dense(a_scales, torch.uint8, (M, K // 32), "a_scales")
    _dense(b_scales, torch.uint8, (N, K // 32), "b_scales")
    ldc = _out_2d(c, M, N, "c")
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" or not workspace.is_contiguous() \
            or workspace.numel() * workspace.element_size() < mxfp4_gemm_workspace_bytes(M, N, K):
        raise ValueError("workspace: expected a contiguous device tensor of mxfp4_gemm_workspace_bytes(M, N, K)")
    st = lib().fp4q_mxfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M, N, K, _ptr(c),
                               dtype_code(c), ldc, _ptr(workspace), _stream(stream))
    _check(st, "fp4q_mxfp4_gemm")


def nvfp4_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return lib().fp4q_nvfp4_gemm_workspace_bytes(M, N, K)


def _g_ptr(g, name):
    if g is None:
        return None
    _dense(g, torch.float32, (1,), name)
    return _ptr(g)


def fp4q_nvfp4_gemm(a_codes, a_scales, a_g, b_codes, b_scales, b_g, c, workspace, stream=None):
    """Raw entry point: a_g / b_g are one-element fp32 device tensors (the g
    fp4q_quantize writes) or None (1)."""
    if a_codes.dim() != 2 or b_codes.dim() != 2:
        raise ValueError("codes: expected 2-D tensors [rows, K/2]")
    M, N = a_codes.shape[0], b_codes.shape[0]
    K = 2 * a_codes.shape[1]
    _dense(a_codes, torch.uint8, (M, K // 2), "a_codes")
    _dense(b_codes, torch.uint8, (N, K // 2), "b_codes")
    _dense(a_scales, torch.uint8, (M, K // 16), "a_scales")
    _dense(b_scales, torch.uint8, (N, K // 16), "b_scales")
    ldc = _out_2d(c, M, N, "c")
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" or not workspace.is_contiguous() \
            or workspace.numel() * workspace.element_size() < nvfp4_gemm_workspace_bytes(M, N, K):
        raise ValueError("workspace: expected a contiguous device tensor of nvfp4_gemm_workspace_bytes(M, N, K)")
    st = lib().fp4q_nvfp4_gemm(_ptr(a_codes), _ptr(a_scales), _g_ptr(a_g, "a_g"), _ptr(b_codes), _ptr(b_scales),
                               _g_ptr(b_g, "b_g"), M, N, K, _ptr(c), dtype_code(c), ldc, _ptr(workspace),
                               _stream(stream))
    _check(st, "fp4q_nvfp4_gemm")


# --------------------------------------------------------------------------
# allocating wrappers
# --------------------------------------------------------------------------

def _workspace(cfg, rows, cols, device):
    n = workspace_bytes(cfg, rows, cols)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device) if n else None


def quantize(x, cfg, dequant_dtype=None, want_mse=True, scales=None, counts=None, stream=None):
    """Quantize a 2-D device tensor; returns dict(codes, scales, g, dequant, mse).
    counts: an int64 device tensor [COUNT_REPLICAS, 16] (counts_buffer())
    to which the written codes' occupancy is added, fused into the quantize
    kernels; occupancy(counts) sums its rows.  With stream, the outputs are
    allocated on and the kernels run on it."""
    rows, cols, _ = _rows_cols_ld(x)
    dev = x.device
    with _on(stream):
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        if scales is None:
            scales = torch.empty((rows, cols // cfg.block), dtype=torch.uint8, device=dev)
        g = torch.empty(1, dtype=torch.float32, device=dev)
        dq = None if dequant_dtype is None else torch.empty((rows, cols), dtype=dequant_dtype, device=dev)
        mse = torch.empty((rows, cols // cfg.block), dtype=torch.float32, device=dev) if want_mse else None
        ws = _workspace(cfg, rows, cols, dev)
        if counts is None:
            fp4q_quantize(cfg, x, codes, scales, g, dq, mse, ws, stream)
        else:
            fp4q_quantize_histogram(cfg, x, codes, scales, counts, g, dq, mse, ws, stream)
    return dict(codes=codes, scales=scales, g=g, dequant=dq, mse=mse)


def scale_search(x, cfg, want_sse=True, stream=None):
    rows, cols, _ = _rows_cols_ld(x)
    dev = x.device
    with _on(stream):
        scales = torch.empty((rows, cols // cfg.block), dtype=torch.uint8, device=dev)
        g = torch.empty(1, dtype=torch.float32, device=dev)
        sse = torch.empty((rows, cols // cfg.block), dtype=torch.float32, device=dev) if want_sse else None
        fp4q_scale_search(cfg, x, scales, g, sse, _workspace(cfg, rows, cols, dev), stream)
    return dict(scales=scales, g=g, sse=sse)


def dequantize(codes, scales, cfg, g=None, out_dtype=torch.float32, stream=None):
    rows, cols = codes.shape[0], codes.shape[1] * 2
    with _on(stream):
        out = torch.empty((rows, cols), dtype=out_dtype, device=codes.device)
        fp4q_dequantize(cfg, codes, scales, out, g, stream)
    return out


def block_mse(x, codes, scales, cfg, g=None, stream=None):
    rows, cols, _ = _rows_cols_ld(x)
    with _on(stream):
        out = torch.empty((rows, cols // cfg.block), dtype=torch.float32, device=x.device)
        fp4q_block_mse(cfg, x, codes, scales, out, g, stream)
    return out


def relaxed_fakequant_fwd(w, scales, c, cfg, sub_block=8, g=None, out_dtype=None, want_codes=False, stream=None):
    rows, cols, _ = _rows_cols_ld(w)
    with _on(stream):
        w_hat = torch.empty((rows, cols), dtype=out_dtype or w.dtype, device=w.device)
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=w.device) if want_codes else None
        fp4q_relaxed_fakequant_fwd(cfg, w, scales, c, sub_block, w_hat, g, codes, stream)
    return w_hat, codes


def relaxed_fakequant_bwd(w, scales, c, grad_out, cfg, sub_block=8, g=None, stream=None):
    rows, cols, _ = _rows_cols_ld(w)
    with _on(stream):
        grad_c = torch.empty((rows, cols // sub_block), dtype=torch.float32, device=w.device)
        fp4q_relaxed_fakequant_bwd(cfg, w, scales, c, sub_block, grad_out, grad_c, g, stream)
    return grad_c


def counts_buffer(device):
    """A zeroed buffer for the fused code counts of quantize(counts=...)."""
    return torch.zeros((COUNT_REPLICAS, 16), dtype=torch.int64, device=device)


def occupancy(counts):
    """The 16 code counts of a fused-count buffer (the sum of its rows)."""
    return counts.sum(0)


def code_histogram(codes, stream=None):
    """Counts of the 16 nibble codes in packed codes [rows, cols/2] (int64 tensor of 16)."""
    with _on(stream):
        counts = torch.zeros(16, dtype=torch.int64, device=codes.device)
        fp4q_code_histogram(codes, counts, stream)
    return counts


def gemm_workspace(M, N, K, device):
    """Device workspace for fp4q_mxfp4_gemm (256-byte aligned by torch's allocator)."""
    return torch.empty(max(mxfp4_gemm_workspace_bytes(M, N, K), 256), dtype=torch.uint8, device=device)


def nvfp4_gemm(a_codes, a_scales, a_g, b_codes, b_scales, b_g, out_dtype=torch.float32, workspace=None,
               stream=None):
    """C [M, N] = dq(A) dq(B)^T for NVFP4 operands (codes [rows, K/2], E4M3
    scales [rows, K/16], per-tensor scales a_g / b_g: one-element fp32 device
    tensors as quantize() returns them, or None for 1).  C is a view of N
    columns of an [M, ldc] buffer with rows padded to 16 bytes."""
    M, N, K = a_codes.shape[0], b_codes.shape[0], 2 * a_codes.shape[1]
    per16 = 16 // torch.empty(0, dtype=out_dtype).element_size()
    ldc = (N + per16 - 1) // per16 * per16
    with _on(stream):
        c = torch.empty((M, ldc), dtype=out_dtype, device=a_codes.device)[:, :N]
        if workspace is None:
            n = nvfp4_gemm_workspace_bytes(M, N, K)
            workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=a_codes.device)
        fp4q_nvfp4_gemm(a_codes, a_scales, a_g, b_codes, b_scales, b_g, c, workspace, stream)
    return c


def mxfp4_gemm(a_codes, a_scales, b_codes, b_scales, out_dtype=torch.float32, workspace=None, stream=None):
    """C [M, N] = dq(A) dq(B)^T for MXFP4 operands (codes [rows, K/2], E8M0 scales [rows, K/32]).

    C is returned as a view of N columns of an [M, ldc] buffer whose rows are
    padded to whole 16-byte chunks (the entry point's row alignment)."""
    M, N, K = a_codes.shape[0], b_codes.shape[0], 2 * a_codes.shape[1]
    per16 = 16 // torch.empty(0, dtype=out_dtype).element_size()
    ldc = (N + per16 - 1) // per16 * per16
    with _on(stream):
        c = torch.empty((M, ldc), dtype=out_dtype, device=a_codes.device)[:, :N]
        if workspace is None:
            workspace = gemm_workspace(M, N, K, a_codes.device)
        fp4q_mxfp4_gemm(a_codes, a_scales, b_codes, b_scales, c, workspace, stream)
    return c
