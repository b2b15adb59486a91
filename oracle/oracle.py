"""ctypes wrapper of the CPU oracle (oracle/fp4q_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check in
__graft_entry__.py and by the cpu_baseline leg of bench.py -- never by the
library in microscaling_fp4_block_fp4q_amd/.

Tensors cross this boundary as numpy arrays on the host: fp32 as float32,
bf16 / fp16 as uint16 bit patterns together with a dtype tag (DT_*).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp4q_oracle.c")
LIB = os.path.join(HERE, "liboracle_fp4q.so")
# A prebuilt oracle library to load instead of building SRC: the mutation
# test points this at deliberately broken copies of the oracle to show that
# the pins catch them.
ALT_LIB = os.environ.get("FP4Q_ORACLE_LIB")

DT_F32, DT_BF16, DT_F16 = 0, 1, 2
SF_E8M0, SF_E4M3, SF_UE5M3 = 0, 1, 2
ABSMAX, PREVENT_ZERO, FOUR_OVER_SIX, BRUTE_FORCE, GIVEN = 0, 1, 2, 3, 4
GLOBAL_NONE, GLOBAL_TENSOR_AMAX, GLOBAL_USER, GLOBAL_SEARCH = 0, 1, 2, 3
SEARCH_CANDIDATES = 32

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, no intrinsics, no fast-math)."""
    if ALT_LIB:
        return ALT_LIB
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        f, i, i64, p = ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        L.oracle_e2m1_mag.argtypes, L.oracle_e2m1_mag.restype = [f], i
        L.oracle_e2m1_value.argtypes, L.oracle_e2m1_value.restype = [i], ctypes.c_double
        L.oracle_e4m3_decode.argtypes, L.oracle_e4m3_decode.restype = [i], ctypes.c_double
        L.oracle_e4m3_encode.argtypes, L.oracle_e4m3_encode.restype = [f], i
        L.oracle_e8m0_decode.argtypes, L.oracle_e8m0_decode.restype = [i], ctypes.c_double
        L.oracle_ue5m3_decode.argtypes, L.oracle_ue5m3_decode.restype = [i], ctypes.c_double
        L.oracle_ue5m3_encode.argtypes, L.oracle_ue5m3_encode.restype = [f], i
        L.oracle_e8m0_absmax_code.argtypes, L.oracle_e8m0_absmax_code.restype = [f], i
        L.oracle_bf16_to_f32.argtypes, L.oracle_bf16_to_f32.restype = [ctypes.c_uint16], f
        L.oracle_f16_to_f32.argtypes, L.oracle_f16_to_f32.restype = [ctypes.c_uint16], f
        L.oracle_bf16_from_f32.argtypes, L.oracle_bf16_from_f32.restype = [f], ctypes.c_uint16
        L.oracle_f16_from_f32.argtypes, L.oracle_f16_from_f32.restype = [f], ctypes.c_uint16
        L.oracle_hadamard_coef.argtypes, L.oracle_hadamard_coef.restype = [i], f
        L.oracle_fwht.argtypes, L.oracle_fwht.restype = [p, i], None
        L.oracle_tree_sum.argtypes, L.oracle_tree_sum.restype = [p, i], f
        L.oracle_block_sse.argtypes, L.oracle_block_sse.restype = [p, i, f], f
        L.oracle_global_scale.argtypes, L.oracle_global_scale.restype = [p, i64], f
        L.oracle_tensor_global_scale.argtypes = [p, i, i64, i64, i64, i]
        L.oracle_tensor_global_scale.restype = f
        L.oracle_global_scale_search.argtypes = [i, i, i, p, i, i64, i64, i64, p]
        L.oracle_global_scale_search.restype = f
        L.oracle_code_histogram.argtypes, L.oracle_code_histogram.restype = [p, i64, i64, p], i
        L.oracle_mxfp4_gemm.argtypes, L.oracle_mxfp4_gemm.restype = [p, p, p, p, i64, i64, i64, p], i
        L.oracle_nvfp4_gemm.argtypes = [p, p, f, p, p, f, i64, i64, i64, p]
        L.oracle_nvfp4_gemm.restype = i
        L.oracle_quantize.argtypes = [i, i, i, i, f, i, p, i, i64, i64, i64,
                                      p, p, p, p, i, i64, p, p]
        L.oracle_quantize.restype = i
        L.oracle_dequantize.argtypes = [i, i, p, p, f, i64, i64, p, i, i64]
        L.oracle_dequantize.restype = i
        L.oracle_block_mse.argtypes = [i, i, i, p, i, i64, i64, i64, p, p, f, p]
        L.oracle_block_mse.restype = i
        L.oracle_relaxed_fwd.argtypes = [i, i, p, i, i64, i64, i64, p, f, p, i, p, i, i64, p]
        L.oracle_relaxed_fwd.restype = i
        L.oracle_relaxed_bwd.argtypes = [i, i, p, i, i64, i64, i64, p, f, p, i, p, i, i64, p]
        L.oracle_relaxed_bwd.restype = i
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dt_of(a: np.ndarray, dt: int | None) -> int:
    if a.dtype == np.float32:
        return DT_F32
    if a.dtype == np.uint16:
        if dt not in (DT_BF16, DT_F16):
            raise ValueError("uint16 arrays need dt=DT_BF16 or DT_F16")
        return dt
    raise TypeError(f"unsupported array dtype {a.dtype}")


def _out_array(rows, cols, dt):
    return np.zeros((rows, cols), dtype=np.float32 if dt == DT_F32 else np.uint16)


# --------------------------------------------------------------------------
# scalar primitives (pins)
# --------------------------------------------------------------------------

def e2m1_mag(u: float) -> int:
    return lib().oracle_e2m1_mag(float(np.float32(u)))


def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(int(code))


def e4m3_encode(v) -> int:
    return lib().oracle_e4m3_encode(float(np.float32(v)))


def ue5m3_decode(code: int) -> float:
    return lib().oracle_ue5m3_decode(int(code))


def ue5m3_encode(v) -> int:
    return lib().oracle_ue5m3_encode(float(np.float32(v)))


def e8m0_decode(code: int) -> float:
    return lib().oracle_e8m0_decode(int(code))


def e8m0_absmax_code(a) -> int:
    return lib().oracle_e8m0_absmax_code(float(np.float32(a)))


def bf16_from_f32(v) -> int:
    return lib().oracle_bf16_from_f32(float(np.float32(v)))


def f16_from_f32(v) -> int:
    return lib().oracle_f16_from_f32(float(np.float32(v)))


def bf16_to_f32(h: int) -> float:
    return lib().oracle_bf16_to_f32(int(h))


def f16_to_f32(h: int) -> float:
    return lib().oracle_f16_to_f32(int(h))


def hadamard_coef(n: int) -> np.float32:
    return np.float32(lib().oracle_hadamard_coef(n))


def fwht(v: np.ndarray) -> np.ndarray:
    """Normalised FWHT of each length-n row of a float32 array (copy)."""
    a = np.ascontiguousarray(v, dtype=np.float32).copy()
    n = a.shape[-1]
    flat = a.reshape(-1, n)
    for r in range(flat.shape[0]):
        row = flat[r]
        lib().oracle_fwht(_ptr(row), n)
    return a


def tree_sum(v: np.ndarray) -> np.float32:
    a = np.ascontiguousarray(v, dtype=np.float32)
    return np.float32(lib().oracle_tree_sum(_ptr(a), a.size))


def block_sse(y: np.ndarray, S: float) -> np.float32:
    a = np.ascontiguousarray(y, dtype=np.float32)
    return np.float32(lib().oracle_block_sse(_ptr(a), a.size, float(np.float32(S))))


def global_scale(y: np.ndarray) -> np.float32:
    a = np.ascontiguousarray(y, dtype=np.float32)
    return np.float32(lib().oracle_global_scale(_ptr(a), a.size))


def tensor_global_scale(x: np.ndarray, *, hadamard: int = 0, x_dt: int | None = None) -> np.float32:
    """g of hierarchical scaling for a whole tensor (rotated when hadamard != 0)."""
    rows, cols = x.shape
    xd = _dt_of(x, x_dt)
    x = np.ascontiguousarray(x)
    return np.float32(lib().oracle_tensor_global_scale(_ptr(x), xd, rows, cols, cols, hadamard))


# --------------------------------------------------------------------------
# tensor entry points
# --------------------------------------------------------------------------

def global_scale_search(x: np.ndarray, *, block: int, strategy: int = ABSMAX, hadamard: int = 0,
                        x_dt: int | None = None):
    """The MSE-searched per-tensor scale of x (E4M3 block scales) and the
    fp64 total SSE of each of the SEARCH_CANDIDATES candidates."""
    rows, cols = x.shape
    xd = _dt_of(x, x_dt)
    x = np.ascontiguousarray(x)
    totals = np.zeros(SEARCH_CANDIDATES, np.float64)
    g = lib().oracle_global_scale_search(strategy, block, hadamard, _ptr(x), xd, rows, cols, cols, _ptr(totals))
    return np.float32(g), totals


def quantize(x: np.ndarray, *, fmt: int, block: int, strategy: int = ABSMAX,
             global_mode: int = GLOBAL_NONE, user_g: float = 1.0, hadamard: int = 0,
             x_dt: int | None = None, dq_dt: int | None = DT_F32,
             scales_in: np.ndarray | None = None, want_codes: bool = True) -> dict:
    """Quantize a 2-D tensor; returns codes, scales, g, dequant, mse, sse."""
    rows, cols = x.shape
    xd = _dt_of(x, x_dt)
    x = np.ascontiguousarray(x)
    nb = cols // block
    codes = np.zeros((rows, cols // 2), np.uint8) if want_codes else None
    if strategy == GIVEN:
        scales = np.ascontiguousarray(scales_in, dtype=np.uint8).copy()
    else:
        scales = np.zeros((rows, nb), np.uint8)
    g = np.zeros(1, np.float32)
    dq = _out_array(rows, cols, dq_dt) if dq_dt is not None else None
    mse = np.zeros((rows, nb), np.float32)
    sse = np.zeros((rows, nb), np.float32)
    rc = lib().oracle_quantize(fmt, block, strategy, global_mode, float(np.float32(user_g)), hadamard,
                               _ptr(x), xd, rows, cols, cols, _ptr(codes), _ptr(scales), _ptr(g),
                               _ptr(dq), -1 if dq_dt is None else dq_dt, cols, _ptr(mse), _ptr(sse))
    if rc != 0:
        raise ValueError("oracle_quantize rejected its arguments")
    return dict(codes=codes, scales=scales, g=np.float32(g[0]), dequant=dq, mse=mse, sse=sse)


def code_histogram(codes: np.ndarray) -> np.ndarray:
    """Counts of the 16 nibble codes in packed codes [rows, cols/2]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    counts = np.zeros(16, np.uint64)
    if lib().oracle_code_histogram(_ptr(codes), rows, 2 * half, _ptr(counts)) != 0:
        raise ValueError("oracle_code_histogram rejected its arguments")
    return counts


def mxfp4_gemm(a_codes, a_scales, b_codes, b_scales) -> np.ndarray:
    """C = dq(A) dq(B)^T in fp64 for MXFP4 operands (codes [rows, K/2], E8M0 scales [rows, K/32])."""
    a_codes, b_codes = (np.ascontiguousarray(t, dtype=np.uint8) for t in (a_codes, b_codes))
    a_scales, b_scales = (np.ascontiguousarray(t, dtype=np.uint8) for t in (a_scales, b_scales))
    M, N, K = a_codes.shape[0], b_codes.shape[0], 2 * a_codes.shape[1]
    c = np.zeros((M, N), np.float64)
    if lib().oracle_mxfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M, N, K, _ptr(c)) != 0:
        raise ValueError("oracle_mxfp4_gemm rejected its arguments")
    return c


def nvfp4_gemm(a_codes, a_scales, g_a, b_codes, b_scales, g_b) -> np.ndarray:
    """C = dq(A) dq(B)^T in fp64 for NVFP4 operands (codes [rows, K/2], E4M3
    scales [rows, K/16], per-tensor scales g_a, g_b)."""
    a_codes, b_codes = (np.ascontiguousarray(t, dtype=np.uint8) for t in (a_codes, b_codes))
    a_scales, b_scales = (np.ascontiguousarray(t, dtype=np.uint8) for t in (a_scales, b_scales))
    M, N, K = a_codes.shape[0], b_codes.shape[0], 2 * a_codes.shape[1]
    c = np.zeros((M, N), np.float64)
    if lib().oracle_nvfp4_gemm(_ptr(a_codes), _ptr(a_scales), float(g_a), _ptr(b_codes), _ptr(b_scales),
                               float(g_b), M, N, K, _ptr(c)) != 0:
        raise ValueError("oracle_nvfp4_gemm rejected its arguments")
    return c


def dequantize(codes, scales, g, *, fmt, block, rows, cols, out_dt=DT_F32):
    out = _out_array(rows, cols, out_dt)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rc = lib().oracle_dequantize(fmt, block, _ptr(codes), _ptr(scales), float(np.float32(g)),
                                 rows, cols, _ptr(out), out_dt, cols)
    if rc != 0:
        raise ValueError("oracle_dequantize rejected its arguments")
    return out


def block_mse(x, codes, scales, g, *, fmt, block, hadamard=0, x_dt=None):
    rows, cols = x.shape
    xd = _dt_of(x, x_dt)
    x = np.ascontiguousarray(x)
    mse = np.zeros((rows, cols // block), np.float32)
    rc = lib().oracle_block_mse(fmt, block, hadamard, _ptr(x), xd, rows, cols, cols,
                                _ptr(np.ascontiguousarray(codes, dtype=np.uint8)),
                                _ptr(np.ascontiguousarray(scales, dtype=np.uint8)),
                                float(np.float32(g)), _ptr(mse))
    if rc != 0:
        raise ValueError("oracle_block_mse rejected its arguments")
    return mse


def relaxed_fwd(w, scales, g, c_f16, *, fmt, block, sub_block, w_dt=None, out_dt=None, want_codes=True):
    rows, cols = w.shape
    wd = _dt_of(w, w_dt)
    od = wd if out_dt is None else out_dt
    w = np.ascontiguousarray(w)
    out = _out_array(rows, cols, od)
    codes = np.zeros((rows, cols // 2), np.uint8) if want_codes else None
    c = np.ascontiguousarray(c_f16, dtype=np.uint16)
    rc = lib().oracle_relaxed_fwd(fmt, block, _ptr(w), wd, rows, cols, cols,
                                  _ptr(np.ascontiguousarray(scales, dtype=np.uint8)),
                                  float(np.float32(g)), _ptr(c), sub_block, _ptr(out), od, cols,
                                  _ptr(codes))
    if rc != 0:
        raise ValueError("oracle_relaxed_fwd rejected its arguments")
    return out, codes


def relaxed_bwd(w, scales, g, c_f16, grad, *, fmt, block, sub_block, w_dt=None, g_dt=None):
    rows, cols = w.shape
    wd = _dt_of(w, w_dt)
    gd = _dt_of(grad, g_dt)
    w = np.ascontiguousarray(w)
    grad = np.ascontiguousarray(grad)
    out = np.zeros((rows, cols // sub_block), np.float32)
    c = np.ascontiguousarray(c_f16, dtype=np.uint16)
    rc = lib().oracle_relaxed_bwd(fmt, block, _ptr(w), wd, rows, cols, cols,
                                  _ptr(np.ascontiguousarray(scales, dtype=np.uint8)),
                                  float(np.float32(g)), _ptr(c), sub_block, _ptr(grad), gd, cols,
                                  _ptr(out))
    if rc != 0:
        raise ValueError("oracle_relaxed_bwd rejected its arguments")
    return out
