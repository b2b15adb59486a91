"""Shared helpers of the GPU parity tests: run the HIP library through its
C ABI (ctypes binding) and the oracle on the same seeded host arrays, and
compare element by element.  Expected values always come from oracle/."""
from __future__ import annotations

import sys

import numpy as np
import torch

from microscaling_fp4_block_fp4q_amd import fp4q as F
from microscaling_fp4_block_fp4q_amd import synth as S
from oracle import oracle as O

DEV = "cuda"
TORCH_DT = {S.F32: torch.float32, S.BF16: torch.bfloat16, S.F16: torch.float16}


def note(msg: str):
    """Name the case on stdout before it touches the GPU."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def gpu_quantize(x: np.ndarray, x_dt: int, cfg, dq_dt: int | None = S.F32, want_mse=True, scales_in=None):
    xt = S.to_torch(x, x_dt, DEV)
    sc = None if scales_in is None else torch.from_numpy(np.ascontiguousarray(scales_in)).to(DEV)
    r = F.quantize(xt, cfg, dequant_dtype=None if dq_dt is None else TORCH_DT[dq_dt], want_mse=want_mse,
                   scales=sc)
    torch.cuda.synchronize()
    out = {k: (None if v is None else S.from_torch(v)) for k, v in r.items()}
    out["g"] = np.float32(out["g"][0])
    return out


def oracle_quantize(x, x_dt, cfg, dq_dt=S.F32, user_g=None, scales_in=None):
    gm, g = cfg.global_mode, cfg.global_scale
    if user_g is not None:            # a row sample quantized with the full tensor's g
        gm, g = O.GLOBAL_USER, user_g
    return O.quantize(x, x_dt=x_dt, fmt=cfg.scale_fmt, block=cfg.block, strategy=cfg.strategy,
                      global_mode=gm, user_g=g, hadamard=cfg.hadamard, dq_dt=dq_dt, scales_in=scales_in)


def bits(a):
    a = np.asarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    return a


def assert_same(got, want, what):
    g, w = bits(got), bits(want)
    if not np.array_equal(g, w):
        bad = np.argwhere(g != w)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: gpu {np.asarray(got)[i]!r} "
                             f"({g[i]:#x}) vs oracle {np.asarray(want)[i]!r} ({w[i]:#x})")


def compare_quant(gpu, ref, rows=None, keys=("codes", "scales", "dequant", "mse")):
    for k in keys:
        if gpu.get(k) is None or ref.get(k) is None:
            continue
        got = gpu[k] if rows is None else gpu[k][rows]
        assert_same(got, ref[k], k)


def sample_rows(n_rows: int, seed: int = 0, k: int = 6) -> np.ndarray:
    rng = np.random.default_rng(seed)
    pick = {0, 1, n_rows // 2, n_rows - 1} | set(rng.choice(n_rows, size=min(k, n_rows), replace=False).tolist())
    return np.array(sorted(pick))


def host_threads() -> int:
    """Threads for the oracle on the host: this process's CPUs, at most 16."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_rows(fn, arrays, chunk=64, **kw):
    """Run an oracle entry point over row chunks of the given arrays on the
    host's cores (ctypes releases the GIL) and stack the results by rows.
    fn(*row_slices, **kw) returns an array, a tuple of arrays or a dict of
    arrays with a leading row axis (scalars and None pass through from the
    first chunk).  Every row of the result is the oracle's own; rows are
    independent in every entry point called this way (a per-tensor scale is
    passed in as the user scale)."""
    import concurrent.futures as cf
    rows = arrays[0].shape[0]
    starts = list(range(0, rows, chunk))

    def run(r0):
        return fn(*(np.ascontiguousarray(a[r0:r0 + chunk]) for a in arrays), **kw)

    with cf.ThreadPoolExecutor(host_threads()) as ex:
        parts = list(ex.map(run, starts))

    def stack(vals):
        v0 = vals[0]
        if isinstance(v0, np.ndarray) and v0.ndim >= 1:
            return np.concatenate(vals, axis=0)
        return v0

    first = parts[0]
    if isinstance(first, dict):
        return {k: stack([p[k] for p in parts]) for k in first}
    if isinstance(first, tuple):
        return tuple(stack([p[i] for p in parts]) for i in range(len(first)))
    return stack(parts)
