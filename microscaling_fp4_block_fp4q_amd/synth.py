"""Seeded synthetic tensors shaped like the pages' workloads.

This module only draws random numbers and casts them; it holds none of the
quantizer's arithmetic.  The same generators feed the CPU oracle (tests,
bench baseline) and the GPU library, so both sides see identical bits.

The pages quantize LLM weights and activations (Llama-3.1-8B MLP layers,
Qwen3 / LLaMA families); no model weights or datasets are used.  Instead:
  * i.i.d. N(0,1) / Laplace(0,1) tensors -- the numerical study of "Finer is
    Better (with the Right Scaling)" (method part 1) samples a normal
    distribution; the MR-GPTQ page (section 2.1) models weights and
    activations as Laplace before rotation.
  * heavy-tailed weights: 0.02 * Student-t(df=3) with 0.5 % of input columns
    scaled by 20 (outlier channels), shaped like Llama-3.1-8B MLP matrices.
  * activations: Laplace(0,1) tokens x hidden with 0.1 % outlier channels x50.
  * FOCUS fake-quant: N(0, 0.02) weights, fp16 c_k ~ U[0.8, 1.25], upstream
    gradient N(0,1).

Every draw is numpy PCG64 (`default_rng(seed)`) in float64, then cast with
round-half-to-even: fp32 via numpy, bf16 via torch, fp16 via numpy.  bf16 and
fp16 tensors are returned as uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np
import torch

F32, BF16, F16 = 0, 1, 2


def cast(a64: np.ndarray, dt: int) -> np.ndarray:
    """float64 -> fp32 array, or bf16 / fp16 bit patterns as uint16."""
    if dt == F32:
        return np.ascontiguousarray(a64.astype(np.float32))
    if dt == F16:
        return np.ascontiguousarray(a64.astype(np.float16)).view(np.uint16)
    t = torch.from_numpy(np.ascontiguousarray(a64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def normal(rows, cols, seed, dt=F32, sigma=1.0):
    rng = np.random.default_rng(seed)
    return cast(rng.standard_normal((rows, cols)) * sigma, dt)


def laplace(rows, cols, seed, dt=F32):
    rng = np.random.default_rng(seed)
    return cast(rng.laplace(0.0, 1.0, (rows, cols)), dt)


def scaled_fp32(x: np.ndarray, factor: float) -> np.ndarray:
    """x * fp32(factor) evaluated in fp32 (the x1e-4 underflow variants)."""
    return (x.astype(np.float32) * np.float32(factor)).astype(np.float32)


def outlier_columns(cols: int, frac: float, rng) -> np.ndarray:
    k = int(round(frac * cols))
    return np.sort(rng.choice(cols, size=k, replace=False))


def llama_mlp_weight(rows, cols, seed, dt=BF16):
    """0.02 * Student-t(df=3), round(0.005 * cols) input columns x20."""
    rng = np.random.default_rng(seed)
    w = 0.02 * rng.standard_t(3.0, (rows, cols))
    w[:, outlier_columns(cols, 0.005, rng)] *= 20.0
    return cast(w, dt)


def activations(tokens, hidden, seed, dt=BF16):
    """Laplace(0,1), round(0.001 * hidden) channels x50."""
    rng = np.random.default_rng(seed)
    a = rng.laplace(0.0, 1.0, (tokens, hidden))
    a[:, outlier_columns(hidden, 0.001, rng)] *= 50.0
    return cast(a, dt)


def focus_inputs(rows, cols, sub_block, seeds=(6, 7, 8), dt=BF16):
    """(W ~ N(0, 0.02), c ~ U[0.8, 1.25] as fp16 bits, G ~ N(0, 1))."""
    w = normal(rows, cols, seeds[0], dt, sigma=0.02)
    rng = np.random.default_rng(seeds[1])
    c = cast(rng.uniform(0.8, 1.25, (rows, cols // sub_block)), F16)
    g = normal(rows, cols, seeds[2], dt)
    return w, c, g


# --------------------------------------------------------------------------
# Named workloads (full sizes); tests draw smaller tensors with the same
# recipes by passing other shapes to the functions above.
# --------------------------------------------------------------------------

def config1():
    """fp32 1024 x 1024 N(0,1), seed 0."""
    return normal(1024, 1024, 0)


def config2():
    """fp32 4096 x 4096: N(0,1) seed 1, Laplace(0,1) seed 2, each also x1e-4."""
    n = normal(4096, 4096, 1)
    l = laplace(4096, 4096, 2)
    return {"normal": n, "laplace": l,
            "normal_1e-4": scaled_fp32(n, 1e-4), "laplace_1e-4": scaled_fp32(l, 1e-4)}


def config3():
    """bf16 Llama-3.1-8B-shaped MLP weights: W_down [4096, 14336] seed 3,
    W_gate/up [14336, 4096] seed 4."""
    return {"w_down": llama_mlp_weight(4096, 14336, 3), "w_up": llama_mlp_weight(14336, 4096, 4)}


def config4():
    """bf16 activations [8192 tokens, 4096 hidden], seed 5."""
    return activations(8192, 4096, 5)


def config5(sub_block=8):
    """bf16 W [4096, 12288] N(0, 0.02) seed 6; c fp16 seed 7; G bf16 seed 8."""
    return focus_inputs(4096, 12288, sub_block)


def to_torch(a: np.ndarray, dt: int, device="cpu") -> torch.Tensor:
    """Host array (fp32, or uint16 bit patterns) -> torch tensor of that dtype."""
    if dt == F32:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16))
        t = t.view(torch.bfloat16 if dt == BF16 else torch.float16)
    return t.to(device)


def from_torch(t: torch.Tensor) -> np.ndarray:
    """torch tensor (fp32 / bf16 / fp16 / uint8) -> host numpy array."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
