"""Brute force at blocks 4 and 8 with E4M3 scales, every block against the oracle's
exhaustive search, on inputs built to stress the candidate masks that prune
the search ("Finer is Better (with the Right Scaling)", method part 2: the
scale of least block squared error among all representable ones, ties to
the smaller code).

The masks keep a code only if both the largest and the second largest
element of the block can reach an error within the best start SSE there
(blocks of 8 also within the branch-and-bound window),
with admissible intervals around S = a / r for the E2M1 grid values r.  The
cases below aim at every branch of that reasoning: blocks on exact grid
points (zero SSE, ties between codes), near-ties from tiny perturbations,
scales that fall on subnormal E4M3 codes and on the top code 126
(saturation), one dominant element with three tiny ones (the second element
admissible everywhere), equal magnitudes, and magnitudes spread over many
binades so that the per-tensor scale pushes blocks to both ends of the
code range."""
import numpy as np
import pytest

from microscaling_fp4_block_fp4q_amd import fp4q as F
from microscaling_fp4_block_fp4q_amd import synth as S

from gpu_helpers import compare_quant, gpu_quantize, note, oracle_quantize

pytestmark = pytest.mark.gpu

GRID = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def stress_blocks(rows: int, cols: int, seed: int, B: int = 4) -> np.ndarray:
    """fp32 [rows, cols] whose blocks of B cycle through the stress kinds."""
    rng = np.random.default_rng(seed)
    nb = rows * cols // B
    kind = np.arange(nb) % 8
    out = np.empty((nb, B), dtype=np.float64)
    sign = rng.choice([-1.0, 1.0], size=(nb, B))
    scale = 2.0 ** rng.integers(-12, 12, size=(nb, 1))
    g4 = GRID[rng.integers(0, 7, size=(nb, B))]
    base = rng.standard_normal((nb, B))
    out[:] = base
    # 0: exact grid values times a power of two (SSE 0 at some codes, ties)
    out[kind == 0] = (g4 * scale)[kind == 0]
    # 1: grid values with relative perturbations of a few ulps (near-ties)
    pert = 1.0 + rng.integers(-3, 4, size=(nb, B)) * 2.0 ** -23
    out[kind == 1] = (g4 * scale * pert)[kind == 1]
    # 2: one dominant element, three tiny ones
    dom = base.copy()
    dom[:, 1:] *= 1e-6
    out[kind == 2] = dom[kind == 2]
    # 3: equal magnitudes
    out[kind == 3] = (np.abs(base[:, :1]) * np.ones((1, B)))[kind == 3]
    # 4: magnitudes over many binades (per-tensor g pushes blocks to both code ends)
    out[kind == 4] = (base * 10.0 ** rng.uniform(-8, 8, size=(nb, 1)))[kind == 4]
    # 5: very small blocks (subnormal E4M3 codes at g = 1)
    out[kind == 5] = (base * 10.0 ** rng.uniform(-5, -2, size=(nb, 1)))[kind == 5]
    # 6: very large blocks (the top code saturates at g = 1)
    out[kind == 6] = (base * 10.0 ** rng.uniform(2, 4, size=(nb, 1)))[kind == 6]
    # 7: plain normal
    out = np.abs(out) * sign
    return S.cast(out.reshape(rows, cols), S.F32)


@pytest.mark.parametrize("gm,g", [(F.GLOBAL_NONE, 1.0), (F.GLOBAL_TENSOR_AMAX, None),
                                  (F.GLOBAL_USER, 0.0009765625), (F.GLOBAL_USER, 37.5)])
@pytest.mark.parametrize("seed", [1, 2])
@pytest.mark.parametrize("B", [4, 8])
def test_bf_stress(O_lib, gm, g, seed, B):
    x = stress_blocks(64, 1024, seed, B)
    cfg = F.config(F.E4M3, B, F.BRUTE_FORCE, gm, global_scale=g if g is not None else 1.0)
    note(f"bf stress B={B} gm={gm} g={g} seed={seed}")
    gpu = gpu_quantize(x, S.F32, cfg, dq_dt=None)
    ref = oracle_quantize(x, S.F32, cfg, dq_dt=None)
    assert gpu["g"].view(np.uint32) == ref["g"].view(np.uint32)
    compare_quant(gpu, ref, keys=("scales", "codes", "mse"))


@pytest.mark.parametrize("dt", [S.BF16, S.F16])
@pytest.mark.parametrize("H", [0, 16, 32])
@pytest.mark.parametrize("B", [4, 8])
def test_bf_stress_narrow_inputs(O_lib, dt, H, B):
    """bf16 / fp16 inputs (several blocks per lane) with and without rotation."""
    x = S.cast(stress_blocks(32, 2048, 7 + H, B).astype(np.float64) * 0.25, dt)
    cfg = F.config(F.E4M3, B, F.BRUTE_FORCE, F.GLOBAL_TENSOR_AMAX, hadamard=H)
    note(f"bf stress B={B} dt={dt} H={H}")
    gpu = gpu_quantize(x, dt, cfg, dq_dt=None)
    ref = oracle_quantize(x, dt, cfg, dq_dt=None)
    compare_quant(gpu, ref, keys=("scales", "codes", "mse"))
