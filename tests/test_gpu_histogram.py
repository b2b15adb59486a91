"""GPU parity of the codebook-occupancy histogram (TORQ page, section 2.B)
against the oracle: exact integer counts on random bytes with ragged sizes,
an empty tensor, and the codes the library itself produces on the 4096 x
4096 workload (including the collapse onto the zero codes at 1e-4)."""
import numpy as np
import pytest
import torch

from microscaling_fp4_block_fp4q_amd import fp4q as F
from microscaling_fp4_block_fp4q_amd import synth as S
from oracle import oracle as O

from gpu_helpers import DEV, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols", [(1, 2), (3, 30), (37, 4002), (1000, 8192), (0, 64), (5, 0)])
def test_random_bytes(O_lib, rows, cols):
    codes = np.random.default_rng(rows + cols).integers(0, 256, (rows, cols // 2)).astype(np.uint8)
    note(f"histogram random {rows}x{cols}")
    got = F.code_histogram(torch.from_numpy(codes).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().astype(np.uint64), O.code_histogram(codes))


@pytest.mark.parametrize("kind", ["normal", "normal_1e-4"])
def test_codes_of_the_workload(O_lib, kind):
    x = S.config2()[kind]
    cfg = F.config(F.E4M3, 16, F.ABSMAX, F.GLOBAL_NONE)
    note(f"histogram of quantized {kind} 4096x4096")
    r = F.quantize(S.to_torch(x, S.F32, DEV), cfg, want_mse=False)
    got = F.code_histogram(r["codes"])
    torch.cuda.synchronize()
    want = O.code_histogram(r["codes"].cpu().numpy())
    assert np.array_equal(got.cpu().numpy().astype(np.uint64), want)
    assert int(want.sum()) == x.size
    if kind == "normal_1e-4":
        assert int(want[0] + want[8]) == x.size          # every E4M3 scale underflows without g
