"""The library on a caller's stream and inside a captured HIP graph.

Every entry point enqueues on the stream it is given and records no memset,
copy, allocation or synchronisation, so a sequence of calls can be captured
once and replayed.  The graph test captures five calls (NVFP4 4-over-6 with
the abs-max pre-pass, E4M3 brute force, the MSE-searched per-tensor scale,
dequantize, code histogram), refills the static input between replays, runs
the same calls eagerly between replays, and checks every replay against the
eager results and against the oracle.
"""
import numpy as np
import pytest
import torch

from microscaling_fp4_block_fp4q_amd import fp4q as F
from microscaling_fp4_block_fp4q_amd import synth as S
from oracle import oracle as O

from gpu_helpers import DEV, assert_same, note

pytestmark = pytest.mark.gpu

ROWS, COLS = 48, 1024
CFG_AMAX = F.nvfp4(F.FOUR_OVER_SIX)
CFG_BF = F.config(F.E4M3, 8, F.BRUTE_FORCE, F.GLOBAL_NONE)
CFG_SEARCH = F.config(F.E4M3, 16, F.ABSMAX, F.GLOBAL_SEARCH)


def u8(shape):
    return torch.empty(shape, dtype=torch.uint8, device=DEV)


def f32(shape):
    return torch.empty(shape, dtype=torch.float32, device=DEV)


class Buffers:
    """Every output of the five calls, preallocated."""

    def __init__(self):
        self.c1, self.s1, self.g1 = u8((ROWS, COLS // 2)), u8((ROWS, COLS // 16)), f32(1)
        self.dq1 = torch.empty((ROWS, COLS), dtype=torch.bfloat16, device=DEV)
        self.m1, self.w1 = f32((ROWS, COLS // 16)), u8(F.workspace_bytes(CFG_AMAX, ROWS, COLS))
        self.c2, self.s2 = u8((ROWS, COLS // 2)), u8((ROWS, COLS // 8))
        self.dq2, self.m2 = f32((ROWS, COLS)), f32((ROWS, COLS // 8))
        self.c3, self.s3, self.g3 = u8((ROWS, COLS // 2)), u8((ROWS, COLS // 16)), f32(1)
        self.w3 = u8(F.workspace_bytes(CFG_SEARCH, ROWS, COLS))
        self.dq4 = f32((ROWS, COLS))
        self.counts = torch.zeros(16, dtype=torch.int64, device=DEV)   # uint64 counts, small values

    def run(self, x):
        F.fp4q_quantize(CFG_AMAX, x, self.c1, self.s1, self.g1, self.dq1, self.m1, self.w1)
        F.fp4q_quantize(CFG_BF, x, self.c2, self.s2, None, self.dq2, self.m2, None)
        F.fp4q_quantize(CFG_SEARCH, x, self.c3, self.s3, self.g3, None, None, self.w3)
        F.fp4q_dequantize(CFG_AMAX, self.c1, self.s1, self.dq4, self.g1)
        F.fp4q_code_histogram(self.c2, self.counts)

    def host(self):
        names = ("c1", "s1", "g1", "dq1", "m1", "c2", "s2", "dq2", "m2", "c3", "s3", "g3", "dq4", "counts")
        return {n: S.from_torch(getattr(self, n)) for n in names}


def check_against_oracle(x, out, counts_before):
    """Compare one run's outputs with the oracle; the histogram accumulates
    onto counts_before.  Returns the expected counts after this run."""
    r1 = O.quantize(x, fmt=F.E4M3, block=16, strategy=F.FOUR_OVER_SIX, global_mode=F.GLOBAL_TENSOR_AMAX,
                    dq_dt=S.BF16)
    for k, v in (("c1", "codes"), ("s1", "scales"), ("dq1", "dequant"), ("m1", "mse")):
        assert_same(out[k], r1[v], k)
    assert out["g1"][0].view(np.uint32) == np.float32(r1["g"]).view(np.uint32)
    r2 = O.quantize(x, fmt=F.E4M3, block=8, strategy=F.BRUTE_FORCE, global_mode=F.GLOBAL_NONE)
    for k, v in (("c2", "codes"), ("s2", "scales"), ("dq2", "dequant"), ("m2", "mse")):
        assert_same(out[k], r2[v], k)
    r3 = O.quantize(x, fmt=F.E4M3, block=16, strategy=F.ABSMAX, global_mode=F.GLOBAL_SEARCH, dq_dt=None)
    assert_same(out["c3"], r3["codes"], "c3")
    assert_same(out["s3"], r3["scales"], "s3")
    assert out["g3"][0].view(np.uint32) == np.float32(r3["g"]).view(np.uint32)
    r4 = O.dequantize(r1["codes"], r1["scales"], r1["g"], fmt=F.E4M3, block=16, rows=ROWS, cols=COLS)
    assert_same(out["dq4"], r4, "dq4")
    counts = counts_before + O.code_histogram(r2["codes"])
    assert np.array_equal(out["counts"].astype(np.uint64), counts), "counts"
    return counts


def test_side_stream(O_lib):
    x = S.laplace(ROWS, COLS, 51)
    note("calls on a side stream")
    s = torch.cuda.Stream()
    xt = S.to_torch(x, S.F32, DEV)
    s.wait_stream(torch.cuda.current_stream())      # xt was written on the current stream
    with torch.cuda.stream(s):
        b = Buffers()
        b.run(xt)
    s.synchronize()
    out = b.host()
    check_against_oracle(x, out, np.zeros(16, np.uint64))


def test_graph_replay_matches_eager(O_lib):
    inputs = [S.laplace(ROWS, COLS, 60), S.normal(ROWS, COLS, 61), S.scaled_fp32(S.normal(ROWS, COLS, 62), 1e-4),
              S.laplace(ROWS, COLS, 63)]
    x_static = S.to_torch(inputs[0], S.F32, DEV)
    graph_bufs, eager_bufs = Buffers(), Buffers()
    note("graph warm-up (eager)")
    graph_bufs.run(x_static)                      # loads every kernel before capture
    torch.cuda.synchronize()
    graph_bufs.counts.zero_()
    torch.cuda.synchronize()
    note("graph capture")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        graph_bufs.run(x_static)
    torch.cuda.synchronize()
    counts_sum = np.zeros(16, np.uint64)
    for k, x in enumerate(inputs):
        note(f"graph replay {k}")
        x_static.copy_(S.to_torch(x, S.F32, DEV))
        graph.replay()
        torch.cuda.synchronize()
        got = graph_bufs.host()
        # the same calls eagerly, into other buffers, between the replays
        eager_bufs.counts.zero_()
        eager_bufs.run(S.to_torch(x, S.F32, DEV))
        torch.cuda.synchronize()
        want = eager_bufs.host()
        for name in got:
            if name != "counts":
                assert_same(got[name], want[name], f"replay {k}: {name}")
        counts_sum = check_against_oracle(x, got, counts_sum)


def test_allocating_wrappers_take_the_stream_argument(O_lib):
    """quantize(..., stream=s) with s not the current stream: outputs and
    workspace are allocated on s and the kernels run on s, while the current
    stream keeps allocating and filling buffers of the workspace's size (which
    would reuse a workspace released to the wrong stream)."""
    x = S.laplace(ROWS, COLS, 61)
    xt = S.to_torch(x, S.F32, DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    note("allocating wrappers on a stream argument")
    nbytes = max(F.workspace_bytes(CFG_AMAX, ROWS, COLS), 16)
    results, junk = [], []
    for _ in range(6):
        results.append(F.quantize(xt, CFG_AMAX, dequant_dtype=torch.float32, stream=s))
        junk.append(torch.full((nbytes,), 255, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    ref = O.quantize(x, fmt=CFG_AMAX.scale_fmt, block=16, strategy=F.FOUR_OVER_SIX,
                     global_mode=F.GLOBAL_TENSOR_AMAX)
    for r in results:
        assert S.from_torch(r["g"])[0].view(np.uint32) == np.float32(ref["g"]).view(np.uint32)
        for k in ("codes", "scales", "dequant", "mse"):
            assert_same(S.from_torch(r[k]), ref[k], k)
