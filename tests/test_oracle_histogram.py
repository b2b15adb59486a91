"""Pins of the oracle's codebook-occupancy histogram (the TORQ page,
section 2.B: codeword usage and its collapse onto the smallest codes)."""
import numpy as np

E4M3, E8M0 = 1, 0


def test_counts_of_a_hand_built_array(O):
    # bytes 0x10, 0x32, 0xF8: nibbles (low first) 0, 1, 2, 3, 8, 15
    codes = np.array([[0x10, 0x32, 0xF8]], np.uint8)
    want = np.zeros(16, np.uint64)
    for q in (0, 1, 2, 3, 8, 15):
        want[q] += 1
    assert np.array_equal(O.code_histogram(codes), want)


def test_matches_numpy_bincount_on_quantized_tensors(O):
    rng = np.random.default_rng(8)
    for fmt, B, gm in ((E4M3, 16, 1), (E8M0, 32, 0), (E4M3, 4, 0)):
        x = rng.laplace(0, 1, (33, 256)).astype(np.float32)
        codes = O.quantize(x, fmt=fmt, block=B, global_mode=gm, dq_dt=None)["codes"]
        nibbles = np.stack([codes & 15, codes >> 4], axis=-1).reshape(-1)
        want = np.bincount(nibbles, minlength=16).astype(np.uint64)
        got = O.code_histogram(codes)
        assert np.array_equal(got, want)
        assert int(got.sum()) == x.size


def test_collapse_at_tiny_scale(O):
    """At 1e-4 with no per-tensor scale every E4M3 abs-max scale underflows
    and all codes collapse onto the two zero codes (region A of the
    Finer-is-Better page)."""
    x = (np.random.default_rng(1).standard_normal((8, 64)) * 1e-4).astype(np.float32)
    h = O.code_histogram(O.quantize(x, fmt=E4M3, block=16, dq_dt=None)["codes"])
    assert int(h[0] + h[8]) == x.size


def test_empty(O):
    assert not O.code_histogram(np.zeros((0, 8), np.uint8)).any()
