"""Exhaustive CPU check that the division-free quotient of the GPU kernels
(reciprocal + two FMAs) puts every element in the same E2M1 bin as the
correctly rounded quotient fl(a / S) that the specification uses, for every
fp32 scale mantissa (tests/support/check_markstein.c explains why that
covers every scale in [2^-100, 2^100])."""
import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "support", "check_markstein.c")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    so = str(tmp_path_factory.mktemp("mk") / "libcheck_markstein.so")
    subprocess.check_call(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fPIC", "-shared", "-o", so, SRC, "-lm"])
    lib = ctypes.CDLL(so)
    lib.check_markstein.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint64)]
    lib.check_markstein.restype = ctypes.c_int
    return lib


def test_bins_agree_for_every_scale_mantissa(checker):
    parts = 16
    step = (1 << 23) // parts

    def run(i):
        n, qm = ctypes.c_uint64(0), ctypes.c_uint64(0)
        bad = checker.check_markstein(i * step, (i + 1) * step, 6, ctypes.byref(n), ctypes.byref(qm))
        return bad, n.value, qm.value

    with ThreadPoolExecutor(8) as ex:
        res = list(ex.map(run, range(parts)))
    bad = sum(r[0] for r in res)
    checked = sum(r[1] for r in res)
    assert checked == (1 << 23) * 8 * 13
    assert bad == 0
    assert sum(r[2] for r in res) == 0       # the quotients themselves agree


def test_scale_code_quotient_for_every_divisor_mantissa(checker):
    """The block scale code rounds fl(a_b / fl(M g)) to a 3-bit mantissa
    (E4M3, UE5M3); the kernels form that quotient from fl(1 / fl(M g)) with
    the same two FMAs.  Around every grid point and midpoint of such a format
    (relative values 1 + k/16) and for every divisor mantissa, the quotients
    must equal the IEEE division's."""
    checker.check_markstein_scale.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int,
                                              ctypes.POINTER(ctypes.c_uint64)]
    checker.check_markstein_scale.restype = ctypes.c_int
    parts = 16
    step = (1 << 23) // parts

    def run(i):
        n = ctypes.c_uint64(0)
        bad = checker.check_markstein_scale(i * step, (i + 1) * step, 6, ctypes.byref(n))
        return bad, n.value

    with ThreadPoolExecutor(8) as ex:
        res = list(ex.map(run, range(parts)))
    assert sum(r[1] for r in res) == (1 << 23) * 16 * 13
    assert sum(r[0] for r in res) == 0
