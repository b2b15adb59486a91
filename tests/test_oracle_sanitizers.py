"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/support/oracle_sanitize.c drives every oracle entry point (all
formats, blocks, strategies, global modes, rotations, element types,
invalid combinations, NaN / infinity / signed zero / subnormal inputs, the
FOCUS pair, the histogram and the MXFP4 GEMM) and prints a hash of every
output.  It is built twice with the oracle's own flags, once plainly and
once with -fsanitize=address,undefined (no recovery, leak checks on); both
must exit cleanly and print the same hashes.  The sanitizers run on host
code only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DRIVER = os.path.join(HERE, "support", "oracle_sanitize.c")
ORACLE = os.path.join(ROOT, "oracle", "fp4q_oracle.c")
FLAGS = ["-std=c11", "-O1", "-ffp-contract=off", "-fno-fast-math", "-g"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]

needs_gcc = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")


def _build(out, extra):
    subprocess.check_call(["gcc", *FLAGS, *extra, "-o", out, DRIVER, ORACLE, "-lm"])


def _run(exe):
    # verify_asan_link_order=0: the environment may preload other libraries
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)


@needs_gcc
def test_oracle_clean_under_asan_ubsan(tmp_path):
    plain, san = str(tmp_path / "plain"), str(tmp_path / "san")
    _build(plain, [])
    try:
        _build(san, SAN)
    except subprocess.CalledProcessError:
        pytest.skip("this gcc cannot link the sanitizer runtimes")
    a, b = _run(plain), _run(san)
    assert a.returncode == 0, a.stderr[-2000:]
    assert b.returncode == 0, b.stderr[-4000:]
    assert "runtime error" not in b.stderr and "AddressSanitizer" not in b.stderr, b.stderr[-4000:]
    lines = a.stdout.splitlines()
    assert len(lines) > 3000 and sum(" rc=0" in ln for ln in lines) > 500
    assert a.stdout == b.stdout
