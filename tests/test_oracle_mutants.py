"""Mutation check of the oracle's pins.

Each mutant below is a copy of oracle/fp4q_oracle.c with one plausible
mistake planted (a wrong constant, sign, index, tie rule, bound or operand).
The oracle pin suite (tests/test_oracle_*.py) is run against every mutant
through FP4Q_ORACLE_LIB; a mutant that passes the whole suite would be a
mistake the pins cannot see, so every mutant must make the suite fail.
Mistakes are planted in copies on the CPU only; the real oracle source is
never modified.

Left out as equivalent (no input can tell them apart from the oracle): an
E8M0 brute force that stops before code 254.  The E2M1 grid at scale 2^126
contains every finite point of the grid at 2^127 (the larger points
overflow to infinity), so code 254 never has a strictly smaller SSE than
code 253 and ties go to the smaller code.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fp4q_oracle.c")
PIN_FILES = ["test_oracle_formats.py", "test_oracle_quant.py", "test_oracle_golden.py",
             "test_oracle_rotation.py", "test_oracle_focus.py", "test_oracle_search.py",
             "test_oracle_ue5m3.py", "test_oracle_histogram.py", "test_oracle_gemm.py"]

# (name, text in the oracle, replacement, which occurrence (1-based))
MUTANTS = [
    ("e2m1 tie to odd", "(d == best_d && (m & 1) == 0)", "(d == best_d && (m & 1) == 1)", 1),
    ("e2m1 NaN saturates", "if (isnan(u)) return 0;", "if (isnan(u)) return 7;", 1),
    ("e2m1 grid 5 for 6", "3.0, 4.0, 6.0}", "3.0, 4.0, 5.0}", 1),
    ("e4m3 subnormal step", "m * ldexp(1.0, -9)", "m * ldexp(1.0, -10)", 1),
    ("e4m3 exponent bias", "ldexp(1.0, e - 7)", "ldexp(1.0, e - 8)", 1),
    ("e4m3 tie to odd", "(d == best_d && (c & 1) == 0)", "(d == best_d && (c & 1) == 1)", 1),
    ("e8m0 abs-max maps onto 4", "(e - 1) - 2 + 127", "(e - 1) - 3 + 127", 1),
    ("e8m0 decode bias", "ldexp(1.0, code - 127)", "ldexp(1.0, code - 126)", 1),
    ("bf16 narrowing truncates", "double m = rne(ldexp(a, 7 - E));", "double m = floor(ldexp(a, 7 - E));", 1),
    ("f16 decode exponent", "(1024 + m) * ldexp(1.0, e - 25)", "(1024 + m) * ldexp(1.0, e - 24)", 1),
    ("fwht butterfly sign", "v[i + h] = a - b;", "v[i + h] = b - a;", 1),
    ("fwht unnormalised", "(float)(1.0 / sqrt((double)n))", "(float)(1.0 / (double)n)", 1),
    ("sse summed left to right",
     "if (n == 1) return v[0];",
     "if (n >= 1) { float s = 0.0f; for (int i = 0; i < n; ++i) s = s + v[i]; return s; }", 1),
    ("quotient by reciprocal", "float u = (S == 0.0f) ? 0.0f : y / S;",
     "float u = (S == 0.0f) ? 0.0f : y * (1.0f / S);", 1),
    ("sign of zero codes lost", "int neg = signbit(y) ? 1 : 0;", "int neg = (y < 0.0f) ? 1 : 0;", 1),
    ("dequant drops the sign", "*yhat = copysignf(v, neg ? -1.0f : 1.0f);", "*yhat = v;", 1),
    ("error with + instead of -", "float d = y[i] - yh;", "float d = y[i] + yh;", 1),
    ("block amax without abs", "uint32_t b = bits_of_f32(y[i]) & 0x7FFFFFFFu;\n        if (b > m) m = b;\n    }\n    return m;",
     "uint32_t b = bits_of_f32(y[i]);\n        if (b > m) m = b;\n    }\n    return m;", 1),
    ("global scale without the 6", "f32_of_bits(m) / 2688.0f", "f32_of_bits(m) / 448.0f", 1),
    ("zero tensor keeps g = 0", "return (g == 0.0f) ? 1.0f : g;", "return g;", 1),
    ("abs-max divides by 4", "int s6 = encode(a_b / six_g);", "int s6 = encode(a_b / (4.0f * g));", 1),
    ("prevent-zero missing", "return s6 < 1 ? 1 : s6;", "return s6;", 1),
    ("4-over-6 ties to s4", "return (sse4 < sse6) ? s4 : s6;", "return (sse4 <= sse6) ? s4 : s6;", 1),
    ("brute force skips 448", "int top_code = (fmt == SF_E4M3) ? 0x7E : 0xFE;",
     "int top_code = (fmt == SF_E4M3) ? 0x7D : 0xFE;", 1),
    ("ue5m3 exponent bias", "ldexp(1.0, e - 15)", "ldexp(1.0, e - 14)", 1),
    ("ue5m3 subnormal step", "m * ldexp(1.0, -17)", "m * ldexp(1.0, -18)", 1),
    ("ue5m3 tie to odd", "if (d < best_d || (d == best_d && (c & 1) == 0)) { best = c; best_d = d; }\n    }\n    return best;\n}\n\n/* MXFP4",
     "if (d < best_d || (d == best_d && (c & 1) == 1)) { best = c; best_d = d; }\n    }\n    return best;\n}\n\n/* MXFP4", 1),
    ("ue5m3 brute force skips the top code", "int top_code = (fmt == SF_E4M3) ? 0x7E : 0xFE;",
     "int top_code = (fmt == SF_E4M3) ? 0x7E : 0xFD;", 1),
    ("brute force ties to larger code", "if (best < 0 || sse < best_sse) { best = c; best_sse = sse; }",
     "if (best < 0 || sse <= best_sse) { best = c; best_sse = sse; }", 2),
    ("mse divides by B - 1", "float m = sse / (float)B;", "float m = sse / (float)(B - 1);", 1),
    ("nibbles swapped", "if ((col & 1) == 0) *byte = (uint8_t)q;\n                    else *byte = (uint8_t)(*byte | (q << 4));",
     "if ((col & 1) == 0) *byte = (uint8_t)(q << 4);\n                    else *byte = (uint8_t)(*byte | q);", 1),
    ("dequantize reads the wrong nibble", "int q = (c & 1) ? (byte >> 4) : (byte & 15);",
     "int q = (c & 1) ? (byte & 15) : (byte >> 4);", 1),
    ("focus S_q divides by c", "float S_q = S_dq * c_k;", "float S_q = S_dq / c_k;", 1),
    ("focus dequant with S_q", "wh = copysignf((float)E2M1_MAG[mag] * S_dq", "wh = copysignf((float)E2M1_MAG[mag] * S_q", 1),
    ("focus quotient ignores c", "float u = (S_q == 0.0f) ? 0.0f : W / S_q;", "float u = (S_q == 0.0f) ? 0.0f : W / S_dq;", 1),
    ("focus gradient sign", "out = -A / cc;", "out = A / cc;", 1),
    ("focus clip bound exclusive", "inside = fabsf(u) <= 6.0f;", "inside = fabsf(u) < 6.0f;", 1),
    ("focus gradient over c not c^2", "float cc = c_k * c_k;", "float cc = c_k;", 1),
    ("histogram drops the sign bit", "counts[q] += 1;", "counts[q & 7] += 1;", 1),
    ("gemm reads A's nibbles swapped", "int qa = (k & 1) ? (ab >> 4) : (ab & 15),",
     "int qa = (k & 1) ? (ab & 15) : (ab >> 4),", 1),
    ("gemm ignores B's scale", "double sb = oracle_e8m0_decode(b_scales[n * (K / 32) + k / 32]);", "double sb = 1.0;", 1),
    ("search ties to the larger shrink", "if (j == 0 || total < best_total ||", "if (j == 0 || total <= best_total ||", 1),
    ("search candidate step 1/32", "float g = g0 * (float)(1.0 - j / 64.0);", "float g = g0 * (float)(1.0 - j / 32.0);", 1),
    ("search result ignores the winner", "return g0 * (float)(1.0 - best / 64.0);", "return g0;", 1),
    ("search scores brute force as abs-max", "int code = choose_scale(SF_E4M3, strategy, yb, B, g, 0);",
     "int code = choose_scale(SF_E4M3, strategy == ST_BRUTE_FORCE ? ST_ABSMAX : strategy, yb, B, g, 0);", 1),
]


def _mutate(text, old, new, occurrence):
    if occurrence == 0:
        return text
    start = -1
    for _ in range(occurrence):
        start = text.index(old, start + 1)
    return text[:start] + new + text[start + len(old):]


def _run_mutant(tmp, k, name, old, new, occ, source):
    src = os.path.join(tmp, f"mutant_{k}.c")
    lib = os.path.join(tmp, f"libmutant_{k}.so")
    with open(src, "w") as f:
        f.write(_mutate(source, old, new, occ))
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                           "-o", lib, src, "-lm"])
    env = dict(os.environ, FP4Q_ORACLE_LIB=lib)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(ROOT, "tests", t) for t in PIN_FILES]]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-600:]


def test_mutant_table_applies():
    """Every planted mistake names text that exists in the oracle."""
    source = open(SRC).read()
    for name, old, new, occ in MUTANTS:
        assert source.count(old) >= occ, name
        assert _mutate(source, old, new, occ) != source, name


def test_every_mutant_is_caught():
    source = open(SRC).read()
    control = ("control (no mistake)", "", "", 0)     # the harness itself must pass the real oracle
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=4) as pool:
            results = list(pool.map(lambda a: _run_mutant(tmp, a[0], *a[1], source),
                                    enumerate([control] + MUTANTS)))
    (_, rc0, out0), results = results[0], results[1:]
    assert rc0 == 0, "the pin suite fails on an unmodified copy of the oracle:\n" + out0
    survivors = [name for name, rc, _ in results if rc == 0]
    unusual = [(name, rc, out) for name, rc, out in results if rc not in (0, 1)]
    assert not unusual, unusual      # collection errors or crashes are not a caught mistake
    assert not survivors, "mutants not caught by any pin: " + ", ".join(survivors)
