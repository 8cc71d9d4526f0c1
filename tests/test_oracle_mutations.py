"""Planted mistakes in the oracle must each fail a pin (CPU only).

Each case copies oracle/moe_oracle.c, plants one plausible mistake in the
copy (a wrong bit position, index, sign, operand, tie rule, bias or order),
builds it with gcc, and runs tests/test_oracle_pins.py against it in a
subprocess (MOE_ORACLE_SOURCE / MOE_ORACLE_LIBRARY point the oracle package
at the copy). The pins pass on the unchanged copy and fail on every mutant.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (label, text in moe_oracle.c, replacement)
MUTANTS = [
    ("fp16 exponent bias", "ldexp(1.0 + man / 1024.0, ex - 15)", "ldexp(1.0 + man / 1024.0, ex - 14)"),
    ("bf16 shift", "(uint32_t)b << 16", "(uint32_t)b << 15"),
    ("e2m1 exponent bias", "ldexp(1.0 + 0.5 * man, ex - 1)", "ldexp(1.0 + 0.5 * man, ex - 2)"),
    ("e4m3 exponent bias", "ldexp(1.0 + man / 8.0, ex - 7)", "ldexp(1.0 + man / 8.0, ex - 8)"),
    ("FWHT butterfly sign", "v[j + h] = a - b;", "v[j + h] = b - a;"),
    ("rotation drops the signs", "t[i] = (double)signs[b + i] * in[b + i];", "t[i] = in[b + i];"),
    ("2-bit code bit position", "bit[k] = 8 * (kk % 4) + 2 * (kk / 4) + k;",
     "bit[k] = 8 * (kk / 4) + 2 * (kk % 4) + k;"),
    ("3-bit code byte mapping", "bit[k] = 8 * (i % 4) + 3 * (i / 4) + k;",
     "bit[k] = 8 * (i / 2) + 3 * (i % 2) + k;"),
    ("3-bit high bit position", "bit[2] = 8 * (i % 4) + 6 + i / 4;", "bit[2] = 8 * (i % 4) + 7 - i / 4;"),
    ("6-bit code bit order", "bit[k] = (6 * jj + k) % 32;", "bit[k] = (6 * jj + 5 - k) % 32;"),
    ("6-bit tile not split", "tau * 384 + (word[k] / 3) * 192 + slot * 3 + word[k] % 3",
     "tau * 384 + slot * 6 + word[k]"),
    ("slot transposed", "int slot = q * 16 + r;", "int slot = r * 4 + q;"),
    ("group scale row-major", "orc_f16_to_double(scales[((long)(n / 16) * (C / 128) + c / 128) * 16 + n % 16]);",
     "orc_f16_to_double(scales[(long)n * (C / 128) + c / 128]);"),
    ("NVFP4 block scale row-major",
     "scales[((long)(n / 16) * (C / 128) + c / 128) * 128 + (n % 16) * 8 + (c % 128) / 16]);",
     "scales[(long)n * (C / 16) + c / 16]);"),
    ("NVFP4 nibble order", "return (jj % 2) ? (byte >> 4) : (byte & 0xF);",
     "return (jj % 2) ? (byte & 0xF) : (byte >> 4);"),
    ("top-k ties to the higher id", "if (best < 0 || l[e] > l[best])", "if (best < 0 || l[e] >= l[best])"),
    ("softmax denominator", "w[t * k + j] = exp((double)l[ids[t * k + j]] - l0) / den;",
     "w[t * k + j] = exp((double)l[ids[t * k + j]] - l0) / (den + 1.0);"),
    ("SiLU on the up projection", "h[n] = g[n] / (1.0 + exp(-g[n])) * u[n];",
     "h[n] = u[n] / (1.0 + exp(-u[n])) * g[n];"),
    ("down input not rotated", "orc_rotate(I, L->signs_inter, h, hr);", "memcpy(hr, h, sizeof(double) * I);"),
    ("combine slots reversed", "acc += w[t * k + j] * ys[(size_t)(p0 + j) * H + i];",
     "acc += w[t * k + (k - 1 - j)] * ys[(size_t)(p0 + j) * H + i];"),
    ("shared expert weight", "acc += ysh[(size_t)t * H + i];", "acc += 0.5 * ysh[(size_t)t * H + i];"),
]


def run_pins(tmp_path, text):
    src = tmp_path / "moe_oracle.c"
    src.write_text(text)
    env = dict(os.environ, MOE_ORACLE_SOURCE=str(src),
               MOE_ORACLE_LIBRARY=str(tmp_path / "liboracle.so"))
    return subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-m", "not gpu",
                           "-p", "no:cacheprovider"],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def test_pins_pass_on_an_unchanged_copy(tmp_path):
    r = run_pins(tmp_path, open(SRC).read())
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]
    assert (tmp_path / "liboracle.so").exists()  # the copy was built and used


@pytest.mark.parametrize("label,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, label, old, new):
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation anchor not found: {old}"
    r = run_pins(tmp_path, text.replace(old, new, 1))
    assert r.returncode == 1 and " failed" in r.stdout, (
        f"{label}: no pin failed\n" + r.stdout[-3000:] + r.stderr[-2000:])
