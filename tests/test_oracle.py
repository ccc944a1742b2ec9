"""The oracle against its pins (see oracle_pins.py), and proof that the pins
catch plausible mistakes: each mutation below plants one mistake in a copy of
oracle.c, builds it on the CPU, and at least one pin must fail."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.default())


# (what the mistake is, text in oracle.c, replacement)
MUTATIONS = [
    ("drop the last k term", "k < K; ++k", "k + 1 < K; ++k"),
    ("skip the first k term", "int64_t k = 0; k < K", "int64_t k = 1; k < K"),
    ("wrong sign", "acc += a * b;", "acc -= a * b;"),
    ("wrong sign (k-outer path)", "c[j] += a * b;", "c[j] -= a * b;"),
    ("transposed A strides", "A[i * sam + k * sak]", "A[i * sak + k * sam]"),
    ("B read transposed (k-inner path)", "B[k + j * sbn]", "B[j + k * sbn]"),
    ("B stride ignored (k-outer path)", "brow[j * sbn]", "brow[j]"),
    ("swapped B scale indices", "SB[(j / 128) * ssbn + (k / 128) * ssbk]",
     "SB[(k / 128) * ssbn + (j / 128) * ssbk]"),
    ("A scale by column block", "SA[i * ssam + (k / 128) * ssak]", "SA[i * ssam + (k / 127) * ssak]"),
    ("magnitude sum without abs", "mag += fabs(a) * fabs(b);", "mag += a * b;"),
    ("subnormal decode off by one", "v = ldexp((double)m, 1 - bias - mbits);",
     "v = ldexp((double)m, -bias - mbits);"),
    ("e4m3 exponent bias", "(int)e - 7 - 3", "(int)e - 8 - 3"),
    ("rounding by truncation", "ldexp(nearbyint(ldexp(x, -q)), q)", "ldexp(trunc(ldexp(x, -q)), q)"),
    ("rounding ties away", "ldexp(nearbyint(ldexp(x, -q)), q)", "ldexp(round(ldexp(x, -q)), q)"),
    ("quantiser scale over 447", "(double)amax / 448.0", "(double)amax / 447.0"),
    ("zero block keeps scale 0", "S[ib * ssr + kb * ssk] = zero ? 1.0f : sc;",
     "S[ib * ssr + kb * ssk] = sc;"),
    ("128 x 128 blocks one row tall", "r1 = r0 + br < R ? r0 + br : R;", "r1 = r0 + 1 < R ? r0 + 1 : R;"),
    ("quantiser drops the sign", "return (uint8_t)(lo | (signbit(v) ? 0x80 : 0));",
     "return (uint8_t)lo;"),
    ("quantiser amax of the first column only", "for (int64_t k = k0; k < k1; ++k) {\n          float a",
     "for (int64_t k = k0; k < k0 + 1; ++k) {\n          float a"),
    ("silu with e^g", "G[t] / (1.0 + exp(-G[t])) * U[t]", "G[t] / (1.0 + exp(G[t])) * U[t]"),
    ("gate and up swapped", "G[t] / (1.0 + exp(-G[t])) * U[t]", "U[t] / (1.0 + exp(-U[t])) * G[t]"),
    ("no sigmoid on the gate", "G[t] / (1.0 + exp(-G[t])) * U[t]", "G[t] * U[t]"),
    ("sigmoid without the gate factor", "G[t] / (1.0 + exp(-G[t])) * U[t]",
     "1.0 / (1.0 + exp(-G[t])) * U[t]"),
    ("bound constants of bf16 and fp16 swapped", "const int p = fmt == FMT_F16 ? 11 : 8;",
     "const int p = fmt == FMT_F16 ? 8 : 11;"),
    ("bound of eight unit roundoffs", "ldexp(4.0, -p) * S[t]", "ldexp(8.0, -p) * S[t]"),
    ("bound of one unit roundoff", "ldexp(4.0, -p) * S[t]", "ldexp(1.0, -p) * S[t]"),
]


_RUN_PINS = """
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_pins
orc = oracle.Oracle({lib!r})
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(orc)
    except Exception as e:
        failed.append(pin.__name__)
print("FAILED:" + ",".join(failed))
"""


@pytest.mark.parametrize("what,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(what, old, new):
    src = open(oracle._SRC).read()
    assert old in src, f"mutation target not found: {old}"
    tmp = tempfile.mkdtemp()
    try:
        path = os.path.join(tmp, "oracle_mut.c")
        open(path, "w").write(src.replace(old, new))
        lib = oracle.build(path, os.path.join(tmp, "liboracle_mut.so"))
        # a planted indexing mistake may read out of bounds, so the pins run in
        # a child process; a crash there also counts as caught
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        r = subprocess.run([sys.executable, "-c", _RUN_PINS.format(root=root, lib=lib)],
                           capture_output=True, text=True, timeout=600)
        caught = r.returncode != 0 or "FAILED:" in r.stdout and \
            r.stdout.strip().split("FAILED:")[-1] != ""
        assert caught, f"no pin caught the planted mistake: {what}\n{r.stdout}{r.stderr}"
    finally:
        shutil.rmtree(tmp)
