"""Pins from values the pages print (tests/golden/, each line cited there)."""
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _facts(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            out[k] = v
    return out


def test_e4m3fn_max_is_448():
    f = _facts("e4m3fn_facts.txt")
    vals = oracle.decode("e4m3fn", np.arange(256, dtype=np.uint16).astype(np.uint8))
    assert np.nanmax(np.abs(vals)) == float(f["e4m3fn_max"])
    assert vals[int(f["e4m3fn_max_code"], 16)] == float(f["e4m3fn_max"])
