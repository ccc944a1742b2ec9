"""Exhaustive pins of the number-format codecs used by the oracle and the
input generator, against torch / numpy dtype conversions and a brute-force
nearest-value search over every code of the format."""
import numpy as np
import pytest
import torch

import gen
import oracle


def _torch_decode(codes: np.ndarray, dtype) -> np.ndarray:
    t = torch.from_numpy(codes.copy())
    if dtype == torch.float8_e4m3fn:
        return t.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    return t.view(torch.int16).view(dtype).to(torch.float32).double().numpy()


def _same(a, b):
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_decode_bf16_exhaustive():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    assert _same(oracle.decode("bf16", codes), _torch_decode(codes, torch.bfloat16))


def test_decode_f16_exhaustive():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    assert _same(oracle.decode("f16", codes), ref)


def test_decode_e4m3fn_exhaustive():
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    got = oracle.decode("e4m3fn", codes)
    assert _same(got, _torch_decode(codes, torch.float8_e4m3fn))
    # "TileKernels deep dive" section 7.2: 448 is the largest E4M3 magnitude.
    assert np.nanmax(np.abs(got)) == 448.0
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0 and np.isnan(got[0x7F])


def _grid(fmt):
    """Sorted finite non-negative values and their codes for fp16 / bf16."""
    codes = np.arange(0x8000, dtype=np.uint16)
    vals = codes.view(np.float16).astype(np.float64) if fmt == "f16" else \
        _torch_decode(codes, torch.bfloat16)
    keep = np.isfinite(vals)
    return vals[keep], codes[keep]


def _nearest_even(x: np.ndarray, fmt: str) -> np.ndarray:
    """Brute-force round-to-nearest-even of |x| on the format's finite grid;
    returns codes with the sign of x; beyond the overflow threshold -> inf."""
    vals, codes = _grid(fmt)
    a = np.abs(x)
    hi = np.searchsorted(vals, a, side="left").clip(1, len(vals) - 1)
    lo = hi - 1
    exact = vals[hi] == a
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[hi] % 2 == 0))
    out = np.where(exact | pick_hi, codes[hi], codes[lo]).astype(np.uint16)
    top = vals[-1]
    half_ulp = (vals[-1] - vals[-2]) / 2
    inf_code = 0x7C00 if fmt == "f16" else 0x7F80
    out = np.where(a >= top + half_ulp, inf_code, out).astype(np.uint16)
    sign = np.where(np.signbit(x), 0x8000, 0).astype(np.uint16)
    return out | sign


def _probe_values(fmt, n=200000, seed=7):
    rng = np.random.default_rng(seed)
    vals, _ = _grid(fmt)
    # random magnitudes across the whole exponent range, plus exact ties and
    # values one fp64 ulp either side of each tie
    e = rng.uniform(np.log2(vals[1]) - 2, np.log2(vals[-1]) + 0.5, n)
    x = np.exp2(e) * rng.choice([-1.0, 1.0], n)
    i = rng.integers(0, len(vals) - 1, 20000)
    ties = (vals[i] + vals[i + 1]) / 2
    x = np.concatenate([x, ties, np.nextafter(ties, 0), np.nextafter(ties, np.inf), -ties,
                        vals, [0.0, -0.0]])
    return x


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_oracle_round_matches_bruteforce(fmt):
    x = _probe_values(fmt)
    assert np.array_equal(oracle.round_to(fmt, x), _nearest_even(x, fmt))


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_gen_round_matches_bruteforce(fmt):
    x = _probe_values(fmt, seed=11)
    got = gen.round_bf16(x) if fmt == "bf16" else gen.round_f16(x)
    assert np.array_equal(got, _nearest_even(x, fmt))


def test_round_matches_library_casts():
    rng = np.random.default_rng(3)
    x32 = rng.standard_normal(100000).astype(np.float32) * np.float32(37.0)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_to("bf16", x32.astype(np.float64)), ref)
    x64 = rng.standard_normal(100000) * 300.0
    assert np.array_equal(oracle.round_to("f16", x64), x64.astype(np.float16).view(np.uint16))


def test_gen_e4m3_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = (rng.uniform(-1, 1, 200000) * np.exp2(rng.uniform(-12, 8.8, 200000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    grid = _torch_decode(np.arange(256, dtype=np.uint16).astype(np.uint8), torch.float8_e4m3fn)
    i = np.arange(0, 0x7E)
    ties = ((grid[i] + grid[i + 1]) / 2).astype(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 448.0, -448.0])])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(gen.round_e4m3fn(x), ref)
