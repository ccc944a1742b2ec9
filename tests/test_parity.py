"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle.

Two acceptance modes, element by element:
  bound mode      |C_gpu - C_ref| <= 4*2^-8 * sum_k |a||b|  (bf16 output),
                                    4*2^-11 * sum_k |a||b| (fp16 output);
  bit-exact mode  integer inputs with K*r^2 <= 2^24, so every fp32 partial sum
                  is exact: C_gpu must equal round-to-nearest-even(C_ref).
Small cases span several tiles and ragged tails and are checked in full; the
five workloads run at their real sizes in the launch configuration the
benchmark times: fp16 256^3, bf16 4096^3 and the skinny product checked in
full, the two 4096 x 7168 x 16384 products on 256 seeded rows (and fully
through a selection matrix, whose product is known without the oracle).
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import gen
import oracle
from gen import configs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

FULL = os.environ.get("TG_FULL_TEST") == "1"


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    return gpu_lib


# ------------------------------------------------------------ small shapes

SHAPES = [(1, 1, 1), (13, 7, 5), (64, 64, 64), (65, 129, 33), (128, 256, 512), (200, 300, 170),
          (256, 256, 256), (1, 257, 1000), (300, 1, 77), (5, 3, 0), (257, 255, 4100)]


def _layout_args(fmt, M, N, K, layout, seed, int_r=None):
    """Device operands for a storage layout; returns (A, sam, sak, B, sbk, sbn,
    a_host_view, b_host_view) where the host views give A[i,k] and B[k,j]
    through (flat array, strides) for the oracle."""
    draw = (lambda shape, stream: gen.integers(shape, seed, stream, int_r, fmt)) if int_r \
        else (lambda shape, stream: gen.normal(shape, seed, stream, fmt))
    if layout == "nk":                  # A row-major, B stored N x K
        A, B = draw((M, K), 0), draw((N, K), 1)
        return A, K, 1, B, 1, K
    if layout == "kn":                  # A row-major, B stored K x N
        A, B = draw((M, K), 0), draw((K, N), 1)
        return A, K, 1, B, N, 1
    if layout == "padded":              # leading dimensions padded by 24 elements
        A = np.zeros((M, K + 24), np.uint16)
        A[:, :K] = draw((M, K), 0)
        B = np.zeros((N, K + 24), np.uint16)
        B[:, :K] = draw((N, K), 1)
        return A, K + 24, 1, B, 1, K + 24
    if layout == "kn_padded":           # B stored K x N with rows padded by 40 elements
        A = draw((M, K), 0)
        B = np.zeros((K, N + 40), np.uint16)
        B[:, :N] = draw((K, N), 1)
        return A, K, 1, B, N + 40, 1
    if layout == "colmajor":            # A stored K x M (A^T row-major), B K x N
        A, B = draw((K, M), 0), draw((K, N), 1)
        return A, 1, M, B, N, 1
    raise ValueError(layout)


def _check16(fmt, M, N, K, layout, seed, int_r=None, scm=None, ws=None):
    A, sam, sak, B, sbk, sbn = _layout_args(fmt, M, N, K, layout, seed, int_r)
    H.log(f"gemm {fmt} M={M} N={N} K={K} layout={layout} int_r={int_r} scm={scm} ws={bool(ws)}")
    c, plan = H.run16(fmt, M, N, K, H.dev(A), sam, sak, H.dev(B), sbk, sbn, scm=scm, ws=ws)
    C_ref, S = oracle.gemm(fmt, M, N, K, A, sam, sak, B, sbk, sbn)
    what = f"{fmt} {M}x{N}x{K} {layout} [{plan}]"
    if int_r:
        H.assert_bit_exact(fmt, c, C_ref, what)
    else:
        H.assert_within_bound(fmt, c, C_ref, S, what)
    return plan


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
@pytest.mark.parametrize("layout", ["nk", "kn", "padded", "colmajor"])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_small_bound(fmt, layout, shape):
    M, N, K = shape
    _check16(fmt, M, N, K, layout, seed=100 + M + N + K)


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
@pytest.mark.parametrize("layout", ["nk", "kn"])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_small_bit_exact(fmt, layout, shape):
    M, N, K = shape
    # K*r^2 <= 2^24 keeps every fp32 partial sum exact; fp16 output also keeps
    # typical sums below its 65504 maximum
    r = max(1, min(64 if fmt == "bf16" else 16, int(math.sqrt(2 ** 24 / max(K, 1)))))
    _check16(fmt, M, N, K, layout, seed=200 + M + N + K, int_r=r)


def test_padded_c_rows():
    _check16("bf16", 100, 90, 64, "nk", seed=7, scm=96)
    _check16("f16", 100, 90, 64, "kn", seed=8, scm=130)


def test_rne_ties_bf16():
    """Sums that are exact ties between bf16 neighbours round to even:
    257 -> 256, 259 -> 260, 261 -> 260, 263 -> 264, -257 -> -256."""
    M, N, K = 64, 64, 64
    a = np.zeros((M, K))
    a[:, 0] = 1.0
    a[:, 1] = 1.0
    b = np.zeros((K, N))
    b[0, :] = 256.0
    b[1, :] = np.resize([1.0, 3.0, 5.0, 7.0, -513.0], N)
    A = gen.round_bf16(a)
    B = gen.round_bf16(b)
    c, plan = H.run16("bf16", M, N, K, H.dev(A), K, 1, H.dev(B), N, 1)
    want = gen.round_bf16(np.resize([256.0, 260.0, 260.0, 264.0, -256.0], N)[None, :].repeat(M, 0))
    assert np.array_equal(c, want), plan


# --------------------------------------------------------------- workloads

def _wl_rows(w):
    """None (every row) for the workloads checked in full -- fp16 256^3, bf16
    4096^3 and the skinny 64 x 7168 x 7168 -- else the workload's seeded
    sample of rows (256 for the two 4096 x 7168 x 16384 products)."""
    if FULL or w.check_rows == 0:
        return None
    return gen.sample_rows(w.M, w.check_rows, w.seed)


def _run_workload16(w, d, ws=False):
    A, B = H.dev(d["A"]), H.dev(d["B"])
    H.log(f"workload {w.name}: {w.M}x{w.N}x{w.K} layout={d['layout']} ws={ws}")
    return H.run16(w.dtype, w.M, w.N, w.K, A, w.K, 1, B, d["sbk"], d["sbn"], ws=ws)


def _oracle16(w, d, rows):
    return oracle.gemm(w.dtype, w.M, w.N, w.K, d["A"], w.K, 1, d["B"], d["sbk"], d["sbn"],
                       rows=rows)


WL16 = [k for k in configs.ORDER if configs.WORKLOADS[k].dtype != "fp8"]


# Each workload through the allocation-free entry point and, where it has a
# split plan (the skinny product), through the workspace entry point too.
WL16_CALLS = [(k, False) for k in WL16] + [("bf16_skinny_64x7168x7168", True)]
WL16_IDS = [f"{k}{'-ws' if ws else ''}" for k, ws in WL16_CALLS]


@pytest.mark.parametrize("name,ws", WL16_CALLS, ids=WL16_IDS)
def test_workload_bound(name, ws):
    w = configs.WORKLOADS[name]
    d = configs.make_inputs(w)
    c, plan = _run_workload16(w, d, ws)
    rows = _wl_rows(w)
    C_ref, S = _oracle16(w, d, rows)
    H.assert_within_bound(w.dtype, c if rows is None else c[rows], C_ref, S, f"{name} [{plan}]")


@pytest.mark.parametrize("name,ws", WL16_CALLS, ids=WL16_IDS)
def test_workload_bit_exact(name, ws):
    w = configs.WORKLOADS[name]
    r = int(math.sqrt(2 ** 24 / w.K))
    if w.dtype == "f16":
        r = min(r, 16)
    d = configs.make_inputs(w, int_r=r)
    c, plan = _run_workload16(w, d, ws)
    rows = _wl_rows(w)
    C_ref, _ = _oracle16(w, d, rows)
    H.assert_bit_exact(w.dtype, c if rows is None else c[rows], C_ref, f"{name} int r={r} [{plan}]")


@pytest.mark.parametrize("name", ["bf16_4096x7168x16384", "bf16_4096", "bf16_skinny_64x7168x7168"])
def test_workload_selection_full(name):
    """A[i,k] = 1 iff k = pi(i): every element of C must equal B[pi(i), j]."""
    w = configs.WORKLOADS[name]
    d = configs.make_inputs(w)
    pi = np.random.default_rng(w.seed).permutation(w.K)[: w.M]
    A = np.zeros((w.M, w.K), np.uint16)
    A[np.arange(w.M), pi] = 0x3F80
    H.log(f"selection {name}")
    c, plan = H.run16(w.dtype, w.M, w.N, w.K, H.dev(A), w.K, 1, H.dev(d["B"]), d["sbk"], d["sbn"])
    Bkn = d["B"] if d["layout"] == "kn" else d["B"].T
    assert np.array_equal(c, Bkn[pi, :]), f"{name} selection [{plan}]"


def test_workload_deterministic():
    w = configs.WORKLOADS["bf16_4096x7168x16384"]
    d = configs.make_inputs(w)
    A, B = H.dev(d["A"]), H.dev(d["B"])
    H.log("determinism bf16_4096x7168x16384")
    c1, _ = H.run16("bf16", w.M, w.N, w.K, A, w.K, 1, B, d["sbk"], d["sbn"])
    c2, _ = H.run16("bf16", w.M, w.N, w.K, A, w.K, 1, B, d["sbk"], d["sbn"])
    assert np.array_equal(c1, c2)


# ----------------------------------------------------------------- fp8

def _fp8_inputs(M, N, K, seed, layout="nk", int_r=None, pow2_scales=False):
    w = configs.Workload("t", "fp8", M, N, K, layout, "normal", seed, 0)
    d = configs.make_inputs(w, int_r=int_r)
    if pow2_scales:
        rng = np.random.default_rng(seed)
        d["SA"] = np.exp2(rng.integers(-2, 3, d["SA"].shape)).astype(np.float32)
        d["SB"] = np.exp2(rng.integers(-2, 3, d["SB"].shape)).astype(np.float32)
    return d


def _check_fp8(M, N, K, d, rows=None, exact=False, what="", ws=None):
    nkb = d["SA"].shape[1]
    A, B, SA, SB = H.dev(d["A"]), H.dev(d["B"]), H.dev(d["SA"]), H.dev(d["SB"])
    H.log(f"fp8 {what} M={M} N={N} K={K} layout={d['layout']} ws={ws is not None}")
    c, plan = H.run_fp8(M, N, K, A, K, 1, SA, nkb, 1, B, d["sbk"], d["sbn"], SB, nkb, 1, ws=ws)
    C_ref, S = oracle.gemm_fp8_blockscaled(M, N, K, d["A"], K, 1, d["SA"], nkb, 1, d["B"],
                                           d["sbk"], d["sbn"], d["SB"], nkb, 1, rows=rows)
    cc = c if rows is None else c[rows]
    if exact:
        H.assert_bit_exact("bf16", cc, C_ref, f"fp8 {what} [{plan}]")
    else:
        H.assert_within_bound("bf16", cc, C_ref, S, f"fp8 {what} [{plan}]")
    return plan


FP8_SHAPES = [(1, 1, 1), (64, 64, 128), (13, 200, 300), (130, 129, 257), (256, 256, 1024),
              (512, 384, 640), (5, 3, 0)]


@pytest.mark.parametrize("shape", FP8_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in FP8_SHAPES])
@pytest.mark.parametrize("layout", ["nk", "kn"])
def test_fp8_small(layout, shape):
    M, N, K = shape
    _check_fp8(M, N, K, _fp8_inputs(M, N, K, 300 + M + K, layout), what="bound")
    _check_fp8(M, N, K, _fp8_inputs(M, N, K, 400 + M + K, layout, int_r=16), exact=True,
               what="int unit scales")
    _check_fp8(M, N, K, _fp8_inputs(M, N, K, 500 + M + K, layout, int_r=4, pow2_scales=True),
               exact=True, what="int pow2 scales")


# Shapes the 256 x 256 fp8 tiles take (grids large enough): ragged M, N and K,
# N not a multiple of 256 (the last tile's second half has no B scale row) or
# of 128, one partial slice.  Rows checked: the first and last 40 (ragged
# last tile row) and 128 seeded ones, every column of each.
FP8_WIDE_CASES = [(4000, 4000, 400), (4096, 3968, 1040), (4097, 4000, 16), (2500, 7000, 2064)]


def _edge_rows(M, seed):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(min(40, M)), np.arange(max(0, M - 40), M),
                           rng.choice(M, size=min(128, M), replace=False)])
    return np.unique(rows)


@pytest.mark.parametrize("case", FP8_WIDE_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in FP8_WIDE_CASES])
def test_fp8_wide_tile(case):
    M, N, K = case
    rows = _edge_rows(M, M + N + K)
    plan = _check_fp8(M, N, K, _fp8_inputs(M, N, K, 1500 + M + K), rows=rows, what="wide bound")
    assert plan == "tile_fp8_256x256", plan
    plan = _check_fp8(M, N, K, _fp8_inputs(M, N, K, 1600 + M + K, int_r=16), rows=rows,
                      exact=True, what="wide int unit scales")
    assert plan == "tile_fp8_256x256", plan
    plan = _check_fp8(M, N, K, _fp8_inputs(M, N, K, 1700 + M + K, int_r=4, pow2_scales=True),
                      rows=rows, exact=True, what="wide int pow2 scales")
    assert plan == "tile_fp8_256x256", plan


def test_fp8_workload_bound():
    w = configs.WORKLOADS["fp8_4096x7168x16384"]
    d = configs.make_inputs(w)
    _check_fp8(w.M, w.N, w.K, d, rows=_wl_rows(w), what=w.name)


def test_fp8_workload_bit_exact():
    w = configs.WORKLOADS["fp8_4096x7168x16384"]
    d = configs.make_inputs(w, int_r=16)
    _check_fp8(w.M, w.N, w.K, d, rows=_wl_rows(w), exact=True, what=w.name + " int")


# ------------------------------------------------------- tuned tile kernels

# (M, N, K, expected plan): ragged edges in M, N and K (K a multiple of 8 but
# not of the 64-wide slice; a single slice, so every slice the deeper stage
# rings prefetch lies past K), each tile shape of the N x K kernel.
TILE_CASES = [
    (4000, 3000, 8, "tile_nt_256x224"),
    (2200, 2000, 8, "tile_nt_128x128_2stage"),
    (3900, 3100, 72, "tile_nt_256x224"),
    (4000, 3000, 136, "tile_nt_256x224"),
    (4000, 4000, 136, "tile_nt_256x256"),
    (300, 500, 136, "tile_nt_128x128"),
    (513, 449, 72, "tile_nt_128x128"),
    (256, 224, 64, "tile_nt_128x128"),
    (65, 1, 8, "tile_nt_128x128"),
]


@pytest.mark.parametrize("case", TILE_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in TILE_CASES])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_tile_nt_ragged(fmt, case):
    M, N, K, want = case
    plan = _check16(fmt, M, N, K, "nk", seed=600 + M + N + K)
    assert plan == want
    r = max(1, min(64 if fmt == "bf16" else 16, int(math.sqrt(2 ** 24 / K))))
    plan = _check16(fmt, M, N, K, "nk", seed=700 + M + N + K, int_r=r)
    assert plan == want


# Grids of more than one round of eight-wave tiles (256 run at once): the
# workgroups of the second round take their K slices from the top down, the
# first of them a partial slice here (K not a multiple of 64).
ROUND_CASES = [
    (4000, 4600, 1000, "nk", "tile_nt_256x224"),
    (4100, 4400, 520, "nk", "tile_nt_256x224"),
    (4400, 4200, 1000, "kn", "tile_nn_256x256"),
]


@pytest.mark.parametrize("case", ROUND_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}{c[3]}" for c in ROUND_CASES])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_two_round_grids(fmt, case):
    M, N, K, layout, want = case
    plan = _check16(fmt, M, N, K, layout, seed=800 + M + N + K)
    assert plan == want
    r = max(1, min(64 if fmt == "bf16" else 16, int(math.sqrt(2 ** 24 / K))))
    plan = _check16(fmt, M, N, K, layout, seed=900 + M + N + K, int_r=r)
    assert plan == want


def test_tile_nt_padded_leading_dims():
    """Leading dimensions padded to multiples of 8 (not of the tile)."""
    M, N, K = 520, 460, 200
    plan = _check16("bf16", M, N, K, "padded", seed=31)
    assert plan.startswith("tile_nt"), plan


# ---------------------------------------------------- split-K tile kernel

# (M, N, K, expected plan): too few 256 x 224 tiles to fill the CUs.  With
# K of more than 128 slices of 64 the 256 x 224 tile splits K across each
# tile's workgroups, every split count 2 .. 8 (each its own combine); ragged
# M, N and K tails.  Checked on sampled rows (and the last row).
SPLITK_CASES = [
    (2000, 3500, 8200, "tile_nt_256x224_splitk2"),
    (1200, 3500, 8200, "tile_nt_256x224_splitk3"),
    (1000, 3500, 8264, "tile_nt_256x224_splitk4"),
    (1000, 2600, 8200, "tile_nt_256x224_splitk5"),
    (700, 3000, 8200, "tile_nt_256x224_splitk6"),
    (700, 2600, 8456, "tile_nt_256x224_splitk7"),
    (200, 300, 8200, "tile_nt_256x224_splitk7"),
]


def _check16_rows(fmt, M, N, K, seed, int_r=None, extra_rows=(), ws=None):
    """B stored N x K; the GPU result on sampled rows (and the last row, and
    `extra_rows`)."""
    draw = (lambda shape, st: gen.integers(shape, seed, st, int_r, fmt)) if int_r \
        else (lambda shape, st: gen.normal(shape, seed, st, fmt))
    A, B = draw((M, K), 0), draw((N, K), 1)
    H.log(f"gemm {fmt} M={M} N={N} K={K} rows int_r={int_r} ws={bool(ws)}")
    c, plan = H.run16(fmt, M, N, K, H.dev(A), K, 1, H.dev(B), 1, K, ws=ws)
    rows = np.union1d(np.union1d(gen.sample_rows(M, 48, seed), [M - 1]),
                      np.asarray(extra_rows, dtype=np.int64))
    C_ref, S = oracle.gemm(fmt, M, N, K, A, K, 1, B, 1, K, rows=rows)
    what = f"{fmt} {M}x{N}x{K} rows [{plan}]"
    if int_r:
        H.assert_bit_exact(fmt, c[rows], C_ref, what)
    else:
        H.assert_within_bound(fmt, c[rows], C_ref, S, what)
    return plan


@pytest.mark.parametrize("case", SPLITK_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in SPLITK_CASES])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_tile_nt_split_k(fmt, case):
    M, N, K, want = case
    plan = _check16_rows(fmt, M, N, K, seed=1500 + M + N + K, ws=True)
    assert plan == want, plan
    r = max(1, min(64 if fmt == "bf16" else 16, int(math.sqrt(2 ** 24 / K))))
    plan = _check16_rows(fmt, M, N, K, seed=1600 + M + N + K, int_r=r, ws=True)
    assert plan == want, plan
    # the allocation-free plan of the same call (128 x 128 tiles, unsplit)
    plan = _check16_rows(fmt, M, N, K, seed=1600 + M + N + K, int_r=r)
    assert plan.startswith("tile_nt_128x128") and "split" not in plan, plan


# (M, N, K, expected plan): grids of one whole wave (256 workgroups) of
# 256 x 224 tiles and a partial one split the partial wave's tiles over K --
# whole tiles and split tiles in one launch; ragged M, N and K; 2 and 3
# splits.  Checked in full.
TAIL_CASES = [
    (4352, 4096, 1024, "tile_nt_256x224_tail2"),
    (4400, 4000, 2056, "tile_nt_256x224_tail3"),
]


@pytest.mark.parametrize("case", TAIL_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in TAIL_CASES])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_tile_nt_tail(fmt, case):
    M, N, K, want = case
    plan = _check16(fmt, M, N, K, "nk", seed=1900 + M + N + K, ws=True)
    assert plan == want, plan
    r = max(1, min(64 if fmt == "bf16" else 16, int(math.sqrt(2 ** 24 / K))))
    plan = _check16(fmt, M, N, K, "nk", seed=2000 + M + N + K, int_r=r, ws=True)
    assert plan == want, plan
    plan = _check16(fmt, M, N, K, "nk", seed=2000 + M + N + K, int_r=r)
    assert plan == "tile_nt_256x224", plan


def test_tile_nt_tail5_rows():
    """4300 x 4000 x 4104: 306 tiles of 256 x 224, the last 50 (tile rows 12
    to 16) split 5 ways; sampled rows plus rows of every split tile row,
    bound and bit-exact."""
    M, N, K = 4300, 4000, 4104
    extra = list(range(3072, M, 37))
    plan = _check16_rows("bf16", M, N, K, seed=2101, extra_rows=extra, ws=True)
    assert plan == "tile_nt_256x224_tail5", plan
    plan = _check16_rows("bf16", M, N, K, seed=2102, int_r=63, extra_rows=extra, ws=True)
    assert plan == "tile_nt_256x224_tail5", plan


# (M, N, K, expected plan): small grids with K of at most 128 slices take
# 128 x 128 tiles, split K across up to 8 workgroups per tile (at least 16
# slices each); every split count, ragged tails; checked in full.  Grids of
# more than 256 such tiles take the two-stage version (two workgroups per CU).
SPLITK128_CASES = [
    (1000, 1000, 1000, "tile_nt_128x128"),
    (300, 500, 2048, "tile_nt_128x128_splitk2"),
    (257, 223, 3080, "tile_nt_128x128_splitk3"),
    (520, 230, 4104, "tile_nt_128x128_splitk4"),
    (130, 250, 5504, "tile_nt_128x128_splitk5"),
    (96, 700, 6504, "tile_nt_128x128_splitk6"),
    (65, 100, 7496, "tile_nt_128x128_splitk7"),
    (200, 300, 8192, "tile_nt_128x128_splitk8"),
    (2200, 2000, 200, "tile_nt_128x128_2stage"),
]


@pytest.mark.parametrize("case", SPLITK128_CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in SPLITK128_CASES])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_tile_nt_128(fmt, case):
    M, N, K, want = case
    plan = _check16(fmt, M, N, K, "nk", seed=1700 + M + N + K, ws=True)
    assert plan == want, plan
    r = max(1, min(64 if fmt == "bf16" else 16, int(math.sqrt(2 ** 24 / K))))
    plan = _check16(fmt, M, N, K, "nk", seed=1800 + M + N + K, int_r=r, ws=True)
    assert plan == want, plan
    if "split" in want:
        plan = _check16(fmt, M, N, K, "nk", seed=1800 + M + N + K, int_r=r)
        assert plan == "tile_nt_128x128", plan


def test_split_k_shard_shape():
    """One GPU's N-shard of the 4096 x 7168 x 16384 product, 4096 x 896 x
    16384 (64 tiles): split 4 ways; sampled rows within the bound, integer
    inputs bit-exact, two runs (and a second stream) bit-identical."""
    M, N, K = 4096, 896, 16384
    w = configs.Workload("shard", "bf16", M, N, K, "nk", "normal_sqrtk", 3, 256)
    rows = gen.sample_rows(M, 256, 3)
    d = configs.make_inputs(w)
    A, B = H.dev(d["A"]), H.dev(d["B"])
    H.log("split-K shard 4096x896x16384")
    c1, plan = H.run16("bf16", M, N, K, A, K, 1, B, 1, K, ws=True)
    assert plan == "tile_nt_256x224_splitk4", plan
    C_ref, S = oracle.gemm("bf16", M, N, K, d["A"], K, 1, d["B"], 1, K, rows=rows)
    H.assert_within_bound("bf16", c1[rows], C_ref, S, f"shard [{plan}]")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c2, _ = H.run16("bf16", M, N, K, A, K, 1, B, 1, K, stream=s.cuda_stream, ws=True)
    torch.cuda.synchronize()
    assert np.array_equal(c1, c2)
    c3, plan3 = H.run16("bf16", M, N, K, A, K, 1, B, 1, K)
    assert plan3 == "tile_nt_128x128", plan3
    H.assert_within_bound("bf16", c3[rows], C_ref, S, f"shard [{plan3}]")
    d = configs.make_inputs(w, int_r=32)
    Ai, Bi = H.dev(d["A"]), H.dev(d["B"])
    c, _ = H.run16("bf16", M, N, K, Ai, K, 1, Bi, 1, K, ws=True)
    C_ref, _ = oracle.gemm("bf16", M, N, K, d["A"], K, 1, d["B"], 1, K, rows=rows)
    H.assert_bit_exact("bf16", c[rows], C_ref, "shard int")
    c4, _ = H.run16("bf16", M, N, K, Ai, K, 1, Bi, 1, K)
    assert np.array_equal(c, c4), "split and unsplit plans differ on integer inputs"



def test_tail_after_split_k_and_repeatable():
    """The partial-wave split shares the stream's scratch with split K: the
    4096 x 896 x 16384 shard (64 tiles split 4 ways) and then 4352 x 4096 x
    4096 (67 tiles past the first wave split 3 ways) on one stream, integer
    inputs bit-exact on sampled rows and rows of the split tiles; normal
    inputs bit-identical over two runs on two streams."""
    M, N, K = 4352, 4096, 4096
    rows = np.union1d(gen.sample_rows(M, 64, 7), np.arange(3072, M, 53))
    ws = configs.Workload("shard", "bf16", 4096, 896, 16384, "nk", "integers", 3, 0)
    wt = configs.Workload("tail", "bf16", M, N, K, "nk", "normal_sqrtk", 8, 0)
    ds = configs.make_inputs(ws, int_r=16)
    dt = configs.make_inputs(wt, int_r=32)
    H.log("split-K shard then partial-wave split, one stream, one workspace")
    shared = H.Workspace(16384 + 64 * 4 * 256 * 224 * 4)
    _, plan = H.run16("bf16", 4096, 896, 16384, H.dev(ds["A"]), 16384, 1, H.dev(ds["B"]), 1,
                      16384, ws=shared)
    assert plan == "tile_nt_256x224_splitk4", plan
    c, plan = H.run16("bf16", M, N, K, H.dev(dt["A"]), K, 1, H.dev(dt["B"]), 1, K, ws=shared)
    assert plan == "tile_nt_256x224_tail3", plan
    C_ref, _ = oracle.gemm("bf16", M, N, K, dt["A"], K, 1, dt["B"], 1, K, rows=rows)
    H.assert_bit_exact("bf16", c[rows], C_ref, f"tail after split K [{plan}]")
    dn = configs.make_inputs(wt)
    A, B = H.dev(dn["A"]), H.dev(dn["B"])
    c1, _ = H.run16("bf16", M, N, K, A, K, 1, B, 1, K, ws=shared)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c2, _ = H.run16("bf16", M, N, K, A, K, 1, B, 1, K, stream=s.cuda_stream, ws=True)
    torch.cuda.synchronize()
    assert np.array_equal(c1, c2)


def test_split_k_scratch_reused_by_more_tiles():
    """Two split-K products in a row on one stream and one workspace: 64
    tiles of 256 x 224 split 4 ways (large partials, few counters), then 80
    tiles split 3 ways, which fits the same workspace.  The second call's counters for tiles 64..79 must not
    start from the first call's partial data: bit-exact on integer inputs."""
    K = 8256
    s = torch.cuda.Stream()
    shared = H.Workspace(16384 + 64 * 4 * 256 * 224 * 4)
    with torch.cuda.stream(s):
        M, N = 2048, 1792
        a, b = gen.normal((M, K), 71, 0, "bf16"), gen.normal((N, K), 71, 1, "bf16")
        H.log(f"split-K scratch reuse, first call {M}x{N}x{K}")
        c, plan = H.run16("bf16", M, N, K, H.dev(a), K, 1, H.dev(b), 1, K, stream=s.cuda_stream,
                          ws=shared)
        assert plan == "tile_nt_256x224_splitk4", plan
        rows = gen.sample_rows(M, 128, 71)
        C_ref, S = oracle.gemm("bf16", M, N, K, a, K, 1, b, 1, K, rows=rows)
        H.assert_within_bound("bf16", c[rows], C_ref, S, f"first call [{plan}]")
        N = 2240
        a, b = gen.integers((M, K), 72, 0, 64, "bf16"), gen.integers((N, K), 72, 1, 64, "bf16")
        H.log(f"split-K scratch reuse, second call {M}x{N}x{K}")
        c, plan = H.run16("bf16", M, N, K, H.dev(a), K, 1, H.dev(b), 1, K, stream=s.cuda_stream,
                          ws=shared)
        assert plan == "tile_nt_256x224_splitk3", plan
        rows = np.union1d(gen.sample_rows(M, 128, 72), np.arange(1024, 2048, 61))
        C_ref, _ = oracle.gemm("bf16", M, N, K, a, K, 1, b, 1, K, rows=rows)
        H.assert_bit_exact("bf16", c[rows], C_ref, f"second call [{plan}]")
    torch.cuda.synchronize()

# ------------------------------------------------------------ skinny kernel

# (M, N, K): no split wanted (short K), and K split across workgroups with a
# workspace / across the waves of 32-column strips without one (K of 16 or
# more 64-wide slices), ragged N strips, K not a multiple of the slice.  The
# 32-column strips take their slices four to a barrier: 16, 18, 19, 33, 65
# and 112 slices leave 0, 2, 3, 1, 1 and 0 over.
SKINNY_CASES = [(1, 100, 64), (17, 300, 200), (64, 64, 8), (64, 33, 1000), (40, 7168, 1024),
                (63, 95, 4104), (64, 1000, 2056), (64, 7168, 520), (64, 7168, 7168),
                (64, 512, 1152), (48, 600, 1192),
                # M <= 32 (the allocation-free plan's 32-row form, 28 B stages):
                # more slices than the deeper ring holds, a ragged last group
                (32, 7168, 7168), (1, 300, 7176), (9, 130, 1800)]
# a full grid of 32-column strips with 16 K slices: the split does not pay,
# so the workspace call runs the strips too
SKINNY_WS_STRIPS = {(40, 7168, 1024)}


@pytest.mark.parametrize("case", SKINNY_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in SKINNY_CASES])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_skinny(fmt, case):
    M, N, K = case
    r = max(1, min(64 if fmt == "bf16" else 16, int(math.sqrt(2 ** 24 / K))))
    c_int = {}
    for ws in (False, True):
        plan = _check16(fmt, M, N, K, "nk", seed=800 + M + N + K, ws=ws)
        assert plan.startswith("skinny_64x"), plan
        if ws:
            want = "skinny_64x32" if (M, N, K) in SKINNY_WS_STRIPS else "skinny_64x128"
            assert plan.startswith(want), plan
        plan = _check16(fmt, M, N, K, "nk", seed=900 + M + N + K, int_r=r, ws=ws)
        assert plan.startswith("skinny_64x"), plan
        A, sam, sak, B, sbk, sbn = _layout_args(fmt, M, N, K, "nk", 900 + M + N + K, r)
        c_int[ws], _ = H.run16(fmt, M, N, K, H.dev(A), sam, sak, H.dev(B), sbk, sbn, ws=ws)
    assert np.array_equal(c_int[False], c_int[True]), "skinny plans differ on integer inputs"


def test_skinny_padded():
    for ws in (False, True):
        plan = _check16("bf16", 50, 70, 136, "padded", seed=41, ws=ws)
        assert plan.startswith("skinny_64x"), plan
        plan = _check16("bf16", 64, 300, 3000, "padded", seed=42, ws=ws)
        assert plan.startswith("skinny_64x"), plan


def test_skinny_split_k_deterministic_and_per_stream():
    """The split-K combination adds the partial tiles in a fixed order: two
    runs agree bit for bit, on the default stream and on a second stream
    (with a workspace of its own), with calls of other shapes in between;
    the allocation-free plan is repeatable too."""
    w = configs.WORKLOADS["bf16_skinny_64x7168x7168"]
    d = configs.make_inputs(w)
    A, B = H.dev(d["A"]), H.dev(d["B"])
    H.log("skinny determinism / second stream")
    ws1 = H.Workspace(16384 + 56 * 4 * 64 * 128 * 4)
    c1, plan = H.run16("bf16", w.M, w.N, w.K, A, w.K, 1, B, d["sbk"], d["sbn"], ws=ws1)
    assert plan == "skinny_64x128_splitk4", plan
    _check16("bf16", 64, 1000, 2056, "nk", seed=61, ws=ws1)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c2, _ = H.run16("bf16", w.M, w.N, w.K, A, w.K, 1, B, d["sbk"], d["sbn"],
                        stream=s.cuda_stream, ws=True)
    torch.cuda.synchronize()
    c3, _ = H.run16("bf16", w.M, w.N, w.K, A, w.K, 1, B, d["sbk"], d["sbn"], ws=ws1)
    assert np.array_equal(c1, c2) and np.array_equal(c1, c3)
    c4, plan4 = H.run16("bf16", w.M, w.N, w.K, A, w.K, 1, B, d["sbk"], d["sbn"])
    c5, _ = H.run16("bf16", w.M, w.N, w.K, A, w.K, 1, B, d["sbk"], d["sbn"])
    assert plan4 == "skinny_64x32", plan4
    assert np.array_equal(c4, c5)


def _capture(stream, M, N, K, A, B, C, ws=None):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        if ws is None:
            H.tg.tg_gemm_bf16(M, N, K, A.data_ptr(), K, 1, B.data_ptr(), 1, K, C.data_ptr(), N, 1,
                              stream.cuda_stream)
        else:
            H.tg.tg_gemm_bf16_ws(M, N, K, A.data_ptr(), K, 1, B.data_ptr(), 1, K, C.data_ptr(), N,
                                 1, ws.ptr, ws.nbytes, stream.cuda_stream)
    return g


def _graph_case(M, N, K, seed, want_ws, want_free):
    """Graphs captured from the allocation-free entry point and from the
    workspace one (its own workspace), replayed several times with eager
    split-K work on another workspace in between, each replay checked
    against the eager result bit for bit (integer inputs: every split order
    sums exactly)."""
    w = configs.Workload("t", "bf16", M, N, K, "nk", "normal", seed, 0)
    d = configs.make_inputs(w, int_r=32)
    A, B = H.dev(d["A"]), H.dev(d["B"])
    c_eager, plan = H.run16("bf16", M, N, K, A, K, 1, B, 1, K, ws=True)
    assert plan == want_ws, plan
    C_ref, _ = oracle.gemm("bf16", M, N, K, d["A"], K, 1, d["B"], 1, K)
    H.assert_bit_exact("bf16", c_eager, C_ref, f"eager [{plan}]")
    c_free, plan = H.run16("bf16", M, N, K, A, K, 1, B, 1, K)
    assert plan == want_free, plan
    assert np.array_equal(c_free, c_eager)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    C1 = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    C2 = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    gws = H.Workspace(H.tg.tg_gemm_workspace_size(H.tg.OP_BF16, M, N, K, A.data_ptr(), K, 1,
                                                  B.data_ptr(), 1, K, C2.data_ptr(), N, 1))
    torch.cuda.synchronize()
    g1 = _capture(s1, M, N, K, A, B, C1)
    g2 = _capture(s2, M, N, K, A, B, C2, gws)
    torch.cuda.synchronize()
    other = H.Workspace(gws.nbytes)
    for _ in range(3):
        C1.zero_()
        C2.zero_()
        H.run16("bf16", M, N, K, A, K, 1, B, 1, K, ws=other)   # eager split-K work in between
        torch.cuda.synchronize()
        g1.replay()
        g2.replay()
        torch.cuda.synchronize()
        assert np.array_equal(C1.cpu().numpy().view(np.uint16), c_eager)
        assert np.array_equal(C2.cpu().numpy().view(np.uint16), c_eager)
        assert gws.counters_zero()


def test_skinny_graph_capture():
    H.log("skinny graph capture")
    _graph_case(64, 2048, 4096, 77, "skinny_64x128_splitk8", "skinny_64x32")


def test_split_k_graph_capture():
    H.log("split-K graph capture")
    _graph_case(1024, 1024, 4096, 78, "tile_nt_128x128_splitk4", "tile_nt_128x128")


def test_pp_split_k_graph_capture():
    H.log("eight-wave split-K graph capture")
    _graph_case(1000, 2600, 8200, 80, "tile_nt_256x224_splitk5", "tile_nt_128x128")


def test_pp_tail_graph_capture():
    H.log("eight-wave partial-wave graph capture")
    _graph_case(4352, 4096, 1024, 81, "tile_nt_256x224_tail2", "tile_nt_256x224")


def test_workspace_short_runs_allocation_free_plan():
    """A workspace one byte short of the split plan's need: the call runs the
    allocation-free plan and leaves the workspace untouched."""
    M, N, K = 64, 2048, 4096
    w = configs.Workload("t", "bf16", M, N, K, "nk", "normal", 79, 0)
    d = configs.make_inputs(w, int_r=32)
    A, B = H.dev(d["A"]), H.dev(d["B"])
    need = H.tg.tg_gemm_workspace_size(H.tg.OP_BF16, M, N, K, A.data_ptr(), K, 1, B.data_ptr(),
                                       1, K, A.data_ptr(), N, 1)
    short = H.Workspace(need - 1)
    short.buf.fill_(0)
    H.log("workspace one byte short")
    c, plan = H.run16("bf16", M, N, K, A, K, 1, B, 1, K, ws=short)
    assert plan == "skinny_64x32", plan
    assert int(short.buf.count_nonzero().item()) == 0
    C_ref, _ = oracle.gemm("bf16", M, N, K, d["A"], K, 1, d["B"], 1, K)
    H.assert_bit_exact("bf16", c, C_ref, "short workspace")

# ------------------------------------------------------ K x N tile kernel

NN_CASES = [(300, 512, 136), (513, 264, 72), (4000, 4000, 136), (256, 256, 64), (65, 8, 8),
            (257, 1032, 1000)]


@pytest.mark.parametrize("case", NN_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in NN_CASES])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_tile_nn(fmt, case):
    M, N, K = case
    plan = _check16(fmt, M, N, K, "kn", seed=1000 + M + N + K)
    assert plan == "tile_nn_256x256", plan
    r = max(1, min(64 if fmt == "bf16" else 16, int(math.sqrt(2 ** 24 / K))))
    plan = _check16(fmt, M, N, K, "kn", seed=1100 + M + N + K, int_r=r)
    assert plan == "tile_nn_256x256", plan


def test_tile_nn_padded():
    plan = _check16("bf16", 300, 264, 200, "kn_padded", seed=51)
    assert plan == "tile_nn_256x256", plan
    plan = _check16("f16", 70, 96, 64, "kn_padded", seed=52)
    assert plan == "tile_nn_256x256", plan


# ------------------------------------------------------- fp8 tile kernel

FP8_TILE_CASES = [(256, 128, 128), (384, 256, 208), (300, 200, 400), (513, 384, 1040),
                  (65, 1000, 2048), (1000, 136, 16), (257, 129, 3072)]


@pytest.mark.parametrize("case", FP8_TILE_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in FP8_TILE_CASES])
def test_fp8_tile(case):
    M, N, K = case
    plan = _check_fp8(M, N, K, _fp8_inputs(M, N, K, 1200 + M + K), what="tile bound")
    assert plan == "tile_fp8_256x128", plan
    plan = _check_fp8(M, N, K, _fp8_inputs(M, N, K, 1300 + M + K, int_r=16), exact=True,
                      what="tile int unit scales")
    assert plan == "tile_fp8_256x128", plan
    plan = _check_fp8(M, N, K, _fp8_inputs(M, N, K, 1400 + M + K, int_r=4, pow2_scales=True),
                      exact=True, what="tile int pow2 scales")
    assert plan == "tile_fp8_256x128", plan


# ------------------------------------------------------- fp8 skinny kernel

# M <= 64: 32-column strips over the whole of K, each wave one 128-wide block
# of every four.  Fewer blocks than waves (K = 256), a partial last block
# (K = 1936, 400), strips past N (N = 300, 130: the last strip partly empty,
# and strips in the second 128-column B scale block), one row, and the
# 64 x 7168 x 7168 decode shape in full.
FP8_SKINNY_CASES = [(1, 1000, 2048), (20, 200, 256), (17, 300, 400), (64, 96, 128),
                    (33, 40, 1936), (8, 130, 256), (5, 16, 256), (64, 7168, 7168)]


@pytest.mark.parametrize("case", FP8_SKINNY_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in FP8_SKINNY_CASES])
def test_fp8_skinny(case):
    M, N, K = case
    plan = _check_fp8(M, N, K, _fp8_inputs(M, N, K, 1800 + M + K), what="skinny bound")
    assert plan == "skinny_fp8_64x32", plan
    plan = _check_fp8(M, N, K, _fp8_inputs(M, N, K, 1900 + M + K, int_r=16), exact=True,
                      what="skinny int unit scales")
    assert plan == "skinny_fp8_64x32", plan
    plan = _check_fp8(M, N, K, _fp8_inputs(M, N, K, 2000 + M + K, int_r=4, pow2_scales=True),
                      exact=True, what="skinny int pow2 scales")
    assert plan == "skinny_fp8_64x32", plan


# The split plan of the fp8 decode product (a caller's workspace): 64 x 128
# strips over ranges of the K blocks, partial tiles added in split order; it
# runs for 33 .. 64 rows with long strips or half-empty strip grids.  Cases:
# a 64 x 7168 x 16384 down projection (4 splits); 64 x 16384 x 7168 (2
# splits); 8 splits (40 x 4096 x 7168); a ragged last strip and a ragged
# last K block in the last of 14 splits (33 x 300 x 7184: 57 blocks); one
# partial strip with 14 splits; 16 splits, summed four at a time (48 x 100 x
# 8192); 14 splits over 16 strips (64 x 2048 x 7168); a 2-column strip in
# the second B scale block; 63 rows of a 16-column strip.
FP8_SPLIT_CASES = [(64, 7168, 16384), (64, 16384, 7168), (40, 4096, 7168), (33, 300, 7184),
                   (40, 40, 7184), (48, 100, 8192), (64, 2048, 7168), (64, 130, 7168),
                   (63, 16, 7168)]


@pytest.mark.parametrize("case", FP8_SPLIT_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in FP8_SPLIT_CASES])
def test_fp8_skinny_split(case):
    M, N, K = case
    for d, exact, what in (
            (_fp8_inputs(M, N, K, 2200 + M + K), False, "split bound"),
            (_fp8_inputs(M, N, K, 2300 + M + K, int_r=16), True, "split int unit scales"),
            (_fp8_inputs(M, N, K, 2400 + M + K, int_r=4, pow2_scales=True), True,
             "split int pow2 scales")):
        plan = _check_fp8(M, N, K, d, exact=exact, what=what, ws=True)
        assert plan.startswith("skinny_fp8_64x128_splitk"), plan


def test_fp8_split_workspace_reuse():
    """One workspace through three calls in a row -- a 64 x 7168 x 16384 down
    projection, a smaller call (fewer strips and splits), the first again: each
    leaves the counters zero and is bit-exact on integer inputs."""
    M0, N0, K0 = big = (64, 7168, 16384)
    ws = H.Workspace(H.tg.tg_gemm_workspace_size(H.tg.OP_FP8, M0, N0, K0, 0x100, K0, 1, 0x200, 1,
                                                 K0, 0x300, N0, 1))
    assert ws.nbytes == 16384 + 56 * 4 * 64 * 128 * 4
    for i, (M, N, K) in enumerate((big, (33, 300, 7184), big)):
        plan = _check_fp8(M, N, K, _fp8_inputs(M, N, K, 2500 + i, int_r=16), exact=True,
                          what=f"split reuse {i}", ws=ws)
        assert plan.startswith("skinny_fp8_64x128_splitk"), plan


def test_fp8_split_padded_c():
    """The split plan storing into C rows padded by 40 elements, behind guard
    bands, with B stored K x N-contiguous rows padded (sbn = K + 32)."""
    M, N, K = 40, 300, 7168
    d = _fp8_inputs(M, N, K, 2600, int_r=16)
    assert (d["sbk"], d["sbn"]) == (1, K)
    Bp = np.zeros((N, K + 32), np.uint8)
    Bp[:, :K] = np.asarray(d["B"]).view(np.uint8).reshape(N, K)
    nkb = d["SA"].shape[1]
    c, plan = H.run_fp8(M, N, K, H.dev(d["A"]), K, 1, H.dev(d["SA"]), nkb, 1, H.dev(Bp),
                        1, K + 32, H.dev(d["SB"]), nkb, 1, scm=N + 40, ws=True)
    assert plan == "skinny_fp8_64x128_splitk", plan     # 14 splits
    C_ref, _ = oracle.gemm_fp8_blockscaled(M, N, K, d["A"], K, 1, d["SA"], nkb, 1, Bp, 1, K + 32,
                                           d["SB"], nkb, 1)
    H.assert_bit_exact("bf16", c, C_ref, f"fp8 split, padded C [{plan}]")


def test_fp8_skinny_padded_c():
    """The skinny fp8 product storing into C rows padded by 40 elements, behind
    guard bands (nothing outside the M x N block is written)."""
    M, N, K = 20, 100, 512
    d = _fp8_inputs(M, N, K, 2100, int_r=16)
    nkb = d["SA"].shape[1]
    c, plan = H.run_fp8(M, N, K, H.dev(d["A"]), K, 1, H.dev(d["SA"]), nkb, 1, H.dev(d["B"]),
                        d["sbk"], d["sbn"], H.dev(d["SB"]), nkb, 1, scm=N + 40)
    assert plan == "skinny_fp8_64x32", plan
    C_ref, _ = oracle.gemm_fp8_blockscaled(M, N, K, d["A"], K, 1, d["SA"], nkb, 1, d["B"],
                                           d["sbk"], d["sbn"], d["SB"], nkb, 1)
    H.assert_bit_exact("bf16", c, C_ref, f"fp8 skinny, padded C [{plan}]")
