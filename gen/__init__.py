"""Seeded synthetic inputs for the tiled GEMM tests and benchmark.

This package holds none of the GEMM's arithmetic: it draws matrices from a
counter-based generator, rounds them once to the storage format (bf16, fp16,
fp32), and block-quantises fp32 matrices to e4m3fn with amax/448 scales (the
per-block convention of the fused RMSNorm + FP8 quantisation listing in
"TileKernels deep dive", section 7.2).  Both the CPU oracle and the GPU path
consume what it produces; it imports neither.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libtg_gen.so")

DIST_UNIFORM, DIST_NORMAL, DIST_INT = 0, 1, 2
OUT_F64, OUT_F32, OUT_BF16, OUT_F16 = 0, 1, 2, 3
_OUT_DTYPE = {OUT_F64: np.float64, OUT_F32: np.float32, OUT_BF16: np.uint16, OUT_F16: np.uint16}
FORMATS = {"f64": OUT_F64, "f32": OUT_F32, "bf16": OUT_BF16, "f16": OUT_F16}


def build() -> str:
    """Compile gen.c into libtg_gen.so next to it (host code, gcc, OpenMP)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, u64, vp, dbl, c_int = (ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p,
                                   ctypes.c_double, ctypes.c_int)
        lib.tg_gen_fill.argtypes = [c_int, u64, u64, i64, i64, dbl, dbl, c_int, vp]
        lib.tg_gen_fill.restype = None
        lib.tg_gen_draws.argtypes = [u64, u64, i64, i64, vp]
        lib.tg_gen_draws.restype = None
        for name in ("tg_gen_round_bf16", "tg_gen_round_f16"):
            getattr(lib, name).argtypes = [vp, i64, vp]
            getattr(lib, name).restype = None
        lib.tg_gen_round_e4m3fn.argtypes = [vp, i64, vp]
        lib.tg_gen_round_e4m3fn.restype = None
        lib.tg_gen_quant_e4m3fn.argtypes = [vp, i64, i64, i64, i64, vp, vp]
        lib.tg_gen_quant_e4m3fn.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def fill(shape, dist: int, seed: int, stream: int, fmt: str, param: float = 0.0,
         divisor: float = 1.0, offset: int = 0) -> np.ndarray:
    """Elements offset.. of (seed, stream), in row-major order of `shape`."""
    out_fmt = FORMATS[fmt]
    out = np.empty(shape, dtype=_OUT_DTYPE[out_fmt])
    _load().tg_gen_fill(dist, seed, stream, offset, out.size, float(param), float(divisor),
                        out_fmt, _ptr(out))
    return out


def uniform_pm1(shape, seed, stream, fmt):
    return fill(shape, DIST_UNIFORM, seed, stream, fmt)


def normal(shape, seed, stream, fmt, divisor=1.0):
    return fill(shape, DIST_NORMAL, seed, stream, fmt, divisor=divisor)


def integers(shape, seed, stream, r, fmt):
    """Integers uniform on [-r, r], stored exactly in `fmt`."""
    return fill(shape, DIST_INT, seed, stream, fmt, param=r)


def draws(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().tg_gen_draws(seed, stream, offset, n, _ptr(out))
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().tg_gen_round_bf16(_ptr(x), x.size, _ptr(out))
    return out


def round_f16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().tg_gen_round_f16(_ptr(x), x.size, _ptr(out))
    return out


def round_e4m3fn(x: np.ndarray) -> np.ndarray:
    """fp32 -> e4m3fn codes, round-to-nearest-even, for |x| <= 448."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().tg_gen_round_e4m3fn(_ptr(x), x.size, _ptr(out))
    return out


def quant_e4m3fn(x: np.ndarray, br: int, bc: int):
    """Block-quantise a rows x cols fp32 matrix: returns (codes, scales) with
    codes rows x cols uint8 and scales ceil(rows/br) x ceil(cols/bc) fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty(((rows + br - 1) // br, (cols + bc - 1) // bc), np.float32)
    _load().tg_gen_quant_e4m3fn(_ptr(x), rows, cols, br, bc, _ptr(q), _ptr(s))
    return q, s


def sample_rows(m: int, count: int, seed: int, stream: int = 2) -> np.ndarray:
    """`count` distinct row indices of 0..m-1 (partial Fisher-Yates shuffle on
    the draws of (seed, stream)), returned sorted."""
    count = min(count, m)
    d = draws(seed, stream, count)
    perm = list(range(m))
    for t in range(count):
        j = t + int(d[t]) % (m - t)
        perm[t], perm[j] = perm[j], perm[t]
    return np.array(sorted(perm[:count]), dtype=np.int64)
