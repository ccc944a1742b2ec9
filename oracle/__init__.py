"""CPU oracle for the tiled dense GEMM -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package; the library path never imports it.  It shares no code with the
GPU path.  The arithmetic lives in oracle.c (plain fp64 loops, own decoders);
this module only marshals numpy arrays through ctypes.

Every function is pinned by tests/test_oracle.py against identities,
permutations, rank-1 closed forms, exact-integer brute force and NumPy's fp64
matmul; the decoders and the rounding are pinned exhaustively against
torch / numpy dtype conversions (tests/test_codecs.py); the fp8 block
quantiser against torch's e4m3fn cast, numpy's fp32 division, the block
invariants of its definition and the input generator's own quantiser; the
product with fp8 output against an identity product and numpy's integer
matmul; the SwiGLU combination against closed forms of silu, a selection
product and exact integer products; the acceptance bound against its stated constants, the unit
roundoffs of torch's format descriptions and an fp32-accumulating model of
the GPU arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "libtg_oracle.so")

FMT = {"f16": 1, "bf16": 2, "e4m3fn": 3}


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile oracle.c (gcc -O2, OpenMP, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class Oracle:
    """ctypes view of one build of oracle.c (the default build, or a test build)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, vp, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.tg_oracle_gemm.argtypes = [c_int, i64, i64, i64, vp, i64, i64, vp, i64, i64,
                                       vp, i64, vp, vp]
        lib.tg_oracle_gemm.restype = c_int
        lib.tg_oracle_gemm_fp8_blockscaled.argtypes = [i64, i64, i64, vp, i64, i64, vp, i64, i64,
                                                       vp, i64, i64, vp, i64, i64, vp, i64, vp, vp]
        lib.tg_oracle_gemm_fp8_blockscaled.restype = c_int
        lib.tg_oracle_round.argtypes = [c_int, vp, i64, vp]
        lib.tg_oracle_round.restype = None
        lib.tg_oracle_decode.argtypes = [c_int, vp, i64, vp]
        lib.tg_oracle_decode.restype = None
        lib.tg_oracle_quant_fp8.argtypes = [i64, i64, vp, i64, i64, vp, i64, vp, i64, i64]
        lib.tg_oracle_quant_fp8.restype = c_int
        lib.tg_oracle_swiglu.argtypes = [i64, vp, vp, vp]
        lib.tg_oracle_swiglu.restype = c_int
        lib.tg_oracle_bound.argtypes = [c_int, vp, i64, vp]
        lib.tg_oracle_bound.restype = None
        lib.tg_oracle_threads.argtypes = [c_int]
        lib.tg_oracle_threads.restype = None
        lib.tg_oracle_init()
        self.lib = lib

    def gemm(self, fmt: str, M: int, N: int, K: int, A: np.ndarray, sam: int, sak: int,
             B: np.ndarray, sbk: int, sbn: int, rows=None):
        """fp64 C and S = sum |a||b| for the requested rows of C (all if None).

        A and B are uint16 code buffers (fp16 or bf16) addressed with element
        strides: A[i,k] = A.flat[i*sam + k*sak], B[k,j] = B.flat[k*sbk + j*sbn].
        """
        A = np.ascontiguousarray(A).view(np.uint16)
        B = np.ascontiguousarray(B).view(np.uint16)
        rows, nrows = _rows_arg(rows, M)
        C = np.empty((nrows, N), np.float64)
        S = np.empty((nrows, N), np.float64)
        rc = self.lib.tg_oracle_gemm(FMT[fmt], M, N, K, _p(A), sam, sak, _p(B), sbk, sbn,
                                     _p(rows), nrows, _p(C), _p(S))
        if rc != 0:
            raise ValueError("oracle: bad arguments")
        return C, S

    def gemm_fp8_blockscaled(self, M, N, K, QA, sam, sak, SA, ssam, ssak, QB, sbk, sbn, SB,
                             ssbn, ssbk, rows=None):
        """fp64 C and S for the e4m3fn block-scaled product (see oracle.c)."""
        QA = np.ascontiguousarray(QA).view(np.uint8)
        QB = np.ascontiguousarray(QB).view(np.uint8)
        SA = np.ascontiguousarray(SA, dtype=np.float32)
        SB = np.ascontiguousarray(SB, dtype=np.float32)
        rows, nrows = _rows_arg(rows, M)
        C = np.empty((nrows, N), np.float64)
        S = np.empty((nrows, N), np.float64)
        rc = self.lib.tg_oracle_gemm_fp8_blockscaled(M, N, K, _p(QA), sam, sak, _p(SA), ssam,
                                                     ssak, _p(QB), sbk, sbn, _p(SB), ssbn, ssbk,
                                                     _p(rows), nrows, _p(C), _p(S))
        if rc != 0:
            raise ValueError("oracle: bad arguments")
        return C, S

    def quant_fp8(self, X: np.ndarray, br: int):
        """Block quantisation of an R x K fp32 matrix to e4m3fn codes with one
        fp32 scale per br x 128 block, br = 1 or 128 (see oracle.c): returns
        (codes R x K uint8, scales ceil(R / br) x ceil(K / 128) fp32)."""
        X = np.ascontiguousarray(X, dtype=np.float32)
        R, K = X.shape
        Q = np.empty((R, K), np.uint8)
        S = np.empty(((R + br - 1) // br, (K + 127) // 128), np.float32)
        rc = self.lib.tg_oracle_quant_fp8(R, K, _p(X), K, br, _p(Q), K, _p(S), S.shape[1], 1)
        if rc != 0:
            raise ValueError("oracle: bad arguments")
        return Q, S

    def gemm_quant_fp8(self, fmt: str, M: int, N: int, K: int, A: np.ndarray, sam: int,
                       sak: int, B: np.ndarray, sbk: int, sbn: int, rows=None):
        """The product with an fp8 output ("TileKernels deep dive" section 7.2:
        the result quantised to FP8 where it is computed, per row slice of 128,
        scale = slice maximum over 448): the fp64 product, rounded once to fp32
        (the accumulator type, with no rounding to 16 bits in between), then
        quantised with one scale per 1 x 128 row slice.  Returns (codes
        nrows x N, scales nrows x ceil(N / 128), fp64 C, S = sum |a||b|) for
        the requested rows (all if None)."""
        C, S = self.gemm(fmt, M, N, K, A, sam, sak, B, sbk, sbn, rows=rows)
        Q, SC = self.quant_fp8(C.astype(np.float32), 1)
        return Q, SC, C, S

    def swiglu(self, G: np.ndarray, U: np.ndarray) -> np.ndarray:
        """h = silu(g) * u element by element, silu(g) = g / (1 + e^-g), in
        fp64 (see oracle.c)."""
        G = np.ascontiguousarray(G, dtype=np.float64)
        U = np.ascontiguousarray(U, dtype=np.float64)
        if G.shape != U.shape:
            raise ValueError("oracle: gate and up shapes differ")
        H = np.empty(G.shape, np.float64)
        if self.lib.tg_oracle_swiglu(G.size, _p(G), _p(U), _p(H)) != 0:
            raise ValueError("oracle: bad arguments")
        return H

    def swiglu_quant_fp8(self, fmt: str, M: int, N: int, K: int, A: np.ndarray, sam: int,
                         sak: int, Bg: np.ndarray, Bu: np.ndarray, sbk: int, sbn: int, rows=None):
        """The fused SwiGLU with an fp8 output ("TileKernels deep dive" section
        4.3): the gate product G = A Bg and the up product U = A Bu in fp64,
        h = silu(g) * u in fp64, rounded once to fp32, then quantised with one
        scale per 1 x 128 row slice as in gemm_quant_fp8.  Bg and Bu share the
        strides (B[k,j] at k*sbk + j*sbn).  Returns (codes nrows x N, scales
        nrows x ceil(N / 128), fp64 H, fp64 G, fp64 U, S_g, S_u) for the
        requested rows (all if None); S = sum |a||b| of each product."""
        G, Sg = self.gemm(fmt, M, N, K, A, sam, sak, Bg, sbk, sbn, rows=rows)
        U, Su = self.gemm(fmt, M, N, K, A, sam, sak, Bu, sbk, sbn, rows=rows)
        H = self.swiglu(G, U)
        Q, SC = self.quant_fp8(H.astype(np.float32), 1)
        return Q, SC, H, G, U, Sg, Su

    def round_to(self, fmt: str, x: np.ndarray) -> np.ndarray:
        """Round fp64 values to fp16 / bf16 codes, nearest-even (overflow -> inf)."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, np.uint16)
        self.lib.tg_oracle_round(FMT[fmt], _p(x), x.size, _p(out))
        return out

    def threads(self, n: int) -> None:
        """Threads of the oracle's parallel row loops (0: every core)."""
        self.lib.tg_oracle_threads(int(n))

    def bound(self, fmt_out: str, S: np.ndarray) -> np.ndarray:
        """Per-element acceptance bound on |C_gpu - C_ref| (see oracle.c):
        four unit roundoffs of the output format times S = sum_k |a||b|."""
        S = np.ascontiguousarray(S, dtype=np.float64)
        out = np.empty(S.shape, np.float64)
        self.lib.tg_oracle_bound(FMT[fmt_out], _p(S), S.size, _p(out))
        return out

    def decode(self, fmt: str, codes: np.ndarray) -> np.ndarray:
        """Exact fp64 values of fp16 / bf16 / e4m3fn codes."""
        dt = np.uint8 if fmt == "e4m3fn" else np.uint16
        codes = np.ascontiguousarray(codes).view(dt)
        out = np.empty(codes.shape, np.float64)
        self.lib.tg_oracle_decode(FMT[fmt], _p(codes), codes.size, _p(out))
        return out


def _p(a):
    return None if a is None else a.ctypes.data


def _rows_arg(rows, M):
    if rows is None:
        return None, M
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    return rows, rows.size


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build()
        _default = Oracle(_LIB)
    return _default


def gemm(*args, **kw):
    return default().gemm(*args, **kw)


def gemm_fp8_blockscaled(*args, **kw):
    return default().gemm_fp8_blockscaled(*args, **kw)


def gemm_quant_fp8(*args, **kw):
    return default().gemm_quant_fp8(*args, **kw)


def swiglu(*args, **kw):
    return default().swiglu(*args, **kw)


def swiglu_quant_fp8(*args, **kw):
    return default().swiglu_quant_fp8(*args, **kw)


def threads(n):
    default().threads(n)


def round_to(fmt, x):
    return default().round_to(fmt, x)


def quant_fp8(X, br):
    return default().quant_fp8(X, br)


def decode(fmt, codes):
    return default().decode(fmt, codes)


def bound(fmt_out: str, S: np.ndarray) -> np.ndarray:
    """Per-element tolerance: 4*2^-8*S for bf16 output, 4*2^-11*S for fp16."""
    return default().bound(fmt_out, S)
