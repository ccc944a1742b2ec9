"""The GEMM workloads and their seeded input recipes.

Shapes follow the pages' workloads: the 4096 x 7168 x 16384 bf16 product of
the Ascend "six-piece" release ("Getting to know TileLang"), the 7168 hidden
size of "TileKernels deep dive" (sections 5.1 and 8.1), and the fp16 first-GEMM
listing of "Getting to know TileLang".  Inputs are synthetic and seeded:
workload n draws with seed n, stream 0 for A, stream 1 for B, stream 2 for
the sampled check rows.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import DIST_INT, DIST_NORMAL, DIST_UNIFORM, fill, quant_e4m3fn


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str           # "f16", "bf16" (inputs and output) or "fp8" (e4m3fn in, bf16 out)
    M: int
    N: int
    K: int
    b_layout: str        # "kn": B stored K x N row-major; "nk": B stored N x K row-major
    dist: str            # "uniform", "normal", "normal_sqrtk"
    seed: int
    check_rows: int      # 0: check every row; else this many sampled rows

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    @property
    def elem_bytes(self) -> int:
        return 1 if self.dtype == "fp8" else 2

    @property
    def compulsory_bytes(self) -> int:
        """A + B read once, C written once (+ fp32 scales for fp8)."""
        e = self.elem_bytes
        b = (self.M * self.K + self.N * self.K) * e + self.M * self.N * 2
        if self.dtype == "fp8":
            kb = -(-self.K // 128)
            b += 4 * (self.M * kb + (-(-self.N // 128)) * kb)
        return b


WORKLOADS = {
    "fp16_256": Workload("fp16_256", "f16", 256, 256, 256, "kn", "uniform", 1, 0),
    "bf16_4096": Workload("bf16_4096", "bf16", 4096, 4096, 4096, "kn", "normal", 2, 0),
    "bf16_4096x7168x16384": Workload("bf16_4096x7168x16384", "bf16", 4096, 7168, 16384, "nk",
                                     "normal_sqrtk", 3, 256),
    "bf16_skinny_64x7168x7168": Workload("bf16_skinny_64x7168x7168", "bf16", 64, 7168, 7168, "nk",
                                         "normal_sqrtk", 4, 0),
    "fp8_4096x7168x16384": Workload("fp8_4096x7168x16384", "fp8", 4096, 7168, 16384, "nk",
                                    "normal", 5, 256),
}
ORDER = list(WORKLOADS)


def b_strides(layout: str, N: int, K: int):
    """(sbk, sbn) element strides of B[k, j] for the storage layout."""
    return (N, 1) if layout == "kn" else (1, K)


def _draw(shape, dist, seed, stream, fmt, K, int_r):
    if int_r is not None:
        return fill(shape, DIST_INT, seed, stream, fmt, param=int_r)
    if dist == "uniform":
        return fill(shape, DIST_UNIFORM, seed, stream, fmt)
    div = math.sqrt(K) if dist == "normal_sqrtk" else 1.0
    return fill(shape, DIST_NORMAL, seed, stream, fmt, divisor=div)


def make_inputs(w: Workload, int_r: int | None = None, M: int | None = None,
                N: int | None = None, K: int | None = None, b_layout: str | None = None):
    """Storage-format inputs for workload `w` (shape overrides allowed).

    int_r: draw integers uniform on [-int_r, int_r] instead of the workload's
    distribution (for bit-exact checks; for fp8 the scales are then 1.0).
    Returns a dict: A (M x K codes), B (K x N or N x K codes), sbk, sbn and,
    for fp8, SA (M x ceil(K/128)) and SB (ceil(N/128) x ceil(K/128)).
    """
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    layout = w.b_layout if b_layout is None else b_layout
    bshape = (K, N) if layout == "kn" else (N, K)
    out = {"M": M, "N": N, "K": K, "layout": layout}
    if w.dtype == "fp8":
        if int_r is not None:
            A = fill((M, K), DIST_INT, w.seed, 0, "f32", param=int_r)
            Bnk = fill((N, K), DIST_INT, w.seed, 1, "f32", param=int_r)
            qa = _f32_ints_to_e4m3(A)
            qb = _f32_ints_to_e4m3(Bnk)
            sa = np.ones((M, -(-K // 128)), np.float32)
            sb = np.ones((-(-N // 128), -(-K // 128)), np.float32)
        else:
            A = _draw((M, K), w.dist, w.seed, 0, "f32", K, None)
            Bnk = _draw((N, K), w.dist, w.seed, 1, "f32", K, None)
            qa, sa = quant_e4m3fn(A, 1, 128)
            qb, sb = quant_e4m3fn(Bnk, 128, 128)
        if layout == "kn":
            qb = np.ascontiguousarray(qb.T)
        out.update(A=qa, B=qb, SA=sa, SB=sb)
    else:
        out["A"] = _draw((M, K), w.dist, w.seed, 0, w.dtype, K, int_r)
        out["B"] = _draw(bshape, w.dist, w.seed, 1, w.dtype, K, int_r)
    out["sbk"], out["sbn"] = b_strides(layout, N, K)
    return out


def _f32_ints_to_e4m3(x: np.ndarray) -> np.ndarray:
    from . import round_e4m3fn
    return round_e4m3fn(x)


def group_sizes(total: int, G: int, seed: int) -> np.ndarray:
    """Row counts of G groups summing to `total`: a seeded uneven split (the
    token counts of G experts).  Weights are 0.25 + u with u uniform from
    (seed, stream 3); counts are floor(total * w / sum w) with the remainder
    spread over the first groups."""
    from . import draws
    u = draws(seed, 3, G).astype(np.float64) / 2.0 ** 64
    w = 0.25 + u
    n = np.floor(total * w / w.sum()).astype(np.int64)
    n[: total - int(n.sum())] += 1
    return n


# The grouped product measured by the benchmark: 8 experts over 8192 tokens,
# N = 4096, K = 7168 (the 7168 hidden size), bf16, B_g stored N x K.
GROUPED = {"name": "grouped_bf16_8x8192x4096x7168", "G": 8, "rows": 8192, "N": 4096, "K": 7168,
           "seed": 6}


# The fused SwiGLU measured by the benchmark: the gate and up projections
# whose h feeds the 4096 x 7168 x 16384 down projection above -- 4096 rows,
# hidden size K = 7168, intermediate size N = 16384 per projection, bf16,
# both weights stored N x K.
SWIGLU = {"name": "swiglu_bf16_4096x16384x7168", "M": 4096, "N": 16384, "K": 7168, "seed": 7}


def swiglu_inputs(M: int, N: int, K: int, seed: int, fmt: str = "bf16"):
    """Input x (M x K, N(0, 1)) and the gate and up weights (each N x K,
    N(0, 1) / sqrt(K), so each product element is about N(0, 1)), drawn from
    streams 0, 1 and 4 of `seed`."""
    div = math.sqrt(max(K, 1))
    return {"A": fill((M, K), DIST_NORMAL, seed, 0, fmt),
            "Bg": fill((N, K), DIST_NORMAL, seed, 1, fmt, divisor=div),
            "Bu": fill((N, K), DIST_NORMAL, seed, 4, fmt, divisor=div)}
