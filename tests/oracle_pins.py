"""Pins of the CPU oracle against facts fixed outside it.

Each pin takes an `oracle.Oracle` (the default build, or a build with a
planted mistake) and raises AssertionError if the oracle disagrees with:
identity and selection matrices, rank-1 closed forms, exact integer / rational
brute force, NumPy's fp64 matmul, layout (stride) invariance, the magnitude-sum
invariants, the fp8 block-scale closed form, and exhaustive decoder tables
from torch / numpy.  Reference values come from Python integers, fractions,
numpy / torch dtype conversions -- never from the oracle itself.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

import gen

ONE = {"bf16": 0x3F80, "f16": 0x3C00}
E4M3_ONE = 0x38


def lib_decode(fmt: str, codes: np.ndarray) -> np.ndarray:
    """Exact fp64 values of codes via torch / numpy dtype conversion."""
    codes = np.ascontiguousarray(codes)
    if fmt == "f16":
        return codes.view(np.float16).astype(np.float64)
    if fmt == "bf16":
        return torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16) \
            .to(torch.float32).double().numpy()
    return torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32) \
        .double().numpy()


def lib_encode(fmt: str, values: np.ndarray) -> np.ndarray:
    """Codes of values exactly representable in fp16 / bf16 (library casts)."""
    values = np.asarray(values, dtype=np.float64)
    if fmt == "f16":
        return values.astype(np.float16).view(np.uint16)
    return torch.from_numpy(values.astype(np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _strides(layout, N, K):
    return (N, 1) if layout == "kn" else (1, K)


def _store_b(bvals_kn: np.ndarray, layout: str) -> np.ndarray:
    return np.ascontiguousarray(bvals_kn if layout == "kn" else bvals_kn.T)


# ---------------------------------------------------------------- 16-bit GEMM

def pin_identity(orc):
    for fmt in ("bf16", "f16"):
        for layout in ("kn", "nk"):
            M = K = 37
            N = 29
            A = np.zeros((M, K), np.uint16)
            A[np.arange(M), np.arange(K)] = ONE[fmt]
            Bkn = gen.normal((K, N), 21, 1, fmt)
            sbk, sbn = _strides(layout, N, K)
            C, S = orc.gemm(fmt, M, N, K, A, K, 1, _store_b(Bkn, layout), sbk, sbn)
            want = lib_decode(fmt, Bkn)
            assert np.array_equal(C, want), "identity: C != B"
            assert np.array_equal(S, np.abs(want)), "identity: S != |B|"


def pin_selection(orc):
    """A[i,k] = 1 iff k = pi(i) (M < K): C[i,:] = B[pi(i),:] exactly."""
    for fmt in ("bf16", "f16"):
        for layout in ("kn", "nk"):
            M, N, K = 23, 31, 41
            pi = np.random.default_rng(4).permutation(K)[:M]
            A = np.zeros((M, K), np.uint16)
            A[np.arange(M), pi] = ONE[fmt]
            Bkn = gen.uniform_pm1((K, N), 22, 1, fmt)
            sbk, sbn = _strides(layout, N, K)
            C, _ = orc.gemm(fmt, M, N, K, A, K, 1, _store_b(Bkn, layout), sbk, sbn)
            assert np.array_equal(C, lib_decode(fmt, Bkn)[pi, :]), "selection: wrong rows"


def pin_rank1(orc):
    """A = u w^T, B = w v^T with small integers: C = (w.w) u v^T exactly."""
    rng = np.random.default_rng(5)
    M, N, K = 19, 13, 27
    u = rng.integers(-15, 16, M)
    v = rng.integers(-15, 16, N)
    w = rng.integers(-15, 16, K)
    for fmt in ("bf16", "f16"):
        for layout in ("kn", "nk"):
            A = lib_encode(fmt, np.outer(u, w))
            Bkn = lib_encode(fmt, np.outer(w, v))
            sbk, sbn = _strides(layout, N, K)
            C, S = orc.gemm(fmt, M, N, K, A, K, 1, _store_b(Bkn, layout), sbk, sbn)
            ww = int(np.dot(w, w))
            assert np.array_equal(C, (ww * np.outer(u, v)).astype(np.float64)), "rank-1"
            assert np.array_equal(S, (ww * np.outer(np.abs(u), np.abs(v))).astype(np.float64))


def pin_all_ones(orc):
    for K in (1, 7, 256, 1000):
        M, N = 3, 5
        A = np.full((M, K), ONE["bf16"], np.uint16)
        B = np.full((K, N), ONE["bf16"], np.uint16)
        C, S = orc.gemm("bf16", M, N, K, A, K, 1, B, N, 1)
        assert np.all(C == K) and np.all(S == K), "all-ones: C != K"
    C, S = orc.gemm("bf16", 2, 3, 0, np.zeros(1, np.uint16), 0, 1, np.zeros(1, np.uint16), 3, 1)
    assert np.all(C == 0) and np.all(S == 0), "K = 0 must give zeros"


def pin_bruteforce_integers(orc):
    """Tiny integer inputs: C and S equal Python exact-integer sums."""
    rng = np.random.default_rng(6)
    for trial in range(40):
        M, N, K = (int(x) for x in rng.integers(1, 10, 3))
        fmt = ("bf16", "f16")[trial % 2]
        layout = ("kn", "nk")[(trial // 2) % 2]
        a = rng.integers(-8, 9, (M, K))
        b = rng.integers(-8, 9, (K, N))
        sbk, sbn = _strides(layout, N, K)
        C, S = orc.gemm(fmt, M, N, K, lib_encode(fmt, a), K, 1,
                        _store_b(lib_encode(fmt, b), layout), sbk, sbn)
        for i in range(M):
            for j in range(N):
                c = sum(int(a[i, k]) * int(b[k, j]) for k in range(K))
                s = sum(abs(int(a[i, k])) * abs(int(b[k, j])) for k in range(K))
                assert C[i, j] == c and S[i, j] == s, f"brute force ({M},{N},{K}) at {i},{j}"


def pin_bruteforce_rationals(orc):
    """Random (non-integer) codes: C within fp64 summation error of the exact
    rational sum; the products of two 16-bit values are exact in fp64."""
    for fmt in ("bf16", "f16"):
        for layout in ("kn", "nk"):
            M, N, K = 4, 5, 33
            A = gen.normal((M, K), 23, 0, fmt)
            Bkn = gen.normal((K, N), 23, 1, fmt)
            a, b = lib_decode(fmt, A), lib_decode(fmt, Bkn)
            sbk, sbn = _strides(layout, N, K)
            C, S = orc.gemm(fmt, M, N, K, A, K, 1, _store_b(Bkn, layout), sbk, sbn)
            for i in range(M):
                for j in range(N):
                    exact = sum(Fraction(a[i, k]) * Fraction(b[k, j]) for k in range(K))
                    mag = sum(abs(Fraction(a[i, k]) * Fraction(b[k, j])) for k in range(K))
                    tol = Fraction(2 * K) * Fraction(2.0 ** -53) * mag
                    assert abs(Fraction(C[i, j]) - exact) <= tol, "rational brute force"
                    assert abs(Fraction(S[i, j]) - mag) <= tol


def pin_numpy_matmul(orc):
    """Against NumPy's fp64 matmul (a library routine) on a larger shape."""
    M, N, K = 70, 45, 300
    for fmt in ("bf16", "f16"):
        A = gen.normal((M, K), 24, 0, fmt)
        Bnk = gen.normal((N, K), 24, 1, fmt)
        a, bt = lib_decode(fmt, A), lib_decode(fmt, Bnk)
        C, S = orc.gemm(fmt, M, N, K, A, K, 1, Bnk, 1, K)
        ref = a @ bt.T
        sref = np.abs(a) @ np.abs(bt).T
        assert np.all(np.abs(C - ref) <= 1e-12 * sref), "numpy matmul"
        assert np.all(np.abs(S - sref) <= 1e-12 * sref), "numpy |a||b|"
        assert np.all(S >= np.abs(C)), "S >= |C|"


def pin_layout_invariance(orc):
    """The same logical A and B in different storage give identical bits."""
    M, N, K = 17, 23, 29
    A = gen.normal((M, K), 25, 0, "bf16")
    Bkn = gen.normal((K, N), 25, 1, "bf16")
    C0, S0 = orc.gemm("bf16", M, N, K, A, K, 1, Bkn, N, 1)
    C1, S1 = orc.gemm("bf16", M, N, K, A, K, 1, np.ascontiguousarray(Bkn.T), 1, K)
    # A column-major, B K x N with a padded leading stride
    Acm = np.ascontiguousarray(A.T)
    Bpad = np.zeros((K, N + 3), np.uint16)
    Bpad[:, :N] = Bkn
    C2, S2 = orc.gemm("bf16", M, N, K, Acm, 1, M, Bpad, N + 3, 1)
    # every other column / element: non-unit strides along both k and j
    Bwide = np.zeros((K, 2 * N), np.uint16)
    Bwide[:, ::2] = Bkn
    Awide = np.zeros((M, 2 * K), np.uint16)
    Awide[:, ::2] = A
    C3, S3 = orc.gemm("bf16", M, N, K, Awide, 2 * K, 2, Bwide, 2 * N, 2)
    for C, S in ((C1, S1), (C2, S2), (C3, S3)):
        assert np.array_equal(C, C0) and np.array_equal(S, S0), "layout changed the result"
    # asymmetric check that catches swapped A strides
    a, b = lib_decode("bf16", A), lib_decode("bf16", Bkn)
    assert np.all(np.abs(C0 - a @ b) <= 1e-12 * (np.abs(a) @ np.abs(b))), "strided A/B"


def pin_row_subset(orc):
    M, N, K = 40, 11, 13
    A = gen.normal((M, K), 26, 0, "f16")
    B = gen.normal((K, N), 26, 1, "f16")
    Cf, Sf = orc.gemm("f16", M, N, K, A, K, 1, B, N, 1)
    rows = np.array([39, 0, 17, 5])
    Cr, Sr = orc.gemm("f16", M, N, K, A, K, 1, B, N, 1, rows=rows)
    assert np.array_equal(Cr, Cf[rows]) and np.array_equal(Sr, Sf[rows]), "row subset"


def pin_nonnegative_s_equals_c(orc):
    M, N, K = 9, 8, 50
    A = gen.fill((M, K), gen.DIST_UNIFORM, 27, 0, "f64")
    B = gen.fill((K, N), gen.DIST_UNIFORM, 27, 1, "f64")
    A = lib_encode("bf16", np.abs(A))
    B = lib_encode("bf16", np.abs(B))
    C, S = orc.gemm("bf16", M, N, K, A, K, 1, B, N, 1)
    assert np.array_equal(C, S), "S must equal C for non-negative inputs"


# ------------------------------------------------------- fp8 block-scaled GEMM

def _dyadic_scales(rng, shape):
    """Scales m * 2^e with 6-bit m: every product and partial sum stays exact."""
    m = rng.integers(1, 64, shape).astype(np.float64)
    e = rng.integers(-8, 3, shape).astype(np.float64)
    return (m * np.exp2(e)).astype(np.float32)


def pin_fp8_unit_codes(orc):
    """qa = qb = 1: C[i,j] = sum_kb n_kb * sa[i,kb] * sb[j/128,kb] exactly,
    n_kb = number of k in block kb (128, or the tail length)."""
    rng = np.random.default_rng(8)
    M, N, K = 5, 300, 400
    nkb, nnb = -(-K // 128), -(-N // 128)
    QA = np.full((M, K), E4M3_ONE, np.uint8)
    QB = np.full((N, K), E4M3_ONE, np.uint8)
    SA = _dyadic_scales(rng, (M, nkb))
    SB = _dyadic_scales(rng, (nnb, nkb))
    C, S = orc.gemm_fp8_blockscaled(M, N, K, QA, K, 1, SA, nkb, 1, QB, 1, K, SB, nkb, 1)
    for i in range(M):
        for j in range(N):
            want = sum(Fraction(min(128, K - 128 * kb)) * Fraction(float(SA[i, kb]))
                       * Fraction(float(SB[j // 128, kb])) for kb in range(nkb))
            assert Fraction(C[i, j]) == want, f"fp8 closed form at {i},{j}"
            assert Fraction(S[i, j]) == want


def pin_fp8_bruteforce(orc):
    """Random codes and fp32 scales, partial blocks in K and N: C within fp64
    rounding of the exact rational sum of (code * scale) products."""
    rng = np.random.default_rng(9)
    M, N, K = 3, 150, 300
    nkb, nnb = -(-K // 128), -(-N // 128)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    QA = rng.choice(finite, (M, K)).astype(np.uint8)
    QB = rng.choice(finite, (N, K)).astype(np.uint8)
    SA = rng.uniform(0.001, 0.01, (M, nkb)).astype(np.float32)
    SB = rng.uniform(0.001, 0.01, (nnb, nkb)).astype(np.float32)
    a, b = lib_decode("e4m3fn", QA), lib_decode("e4m3fn", QB)
    for layout in ("nk", "kn"):
        if layout == "nk":
            C, S = orc.gemm_fp8_blockscaled(M, N, K, QA, K, 1, SA, nkb, 1, QB, 1, K, SB, nkb, 1)
        else:
            QBkn = np.ascontiguousarray(QB.T)
            C, S = orc.gemm_fp8_blockscaled(M, N, K, QA, K, 1, SA, nkb, 1, QBkn, N, 1, SB, nkb, 1)
        for i in range(M):
            for j in range(0, N, 7):
                terms = [Fraction(a[i, k]) * Fraction(float(SA[i, k // 128]))
                         * Fraction(b[j, k]) * Fraction(float(SB[j // 128, k // 128]))
                         for k in range(K)]
                exact = sum(terms)
                mag = sum(abs(t) for t in terms)
                tol = Fraction(4 * K) * Fraction(2.0 ** -53) * mag
                assert abs(Fraction(C[i, j]) - exact) <= tol, f"fp8 brute force {layout} {i},{j}"
                assert abs(Fraction(S[i, j]) - mag) <= tol


def pin_fp8_layout_and_rows(orc):
    rng = np.random.default_rng(10)
    M, N, K = 6, 130, 260
    nkb, nnb = -(-K // 128), -(-N // 128)
    QA = rng.integers(0, 0x7E, (M, K)).astype(np.uint8)
    QB = rng.integers(0x80, 0xFE, (N, K)).astype(np.uint8)
    SA = rng.uniform(0.5, 2, (M, nkb)).astype(np.float32)
    SB = rng.uniform(0.5, 2, (nnb, nkb)).astype(np.float32)
    C0, S0 = orc.gemm_fp8_blockscaled(M, N, K, QA, K, 1, SA, nkb, 1, QB, 1, K, SB, nkb, 1)
    C1, S1 = orc.gemm_fp8_blockscaled(M, N, K, QA, K, 1, SA, nkb, 1, np.ascontiguousarray(QB.T),
                                      N, 1, SB, nkb, 1)
    assert np.array_equal(C0, C1) and np.array_equal(S0, S1), "fp8 layout"
    rows = np.array([5, 2])
    Cr, _ = orc.gemm_fp8_blockscaled(M, N, K, QA, K, 1, SA, nkb, 1, QB, 1, K, SB, nkb, 1,
                                     rows=rows)
    assert np.array_equal(Cr, C0[rows]), "fp8 row subset"
    assert np.all(C0 <= 0), "positive A codes times negative B codes must give C <= 0"


# ------------------------------------------------------------------ codecs

def pin_decoders(orc):
    codes16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    codes8 = np.arange(256, dtype=np.uint16).astype(np.uint8)
    for fmt, codes in (("bf16", codes16), ("f16", codes16), ("e4m3fn", codes8)):
        got, want = orc.decode(fmt, codes), lib_decode(fmt, codes)
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan], want[~nan]), \
            f"decoder {fmt}"


def pin_rounding(orc):
    """RNE to the output format against library casts (single rounding) and
    constructed ties."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal(50000) * 100.0
    assert np.array_equal(orc.round_to("f16", x), x.astype(np.float16).view(np.uint16)), "f16"
    x32 = (rng.standard_normal(50000) * 100.0).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.round_to("bf16", x32.astype(np.float64)), want), "bf16"
    # ties: 257 lies halfway between 256 and 258 in bf16 -> 256 (even); 259 -> 260
    assert orc.round_to("bf16", np.array([257.0, 259.0, -257.0])).tolist() == \
        lib_encode("bf16", np.array([256.0, 260.0, -256.0])).tolist(), "bf16 ties"
    assert orc.round_to("f16", np.array([2049.0, 2051.0])).tolist() == \
        lib_encode("f16", np.array([2048.0, 2052.0])).tolist(), "f16 ties"



# ------------------------------------------------------- fp8 block quantiser

def _fp32_div(a, b):
    """IEEE fp32 quotient (numpy's float32 division)."""
    return (np.float32(a) / np.float32(b)).astype(np.float32)


def _blocks(R, K, br):
    for ib in range((R + br - 1) // br):
        for kb in range((K + 127) // 128):
            yield ib, kb, slice(ib * br, min(R, ib * br + br)), slice(kb * 128, min(K, kb * 128 + 128))


def pin_quant_codes_match_torch(orc):
    """With 448 in every block the scale is exactly 1, so the codes are the
    e4m3fn rounding of the inputs themselves: torch's float8_e4m3fn cast
    (round to nearest even) must agree -- on every representable value, every
    midpoint between neighbours (ties), random values, tiny values in the
    subnormal range and signed zeros."""
    pos = lib_decode("e4m3fn", np.arange(0, 127, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(11)
    vals = np.concatenate([pos, -pos, mids, -mids, rng.uniform(-448, 448, 4000),
                           np.exp2(rng.uniform(-13, -5, 2000)) * rng.choice([-1, 1], 2000),
                           [0.0, -0.0, 448.0, -448.0]]).astype(np.float32)
    per = 127
    rows = -(-vals.size // per)
    X = np.zeros((rows, 128), np.float32)
    X[:, 0] = 448.0
    flat = np.zeros(rows * per, np.float32)
    flat[:vals.size] = vals
    X[:, 1:] = flat.reshape(rows, per)
    for br in (1, 128):
        Q, S = orc.quant_fp8(X, br)
        assert np.all(S == 1.0), "scale of a block whose maximum is 448"
        want = torch.from_numpy(X.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(Q, want), "e4m3fn rounding differs from torch's cast"


def _quant_data(R, K, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((R, K)).astype(np.float32)
    X *= np.exp2(rng.integers(-20, 20, (R, 1))).astype(np.float32)   # rows of varied scale
    return X


def pin_quant_scales_and_bounds(orc):
    """Each scale is the fp32 quotient amax / 448 (numpy's IEEE division);
    in every block the largest code decodes to +-448 exactly and every code
    is within half an e4m3fn step of x / s (plus the fp32 quotient's own
    rounding)."""
    for R, K, br in ((130, 300, 1), (300, 257, 128), (1, 128, 1), (129, 1, 128)):
        X = _quant_data(R, K, 100 + R + K)
        Q, S = orc.quant_fp8(X, br)
        dq = lib_decode("e4m3fn", Q)
        for ib, kb, rs, ks in _blocks(R, K, br):
            blk = X[rs, ks]
            amax = np.abs(blk).max()
            s = _fp32_div(amax, 448.0)
            assert S[ib, kb] == s, (R, K, br, ib, kb)
            d = dq[rs, ks]
            assert np.abs(d).max() == 448.0, "the block maximum maps to 448"
            y = np.abs(blk.astype(np.float64) / np.float64(s))
            step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(y, 2.0 ** -30))) - 3, -9))
            assert np.all(np.abs(np.abs(d) - np.minimum(y, 448.0)) <= step / 2 + 448 * 2.0 ** -22)
            assert np.all((d == 0) | (np.sign(d) == np.sign(blk)))


def pin_quant_edge_blocks(orc):
    """A zero block, and a block whose maximum over 448 underflows fp32, get
    scale 1 and zero codes; a block whose scale is a coarse fp32 subnormal
    (2 x 2^-149 for a maximum of 1075 x 2^-149) gives quotients above 448,
    which clamp to 448, and rounds the rest on the e4m3fn grid."""
    t = np.float32(2.0 ** -149)
    X = np.zeros((3, 128), np.float32)
    X[1, 5] = t                      # 2^-149 / 448 underflows
    X[2, 0] = 1075 * t               # s = fl(1075/448 * 2^-149) = 2 * 2^-149
    X[2, 1] = -300 * t               # -150 -> -144 on the grid
    X[2, 2] = 32 * t                 # 16 exactly
    Q, S = orc.quant_fp8(X, 1)
    assert S[0, 0] == 1.0 and not Q[0].any()
    assert S[1, 0] == 1.0 and not Q[1].any()
    assert S[2, 0] == np.float32(2 * t)
    got = lib_decode("e4m3fn", Q[2, :3])
    assert list(got) == [448.0, -144.0, 16.0], got
    assert not Q[2, 3:].any()


def pin_quant_block_relation(orc):
    """The 128 x 128 scale of a block is the largest of its rows' 1 x 128
    scales (the maximum commutes with the monotone, correctly rounded
    division)."""
    X = _quant_data(300, 400, 7)
    _, S1 = orc.quant_fp8(X, 1)
    _, S2 = orc.quant_fp8(X, 128)
    for ib in range(S2.shape[0]):
        assert np.array_equal(S2[ib], S1[ib * 128:(ib + 1) * 128].max(axis=0))


def pin_quant_matches_generator(orc):
    """The input generator's own block quantiser (separate code, same
    reading) agrees bit for bit on ordinary data."""
    for R, K, br in ((200, 333, 1), (260, 384, 128)):
        X = _quant_data(R, K, 3 + R)
        Q, S = orc.quant_fp8(X, br)
        Qg, Sg = gen.quant_e4m3fn(X, br, 128)
        assert np.array_equal(Q, Qg) and np.array_equal(S, Sg)


def pin_gemm_quant_identity(orc):
    """An identity A selects the rows of B, so C = B exactly: with a 448 in
    every 128-column slice the scale is 1 and the codes are torch's e4m3fn
    cast of B's values (a transposed operand, a wrong slice width or a slice
    taken down a column instead of along a row would all differ)."""
    rng = np.random.default_rng(21)
    for fmt in ("bf16", "f16"):
        M = K = 40
        N = 300
        vals = lib_decode(fmt, lib_encode(fmt, rng.uniform(-440, 440, (K, N))))
        vals[:, ::128] = 448.0 * rng.choice([-1.0, 1.0], (K, (N + 127) // 128))
        B = lib_encode(fmt, vals)                     # K x N, N-contiguous
        A = lib_encode(fmt, np.eye(M, K))
        Q, S, C, _ = orc.gemm_quant_fp8(fmt, M, N, K, A, K, 1, B, N, 1)
        assert np.array_equal(C, vals)
        assert np.all(S == 1.0), "slice maximum 448 gives scale 1"
        want = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn)
        assert np.array_equal(Q, want.view(torch.uint8).numpy())


def pin_gemm_quant_integers(orc):
    """Small integer operands: the product is numpy's exact int64 matmul; each
    slice's scale is numpy's fp32 quotient of its maximum by 448 and each code
    torch's e4m3fn cast of the fp32 quotient C / scale.  Ragged last slice
    (N = 333), rows of very different size, and a zero row (scale 1, codes 0)."""
    rng = np.random.default_rng(22)
    M, N, K = 37, 333, 50
    Ai = rng.integers(-8, 9, (M, K)) * (2 ** rng.integers(0, 6, (M, 1)))
    Ai[5] = 0
    Bi = rng.integers(-8, 9, (K, N))
    Ci = Ai @ Bi
    A, B = lib_encode("bf16", Ai), lib_encode("bf16", Bi)
    Q, S, C, _ = orc.gemm_quant_fp8("bf16", M, N, K, A, K, 1, B, N, 1)
    assert np.array_equal(C, Ci)
    for i in range(M):
        for j in range((N + 127) // 128):
            blk = Ci[i, j * 128:(j + 1) * 128].astype(np.float32)
            s = _fp32_div(np.abs(blk).max(), 448.0)
            if s == 0:
                assert S[i, j] == 1.0 and not Q[i, j * 128:(j + 1) * 128].any()
                continue
            assert S[i, j] == s, (i, j)
            y = np.clip(blk / s, -448, 448).astype(np.float32)
            want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(Q[i, j * 128:(j + 1) * 128], want), (i, j)


# ---------------------------------------------------------- SwiGLU

def pin_swiglu_closed_forms(orc):
    """silu(g) = g / (1 + e^-g) at points with closed forms, with u = 1:
    silu(0) = 0; silu(ln 3) = (3/4) ln 3 and silu(-ln 3) = -(1/4) ln 3 (e^-ln3
    = 1/3); silu(t) - silu(-t) = t for every t; silu(50) = 50 in fp64.  And
    h = silu(g) * u scales with u: u = -2.5 gives -2.5 silu(g).  (A sign slip
    in the exponent, the gate and up roles swapped, a missing division or a
    missing factor g each break one of these.)"""
    ln3 = np.log(3.0)
    G = np.array([0.0, ln3, -ln3, 50.0, 0.7, -0.7, 3.25, -3.25])
    H = orc.swiglu(G, np.ones_like(G))
    assert H[0] == 0.0
    assert abs(H[1] - 0.75 * ln3) <= 1e-15 and abs(H[2] + 0.25 * ln3) <= 1e-15
    assert H[3] == 50.0
    for a, b in ((4, 5), (6, 7)):
        assert abs((H[a] - H[b]) - G[a]) <= 1e-15, (H[a], H[b], G[a])
    H2 = orc.swiglu(G, np.full_like(G, -2.5))
    assert np.all(np.abs(H2 - (-2.5) * H) <= 1e-15 * np.abs(H) + 1e-300)


def pin_swiglu_selection(orc):
    """With A = I the gate and up products select the weights' rows, so h at
    (i, n) is silu(Bg[n, i]) * Bu[n, i] (weights stored N x K): element by
    element on exactly representable values, in both formats (a transposed
    weight, a swapped gate and up, or a row offset would all differ)."""
    rng = np.random.default_rng(31)
    for fmt in ("bf16", "f16"):
        M = K = 24
        N = 150
        gv = lib_decode(fmt, lib_encode(fmt, rng.uniform(-6, 6, (N, K))))
        uv = lib_decode(fmt, lib_encode(fmt, rng.uniform(-3, 3, (N, K))))
        Bg, Bu = lib_encode(fmt, gv), lib_encode(fmt, uv)   # N x K, K-contiguous
        A = lib_encode(fmt, np.eye(M, K))
        Q, SC, H, G, U, _, _ = orc.swiglu_quant_fp8(fmt, M, N, K, A, K, 1, Bg, Bu, 1, K)
        assert np.array_equal(G, gv.T) and np.array_equal(U, uv.T)
        want = gv.T / (1.0 + np.exp(-gv.T)) * uv.T
        assert np.all(np.abs(H - want) <= 1e-15 * np.abs(want))


def pin_swiglu_quant_large_gate(orc):
    """Positive integer inputs and gate weights make every gate value at least
    K = 200, where 1 + e^-g rounds to 1 and silu(g) = g exactly: h is numpy's
    exact integer product (A Bg) * (A Bu), and each 1 x 128 slice's scale and
    codes are numpy's fp32 quotient of its maximum by 448 and torch's e4m3fn
    cast of h / scale (ragged last slice, N = 300)."""
    rng = np.random.default_rng(32)
    M, N, K = 20, 300, 200
    Ai = rng.integers(1, 4, (M, K))
    Gw = rng.integers(1, 4, (N, K))
    Uw = rng.integers(-3, 4, (N, K))
    A, Bg, Bu = lib_encode("bf16", Ai), lib_encode("bf16", Gw), lib_encode("bf16", Uw)
    Q, SC, H, G, U, _, _ = orc.swiglu_quant_fp8("bf16", M, N, K, A, K, 1, Bg, Bu, 1, K)
    Hi = (Ai @ Gw.T) * (Ai @ Uw.T)
    assert np.array_equal(H, Hi)
    for i in range(M):
        for j in range((N + 127) // 128):
            blk = Hi[i, j * 128:(j + 1) * 128].astype(np.float32)
            s = _fp32_div(np.abs(blk).max(), 448.0)
            assert SC[i, j] == s, (i, j)
            y = np.clip(blk / s, -448, 448).astype(np.float32)
            want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(Q[i, j * 128:(j + 1) * 128], want), (i, j)


# ---------------------------------------------------------- acceptance bound

def pin_bound_constants(orc):
    """The tolerance is 4 * 2^-8 * S for bf16 output and 4 * 2^-11 * S for
    fp16 output (the constants written out here), i.e. four unit roundoffs of
    the output format, the unit roundoff being half the format's epsilon as
    torch describes it; S = 0 gives a zero tolerance."""
    rng = np.random.default_rng(21)
    S = np.concatenate([[0.0, 1.0, 3.0, 1e-30, 1e30], rng.exponential(5.0, 1000)])
    for fmt, const, dtype in (("bf16", 4.0 * 2.0 ** -8, torch.bfloat16),
                              ("f16", 4.0 * 2.0 ** -11, torch.float16)):
        got = orc.bound(fmt, S)
        assert np.array_equal(got, const * S), f"bound constant {fmt}"
        unit = torch.finfo(dtype).eps / 2.0
        assert np.array_equal(got, 4.0 * unit * S), f"bound vs unit roundoff {fmt}"
        assert got[0] == 0.0


def _fp32_sequential(a: np.ndarray, b: np.ndarray, order) -> np.ndarray:
    """sum_k a[i,k] b[k,j] accumulated in fp32 (products exact for 16-bit
    inputs) in the given k order: a model of the GPU's accumulation."""
    acc = np.zeros((a.shape[0], b.shape[1]), np.float32)
    for k in order:
        acc = (acc + np.outer(a[:, k], b[k, :]).astype(np.float32)).astype(np.float32)
    return acc


def pin_bound_model(orc):
    """An fp32-accumulating product rounded once to the output format stays
    within the tolerance (in ascending, descending and shuffled k order, at
    K = 16384 and on cancelling sums), while a result off by 2^-5 * S does
    not: the bound admits the arithmetic the method allows and no more."""
    rng = np.random.default_rng(22)
    for fmt in ("bf16", "f16"):
        for K in (16384, 1000):
            M, N = 3, 4
            a = lib_decode(fmt, lib_encode(fmt, rng.standard_normal((M, K)) / np.sqrt(K)))
            b = lib_decode(fmt, lib_encode(fmt, rng.standard_normal((K, N))))
            a[0, :] = np.abs(a[0, :])                 # a row of same-sign terms
            c_ref = a @ b
            S = np.abs(a) @ np.abs(b)
            tol = orc.bound(fmt, S)
            for order in (range(K), range(K - 1, -1, -1), rng.permutation(K)):
                c32 = _fp32_sequential(a, b, order).astype(np.float64)
                got = lib_decode(fmt, lib_encode(fmt, c32 if fmt == "f16" else
                                                 c32.astype(np.float32)))
                assert np.all(np.abs(got - c_ref) <= tol), f"model outside bound {fmt} K={K}"
            assert np.all(2.0 ** -5 * S > tol), f"bound too loose {fmt}"


ALL_PINS = [pin_identity, pin_selection, pin_rank1, pin_all_ones, pin_bruteforce_integers,
            pin_bruteforce_rationals, pin_numpy_matmul, pin_layout_invariance, pin_row_subset,
            pin_nonnegative_s_equals_c, pin_fp8_unit_codes, pin_fp8_bruteforce,
            pin_fp8_layout_and_rows, pin_decoders, pin_rounding, pin_quant_codes_match_torch,
            pin_quant_scales_and_bounds, pin_quant_edge_blocks, pin_quant_block_relation,
            pin_quant_matches_generator, pin_gemm_quant_identity, pin_gemm_quant_integers,
            pin_swiglu_closed_forms, pin_swiglu_selection, pin_swiglu_quant_large_gate,
            pin_bound_constants, pin_bound_model]
