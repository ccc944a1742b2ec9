"""The fp8 block quantiser on the GPU (tg_quant_fp8_1x128 / _128x128, through
the C-ABI) against the CPU oracle: codes and scales must agree bit for bit.

Inputs: seeded N(0, 1) fp32 with rows of varied magnitude, the fp8
workload's own operands at full size (A 4096 x 16384 with 1 x 128 scales, B
7168 x 16384 with 128 x 128 scales), ragged and padded shapes, and
constructed blocks (zeros, a maximum whose scale underflows, a coarse
subnormal scale, e4m3fn ties, signed zeros), rows of extreme scale, and a
strided sweep of every fp32 value up to 448 with scale 1.  The quantised
operands then go through the block-scaled product and are checked against
the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_tiled_gemm_03_amd as tg
import gen
import oracle
from gen import configs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    return gpu_lib


def _gpu_quant(X: np.ndarray, br: int, ldx=None, ldq=None):
    """Quantise X (R x K fp32) on the GPU; optional padded leading dims."""
    R, K = X.shape
    ldx = K if ldx is None else ldx
    ldq = K if ldq is None else ldq
    xb = np.zeros((R, ldx), np.float32)
    xb[:, :K] = X
    Xd = torch.from_numpy(xb).cuda()
    Qd = torch.full((R * ldq + 64,), 0x5A, dtype=torch.uint8, device="cuda")
    nrb, nkb = -(-R // br), -(-K // 128)
    Sd = torch.full((nrb * nkb + 16,), -7.0, dtype=torch.float32, device="cuda")
    fn = tg.tg_quant_fp8_1x128 if br == 1 else tg.tg_quant_fp8_128x128
    H.log(f"quant br={br} R={R} K={K} ldx={ldx} ldq={ldq}")
    fn(R, K, Xd.data_ptr(), ldx, Qd.data_ptr(), ldq, Sd.data_ptr(), nkb, 1,
       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    q = Qd.cpu().numpy()
    s = Sd.cpu().numpy()
    # nothing written past the codes / scales
    assert np.all(q[R * ldq:] == 0x5A) and np.all(s[nrb * nkb:] == -7.0)
    if ldq > K:
        assert np.all(q[:R * ldq].reshape(R, ldq)[:, K:] == 0x5A), "padding of Q written"
    return q[:R * ldq].reshape(R, ldq)[:, :K], s[:nrb * nkb].reshape(nrb, nkb)


def _check(X, br, **kw):
    q, s = _gpu_quant(X, br, **kw)
    Qo, So = oracle.quant_fp8(X, br)
    R, K = X.shape
    assert np.array_equal(s.view(np.uint32), So.view(np.uint32)), f"scales differ {R}x{K} br={br}"
    bad = q != Qo
    if bad.any():
        i, k = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} codes differ ({R}x{K} br={br}); first at ({i},{k}): "
                             f"x={X[i, k]!r} got {q[i, k]:#04x} want {Qo[i, k]:#04x}")


def _data(R, K, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((R, K)).astype(np.float32)
    return X * np.exp2(rng.integers(-20, 20, (R, 1))).astype(np.float32)


SHAPES = [(1, 1), (3, 130), (130, 257), (129, 1000), (257, 129), (64, 128), (300, 384)]


@pytest.mark.parametrize("br", [1, 128])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{r}x{k}" for r, k in SHAPES])
def test_quant_shapes(shape, br):
    R, K = shape
    _check(_data(R, K, 10 + R + K), br)


@pytest.mark.parametrize("br", [1, 128])
def test_quant_padded(br):
    """Padded leading dimensions: aligned (vector path) and not (element path)."""
    X = _data(200, 300, 5)
    _check(X, br, ldx=304, ldq=320)
    _check(X, br, ldx=301, ldq=303)


@pytest.mark.parametrize("br", [1, 128])
def test_quant_edge_blocks(br):
    """Zero blocks, a maximum whose quotient by 448 underflows, a coarse
    subnormal scale (quotients above 448 clamp), e4m3fn midpoints with a
    scale of exactly 1, and signed zeros."""
    t = np.float32(2.0 ** -149)
    X = np.zeros((256, 384), np.float32)
    X[1, 5] = t
    X[2, 0], X[2, 1], X[2, 2] = 1075 * t, -300 * t, 32 * t
    pos = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = (pos[:-1] + pos[1:]) / 2
    ties = np.zeros(3 * 127, np.float32)
    vals = np.concatenate([mids, -mids, [-0.0, 0.0, -1e-6, 1e-6]]).astype(np.float32)
    ties[:vals.size] = vals
    for r in range(3, 6):
        X[r, 128] = 448.0
        X[r, 129:256] = ties[(r - 3) * 127:(r - 2) * 127]
    X[6, 256:] = -0.0
    _check(X, br)


def test_quant_e4m3_grid():
    """Blocks whose maximum is 448 have scale 1, so their codes are the
    e4m3fn rounding of the inputs themselves: every 61st fp32 bit pattern of
    magnitude up to 448 in both signs, and every e4m3fn midpoint with its
    four neighbours on each side, against the oracle bit for bit."""
    lim = 0x43E00000                                   # 448.0
    mags = np.arange(0, lim + 1, 61, dtype=np.uint32)
    pos = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32).view(np.uint32)
    near = (mids[:, None].astype(np.int64) + np.arange(-4, 5)[None, :]).ravel()
    mags = np.concatenate([mags, near[(near >= 0) & (near <= lim)].astype(np.uint32)])
    vals = np.concatenate([mags, mags | np.uint32(0x80000000)]).view(np.float32)
    rows = -(-vals.size // 127)
    X = np.zeros((rows, 128), np.float32)
    X[:, 0] = 448.0
    flat = np.zeros(rows * 127, np.float32)
    flat[:vals.size] = vals
    X[:, 1:] = flat.reshape(rows, 127)
    _check(X, 1)


@pytest.mark.parametrize("br", [1, 128])
def test_quant_extreme_scales(br):
    """Rows whose scales lie far outside 2^-60 .. 2^60 (divided exactly)
    next to ordinary rows (reciprocal and one correction), so waves and
    workgroups mix both ways of forming x / s."""
    rng = np.random.default_rng(77)
    R, K = 384, 512
    X = rng.standard_normal((R, K)).astype(np.float32)
    exps = rng.choice([-100, -75, -62, -58, 0, 20, 58, 62, 75, 100], R)
    X *= np.exp2(exps.astype(np.float64))[:, None].astype(np.float32)
    _check(X, br)


def test_quant_workload_operands():
    """The fp8 workload's operands at full size: A with 1 x 128 scales, B
    (stored N x K) with 128 x 128 scales."""
    w = configs.WORKLOADS["fp8_4096x7168x16384"]
    A = gen.normal((w.M, w.K), w.seed, 0, "f32")
    _check(A, 1)
    del A
    B = gen.normal((w.N, w.K), w.seed, 1, "f32")
    _check(B, 128)


def test_quant_then_product():
    """Quantise A (1 x 128) and B (128 x 128) on the GPU and multiply them
    with tg_gemm_fp8_blockscaled: the operands are the oracle's bit for bit,
    and the product is within the bound of the oracle's product of them."""
    M, N, K = 300, 260, 1000
    A, B = _data(M, K, 1), _data(N, K, 2)
    qa, sa = _gpu_quant(A, 1)
    qb, sb = _gpu_quant(B, 128)
    Qa, Sa = oracle.quant_fp8(A, 1)
    Qb, Sb = oracle.quant_fp8(B, 128)
    assert np.array_equal(qa, Qa) and np.array_equal(qb, Qb)
    assert np.array_equal(sa, Sa) and np.array_equal(sb, Sb)
    nkb = sa.shape[1]
    c, plan = H.run_fp8(M, N, K, H.dev(qa), K, 1, H.dev(sa), nkb, 1, H.dev(qb), 1, K, H.dev(sb),
                        nkb, 1)
    C_ref, S = oracle.gemm_fp8_blockscaled(M, N, K, Qa, K, 1, Sa, nkb, 1, Qb, 1, K, Sb, nkb, 1)
    H.assert_within_bound("bf16", c, C_ref, S, f"quantised product [{plan}]")
