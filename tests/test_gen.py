"""The seeded input generator: reproducible bytes, thread-count independence,
the published SplitMix64 output function, sane moments, and the e4m3fn block
quantiser's invariants."""
import hashlib
import os
import subprocess
import sys

import numpy as np
import pytest

import gen
from gen import configs
from tests.oracle_pins import lib_decode

MASK = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15


def _splitmix_out(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def test_draws_follow_splitmix64_definition():
    for seed, stream in ((0, 0), (3, 1), (12345, 2)):
        key = _splitmix_out(_splitmix_out((seed + GOLDEN) & MASK) + stream * GOLDEN & MASK)
        want = [_splitmix_out((key + (i + 1) * GOLDEN) & MASK) for i in range(50)]
        assert gen.draws(seed, stream, 50).tolist() == want


# SHA-256 of the first 1000 elements, pinned when the generator was written.
PINNED = [
    (((1000,), gen.DIST_UNIFORM, 1, 0, "f16"), 0,
     "1eaf1e0ab5307ab16885d7043aef6c710682af2c39a7d3b3da803c54a5f156eb"),
    (((1000,), gen.DIST_NORMAL, 3, 1, "bf16"), 0,
     "7160560b6557c6e2c8e96d00f6632de6ec8fc5920ff551f3dc7d6795d8c3d65a"),
    (((1000,), gen.DIST_NORMAL, 5, 0, "f32"), 0,
     "f456eb03cdcb9abdea63ec932a345772bad0b53c70bbe85354101bae22b8d033"),
    (((1000,), gen.DIST_INT, 2, 0, "bf16"), 32,
     "555745ce2b1abde6d7341ce2e0b278ea0fdf07dc8eb550b9f55a6ff0800e2e0b"),
]


@pytest.mark.parametrize("args,param,digest", PINNED)
def test_pinned_bytes(args, param, digest):
    assert hashlib.sha256(gen.fill(*args, param=param).tobytes()).hexdigest() == digest


def test_thread_count_independent():
    code = ("import sys, hashlib; sys.path.insert(0, %r); import gen; "
            "print(hashlib.sha256(gen.normal((300001,), 9, 1, 'bf16').tobytes()).hexdigest())"
            % os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    outs = set()
    for threads in ("1", "3", "8"):
        env = dict(os.environ, OMP_NUM_THREADS=threads)
        outs.add(subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                                text=True, check=True).stdout)
    assert len(outs) == 1


def test_offset_is_a_window():
    full = gen.normal((5000,), 4, 1, "f64")
    part = gen.fill((1000,), gen.DIST_NORMAL, 4, 1, "f64", offset=2500)
    assert np.array_equal(full[2500:3500], part)


def test_moments():
    u = gen.uniform_pm1((400000,), 1, 0, "f64")
    assert u.min() >= -1 and u.max() < 1 and abs(u.mean()) < 0.01 and abs(u.var() - 1 / 3) < 0.01
    z = gen.normal((400000,), 2, 0, "f64")
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1) < 0.01
    zk = gen.normal((400000,), 3, 0, "f64", divisor=128.0)
    assert abs(zk.var() * 16384 - 1) < 0.01
    r = gen.integers((100000,), 4, 0, 32, "f64")
    assert r.min() == -32 and r.max() == 32 and np.all(r == np.round(r))


def test_rounding_of_draws_is_single_rne():
    x = gen.normal((20000,), 6, 0, "f64")
    assert np.array_equal(gen.normal((20000,), 6, 0, "bf16"), gen.round_bf16(x))
    assert np.array_equal(gen.normal((20000,), 6, 0, "f16"), x.astype(np.float16).view(np.uint16))
    assert np.array_equal(gen.normal((20000,), 6, 0, "f32"), x.astype(np.float32))


@pytest.mark.parametrize("br,bc", [(1, 128), (128, 128)])
def test_block_quantiser(br, bc):
    rows, cols = 300, 400
    x = gen.normal((rows, cols), 7, 0, "f32")
    x[5, :] = 0.0                              # an all-zero 1x128 row slice
    q, s = gen.quant_e4m3fn(x, br, bc)
    assert s.shape == (-(-rows // br), -(-cols // bc))
    v = lib_decode("e4m3fn", q)
    assert np.all(np.abs(v) <= 448)
    grid = np.unique(np.abs(lib_decode("e4m3fn", np.arange(0, 0x7F, dtype=np.uint8))))
    for bi in range(s.shape[0]):
        for bj in range(s.shape[1]):
            blk = (slice(bi * br, (bi + 1) * br), slice(bj * bc, (bj + 1) * bc))
            xb, vb, sc = x[blk], v[blk], s[bi, bj]
            amax = np.max(np.abs(xb))
            if amax == 0:
                assert sc == 1.0 and np.all(vb == 0)
                continue
            assert sc == np.float32(amax) / np.float32(448.0)
            assert np.max(np.abs(vb)) == 448.0       # the block maximum lands on +-448
            y = np.clip(xb / sc, -448, 448).astype(np.float64)  # fp32 division, as specified
            # nearest e4m3 value (brute force over the grid), ties to even code
            d = np.abs(np.abs(y)[..., None] - grid[None, None, :])
            best = d.min(axis=-1)
            assert np.all(np.abs(np.abs(vb) - np.abs(y)) == best)
            assert np.all((vb == 0) | (np.sign(vb) == np.sign(y)))


def test_sample_rows():
    r = gen.sample_rows(4096, 256, 3)
    assert len(set(r.tolist())) == 256 and r.min() >= 0 and r.max() < 4096
    assert np.array_equal(r, gen.sample_rows(4096, 256, 3))
    assert not np.array_equal(r, gen.sample_rows(4096, 256, 5))


def test_workload_table():
    w = configs.WORKLOADS
    assert [w[k].seed for k in configs.ORDER] == [1, 2, 3, 4, 5]
    big = w["bf16_4096x7168x16384"]
    assert (big.M, big.N, big.K, big.b_layout) == (4096, 7168, 16384, "nk")
    assert big.compulsory_bytes == 427_819_008
    assert w["bf16_skinny_64x7168x7168"].compulsory_bytes == 104_595_456
    assert w["fp8_4096x7168x16384"].compulsory_bytes == 245_395_456
    small = configs.make_inputs(w["fp8_4096x7168x16384"], M=8, N=200, K=300)
    assert small["A"].shape == (8, 300) and small["B"].shape == (200, 300)
    assert small["SA"].shape == (8, 3) and small["SB"].shape == (2, 3)
