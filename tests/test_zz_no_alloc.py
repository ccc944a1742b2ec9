"""The fixed-scratch entry point tg_gemm_bf16_static_scratch (no allocation:
its split plans use the library's own device array) against the workspace
entry point tg_gemm_bf16_ws it varies: the same plan and the same bits, on
two calls in a row with the second smaller, for the skinny split plan and
the split-K tile plan; on integer inputs also bit-exact against the oracle."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import gen
import oracle
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

STATIC_BYTES = 64 << 20


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    return gpu_lib


def _static(M, N, K, A, B):
    """tg_gemm_bf16_static_scratch on device codes A (M x K), B (N x K);
    returns (C codes, plan)."""
    buf, off, scm = H.alloc_c(M, N)
    args = (M, N, K, A.data_ptr(), K, 1, B.data_ptr(), 1, K, buf.data_ptr() + 2 * off, scm, 1)
    plan = H.tg.tg_gemm_plan_ws(H.tg.OP_BF16, *args, STATIC_BYTES)
    H.tg.tg_gemm_bf16_static_scratch(*args, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    H.check_guards(buf, off, M, N, scm)
    return H.c_view(buf, off, M, N, scm), plan


# (first call, second smaller call, split plan of each)
CASES = [
    ((64, 7168, 7168), (64, 2048, 4096), ("skinny_64x128_splitk4", "skinny_64x128_splitk8")),
    ((4096, 896, 16384), (1024, 1024, 4096), ("tile_nt_256x224_splitk4",
                                              "tile_nt_128x128_splitk4")),
]


@pytest.mark.parametrize("case", CASES, ids=["skinny", "tile_split_k"])
def test_static_scratch_matches_workspace_entry(case):
    for (M, N, K), want in zip(case[:2], case[2]):
        seed = 3000 + M + N + K
        a = gen.normal((M, K), seed, 0, "bf16", divisor=math.sqrt(K))
        b = gen.normal((N, K), seed, 1, "bf16", divisor=math.sqrt(K))
        A, B = H.dev(a), H.dev(b)
        H.log(f"static scratch {M}x{N}x{K}")
        c_static, plan = _static(M, N, K, A, B)
        assert plan == want, plan
        c_ws, plan_ws = H.run16("bf16", M, N, K, A, K, 1, B, 1, K, ws=True)
        assert plan_ws == want, plan_ws
        assert np.array_equal(c_static, c_ws), f"static scratch differs from workspace {M}x{N}x{K}"
        rows = None if M <= 1024 else gen.sample_rows(M, 128, seed)
        C_ref, S = oracle.gemm("bf16", M, N, K, a, K, 1, b, 1, K, rows=rows)
        H.assert_within_bound("bf16", c_static if rows is None else c_static[rows], C_ref, S,
                              f"static {M}x{N}x{K} [{plan}]")
        # integer inputs: every fp32 partial sum exact, so bit-exact
        r = int(math.sqrt(2 ** 24 / K))
        ai, bi = gen.integers((M, K), seed, 0, r, "bf16"), gen.integers((N, K), seed, 1, r, "bf16")
        c_int, _ = _static(M, N, K, H.dev(ai), H.dev(bi))
        C_ref, _ = oracle.gemm("bf16", M, N, K, ai, K, 1, bi, 1, K, rows=rows)
        H.assert_bit_exact("bf16", c_int if rows is None else c_int[rows], C_ref,
                           f"static int {M}x{N}x{K}")


def test_static_scratch_rejects_and_noops():
    """A split plan larger than the array: TG_ERR_SCRATCH_LIMIT and C
    untouched; an empty call is a no-op; an unsplit call runs as
    tg_gemm_bf16."""
    M, N, K = 4096, 4896, 4096
    A = torch.zeros((M, K), dtype=torch.int16, device="cuda")
    B = torch.zeros((N, K), dtype=torch.int16, device="cuda")
    C = torch.full((M, N), 0x7BAD, dtype=torch.int16, device="cuda")
    st = H.tg.load().tg_gemm_bf16_static_scratch(M, N, K, A.data_ptr(), K, 1, B.data_ptr(), 1, K,
                                                 C.data_ptr(), N, 1, None)
    assert st == H.tg.TG_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert bool(torch.all(C == 0x7BAD).item())
    assert H.tg.load().tg_gemm_bf16_static_scratch(0, N, K, A.data_ptr(), K, 1, B.data_ptr(), 1,
                                                   K, C.data_ptr(), N, 1, None) == 0
    Mh, Nh, Kh = 512, 7168, 1024
    a = gen.integers((Mh, Kh), 5, 0, 64, "bf16")
    b = gen.integers((Nh, Kh), 5, 1, 64, "bf16")
    c, plan = _static(Mh, Nh, Kh, H.dev(a), H.dev(b))
    c_plain, plan_plain = H.run16("bf16", Mh, Nh, Kh, H.dev(a), Kh, 1, H.dev(b), 1, Kh)
    assert plan == plan_plain and np.array_equal(c, c_plain), (plan, plan_plain)
