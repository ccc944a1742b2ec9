"""The grouped product on the GPU (tg_gemm_grouped_f16 / _bf16, through the
C-ABI) against the CPU oracle applied group by group: bit-exact on integer
inputs, within the bound otherwise.  Uneven and empty groups, ragged row
counts, N and K, the group-by-group path for operands the one-launch kernel
does not take, and the benchmark's 8-expert workload on sampled rows."""
from __future__ import annotations

import math

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


def _inputs(fmt, rows, G, N, K, seed, int_r=None, lda=None, ldb=None):
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    draw = (lambda shape, stream: gen.integers(shape, seed, stream, int_r, fmt)) if int_r \
        else (lambda shape, stream: gen.normal(shape, seed, stream, fmt, divisor=math.sqrt(K)))
    A = np.zeros((rows, lda), np.uint16)
    A[:, :K] = draw((rows, K), 0)
    B = np.zeros((G, N, ldb), np.uint16)
    B[:, :, :K] = draw((G, N, K), 1)
    return A, B


def _run(fmt, offsets, N, K, A, B, lda, ldb):
    G = len(offsets) - 1
    rows = int(offsets[-1])
    Ad, Bd = H.dev(A), H.dev(B)
    buf = torch.full((rows * N + 64,), 0x7E01, dtype=torch.int16, device="cuda")
    args = (G, offsets, N, K, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, N * ldb, buf.data_ptr(), N)
    plan = tg.tg_gemm_grouped_plan(*args)
    fn = tg.tg_gemm_grouped_bf16 if fmt == "bf16" else tg.tg_gemm_grouped_f16
    H.log(f"grouped {fmt} G={G} rows={rows} N={N} K={K} lda={lda} ldb={ldb} [{plan}]")
    fn(*args, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    out = buf.cpu().numpy().view(np.uint16)
    assert np.all(out[rows * N:] == 0x7E01), "written past C"
    return out[:rows * N].reshape(rows, N), plan


def _ref(fmt, offsets, N, K, A, B, lda, ldb, rows=None):
    """The oracle product of each group, stacked (rows: a subset of C's rows)."""
    want = range(int(offsets[-1])) if rows is None else rows
    C = np.zeros((len(want), N))
    S = np.zeros((len(want), N))
    for g in range(len(offsets) - 1):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        sel = [(t, r) for t, r in enumerate(want) if lo <= r < hi]
        if not sel:
            continue
        local = np.array([r - lo for _, r in sel], np.int64)
        Cg, Sg = oracle.gemm(fmt, hi - lo, N, K, A[lo:hi], lda, 1, B[g], 1, ldb, rows=local)
        idx = [t for t, _ in sel]
        C[idx], S[idx] = Cg, Sg
    return C, S


CASES = [
    ([0, 300], 200, 136),                          # one group
    ([0, 100, 100, 357, 600, 601], 250, 64),       # an empty group, tiny and ragged groups
    ([0, 256, 512, 768], 224, 72),                 # tile-aligned groups
    ([0, 37, 400, 401, 1100], 129, 1000),          # ragged everything
    # more than one wave of tiles (330 and 385 of 256 x 224)
    ([0, 5000, 9000, 16700], 1024, 1032),
    ([0, 3000, 3001, 9000, 16700], 1000, 2056),
]


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("case", CASES, ids=[f"{len(c[0]) - 1}g_{c[1]}x{c[2]}" for c in CASES])
def test_grouped(fmt, case):
    offsets, N, K = case
    offsets = np.array(offsets, np.int64)
    G, rows = len(offsets) - 1, int(offsets[-1])
    A, B = _inputs(fmt, rows, G, N, K, 20 + N + K)
    c, plan = _run(fmt, offsets, N, K, A, B, K, K)
    assert plan.startswith("grouped_tile_nt"), plan
    C_ref, S = _ref(fmt, offsets, N, K, A, B, K, K)
    H.assert_within_bound(fmt, c, C_ref, S, f"grouped {fmt} [{plan}]")
    r = max(1, min(64 if fmt == "bf16" else 16, int(math.sqrt(2 ** 24 / K))))
    A, B = _inputs(fmt, rows, G, N, K, 30 + N + K, int_r=r)
    c, _ = _run(fmt, offsets, N, K, A, B, K, K)
    C_ref, _ = _ref(fmt, offsets, N, K, A, B, K, K)
    H.assert_bit_exact(fmt, c, C_ref, f"grouped {fmt} int [{plan}]")


def test_grouped_per_group_path():
    """Leading dimensions the one-launch kernel does not take (not multiples
    of 8) run group by group, with the same results."""
    offsets = np.array([0, 70, 70, 300], np.int64)
    N, K = 90, 100
    A, B = _inputs("bf16", 300, 3, N, K, 9, int_r=16, lda=101, ldb=103)
    c, plan = _run("bf16", offsets, N, K, A, B, 101, 103)
    assert plan == "per_group", plan
    C_ref, _ = _ref("bf16", offsets, N, K, A, B, 101, 103)
    H.assert_bit_exact("bf16", c, C_ref, "grouped per-group path")


def test_grouped_workload_sampled():
    """The benchmark's 8-expert product at full size, on 256 seeded rows and
    rows of the last group: within the bound on N(0,1)/sqrt(K) inputs,
    bit-exact on integers."""
    w = configs.GROUPED
    sizes = configs.group_sizes(w["rows"], w["G"], w["seed"])
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    N, K = w["N"], w["K"]
    rows = np.union1d(gen.sample_rows(w["rows"], 256, w["seed"]),
                      np.arange(offsets[-2], offsets[-1], 29))
    A, B = _inputs("bf16", w["rows"], w["G"], N, K, w["seed"])
    c, plan = _run("bf16", offsets, N, K, A, B, K, K)
    assert plan == "grouped_tile_nt_256x224", plan
    C_ref, S = _ref("bf16", offsets, N, K, A, B, K, K, rows=rows)
    H.assert_within_bound("bf16", c[rows], C_ref, S, f"grouped workload [{plan}]")
    A, B = _inputs("bf16", w["rows"], w["G"], N, K, w["seed"], int_r=48)
    c, _ = _run("bf16", offsets, N, K, A, B, K, K)
    C_ref, _ = _ref("bf16", offsets, N, K, A, B, K, K, rows=rows)
    H.assert_bit_exact("bf16", c[rows], C_ref, "grouped workload int")


# ------------------------------------------------------------------ fp8

def _fp8_inputs(rows, G, N, K, seed, int_r=None):
    """e4m3fn codes and fp32 scales: A (rows x K) with 1 x 128 row scales,
    B (G x N x K) with 128 x 128 block scales per group (SB stacked G x
    ceil(N/128) x ceil(K/128)).  int_r: integer codes and unit scales."""
    nkb, nnb = -(-K // 128), -(-N // 128)
    if int_r:
        qa = gen.round_e4m3fn(gen.integers((rows, K), seed, 0, int_r, "f32"))
        qb = gen.round_e4m3fn(gen.integers((G, N, K), seed, 1, int_r, "f32"))
        return qa, np.ones((rows, nkb), np.float32), qb, np.ones((G, nnb, nkb), np.float32)
    qa, sa = gen.quant_e4m3fn(gen.normal((rows, K), seed, 0, "f32"), 1, 128)
    xb = gen.normal((G * N, K), seed, 1, "f32").reshape(G, N, K)
    qb = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, nnb, nkb), np.float32)
    for g in range(G):
        qb[g], sb[g] = gen.quant_e4m3fn(xb[g], 128, 128)
    return qa, sa, qb, sb


def _run_fp8(offsets, N, K, qa, sa, qb, sb):
    G = len(offsets) - 1
    rows = int(offsets[-1])
    nkb, nnb = sa.shape[1], sb.shape[1]
    d = [H.dev(x) for x in (qa, sa, qb, sb)]
    buf = torch.full((rows * N + 64,), 0x7E01, dtype=torch.int16, device="cuda")
    args = (G, offsets, N, K, d[0].data_ptr(), K, d[1].data_ptr(), nkb, 1, d[2].data_ptr(), K,
            N * K, d[3].data_ptr(), nkb, 1, nnb * nkb, buf.data_ptr(), N)
    plan = tg.tg_gemm_grouped_fp8_plan(*args)
    H.log(f"grouped fp8 G={G} rows={rows} N={N} K={K} [{plan}]")
    tg.tg_gemm_grouped_fp8_blockscaled(*args, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    out = buf.cpu().numpy().view(np.uint16)
    assert np.all(out[rows * N:] == 0x7E01), "written past C"
    return out[:rows * N].reshape(rows, N), plan


def _ref_fp8(offsets, N, K, qa, sa, qb, sb, rows=None):
    want = range(int(offsets[-1])) if rows is None else rows
    nkb = sa.shape[1]
    C = np.zeros((len(want), N))
    S = np.zeros((len(want), N))
    for g in range(len(offsets) - 1):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        sel = [(t, r) for t, r in enumerate(want) if lo <= r < hi]
        if not sel:
            continue
        local = np.array([r - lo for _, r in sel], np.int64)
        Cg, Sg = oracle.gemm_fp8_blockscaled(hi - lo, N, K, qa[lo:hi], K, 1, sa[lo:hi], nkb, 1,
                                             qb[g], 1, K, sb[g], nkb, 1, rows=local)
        idx = [t for t, _ in sel]
        C[idx], S[idx] = Cg, Sg
    return C, S


FP8_CASES = [([0, 300], 200, 1024), ([0, 100, 100, 357, 600], 250, 384),
             ([0, 1, 257, 700], 129, 272)]


@pytest.mark.parametrize("case", FP8_CASES, ids=[f"{len(c[0]) - 1}g_{c[1]}x{c[2]}" for c in FP8_CASES])
def test_grouped_fp8(case):
    offsets, N, K = case
    offsets = np.array(offsets, np.int64)
    G, rows = len(offsets) - 1, int(offsets[-1])
    x = _fp8_inputs(rows, G, N, K, 40 + N + K)
    c, plan = _run_fp8(offsets, N, K, *x)
    assert plan == "grouped_tile_fp8_256x128", plan
    C_ref, S = _ref_fp8(offsets, N, K, *x)
    H.assert_within_bound("bf16", c, C_ref, S, f"grouped fp8 [{plan}]")
    x = _fp8_inputs(rows, G, N, K, 50 + N + K, int_r=16)
    c, _ = _run_fp8(offsets, N, K, *x)
    C_ref, _ = _ref_fp8(offsets, N, K, *x)
    H.assert_bit_exact("bf16", c, C_ref, "grouped fp8 int")


def test_grouped_fp8_workload_sampled():
    """The 8-expert shape (8192 x 4096 x 7168 in all) in fp8, 256 seeded rows."""
    w = configs.GROUPED
    sizes = configs.group_sizes(w["rows"], w["G"], w["seed"])
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    N, K = w["N"], w["K"]
    rows = gen.sample_rows(w["rows"], 256, w["seed"])
    x = _fp8_inputs(w["rows"], w["G"], N, K, w["seed"])
    c, plan = _run_fp8(offsets, N, K, *x)
    assert plan == "grouped_tile_fp8_256x256", plan
    C_ref, S = _ref_fp8(offsets, N, K, *x, rows=rows)
    H.assert_within_bound("bf16", c[rows], C_ref, S, f"grouped fp8 workload [{plan}]")
    x = _fp8_inputs(w["rows"], w["G"], N, K, w["seed"], int_r=16)
    c, _ = _run_fp8(offsets, N, K, *x)
    C_ref, _ = _ref_fp8(offsets, N, K, *x, rows=rows)
    H.assert_bit_exact("bf16", c[rows], C_ref, "grouped fp8 workload int")
