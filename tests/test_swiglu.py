"""The fused SwiGLU with an fp8 output (tg_gemm_f16_swiglu_quant_fp8 /
tg_gemm_bf16_swiglu_quant_fp8, through the C-ABI) against the oracle: the
fp64 gate and up products, h = silu(g) u in fp64 rounded once to fp32, then
quantised per 1 x 128 row slice.

Exact mode: positive integer inputs and gate weights with every gate value at
least 37, where 1 + e^-g is 1 in fp32 and in fp64, and |g u| < 2^24, so both
sides hold h = g u exactly and codes and scales must agree bit for bit (the
preconditions are asserted on the oracle's values).  Normal mode: seeded
N(0, 1) input and N(0, 1)/sqrt(K) weights (gate values about N(0, 1), the
curved part of silu); each scale and dequantised value must lie within the
bound that the products' fp32 accumulation error, carried through h, and half
an e4m3fn step allow.  The cases reach all three kernels, ragged edges, a grid of
more than one round of workgroups, padded code and scale strides behind guard
bytes, K = 0, weight rows closer than K apart, the 4096 x 16384 x 7168 shape on
sampled rows, the 64 x 16384 x 7168 decode shape in full, and the output fed
to tg_gemm_fp8_blockscaled as the down projection's A operand; the workspace
entry points' split plan on 2, 4 and 8 splits, workspace reuse and graph
capture.
"""
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
from tests.test_quant_out import assert_exact, assert_within_err, run_guarded

pytestmark = pytest.mark.gpu

GATE_MIN = 37   # e^-37 < 2^-53: 1 + e^-g rounds to 1 in fp64 (and in fp32)


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    return gpu_lib


def _encode(fmt, x):
    return gen.round_bf16(x) if fmt == "bf16" else gen.round_f16(x)


def _ints(shape, seed, stream, lo, hi, fmt):
    """Seeded integers on [lo, hi] as fp64 (folded from the generator's
    integers on [-64, 64])."""
    x = oracle.decode(fmt, gen.integers(shape, seed, stream, 64, fmt))
    return lo + np.mod(x + 64, hi - lo + 1)


def _operands(fmt, M, N, K, layout, seed, exact):
    """Logical x (M x K), gate and up weights (K x N) in a storage layout;
    returns (A, sam, sak, Bg, Bu, sbk, sbn) as codes."""
    if exact:
        # x in [1, 2], gate weights in [c, c + 1] with K c >= 37, up weights in
        # [-2, 2]: 37 <= g <= 2 K (c + 1) and |u| <= 4 K, so |g u| < 2^24 for
        # K <= 1024
        assert K <= 1024
        g_lo = max(1, -(-GATE_MIN // max(K, 1)))
        A = _ints((M, K), seed, 0, 1, 2, fmt)
        Bg = _ints((K, N), seed, 1, g_lo, g_lo + 1, fmt)
        Bu = _ints((K, N), seed, 4, -2, 2, fmt)
    else:
        div = math.sqrt(max(K, 1))
        A = oracle.decode(fmt, gen.normal((M, K), seed, 0, fmt))
        Bg = oracle.decode(fmt, gen.normal((K, N), seed, 1, fmt, divisor=div))
        Bu = oracle.decode(fmt, gen.normal((K, N), seed, 4, fmt, divisor=div))
    if layout == "nk":                       # weights stored N x K
        return (_encode(fmt, A), K, 1, _encode(fmt, Bg.T), _encode(fmt, Bu.T), 1, K)
    if layout == "kn":                       # weights stored K x N
        return (_encode(fmt, A), K, 1, _encode(fmt, Bg), _encode(fmt, Bu), N, 1)
    if layout == "padded":                   # leading dimensions padded by 24 elements
        pad = lambda x: np.pad(x, ((0, 0), (0, 24)))  # noqa: E731
        return (_encode(fmt, pad(A)), K + 24, 1, _encode(fmt, pad(Bg.T)), _encode(fmt, pad(Bu.T)),
                1, K + 24)
    raise ValueError(layout)


def _run(fmt, M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, sqm=None, ssm=None, ssj=1, ws=None):
    """Run the fused SwiGLU on device operands; returns (codes M x N,
    scales M x ceil(N/128), plan).  ws=True: the workspace entry point with a
    fresh zeroed workspace of the size its split plan asks for; ws=<Workspace>:
    with that one (its counters must be zero again afterwards)."""
    op = 1 if fmt == "bf16" else 0
    if ws is None:
        fn = tg.tg_gemm_bf16_swiglu_quant_fp8 if fmt == "bf16" else tg.tg_gemm_f16_swiglu_quant_fp8
    else:
        fn = (tg.tg_gemm_bf16_swiglu_quant_fp8_ws if fmt == "bf16"
              else tg.tg_gemm_f16_swiglu_quant_fp8_ws)
    box = [ws]

    def launch(Q, sqm, S, ssm, ssj):
        args = (M, N, K, A.data_ptr(), sam, sak, Bg.data_ptr(), Bu.data_ptr(), sbk, sbn, Q, sqm,
                S, ssm, ssj)
        st = torch.cuda.current_stream().cuda_stream
        if box[0] is None:
            plan = tg.tg_gemm_swiglu_quant_fp8_plan(op, *args)
            H.log(f"swiglu->fp8 {fmt} M={M} N={N} K={K} sqm={sqm} ssm={ssm} ssj={ssj} [{plan}]")
            fn(*args, st)
            return plan
        if box[0] is True:
            box[0] = H.Workspace(tg.tg_gemm_swiglu_quant_fp8_workspace_size(op, *args))
        w = box[0]
        plan = tg.tg_gemm_swiglu_quant_fp8_plan_ws(op, *args, w.nbytes)
        H.log(f"swiglu->fp8 ws {fmt} M={M} N={N} K={K} bytes={w.nbytes} [{plan}]")
        fn(*args, w.ptr, w.nbytes, st)
        return plan

    Q, S, plan = run_guarded(M, N, launch, sqm, ssm, ssj)
    if ws is not None:
        assert box[0].counters_zero(), "workspace counters left nonzero"
    return Q, S, plan


def _h_error(K, G, U, Sg, Su):
    """Bound on |h' - h| for the kernel's fp32 h' = g' u' / (1 + e^-g'):
    the products' accumulation errors eg = K 2^-24 S_g and eu = K 2^-24 S_u
    carried through h (|d silu / dg| <= 1.1 and |silu(g)| <= |g|), plus
    2^-19 |g'| |u'| for the four fp32 operations that form h' (exp within a
    few units in the last place, the product, the sum and the quotient)."""
    eg = K * 2.0 ** -24 * Sg
    eu = K * 2.0 ** -24 * Su
    return 1.1 * (np.abs(U) + eu) * eg + np.abs(G) * eu \
        + 2.0 ** -19 * (np.abs(G) + eg) * (np.abs(U) + eu)


def _check(fmt, M, N, K, layout, seed, want=None, ws=None, modes=(True, False)):
    for exact in modes:
        A, sam, sak, Bg, Bu, sbk, sbn = _operands(fmt, M, N, K, layout, seed, exact)
        Q, S, plan = _run(fmt, M, N, K, H.dev(A), sam, sak, H.dev(Bg), H.dev(Bu), sbk, sbn, ws=ws)
        if want:
            assert plan == want, plan
        Qo, So, Ho, G, U, Sg, Su = oracle.swiglu_quant_fp8(fmt, M, N, K, A, sam, sak, Bg, Bu, sbk,
                                                           sbn)
        what = f"{fmt} {M}x{N}x{K} {layout} {'integers' if exact else 'normal'} [{plan}]"
        if exact:
            assert K == 0 or G.min() >= GATE_MIN, "precondition: every gate value >= 37"
            assert np.abs(Ho).max() < 2.0 ** 24, "precondition: h exact in fp32"
            assert np.array_equal(Ho, G * U), "precondition: silu(g) = g"
            assert_exact(Q, S, Qo, So, what)
        else:
            assert_within_err(Q, S, Ho, _h_error(K, G, U, Sg, Su), what)


# (M, N, K, storage layout, expected plan)
CASES = [
    (300, 500, 256, "nk", "tile_nt_256x256_swiglu_q8"),
    (256, 256, 64, "nk", "tile_nt_256x256_swiglu_q8"),
    (33, 129, 8, "nk", "skinny_64x128_swiglu_q8"),
    (513, 392, 200, "nk", "tile_nt_256x256_swiglu_q8"),
    (65, 300, 136, "nk", "tile_nt_256x256_swiglu_q8"),
    (1, 1000, 520, "nk", "skinny_64x128_swiglu_q8"),
    (64, 600, 1000, "nk", "skinny_64x128_swiglu_q8"),
    (17, 300, 200, "nk", "skinny_64x128_swiglu_q8"),
    (64, 256, 64, "padded", "skinny_64x128_swiglu_q8"),
    (300, 256, 256, "padded", "tile_nt_256x256_swiglu_q8"),
    (100, 300, 100, "padded", "generic16_32x128_swiglu_q8"),
    (70, 200, 96, "kn", "generic16_32x128_swiglu_q8"),
    (1, 1, 1, "nk", "generic16_32x128_swiglu_q8"),
    (40, 130, 77, "nk", "generic16_32x128_swiglu_q8"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}-{c[3]}" for c in CASES])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_swiglu(fmt, case):
    M, N, K, layout, want = case
    _check(fmt, M, N, K, layout, 3100 + M + N + K, want)


def test_swiglu_decode_shape():
    """The gate and up projections of 64 decode rows, 64 x 16384 x 7168 (the
    skinny kernel: one workgroup per 128-column slice over all of K), every
    row, in the workload's normal recipe, within the bound."""
    M, N, K = 64, 16384, 7168
    d = configs.swiglu_inputs(M, N, K, 3700)
    Q, S, plan = _run("bf16", M, N, K, H.dev(d["A"]), K, 1, H.dev(d["Bg"]), H.dev(d["Bu"]), 1, K)
    assert plan == "skinny_64x128_swiglu_q8", plan
    _, _, Ho, G, U, Sg, Su = oracle.swiglu_quant_fp8("bf16", M, N, K, d["A"], K, 1, d["Bg"],
                                                     d["Bu"], 1, K)
    assert_within_err(Q, S, Ho, _h_error(K, G, U, Sg, Su), "decode shape, normal")


@pytest.mark.parametrize("M", [20, 200])
def test_swiglu_overlapping_weight_rows(M):
    """Weight rows 8 elements apart with K = 64 (legal: the weights are only
    read): the rows past N of the last 128-column slice then lie inside the
    buffer, and their products must still stay out of that slice's row
    maxima.  Integer inputs, bit for bit, on both the skinny and the tile
    kernel."""
    N, K, sbn = 200, 64, 8
    fmt = "bf16"
    g_lo = -(-GATE_MIN // K)
    A = _ints((M, K), 3800, 0, 1, 2, fmt)
    span = (N - 1) * sbn + K
    Bg = _ints((span,), 3800, 1, g_lo, g_lo + 1, fmt)
    Bu = _ints((span,), 3800, 4, -2, 2, fmt)
    A, Bg, Bu = _encode(fmt, A), _encode(fmt, Bg), _encode(fmt, Bu)
    Q, S, plan = _run(fmt, M, N, K, H.dev(A), K, 1, H.dev(Bg), H.dev(Bu), 1, sbn)
    assert plan == ("skinny_64x128_swiglu_q8" if M <= 64 else "tile_nt_256x256_swiglu_q8"), plan
    Qo, So, Ho, G, U, _, _ = oracle.swiglu_quant_fp8(fmt, M, N, K, A, K, 1, Bg, Bu, 1, sbn)
    assert G.min() >= GATE_MIN and np.abs(Ho).max() < 2.0 ** 24 and np.array_equal(Ho, G * U)
    assert_exact(Q, S, Qo, So, f"overlapping weight rows [{plan}]")


def test_swiglu_two_rounds():
    """288 workgroups: more than one per CU, so the second round walks K
    from the top down."""
    _check("bf16", 2100, 4000, 136, "nk", 3200, "tile_nt_256x256_swiglu_q8")


def test_swiglu_strides():
    """Codes with a padded row stride; scales row-major with a padded row
    stride, then column-major."""
    M, N, K = 290, 600, 136
    A, sam, sak, Bg, Bu, sbk, sbn = _operands("bf16", M, N, K, "nk", 3300, True)
    Qo, So, _, _, _, _, _ = oracle.swiglu_quant_fp8("bf16", M, N, K, A, sam, sak, Bg, Bu, sbk, sbn)
    Ad, Bgd, Bud = H.dev(A), H.dev(Bg), H.dev(Bu)
    nb = -(-N // 128)
    for sqm, ssm, ssj in ((N + 37, nb + 3, 1), (N + 8, 1, M + 5)):
        Q, S, plan = _run("bf16", M, N, K, Ad, sam, sak, Bgd, Bud, sbk, sbn, sqm=sqm, ssm=ssm,
                          ssj=ssj)
        assert plan == "tile_nt_256x256_swiglu_q8", plan
        assert_exact(Q, S, Qo, So, f"strides sqm={sqm} ssm={ssm} ssj={ssj} [{plan}]")


def test_swiglu_k0_and_zero_gate():
    """K = 0: both products vanish, so h = silu(0) 0 = 0 (scale 1, codes 0).
    A zero gate column gives h = silu(0) u = 0 whatever the up product; a zero
    up column gives 0 whatever the gate."""
    M, N = 70, 300
    Z = torch.zeros(1, dtype=torch.int16, device="cuda")
    Q, S, plan = _run("bf16", M, N, 0, Z, 0, 1, Z, Z, 1, 0)
    assert not Q.any() and np.all(S == 1.0), plan
    K = 64
    A, sam, sak, Bg, Bu, sbk, sbn = _operands("bf16", M, N, K, "nk", 3400, False)
    Bg, Bu = Bg.copy(), Bu.copy()
    Bg[::3] = 0                         # weights stored N x K: rows are output columns
    Bu[1::3] = 0
    Q, S, plan = _run("bf16", M, N, K, H.dev(A), sam, sak, H.dev(Bg), H.dev(Bu), sbk, sbn)
    assert plan == "tile_nt_256x256_swiglu_q8", plan
    assert np.all(oracle.decode("e4m3fn", Q[:, ::3]) == 0)    # +0 or -0 (sign of g u)
    assert np.all(oracle.decode("e4m3fn", Q[:, 1::3]) == 0)
    Qo, So, Ho, G, U, Sg, Su = oracle.swiglu_quant_fp8("bf16", M, N, K, A, sam, sak, Bg, Bu, sbk,
                                                       sbn)
    assert_within_err(Q, S, Ho, _h_error(K, G, U, Sg, Su), "zero gate and up columns")


def test_swiglu_full_shape():
    """The gate and up projections 4096 x 16384 x 7168 on sampled rows, in the
    workload's normal recipe, within the bound."""
    w = configs.SWIGLU
    M, N, K = w["M"], w["N"], w["K"]
    d = configs.swiglu_inputs(M, N, K, w["seed"])
    rows = gen.sample_rows(M, 96, w["seed"])
    Q, S, plan = _run("bf16", M, N, K, H.dev(d["A"]), K, 1, H.dev(d["Bg"]), H.dev(d["Bu"]), 1, K)
    assert plan == "tile_nt_256x256_swiglu_q8", plan
    _, _, Ho, G, U, Sg, Su = oracle.swiglu_quant_fp8("bf16", M, N, K, d["A"], K, 1, d["Bg"],
                                                     d["Bu"], 1, K, rows=rows)
    assert_within_err(Q[rows], S[rows], Ho, _h_error(K, G, U, Sg, Su), "full shape, normal")
    del d
    torch.cuda.empty_cache()


def test_swiglu_feeds_down_projection():
    """h's codes and 1 x 128 scales are the A operand of the block-scaled down
    projection: C = h W_down on the GPU, within the bound of the oracle's
    block-scaled product of the oracle's own codes and scales."""
    M, N, K = 300, 512, 256
    A, sam, sak, Bg, Bu, sbk, sbn = _operands("bf16", M, N, K, "nk", 3500, True)
    Q, S, plan = _run("bf16", M, N, K, H.dev(A), sam, sak, H.dev(Bg), H.dev(Bu), sbk, sbn)
    Qo, So, _, _, _, _, _ = oracle.swiglu_quant_fp8("bf16", M, N, K, A, sam, sak, Bg, Bu, sbk, sbn)
    assert_exact(Q, S, Qo, So, "SwiGLU")
    N2, K2 = 260, N
    Q2, S2 = oracle.quant_fp8(gen.normal((N2, K2), 3501, 0, "f32"), 128)
    nkb = S.shape[1]
    c, plan2 = H.run_fp8(M, N2, K2, H.dev(Q), K2, 1, H.dev(S), nkb, 1, H.dev(Q2), 1, K2,
                         H.dev(S2), nkb, 1)
    C_ref, Sb = oracle.gemm_fp8_blockscaled(M, N2, K2, Qo, K2, 1, So, nkb, 1, Q2, 1, K2, S2, nkb, 1)
    H.assert_within_bound("bf16", c, C_ref, Sb, f"down projection [{plan} -> {plan2}]")


@pytest.mark.parametrize("M", [300, 48])
def test_swiglu_graph_capture(M):
    """The fused SwiGLU allocates nothing, so it can be captured: a graph
    replayed several times with eager work in between gives the eager codes
    and scales bit for bit (the tile kernel, and the decode-sized one)."""
    N, K = 512, 256
    A, sam, sak, Bg, Bu, sbk, sbn = _operands("bf16", M, N, K, "nk", 3600, False)
    Ad, Bgd, Bud = H.dev(A), H.dev(Bg), H.dev(Bu)
    nb = -(-N // 128)
    Q = torch.zeros((M, N), dtype=torch.uint8, device="cuda")
    S = torch.zeros((M, nb), dtype=torch.float32, device="cuda")
    args = lambda q, s: (M, N, K, Ad.data_ptr(), sam, sak, Bgd.data_ptr(), Bud.data_ptr(),  # noqa
                         sbk, sbn, q.data_ptr(), N, s.data_ptr(), nb, 1)
    stream = torch.cuda.Stream()
    plan = tg.tg_gemm_swiglu_quant_fp8_plan(1, *args(Q, S))
    assert plan == ("skinny_64x128_swiglu_q8" if M <= 64 else "tile_nt_256x256_swiglu_q8"), plan
    H.log(f"swiglu graph capture M={M} N={N} K={K} [{plan}]")
    with torch.cuda.stream(stream):
        tg.tg_gemm_bf16_swiglu_quant_fp8(*args(Q, S), stream.cuda_stream)
    stream.synchronize()
    Qe, Se = Q.clone(), S.clone()
    Qg = torch.zeros_like(Q)
    Sg = torch.zeros_like(S)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        tg.tg_gemm_bf16_swiglu_quant_fp8(*args(Qg, Sg), stream.cuda_stream)
    for rep in range(3):
        Qg.fill_(0x5A)
        Sg.fill_(-7.0)
        _run("bf16", min(M, 40), 200, 96, Ad, K, 1, Bgd, Bud, 1, K)  # eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Qg, Qe) and torch.equal(Sg.view(torch.int32), Se.view(torch.int32)), rep


# The skinny kernel's split plan (the workspace entry points): K slices of
# each output slice split over workgroups, the g and u partial sums added in
# split order before the activation.  (M, N, K, layout, splits, modes): 2
# splits with a ragged last output slice; a ragged last K slice in the last
# split; one row, one column past the first slice, padded strides; 4 and 8
# splits (normal inputs only: the exact recipe needs K <= 1024).
SPLIT_CASES = [
    (64, 300, 1024, "nk", 2, (True, False)),
    (33, 1000, 1000, "nk", 2, (True, False)),
    (1, 129, 1024, "padded", 2, (True, False)),
    (64, 7168, 2048, "nk", 4, (False,)),
    (48, 256, 16384, "nk", 8, (False,)),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}-{c[3]}" for c in SPLIT_CASES])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_swiglu_split(fmt, case):
    M, N, K, layout, splits, modes = case
    _check(fmt, M, N, K, layout, 3900 + M + N + K, f"skinny_64x128_swiglu_q8_splitk{splits}",
           ws=True, modes=modes)


def test_swiglu_split_decode_shape():
    """The 64 x 16384 x 7168 decode shape with a workspace (K split 2 ways,
    256 workgroups), every row, within the bound."""
    M, N, K = 64, 16384, 7168
    d = configs.swiglu_inputs(M, N, K, 3710)
    Q, S, plan = _run("bf16", M, N, K, H.dev(d["A"]), K, 1, H.dev(d["Bg"]), H.dev(d["Bu"]), 1, K,
                      ws=True)
    assert plan == "skinny_64x128_swiglu_q8_splitk2", plan
    _, _, Ho, G, U, Sg, Su = oracle.swiglu_quant_fp8("bf16", M, N, K, d["A"], K, 1, d["Bg"],
                                                     d["Bu"], 1, K)
    assert_within_err(Q, S, Ho, _h_error(K, G, U, Sg, Su), "decode shape, split, normal")


def test_swiglu_split_workspace_reuse():
    """One workspace through three calls in a row: 2 splits over 56 output
    slices, then 2 over 3 (a smaller call), then the first again; integer
    inputs, bit for bit against the oracle, counters zero after each."""
    fmt = "bf16"
    big, small = (64, 7168, 1024), (40, 300, 1024)
    ws = None
    for i, (M, N, K) in enumerate((big, small, big)):
        A, sam, sak, Bg, Bu, sbk, sbn = _operands(fmt, M, N, K, "nk", 4000 + i, True)
        if ws is None:
            nb = -(-N // 128)
            ws = H.Workspace(tg.tg_gemm_swiglu_quant_fp8_workspace_size(
                1, M, N, K, 0x100, sam, sak, 0x200, 0x300, sbk, sbn, 0x400, N, 0x500, nb, 1))
            assert ws.nbytes == 16384 + 56 * 2 * 64 * 1024
        Q, S, plan = _run(fmt, M, N, K, H.dev(A), sam, sak, H.dev(Bg), H.dev(Bu), sbk, sbn, ws=ws)
        assert plan.startswith("skinny_64x128_swiglu_q8_splitk"), plan
        Qo, So, Ho, G, U, _, _ = oracle.swiglu_quant_fp8(fmt, M, N, K, A, sam, sak, Bg, Bu, sbk,
                                                         sbn)
        assert G.min() >= GATE_MIN and np.abs(Ho).max() < 2.0 ** 24 and np.array_equal(Ho, G * U)
        assert_exact(Q, S, Qo, So, f"workspace reuse {i} [{plan}]")


def test_swiglu_split_graph_capture():
    """The split plan under graph capture: the kernel clears its own counters,
    so replays (with eager calls on the same workspace in between) give the
    eager codes and scales bit for bit."""
    M, N, K = 48, 512, 2048
    A, sam, sak, Bg, Bu, sbk, sbn = _operands("bf16", M, N, K, "nk", 4100, False)
    Ad, Bgd, Bud = H.dev(A), H.dev(Bg), H.dev(Bu)
    nb = -(-N // 128)
    Q = torch.zeros((M, N), dtype=torch.uint8, device="cuda")
    S = torch.zeros((M, nb), dtype=torch.float32, device="cuda")
    args = lambda q, s: (M, N, K, Ad.data_ptr(), sam, sak, Bgd.data_ptr(), Bud.data_ptr(),  # noqa
                         sbk, sbn, q.data_ptr(), N, s.data_ptr(), nb, 1)
    ws = H.Workspace(tg.tg_gemm_swiglu_quant_fp8_workspace_size(1, *args(Q, S)))
    plan = tg.tg_gemm_swiglu_quant_fp8_plan_ws(1, *args(Q, S), ws.nbytes)
    assert plan == "skinny_64x128_swiglu_q8_splitk4", plan
    H.log(f"swiglu split graph capture M={M} N={N} K={K} [{plan}]")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        tg.tg_gemm_bf16_swiglu_quant_fp8_ws(*args(Q, S), ws.ptr, ws.nbytes, stream.cuda_stream)
    stream.synchronize()
    Qe, Se = Q.clone(), S.clone()
    Qg, Sg = torch.zeros_like(Q), torch.zeros_like(S)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        tg.tg_gemm_bf16_swiglu_quant_fp8_ws(*args(Qg, Sg), ws.ptr, ws.nbytes, stream.cuda_stream)
    for rep in range(3):
        Qg.fill_(0x5A)
        Sg.fill_(-7.0)
        _run("bf16", M, N, K, Ad, sam, sak, Bgd, Bud, sbk, sbn, ws=ws)  # eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert ws.counters_zero(), rep
        assert torch.equal(Qg, Qe) and torch.equal(Sg.view(torch.int32), Se.view(torch.int32)), rep
