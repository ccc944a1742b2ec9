"""The C-ABI boundary on the CPU: the library loads, exports every function
include/tg_gemm.h declares, and rejects invalid arguments on the host before
any HIP call (so no GPU is needed here).  Valid calls are never made on the
CPU; the parity tests make them on the GPU."""
import ctypes
import os
import re

import pytest

import dense_tiled_gemm_03_amd as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tg_gemm.h")

# Distinct fake device addresses: validation must reject before touching them.
PA, PB, PC, PS = 0x10000, 0x20000, 0x30000, 0x40000


@pytest.fixture(scope="module")
def lib():
    return tg.ensure_built()


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(tg_\w+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(tg.EXPORTS)
    for name in names:
        assert hasattr(lib, name), f"{name} not exported"
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    for code, tag in ((0, "TG_SUCCESS"), (1, "TG_ERR_INVALID_VALUE"), (2, "TG_ERR_UNSUPPORTED"),
                      (3, "TG_ERR_LAUNCH"), (4, "TG_ERR_SCRATCH_LIMIT")):
        assert tg.tg_status_string(code).startswith(tag)
    assert "unknown" in tg.tg_status_string(99)


def _call16(fn, M=8, N=8, K=8, A=PA, sam=8, sak=1, B=PB, sbk=8, sbn=1, C=PC, scm=8, scn=1):
    return fn(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, None)


INVALID16 = [
    dict(M=-1), dict(N=-2), dict(K=-3),
    dict(sam=-1), dict(sak=-1), dict(sbk=-1), dict(sbn=-1), dict(scm=-1), dict(scn=-1),
    dict(A=0), dict(B=0), dict(C=0),
    dict(scm=7),                                   # rows of C overlap
    dict(M=2, sam=1 << 62, K=8, sak=1 << 62),      # A extent overflows int64
    dict(N=3, sbn=1 << 62),                        # B extent overflows
    dict(M=1 << 40, scm=1 << 40),                  # C extent overflows
]


@pytest.mark.parametrize("kw", INVALID16, ids=[str(k) for k in INVALID16])
@pytest.mark.parametrize("name", ["tg_gemm_f16", "tg_gemm_bf16"])
def test_invalid_16bit(lib, name, kw):
    assert _call16(getattr(lib, name), **kw) == tg.TG_ERR_INVALID_VALUE


@pytest.mark.parametrize("kw", [dict(scn=2), dict(scn=0), dict(M=1 << 31, scm=8),
                                dict(K=1 << 31, sak=1, sbk=8)])
def test_unsupported_16bit(lib, kw):
    assert _call16(lib.tg_gemm_bf16, **kw) == tg.TG_ERR_UNSUPPORTED


def test_empty_calls_are_noops(lib):
    # M == 0 or N == 0: success without any HIP call (pointers may be NULL)
    for kw in (dict(M=0), dict(N=0), dict(M=0, A=0, B=0, C=0), dict(N=0, C=0, scm=0)):
        assert _call16(lib.tg_gemm_bf16, **kw) == tg.TG_SUCCESS
        assert _call16(lib.tg_gemm_f16, **kw) == tg.TG_SUCCESS


def test_k_zero_needs_no_operands(lib):
    # K == 0 only writes C, so NULL A/B pass validation (checked via the plan)
    assert tg.tg_gemm_plan(tg.OP_BF16, 8, 8, 0, 0, 0, 0, 0, 0, 0, PC, 8, 1) is not None
    assert tg.tg_gemm_plan(tg.OP_BF16, 8, 8, 0, 0, 0, 0, 0, 0, 0, 0, 8, 1) is None


def _call8(lib, M=8, N=8, K=256, A=PA, sam=256, sak=1, SA=PS, ssam=2, ssak=1, B=PB, sbk=1,
           sbn=256, SB=PS, ssbn=2, ssbk=1, C=PC, scm=8, scn=1):
    return lib.tg_gemm_fp8_blockscaled(M, N, K, A, sam, sak, SA, ssam, ssak, B, sbk, sbn, SB,
                                       ssbn, ssbk, C, scm, scn, None)


INVALID8 = [dict(M=-1), dict(K=-1), dict(ssam=-1), dict(ssak=-1), dict(ssbn=-1), dict(ssbk=-1),
            dict(SA=0), dict(SB=0), dict(A=0), dict(B=0), dict(C=0), dict(scm=3),
            dict(M=3, ssam=1 << 62)]


@pytest.mark.parametrize("kw", INVALID8, ids=[str(k) for k in INVALID8])
def test_invalid_fp8(lib, kw):
    assert _call8(lib, **kw) == tg.TG_ERR_INVALID_VALUE


def test_fp8_unsupported_and_noop(lib):
    assert _call8(lib, scn=4) == tg.TG_ERR_UNSUPPORTED
    assert _call8(lib, M=0, SA=0, SB=0, A=0, B=0, C=0) == tg.TG_SUCCESS


def _callq(lib, name, **kw):
    a = dict(R=8, K=300, X=PA, ldx=300, Q=PB, ldq=300, S=PS, ssr=3, ssk=1)
    a.update(kw)
    return getattr(lib, name)(a["R"], a["K"], a["X"], a["ldx"], a["Q"], a["ldq"], a["S"],
                              a["ssr"], a["ssk"], None)


INVALIDQ = [dict(R=-1), dict(K=-1), dict(ldx=-1), dict(ssk=-1), dict(X=0), dict(Q=0), dict(S=0),
            dict(ldx=299), dict(ldq=299), dict(ssk=0), dict(R=300, ssr=0),
            dict(R=1 << 62, ldx=1 << 20)]


@pytest.mark.parametrize("kw", INVALIDQ, ids=[str(k) for k in INVALIDQ])
@pytest.mark.parametrize("name", ["tg_quant_fp8_1x128", "tg_quant_fp8_128x128"])
def test_quant_invalid(lib, name, kw):
    assert _callq(lib, name, **kw) == tg.TG_ERR_INVALID_VALUE


@pytest.mark.parametrize("name", ["tg_quant_fp8_1x128", "tg_quant_fp8_128x128"])
def test_quant_noop(lib, name):
    assert _callq(lib, name, R=0, X=0, Q=0, S=0) == tg.TG_SUCCESS
    assert _callq(lib, name, K=0, X=0, Q=0, S=0) == tg.TG_SUCCESS


def _callqo(lib, name, **kw):
    a = dict(M=8, N=300, K=64, A=PA, sam=64, sak=1, B=PB, sbk=1, sbn=64, Q=PC, sqm=300, S=PS,
             ssm=3, ssj=1)
    a.update(kw)
    args = [a[k] for k in ("M", "N", "K", "A", "sam", "sak", "B", "sbk", "sbn", "Q", "sqm", "S",
                           "ssm", "ssj")]
    if name == "plan":
        return lib.tg_gemm_quant_fp8_plan(a.get("op", 1), *args)
    return getattr(lib, name)(*args, None)


INVALIDQO = [dict(M=-1), dict(N=-1), dict(K=-1), dict(sam=-1), dict(sbn=-1), dict(sqm=-1),
             dict(ssm=-1), dict(ssj=-1), dict(A=0), dict(B=0), dict(Q=0), dict(S=0),
             dict(sqm=299),                        # rows of the codes overlap
             dict(ssj=0),                          # three slices in one place
             dict(ssm=0),                          # eight rows' scales in one place
             dict(M=2, ssm=1 << 62),               # scale range overflows
             dict(M=1 << 40, sqm=1 << 40)]         # code range overflows


@pytest.mark.parametrize("kw", INVALIDQO, ids=[str(k) for k in INVALIDQO])
@pytest.mark.parametrize("name", ["tg_gemm_f16_quant_fp8", "tg_gemm_bf16_quant_fp8", "plan"])
def test_quant_out_invalid(lib, name, kw):
    r = _callqo(lib, name, **kw)
    assert (r is None) if name == "plan" else (r == tg.TG_ERR_INVALID_VALUE)


def test_quant_out_noop_and_plans(lib):
    assert _callqo(lib, "tg_gemm_bf16_quant_fp8", M=0, A=0, B=0, Q=0, S=0) == tg.TG_SUCCESS
    assert _callqo(lib, "tg_gemm_bf16_quant_fp8", N=0, A=0, B=0, Q=0, S=0) == tg.TG_SUCCESS
    base = dict(op=1, M=8, N=300, K=64, A=PA, sam=64, sak=1, B=PB, sbk=1, sbn=64, Q=PC, sqm=300,
                S=PS, ssm=3, ssj=1)
    order = ("op", "M", "N", "K", "A", "sam", "sak", "B", "sbk", "sbn", "Q", "sqm", "S", "ssm",
             "ssj")
    plan = lambda **kw: tg.tg_gemm_quant_fp8_plan(*[{**base, **kw}[k] for k in order])  # noqa
    assert plan() == "tile_nt_256x256_q8"
    assert plan(op=0) == "tile_nt_256x256_q8"
    assert plan(op=2) is None                                  # fp8 inputs: not this entry
    assert plan(sbk=304, sbn=1, N=304, sqm=304) == "tile_nn_256x256_q8"
    assert plan(A=PA + 2) == "generic16_32x128_q8"             # misaligned A
    assert plan(K=0, A=0, B=0) == "generic16_32x128_q8"        # zero codes, unit scales
    assert plan(M=0) == "none"
    # the fused path of the 4096 x 7168 x 16384 product
    assert plan(M=4096, N=7168, K=16384, sam=16384, sbn=16384, sqm=7168, ssm=56) \
        == "tile_nt_256x256_q8"


def _callsw(lib, name, **kw):
    a = dict(M=8, N=300, K=64, A=PA, sam=64, sak=1, Bg=PB, Bu=PB + 0x8000, sbk=1, sbn=64, Q=PC,
             sqm=300, S=PS, ssm=3, ssj=1)
    a.update(kw)
    args = [a[k] for k in ("M", "N", "K", "A", "sam", "sak", "Bg", "Bu", "sbk", "sbn", "Q", "sqm",
                           "S", "ssm", "ssj")]
    if name == "plan":
        r = lib.tg_gemm_swiglu_quant_fp8_plan(a.get("op", 1), *args)
        return None if r is None else r.decode()
    if name == "plan_ws":
        r = lib.tg_gemm_swiglu_quant_fp8_plan_ws(a.get("op", 1), *args, a.get("ws_bytes", 0))
        return None if r is None else r.decode()
    if name == "ws_size":
        return tg.tg_gemm_swiglu_quant_fp8_workspace_size(a.get("op", 1), *args)
    if name.endswith("_ws"):
        return getattr(lib, name)(*args, a.get("ws", 0), a.get("ws_bytes", 0), None)
    return getattr(lib, name)(*args, None)


INVALIDSW = INVALIDQO[:9] + [dict(Bg=0), dict(Bu=0)] + INVALIDQO[10:]


@pytest.mark.parametrize("kw", INVALIDSW, ids=[str(k) for k in INVALIDSW])
@pytest.mark.parametrize("name", ["tg_gemm_f16_swiglu_quant_fp8", "tg_gemm_bf16_swiglu_quant_fp8",
                                  "tg_gemm_f16_swiglu_quant_fp8_ws",
                                  "tg_gemm_bf16_swiglu_quant_fp8_ws", "plan", "plan_ws", "ws_size"])
def test_swiglu_invalid(lib, name, kw):
    if name == "ws_size":
        with pytest.raises(tg.TgError):
            _callsw(lib, name, **kw)
        return
    r = _callsw(lib, name, **kw)
    assert (r is None) if name.startswith("plan") else (r == tg.TG_ERR_INVALID_VALUE)


# The fused SwiGLU's split plan (with a workspace): the K slices of each
# 128-column output slice split so that slices x splits stays within 256
# workgroups, with at least 8 slices per split and at most 8 splits, and
# none for more than 64 output slices with fewer than 16 K slices per split;
# 64 KiB of g and u partial tiles per slice and split after the 16 KiB of
# counters.
SWIGLU_WS_PLANS = [
    ((64, 16384, 7168), 2),     # the decode shape: 128 slices
    ((1, 7168, 7168), 4),       # 56 slices
    ((64, 300, 2048), 4),       # 3 slices, 32 K slices
    ((64, 256, 16384), 8),      # 2 slices, capped at 8 splits
    ((33, 200, 1040), 2),       # 17 K slices
    ((64, 32768, 7168), 1),     # 256 slices: no split
    ((64, 16384, 1024), 1),     # 128 slices, 2 splits would get 8 K slices each
    ((64, 16384, 2048), 2),     # 16 K slices per split
    ((16, 7168, 2048), 4),      # 56 slices
    ((8, 300, 64), 1),          # one K slice
]


@pytest.mark.parametrize("case", SWIGLU_WS_PLANS, ids=[f"{m}x{n}x{k}" for (m, n, k), _ in SWIGLU_WS_PLANS])
def test_swiglu_workspace_plans(lib, case):
    (M, N, K), splits = case
    kw = dict(M=M, N=N, K=K, sam=K, sbn=K, sqm=N, ssm=-(-N // 128))
    need = _callsw(lib, "ws_size", **kw)
    base = "skinny_64x128_swiglu_q8"
    assert _callsw(lib, "plan", **kw) == base
    if splits == 1:
        assert need == 0
        assert _callsw(lib, "plan_ws", ws_bytes=1 << 40, **kw) == base
        return
    assert need == 16384 + -(-N // 128) * splits * 64 * 1024
    want = f"{base}_splitk{splits}"
    assert _callsw(lib, "plan_ws", ws_bytes=need, **kw) == want
    assert _callsw(lib, "plan_ws", ws_bytes=1 << 40, **kw) == want
    assert _callsw(lib, "plan_ws", ws_bytes=need - 1, **kw) == base
    assert _callsw(lib, "plan_ws", op=0, ws_bytes=need, **kw) == want


def test_swiglu_workspace_other_paths_and_errors(lib):
    # larger M (the tile kernel) and misaligned weights (the masked kernel): no split plan
    kw = dict(M=4096, N=7168, K=7168, sam=7168, sbn=7168, sqm=7168, ssm=56)
    assert _callsw(lib, "ws_size", **kw) == 0
    assert _callsw(lib, "plan_ws", ws_bytes=1 << 40, **kw) == "tile_nt_256x256_swiglu_q8"
    assert _callsw(lib, "ws_size", M=8, Bu=PB + 2) == 0
    assert _callsw(lib, "plan_ws", M=8, Bu=PB + 2, ws_bytes=1 << 40) == \
        "generic16_32x128_swiglu_q8"
    assert _callsw(lib, "plan_ws", M=0, ws_bytes=1 << 20) == "none"
    assert _callsw(lib, "ws_size", M=0) == 0
    for name in ("tg_gemm_f16_swiglu_quant_fp8_ws", "tg_gemm_bf16_swiglu_quant_fp8_ws"):
        assert _callsw(lib, name, ws=0, ws_bytes=1 << 20) == tg.TG_ERR_INVALID_VALUE
        assert _callsw(lib, name, ws=PS + 16, ws_bytes=1 << 20) == tg.TG_ERR_INVALID_VALUE
        assert _callsw(lib, name, M=0, A=0, Bg=0, Bu=0, Q=0, S=0, ws=PS, ws_bytes=1 << 20) == \
            tg.TG_SUCCESS
    assert lib.tg_gemm_swiglu_quant_fp8_workspace_size(1, 8, 300, 64, PA, 64, 1, PB, PB + 0x8000,
                                                       1, 64, PC, 300, PS, 3, 1, None) == \
        tg.TG_ERR_INVALID_VALUE
    with pytest.raises(tg.TgError):
        _callsw(lib, "ws_size", op=2)


def test_swiglu_noop_and_plans(lib):
    for name in ("tg_gemm_f16_swiglu_quant_fp8", "tg_gemm_bf16_swiglu_quant_fp8"):
        assert _callsw(lib, name, M=0, A=0, Bg=0, Bu=0, Q=0, S=0) == tg.TG_SUCCESS
        assert _callsw(lib, name, N=0, A=0, Bg=0, Bu=0, Q=0, S=0) == tg.TG_SUCCESS
    plan = lambda **kw: _callsw(lib, "plan", **kw)  # noqa
    assert plan() == "skinny_64x128_swiglu_q8"                 # M <= 64
    assert plan(op=0) == "skinny_64x128_swiglu_q8"
    assert plan(M=64) == "skinny_64x128_swiglu_q8"
    assert plan(M=65, ssm=3) == "tile_nt_256x256_swiglu_q8"
    assert plan(M=1, K=7168, sam=7168, sbn=7168) == "skinny_64x128_swiglu_q8"
    assert plan(op=2) is None                                  # fp8 inputs: not this entry
    for M in (8, 300):
        assert plan(M=M, Bu=PB + 2) == "generic16_32x128_swiglu_q8"  # misaligned up weights
        assert plan(M=M, Bg=PB + 2) == "generic16_32x128_swiglu_q8"  # misaligned gate weights
        assert plan(M=M, sbk=304, sbn=1, N=304, sqm=304) == "generic16_32x128_swiglu_q8"  # K x N
    assert plan(K=0, A=0, Bg=0, Bu=0) == "generic16_32x128_swiglu_q8"
    assert plan(M=0) == "none"
    # gate and up projections of a 7168-wide layer over 4096 rows
    assert plan(M=4096, N=7168, K=7168, sam=7168, sbn=7168, sqm=7168, ssm=56) \
        == "tile_nt_256x256_swiglu_q8"


def _grouped(lib, fn, **kw):
    import numpy as np
    a = dict(G=2, off=[0, 100, 300], N=64, K=128, A=PA, lda=128, B=PB, ldb=128, sbg=64 * 128,
             C=PC, ldc=64)
    a.update(kw)
    off = None if a["off"] is None else np.ascontiguousarray(a["off"], dtype=np.int64)
    ptr = 0 if off is None else off.ctypes.data
    args = [a["G"], ptr, a["N"], a["K"], a["A"], a["lda"], a["B"], a["ldb"], a["sbg"], a["C"],
            a["ldc"]]
    if fn == "plan":
        r = lib.tg_gemm_grouped_plan(*args)
        return None if r is None else r.decode()
    return getattr(lib, fn)(*args, None)


INVALIDG = [dict(G=-1), dict(N=-1), dict(K=-1), dict(lda=-1), dict(sbg=-1), dict(off=[0, 200, 100]),
            dict(off=[-1, 100, 300]), dict(off=None), dict(lda=100), dict(ldc=63), dict(ldb=127),
            dict(C=0), dict(A=0), dict(B=0), dict(G=2, sbg=1 << 62)]


@pytest.mark.parametrize("kw", INVALIDG, ids=[str(k) for k in INVALIDG])
@pytest.mark.parametrize("fn", ["tg_gemm_grouped_f16", "tg_gemm_grouped_bf16"])
def test_grouped_invalid(lib, fn, kw):
    assert _grouped(lib, fn, **kw) == tg.TG_ERR_INVALID_VALUE
    assert _grouped(lib, "plan", **kw) is None


def test_grouped_noop_and_plans(lib):
    for kw in (dict(G=0, off=[0]), dict(off=[0, 0, 0]), dict(N=0)):
        assert _grouped(lib, "tg_gemm_grouped_bf16", **kw) == tg.TG_SUCCESS
        assert _grouped(lib, "plan", **kw) == "none"
    assert _grouped(lib, "plan") == "grouped_tile_nt_256x224"
    assert _grouped(lib, "plan", lda=129) == "per_group"          # rows not 16-byte multiples
    assert _grouped(lib, "plan", K=100, lda=128, ldb=128) == "per_group"   # K % 8 != 0
    assert _grouped(lib, "plan", G=129, off=list(range(0, 130 * 2, 2))) == "per_group"
    assert _grouped(lib, "plan", off=[0, 2048, 4096], N=4096, ldc=4096,
                    sbg=4096 * 128) == "grouped_tile_nt_256x256"
    # 8192 rows in 8 uneven groups x 4096 x 7168: 684 tiles of 256 x 224
    # (3 waves) against 576 of 256 x 256 (also 3)
    off = [0, 1246, 2575, 3497, 4713, 5522, 6122, 6748, 8192]
    assert _grouped(lib, "plan", G=8, off=off, N=4096, K=7168, lda=7168, ldb=7168,
                    sbg=4096 * 7168, ldc=4096) == "grouped_tile_nt_256x224"


def _grouped8(lib, plan=False, **kw):
    import numpy as np
    a = dict(G=2, off=[0, 100, 300], N=64, K=128, A=PA, lda=128, SA=PS, ssam=1, ssak=1, B=PB,
             ldb=128, sbg=64 * 128, SB=PS + 4096, ssbn=1, ssbk=1, ssbg=1, C=PC, ldc=64)
    a.update(kw)
    off = None if a["off"] is None else np.ascontiguousarray(a["off"], dtype=np.int64)
    args = [a["G"], 0 if off is None else off.ctypes.data, a["N"], a["K"], a["A"], a["lda"],
            a["SA"], a["ssam"], a["ssak"], a["B"], a["ldb"], a["sbg"], a["SB"], a["ssbn"],
            a["ssbk"], a["ssbg"], a["C"], a["ldc"]]
    if plan:
        r = lib.tg_gemm_grouped_fp8_plan(*args)
        return None if r is None else r.decode()
    return lib.tg_gemm_grouped_fp8_blockscaled(*args, None)


INVALIDG8 = INVALIDG + [dict(SA=0), dict(SB=0), dict(ssbg=-1), dict(ssak=-1),
                        dict(ssbg=1 << 62)]


@pytest.mark.parametrize("kw", INVALIDG8, ids=[str(k) for k in INVALIDG8])
def test_grouped_fp8_invalid(lib, kw):
    assert _grouped8(lib, **kw) == tg.TG_ERR_INVALID_VALUE
    assert _grouped8(lib, plan=True, **kw) is None


def test_grouped_fp8_noop_and_plans(lib):
    for kw in (dict(G=0, off=[0]), dict(off=[0, 0, 0]), dict(N=0)):
        assert _grouped8(lib, **kw) == tg.TG_SUCCESS
        assert _grouped8(lib, plan=True, **kw) == "none"
    assert _grouped8(lib, plan=True) == "grouped_tile_fp8_256x128"
    # 8 x 1024 rows x 4096 columns: 32 tile rows, 512 tiles of 256 x 256 (2 rounds on 256
    # CUs) against 1024 of 256 x 128 (4 rounds)
    wide = dict(G=8, off=[1024 * g for g in range(9)], N=4096, ldc=4096, sbg=4096 * 128)
    assert _grouped8(lib, plan=True, **wide) == "grouped_tile_fp8_256x256"
    assert _grouped8(lib, plan=True, lda=136) == "per_group"       # rows not 16-byte multiples
    assert _grouped8(lib, plan=True, sbg=64 * 128 + 8) == "per_group"


def test_python_wrapper_raises(lib):
    with pytest.raises(tg.TgError) as e:
        tg.tg_gemm_bf16(-1, 8, 8, PA, 8, 1, PB, 8, 1, PC, 8, 1, 0)
    assert e.value.status == tg.TG_ERR_INVALID_VALUE


def test_plan_names(lib):
    plan = lambda *a: tg.tg_gemm_plan(*a)  # noqa: E731
    assert plan(tg.OP_BF16, 0, 8, 8, PA, 8, 1, PB, 8, 1, PC, 8, 1) == "none"
    assert plan(tg.OP_BF16, -1, 8, 8, PA, 8, 1, PB, 8, 1, PC, 8, 1) is None
    assert plan(7, 8, 8, 8, PA, 8, 1, PB, 8, 1, PC, 8, 1) is None
    # a ragged, odd-strided call must go to the general kernel
    assert plan(tg.OP_F16, 13, 7, 5, PA + 2, 5, 1, PB, 1, 5, PC, 7, 1).startswith("generic")
    assert plan(tg.OP_FP8, 13, 7, 5, PA + 1, 5, 1, PB, 1, 5, PC, 7, 1).startswith("generic")


# The kernel each benchmark workload is planned onto (host-side choice; no
# launch), by the allocation-free entry points and by the workspace ones
# given all the workspace their split plans ask for.  A silent fallback to
# the general kernel fails here.
EXPECTED_PLANS = {
    "fp16_256": ("tile_nn_256x256", "tile_nn_256x256"),
    "bf16_4096": ("tile_nn_256x256", "tile_nn_256x256"),
    "bf16_4096x7168x16384": ("tile_nt_256x224", "tile_nt_256x224"),
    "bf16_skinny_64x7168x7168": ("skinny_64x32", "skinny_64x128_splitk4"),
    "fp8_4096x7168x16384": ("tile_fp8_256x256", "tile_fp8_256x256"),
}


# The plan for each shape of the benchmark's sweep (bf16, B stored N x K) and
# for the boundaries of the small-grid rule, without and with a workspace:
# small grids (at most half the CUs in 256 x 224 tiles) take 128 x 128 tiles
# (two-stage when there are more than 256 of them), with K split when a
# workspace is given and K is at most 128 slices of 64; with longer K and a
# workspace, 256 x 224 with split K; larger grids 256 x 224 or 256 x 256 by
# wave quantisation, and with a workspace a partial second wave of 256 x 224
# tiles may be split over K.
SWEEP_PLANS = [
    (4096, 7168, 7168, "tile_nt_256x224", "tile_nt_256x224"),
    (4096, 896, 16384, "tile_nt_128x128", "tile_nt_256x224_splitk4"),
    (1024, 1024, 4096, "tile_nt_128x128", "tile_nt_128x128_splitk4"),
    (2048, 2048, 2048, "tile_nt_128x128", "tile_nt_128x128"),
    (8192, 8192, 8192, "tile_nt_256x256", "tile_nt_256x256"),
    (2048, 7168, 16384, "tile_nt_256x224", "tile_nt_256x224"),
    (1024, 1024, 8192, "tile_nt_128x128", "tile_nt_128x128_splitk4"),
    (1024, 1024, 8200, "tile_nt_128x128", "tile_nt_256x224_splitk7"),
    (2048, 2048, 8192, "tile_nt_128x128", "tile_nt_128x128"),
    (4096, 4096, 1024, "tile_nt_256x256", "tile_nt_256x256"),
    (4096, 1792, 4096, "tile_nt_128x128_2stage", "tile_nt_128x128_2stage"),
    (4096, 1024, 4096, "tile_nt_128x128", "tile_nt_128x128"),
    # one whole wave and a partial one: the partial wave's tiles split over K
    (4352, 4096, 1024, "tile_nt_256x224", "tile_nt_256x224_tail2"),
    (4400, 4000, 2056, "tile_nt_256x224", "tile_nt_256x224_tail3"),
    (4300, 4000, 4104, "tile_nt_256x224", "tile_nt_256x224_tail5"),
    (4352, 4096, 4096, "tile_nt_256x224", "tile_nt_256x224_tail3"),
    (4352, 4096, 448, "tile_nt_256x224", "tile_nt_256x224"),      # K too short to split
    (6144, 6144, 2048, "tile_nt_256x224", "tile_nt_256x224"),     # three waves: unsplit
]


def _ws_bytes(op, M, N, K, sbk, sbn):
    return tg.tg_gemm_workspace_size(op, M, N, K, PA, K, 1, PB, sbk, sbn, PC, N, 1)


@pytest.mark.parametrize("case", SWEEP_PLANS, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in SWEEP_PLANS])
def test_sweep_plans(lib, case):
    M, N, K, want, want_ws = case
    got = tg.tg_gemm_plan(tg.OP_BF16, M, N, K, PA, K, 1, PB, 1, K, PC, N, 1)
    assert got == want
    need = _ws_bytes(tg.OP_BF16, M, N, K, 1, K)
    assert (need > 0) == (want != want_ws)
    args = (tg.OP_BF16, M, N, K, PA, K, 1, PB, 1, K, PC, N, 1)
    assert tg.tg_gemm_plan_ws(*args, need) == want_ws
    assert tg.tg_gemm_plan_ws(*args, 1 << 40) == want_ws
    if need:
        # one byte short of the split plan's scratch: the allocation-free plan
        assert tg.tg_gemm_plan_ws(*args, need - 1) == want
        assert tg.tg_gemm_plan_ws(*args, 0) == want


@pytest.mark.parametrize("name", sorted(EXPECTED_PLANS))
def test_workload_plans(lib, name):
    from gen import configs
    w = configs.WORKLOADS[name]
    sbk, sbn = configs.b_strides(w.b_layout, w.N, w.K)
    op = {"f16": tg.OP_F16, "bf16": tg.OP_BF16, "fp8": tg.OP_FP8}[w.dtype]
    args = (op, w.M, w.N, w.K, PA, w.K, 1, PB, sbk, sbn, PC, w.N, 1)
    assert tg.tg_gemm_plan(*args) == EXPECTED_PLANS[name][0]
    assert tg.tg_gemm_plan_ws(*args, _ws_bytes(op, w.M, w.N, w.K, sbk, sbn)) == \
        EXPECTED_PLANS[name][1]


# The fp8 tile shape by grid size: 256 x 256 tiles unless 256 x 128 tiles take
# fewer tile rounds on 256 CUs, a round of 256 x 256 counting 4/3 of one of
# 256 x 128 (64 against 48 KiB moved per slice).
FP8_TILE_PLANS = [
    ((64, 7168, 7168), "skinny_fp8_64x32"),     # M <= 64: 32-column strips over all of K
    ((1, 100, 16), "skinny_fp8_64x32"),
    ((65, 7168, 7168), "tile_fp8_256x128"),     # 28 tiles
    ((64, 100, 24), "generic_fp8_64x64"),       # K not a multiple of 16
    ((256, 128, 128), "tile_fp8_256x128"),      # 1 tile either way
    ((2048, 2048, 1024), "tile_fp8_256x128"),   # 64 or 128 tiles: one round each
    ((1024, 8192, 512), "tile_fp8_256x128"),    # 128 or 256 tiles: one round each
    ((4096, 4096, 256), "tile_fp8_256x256"),    # 256 tiles (1 round) or 512 (2)
    ((4000, 4000, 400), "tile_fp8_256x256"),
    ((4097, 4000, 16), "tile_fp8_256x256"),     # 272 (2 rounds) or 544 (3)
    ((4096, 3968, 1040), "tile_fp8_256x256"),   # 256 or 496
    ((2500, 7000, 2064), "tile_fp8_256x256"),   # 280 or 550
    ((4096, 7168, 16384), "tile_fp8_256x256"),  # 448 (2 rounds) or 896 (4)
]


@pytest.mark.parametrize("case", FP8_TILE_PLANS, ids=[f"{m}x{n}x{k}" for (m, n, k), _ in FP8_TILE_PLANS])
def test_fp8_tile_plans(lib, case):
    (M, N, K), want = case
    assert tg.tg_gemm_plan(tg.OP_FP8, M, N, K, PA, K, 1, PB, 1, K, PC, N, 1) == want


# The fp8 decode product with a workspace: 64 x 128 strips, the K blocks
# split so that strips x splits stays within 256 workgroups, with at least 4
# blocks per split -- for more than 32 rows, where the strip grid's rounds
# times the K blocks reach 96, or the strip grid (32-column strips) fills at
# most half the CUs and K has at least 56 blocks.  Otherwise (and for M > 64,
# or K not a multiple of 16) the plan without workspace.
FP8_WS_PLANS = [
    ((64, 7168, 16384), "skinny_fp8_64x128_splitk4"),    # 1 round x 128 blocks
    ((33, 7168, 18432), "skinny_fp8_64x128_splitk4"),    # 1 round x 144 blocks
    ((64, 16384, 7168), "skinny_fp8_64x128_splitk2"),    # 2 rounds x 56 blocks
    ((48, 8192, 12288), "skinny_fp8_64x128_splitk4"),    # 1 round x 96 blocks
    ((40, 4096, 7168), "skinny_fp8_64x128_splitk8"),     # 128 strip workgroups, 56 blocks
    ((64, 2048, 7168), "skinny_fp8_64x128_splitk"),      # 64 strip workgroups: 14 splits
    ((64, 4096, 6144), "skinny_fp8_64x32"),              # half grid, but 48 blocks
    ((64, 7168, 7168), "skinny_fp8_64x32"),              # 1 round x 56 blocks
    ((64, 4096, 4096), "skinny_fp8_64x32"),              # half grid, but 32 blocks
    ((64, 1024, 4096), "skinny_fp8_64x32"),
    ((32, 16384, 7168), "skinny_fp8_64x32"),             # 32 rows
    ((1, 7168, 16384), "skinny_fp8_64x32"),
    ((64, 32768, 7168), "skinny_fp8_64x32"),             # 256 strips: no split
    ((64, 1000, 384), "skinny_fp8_64x32"),               # 3 blocks: too short to split
    ((65, 7168, 7168), "tile_fp8_256x128"),
    ((64, 100, 24), "generic_fp8_64x64"),
]


@pytest.mark.parametrize("case", FP8_WS_PLANS, ids=[f"{m}x{n}x{k}" for (m, n, k), _ in FP8_WS_PLANS])
def test_fp8_workspace_plans(lib, case):
    (M, N, K), want = case
    args = (tg.OP_FP8, M, N, K, PA, K, 1, PB, 1, K, PC, N, 1)
    need = _ws_bytes(tg.OP_FP8, M, N, K, 1, K)
    plain = tg.tg_gemm_plan(*args)
    assert (need > 0) == (want != plain)
    assert tg.tg_gemm_plan_ws(*args, need) == want
    assert tg.tg_gemm_plan_ws(*args, 1 << 40) == want
    if need:
        assert plain == "skinny_fp8_64x32"
        assert tg.tg_gemm_plan_ws(*args, need - 1) == plain
        assert tg.tg_gemm_plan_ws(*args, 0) == plain
        strips = -(-N // 128)
        splits = int(want.rsplit("splitk", 1)[1] or 14)    # the names go to splitk8
        assert need == 16384 + strips * splits * 64 * 128 * 4


# The 16-bit skinny product with a workspace: its split plan where it pays --
# the strip grid's rounds times the K slices (64 wide) reach 96, or the
# strip grid (32-column strips) fills at most half the CUs; otherwise the
# allocation-free 32-column strips.
BF16_WS_PLANS = [
    ((64, 7168, 7168), "skinny_64x128_splitk4"),     # 1 round x 112 slices
    ((1, 7168, 7168), "skinny_64x128_splitk4"),
    ((64, 16384, 7168), "skinny_64x128_splitk2"),    # 2 rounds x 112
    ((64, 7168, 16384), "skinny_64x128_splitk4"),
    ((64, 4096, 4096), "skinny_64x128_splitk8"),     # 128 strip workgroups
    ((64, 1024, 4096), "skinny_64x128_splitk8"),
    ((64, 7168, 4096), "skinny_64x32"),              # 1 round x 64 slices
    ((64, 7168, 2048), "skinny_64x32"),              # 1 round x 32 slices
    ((40, 7168, 1024), "skinny_64x32"),
    ((64, 7168, 520), "skinny_64x128"),              # 9 slices: too short to split
]


@pytest.mark.parametrize("case", BF16_WS_PLANS, ids=[f"{m}x{n}x{k}" for (m, n, k), _ in BF16_WS_PLANS])
def test_bf16_skinny_workspace_plans(lib, case):
    (M, N, K), want = case
    args = (tg.OP_BF16, M, N, K, PA, K, 1, PB, 1, K, PC, N, 1)
    need = _ws_bytes(tg.OP_BF16, M, N, K, 1, K)
    assert tg.tg_gemm_plan_ws(*args, 1 << 40) == want
    assert (need > 0) == ("splitk" in want)
    if need:
        assert tg.tg_gemm_plan_ws(*args, need) == want
        assert tg.tg_gemm_plan_ws(*args, need - 1) == tg.tg_gemm_plan(*args) == "skinny_64x32"


def test_workspace_sizes(lib):
    """The split plans' scratch: a 16 KiB counter area, then 4 bytes per
    element of each split's partial tile."""
    assert _ws_bytes(tg.OP_BF16, 64, 7168, 7168, 1, 7168) == 16384 + 56 * 4 * 64 * 128 * 4
    assert _ws_bytes(tg.OP_BF16, 4096, 896, 16384, 1, 16384) == 16384 + 64 * 4 * 256 * 224 * 4
    assert _ws_bytes(tg.OP_F16, 1024, 1024, 4096, 1, 4096) == 16384 + 64 * 4 * 128 * 128 * 4
    assert _ws_bytes(tg.OP_BF16, 4352, 4096, 4096, 1, 4096) == 16384 + 67 * 3 * 256 * 224 * 4
    assert _ws_bytes(tg.OP_BF16, 4096, 7168, 16384, 1, 16384) == 0
    assert _ws_bytes(tg.OP_FP8, 64, 7168, 16384, 1, 16384) == 16384 + 56 * 4 * 64 * 128 * 4
    assert _ws_bytes(tg.OP_FP8, 64, 7168, 7168, 1, 7168) == 0
    assert _ws_bytes(tg.OP_FP8, 65, 7168, 7168, 1, 7168) == 0
    assert _ws_bytes(tg.OP_BF16, 0, 8, 8, 1, 8) == 0
    with pytest.raises(tg.TgError):
        _ws_bytes(tg.OP_BF16, -1, 8, 8, 1, 8)
    with pytest.raises(tg.TgError):
        _ws_bytes(5, 8, 8, 8, 1, 8)
    out = ctypes.c_size_t(0)
    assert lib.tg_gemm_workspace_size(1, 8, 8, 8, PA, 8, 1, PB, 1, 8, PC, 8, 1, None) == \
        tg.TG_ERR_INVALID_VALUE
    assert lib.tg_gemm_workspace_size(1, 8, 8, 8, PA, 8, 1, PB, 1, 8, PC, 8, 1,
                                      ctypes.byref(out)) == tg.TG_SUCCESS and out.value == 0


@pytest.mark.parametrize("name", ["tg_gemm_f16_ws", "tg_gemm_bf16_ws"])
def test_workspace_invalid(lib, name):
    fn = getattr(lib, name)
    args = (64, 7168, 7168, PA, 7168, 1, PB, 1, 7168, PC, 7168, 1)
    assert fn(*args, 0, 1 << 20, None) == tg.TG_ERR_INVALID_VALUE          # NULL workspace
    assert fn(*args, PS + 16, 1 << 20, None) == tg.TG_ERR_INVALID_VALUE    # not 256-byte aligned
    bad = (-1,) + args[1:]
    assert fn(*bad, PS, 1 << 20, None) == tg.TG_ERR_INVALID_VALUE
    assert fn(0, *args[1:], PS, 1 << 20, None) == tg.TG_SUCCESS             # no-op


def test_fp8_workspace_invalid(lib):
    fn = lib.tg_gemm_fp8_blockscaled_ws
    args = (64, 7168, 7168, PA, 7168, 1, PS, 56, 1, PB, 1, 7168, PS, 56, 1, PC, 7168, 1)
    assert fn(*args, 0, 1 << 20, None) == tg.TG_ERR_INVALID_VALUE          # NULL workspace
    assert fn(*args, PS + 16, 1 << 20, None) == tg.TG_ERR_INVALID_VALUE    # not 256-byte aligned
    bad = args[:6] + (0,) + args[7:]                                         # NULL SA
    assert fn(*bad, PS, 1 << 20, None) == tg.TG_ERR_INVALID_VALUE
    bad = (-1,) + args[1:]
    assert fn(*bad, PS, 1 << 20, None) == tg.TG_ERR_INVALID_VALUE
    assert fn(0, *args[1:], PS, 1 << 20, None) == tg.TG_SUCCESS             # no-op


def test_static_scratch_host_checks(lib):
    """The fixed-scratch entry point validates and sizes on the host before
    any HIP call: invalid arguments, a split plan larger than its 64 MiB
    array (4096 x 4896 x 4096: 96 tiles past the first wave split 5 ways,
    105 MiB) and empty calls return without touching the device."""
    fn = lib.tg_gemm_bf16_static_scratch
    assert fn(4096, 4896, 4096, PA, 4096, 1, PB, 1, 4096, PC, 4896, 1, None) == \
        tg.TG_ERR_SCRATCH_LIMIT
    assert tg.tg_gemm_workspace_size(tg.OP_BF16, 4096, 4896, 4096, PA, 4096, 1, PB, 1, 4096, PC,
                                     4896, 1) > 64 << 20
    assert fn(-1, 8, 8, PA, 8, 1, PB, 1, 8, PC, 8, 1, None) == tg.TG_ERR_INVALID_VALUE
    assert fn(8, 8, 8, PA, 8, 1, PB, 1, 8, PC, 8, 2, None) == tg.TG_ERR_UNSUPPORTED
    assert fn(0, 8, 8, PA, 8, 1, PB, 1, 8, PC, 8, 1, None) == tg.TG_SUCCESS
