"""Python binding of libtg_gemm.so: the tiled dense GEMM C = A * B on MI355X.

Argument marshalling only -- every step of the product runs in the library's
HIP kernels.  The functions carry the C-ABI's names (include/tg_gemm.h) and
take device pointers as integers, element strides and a hipStream_t handle.
The `*_t` helpers read those arguments off torch tensors (torch only owns the
device memory and the streams).  There is no fallback: if the library is not
built, `load()` raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtg_gemm.so")

TG_SUCCESS, TG_ERR_INVALID_VALUE, TG_ERR_UNSUPPORTED, TG_ERR_LAUNCH = 0, 1, 2, 3
TG_ERR_SCRATCH_LIMIT = 4
OP_F16, OP_BF16, OP_FP8 = 0, 1, 2
EXPORTS = ("tg_status_string", "tg_gemm_f16", "tg_gemm_bf16", "tg_gemm_fp8_blockscaled",
           "tg_gemm_plan", "tg_quant_fp8_1x128", "tg_quant_fp8_128x128", "tg_gemm_grouped_f16",
           "tg_gemm_grouped_bf16", "tg_gemm_grouped_plan", "tg_gemm_grouped_fp8_blockscaled",
           "tg_gemm_grouped_fp8_plan", "tg_gemm_f16_quant_fp8", "tg_gemm_bf16_quant_fp8",
           "tg_gemm_quant_fp8_plan", "tg_gemm_f16_ws", "tg_gemm_bf16_ws", "tg_gemm_workspace_size",
           "tg_gemm_plan_ws", "tg_gemm_bf16_static_scratch", "tg_gemm_f16_swiglu_quant_fp8",
           "tg_gemm_bf16_swiglu_quant_fp8", "tg_gemm_swiglu_quant_fp8_plan",
           "tg_gemm_fp8_blockscaled_ws", "tg_gemm_f16_swiglu_quant_fp8_ws",
           "tg_gemm_bf16_swiglu_quant_fp8_ws", "tg_gemm_swiglu_quant_fp8_workspace_size",
           "tg_gemm_swiglu_quant_fp8_plan_ws")


class TgError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def load():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m dense_tiled_gemm_03_amd.build`"
                           " (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.tg_status_string.argtypes = [c_int]
    lib.tg_status_string.restype = ctypes.c_char_p
    sig16 = [i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64, vp]
    for name in ("tg_gemm_f16", "tg_gemm_bf16"):
        getattr(lib, name).argtypes = sig16
        getattr(lib, name).restype = c_int
    lib.tg_gemm_fp8_blockscaled.argtypes = [i64, i64, i64, vp, i64, i64, vp, i64, i64,
                                            vp, i64, i64, vp, i64, i64, vp, i64, i64, vp]
    lib.tg_gemm_fp8_blockscaled.restype = c_int
    lib.tg_gemm_fp8_blockscaled_ws.argtypes = (lib.tg_gemm_fp8_blockscaled.argtypes[:-1]
                                               + [vp, ctypes.c_size_t, vp])
    lib.tg_gemm_fp8_blockscaled_ws.restype = c_int
    lib.tg_gemm_plan.argtypes = [c_int, i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64]
    lib.tg_gemm_plan.restype = ctypes.c_char_p
    sz = ctypes.c_size_t
    for name in ("tg_gemm_f16_ws", "tg_gemm_bf16_ws"):
        getattr(lib, name).argtypes = sig16[:-1] + [vp, sz, vp]
        getattr(lib, name).restype = c_int
    lib.tg_gemm_bf16_static_scratch.argtypes = sig16
    lib.tg_gemm_bf16_static_scratch.restype = c_int
    lib.tg_gemm_workspace_size.argtypes = [c_int, i64, i64, i64, vp, i64, i64, vp, i64, i64, vp,
                                           i64, i64, ctypes.POINTER(sz)]
    lib.tg_gemm_workspace_size.restype = c_int
    lib.tg_gemm_plan_ws.argtypes = [c_int, i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64,
                                    sz]
    lib.tg_gemm_plan_ws.restype = ctypes.c_char_p
    sigg = [i64, vp, i64, i64, vp, i64, vp, i64, i64, vp, i64]
    for name in ("tg_gemm_grouped_f16", "tg_gemm_grouped_bf16"):
        getattr(lib, name).argtypes = sigg + [vp]
        getattr(lib, name).restype = c_int
    lib.tg_gemm_grouped_plan.argtypes = sigg
    lib.tg_gemm_grouped_plan.restype = ctypes.c_char_p
    sig8 = [i64, vp, i64, i64, vp, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64, i64, vp, i64]
    lib.tg_gemm_grouped_fp8_blockscaled.argtypes = sig8 + [vp]
    lib.tg_gemm_grouped_fp8_blockscaled.restype = c_int
    lib.tg_gemm_grouped_fp8_plan.argtypes = sig8
    lib.tg_gemm_grouped_fp8_plan.restype = ctypes.c_char_p
    for name in ("tg_quant_fp8_1x128", "tg_quant_fp8_128x128"):
        getattr(lib, name).argtypes = [i64, i64, vp, i64, vp, i64, vp, i64, i64, vp]
        getattr(lib, name).restype = c_int
    sigq = [i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, vp, i64, i64]
    for name in ("tg_gemm_f16_quant_fp8", "tg_gemm_bf16_quant_fp8"):
        getattr(lib, name).argtypes = sigq + [vp]
        getattr(lib, name).restype = c_int
    lib.tg_gemm_quant_fp8_plan.argtypes = [c_int] + sigq
    lib.tg_gemm_quant_fp8_plan.restype = ctypes.c_char_p
    sigs = [i64, i64, i64, vp, i64, i64, vp, vp, i64, i64, vp, i64, vp, i64, i64]
    for name in ("tg_gemm_f16_swiglu_quant_fp8", "tg_gemm_bf16_swiglu_quant_fp8"):
        getattr(lib, name).argtypes = sigs + [vp]
        getattr(lib, name).restype = c_int
    lib.tg_gemm_swiglu_quant_fp8_plan.argtypes = [c_int] + sigs
    lib.tg_gemm_swiglu_quant_fp8_plan.restype = ctypes.c_char_p
    for name in ("tg_gemm_f16_swiglu_quant_fp8_ws", "tg_gemm_bf16_swiglu_quant_fp8_ws"):
        getattr(lib, name).argtypes = sigs + [vp, ctypes.c_size_t, vp]
        getattr(lib, name).restype = c_int
    lib.tg_gemm_swiglu_quant_fp8_workspace_size.argtypes = (
        [c_int] + sigs + [ctypes.POINTER(ctypes.c_size_t)])
    lib.tg_gemm_swiglu_quant_fp8_workspace_size.restype = c_int
    lib.tg_gemm_swiglu_quant_fp8_plan_ws.argtypes = [c_int] + sigs + [ctypes.c_size_t]
    lib.tg_gemm_swiglu_quant_fp8_plan_ws.restype = ctypes.c_char_p
    _lib = lib
    return lib


def ensure_built():
    """Build the library if it is missing (tests, smoke and bench use this)."""
    if not os.path.exists(LIB_PATH):
        from . import build
        build.build()
    return load()


def tg_status_string(status: int) -> str:
    return load().tg_status_string(status).decode()


def _check(status: int) -> int:
    if status != TG_SUCCESS:
        raise TgError(status, tg_status_string(status))
    return status


def tg_gemm_f16(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, stream=0):
    return _check(load().tg_gemm_f16(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, stream))


def tg_gemm_bf16(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, stream=0):
    return _check(load().tg_gemm_bf16(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, stream))


def tg_gemm_f16_ws(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, workspace, workspace_bytes,
                   stream=0):
    return _check(load().tg_gemm_f16_ws(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, workspace,
                                        workspace_bytes, stream))


def tg_gemm_bf16_ws(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, workspace, workspace_bytes,
                    stream=0):
    return _check(load().tg_gemm_bf16_ws(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn,
                                         workspace, workspace_bytes, stream))


def tg_gemm_bf16_static_scratch(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, stream=0):
    return _check(load().tg_gemm_bf16_static_scratch(M, N, K, A, sam, sak, B, sbk, sbn, C, scm,
                                                     scn, stream))


def tg_gemm_workspace_size(op, M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn):
    """Workspace bytes of the call's split plan (0: none)."""
    out = ctypes.c_size_t(0)
    _check(load().tg_gemm_workspace_size(op, M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn,
                                         ctypes.byref(out)))
    return out.value


def tg_gemm_plan_ws(op, M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, workspace_bytes):
    r = load().tg_gemm_plan_ws(op, M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn,
                               workspace_bytes)
    return None if r is None else r.decode()


def tg_gemm_fp8_blockscaled(M, N, K, A, sam, sak, SA, ssam, ssak, B, sbk, sbn, SB, ssbn, ssbk,
                            C, scm, scn, stream=0):
    return _check(load().tg_gemm_fp8_blockscaled(M, N, K, A, sam, sak, SA, ssam, ssak, B, sbk,
                                                 sbn, SB, ssbn, ssbk, C, scm, scn, stream))


def tg_gemm_fp8_blockscaled_ws(M, N, K, A, sam, sak, SA, ssam, ssak, B, sbk, sbn, SB, ssbn,
                               ssbk, C, scm, scn, workspace, workspace_bytes, stream=0):
    return _check(load().tg_gemm_fp8_blockscaled_ws(M, N, K, A, sam, sak, SA, ssam, ssak, B, sbk,
                                                    sbn, SB, ssbn, ssbk, C, scm, scn, workspace,
                                                    workspace_bytes, stream))


def tg_quant_fp8_1x128(R, K, X, ldx, Q, ldq, S, ssr, ssk, stream=0):
    return _check(load().tg_quant_fp8_1x128(R, K, X, ldx, Q, ldq, S, ssr, ssk, stream))


def tg_quant_fp8_128x128(R, K, X, ldx, Q, ldq, S, ssr, ssk, stream=0):
    return _check(load().tg_quant_fp8_128x128(R, K, X, ldx, Q, ldq, S, ssr, ssk, stream))


def tg_gemm_f16_quant_fp8(M, N, K, A, sam, sak, B, sbk, sbn, Q, sqm, S, ssm, ssj, stream=0):
    return _check(load().tg_gemm_f16_quant_fp8(M, N, K, A, sam, sak, B, sbk, sbn, Q, sqm, S, ssm,
                                               ssj, stream))


def tg_gemm_bf16_quant_fp8(M, N, K, A, sam, sak, B, sbk, sbn, Q, sqm, S, ssm, ssj, stream=0):
    return _check(load().tg_gemm_bf16_quant_fp8(M, N, K, A, sam, sak, B, sbk, sbn, Q, sqm, S, ssm,
                                                ssj, stream))


def tg_gemm_quant_fp8_plan(op, M, N, K, A, sam, sak, B, sbk, sbn, Q, sqm, S, ssm, ssj):
    r = load().tg_gemm_quant_fp8_plan(op, M, N, K, A, sam, sak, B, sbk, sbn, Q, sqm, S, ssm, ssj)
    return None if r is None else r.decode()


def tg_gemm_f16_swiglu_quant_fp8(M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q, sqm, S, ssm, ssj,
                                 stream=0):
    return _check(load().tg_gemm_f16_swiglu_quant_fp8(M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q,
                                                      sqm, S, ssm, ssj, stream))


def tg_gemm_bf16_swiglu_quant_fp8(M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q, sqm, S, ssm, ssj,
                                  stream=0):
    return _check(load().tg_gemm_bf16_swiglu_quant_fp8(M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q,
                                                       sqm, S, ssm, ssj, stream))


def tg_gemm_swiglu_quant_fp8_plan(op, M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q, sqm, S, ssm,
                                  ssj):
    r = load().tg_gemm_swiglu_quant_fp8_plan(op, M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q, sqm,
                                             S, ssm, ssj)
    return None if r is None else r.decode()


def tg_gemm_f16_swiglu_quant_fp8_ws(M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q, sqm, S, ssm, ssj,
                                    workspace, workspace_bytes, stream=0):
    return _check(load().tg_gemm_f16_swiglu_quant_fp8_ws(M, N, K, A, sam, sak, Bg, Bu, sbk, sbn,
                                                         Q, sqm, S, ssm, ssj, workspace,
                                                         workspace_bytes, stream))


def tg_gemm_bf16_swiglu_quant_fp8_ws(M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q, sqm, S, ssm, ssj,
                                     workspace, workspace_bytes, stream=0):
    return _check(load().tg_gemm_bf16_swiglu_quant_fp8_ws(M, N, K, A, sam, sak, Bg, Bu, sbk, sbn,
                                                          Q, sqm, S, ssm, ssj, workspace,
                                                          workspace_bytes, stream))


def tg_gemm_swiglu_quant_fp8_workspace_size(op, M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q, sqm, S,
                                            ssm, ssj):
    """Workspace bytes of the fused SwiGLU call's split plan (0: none)."""
    out = ctypes.c_size_t(0)
    _check(load().tg_gemm_swiglu_quant_fp8_workspace_size(op, M, N, K, A, sam, sak, Bg, Bu, sbk,
                                                          sbn, Q, sqm, S, ssm, ssj,
                                                          ctypes.byref(out)))
    return out.value


def tg_gemm_swiglu_quant_fp8_plan_ws(op, M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q, sqm, S, ssm,
                                     ssj, workspace_bytes):
    r = load().tg_gemm_swiglu_quant_fp8_plan_ws(op, M, N, K, A, sam, sak, Bg, Bu, sbk, sbn, Q,
                                                sqm, S, ssm, ssj, workspace_bytes)
    return None if r is None else r.decode()


def _offsets(offsets):
    """A host int64 array of the G + 1 group row offsets (kept alive by the
    caller for the duration of the call)."""
    import numpy as np
    return np.ascontiguousarray(offsets, dtype=np.int64)


def tg_gemm_grouped_f16(G, offsets, N, K, A, lda, B, ldb, sbg, C, ldc, stream=0):
    off = _offsets(offsets)
    return _check(load().tg_gemm_grouped_f16(G, off.ctypes.data, N, K, A, lda, B, ldb, sbg, C,
                                             ldc, stream))


def tg_gemm_grouped_bf16(G, offsets, N, K, A, lda, B, ldb, sbg, C, ldc, stream=0):
    off = _offsets(offsets)
    return _check(load().tg_gemm_grouped_bf16(G, off.ctypes.data, N, K, A, lda, B, ldb, sbg, C,
                                              ldc, stream))


def tg_gemm_grouped_plan(G, offsets, N, K, A, lda, B, ldb, sbg, C, ldc):
    off = _offsets(offsets)
    r = load().tg_gemm_grouped_plan(G, off.ctypes.data, N, K, A, lda, B, ldb, sbg, C, ldc)
    return None if r is None else r.decode()


def tg_gemm_grouped_fp8_blockscaled(G, offsets, N, K, A, lda, SA, ssam, ssak, B, ldb, sbg, SB,
                                    ssbn, ssbk, ssbg, C, ldc, stream=0):
    off = _offsets(offsets)
    return _check(load().tg_gemm_grouped_fp8_blockscaled(G, off.ctypes.data, N, K, A, lda, SA,
                                                         ssam, ssak, B, ldb, sbg, SB, ssbn, ssbk,
                                                         ssbg, C, ldc, stream))


def tg_gemm_grouped_fp8_plan(G, offsets, N, K, A, lda, SA, ssam, ssak, B, ldb, sbg, SB, ssbn,
                             ssbk, ssbg, C, ldc):
    off = _offsets(offsets)
    r = load().tg_gemm_grouped_fp8_plan(G, off.ctypes.data, N, K, A, lda, SA, ssam, ssak, B, ldb,
                                        sbg, SB, ssbn, ssbk, ssbg, C, ldc)
    return None if r is None else r.decode()


def tg_gemm_plan(op, M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn):
    r = load().tg_gemm_plan(op, M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn)
    return None if r is None else r.decode()


# ------------------------------------------------------------ torch helpers

def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _mnk(A, B, C):
    """(M, N, K) and element strides from A (M x K), B (K x N), C (M x N) views."""
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    return M, N, K


def gemm_t(A, B, C, stream=None, plan_only=False):
    """C = A @ B for fp16 / bf16 torch tensors (B may be any strided K x N view,
    e.g. W.t() of an N x K weight).  Runs on `stream` (default: current)."""
    import torch
    M, N, K = _mnk(A, B, C)
    if not (A.dtype == B.dtype == C.dtype) or A.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("gemm_t: A, B, C must all be float16 or all bfloat16")
    args = (M, N, K, A.data_ptr(), A.stride(0), A.stride(1), B.data_ptr(), B.stride(0),
            B.stride(1), C.data_ptr(), C.stride(0), C.stride(1))
    op = OP_F16 if A.dtype == torch.float16 else OP_BF16
    if plan_only:
        return tg_gemm_plan(op, *args)
    fn = tg_gemm_f16 if op == OP_F16 else tg_gemm_bf16
    return fn(*args, _stream_handle(stream))


def gemm_fp8_blockscaled_t(A, SA, B, SB, C, stream=None, plan_only=False):
    """C (bf16, M x N) = block-scaled product of e4m3fn codes A (M x K) and
    B (K x N view) with fp32 scales SA (M x ceil(K/128)) and
    SB (ceil(N/128) x ceil(K/128)).  Code tensors may be uint8 or float8_e4m3fn."""
    M, N, K = _mnk(A, B, C)
    if plan_only:
        return tg_gemm_plan(OP_FP8, M, N, K, A.data_ptr(), A.stride(0), A.stride(1),
                            B.data_ptr(), B.stride(0), B.stride(1), C.data_ptr(), C.stride(0),
                            C.stride(1))
    return tg_gemm_fp8_blockscaled(M, N, K, A.data_ptr(), A.stride(0), A.stride(1),
                                   SA.data_ptr(), SA.stride(0), SA.stride(1),
                                   B.data_ptr(), B.stride(0), B.stride(1),
                                   SB.data_ptr(), SB.stride(0), SB.stride(1),
                                   C.data_ptr(), C.stride(0), C.stride(1), _stream_handle(stream))
