"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
library through its C-ABI binding, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import dense_tiled_gemm_03_amd as tg
import oracle

CANARY = 0x7BAD  # a finite fp16 / bf16 pattern the kernels never write by chance


def log(msg):
    """Names the case before each GPU step (flushed, so a crash still shows it)."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    """Raw codes to the GPU (int16 for 16-bit codes, uint8 for fp8, fp32 scales)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def alloc_c(M: int, N: int, scm: int | None = None, guard: int = 64):
    """C buffer with a guard band of canaries before and after, plus canaries
    in the padding columns when scm > N.  Returns (buffer, offset, scm)."""
    scm = N if scm is None else scm
    rows_span = (M - 1) * scm + N if M > 0 else 0
    buf = torch.full((guard + rows_span + guard,), CANARY, dtype=torch.int16, device="cuda")
    return buf, guard, scm


def c_view(buf, off, M, N, scm) -> np.ndarray:
    h = buf.cpu().numpy().view(np.uint16)
    out = np.empty((M, N), np.uint16)
    for i in range(M):
        out[i] = h[off + i * scm: off + i * scm + N]
    return out


def check_guards(buf, off, M, N, scm):
    h = buf.cpu().numpy().view(np.uint16)
    span = (M - 1) * scm + N if M > 0 else 0
    assert np.all(h[:off] == CANARY), "write before C"
    assert np.all(h[off + span:] == CANARY), "write after C"
    if scm > N:
        for i in range(M - 1):
            gap = h[off + i * scm + N: off + (i + 1) * scm]
            assert np.all(gap == CANARY), f"write into padding after row {i}"


class Workspace:
    """A caller-owned workspace for the *_ws entry points: zero-filled device
    memory (the completion counters must start at zero), 256-byte aligned."""

    COUNTER_BYTES = 16384

    def __init__(self, nbytes: int):
        self.nbytes = int(nbytes)
        self.buf = torch.zeros(self.nbytes + 256, dtype=torch.uint8, device="cuda")
        self.ptr = (self.buf.data_ptr() + 255) & ~255
        self.off = self.ptr - self.buf.data_ptr()

    def counters_zero(self) -> bool:
        n = min(self.nbytes, self.COUNTER_BYTES)
        return bool(torch.all(self.buf[self.off:self.off + n] == 0).item())


def run16(fmt: str, M, N, K, A, sam, sak, B, sbk, sbn, scm=None, a_off=0, b_off=0,
          stream=None, ws=None):
    """Call tg_gemm_f16 / tg_gemm_bf16 on device tensors A, B (codes, element
    offsets a_off / b_off); returns (C codes M x N, plan name).  Checks guards.
    ws=True: call tg_gemm_f16_ws / tg_gemm_bf16_ws with a fresh zeroed
    workspace of the size the split plan asks for; ws=<Workspace>: with that
    one.  After a workspace call its counters must be zero again."""
    buf, off, scm = alloc_c(M, N, scm)
    esz = 2
    args = (M, N, K, A.data_ptr() + a_off * esz, sam, sak, B.data_ptr() + b_off * esz, sbk, sbn,
            buf.data_ptr() + off * esz, scm, 1)
    op = tg.OP_BF16 if fmt == "bf16" else tg.OP_F16
    st = torch.cuda.current_stream().cuda_stream if stream is None else stream
    if ws is None or ws is False:
        plan = tg.tg_gemm_plan(op, *args)
        fn = tg.tg_gemm_bf16 if fmt == "bf16" else tg.tg_gemm_f16
        fn(*args, st)
    else:
        if ws is True:
            ws = Workspace(tg.tg_gemm_workspace_size(op, *args))
        plan = tg.tg_gemm_plan_ws(op, *args, ws.nbytes)
        fn = tg.tg_gemm_bf16_ws if fmt == "bf16" else tg.tg_gemm_f16_ws
        fn(*args, ws.ptr, ws.nbytes, st)
    torch.cuda.synchronize()
    check_guards(buf, off, M, N, scm)
    if ws is not None and ws is not False:
        assert ws.counters_zero(), "workspace counters left nonzero"
    return c_view(buf, off, M, N, scm), plan


def run_fp8(M, N, K, A, sam, sak, SA, ssam, ssak, B, sbk, sbn, SB, ssbn, ssbk, scm=None,
            ws=None):
    """tg_gemm_fp8_blockscaled on device tensors; returns (C codes, plan).
    ws=True / <Workspace>: tg_gemm_fp8_blockscaled_ws, as run16 does."""
    buf, off, scm = alloc_c(M, N, scm)
    args = (M, N, K, A.data_ptr(), sam, sak, B.data_ptr(), sbk, sbn, buf.data_ptr() + off * 2,
            scm, 1)
    full = (M, N, K, A.data_ptr(), sam, sak, SA.data_ptr(), ssam, ssak, B.data_ptr(), sbk, sbn,
            SB.data_ptr(), ssbn, ssbk, buf.data_ptr() + off * 2, scm, 1)
    st = torch.cuda.current_stream().cuda_stream
    if ws is None or ws is False:
        plan = tg.tg_gemm_plan(tg.OP_FP8, *args)
        tg.tg_gemm_fp8_blockscaled(*full, st)
    else:
        if ws is True:
            ws = Workspace(tg.tg_gemm_workspace_size(tg.OP_FP8, *args))
        plan = tg.tg_gemm_plan_ws(tg.OP_FP8, *args, ws.nbytes)
        tg.tg_gemm_fp8_blockscaled_ws(*full, ws.ptr, ws.nbytes, st)
    torch.cuda.synchronize()
    check_guards(buf, off, M, N, scm)
    if ws is not None and ws is not False:
        assert ws.counters_zero(), "workspace counters left nonzero"
    return c_view(buf, off, M, N, scm), plan


def assert_within_bound(out_fmt: str, c_codes: np.ndarray, C_ref: np.ndarray, S: np.ndarray,
                        what: str = ""):
    """|C_gpu - C_ref| <= c * S per element (c = 4*2^-8 bf16, 4*2^-11 fp16)."""
    got = oracle.decode(out_fmt, c_codes)
    err = np.abs(got - C_ref)
    tol = oracle.bound(out_fmt, S)
    bad = ~(err <= tol)
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements outside the bound; first at ({i},{j}):"
                             f" got {got[i, j]!r} ref {C_ref[i, j]!r} tol {tol[i, j]!r}")
    ratio = float(np.max(err / np.where(tol > 0, tol, 1.0))) if err.size else 0.0
    return ratio


def assert_bit_exact(out_fmt: str, c_codes: np.ndarray, C_ref: np.ndarray, what: str = ""):
    want = oracle.round_to(out_fmt, C_ref)
    bad = c_codes != want
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} codes differ; first at ({i},{j}): "
                             f"got {c_codes[i, j]:#06x} want {want[i, j]:#06x} "
                             f"(ref {C_ref[i, j]!r})")
