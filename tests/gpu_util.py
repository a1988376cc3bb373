"""Helpers for the GPU parity tests: run the HIP library through the C ABI on seeded
inputs and compute the oracle on the same inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import oracle
from tiled_stage_software_amd import inputs, libgemm as lg

DEV = torch.device("cuda:0")
TOL = {"f32": 1e-6, "bf16": 1e-5, "f16": 1e-5}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


DT_CODE = {"f32": lg.GEMM_F32, "bf16": lg.GEMM_BF16, "f16": lg.GEMM_F16}


def workspace_bytes(p: inputs.Problem, ldc: int, A_ptr: int, B_ptr: int, C_ptr: int, **opts) -> tuple:
    """(bytes, plan) that gemm_*_ws needs for this problem (gemm_workspace_size)."""
    s, n, plan = lg.gemm_workspace_size(DT_CODE[p.dtype], DT_CODE[p.out], p.A.layout, p.B.layout, p.M, p.N, p.K,
                                        p.alpha, A_ptr, p.A.ld, B_ptr, p.B.ld, p.beta, C_ptr, ldc,
                                        lg._opts(**opts))
    lg.check(s)
    return n, plan


def gpu_gemm(p: inputs.Problem, ldc: int | None = None, c_fill=None, ws=None, **opts):
    """Run C = alpha*A*B + beta*C0 on the GPU; returns the C storage (CPU tensor, M x ldc)
    and the status.  c_fill: value the C buffer holds before the call when beta == 0.
    ws: None = gemm_*_ex; "auto" = gemm_*_ws with the workspace gemm_workspace_size asks
    for (NaN-filled, so that stale bytes would show); an int = a workspace of that many
    bytes; a device tensor = that workspace."""
    M, N, K = p.M, p.N, p.K
    ldc = ldc or max(N, 1)
    out_dt = inputs.DTYPES[p.out]
    if p.C0 is not None:
        C0 = p.C0
        if C0.ld != ldc:
            C0 = inputs.place(C0.logical(), inputs.ROW, ldc)
        Cst = C0.storage.clone()
    else:
        fill = float("nan") if c_fill is None else c_fill
        Cst = torch.full((max(M * ldc, 1),), fill, dtype=out_dt)
    Cd = Cst.to(DEV)
    Ad = p.A.storage.to(DEV) if p.A.storage.numel() else torch.empty(1, dtype=p.A.storage.dtype, device=DEV)
    Bd = p.B.storage.to(DEV) if p.B.storage.numel() else torch.empty(1, dtype=p.B.storage.dtype, device=DEV)
    wptr, wbytes = 0, 0
    if ws is not None:
        if isinstance(ws, torch.Tensor):
            W, wbytes = ws, ws.numel() * ws.element_size()
        else:
            wbytes = int(ws) if ws != "auto" else \
                workspace_bytes(p, ldc, Ad.data_ptr(), Bd.data_ptr(), Cd.data_ptr(), **opts)[0]
            W = torch.full((wbytes // 2 + 1,), float("nan"), dtype=torch.bfloat16, device=DEV)
        wptr = W.data_ptr()
    s = lg.gemm_operands(p.dtype, p.out, p.A.layout, p.B.layout, M, N, K, p.alpha,
                         Ad.data_ptr(), p.A.ld, Bd.data_ptr(), p.B.ld, p.beta, Cd.data_ptr(), ldc,
                         torch.cuda.current_stream().cuda_stream, ws_ptr=wptr, ws_bytes=wbytes, **opts)
    if s != lg.GEMM_OK:
        raise lg.GemmError(s, lg.gemm_last_error())
    torch.cuda.synchronize()
    return Cd.cpu(), ldc


def c_logical(Cst: torch.Tensor, M: int, N: int, ldc: int) -> torch.Tensor:
    if M == 0 or N == 0:
        return Cst.new_empty((M, N))
    return Cst[: (M - 1) * ldc + N].as_strided((M, N), (ldc, 1))


def oracle_ref(p: inputs.Problem, rows=None) -> np.ndarray:
    return oracle.gemm_f64(p.A.layout == inputs.COL, p.B.layout == inputs.COL, p.M, p.N, p.K, p.alpha,
                           p.A.storage, p.A.ld, p.B.storage, p.B.ld, p.beta,
                           None if p.C0 is None else p.C0.storage, 0 if p.C0 is None else p.C0.ld, rows=rows)


def max_abs(op: inputs.Operand) -> float:
    if op.rows == 0 or op.cols == 0:
        return 0.0
    return float(op.logical().abs().max().item())


HALF_ULP_BITS = {"bf16": 8, "f16": 11}   # significand bits (hidden bit included)


def output_rounding_allowance(ref: np.ndarray, out: str) -> np.ndarray:
    """Half an ulp of the 16-bit output format at |ref| (taken at the upper end of the
    binade): the error that rounding even the exact result to the output type makes.
    Zero for fp32 output, where the tolerance is applied to the unrounded result."""
    if out not in HALF_ULP_BITS:
        return np.zeros_like(ref)
    p = HALF_ULP_BITS[out]
    emin = -126 if out == "bf16" else -14
    a = np.abs(ref) * (1.0 + 2.0 ** (1 - p))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - p).astype(np.int64))   # half of 2^(e - p + 1)


def err_vs_oracle(p: inputs.Problem, C: torch.Tensor, rows=None, raw: bool = False) -> float:
    """Normalised error ||C - Cref||_inf / (K max|A| max|B|) of the device result (rows
    subset optional) against the unrounded oracle.  For bf16 / f16 output the half-ulp
    that rounding the exact result to the output type costs is taken off each element
    first (unless raw=True): the tolerance bounds the fp32 accumulation, not the
    output format."""
    ref = oracle_ref(p, rows)
    got = C.double().numpy() if rows is None else C[rows].double().numpy()
    if not raw and p.out in HALF_ULP_BITS and got.size:
        if np.isnan(got).any():
            return float("inf")
        d = np.maximum(np.abs(got - ref) - output_rounding_allowance(ref, p.out), 0.0)
        den = p.K * max_abs(p.A) * max_abs(p.B)
        return float(d.max()) / den if den else (0.0 if d.max() == 0 else float("inf"))
    return oracle.normalized_error(got, ref, p.K, max_abs(p.A), max_abs(p.B))


def sample_rows(M: int, block: int = 256):
    """One row in every 256-row block at a varying offset, plus the first and last rows."""
    rows = {0, M - 1}
    for b in range((M + block - 1) // block):
        r = b * block + (b * 37) % block
        if r < M:
            rows.add(r)
    return sorted(rows)


def expected_rounded(exact: np.ndarray, out: str) -> np.ndarray:
    """Exact (representable-in-fp64) results rounded to the output type with RNE, as the
    oracle defines it."""
    fmt = {"f32": oracle.FMT_F32, "bf16": oracle.FMT_BF16, "f16": oracle.FMT_F16}[out]
    return oracle.round_to(exact, fmt)


def widened(p: inputs.Problem):
    """The operands' storage widened (exactly) to fp64 once, for repeated oracle calls."""
    a = p.A.storage.double().numpy()
    b = p.B.storage.double().numpy()
    c = None if p.C0 is None else p.C0.storage.double().numpy()
    return a, b, c


def whole_matrix(p: inputs.Problem, C: torch.Tensor, exact: bool = False, batch: int = 512) -> float:
    """Every element of the device result C (M x N, CPU) against the oracle, computed in
    batches of rows so that host memory stays bounded.  exact=False: the normalised error
    ||C - Cref||_inf / (K max|A| max|B|) over the whole matrix, raw (the output rounding
    included).  exact=True: the number of elements that differ from the exact result
    rounded (RNE) to the output type."""
    a, b, c = widened(p)
    la, lb = p.A.layout == inputs.COL, p.B.layout == inputs.COL
    amax, bmax = max_abs(p.A), max_abs(p.B)
    worst, bad = 0.0, 0
    for r0 in range(0, p.M, batch):
        rows = list(range(r0, min(p.M, r0 + batch)))
        ref = oracle.gemm_f64(la, lb, p.M, p.N, p.K, p.alpha, a, p.A.ld, b, p.B.ld, p.beta, c,
                              0 if p.C0 is None else p.C0.ld, rows=rows)
        got = C[r0:r0 + len(rows)].double().numpy()
        if exact:
            bad += int(np.count_nonzero(got != expected_rounded(ref, p.out)))
        else:
            worst = max(worst, oracle.normalized_error(got, ref, p.K, amax, bmax))
    return float(bad) if exact else worst
