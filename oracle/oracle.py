"""Plain CPU oracle for the tiled GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It never imports the HIP library or its
Python binding, and the library never imports it.

What it computes is the GEMM definition (see ``oracle_gemm.c``): per output one fp64
running sum over k ascending, ``out = alpha*sum + beta*C0`` (C0 unread when beta == 0).
The accumulation ``C += A * B`` over K tiles is section 2 ("Thread Block Tile") of the
page "CUTLASS-Cute 初步(6)：CUDA GEMM 计算优化、Multi-Stage 与软流水"; tiling and
stage count only reorder the products (all four pages), so the definition is exact.

Functions:
  gemm_f64        -- the fp64 definition, on the exact (widened) input values.
  sgemm_fma_chain -- fp32 model of one FMA chain per output, k ascending (thread tile,
                     section 4 of the same page); bit-exact target for FP32 VALU kernels.
  round_to        -- IEEE round-to-nearest-even of fp64 values to fp32 / bf16 / f16.
  encode16        -- bf16 / f16 bit patterns of already rounded values.
  normalized_error-- ||C - Cref||_inf / (K * max|A| * max|B|).

Pins (tests/test_oracle_pins.py): exact rational brute force, identity and permutation
matrices, all-ones (C = K), rank-one closed forms, ties in rounding, hand-worked golden
fixtures.  Nothing in the oracle is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

FMT_F32, FMT_BF16, FMT_F16 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, dp, fp = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_float)
        ip = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_gemm_f64.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                        ctypes.c_double, dp, i64, dp, i64,
                                        ctypes.c_double, dp, i64, dp, i64, ip, i64, ctypes.c_int]
        lib.oracle_gemm_f64.restype = ctypes.c_int
        lib.oracle_sgemm_fma_chain.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                               ctypes.c_float, fp, i64, fp, i64,
                                               ctypes.c_float, fp, i64, fp, i64, ip, i64, ctypes.c_int]
        lib.oracle_sgemm_fma_chain.restype = ctypes.c_int
        lib.oracle_round.argtypes = [dp, i64, ctypes.c_int]
        lib.oracle_round.restype = ctypes.c_int
        lib.oracle_encode16.argtypes = [dp, ctypes.POINTER(ctypes.c_uint16), i64, ctypes.c_int]
        lib.oracle_encode16.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = [ctypes.c_int]
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
        return lib


def _as_f64(x) -> np.ndarray:
    """Exact widening of the storage values to fp64 (bf16/f16/fp32 -> fp64 is exact)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor (CPU); widen with the library cast
        import torch
        x = x.detach().to("cpu").to(torch.float64).contiguous().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64)).reshape(-1)


def _as_f32(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):
        import torch
        assert x.dtype == torch.float32
        x = x.detach().to("cpu").contiguous().numpy()
    assert np.asarray(x).dtype == np.float32
    return np.ascontiguousarray(x).reshape(-1)


def _rows_arg(rows, M):
    if rows is None:
        return None, M
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, int(r.size)


def _need(storage: np.ndarray, col: bool, R: int, Cc: int, ld: int, name: str):
    if R == 0 or Cc == 0:
        return
    need = (Cc - 1) * ld + R if col else (R - 1) * ld + Cc
    if storage.size < need:
        raise ValueError(f"{name}: storage holds {storage.size} elements, layout needs {need}")


def max_threads(nthreads: int = 0) -> int:
    return int(_load().oracle_max_threads(int(nthreads)))


def gemm_f64(a_col: bool, b_col: bool, M: int, N: int, K: int, alpha: float,
             A, lda: int, B, ldb: int, beta: float = 0.0, C0=None, ldc0: int = 0,
             rows=None, nthreads: int = 0) -> np.ndarray:
    """fp64 ``alpha*A@B + beta*C0`` on the storage arrays (any float dtype, widened
    exactly).  Returns an (nrows, N) float64 array; with ``rows`` only those C rows."""
    lib = _load()
    a = _as_f64(A)
    b = _as_f64(B)
    _need(a, a_col, M, K, lda, "A")
    _need(b, b_col, K, N, ldb, "B")
    c0 = None
    if beta != 0.0:
        if C0 is None:
            raise ValueError("beta != 0 needs C0")
        c0 = _as_f64(C0)
        _need(c0, False, M, N, ldc0, "C0")
    r, nrows = _rows_arg(rows, M)
    out = np.empty((nrows, max(N, 1)), dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    empty = np.zeros(1, dtype=np.float64)
    rc = lib.oracle_gemm_f64(int(bool(a_col)), int(bool(b_col)), M, N, K, float(alpha),
                             (a if a.size else empty).ctypes.data_as(dp), lda,
                             (b if b.size else empty).ctypes.data_as(dp), ldb,
                             float(beta), (c0 if c0 is not None else empty).ctypes.data_as(dp), ldc0,
                             out.ctypes.data_as(dp), max(N, 1),
                             None if r is None else r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                             nrows, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gemm_f64: bad arguments")
    return out[:, :N]


def sgemm_fma_chain(a_col: bool, b_col: bool, M: int, N: int, K: int, alpha: float,
                    A, lda: int, B, ldb: int, beta: float = 0.0, C0=None, ldc0: int = 0,
                    rows=None, nthreads: int = 0) -> np.ndarray:
    """fp32, one fused-multiply-add chain per output, k ascending (see module doc)."""
    lib = _load()
    a = _as_f32(A)
    b = _as_f32(B)
    _need(a, a_col, M, K, lda, "A")
    _need(b, b_col, K, N, ldb, "B")
    c0 = None
    if beta != 0.0:
        c0 = _as_f32(C0)
        _need(c0, False, M, N, ldc0, "C0")
    r, nrows = _rows_arg(rows, M)
    out = np.empty((nrows, max(N, 1)), dtype=np.float32)
    fp = ctypes.POINTER(ctypes.c_float)
    empty = np.zeros(1, dtype=np.float32)
    rc = lib.oracle_sgemm_fma_chain(int(bool(a_col)), int(bool(b_col)), M, N, K, float(alpha),
                                    (a if a.size else empty).ctypes.data_as(fp), lda,
                                    (b if b.size else empty).ctypes.data_as(fp), ldb,
                                    float(beta), (c0 if c0 is not None else empty).ctypes.data_as(fp), ldc0,
                                    out.ctypes.data_as(fp), max(N, 1),
                                    None if r is None else r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                    nrows, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_sgemm_fma_chain: bad arguments")
    return out[:, :N]


def round_to(x, fmt: int) -> np.ndarray:
    """IEEE round-to-nearest-even of fp64 values to fp32 (0), bf16 (1) or f16 (2);
    the result is returned as fp64 values (exactly representable in the format)."""
    v = np.array(x, dtype=np.float64, copy=True)
    flat = np.ascontiguousarray(v.reshape(-1))
    rc = _load().oracle_round(flat.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), flat.size, int(fmt))
    if rc != 0:
        raise ValueError("unknown format")
    return flat.reshape(v.shape)


def encode16(x, fmt: int) -> np.ndarray:
    """uint16 bit patterns (bf16 fmt=1, f16 fmt=2) of values already rounded to the format."""
    v = np.ascontiguousarray(np.array(x, dtype=np.float64).reshape(-1))
    out = np.empty(v.size, dtype=np.uint16)
    rc = _load().oracle_encode16(v.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                 out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), v.size, int(fmt))
    if rc != 0:
        raise ValueError("unknown format")
    return out.reshape(np.shape(x))


def normalized_error(C, Cref, K: int, max_abs_a: float, max_abs_b: float) -> float:
    """||C - Cref||_inf / (K * max|A| * max|B|); C is the device result widened to
    fp64, Cref the unrounded fp64 oracle.  A zero denominator demands exact equality
    (returns 0.0 if equal, inf otherwise)."""
    C = np.asarray(C, dtype=np.float64)
    Cref = np.asarray(Cref, dtype=np.float64)
    if C.shape != Cref.shape:
        raise ValueError(f"shape mismatch {C.shape} vs {Cref.shape}")
    if C.size == 0:
        return 0.0
    if np.isnan(C).any() or np.isnan(Cref).any():
        same = np.array_equal(np.isnan(C), np.isnan(Cref)) and np.array_equal(C[~np.isnan(C)], Cref[~np.isnan(Cref)])
        return 0.0 if same else float("inf")
    diff = float(np.max(np.abs(C - Cref)))
    den = float(K) * float(max_abs_a) * float(max_abs_b)
    if den == 0.0:
        return 0.0 if diff == 0.0 else float("inf")
    return diff / den
