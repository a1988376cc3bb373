"""Seeded synthetic inputs for the GEMM workloads.

This module only draws numbers and lays them out in memory; it holds none of the
GEMM's arithmetic.  Both the HIP library's tests/benchmark and the CPU oracle consume
what it produces, so neither side generates its own inputs.

Recipe: values are drawn in fp32 from ``torch.Generator().manual_seed(seed)`` (uniform
on [-1, 1) as ``2*rand - 1``, or normal as ``randn * std``) and cast with
round-to-nearest-even to the operand dtype.  Seeds are ``1000*c + o`` for workload c
(1..5) and operand o (1 = A, 2 = B, 3 = C0).  Padding between a row's last element and
the next row (leading dimension larger than the logical extent) is filled with NaN, so
a kernel that reads outside the logical matrix poisons its result.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

ROW, COL = 0, 1

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclasses.dataclass
class Operand:
    """A matrix of logical shape (rows, cols) stored in a flat tensor.

    row-major: element (r, c) at storage[r*ld + c]; column-major: storage[c*ld + r].
    """
    storage: torch.Tensor
    rows: int
    cols: int
    layout: int
    ld: int

    def logical(self) -> torch.Tensor:
        """(rows, cols) strided view of the storage (no copy)."""
        if self.rows == 0 or self.cols == 0:
            return self.storage.new_empty((self.rows, self.cols))
        if self.layout == ROW:
            return self.storage.as_strided((self.rows, self.cols), (self.ld, 1))
        return self.storage.as_strided((self.rows, self.cols), (1, self.ld))

    def to(self, device) -> "Operand":
        return dataclasses.replace(self, storage=self.storage.to(device))


def storage_size(rows: int, cols: int, layout: int, ld: int) -> int:
    if rows == 0 or cols == 0:
        return 0
    return (rows - 1) * ld + cols if layout == ROW else (cols - 1) * ld + rows


def place(values: torch.Tensor, layout: int, ld: Optional[int] = None, pad=float("nan"),
          extra: int = 0) -> Operand:
    """Lay a (rows, cols) tensor out in memory with the given layout and leading
    dimension; ``extra`` elements of padding are appended (also filled with ``pad``)."""
    rows, cols = values.shape
    if ld is None:
        ld = cols if layout == ROW else rows
    ld = max(int(ld), 1)
    n = storage_size(rows, cols, layout, ld) + extra
    storage = torch.full((n,), pad, dtype=values.dtype) if values.dtype.is_floating_point \
        else torch.zeros((n,), dtype=values.dtype)
    op = Operand(storage, rows, cols, layout, ld)
    if rows and cols:
        op.logical().copy_(values)
    return op


def draw(rows: int, cols: int, dist: str, seed: int, dtype: torch.dtype, std: float = 1.0) -> torch.Tensor:
    """Seeded fp32 draw of a (rows, cols) matrix, cast (RNE) to ``dtype``."""
    g = torch.Generator().manual_seed(int(seed))
    if dist == "uniform":
        v = torch.rand((rows, cols), generator=g, dtype=torch.float32) * 2.0 - 1.0
    elif dist == "normal":
        v = torch.randn((rows, cols), generator=g, dtype=torch.float32) * std
    elif dist == "ones":
        v = torch.ones((rows, cols), dtype=torch.float32)
    elif dist.startswith("int"):
        # small integers in [-m, m]: every product and partial sum is an exact fp32 integer
        m = int(dist[3:] or 2)
        v = torch.randint(-m, m + 1, (rows, cols), generator=g).to(torch.float32)
    else:
        raise ValueError(dist)
    return v.to(dtype)


def operand(rows: int, cols: int, layout: int, dtype: torch.dtype, dist: str, seed: int,
            ld: Optional[int] = None, std: float = 1.0) -> Operand:
    return place(draw(rows, cols, dist, seed, dtype, std), layout, ld)


# The five workloads.  Sizes, layouts, value distributions and alpha/beta are those the
# product is measured on; "NT" = A row-major and B column-major (both K-contiguous).
CONFIGS = {
    "c1": dict(index=1, name="fp32 256^3 NN, single vs double buffer", dtype="f32", out="f32",
               M=256, N=256, K=256, la=ROW, lb=ROW, dist="uniform", std=1.0, alpha=1.0, beta=0.0),
    "c2": dict(index=2, name="fp32 4096^3 NN, 128x64 tile, nStage 1/2/3", dtype="f32", out="f32",
               M=4096, N=4096, K=4096, la=ROW, lb=ROW, dist="uniform", std=1.0, alpha=1.0, beta=0.0),
    "c3": dict(index=3, name="bf16 8192^3 NT -> bf16", dtype="bf16", out="bf16",
               M=8192, N=8192, K=8192, la=ROW, lb=COL, dist="normal", std=1.0, alpha=1.0, beta=0.0),
    "c4": dict(index=4, name="f16 16384x14336x4096 NT -> f16 (MLP shape)", dtype="f16", out="f16",
               M=16384, N=14336, K=4096, la=ROW, lb=COL, dist="normal", std=1.0 / 64.0,
               alpha=1.0, beta=0.0),
    "c5": dict(index=5, name="bf16 4000x3000x2049 NN, fp32 C, alpha 0.5 beta 1", dtype="bf16", out="f32",
               M=4000, N=3000, K=2049, la=ROW, lb=ROW, dist="uniform", std=1.0, alpha=0.5, beta=1.0),
}


@dataclasses.dataclass
class Problem:
    M: int
    N: int
    K: int
    A: Operand
    B: Operand
    C0: Optional[Operand]
    alpha: float
    beta: float
    dtype: str
    out: str


def make_problem(cfg: dict, M=None, N=None, K=None, dist=None, lda=None, ldb=None) -> Problem:
    """Inputs of a workload (optionally at other sizes / value distributions)."""
    M = cfg["M"] if M is None else M
    N = cfg["N"] if N is None else N
    K = cfg["K"] if K is None else K
    dist = cfg["dist"] if dist is None else dist
    c = cfg["index"]
    dt = DTYPES[cfg["dtype"]]
    A = operand(M, K, cfg["la"], dt, dist, 1000 * c + 1, ld=lda, std=cfg["std"])
    B = operand(K, N, cfg["lb"], dt, dist, 1000 * c + 2, ld=ldb, std=cfg["std"])
    C0 = None
    if cfg["beta"] != 0.0:
        C0 = operand(M, N, ROW, DTYPES[cfg["out"]], "uniform", 1000 * c + 3)
    return Problem(M, N, K, A, B, C0, cfg["alpha"], cfg["beta"], cfg["dtype"], cfg["out"])
