"""Pins of the CPU oracle against things other than itself (no GPU).

Each test checks the oracle against mathematics it does not share code with: exact
rational arithmetic, identity / permutation matrices, all-ones sums, rank-one closed
forms, hand-worked fixtures in tests/golden, and the library casts of numpy / torch.
A plausible slip in the oracle (a dropped term, a transposed operand, a wrong leading
dimension, alpha/beta swapped, truncation instead of round-to-nearest-even) fails at
least one of them.
"""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from tiled_stage_software_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


def _store(mat: np.ndarray, col: bool, ld_pad: int = 0):
    """Lay out a float64 (R, C) matrix in a flat array (row- or column-major, padded ld)
    with NaN padding; independent of the inputs module on purpose."""
    R, C = mat.shape
    ld = (R if col else C) + ld_pad
    n = ((C - 1) * ld + R) if col else ((R - 1) * ld + C)
    s = np.full(max(n, 0), np.nan)
    for r in range(R):
        for c in range(C):
            s[c * ld + r if col else r * ld + c] = mat[r, c]
    return s, ld


def _exact(A, B, alpha, beta, C0):
    M, K = A.shape
    N = B.shape[1]
    out = [[None] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = sum((Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K)), Fraction(0))
            v = Fraction(alpha) * s
            if beta != 0:
                v += Fraction(beta) * Fraction(float(C0[i, j]))
            out[i][j] = v
    return out


@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (4, 4, 4), (2, 3, 1), (5, 1, 6)])
@pytest.mark.parametrize("ab", [(1.0, 0.0), (0.5, 1.0), (-2.0, 0.5)])
@pytest.mark.parametrize("lay", LAYOUTS)
def test_exact_rationals(oracle, shape, ab, lay):
    """Brute force against exact rational arithmetic, every layout, padded ld."""
    M, N, K = shape
    alpha, beta = ab
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    A = rng.standard_normal((M, K))
    B = rng.standard_normal((K, N))
    C0 = rng.standard_normal((M, N))
    a, lda = _store(A, lay[0], 3)
    b, ldb = _store(B, lay[1], 2)
    c0, ldc = _store(C0, False, 1)
    got = oracle.gemm_f64(lay[0], lay[1], M, N, K, alpha, a, lda, b, ldb, beta, c0, ldc)
    ex = _exact(A, B, alpha, beta, C0)
    for i in range(M):
        for j in range(N):
            scale = abs(alpha) * sum(abs(A[i, k] * B[k, j]) for k in range(K)) + abs(beta * C0[i, j])
            assert abs(Fraction(got[i, j]) - ex[i][j]) <= Fraction(4 * (K + 2) * 2.0 ** -53 * scale)


def test_beta_zero_never_reads_c(oracle):
    A = np.arange(6, dtype=np.float64).reshape(2, 3)
    B = np.arange(12, dtype=np.float64).reshape(3, 4)
    a, lda = _store(A, False)
    b, ldb = _store(B, False)
    c0 = np.full(8, np.nan)
    got = oracle.gemm_f64(False, False, 2, 4, 3, 1.0, a, lda, b, ldb, 0.0, c0, 4)
    assert np.array_equal(got, A @ B)


@pytest.mark.parametrize("lay", LAYOUTS)
def test_identity_and_permutation(oracle, lay):
    """A*I = A, I*B = B, P*B permutes rows, A*P permutes columns -- exactly."""
    rng = np.random.default_rng(7)
    M, K, N = 5, 7, 6
    A = rng.standard_normal((M, K))
    B = rng.standard_normal((K, N))
    a, lda = _store(A, lay[0], 1)
    b, ldb = _store(B, lay[1], 2)
    I_k, ldi = _store(np.eye(K), lay[1])
    assert np.array_equal(oracle.gemm_f64(lay[0], lay[1], M, K, K, 1.0, a, lda, I_k, ldi), A)
    I_k2, ldi2 = _store(np.eye(K), lay[0])
    assert np.array_equal(oracle.gemm_f64(lay[0], lay[1], K, N, K, 1.0, I_k2, ldi2, b, ldb), B)
    perm = rng.permutation(K)
    P = np.eye(K)[perm]                       # (P @ B)[i] = B[perm[i]]
    p, ldp = _store(P, lay[0])
    assert np.array_equal(oracle.gemm_f64(lay[0], lay[1], K, N, K, 1.0, p, ldp, b, ldb), B[perm])
    p2, ldp2 = _store(P, lay[1])               # (A @ P)[:, j] = A[:, inv[j]]
    inv = np.argsort(perm)
    assert np.array_equal(oracle.gemm_f64(lay[0], lay[1], M, K, K, 1.0, a, lda, p2, ldp2), A[:, inv])


@pytest.mark.parametrize("K", [1, 2, 17, 256, 2049])
def test_all_ones(oracle, K):
    M, N = 3, 5
    a, lda = _store(np.ones((M, K)), False)
    b, ldb = _store(np.ones((K, N)), True)
    assert np.all(oracle.gemm_f64(False, True, M, N, K, 1.0, a, lda, b, ldb) == K)
    c0, ldc = _store(np.ones((M, N)), False)
    got = oracle.gemm_f64(False, True, M, N, K, 0.5, a, lda, b, ldb, 1.0, c0, ldc)
    assert np.all(got == 0.5 * K + 1.0)


def test_rank_one_closed_form(oracle):
    """A = u v^T, B = w z^T  =>  C = (v.w) u z^T."""
    rng = np.random.default_rng(11)
    M, K, N = 9, 33, 7
    u, v, w, z = (rng.standard_normal(n) for n in (M, K, K, N))
    A = np.outer(u, v)
    B = np.outer(w, z)
    for la, lb in LAYOUTS:
        a, lda = _store(A, la)
        b, ldb = _store(B, lb)
        got = oracle.gemm_f64(la, lb, M, N, K, 1.0, a, lda, b, ldb)
        want = float(np.dot(v, w)) * np.outer(u, z)
        assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


def _read_golden(name):
    sections, cur, meta = {}, None, {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.endswith(":"):
                cur = line[:-1]
                sections[cur] = []
            elif ":" in line:
                k, v = line.split(":", 1)
                meta[k.strip()] = float(v)
                cur = None
            else:
                sections[cur].append([float(t) for t in line.split()])
    return meta, {k: np.array(v) for k, v in sections.items()}


def test_golden_hand_worked(oracle):
    meta, s = _read_golden("hand_gemm_2x3x2.txt")
    M, N, K = int(meta["M"]), int(meta["N"]), int(meta["K"])
    for la, lb in LAYOUTS:
        a, lda = _store(s["A"], la)
        b, ldb = _store(s["B"], lb)
        assert np.array_equal(oracle.gemm_f64(la, lb, M, N, K, 1.0, a, lda, b, ldb), s["C_alpha1_beta0"])
        c0, ldc = _store(s["C0"], False)
        got = oracle.gemm_f64(la, lb, M, N, K, meta["alpha"], a, lda, b, ldb, meta["beta"], c0, ldc)
        assert np.array_equal(got, s["C_alpha_beta"])


def test_rows_subset_matches_full(oracle):
    rng = np.random.default_rng(3)
    M, N, K = 37, 19, 23
    A = rng.standard_normal((M, K))
    B = rng.standard_normal((K, N))
    for la, lb in LAYOUTS:
        a, lda = _store(A, la, 2)
        b, ldb = _store(B, lb, 1)
        full = oracle.gemm_f64(la, lb, M, N, K, 1.0, a, lda, b, ldb)
        rows = [36, 0, 5, 5, 17]
        assert np.array_equal(oracle.gemm_f64(la, lb, M, N, K, 1.0, a, lda, b, ldb, rows=rows), full[rows])


def test_empty_shapes(oracle):
    got = oracle.gemm_f64(False, False, 0, 4, 3, 1.0, np.zeros(0), 3, np.zeros(12), 4)
    assert got.shape == (0, 4)
    got = oracle.gemm_f64(False, False, 2, 3, 0, 1.0, np.zeros(0), 1, np.zeros(0), 3)
    assert np.array_equal(got, np.zeros((2, 3)))


# ---------------------------------------------------------------- fp32 FMA-chain model

def _f32_rne(q: Fraction) -> Fraction:
    """Exact rational -> nearest binary32 (ties to even), written with integers only."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    n, rem = divmod(q, quantum)
    n = int(n)
    if rem * 2 > quantum or (rem * 2 == quantum and n % 2 == 1):
        n += 1
    return sign * n * quantum


def _fma_chain_exact(a_row, b_col, alpha, beta, c0):
    acc = Fraction(0)
    for a, b in zip(a_row, b_col):
        acc = _f32_rne(Fraction(float(a)) * Fraction(float(b)) + acc)
    if beta == 0:
        return _f32_rne(Fraction(float(alpha)) * acc)
    return _f32_rne(Fraction(float(alpha)) * acc + _f32_rne(Fraction(float(beta)) * Fraction(float(c0))))


@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("ab", [(1.0, 0.0), (0.5, 1.0), (-3.0, 0.25)])
def test_fma_chain_against_exact_single_roundings(oracle, lay, ab):
    """Every step is one correctly rounded fp32 fma: checked with exact rationals and an
    integer-only round-to-nearest-even, so a mul-then-add or double-rounding bug fails."""
    rng = np.random.default_rng(5)
    M, N, K = 4, 3, 9
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((K, N)).astype(np.float32)
    C0 = rng.standard_normal((M, N)).astype(np.float32)
    a, lda = _store(A.astype(np.float64), lay[0], 1)
    b, ldb = _store(B.astype(np.float64), lay[1], 0)
    got = oracle.sgemm_fma_chain(lay[0], lay[1], M, N, K, ab[0], a.astype(np.float32), lda,
                                 b.astype(np.float32), ldb, ab[1], C0.reshape(-1), N)
    for i in range(M):
        for j in range(N):
            assert Fraction(float(got[i, j])) == _fma_chain_exact(A[i], B[:, j], ab[0], ab[1], C0[i, j])


def test_fma_chain_is_fused():
    """A case where fused and unfused differ: (1+2^-12)^2 - (1+2^-11) = 2^-24 exactly;
    the fp32 product alone rounds the 2^-24 away."""
    from oracle import oracle as o
    x = np.float32(1 + 2.0 ** -12)
    A = np.array([x, np.float32(-(1 + 2.0 ** -11))], dtype=np.float32)
    B = np.array([x, np.float32(1.0)], dtype=np.float32)
    # acc1 = rne(x*x) = 1 + 2^-11 (the 2^-24 is lost); acc2 = rne(-(1+2^-11) + acc1) = 0.
    got = o.sgemm_fma_chain(False, True, 1, 1, 2, 1.0, A, 2, B, 2)
    assert got[0, 0] == 0.0
    # Reverse the order: acc1 = -(1+2^-11); acc2 = rne(x*x + acc1) = 2^-24 (fused).
    got2 = o.sgemm_fma_chain(False, True, 1, 1, 2, 1.0, A[::-1].copy(), 2, B[::-1].copy(), 2)
    assert got2[0, 0] == np.float32(2.0 ** -24)


def test_fma_chain_close_to_fp64(oracle):
    rng = np.random.default_rng(9)
    M, N, K = 16, 24, 512
    A = (rng.random((M, K)) * 2 - 1).astype(np.float32)
    B = (rng.random((K, N)) * 2 - 1).astype(np.float32)
    a32 = A.reshape(-1)
    b32 = B.reshape(-1)
    c = oracle.sgemm_fma_chain(False, False, M, N, K, 1.0, a32, K, b32, N)
    r = oracle.gemm_f64(False, False, M, N, K, 1.0, a32, K, b32, N)
    err = oracle.normalized_error(c, r, K, np.abs(A).max(), np.abs(B).max())
    assert 0 < err < 1e-6


# ---------------------------------------------------------------- rounding / encoding

def test_round_matches_library_casts(oracle):
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 8, 20000),
        rng.standard_normal(2000) * 1e-6,           # f16 subnormal range
        rng.standard_normal(2000) * 1e-40,          # bf16 / fp32 subnormal range
        np.array([0.0, -0.0, 65504.0, 65519.9, 65520.0, 1e39, -1e39, 3.4e38]),
    ])
    # ties: midpoints between consecutive bf16 / f16 values
    t = torch.tensor(rng.standard_normal(5000), dtype=torch.float32).to(torch.bfloat16).double().numpy()
    x = np.concatenate([x, t + np.ldexp(1.0, np.frexp(t)[1] - 9)])
    h = np.float16(rng.standard_normal(5000)).astype(np.float64)
    x = np.concatenate([x, h + np.ldexp(1.0, np.frexp(h)[1] - 12)])
    f32 = oracle.round_to(x, 0)
    assert np.array_equal(f32, x.astype(np.float32).astype(np.float64))
    bf = oracle.round_to(x, 1)
    # torch rounds fp64 -> bf16 directly (single rounding)
    want_bf = torch.tensor(x, dtype=torch.float64).to(torch.bfloat16).double().numpy()
    assert np.array_equal(bf, want_bf)
    f16 = oracle.round_to(x, 2)
    assert np.array_equal(f16, x.astype(np.float16).astype(np.float64))


def test_rne_golden_ties(oracle):
    with open(os.path.join(GOLDEN, "rne_ties.txt"), encoding="utf-8") as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for fmt, k, want in rows:
        got = oracle.round_to([float(k)], 1 if fmt == "bf16" else 2)[0]
        assert got == float(want), (fmt, k, want, got)


def test_encode16_matches_library_bits(oracle):
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-6, 6, 4000),
                        [0.0, -0.0, np.inf, -np.inf, 1e-7, -3e-8, 6e-5]])
    bf = oracle.round_to(x, 1)
    want = torch.tensor(bf, dtype=torch.float64).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.encode16(bf, 1), want)
    h = oracle.round_to(x, 2)
    assert np.array_equal(oracle.encode16(h, 2), h.astype(np.float16).view(np.uint16))


def test_normalized_error_definition(oracle):
    C = np.array([[1.0, 2.0], [3.0, 4.5]])
    R = np.array([[1.0, 2.0], [3.0, 4.0]])
    assert oracle.normalized_error(C, R, 10, 2.0, 0.5) == pytest.approx(0.5 / (10 * 2.0 * 0.5))
    assert oracle.normalized_error(R, R, 0, 0.0, 0.0) == 0.0
    assert oracle.normalized_error(C, R, 0, 1.0, 1.0) == math.inf


def test_oracle_consumes_generated_inputs(oracle):
    """The seeded generator's storage layouts are read the way the oracle documents."""
    for la in (inputs.ROW, inputs.COL):
        for lb in (inputs.ROW, inputs.COL):
            A = inputs.operand(6, 5, la, torch.bfloat16, "int2", 1, ld=9)
            B = inputs.operand(5, 4, lb, torch.bfloat16, "int2", 2, ld=8)
            got = oracle.gemm_f64(la == inputs.COL, lb == inputs.COL, 6, 4, 5, 1.0,
                                  A.storage, A.ld, B.storage, B.ld)
            want = A.logical().double().numpy() @ B.logical().double().numpy()
            assert np.array_equal(got, want)
