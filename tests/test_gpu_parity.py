"""Parity of the HIP library (through the C ABI) with the CPU oracle, on an MI355X.

Bars: bit-exact where the exact result is representable (identity, permutation,
all-ones, small-integer inputs) and across stage counts / repeated runs;
||C - Cref||_inf / (K max|A| max|B|) <= 1e-6 (fp32) or 1e-5 (bf16 / f16 inputs) on
random inputs; the fp32 VALU path equal bit for bit to one fmaf chain per output.
"""
import math

import numpy as np
import pytest
import torch

from gpu_util import (DEV, TOL, say, gpu_gemm, c_logical, oracle_ref, err_vs_oracle, sample_rows,
                      expected_rounded, max_abs, whole_matrix)
from oracle import oracle
from tiled_stage_software_amd import inputs, libgemm as lg

pytestmark = pytest.mark.gpu

ROW, COL = inputs.ROW, inputs.COL
K_VALU_RING, K_VALU_STAGED = lg.GEMM_KERNEL_VALU_RING, lg.GEMM_KERNEL_VALU_STAGED
K_MFMA_RING, K_MFMA_STAGED = lg.GEMM_KERNEL_MFMA_RING, lg.GEMM_KERNEL_MFMA_STAGED


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lg.load()  # fails loudly if the library is missing
    torch.zeros(1, device=DEV)


def problem(dtype, out, M, N, K, la, lb, dist="uniform", alpha=1.0, beta=0.0, seed=1, lda=None, ldb=None,
            std=1.0):
    dt = inputs.DTYPES[dtype]
    A = inputs.operand(M, K, la, dt, dist, seed * 10 + 1, ld=lda, std=std)
    B = inputs.operand(K, N, lb, dt, dist, seed * 10 + 2, ld=ldb, std=std)
    C0 = inputs.operand(M, N, ROW, inputs.DTYPES[out], "uniform", seed * 10 + 3) if beta != 0.0 else None
    return inputs.Problem(M, N, K, A, B, C0, alpha, beta, dtype, out)


def run(p, **opts):
    C, ldc = gpu_gemm(p, **opts)
    return c_logical(C, p.M, p.N, ldc)


def same_values(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Equal as numbers (+0 == -0), NaN where NaN."""
    x, y = a.double().numpy(), b.double().numpy()
    return x.shape == y.shape and np.array_equal(np.isnan(x), np.isnan(y)) and np.array_equal(
        np.nan_to_num(x), np.nan_to_num(y))


# --------------------------------------------------------------- exact special cases

FAMILIES = [  # (dtype, out, la, lb, kernel, tile, nstage, M, N, K): M, N, K >= the tile
    ("f32", "f32", ROW, ROW, K_VALU_RING, 1, 2, 256, 192, 128),
    ("f32", "f32", ROW, ROW, K_VALU_RING, 5, 3, 256, 192, 128),
    ("f32", "f32", ROW, ROW, K_VALU_RING, 6, 2, 256, 192, 128),
    ("f32", "f32", ROW, ROW, K_VALU_RING, 10, 2, 256, 256, 128),
    ("f32", "f32", ROW, ROW, K_VALU_RING, 11, 4, 256, 384, 128),
    ("f32", "f32", ROW, ROW, K_VALU_RING, 3, 4, 96, 64, 48),
    ("f32", "f32", COL, COL, K_VALU_STAGED, 1, 2, 130, 70, 45),
    ("bf16", "bf16", ROW, COL, K_MFMA_RING, 1, 2, 512, 512, 256),
    ("f16", "f16", ROW, COL, K_MFMA_RING, 3, 2, 256, 384, 128),
    ("bf16", "bf16", ROW, COL, K_MFMA_RING, 2, 4, 256, 512, 256),
    ("bf16", "bf16", ROW, COL, K_MFMA_RING, 24, 2, 512, 256, 256),
    ("bf16", "bf16", ROW, COL, K_MFMA_RING, 31, 2, 512, 256, 256),
    ("f16", "f32", ROW, COL, K_MFMA_RING, 31, 1, 256, 512, 256),
    ("bf16", "f32", ROW, COL, K_MFMA_RING, 32, 2, 384, 256, 256),
    ("f16", "f32", ROW, COL, K_MFMA_RING, 26, 2, 256, 512, 256),
    ("bf16", "bf16", ROW, COL, K_MFMA_RING, 25, 4, 256, 256, 256),
    ("f16", "f16", ROW, COL, K_MFMA_RING, 29, 1, 384, 256, 256),
    ("bf16", "f32", ROW, ROW, K_MFMA_RING, 30, 2, 384, 512, 256),
    ("f16", "f16", ROW, ROW, K_MFMA_RING, 30, 1, 256, 256, 256),
    ("bf16", "f32", ROW, ROW, K_MFMA_STAGED, 1, 2, 200, 136, 77),
    ("f16", "f16", COL, ROW, K_MFMA_STAGED, 1, 1, 129, 257, 40),
]


def _fid(f):
    return f"{f[0]}-{f[1]}-{'RC'[f[2]]}{'RC'[f[3]]}-k{f[4]}-t{f[5]}-s{f[6]}"


@pytest.mark.parametrize("fam", FAMILIES, ids=_fid)
def test_identity_and_permutation_exact(fam):
    """A@P permutes columns, I@B = B, P@B permutes rows: exact in every precision, so a
    misplaced fragment, lane or swizzle shows up as a wrong element."""
    dtype, out, la, lb, kern, tile, S, M, N, K = fam
    dt, odt = inputs.DTYPES[dtype], inputs.DTYPES[out]
    say(f"[identity/permutation] {_fid(fam)}")
    g = torch.Generator().manual_seed(5)
    Avals = torch.randint(-8, 9, (M, K), generator=g).to(torch.float32) / 4
    Bvals = torch.randint(-8, 9, (K, N), generator=g).to(torch.float32) / 4
    perm = torch.randperm(K, generator=g)
    P = torch.zeros(K, K)
    P[torch.arange(K), perm] = 1.0            # (A @ P)[:, perm[i]] = A[:, i];  (P @ B)[i] = B[perm[i]]
    opts = dict(kernel=kern, tile=tile, nstage=S)
    A = inputs.place(Avals.to(dt), la)
    p = inputs.Problem(M, K, K, A, inputs.place(P.to(dt), lb), None, 1.0, 0.0, dtype, out)
    want = torch.empty(M, K)
    want[:, perm] = Avals
    assert same_values(run(p, **opts), want.to(odt)), "A @ P"
    Bop = inputs.place(Bvals.to(dt), lb)
    p = inputs.Problem(K, N, K, inputs.place(torch.eye(K).to(dt), la), Bop, None, 1.0, 0.0, dtype, out)
    assert same_values(run(p, **opts), Bvals.to(odt)), "I @ B"
    p = inputs.Problem(K, N, K, inputs.place(P.to(dt), la), Bop, None, 1.0, 0.0, dtype, out)
    assert same_values(run(p, **opts), Bvals[perm].to(odt)), "P @ B"


@pytest.mark.parametrize("fam", FAMILIES, ids=_fid)
def test_small_integers_exact(fam):
    """Entries in [-2, 2]: every product and partial sum is an exact fp32 integer, so the
    device result must equal the exact sum rounded (RNE) to the output type."""
    dtype, out, la, lb, kern, tile, S, M, N, K = fam
    say(f"[small integers] {_fid(fam)}")
    p = problem(dtype, out, M, N, K, la, lb, dist="int2", seed=3)
    got = run(p, kernel=kern, tile=tile, nstage=S)
    exact = oracle_ref(p)
    assert np.array_equal(got.double().numpy(), expected_rounded(exact, out))


@pytest.mark.parametrize("dtype,out,K,want", [
    ("bf16", "bf16", 2060, 2064.0),     # nearest
    ("bf16", "bf16", 2056, 2048.0),     # tie -> even
    ("f16", "f16", 2051, 2052.0),       # tie -> even
    ("f32", "f32", 2049, 2049.0),
    ("bf16", "f32", 2049, 2049.0),
])
def test_all_ones_rounding(dtype, out, K, want):
    """All-ones inputs: C = K exactly in fp32, then round-to-nearest-even to the output."""
    say(f"[all ones] {dtype}->{out} K={K}")
    la, lb = (ROW, COL) if dtype != "f32" else (ROW, ROW)
    p = problem(dtype, out, 33, 40, K, la, lb, dist="ones")
    got = run(p)
    assert torch.all(got.double() == want), got.unique()


def test_alpha_beta_all_ones():
    """c5 form: alpha = 0.5, beta = 1 with C0 = 1 gives 0.5*K + 1 exactly."""
    say("[all ones alpha/beta]")
    M, N, K = 100, 60, 2049
    dt = torch.bfloat16
    A = inputs.operand(M, K, ROW, dt, "ones", 1)
    B = inputs.operand(K, N, ROW, dt, "ones", 2)
    C0 = inputs.place(torch.ones(M, N), ROW)
    p = inputs.Problem(M, N, K, A, B, C0, 0.5, 1.0, "bf16", "f32")
    got = run(p)
    assert torch.all(got == 0.5 * K + 1.0)


# --------------------------------------------------------------- the five workloads

SMALL = {  # reduced sizes that span several tiles and leave ragged tails
    "c1": dict(M=256, N=256, K=256),
    "c2": dict(M=640, N=448, K=512),
    "c3": dict(M=768, N=1024, K=512),
    "c4": dict(M=1024, N=768, K=384),
    "c5": dict(M=400, N=300, K=205),
}


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_workload_small_vs_oracle(name):
    cfg = inputs.CONFIGS[name]
    p = inputs.make_problem(cfg, **SMALL[name])
    say(f"[{name} small] {SMALL[name]}")
    got = run(p)
    err = err_vs_oracle(p, got)
    say(f"  err={err:.3e}")
    assert err <= TOL[cfg["dtype"]]


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_workload_full_size_whole_matrix(name):
    """Full configuration sizes in the launch configuration the benchmark times: every
    element against the oracle, the stated bar unadjusted (output rounding included)."""
    cfg = inputs.CONFIGS[name]
    p = inputs.make_problem(cfg)
    s, plan = lg.gemm_plan({"f32": 0, "bf16": 1, "f16": 2}[p.dtype], {"f32": 0, "bf16": 1, "f16": 2}[p.out],
                           p.A.layout, p.B.layout, p.M, p.N, p.K, p.alpha, 16, p.A.ld, 16, p.B.ld, p.beta, 16, p.N)
    say(f"[{name} full] M={p.M} N={p.N} K={p.K} plan={plan.as_dict()}")
    got = run(p)
    assert not torch.isnan(got).any()
    err = whole_matrix(p, got)
    say(f"  all {p.M} rows: err={err:.3e}")
    assert err <= TOL[cfg["dtype"]]


@pytest.mark.parametrize("name", ["c3", "c4"])
def test_full_size_small_integers_bit_exact(name):
    """Whole-matrix bit-exactness at the full MFMA shapes with integer inputs (every sum
    exact in fp32): every element equals the exact result rounded to the output type."""
    cfg = inputs.CONFIGS[name]
    p = inputs.make_problem(cfg, dist="int2")
    say(f"[{name} full int2]")
    got = run(p)
    bad = whole_matrix(p, got, exact=True)
    say(f"  all {p.M} rows: {int(bad)} elements differ")
    assert bad == 0


FULL_STAGES = [  # (workload, kernel family, tile, stage counts): the default tiles at full size
    ("c2", K_VALU_RING, 10, [1, 2, 3, 4]),
    ("c2", K_VALU_RING, 5, [1, 2, 3, 4]),
    ("c3", K_MFMA_RING, 31, [1, 2]),
    ("c4", K_MFMA_RING, 31, [1, 2]),
    ("c5", K_MFMA_RING, 30, [1, 2]),
]


@pytest.mark.parametrize("case", FULL_STAGES, ids=lambda c: f"{c[0]}-t{c[2]}")
def test_full_shape_bit_identical_across_stage_counts(case):
    """At the full configuration shapes: the ring depth changes no bit of the output (every
    accumulator sees the same k order), and a repeated run changes none either."""
    name, kern, tile, stages = case
    p = inputs.make_problem(inputs.CONFIGS[name])
    outs = []
    for S in stages:
        say(f"[{name} full stages] tile={tile} nstage={S}")
        outs.append(run(p, kernel=kern, tile=tile, nstage=S))
    outs.append(run(p, kernel=kern, tile=tile, nstage=stages[-1]))
    bits = torch.int32 if outs[0].dtype == torch.float32 else torch.int16
    for o in outs[1:]:
        assert torch.equal(o.view(bits), outs[0].view(bits))


# --------------------------------------------------------------- stage counts

RING_STAGES = [
    ("f32", "f32", ROW, ROW, K_VALU_RING, 1, [1, 2, 3, 4], 512, 384, 1024),
    ("f32", "f32", ROW, ROW, K_VALU_RING, 5, [1, 2, 3, 4], 512, 384, 1024),
    ("f32", "f32", ROW, ROW, K_VALU_RING, 10, [1, 2, 3, 4], 520, 392, 1024),
    ("f32", "f32", ROW, ROW, K_VALU_RING, 11, [1, 2, 3, 4], 384, 520, 512),
    ("f32", "f32", ROW, ROW, K_VALU_RING, 4, [1, 2, 3, 4], 256, 320, 512),
    ("f32", "f32", ROW, ROW, K_VALU_RING, 7, [1, 2, 3, 4], 96, 64, 320),
    ("f32", "f32", ROW, ROW, K_VALU_RING, 3, [1, 2, 3, 4], 96, 64, 160),
    ("bf16", "bf16", ROW, COL, K_MFMA_RING, 1, [1, 2], 768, 512, 512),
    ("bf16", "bf16", ROW, COL, K_MFMA_RING, 2, [1, 2, 3, 4], 512, 768, 640),
    ("f16", "f32", ROW, COL, K_MFMA_RING, 3, [1, 2, 3, 4], 384, 256, 704),
    ("bf16", "bf16", ROW, COL, K_MFMA_RING, 25, [3, 4], 512, 768, 640),
    ("bf16", "bf16", ROW, COL, K_MFMA_RING, 18, [1, 2, 3], 768, 640, 576),
    ("bf16", "bf16", ROW, COL, K_MFMA_RING, 23, [1, 2], 768, 512, 576),
    ("bf16", "bf16", ROW, COL, K_MFMA_RING, 24, [1, 2], 768, 512, 576),
    ("bf16", "bf16", ROW, COL, K_MFMA_RING, 31, [1, 2], 768, 512, 576),
    ("f16", "f16", ROW, COL, K_MFMA_RING, 32, [1, 2], 576, 768, 448),
    ("f16", "f32", ROW, COL, K_MFMA_RING, 29, [1, 2], 600, 768, 448),
    ("f16", "f16", ROW, COL, K_MFMA_RING, 23, [1, 2], 512, 768, 448),
    ("bf16", "bf16", ROW, COL, K_MFMA_RING, 26, [1, 2], 768, 600, 576),
    ("bf16", "f32", ROW, COL, K_MFMA_RING, 29, [1, 2], 600, 768, 448),
    ("bf16", "f32", ROW, ROW, K_MFMA_RING, 30, [1, 2], 600, 768, 449),
    ("f16", "f16", ROW, ROW, K_MFMA_RING, 30, [1, 2], 400, 512, 384),
    ("f16", "f16", ROW, COL, K_MFMA_RING, 19, [2, 3], 2304, 4352, 320),
    ("bf16", "f32", ROW, ROW, K_MFMA_STAGED, 1, [1, 2], 300, 200, 333),
    ("f32", "f32", COL, ROW, K_VALU_STAGED, 1, [1, 2], 300, 200, 77),
]


@pytest.mark.parametrize("case", RING_STAGES, ids=lambda c: f"{c[0]}-k{c[4]}-t{c[5]}")
def test_bit_identical_across_stage_counts(case):
    """Every accumulator sees the same k order whatever the ring depth: outputs are
    bit-identical for every nStage and across repeated runs."""
    dtype, out, la, lb, kern, tile, stages, M, N, K = case
    p = problem(dtype, out, M, N, K, la, lb, dist="normal", seed=11)
    results = []
    for S in stages:
        say(f"[stages] {case[:6]} nstage={S}")
        results.append(run(p, kernel=kern, tile=tile, nstage=S))
    results.append(run(p, kernel=kern, tile=tile, nstage=stages[-1]))
    ref = results[0]
    for r in results[1:]:
        assert torch.equal(r.view(torch.int32) if r.dtype == torch.float32 else r.view(torch.int16),
                           ref.view(torch.int32) if ref.dtype == torch.float32 else ref.view(torch.int16))
    err = err_vs_oracle(p, ref)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("M,N,K,la,lb,opts", [
    (2048, 2048, 512, ROW, COL, {}),                                             # 64 tiles
    (2000, 1504, 300, ROW, ROW, dict(kernel=K_MFMA_RING, tile=30, nstage=2)),    # row-major ring, 11 x 6 = 66 tiles
    (1000, 1100, 256, ROW, COL, {}),                                             # 4 x 5 = 20 tiles
    (2304, 2304, 256, ROW, COL, dict(kernel=K_MFMA_RING, tile=28, nstage=2)),    # persistent, 81 tiles
    (4352, 4352, 128, ROW, COL, dict(kernel=K_MFMA_RING, tile=28, nstage=2)),    # persistent, 289 tiles > grid
    (1100, 700, 96, ROW, ROW, dict(kernel=K_VALU_RING, tile=5, nstage=2)),       # fp32, 9 x 11 = 99 tiles
])
def test_xcd_order_does_not_change_results(M, N, K, la, lb, opts):
    """The XCD remap (applied when the tile count is a multiple of 8) permutes the tiles:
    every tile is written (C starts as NaN) and the bits equal those of plain order, for
    plain, persistent (more tiles than workgroups) and fp32 grids, with tile counts that are
    and are not multiples of 8."""
    fp32 = opts.get("kernel") == K_VALU_RING
    dt = "f32" if fp32 else "bf16"
    p = problem(dt, dt, M, N, K, la, lb, dist="normal", seed=12)
    say(f"[xcd] {M}x{N}x{K} {opts}")
    a = run(p, **opts)
    b = run(p, flags=lg.GEMM_FLAG_NO_XCD_REMAP, **opts)
    view = torch.int32 if fp32 else torch.int16
    assert not torch.isnan(a.float()).any()
    assert torch.equal(a.view(view), b.view(view))


# --------------------------------------------------------------- fp32 fma-chain model

@pytest.mark.parametrize("kern,tile,S,M,N,K,la,lb", [
    (K_VALU_RING, 3, 2, 256, 256, 256, ROW, ROW),
    (K_VALU_RING, 1, 3, 512, 256, 512, ROW, ROW),
    (K_VALU_RING, 5, 3, 512, 256, 512, ROW, ROW),
    (K_VALU_RING, 4, 2, 256, 192, 256, ROW, ROW),
    (K_VALU_RING, 6, 4, 384, 128, 320, ROW, ROW),
    (K_VALU_RING, 7, 2, 256, 256, 256, ROW, ROW),
    (K_VALU_RING, 9, 4, 272, 208, 224, ROW, ROW),    # 16x16 tiles, 17 x 13 of them
    (K_VALU_RING, 9, 1, 40, 56, 96, ROW, ROW),       # ragged: edge tiles shifted inward
    (K_VALU_RING, 10, 2, 384, 256, 320, ROW, ROW),   # 128x128 tiles of 8x8 per thread
    (K_VALU_RING, 10, 4, 300, 260, 96, ROW, ROW),    # ragged
    (K_VALU_RING, 11, 4, 256, 384, 336, ROW, ROW),   # 128x128 tiles, 512 threads of 8x4
    (K_VALU_RING, 11, 1, 260, 132, 48, ROW, ROW),    # ragged
    (K_VALU_RING, 2, 1, 192, 128, 64, ROW, ROW),
    (K_VALU_STAGED, 1, 2, 131, 77, 50, COL, COL),
    (K_VALU_STAGED, 3, 1, 45, 33, 19, ROW, COL),
])
def test_fp32_matches_fma_chain_bit_for_bit(kern, tile, S, M, N, K, la, lb):
    say(f"[fma chain] kernel={kern} tile={tile} S={S} {M}x{N}x{K}")
    for alpha, beta in ((1.0, 0.0), (0.75, -1.5)):
        p = problem("f32", "f32", M, N, K, la, lb, dist="uniform", alpha=alpha, beta=beta, seed=13)
        got = run(p, kernel=kern, tile=tile, nstage=S)
        want = oracle.sgemm_fma_chain(la == COL, lb == COL, M, N, K, alpha, p.A.storage, p.A.ld,
                                      p.B.storage, p.B.ld, beta, None if p.C0 is None else p.C0.storage, N)
        assert np.array_equal(got.numpy(), want), np.argwhere(got.numpy() != want)[:5]


def test_fp32_4096_whole_matrix_fma_chain():
    """fp32 4096^3 at full size: every element equal, bit for bit, to one fmaf chain per
    output in ascending k."""
    p = inputs.make_problem(inputs.CONFIGS["c2"])
    say("[fma chain c2 full]")
    got = run(p).numpy()
    bad = 0
    for r0 in range(0, p.M, 512):
        rows = list(range(r0, min(p.M, r0 + 512)))
        want = oracle.sgemm_fma_chain(False, False, p.M, p.N, p.K, 1.0, p.A.storage, p.A.ld, p.B.storage, p.B.ld,
                                      rows=rows)
        bad += int(np.count_nonzero(got[r0:r0 + len(rows)] != want))
    say(f"  all {p.M} rows: {bad} elements differ")
    assert bad == 0


# --------------------------------------------------------------- edge sweep

EDGE = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def _edge_cases(n=40, seed=21):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = ["f32", "bf16", "f16"][i % 3]
        out = dtype if (i // 3) % 2 == 0 else "f32"
        M, N, K = (int(rng.choice(EDGE)) for _ in range(3))
        la, lb = int(rng.integers(2)), int(rng.integers(2))
        alpha = float(rng.choice([1.0, 0.5, -2.0, 0.0]))
        beta = float(rng.choice([0.0, 1.0, 0.5]))
        pad = int(rng.choice([0, 0, 1, 8]))
        cases.append((dtype, out, M, N, K, la, lb, alpha, beta, pad))
    return cases


@pytest.mark.parametrize("case", _edge_cases())
def test_edge_sweep(case):
    dtype, out, M, N, K, la, lb, alpha, beta, pad = case
    say(f"[edge] {case}")
    lda = (K if la == ROW else M) + pad
    ldb = (N if lb == ROW else K) + pad
    p = problem(dtype, out, M, N, K, la, lb, dist="uniform", alpha=alpha, beta=beta, seed=M + N + K,
                lda=lda, ldb=ldb)
    C, ldc = gpu_gemm(p, ldc=N + pad)
    got = c_logical(C, M, N, ldc)
    err = err_vs_oracle(p, got)
    assert err <= TOL[dtype], err
    if pad and M > 1 and beta == 0.0:
        # C padding between rows is never written (it held NaN)
        gaps = C[: (M - 1) * ldc].view(M - 1, ldc)[:, N:]
        assert torch.isnan(gaps.float()).all()


def test_beta_zero_ignores_nan_in_c():
    p = problem("bf16", "bf16", 300, 260, 96, ROW, COL, dist="uniform", seed=31)
    C, ldc = gpu_gemm(p, c_fill=float("nan"))
    assert not torch.isnan(c_logical(C, 300, 260, ldc).float()).any()


def test_k_zero_and_alpha_zero_scale_c():
    for K, alpha in ((0, 1.0), (64, 0.0)):
        for beta in (0.0, 0.5):
            p = problem("bf16", "f32", 70, 90, K, ROW, ROW, alpha=alpha, beta=beta, seed=32,
                        lda=max(K, 1))
            got = run(p)
            want = torch.zeros(70, 90) if beta == 0.0 else 0.5 * p.C0.logical()
            assert torch.equal(got, want)


def test_f16_subnormal_inputs_not_flushed():
    """A = 2^-24 * small integers (f16 subnormals), B = small integers: the exact
    result 2^-24 * sum is representable in fp32 and must not be flushed to zero."""
    say("[f16 subnormals]")
    M, N, K = 256, 256, 128
    g = torch.Generator().manual_seed(41)
    ia = torch.randint(-3, 4, (M, K), generator=g).float()
    ib = torch.randint(-3, 4, (K, N), generator=g).float()
    A = inputs.place((ia * 2.0 ** -24).to(torch.float16), ROW)
    B = inputs.place(ib.to(torch.float16), COL)
    assert (A.logical().float() != 0).any()
    p = inputs.Problem(M, N, K, A, B, None, 1.0, 0.0, "f16", "f32")
    for kern in (K_MFMA_RING, K_MFMA_STAGED):
        got = run(p, kernel=kern, tile=3 if kern == K_MFMA_RING else 0)
        want = (ia.double() @ ib.double()) * 2.0 ** -24
        assert torch.equal(got.double(), want)


def test_repeated_runs_identical():
    p = inputs.make_problem(inputs.CONFIGS["c3"], M=1024, N=1024, K=1024)
    a = run(p)
    for _ in range(3):
        assert torch.equal(run(p).view(torch.int16), a.view(torch.int16))


def test_matmul_wrapper_on_strided_views():
    g = torch.Generator().manual_seed(51)
    A = torch.randn(300, 200, generator=g).to(torch.bfloat16).to(DEV)
    Bt = torch.randn(150, 200, generator=g).to(torch.bfloat16).to(DEV)
    C = lg.matmul(A, Bt.t(), out_dtype=torch.float32)     # B column-major view
    torch.cuda.synchronize()
    ref = oracle.gemm_f64(False, True, 300, 150, 200, 1.0, A.cpu(), 200, Bt.cpu(), 200)
    err = oracle.normalized_error(C.cpu().double().numpy(), ref, 200, A.abs().max().item(), Bt.abs().max().item())
    assert err <= 1e-5


# --------------------------------------------------------------- every built variant

def _planned_variants():
    """Every (kernel family, tile, nstage) the planner accepts for a problem that fits
    all tiles; each must launch and agree with the oracle."""
    out = []
    for kern, dt, la, lb in ((K_MFMA_RING, "bf16", ROW, COL), (K_MFMA_STAGED, "f16", ROW, ROW),
                             (K_VALU_RING, "f32", ROW, ROW), (K_VALU_STAGED, "f32", COL, ROW)):
        for tile in range(1, 40):
            for S in range(1, 6):
                code = {"f32": 0, "bf16": 1, "f16": 2}[dt]
                M, N, K = 512, 512, 384
                s, plan = lg.gemm_plan(code, code, la, lb, M, N, K, 1.0, 16, K if la == ROW else M, 16,
                                       N if lb == ROW else K, 0.0, 16, N,
                                       lg.GemmOpts(S, kern, tile, 0))
                if s == lg.GEMM_OK:
                    out.append((kern, dt, la, lb, tile, S))
    return out


@pytest.mark.parametrize("v", _planned_variants(), ids=lambda v: f"k{v[0]}-{v[1]}-t{v[4]}-s{v[5]}")
def test_every_planned_variant_launches_and_matches(v):
    kern, dt, la, lb, tile, S = v
    say(f"[variant] kernel={kern} {dt} tile={tile} nstage={S}")
    p = problem(dt, dt if dt != "f32" else "f32", 512, 512, 384, la, lb, dist="int2", seed=61)
    got = run(p, kernel=kern, tile=tile, nstage=S)
    assert np.array_equal(got.double().numpy(), expected_rounded(oracle_ref(p), p.out))


# --------------------------------------------------------------- persistent tiles

PERSISTENT = [(19, 2), (19, 3), (28, 2)]


@pytest.mark.parametrize("shape", [(4096, 4096, 192), (4100, 3000, 320), (2048, 2560, 128), (8192, 4352, 128)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("ts", PERSISTENT, ids=lambda t: f"t{t[0]}-s{t[1]}")
def test_persistent_tiles_walk_several_tiles_exactly(shape, ts):
    """One workgroup per CU walks more tiles than the grid holds (512, 408 and 1088 tiles
    of 256x128, 544 of 256x256; 160 of 256x128 fit at once); ragged M / N edges; every
    element exact on small integers, and the same bits as the non-persistent tile of the
    same scheme (the producer / consumer tile 18, the split-copy tile 23)."""
    M, N, K = shape
    tile, S = ts
    say(f"[persistent] tile={tile} S={S} {M}x{N}x{K}")
    p = problem("bf16", "f32", M, N, K, ROW, COL, dist="int2", seed=83)
    got = run(p, kernel=K_MFMA_RING, tile=tile, nstage=S)
    assert np.array_equal(got.double().numpy(), expected_rounded(oracle_ref(p), p.out))
    ref = run(p, kernel=K_MFMA_RING, tile=23 if tile == 28 else 18, nstage=S)
    assert torch.equal(got, ref)


EQUAL_LDS = [("f32", "f32", ROW, ROW, K_VALU_RING, 1, [1, 2, 3], 512, 384, 256),
             ("f32", "f32", ROW, ROW, K_VALU_RING, 5, [1, 2, 3], 512, 384, 256),
             ("bf16", "bf16", ROW, COL, K_MFMA_RING, 18, [1, 2], 768, 640, 576),
             ("bf16", "bf16", ROW, COL, K_MFMA_RING, 23, [1, 2], 768, 512, 576),
             ("bf16", "bf16", ROW, COL, K_MFMA_RING, 3, [1, 2, 3], 384, 256, 320)]


@pytest.mark.parametrize("case", EQUAL_LDS, ids=lambda c: f"{c[0]}-k{c[4]}-t{c[5]}")
def test_equal_lds_padding_changes_no_bit(case):
    """The equal-occupancy launches (extra dynamic LDS) give the same bits."""
    dtype, out, la, lb, kern, tile, stages, M, N, K = case
    p = problem(dtype, out, M, N, K, la, lb, dist="normal", seed=29)
    for S in stages:
        say(f"[equal-lds] {case[:6]} nstage={S}")
        a = run(p, kernel=kern, tile=tile, nstage=S)
        b = run(p, kernel=kern, tile=tile, nstage=S, flags=lg.GEMM_FLAG_EQUAL_LDS)
        assert torch.equal(a, b)


RAGGED_TILES = [(23, 2), (24, 2), (24, 1), (31, 2), (31, 1), (32, 2), (18, 3), (18, 1), (25, 3), (26, 2), (26, 1), (29, 1), (29, 2), (1, 2), (2, 4)]


@pytest.mark.parametrize("ts", RAGGED_TILES, ids=lambda t: f"t{t[0]}-s{t[1]}")
def test_ring_tiles_on_ragged_edges(ts):
    """M and N that are not multiples of the tile (edge tiles shifted inward, each element
    stored once), K a few slabs long; exact on small integers, 16-bit and fp32 outputs."""
    tile, S = ts
    for (M, N, K, out) in ((300, 700, 192, "bf16"), (513, 257, 320, "f32")):
        say(f"[ragged] tile={tile} S={S} {M}x{N}x{K} -> {out}")
        p = problem("bf16", out, M, N, K, ROW, COL, dist="int2", seed=97)
        got = run(p, kernel=K_MFMA_RING, tile=tile, nstage=S)
        assert np.array_equal(got.double().numpy(), expected_rounded(oracle_ref(p), p.out))


@pytest.mark.parametrize("tile,S", [(1, 2), (2, 3), (3, 1), (5, 3), (6, 2), (7, 2), (9, 4), (9, 2), (10, 2), (10, 3),
                                    (11, 4), (11, 2)])
def test_valu_ring_on_ragged_edges(tile, S):
    """fp32 direct ring with M and N not multiples of the tile (N a multiple of 4, so the
    shifted last column tile stays 16-byte aligned; row pitch padded): edge tiles shifted
    inward, every element stored once, exact."""
    second = (130, 100, 32, 104) if tile not in (10, 11) else (260, 132, 96, 136)   # >= the 128x128 tiles
    for (M, N, K, ldb) in ((300, 260, 64, 264), second):
        say(f"[ragged valu] tile={tile} S={S} {M}x{N}x{K} ldb={ldb}")
        p = problem("f32", "f32", M, N, K, ROW, ROW, dist="int2", seed=101, ldb=ldb)
        got = run(p, kernel=K_VALU_RING, tile=tile, nstage=S)
        assert np.array_equal(got.double().numpy(), expected_rounded(oracle_ref(p), p.out))


# --------------------------------------------------------------- row-major A and B in place

KN_CASES = [  # (dtype, out, M, N, K, lda pad, ldb pad, alpha, beta): K tails, odd A pitches, ragged M / N
    ("bf16", "f32", 300, 512, 1, 0, 0, 1.0, 0.0),
    ("bf16", "bf16", 193, 264, 17, 1, 8, 1.0, 0.0),
    ("f16", "f16", 400, 520, 63, 3, 0, 1.0, 0.0),
    ("bf16", "f32", 385, 256, 64, 0, 16, 0.5, 1.0),
    ("f16", "f32", 600, 776, 65, 7, 0, -2.0, 0.5),
    ("bf16", "bf16", 577, 1032, 130, 1, 24, 1.0, 0.0),
    ("bf16", "f32", 4000, 3000, 2049, 0, 0, 0.5, 1.0),
]


@pytest.mark.parametrize("case", KN_CASES, ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}x{c[3]}x{c[4]}")
def test_row_major_ring_exact_on_tails_and_pitches(case):
    """Tile 30 reads row-major A (any pitch, through registers) and row-major B (copied as
    [k][n] rows, fragments gathered by transposing LDS reads) as they are, K tail included:
    exact on small integers, and the same bits as the split tile on operands rewritten
    into a workspace (same k order per accumulator)."""
    dtype, out, M, N, K, pa, pb, alpha, beta = case
    p = problem(dtype, out, M, N, K, ROW, ROW, dist="int2", alpha=alpha, beta=beta, seed=7, lda=K + pa, ldb=N + pb)
    for S in (1, 2):
        say(f"[row-major ring] {case} nstage={S}")
        got = run(p, kernel=K_MFMA_RING, tile=30, nstage=S)
        assert np.array_equal(got.double().numpy(), expected_rounded(oracle_ref(p), p.out))
    q = problem(dtype, out, M, N, K, ROW, ROW, dist="normal", alpha=alpha, beta=beta, seed=8, lda=K + pa, ldb=N + pb)
    a = run(q, kernel=K_MFMA_RING, tile=30, nstage=2)
    C, ldc = gpu_gemm(q, ws="auto", kernel=K_MFMA_RING, tile=29, nstage=2)
    b = c_logical(C, M, N, ldc)
    bits = torch.int32 if out == "f32" else torch.int16
    assert torch.equal(a.view(bits), b.view(bits))
    assert err_vs_oracle(q, a) <= TOL[dtype]


# --------------------------------------------------------------- LDS-poisoning variants

POISON_CASES = [  # (dtype, out, la, lb, kernel, tile, stages, M, N, K, alpha, beta): several slabs, ragged M / N
    ("f32", "f32", ROW, ROW, K_VALU_RING, 5, (1, 2, 3, 4), 300, 200, 160, 1.0, 0.0),
    ("f32", "f32", ROW, ROW, K_VALU_RING, 10, (1, 2, 3, 4), 300, 200, 160, 1.0, 0.0),
    ("bf16", "bf16", ROW, COL, K_MFMA_RING, 31, (1, 2), 520, 600, 448, 1.0, 0.0),
    ("bf16", "f32", ROW, COL, K_MFMA_RING, 31, (1, 2), 300, 264, 320, 0.5, 1.0),
    ("bf16", "f32", ROW, ROW, K_MFMA_RING, 30, (1, 2), 400, 520, 449, 0.5, 1.0),
    ("bf16", "bf16", ROW, ROW, K_MFMA_RING, 30, (1, 2), 197, 256, 130, 1.0, 0.0),
]


@pytest.mark.parametrize("case", POISON_CASES,
                         ids=lambda c: f"{c[0]}-{c[1]}-{'RC'[c[2]]}{'RC'[c[3]]}-t{c[5]}-{c[7]}x{c[8]}x{c[9]}")
def test_poisoned_ring_changes_no_bit(case):
    """With every ring slot overwritten by NaN bits as soon as it is released, the default
    ring kernels give the same bits as without it, exact on small integers and on all-ones
    operands (where a stale slab would be indistinguishable from the right one and only the
    poison could show a read outside a slot's live range)."""
    dtype, out, la, lb, kern, tile, stages, M, N, K, alpha, beta = case
    for dist in ("int2", "ones"):
        p = problem(dtype, out, M, N, K, la, lb, dist=dist, alpha=alpha, beta=beta, seed=83)
        want = expected_rounded(oracle_ref(p), p.out)
        for S in stages:
            say(f"[poison] {dtype}->{out} tile={tile} S={S} {M}x{N}x{K} {dist}")
            got = run(p, kernel=kern, tile=tile, nstage=S, flags=lg.GEMM_FLAG_POISON_LDS)
            plain = run(p, kernel=kern, tile=tile, nstage=S)
            assert not torch.isnan(got.float()).any()
            assert np.array_equal(got.double().numpy(), want)
            assert torch.equal(got.contiguous().view(torch.int16 if out != "f32" else torch.int32),
                               plain.contiguous().view(torch.int16 if out != "f32" else torch.int32))
