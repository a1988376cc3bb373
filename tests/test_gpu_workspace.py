"""Parity of the repacking path (gemm_bf16_ws / gemm_f16_ws) with the CPU oracle, on an
MI355X.

The path rewrites operands the direct ring cannot read in place (N- or M-contiguous,
pitch or base off 16 bytes, a K tail) into a workspace as K-contiguous rows padded with
zeros to a multiple of 64, then runs the ring.  Bars: bit-exact on small-integer inputs
in every layout, with K tails and ragged M / N; bit-identical to the ring run on operands
padded and transposed by torch; the full irregular-tail workload within the bf16
tolerance on every element; a too-small workspace behaves exactly as gemm_*_ex.
"""
import numpy as np
import pytest
import torch

from gpu_util import (DEV, TOL, say, gpu_gemm, c_logical, oracle_ref, err_vs_oracle, sample_rows,
                      expected_rounded, workspace_bytes, whole_matrix)
from tiled_stage_software_amd import inputs, libgemm as lg

pytestmark = pytest.mark.gpu

ROW, COL = inputs.ROW, inputs.COL
K_MFMA_RING, K_MFMA_STAGED = lg.GEMM_KERNEL_MFMA_RING, lg.GEMM_KERNEL_MFMA_STAGED


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lg.load()  # fails loudly if the library is missing
    torch.zeros(1, device=DEV)


def problem(dtype, out, M, N, K, la, lb, dist="int2", alpha=1.0, beta=0.0, seed=1, lda=None, ldb=None):
    dt = inputs.DTYPES[dtype]
    A = inputs.operand(M, K, la, dt, dist, seed * 10 + 1, ld=lda)
    B = inputs.operand(K, N, lb, dt, dist, seed * 10 + 2, ld=ldb)
    C0 = inputs.operand(M, N, ROW, inputs.DTYPES[out], "uniform", seed * 10 + 3) if beta != 0.0 else None
    return inputs.Problem(M, N, K, A, B, C0, alpha, beta, dtype, out)


def run(p, **opts):
    C, ldc = gpu_gemm(p, **opts)
    return c_logical(C, p.M, p.N, ldc)


def plan_of(p, **opts):
    return workspace_bytes(p, p.N, 1 << 20, 1 << 21, 1 << 22, **opts)


LAYOUTS = [(ROW, ROW), (COL, ROW), (COL, COL), (ROW, COL)]
SHAPES = [  # (M, N, K, lda pad, ldb pad): K tails, ragged M / N, odd pitches
    (300, 700, 192, 0, 0),
    (513, 257, 100, 3, 1),
    (260, 300, 129, 0, 5),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("lay", LAYOUTS, ids=lambda l: "RC"[l[0]] + "RC"[l[1]])
def test_exact_in_every_layout(dtype, lay):
    la, lb = lay
    for i, (M, N, K, pa, pb) in enumerate(SHAPES):
        for out, alpha, beta in ((dtype, 1.0, 0.0), ("f32", 0.5, 1.0)):
            lda = (K if la == ROW else M) + pa
            ldb = (N if lb == ROW else K) + pb
            p = problem(dtype, out, M, N, K, la, lb, alpha=alpha, beta=beta, seed=31 + i, lda=lda, ldb=ldb)
            n, plan = plan_of(p)
            say(f"[ws] {dtype} {'RC'[la]}{'RC'[lb]} {M}x{N}x{K} lda={lda} ldb={ldb} -> {out} "
                f"packed={plan.packed} bytes={n} tile={plan.tile}")
            direct = la == ROW and lb == COL and K % 64 == 0 and pa == 0 and pb == 0
            assert (plan.packed == 0) == direct and plan.kernel == K_MFMA_RING
            got = run(p, ws="auto")
            # alpha*acc + beta*c is one fp32 rounding of an exact value: RNE of the exact result
            assert np.array_equal(got.double().numpy(), expected_rounded(oracle_ref(p), out))


def test_identical_to_the_ring_on_operands_packed_by_torch():
    """The rewrite only moves bits and appends zeros: the ring on torch's padded,
    transposed copies gives the same result bit for bit (normal inputs, K tail)."""
    M, N, K = 520, 390, 2049
    Kp = 2112
    p = problem("bf16", "f32", M, N, K, ROW, ROW, dist="normal", alpha=0.5, beta=1.0, seed=7, lda=K)
    for tile, S in ((0, 0), (23, 2), (29, 2), (3, 2), (18, 3)):
        opts = dict(kernel=K_MFMA_RING, tile=tile, nstage=S) if tile else {}
        say(f"[ws torch-packed] tile={tile} S={S}")
        got = run(p, ws="auto", **opts)
        A = p.A.logical()
        B = p.B.logical()
        Ap = torch.zeros(M, Kp, dtype=torch.bfloat16)
        Ap[:, :K] = A
        Bp = torch.zeros(N, Kp, dtype=torch.bfloat16)
        Bp[:, :K] = B.t()
        q = inputs.Problem(M, N, Kp, inputs.place(Ap, ROW, Kp), inputs.place(Bp.t(), COL, Kp), p.C0,
                           p.alpha, p.beta, "bf16", "f32")
        ref = run(q, kernel=K_MFMA_RING, tile=tile or plan_of(p)[1].tile, nstage=S)
        assert torch.equal(got, ref)


def test_irregular_tail_workload_full_size():
    """The bf16 4000x3000x2049 NN workload with fp32 C, alpha 0.5, beta 1: with a workspace
    offered, the call reads the operands in place (tile 30, nothing rewritten); forcing the
    split tile rewrites both operands into the workspace.  Both give the same bits, within
    the bf16 tolerance on every element."""
    cfg = inputs.CONFIGS["c5"]
    p = inputs.make_problem(cfg)
    n, plan = plan_of(p)
    say(f"[ws c5] packed={plan.packed} bytes={n} tile={plan.tile} S={plan.nstage} grid={plan.grid}")
    assert plan.packed == 0 and plan.kernel == K_MFMA_RING and plan.tile == 30 and n == 0
    got = run(p, ws="auto")
    assert not torch.isnan(got).any()
    e = whole_matrix(p, got)
    say(f"[ws c5] all rows: err {e:.3e}")
    assert e <= TOL["bf16"]
    n29, plan29 = plan_of(p, kernel=K_MFMA_RING, tile=29)
    assert plan29.packed == 3 and n29 == 4000 * 2112 * 2 + 3000 * 2112 * 2
    packed = run(p, ws="auto", kernel=K_MFMA_RING, tile=29)
    assert torch.equal(got.view(torch.int32), packed.view(torch.int32))


def test_irregular_tail_workload_full_size_bit_identical_across_stage_counts():
    """Full c5 shape through the workspace path (operands rewritten for the split tile):
    one and two ring slots give the same bits."""
    p = inputs.make_problem(inputs.CONFIGS["c5"])
    outs = []
    for S in (1, 2):
        say(f"[ws c5 stages] tile=29 S={S}")
        outs.append(run(p, ws="auto", kernel=K_MFMA_RING, tile=29, nstage=S))
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))


def test_too_small_workspace_is_the_plain_call():
    p = problem("bf16", "bf16", 300, 260, 130, ROW, ROW, dist="normal", seed=5)
    n, plan = plan_of(p)
    assert n > 0 and plan.packed == 3
    base = run(p)                       # gemm_bf16_ex: the staged kernel
    small = run(p, ws=n - 256)          # too small: exactly gemm_bf16_ex
    assert torch.equal(base, small)
    full = run(p, ws="auto")            # the ring: a different k grouping, same tolerance
    assert err_vs_oracle(p, full) <= TOL["bf16"]


def test_workspace_reused_by_consecutive_calls():
    """One workspace, a large call then a smaller one (its stale contents must not leak)."""
    W = torch.full((8 << 20,), float("nan"), dtype=torch.bfloat16, device=DEV)
    for (M, N, K, seed) in ((700, 600, 1000, 11), (300, 270, 77, 12)):
        p = problem("f16", "f32", M, N, K, COL, ROW, seed=seed)
        n, plan = plan_of(p)
        assert 0 < n <= W.numel() * 2 and plan.packed == 3
        say(f"[ws reuse] {M}x{N}x{K}")
        got = run(p, ws=W)
        assert np.array_equal(got.double().numpy(), expected_rounded(oracle_ref(p), "f32"))


def test_forced_staged_kernel_ignores_the_workspace():
    p = problem("bf16", "bf16", 257, 300, 70, ROW, ROW, seed=3)
    n, plan = plan_of(p, kernel=K_MFMA_STAGED)
    assert n == 0 and plan.kernel == K_MFMA_STAGED and plan.packed == 0
    got = run(p, ws=1 << 20, kernel=K_MFMA_STAGED)
    assert np.array_equal(got.double().numpy(), expected_rounded(oracle_ref(p), "bf16"))


def test_irregular_tail_workload_small_integers_bit_exact():
    """Full size, integer inputs: exact sums, so the rewritten-operand path equals the
    oracle rounded to fp32 bit for bit on every element."""
    p = inputs.make_problem(inputs.CONFIGS["c5"], dist="int2")
    say("[ws c5 full int2]")
    got = run(p, ws="auto")
    assert whole_matrix(p, got, exact=True) == 0


def test_irregular_tail_workload_reduced_whole_matrix():
    """The same workload form (NN, K tail, fp32 C, alpha 0.5, beta 1) at 400x300x205:
    every element against the oracle."""
    p = inputs.make_problem(inputs.CONFIGS["c5"], M=400, N=300, K=205)
    n, plan = plan_of(p)
    say(f"[ws c5 small] packed={plan.packed} tile={plan.tile}")
    assert plan.packed == 3
    got = run(p, ws="auto")
    assert err_vs_oracle(p, got) <= TOL["bf16"]


@pytest.mark.parametrize("tile,stages", [(23, (1, 2)), (29, (1, 2)), (18, (1, 2, 3)), (3, (1, 2, 3, 4))])
def test_rewritten_operands_bit_identical_across_stage_counts(tile, stages):
    """Ring depth changes no bit on the rewritten-operand path either."""
    p = problem("bf16", "f32", 700, 600, 2049, ROW, ROW, dist="normal", alpha=0.5, beta=1.0, seed=9, lda=2049)
    outs = []
    for S in stages:
        say(f"[ws stages] tile={tile} S={S}")
        outs.append(run(p, ws="auto", kernel=K_MFMA_RING, tile=tile, nstage=S))
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    assert err_vs_oracle(p, outs[0]) <= TOL["bf16"]


def test_matmul_wrapper_with_an_automatic_workspace():
    """libgemm.matmul(..., workspace="auto") on torch views: B given as a transposed
    (N-contiguous) view, fp32 C with alpha / beta; exact on small integers."""
    g = torch.Generator().manual_seed(17)
    M, N, K = 300, 260, 130
    A = torch.randint(-2, 3, (M, K), generator=g).to(torch.bfloat16)
    Bt = torch.randint(-2, 3, (N, K), generator=g).to(torch.bfloat16)   # B = Bt.T is column-major
    C0 = torch.randint(-4, 5, (M, N), generator=g).to(torch.float32)
    want = 0.5 * (A.double() @ Bt.double().T) + 1.0 * C0.double()
    for B in (Bt.to(DEV).T, Bt.T.contiguous().to(DEV)):                   # column- then row-major B
        say(f"[matmul ws] B strides {tuple(B.stride())}")
        C = C0.to(DEV)
        out = lg.matmul(A.to(DEV), B, C=C, alpha=0.5, beta=1.0, workspace="auto")
        torch.cuda.synchronize()
        assert out.data_ptr() == C.data_ptr()
        assert torch.equal(out.cpu().double(), want)
