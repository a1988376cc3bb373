"""The stage / tile tuner through the C ABI: it returns a variant the planner accepts,
and that variant computes the product exactly on small-integer inputs."""
import numpy as np
import pytest
import torch

from tiled_stage_software_amd import inputs, libgemm as lg
from gpu_util import DEV, say, gpu_gemm, c_logical, oracle_ref, expected_rounded

pytestmark = pytest.mark.gpu

CASES = [("bf16", "bf16", inputs.ROW, inputs.COL, 1024, 768, 512),
         ("f16", "f32", inputs.ROW, inputs.ROW, 300, 200, 129),
         ("f32", "f32", inputs.ROW, inputs.ROW, 512, 256, 256)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[4]}x{c[5]}x{c[6]}")
def test_tuned_variant_is_valid_and_exact(case):
    dt, out, la, lb, M, N, K = case
    say(f"[tune] {case}")
    cfg = dict(dtype=dt, out=out, M=M, N=N, K=K, la=la, lb=lb, dist="int2", std=1.0, alpha=1.0, beta=0.0, index=9)
    p = inputs.make_problem(cfg)
    A, B = p.A.storage.to(DEV), p.B.storage.to(DEV)
    C = torch.zeros(M * N, dtype=inputs.DTYPES[out], device=DEV)
    code = {"f32": lg.GEMM_F32, "bf16": lg.GEMM_BF16, "f16": lg.GEMM_F16}
    s, best, ms = lg.gemm_tune(code[dt], code[out], la, lb, M, N, K, 1.0, A.data_ptr(), p.A.ld, B.data_ptr(), p.B.ld,
                               0.0, C.data_ptr(), N, torch.cuda.current_stream().cuda_stream, reps=3)
    assert s == lg.GEMM_OK, lg.gemm_last_error()
    assert ms > 0.0
    s, plan = lg.gemm_plan(code[dt], code[out], la, lb, M, N, K, 1.0, A.data_ptr(), p.A.ld, B.data_ptr(), p.B.ld,
                           0.0, C.data_ptr(), N, best)
    assert s == lg.GEMM_OK and plan.kernel == best.kernel and plan.tile == best.tile and plan.nstage == best.nstage
    Cst, ldc = gpu_gemm(p, nstage=best.nstage, kernel=best.kernel, tile=best.tile)
    got = c_logical(Cst, M, N, ldc).double().numpy()
    assert np.array_equal(got, expected_rounded(oracle_ref(p), out))


def test_tune_empty_problem_reports_default():
    C = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    d = C.data_ptr()
    s, best, ms = lg.gemm_tune(lg.GEMM_BF16, lg.GEMM_BF16, inputs.ROW, inputs.COL, 0, 16, 16, 1.0, d, 16, d, 16,
                               0.0, d, 16, 0, reps=2)
    assert s == lg.GEMM_OK and ms == 0.0


def test_tune_with_a_workspace_times_the_workspace_call():
    """bf16 NN with a K tail: without a workspace the staged kernel and the ring that reads
    row-major operands in place (tile 30) can run; with one the tuner also times ring
    variants on the rewritten operands, and its pick, passed to gemm_bf16_ws with the same
    workspace, is exact on small integers."""
    M, N, K = 700, 600, 300
    say("[tune ws]")
    cfg = dict(dtype="bf16", out="f32", M=M, N=N, K=K, la=inputs.ROW, lb=inputs.ROW, dist="int2", std=1.0,
               alpha=1.0, beta=0.0, index=9)
    p = inputs.make_problem(cfg)
    A, B = p.A.storage.to(DEV), p.B.storage.to(DEV)
    C = torch.zeros(M * N, dtype=torch.float32, device=DEV)
    args = (lg.GEMM_BF16, lg.GEMM_F32, p.A.layout, p.B.layout, M, N, K, 1.0, A.data_ptr(), p.A.ld, B.data_ptr(),
            p.B.ld, 0.0, C.data_ptr(), N)
    s, n, _ = lg.gemm_workspace_size(*args)
    assert s == lg.GEMM_OK and n > 0
    W = torch.empty(n, dtype=torch.uint8, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    s, best, ms = lg.gemm_tune_ws(*args, st, W.data_ptr(), n, reps=3)
    assert s == lg.GEMM_OK and ms > 0.0, lg.gemm_last_error()
    s, best0, _ = lg.gemm_tune(*args, st, reps=3)
    assert s == lg.GEMM_OK and (best0.kernel == lg.GEMM_KERNEL_MFMA_STAGED or
                                (best0.kernel == lg.GEMM_KERNEL_MFMA_RING and best0.tile == 30))
    Cst, ldc = gpu_gemm(p, nstage=best0.nstage, kernel=best0.kernel, tile=best0.tile)
    assert np.array_equal(c_logical(Cst, M, N, ldc).double().numpy(), expected_rounded(oracle_ref(p), "f32"))
    Cst, ldc = gpu_gemm(p, ws=W, nstage=best.nstage, kernel=best.kernel, tile=best.tile)
    got = c_logical(Cst, M, N, ldc).double().numpy()
    assert np.array_equal(got, expected_rounded(oracle_ref(p), "f32"))
