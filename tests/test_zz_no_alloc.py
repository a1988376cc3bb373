"""gemm_ws_static -- the entry point that allocates nothing (its workspace is a static
device array of the library) -- against gemm_bf16_ws / gemm_f16_ws with a caller
workspace: the same bits on two calls in a row, the second one smaller, and within the
oracle's bar."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, TOL, DT_CODE, say, gpu_gemm, c_logical, expected_rounded, oracle_ref, whole_matrix, \
    workspace_bytes
from tiled_stage_software_amd import inputs, libgemm as lg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lg.load()  # fails loudly if the library is missing
    torch.zeros(1, device=DEV)


# the irregular-tail workload is read in place by default; the split tile rewrites it
SPLIT = dict(kernel=lg.GEMM_KERNEL_MFMA_RING, tile=29)


def static_call(p: inputs.Problem, **opts) -> torch.Tensor:
    """C = alpha*A*B + beta*C0 through gemm_ws_static; C (M x N) on the host."""
    Ad, Bd = p.A.storage.to(DEV), p.B.storage.to(DEV)
    if p.C0 is not None:
        Cd = p.C0.storage.clone().to(DEV)
    else:
        Cd = torch.full((p.M * p.N,), float("nan"), dtype=inputs.DTYPES[p.out], device=DEV)
    s = lg.gemm_ws_static(DT_CODE[p.dtype], p.A.layout, p.B.layout, p.M, p.N, p.K, p.alpha, Ad.data_ptr(), p.A.ld,
                          Bd.data_ptr(), p.B.ld, p.beta, Cd.data_ptr(), DT_CODE[p.out], p.N,
                          torch.cuda.current_stream().cuda_stream, lg._opts(**opts))
    if s != lg.GEMM_OK:
        raise lg.GemmError(s, lg.gemm_last_error())
    torch.cuda.synchronize()
    return c_logical(Cd.cpu(), p.M, p.N, p.N)


def caller_ws_call(p: inputs.Problem, **opts) -> torch.Tensor:
    C, ldc = gpu_gemm(p, ws="auto", **opts)
    return c_logical(C, p.M, p.N, ldc)


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def test_static_workspace_equals_caller_workspace_on_consecutive_calls():
    big = inputs.make_problem(inputs.CONFIGS["c5"])                       # bf16 4000x3000x2049 NN, fp32 C
    dt = inputs.DTYPES["f16"]
    small = inputs.Problem(513, 257, 100,
                           inputs.operand(513, 100, inputs.COL, dt, "int2", 71, ld=516),
                           inputs.operand(100, 257, inputs.ROW, dt, "int2", 72, ld=258),
                           None, 1.0, 0.0, "f16", "f16")
    for name, p, opts in (("c5 full, split tile", big, SPLIT), ("f16 513x257x100 col x row", small, {})):
        n, plan = workspace_bytes(p, p.N, 1 << 20, 1 << 21, 1 << 22, **opts)
        say(f"[no-alloc] {name}: rewrites {plan.packed} ({n} bytes of {lg.GEMM_STATIC_WS_BYTES}), tile {plan.tile}")
        assert plan.packed != 0 and 0 < n <= lg.GEMM_STATIC_WS_BYTES
        got = static_call(p, **opts)
        ref = caller_ws_call(p, **opts)
        assert torch.equal(bits(got), bits(ref)), name
        if p is big:
            e = whole_matrix(p, got)
            say(f"  err {e:.3e}")
            assert e <= TOL["bf16"]
        else:
            assert np.array_equal(got.double().numpy(), expected_rounded(oracle_ref(p), p.out))
