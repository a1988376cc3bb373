"""The compute-bound control (gemm_mfma_ceiling) through the C ABI.  On small-integer
fragments every partial sum is an integer below 2^24, so each lane's accumulator sum is
exact and is checked bit for bit against the same sum formed in int64 from the fragment
and result layouts the header documents (the matrix instruction's own register layout);
every wave of every workgroup must give it, and nothing past the last workgroup's sums is
written."""
import numpy as np
import pytest
import torch

from tiled_stage_software_amd import libgemm as lg
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu
SHAPES = {16: (4, 4, 4), 32: (8, 2, 2)}   # k-steps R, first-operand fragments WA, second WB
TORCH = {lg.GEMM_BF16: torch.bfloat16, lg.GEMM_F16: torch.float16}
NFRAG = lg.GEMM_CEIL_FRAG_ELEMS // (64 * 8)


def expected_lane_sums(frags: np.ndarray, mi: int, iters: int) -> np.ndarray:
    """frags: int64 [NFRAG, 64 lanes, 8].  Lane l of a fragment holds row l mod mi, k =
    8*(l // mi) .. +7 of its mi x (512/mi) block; each instruction adds X Y^T."""
    R, WA, WB = SHAPES[mi]
    ki = 512 // mi
    blk = np.zeros((NFRAG, mi, ki), dtype=np.int64)
    for l in range(64):
        blk[:, l % mi, 8 * (l // mi): 8 * (l // mi) + 8] = frags[:, l, :]
    total = np.zeros((mi, mi), dtype=np.int64)
    for r in range(R):
        for i in range(WA):
            for j in range(WB):
                total += blk[r * (WA + WB) + i] @ blk[r * (WA + WB) + WA + j].T
    total *= iters
    sums = np.zeros(64, dtype=np.int64)
    for l in range(64):
        if mi == 32:
            rows = [8 * q + 4 * (l // 32) + t for q in range(4) for t in range(4)]
        else:
            rows = [4 * (l // 16) + t for t in range(4)]
        sums[l] = total[rows, l % mi].sum()
    return sums


@pytest.mark.parametrize("in_type", [lg.GEMM_BF16, lg.GEMM_F16])
@pytest.mark.parametrize("mi", [16, 32])
@pytest.mark.parametrize("grid,iters", [(1, 1), (3, 3), (300, 2), (5, 0)])
def test_lane_sums_are_exact(in_type, mi, grid, iters):
    say(f"[mfma_ceiling] in_type={in_type} shape={mi} grid={grid} iters={iters}")
    g = torch.Generator().manual_seed(900 + mi + grid)
    ints = torch.randint(-3, 4, (NFRAG, 64, 8), generator=g)
    frags = ints.to(TORCH[in_type]).view(torch.int16).contiguous().to(DEV)
    n = grid * lg.GEMM_CEIL_THREADS
    guard = 256
    sums = torch.full((n + guard,), -7.0, dtype=torch.float32, device=DEV)
    s = lg.gemm_mfma_ceiling(in_type, mi, frags.data_ptr(), sums.data_ptr(), grid, iters,
                             torch.cuda.current_stream().cuda_stream)
    assert s == lg.GEMM_OK, lg.gemm_last_error()
    torch.cuda.synchronize()
    got = sums[:n].cpu().double().numpy().reshape(grid * 8, 64)
    want = expected_lane_sums(ints.numpy().astype(np.int64), mi, iters)
    assert np.abs(want).max() < 2 ** 24
    assert (got == want[None, :].astype(np.float64)).all()
    assert bool((sums[n:] == -7.0).all())


def test_random_operands_give_finite_equal_sums_across_waves():
    """N(0,1) bf16 fragments, as the benchmark times them: every wave holds the same
    operands, so every wave's lane sums agree exactly (the same instructions in the same
    order), and they are finite."""
    say("[mfma_ceiling] random bf16, shape 16, grid 512, iters 64")
    g = torch.Generator().manual_seed(901)
    frags = torch.randn((lg.GEMM_CEIL_FRAG_ELEMS,), generator=g).to(torch.bfloat16).view(torch.int16).to(DEV)
    grid = 512
    sums = torch.empty((grid * lg.GEMM_CEIL_THREADS,), dtype=torch.float32, device=DEV)
    s = lg.gemm_mfma_ceiling(lg.GEMM_BF16, 16, frags.data_ptr(), sums.data_ptr(), grid, 64,
                             torch.cuda.current_stream().cuda_stream)
    assert s == lg.GEMM_OK, lg.gemm_last_error()
    torch.cuda.synchronize()
    v = sums.view(grid * 8, 64)
    assert bool(torch.isfinite(v).all())
    assert bool((v == v[0:1]).all())
