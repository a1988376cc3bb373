"""The pipelined streaming copy (gemm_pipe_copy) through the C ABI: every stage count
copies every byte exactly, for one slab, a ragged number of slabs per workgroup and a
large buffer; the bytes around the destination are never written."""
import pytest
import torch

from tiled_stage_software_amd import libgemm as lg
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu
SLAB = 16384


@pytest.mark.parametrize("nstage", [1, 2, 3, 4])
@pytest.mark.parametrize("slabs", [1, 7, 2048 + 37, 16384])
def test_copy_is_exact(nstage, slabs):
    say(f"[pipe_copy] nstage={nstage} slabs={slabs}")
    n = slabs * SLAB
    g = torch.Generator(device="cpu").manual_seed(70 + slabs)
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).to(DEV)
    guard = 4096
    dst = torch.full((n + 2 * guard,), 0xA5, dtype=torch.uint8, device=DEV)
    s = lg.gemm_pipe_copy(dst.data_ptr() + guard, src.data_ptr(), n, nstage,
                          torch.cuda.current_stream().cuda_stream)
    assert s == lg.GEMM_OK, lg.gemm_last_error()
    torch.cuda.synchronize()
    assert torch.equal(dst[guard:guard + n], src)
    assert bool((dst[:guard] == 0xA5).all()) and bool((dst[guard + n:] == 0xA5).all())
