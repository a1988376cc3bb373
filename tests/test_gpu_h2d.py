"""Host-to-device copy staged through a ring of page-locked slots (gemm_h2d_staged):
every byte arrives, for every slot count, chunk size and a ragged last chunk."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, say
from tiled_stage_software_amd import libgemm as lg

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nstage", [1, 2, 3, 4])
def test_staged_copy_is_exact(nstage):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rng = np.random.default_rng(nstage)
    for nbytes, chunk in ((1, 4096), (1000, 256), ((4 << 20) + 123, 1 << 20), (24 << 20, 3 << 20)):
        say(f"[h2d] nstage={nstage} bytes={nbytes} chunk={chunk}")
        src = rng.integers(0, 256, nbytes, dtype=np.uint8)            # ordinary (pageable) memory
        staging = torch.empty(nstage * chunk, dtype=torch.uint8, pin_memory=True)
        dst = torch.full((nbytes + 64,), 7, dtype=torch.uint8, device=DEV)
        s = lg.gemm_h2d_staged(dst.data_ptr(), src.ctypes.data, nbytes, staging.data_ptr(), chunk, nstage,
                               torch.cuda.current_stream().cuda_stream)
        assert s == lg.GEMM_OK, lg.gemm_last_error()
        out = dst.cpu().numpy()
        assert np.array_equal(out[:nbytes], src)
        assert (out[nbytes:] == 7).all()        # nothing written past the end
