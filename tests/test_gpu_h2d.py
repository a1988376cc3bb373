"""Host-to-device copy staged through a ring of page-locked slots (gemm_h2d_staged and its
asynchronous form): every byte arrives, for every slot count, chunk size and a ragged last
chunk; the asynchronous call returns before its last DMAs finish and overlaps GEMM work
queued on another stream."""
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


@pytest.mark.parametrize("nstage", [1, 2, 4])
def test_async_staged_copy_is_exact_after_the_stream(nstage):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rng = np.random.default_rng(10 + nstage)
    st = torch.cuda.Stream()
    for nbytes, chunk in ((777, 256), ((8 << 20) + 5, 1 << 20)):
        say(f"[h2d async] nstage={nstage} bytes={nbytes} chunk={chunk}")
        src = rng.integers(0, 256, nbytes, dtype=np.uint8)
        staging = torch.empty(nstage * chunk, dtype=torch.uint8, pin_memory=True)
        dst = torch.full((nbytes + 64,), 7, dtype=torch.uint8, device=DEV)
        torch.cuda.synchronize()
        s = lg.gemm_h2d_staged_async(dst.data_ptr(), src.ctypes.data, nbytes, staging.data_ptr(), chunk, nstage,
                                     st.cuda_stream)
        assert s == lg.GEMM_OK, lg.gemm_last_error()
        st.synchronize()
        out = dst.cpu().numpy()
        assert np.array_equal(out[:nbytes], src)
        assert (out[nbytes:] == 7).all()


def test_async_staged_copy_overlaps_gemm_on_another_stream():
    """GEMMs queued on one stream, then a 64 MiB staged copy on another: the copy is exact
    and the GEMM results are those of the same GEMMs run alone."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tiled_stage_software_amd import inputs
    p = inputs.make_problem(inputs.CONFIGS["c3"], M=2048, N=2048, K=2048)
    A, B = p.A.storage.to(DEV), p.B.storage.to(DEV)
    C1 = torch.empty(2048 * 2048, dtype=torch.bfloat16, device=DEV)
    C2 = torch.empty_like(C1)
    g = torch.cuda.Stream()
    h = torch.cuda.Stream()

    def gemm(C):
        s = lg.gemm_bf16(inputs.ROW, inputs.COL, 2048, 2048, 2048, 1.0, A.data_ptr(), 2048, B.data_ptr(), 2048, 0.0,
                         C.data_ptr(), lg.GEMM_BF16, 2048, g.cuda_stream)
        assert s == lg.GEMM_OK
    gemm(C1)
    g.synchronize()
    nbytes, chunk = 64 << 20, 4 << 20
    src = np.random.default_rng(3).integers(0, 256, nbytes, dtype=np.uint8)
    staging = torch.empty(2 * chunk, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    for _ in range(20):
        gemm(C2)
    s = lg.gemm_h2d_staged_async(dst.data_ptr(), src.ctypes.data, nbytes, staging.data_ptr(), chunk, 2, h.cuda_stream)
    assert s == lg.GEMM_OK, lg.gemm_last_error()
    h.synchronize()
    g.synchronize()
    assert np.array_equal(dst.cpu().numpy(), src)
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
