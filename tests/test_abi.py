"""C ABI checks that need no GPU: the library loads, exports what include/libgemm.h
declares, rejects bad arguments before launching anything, and plans the kernel the
problem calls for."""
import ctypes
import os
import re
import subprocess

import pytest

from tiled_stage_software_amd import libgemm as lg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libgemm.h")

ROW, COL = lg.GEMM_ROW_MAJOR, lg.GEMM_COL_MAJOR
A16 = 0x10000   # fake, 16-byte aligned device addresses (never dereferenced by gemm_plan)
B16 = 0x20000
C16 = 0x30000


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(gemm_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert set(names) == set(lg.EXPORTS), names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", lg.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    lib = lg.load()
    for n in declared_functions():
        assert hasattr(lib, n)


def test_status_strings():
    assert lg.gemm_status_string(0) == "GEMM_OK"
    assert lg.gemm_status_string(1) == "GEMM_ERR_INVALID_ARG"
    assert lg.gemm_status_string(2) == "GEMM_ERR_UNSUPPORTED"
    assert lg.gemm_status_string(3) == "GEMM_ERR_HIP"


def plan(in_t, c_t, la, lb, M, N, K, alpha=1.0, A=A16, lda=None, B=B16, ldb=None, beta=0.0, C=C16, ldc=None,
         **opts):
    lda = lda if lda is not None else (K if la == ROW else M)
    ldb = ldb if ldb is not None else (N if lb == ROW else K)
    ldc = ldc if ldc is not None else N
    o = lg.GemmOpts(opts.get("nstage", 0), opts.get("kernel", 0), opts.get("tile", 0), opts.get("flags", 0)) \
        if opts else None
    return lg.gemm_plan(in_t, c_t, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, o)


F32, BF16, F16 = lg.GEMM_F32, lg.GEMM_BF16, lg.GEMM_F16


@pytest.mark.parametrize("case,want", [
    (dict(M=-1), lg.GEMM_ERR_INVALID_ARG),
    (dict(N=-2), lg.GEMM_ERR_INVALID_ARG),
    (dict(K=-3), lg.GEMM_ERR_INVALID_ARG),
    (dict(lda=31), lg.GEMM_ERR_INVALID_ARG),        # row-major A needs lda >= K = 32
    (dict(ldb=47), lg.GEMM_ERR_INVALID_ARG),        # row-major B needs ldb >= N = 48
    (dict(ldc=47), lg.GEMM_ERR_INVALID_ARG),
    (dict(A=0), lg.GEMM_ERR_INVALID_ARG),
    (dict(B=0), lg.GEMM_ERR_INVALID_ARG),
    (dict(C=0), lg.GEMM_ERR_INVALID_ARG),
    (dict(la=7), lg.GEMM_ERR_INVALID_ARG),
    (dict(nstage=6), lg.GEMM_ERR_UNSUPPORTED),
    (dict(nstage=-1), lg.GEMM_ERR_UNSUPPORTED),
    (dict(flags=8), lg.GEMM_ERR_INVALID_ARG),
    (dict(kernel=lg.GEMM_KERNEL_MFMA_RING), lg.GEMM_ERR_UNSUPPORTED),   # fp32 input on the MFMA path
    (dict(kernel=lg.GEMM_KERNEL_VALU_RING, A=A16 + 4), lg.GEMM_ERR_UNSUPPORTED),  # misaligned
    (dict(kernel=lg.GEMM_KERNEL_VALU_STAGED, nstage=3), lg.GEMM_ERR_UNSUPPORTED),
])
def test_invalid_arguments(case, want):
    args = dict(in_t=F32, c_t=F32, la=ROW, lb=ROW, M=40, N=48, K=32)
    args.update(case)
    s, _ = plan(**args)
    assert s == want, (case, lg.gemm_status_string(s), lg.gemm_last_error())
    assert lg.gemm_last_error() != ""


def test_null_pointers_allowed_when_unused():
    assert plan(F32, F32, ROW, ROW, 0, 8, 8, A=0, B=0, C=0)[0] == lg.GEMM_OK      # M == 0
    assert plan(F32, F32, ROW, ROW, 8, 8, 0, A=0, B=0, lda=1)[0] == lg.GEMM_OK    # K == 0: scale only
    assert plan(F32, F32, ROW, ROW, 8, 8, 8, alpha=0.0, A=0, B=0)[0] == lg.GEMM_OK


def test_c_type_must_match_entry_point():
    assert plan(BF16, F16, ROW, COL, 64, 64, 64)[0] == lg.GEMM_ERR_INVALID_ARG
    assert plan(F16, BF16, ROW, COL, 64, 64, 64)[0] == lg.GEMM_ERR_INVALID_ARG
    assert plan(F32, BF16, ROW, ROW, 64, 64, 64)[0] == lg.GEMM_ERR_INVALID_ARG
    # the entry points themselves reject before touching the GPU
    s = lg.gemm_bf16(ROW, COL, 64, 64, 64, 1.0, A16, 64, B16, 64, 0.0, C16, lg.GEMM_F16, 64, 0)
    assert s == lg.GEMM_ERR_INVALID_ARG


def test_quick_returns():
    s, p = plan(BF16, BF16, ROW, COL, 0, 64, 64)
    assert s == lg.GEMM_OK and p.grid == 0
    s, p = plan(BF16, BF16, ROW, COL, 64, 0, 64, ldc=1)
    assert s == lg.GEMM_OK and p.grid == 0
    s, p = plan(BF16, BF16, ROW, COL, 64, 64, 0, lda=1, ldb=1)
    assert s == lg.GEMM_OK and p.kernel == lg.GEMM_KERNEL_SCALE
    s, p = plan(BF16, BF16, ROW, COL, 64, 64, 64, alpha=0.0)
    assert s == lg.GEMM_OK and p.kernel == lg.GEMM_KERNEL_SCALE
    # M == 0 through the entry point: nothing is launched, so this is safe without a GPU
    assert lg.gemm_f32(ROW, ROW, 0, 5, 5, 1.0, 0, 5, 0, 5, 0.0, 0, 5, 0) == lg.GEMM_OK


def test_plans_for_the_workloads():
    # fp32 4096^3 NN -> direct ring, 128x128 tile of 8x8 per thread: 1024 tiles, two full
    # rounds of two workgroups per CU
    s, p = plan(F32, F32, ROW, ROW, 4096, 4096, 4096)
    assert s == 0 and p.kernel == lg.GEMM_KERNEL_VALU_RING and (p.bm, p.bn, p.bk) == (128, 128, 32)
    assert p.grid == 32 * 32 and p.tile == 10 and p.threads == 256 and p.nstage == 2
    # the round model's other picks: 3072^3 and 2048^3 -> 128x64 (576 tiles of 128x128 would
    # leave a second round an eighth full; 256 would fill half the slots of one), 2560^3 ->
    # 128x128 (400 tiles in one round against 800 128x64 tiles in two), and K not a multiple
    # of 32 -> no tile 10
    assert plan(F32, F32, ROW, ROW, 3072, 3072, 3072)[1].tile == 5
    assert plan(F32, F32, ROW, ROW, 2048, 2048, 2048)[1].tile == 5
    assert plan(F32, F32, ROW, ROW, 2560, 2560, 2560)[1].tile == 10
    assert plan(F32, F32, ROW, ROW, 4096, 4096, 4080)[1].tile == 5
    # tile 11 (512 threads of 8x4) only when asked for
    s, p = plan(F32, F32, ROW, ROW, 2048, 2048, 2048, kernel=lg.GEMM_KERNEL_VALU_RING, tile=11)
    assert s == 0 and p.tile == 11 and p.threads == 512 and p.grid == 256 and p.nstage == 4
    # fp32 256^3 NN -> direct ring, 16x16 tiles (64 of 32x32 would leave most CUs idle)
    s, p = plan(F32, F32, ROW, ROW, 256, 256, 256)
    assert s == 0 and p.kernel == lg.GEMM_KERNEL_VALU_RING and (p.bm, p.bn) == (16, 16)
    assert p.tile == 9 and p.threads == 64 and p.grid == 256 and p.nstage == 4
    # fp32 1024^3 NN: 1024 tiles of 32x32, four per CU -> the 32x32 tile
    s, p = plan(F32, F32, ROW, ROW, 1024, 1024, 1024)
    assert s == 0 and p.kernel == lg.GEMM_KERNEL_VALU_RING and p.tile == 7 and (p.bm, p.bn) == (32, 32)
    # bf16 8192^3 NT -> MFMA ring, 256x256 split-copy tile (8 waves), two slots
    s, p = plan(BF16, BF16, ROW, COL, 8192, 8192, 8192)
    assert s == 0 and p.kernel == lg.GEMM_KERNEL_MFMA_RING and (p.bm, p.bn, p.bk) == (256, 256, 64)
    assert p.tile == 31 and p.threads == 512 and p.nstage == 2 and p.grid == 32 * 32 and p.lds_bytes <= 163840
    # f16 MLP shape NT
    s, p = plan(F16, F16, ROW, COL, 16384, 14336, 4096)
    assert s == 0 and p.kernel == lg.GEMM_KERNEL_MFMA_RING and p.grid == 64 * 56
    # bf16 4000x3000x2049 NN, fp32 C: odd K and lda, row-major B -> the 192x256 ring that reads
    # row-major A (any pitch) and B as they are (252 tiles, one round), with or without a
    # workspace; forcing the K-contiguous split tile rewrites both operands instead
    s, p = plan(BF16, F32, ROW, ROW, 4000, 3000, 2049, alpha=0.5, beta=1.0)
    assert s == 0 and p.kernel == lg.GEMM_KERNEL_MFMA_RING and p.tile == 30 and p.grid == 21 * 12
    s, n, p = ws_size(BF16, F32, ROW, ROW, 4000, 3000, 2049, alpha=0.5, beta=1.0)
    assert s == 0 and n == 0 and p.tile == 30 and p.packed == 0
    s, n, p = ws_size(BF16, F32, ROW, ROW, 4000, 3000, 2049, alpha=0.5, beta=1.0, kernel=lg.GEMM_KERNEL_MFMA_RING,
                      tile=29)
    assert s == 0 and p.kernel == lg.GEMM_KERNEL_MFMA_RING and p.tile == 29 and p.grid == 21 * 12 and p.packed == 3


def test_ring_requirements_fall_back_to_staged():
    # misaligned A pointer, odd leading dimension, K tail, small problem, wrong layout
    for kw in (dict(A=A16 + 2), dict(lda=8201), dict(K=8190, lda=8192, ldb=8192), dict(M=100),
               dict(la=COL, lda=8192)):
        args = dict(in_t=BF16, c_t=BF16, la=ROW, lb=COL, M=8192, N=8192, K=8192)
        args.update(kw)
        s, p = plan(**args)
        assert s == 0 and p.kernel == lg.GEMM_KERNEL_MFMA_STAGED, kw


def test_fp32_ring_needs_an_aligned_last_column_tile():
    # row-major B: the shifted last column tile starts at N - bn, which must be 16-byte aligned
    s, p = plan(F32, F32, ROW, ROW, 300, 257, 48, ldb=260)
    assert s == 0 and p.kernel == lg.GEMM_KERNEL_VALU_STAGED
    s, _ = plan(F32, F32, ROW, ROW, 300, 257, 48, ldb=260, kernel=lg.GEMM_KERNEL_VALU_RING)
    assert s == lg.GEMM_ERR_UNSUPPORTED
    s, p = plan(F32, F32, ROW, ROW, 300, 260, 48, kernel=lg.GEMM_KERNEL_VALU_RING)
    assert s == 0 and p.kernel == lg.GEMM_KERNEL_VALU_RING


def test_lds_budget():
    # 256x256x32 tile: 32 KiB per slot; 4 slots fit, 5 exactly fill 160 KiB but are not built
    s, p = plan(BF16, BF16, ROW, COL, 8192, 8192, 8192, kernel=lg.GEMM_KERNEL_MFMA_RING, tile=2, nstage=4)
    assert s == 0 and p.lds_bytes == 4 * 32768
    s, _ = plan(BF16, BF16, ROW, COL, 8192, 8192, 8192, kernel=lg.GEMM_KERNEL_MFMA_RING, tile=1, nstage=3)
    assert s == lg.GEMM_ERR_UNSUPPORTED       # 3 x 64 KiB > 160 KiB
    s, _ = plan(F32, F32, ROW, ROW, 512, 512, 512, kernel=lg.GEMM_KERNEL_VALU_RING, tile=1, nstage=5)
    assert s == lg.GEMM_ERR_UNSUPPORTED


def test_split_tiles_keep_lds_for_the_c_tile():
    # a 16-bit C of 256 columns is staged through LDS after the K loop: the one-slot ring of
    # the 256x256 split tile still allocates the 128 KiB C tile; an fp32 C does not
    s, p = plan(BF16, BF16, ROW, COL, 8192, 8192, 8192, kernel=lg.GEMM_KERNEL_MFMA_RING, tile=24, nstage=1)
    assert s == 0 and p.lds_bytes == 256 * 256 * 2
    s, p = plan(BF16, F32, ROW, COL, 8192, 8192, 8192, kernel=lg.GEMM_KERNEL_MFMA_RING, tile=24, nstage=1)
    assert s == 0 and p.lds_bytes == (256 + 256) * 64 * 2
    s, p = plan(BF16, BF16, ROW, COL, 8192, 8192, 8192, kernel=lg.GEMM_KERNEL_MFMA_RING, tile=24, nstage=1,
                flags=lg.GEMM_FLAG_EQUAL_LDS)
    assert s == 0 and p.lds_bytes == 2 * (256 + 256) * 64 * 2   # the 2-slot ring: no padding needed


def test_forced_kernels_and_stages():
    for S in (1, 2, 3, 4):
        s, p = plan(F32, F32, ROW, ROW, 4096, 4096, 4096, kernel=lg.GEMM_KERNEL_VALU_RING, nstage=S)
        assert s == 0 and p.nstage == S and p.lds_bytes == S * (128 * 16 + 16 * 64) * 4
    s, p = plan(F32, F32, COL, COL, 100, 70, 33, kernel=lg.GEMM_KERNEL_VALU_STAGED, nstage=1)
    assert s == 0 and p.kernel == lg.GEMM_KERNEL_VALU_STAGED and p.nstage == 1


def test_pipe_copy_rejects_bad_arguments_before_launching():
    """Every error path of gemm_pipe_copy returns before any HIP call (runs without a GPU)."""
    S = 16384
    cases = [
        (A16, B16, -S, 2, lg.GEMM_ERR_INVALID_ARG),          # negative size
        (A16, B16, S + 16, 2, lg.GEMM_ERR_INVALID_ARG),      # not a multiple of a slab
        (A16, B16, S, 5, lg.GEMM_ERR_UNSUPPORTED),           # stage count
        (A16, B16, S, -1, lg.GEMM_ERR_UNSUPPORTED),
        (0, B16, S, 2, lg.GEMM_ERR_INVALID_ARG),             # NULL
        (A16, 0, S, 2, lg.GEMM_ERR_INVALID_ARG),
        (A16 + 4, B16, S, 2, lg.GEMM_ERR_INVALID_ARG),       # alignment
        (A16, A16 + S // 2, S, 2, lg.GEMM_ERR_INVALID_ARG),  # overlap
    ]
    for dst, src, n, st, want in cases:
        assert lg.gemm_pipe_copy(dst, src, n, st) == want, (dst, src, n, st)
        assert lg.gemm_last_error()
    assert lg.gemm_pipe_copy(0, 0, 0, 2) == lg.GEMM_OK       # empty copy: nothing launched


def test_mfma_ceiling_rejects_bad_arguments_before_launching():
    """Every error path of gemm_mfma_ceiling returns before any HIP call (runs without a GPU)."""
    cases = [
        (lg.GEMM_F32, 16, A16, C16, 1, 1, lg.GEMM_ERR_UNSUPPORTED),     # fp32 has no matrix instruction here
        (7, 16, A16, C16, 1, 1, lg.GEMM_ERR_UNSUPPORTED),
        (BF16, 8, A16, C16, 1, 1, lg.GEMM_ERR_UNSUPPORTED),             # shape
        (BF16, 64, A16, C16, 1, 1, lg.GEMM_ERR_UNSUPPORTED),
        (BF16, 16, A16, C16, 0, 1, lg.GEMM_ERR_INVALID_ARG),            # grid
        (BF16, 16, A16, C16, lg.GEMM_CEIL_MAX_GRID + 1, 1, lg.GEMM_ERR_INVALID_ARG),
        (BF16, 16, A16, C16, 1, -1, lg.GEMM_ERR_INVALID_ARG),           # iters
        (BF16, 16, 0, C16, 1, 1, lg.GEMM_ERR_INVALID_ARG),              # NULL
        (BF16, 32, A16, 0, 1, 1, lg.GEMM_ERR_INVALID_ARG),
        (lg.GEMM_F16, 16, A16 + 8, C16, 1, 1, lg.GEMM_ERR_INVALID_ARG),  # alignment
        (lg.GEMM_F16, 32, A16, C16 + 2, 1, 1, lg.GEMM_ERR_INVALID_ARG),
    ]
    for t, shape, fr, sums, grid, iters, want in cases:
        assert lg.gemm_mfma_ceiling(t, shape, fr, sums, grid, iters) == want, (t, shape, fr, sums, grid, iters)
        assert lg.gemm_last_error()


def test_tune_rejects_bad_arguments_before_launching():
    import ctypes
    lib = lg.load()
    best = lg.GemmOpts()
    ms = ctypes.c_float()
    args = (BF16, BF16, ROW, COL, 256, 256, 256, 1.0, A16, 256, B16, 256, 0.0, C16, 256, None)
    assert lib.gemm_tune(*args, 0, ctypes.byref(best), ctypes.byref(ms)) == lg.GEMM_ERR_INVALID_ARG
    assert lib.gemm_tune(*args, 5, None, ctypes.byref(ms)) == lg.GEMM_ERR_INVALID_ARG
    assert lib.gemm_tune(*args, 5, ctypes.byref(best), None) == lg.GEMM_ERR_INVALID_ARG
    bad_type = (7,) + args[1:]
    assert lib.gemm_tune(*bad_type, 5, ctypes.byref(best), ctypes.byref(ms)) == lg.GEMM_ERR_INVALID_ARG
    bad_c = (BF16, F16) + args[2:]
    assert lib.gemm_tune(*bad_c, 5, ctypes.byref(best), ctypes.byref(ms)) == lg.GEMM_ERR_INVALID_ARG
    bad_ld = args[:9] + (100,) + args[10:]     # lda < K
    assert lib.gemm_tune(*bad_ld, 5, ctypes.byref(best), ctypes.byref(ms)) == lg.GEMM_ERR_INVALID_ARG


def test_equal_lds_flag_pads_to_the_deepest_ring():
    """GEMM_FLAG_EQUAL_LDS gives every stage count the LDS of the tile's deepest ring."""
    deepest = None
    for S in (1, 2, 3, 4):
        s, p = plan(F32, F32, ROW, ROW, 4096, 4096, 4096, nstage=S, kernel=lg.GEMM_KERNEL_VALU_RING, tile=1,
                    flags=lg.GEMM_FLAG_EQUAL_LDS)
        assert s == 0
        deepest = deepest or p.lds_bytes
        assert p.lds_bytes == deepest == 4 * (128 * 16 + 16 * 64) * 4
        s, q = plan(F32, F32, ROW, ROW, 4096, 4096, 4096, nstage=S, kernel=lg.GEMM_KERNEL_VALU_RING, tile=1)
        assert q.lds_bytes == S * (128 * 16 + 16 * 64) * 4
    s, p = plan(BF16, BF16, ROW, COL, 8192, 8192, 8192, nstage=1, kernel=lg.GEMM_KERNEL_MFMA_RING, tile=18,
                flags=lg.GEMM_FLAG_EQUAL_LDS)
    assert s == 0 and p.lds_bytes == 3 * (256 + 128) * 64 * 2 <= 163840
    s, _ = plan(BF16, BF16, ROW, COL, 8192, 8192, 8192, flags=8)
    assert s == lg.GEMM_ERR_INVALID_ARG


def ws_size(in_t, c_t, la, lb, M, N, K, alpha=1.0, A=A16, lda=None, B=B16, ldb=None, beta=0.0, C=C16, ldc=None,
            **opts):
    lda = lda if lda is not None else (K if la == ROW else M)
    ldb = ldb if ldb is not None else (N if lb == ROW else K)
    ldc = ldc if ldc is not None else N
    o = lg.GemmOpts(opts.get("nstage", 0), opts.get("kernel", 0), opts.get("tile", 0), opts.get("flags", 0)) \
        if opts else None
    return lg.gemm_workspace_size(in_t, c_t, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, o)


def test_workspace_size_of_the_irregular_workload():
    # bf16 4000x3000x2049 NN: read in place by tile 30, nothing to rewrite
    s, n, p = ws_size(BF16, F32, ROW, ROW, 4000, 3000, 2049, alpha=0.5, beta=1.0)
    assert s == 0 and n == 0 and p.packed == 0 and p.tile == 30
    # with the split tile forced: both operands rewritten, K padded to 2112
    s, n, p = ws_size(BF16, F32, ROW, ROW, 4000, 3000, 2049, alpha=0.5, beta=1.0, kernel=lg.GEMM_KERNEL_MFMA_RING,
                      tile=29)
    assert s == 0 and p.packed == 3 and p.kernel == lg.GEMM_KERNEL_MFMA_RING and p.bk in (32, 64)
    assert n == 4000 * 2112 * 2 + 3000 * 2112 * 2


def test_row_major_ring_requirements():
    """Tile 30 reads row-major A and B in place: any A pitch, K tail; B rows 16-byte
    aligned and N a multiple of 8; enough tiles, else the staged kernel."""
    args = dict(in_t=BF16, c_t=F32, la=ROW, lb=ROW, M=4000, N=3000, K=2049)
    s, p = plan(**args)
    assert s == 0 and p.tile == 30 and p.kernel == lg.GEMM_KERNEL_MFMA_RING
    for kw in (dict(N=3004, ldb=3004), dict(ldb=3001), dict(B=B16 + 2), dict(M=500, N=500), dict(la=COL, lda=4000)):
        a = dict(args)
        a.update(kw)
        s, p = plan(**a)
        assert s == 0 and p.kernel == lg.GEMM_KERNEL_MFMA_STAGED, kw
    s, p = plan(**dict(args, lda=2050, K=2050))
    assert s == 0 and p.tile == 30
    s, _ = plan(BF16, BF16, ROW, COL, 8192, 8192, 8192, kernel=lg.GEMM_KERNEL_MFMA_RING, tile=30)
    assert s == lg.GEMM_ERR_UNSUPPORTED and "row-major" in lg.gemm_last_error()
    s, p = plan(**dict(args, kernel=lg.GEMM_KERNEL_MFMA_RING, tile=30, nstage=1))
    assert s == 0 and p.nstage == 1


def test_workspace_size_rewrites_only_what_the_ring_cannot_read():
    M, N, K = 1024, 768, 512
    # K-contiguous, aligned, K a multiple of 64: nothing to rewrite
    s, n, p = ws_size(BF16, BF16, ROW, COL, M, N, K)
    assert s == 0 and n == 0 and p.packed == 0 and p.kernel == lg.GEMM_KERNEL_MFMA_RING
    # A's pitch off 16 bytes: A only
    s, n, p = ws_size(BF16, BF16, ROW, COL, M, N, K, lda=K + 1)
    assert s == 0 and p.packed == 1 and n == M * K * 2
    # A's base off 16 bytes: A only
    s, n, p = ws_size(F16, F16, ROW, COL, M, N, K, A=A16 + 2)
    assert s == 0 and p.packed == 1 and n == M * K * 2
    # B row-major (N-contiguous): B only
    s, n, p = ws_size(F16, F32, ROW, ROW, M, N, K)
    assert s == 0 and p.packed == 2 and n == N * K * 2
    # A column-major: A only
    s, n, p = ws_size(BF16, F32, COL, COL, M, N, K)
    assert s == 0 and p.packed == 1 and n == M * K * 2
    # K tail: both, K rounded up to 64; sizes rounded up to 256 bytes
    s, n, p = ws_size(BF16, BF16, ROW, COL, 1001, 777, 100)
    assert s == 0 and p.packed == 3 and n == (-(-1001 * 128 * 2 // 256) * 256) + (-(-777 * 128 * 2 // 256) * 256)


def test_workspace_size_zero_where_the_ring_does_not_apply():
    for kw in (dict(in_t=F32, c_t=F32, la=ROW, lb=ROW),                     # fp32: VALU kernels
               dict(in_t=BF16, c_t=BF16, la=ROW, lb=ROW, M=100),             # smaller than any ring tile
               dict(in_t=BF16, c_t=BF16, la=ROW, lb=ROW, kernel=lg.GEMM_KERNEL_MFMA_STAGED),
               dict(in_t=BF16, c_t=BF16, la=ROW, lb=ROW, K=0, lda=1),        # only scales C
               dict(in_t=BF16, c_t=BF16, la=ROW, lb=ROW, alpha=0.0)):
        args = dict(M=1024, N=1024, K=1000)
        args.update(kw)
        s, n, p = ws_size(**args)
        assert s == 0 and n == 0 and p.packed == 0, kw
    # a forced ring with a layout it cannot read: planned on the rewritten operands
    s, n, p = ws_size(BF16, BF16, ROW, ROW, 1024, 1024, 1000, kernel=lg.GEMM_KERNEL_MFMA_RING, tile=3)
    assert s == 0 and p.packed == 3 and p.tile == 3 and n > 0


def test_workspace_argument_errors():
    s, n, p = ws_size(BF16, BF16, ROW, ROW, 1024, 1024, 1000, lda=10)
    assert s == lg.GEMM_ERR_INVALID_ARG
    s = lg.load().gemm_workspace_size(BF16, BF16, ROW, ROW, 64, 64, 64, 1.0, A16, 64, B16, 64, 0.0, C16, 64,
                                      None, None, None)
    assert s == lg.GEMM_ERR_INVALID_ARG
    # a workspace off 256 bytes is refused before anything is enqueued
    s = lg.gemm_bf16_ws(ROW, ROW, 1024, 1024, 1000, 1.0, A16, 1000, B16, 1024, 0.0, C16, BF16, 1024, 0, None,
                        A16 + 16, 1 << 30)
    assert s == lg.GEMM_ERR_INVALID_ARG and "aligned" in lg.gemm_last_error()
    # the workspace tuner refuses fp32 input and a misaligned workspace before timing anything
    best, ms = lg.GemmOpts(), ctypes.c_float(0.0)
    s = lg.load().gemm_tune_ws(F32, F32, ROW, ROW, 64, 64, 64, 1.0, A16, 64, B16, 64, 0.0, C16, 64, None,
                               A16, 1 << 20, 2, ctypes.byref(best), ctypes.byref(ms))
    assert s == lg.GEMM_ERR_INVALID_ARG
    s = lg.load().gemm_tune_ws(BF16, BF16, ROW, ROW, 64, 64, 64, 1.0, A16, 64, B16, 64, 0.0, C16, 64, None,
                               A16 + 16, 1 << 20, 2, ctypes.byref(best), ctypes.byref(ms))
    assert s == lg.GEMM_ERR_INVALID_ARG and "aligned" in lg.gemm_last_error()


def test_h2d_staged_rejects_bad_arguments_before_copying():
    H = 0x40000  # fake addresses: every case fails before anything is touched
    for args, want in (((A16, H, -1, H + (1 << 20), 4096, 2), lg.GEMM_ERR_INVALID_ARG),
                       ((A16, H, 8192, H + (1 << 20), 0, 2), lg.GEMM_ERR_INVALID_ARG),
                       ((A16, H, 8192, H + (1 << 20), 4096, 0), lg.GEMM_ERR_UNSUPPORTED),
                       ((A16, H, 8192, H + (1 << 20), 4096, 5), lg.GEMM_ERR_UNSUPPORTED),
                       ((0, H, 8192, H + (1 << 20), 4096, 2), lg.GEMM_ERR_INVALID_ARG),
                       ((A16, H, 8192, 0, 4096, 2), lg.GEMM_ERR_INVALID_ARG),
                       ((A16, H, 8192, H + 4096, 4096, 2), lg.GEMM_ERR_INVALID_ARG)):  # src overlaps the ring
        assert lg.gemm_h2d_staged(*args) == want, args
        assert lg.gemm_h2d_staged_async(*args) == want, args
    assert lg.gemm_h2d_staged(A16, H, 0, H + (1 << 20), 4096, 2) == lg.GEMM_OK   # nothing to copy
    assert lg.gemm_h2d_staged_async(A16, H, 0, H + (1 << 20), 4096, 2) == lg.GEMM_OK


# --------------------------------------------------------------- failure paths without a GPU

def _no_gpu_here():
    import torch
    return torch.cuda.device_count() == 0   # counts devices without initialising HIP


@pytest.mark.skipif(not _no_gpu_here(), reason="needs a host without a GPU: the calls below pass fake device "
                                                "addresses that a real launch would dereference")
def test_launch_without_a_device_reports_hip_error():
    """With no GPU present the HIP runtime refuses every launch: each entry point returns
    GEMM_ERR_HIP with the runtime's message, after its own argument checks passed."""
    cases = [
        ("gemm_f32", lambda: lg.gemm_f32(ROW, ROW, 256, 256, 256, 1.0, A16, 256, B16, 256, 0.0, C16, 256)),
        ("gemm_bf16 ring", lambda: lg.gemm_bf16(ROW, COL, 512, 512, 512, 1.0, A16, 512, B16, 512, 0.0, C16,
                                                 lg.GEMM_BF16, 512)),
        ("gemm_f16 staged", lambda: lg.gemm_f16(COL, ROW, 100, 70, 33, 1.0, A16, 100, B16, 70, 0.5, C16,
                                                 lg.GEMM_F32, 70)),
        ("scale", lambda: lg.gemm_bf16(ROW, COL, 64, 64, 0, 1.0, A16, 1, B16, 1, 0.5, C16, lg.GEMM_F32, 64)),
        ("gemm_bf16_ws pack", lambda: lg.gemm_bf16_ws(ROW, ROW, 4000, 3000, 2049, 0.5, A16, 2049, B16, 3000, 1.0,
                                                     C16, lg.GEMM_F32, 3000, 0, None, 0x40000000, 1 << 26)),
        ("gemm_pipe_copy", lambda: lg.gemm_pipe_copy(A16, 0x800000, 1 << 16, 2)),
        ("gemm_mfma_ceiling", lambda: lg.gemm_mfma_ceiling(BF16, 16, A16, C16, 4, 1)),
    ]
    for name, call in cases:
        s = call()
        msg = lg.gemm_last_error()
        assert s == lg.GEMM_ERR_HIP, (name, s, msg)
        assert msg and ("fail" in msg or "error" in msg.lower()), (name, msg)
    # the tuner's event creation or first launch fails the same way, before any timing
    best, ms = lg.GemmOpts(), ctypes.c_float(0)
    s = lg.load().gemm_tune(BF16, BF16, ROW, COL, 512, 512, 512, 1.0, A16, 512, B16, 512, 0.0, C16, 512, None, 2,
                            ctypes.byref(best), ctypes.byref(ms))
    assert s == lg.GEMM_ERR_HIP and lg.gemm_last_error()
    # a later call's own argument error still wins over the missing device
    assert lg.gemm_f32(ROW, ROW, -1, 1, 1, 1.0, A16, 1, B16, 1, 0.0, C16, 1) == lg.GEMM_ERR_INVALID_ARG


def test_matmul_rejects_overlapping_c_before_any_launch():
    """An expanded (stride 0) or row-overlapping C view would make the kernels write past
    its storage: the binding refuses it before calling the library."""
    import torch
    A = torch.zeros(4, 8, dtype=torch.bfloat16)
    B = torch.zeros(8, 8, dtype=torch.bfloat16)
    for C in (torch.empty(1, 8).expand(4, 8), torch.empty(40).as_strided((4, 8), (4, 1)),
              torch.empty(1, 1).expand(4, 1)):
        Bv = B if C.shape[1] == 8 else B[:, :1]
        with pytest.raises(ValueError, match="overlap"):
            lg.matmul(A, Bv, C=C)


def test_static_workspace_entry_rejects_before_touching_the_device():
    """gemm_ws_static: argument errors and a rewrite larger than the static array are
    refused before any device call (so this runs without a GPU)."""
    big = lg.gemm_ws_static(BF16, COL, ROW, 8192, 8192, 8192, 1.0, A16, 8192, B16, 8192, 0.0, C16, BF16, 8192)
    assert big == lg.GEMM_ERR_UNSUPPORTED and "static workspace" in lg.gemm_last_error()
    s, n, _ = ws_size(BF16, BF16, COL, ROW, 8192, 8192, 8192)
    assert s == 0 and n > lg.GEMM_STATIC_WS_BYTES
    assert lg.gemm_ws_static(F32, ROW, ROW, 64, 64, 64, 1.0, A16, 64, B16, 64, 0.0, C16, F32, 64) == \
        lg.GEMM_ERR_INVALID_ARG
    assert lg.gemm_ws_static(BF16, ROW, ROW, 64, 64, 64, 1.0, A16, 64, B16, 64, 0.0, C16, F16, 64) == \
        lg.GEMM_ERR_INVALID_ARG
    assert lg.gemm_ws_static(F16, ROW, ROW, -1, 64, 64, 1.0, A16, 64, B16, 64, 0.0, C16, F16, 64) == \
        lg.GEMM_ERR_INVALID_ARG
    assert lg.gemm_ws_static(BF16, ROW, ROW, 0, 64, 64, 1.0, A16, 64, B16, 64, 0.0, C16, F32, 64) == lg.GEMM_OK
    # the irregular-tail workload, rewritten for the split tile, fits
    s, n, _ = ws_size(BF16, F32, ROW, ROW, 4000, 3000, 2049, alpha=0.5, lda=2049, beta=1.0,
                      kernel=lg.GEMM_KERNEL_MFMA_RING, tile=29)
    assert s == 0 and 0 < n <= lg.GEMM_STATIC_WS_BYTES


def test_debug_env_prints_every_choice_and_error():
    """GEMM_DEBUG=1: each plan is described on stderr (kernel, tile, stage count, why the
    direct ring was passed over), and so is a refused call; without it, nothing is printed."""
    import subprocess
    import sys
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from tiled_stage_software_amd import libgemm as lg\n"
        "lg.gemm_plan(1, 1, 0, 1, 8192, 8192, 8192, 1.0, 16, 8192, 16, 8192, 0.0, 16, 8192, None)\n"
        "lg.gemm_plan(1, 1, 1, 1, 512, 512, 512, 1.0, 16, 512, 16, 512, 0.0, 16, 512, None)\n"
        "lg.gemm_plan(0, 0, 0, 0, 64, 64, 64, 1.0, 16, 64, 16, 64, 0.0, 16, 64, lg.GemmOpts(9, 0, 0, 0))\n"
    ) % ROOT
    env = dict(os.environ, GEMM_DEBUG="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("libgemm:")]
    assert any("M=8192 N=8192 K=8192" in l and "-> mfma_ring tile 31" in l and "nstage 2" in l for l in lines), lines
    assert any("-> mfma_staged" in l and "direct ring passed over: needs A row-major and B column-major" in l
               for l in lines), lines
    assert any("status 2" in l and "nstage 9" in l for l in lines), lines
    env.pop("GEMM_DEBUG")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "libgemm:" not in r.stderr


def test_poison_flag_is_planned_only_where_its_variant_is_built():
    """GEMM_FLAG_POISON_LDS: the fp32 ring tiles 5 and 10 and the bf16 tiles 31 / 30 plan with
    it; anything else is refused before a launch."""
    P = lg.GEMM_FLAG_POISON_LDS
    s, p = plan(BF16, BF16, ROW, COL, 8192, 8192, 8192, flags=P)
    assert s == 0 and p.tile == 31
    assert plan(BF16, BF16, ROW, COL, 8192, 8192, 8192, kernel=lg.GEMM_KERNEL_MFMA_RING, tile=24,
                flags=P)[0] == lg.GEMM_ERR_UNSUPPORTED                                       # not the default tile
    s, p = plan(BF16, F32, ROW, ROW, 4000, 3000, 2049, alpha=0.5, beta=1.0, lda=2049, flags=P)
    assert s == 0 and p.tile == 30
    s, p = plan(F32, F32, ROW, ROW, 4096, 4096, 4096, flags=P)
    assert s == 0 and p.kernel == lg.GEMM_KERNEL_VALU_RING and p.tile == 10
    for S in (1, 2, 3, 4):
        assert plan(F32, F32, ROW, ROW, 4096, 4096, 4096, nstage=S, flags=P)[0] == 0
        assert plan(F32, F32, ROW, ROW, 4096, 4096, 4096, kernel=lg.GEMM_KERNEL_VALU_RING, tile=5, nstage=S,
                    flags=P)[0] == 0
    assert plan(F32, F32, ROW, ROW, 2048, 2048, 2048, kernel=lg.GEMM_KERNEL_VALU_RING, tile=11,
                flags=P)[0] == lg.GEMM_ERR_UNSUPPORTED                                          # tile 11
    assert plan(F16, F16, ROW, COL, 8192, 8192, 8192, flags=P)[0] == lg.GEMM_ERR_UNSUPPORTED   # not built for f16
    assert plan(F32, F32, ROW, ROW, 256, 256, 256, flags=P)[0] == lg.GEMM_ERR_UNSUPPORTED      # small tile 9
    assert plan(BF16, BF16, COL, COL, 512, 512, 512, flags=P)[0] == lg.GEMM_ERR_UNSUPPORTED    # staged kernel
