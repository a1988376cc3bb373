"""ctypes binding of libgemm.so -- argument marshalling only.

The functions named like the C ABI (``gemm_f32``, ``gemm_bf16``, ``gemm_f16``, their
``_ex`` forms, ``gemm_plan``, ``gemm_schedule``, ``gemm_status_string``,
``gemm_last_error``) take plain integers for device pointers and return the status
code.  ``matmul`` is a convenience wrapper over torch tensors: it reads the layout and
leading dimension of each operand from its strides and passes ``data_ptr()`` and the
current HIP stream; every step of the computation runs in the library's kernels.

There is no fallback: if libgemm.so cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libgemm.so")

GEMM_OK, GEMM_ERR_INVALID_ARG, GEMM_ERR_UNSUPPORTED, GEMM_ERR_HIP = 0, 1, 2, 3
GEMM_ROW_MAJOR, GEMM_COL_MAJOR = 0, 1
GEMM_F32, GEMM_BF16, GEMM_F16 = 0, 1, 2
(GEMM_KERNEL_AUTO, GEMM_KERNEL_VALU_RING, GEMM_KERNEL_VALU_STAGED, GEMM_KERNEL_MFMA_RING,
 GEMM_KERNEL_MFMA_STAGED, GEMM_KERNEL_SCALE) = range(6)
GEMM_FLAG_NO_XCD_REMAP = 1
GEMM_FLAG_EQUAL_LDS = 2
GEMM_FLAG_POISON_LDS = 4
GEMM_MAX_NSTAGE = 4
GEMM_STATIC_WS_BYTES = 33554432
GEMM_CEIL_THREADS = 512
GEMM_CEIL_FRAG_ELEMS = 16384
GEMM_CEIL_MAX_GRID = 65536

KERNEL_NAMES = {0: "none", 1: "valu_ring", 2: "valu_staged", 3: "mfma_ring", 4: "mfma_staged", 5: "scale"}

# Symbols declared in include/libgemm.h.
EXPORTS = ("gemm_f32", "gemm_bf16", "gemm_f16", "gemm_f32_ex", "gemm_bf16_ex", "gemm_f16_ex",
           "gemm_bf16_ws", "gemm_f16_ws", "gemm_ws_static", "gemm_workspace_size", "gemm_plan", "gemm_tune", "gemm_tune_ws",
           "gemm_schedule", "gemm_pipe_copy", "gemm_mfma_ceiling", "gemm_h2d_staged", "gemm_h2d_staged_async", "gemm_status_string",
           "gemm_last_error")


class GemmOpts(ctypes.Structure):
    _fields_ = [("nstage", ctypes.c_int), ("kernel", ctypes.c_int), ("tile", ctypes.c_int),
                ("flags", ctypes.c_int)]


class GemmPlan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("nstage", ctypes.c_int), ("tile", ctypes.c_int),
                ("bm", ctypes.c_int), ("bn", ctypes.c_int), ("bk", ctypes.c_int),
                ("threads", ctypes.c_int), ("lds_bytes", ctypes.c_int), ("grid", ctypes.c_int64),
                ("packed", ctypes.c_int)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["kernel_name"] = KERNEL_NAMES.get(self.kernel, str(self.kernel))
        return d


class GemmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_name(status)}: {msg}")
        self.status = status


_lock = threading.Lock()
_lib = None


def load():
    """Load libgemm.so (built in-tree by ``tiled_stage_software_amd.build``)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(LIB_PATH)
        i64, vp, i32, f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        base = [i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp]
        lib.gemm_f32.argtypes = base + [i64, vp]
        lib.gemm_f32_ex.argtypes = base + [i64, vp, ctypes.POINTER(GemmOpts)]
        for name in ("gemm_bf16", "gemm_f16"):
            getattr(lib, name).argtypes = base + [i32, i64, vp]
            getattr(lib, name + "_ex").argtypes = base + [i32, i64, vp, ctypes.POINTER(GemmOpts)]
            getattr(lib, name + "_ws").argtypes = base + [i32, i64, vp, ctypes.POINTER(GemmOpts), vp,
                                                          ctypes.c_size_t]
        for name in ("gemm_f32", "gemm_bf16", "gemm_f16", "gemm_f32_ex", "gemm_bf16_ex", "gemm_f16_ex",
                     "gemm_bf16_ws", "gemm_f16_ws"):
            getattr(lib, name).restype = i32
        lib.gemm_ws_static.argtypes = [i32] + base + [i32, i64, vp, ctypes.POINTER(GemmOpts)]
        lib.gemm_ws_static.restype = i32
        lib.gemm_workspace_size.argtypes = [i32, i32, i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp,
                                            i64, ctypes.POINTER(GemmOpts), ctypes.POINTER(ctypes.c_size_t),
                                            ctypes.POINTER(GemmPlan)]
        lib.gemm_workspace_size.restype = i32
        lib.gemm_plan.argtypes = [i32, i32, i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64,
                                  ctypes.POINTER(GemmOpts), ctypes.POINTER(GemmPlan)]
        lib.gemm_plan.restype = i32
        lib.gemm_schedule.argtypes = [i32, i32, i32, i32, ctypes.POINTER(ctypes.c_int), i32]
        lib.gemm_schedule.restype = i32
        lib.gemm_tune.argtypes = [i32, i32, i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64,
                                  vp, i32, ctypes.POINTER(GemmOpts), ctypes.POINTER(ctypes.c_float)]
        lib.gemm_tune.restype = i32
        lib.gemm_tune_ws.argtypes = [i32, i32, i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64,
                                     vp, vp, ctypes.c_size_t, i32, ctypes.POINTER(GemmOpts),
                                     ctypes.POINTER(ctypes.c_float)]
        lib.gemm_tune_ws.restype = i32
        lib.gemm_pipe_copy.argtypes = [vp, vp, i64, i32, vp]
        lib.gemm_pipe_copy.restype = i32
        lib.gemm_mfma_ceiling.argtypes = [i32, i32, vp, vp, i64, i64, vp]
        lib.gemm_mfma_ceiling.restype = i32
        for name in ("gemm_h2d_staged", "gemm_h2d_staged_async"):
            getattr(lib, name).argtypes = [vp, vp, i64, vp, i64, i32, vp]
            getattr(lib, name).restype = i32
        lib.gemm_status_string.argtypes = [i32]
        lib.gemm_status_string.restype = ctypes.c_char_p
        lib.gemm_last_error.argtypes = []
        lib.gemm_last_error.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _opts(nstage=0, kernel=0, tile=0, flags=0) -> Optional[GemmOpts]:
    if not (nstage or kernel or tile or flags):
        return None
    return GemmOpts(int(nstage), int(kernel), int(tile), int(flags))


def _ref(o):
    return ctypes.byref(o) if o is not None else None


# ------------------------------------------------------------------ C ABI names

def gemm_f32(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    return load().gemm_f32(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def gemm_bf16(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream=0) -> int:
    return load().gemm_bf16(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream)


def gemm_f16(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream=0) -> int:
    return load().gemm_f16(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream)


def gemm_f32_ex(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0, opts=None) -> int:
    return load().gemm_f32_ex(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, _ref(opts))


def gemm_bf16_ex(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream=0, opts=None) -> int:
    return load().gemm_bf16_ex(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream, _ref(opts))


def gemm_f16_ex(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream=0, opts=None) -> int:
    return load().gemm_f16_ex(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream, _ref(opts))


def gemm_bf16_ws(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream=0, opts=None,
                 workspace=0, workspace_bytes=0) -> int:
    return load().gemm_bf16_ws(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream, _ref(opts),
                               workspace, workspace_bytes)


def gemm_f16_ws(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream=0, opts=None,
                workspace=0, workspace_bytes=0) -> int:
    return load().gemm_f16_ws(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream, _ref(opts),
                              workspace, workspace_bytes)


def gemm_ws_static(in_type, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream=0, opts=None) -> int:
    """gemm_bf16_ws / gemm_f16_ws with the library's static workspace (allocates nothing)."""
    return load().gemm_ws_static(in_type, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream,
                                 _ref(opts))


def gemm_workspace_size(in_type, c_type, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, opts=None):
    """Returns (status, bytes, GemmPlan of the call given that many bytes)."""
    n = ctypes.c_size_t(0)
    plan = GemmPlan()
    s = load().gemm_workspace_size(in_type, c_type, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                   _ref(opts), ctypes.byref(n), ctypes.byref(plan))
    return s, n.value, plan


def gemm_plan(in_type, c_type, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, opts=None):
    """Returns (status, GemmPlan)."""
    plan = GemmPlan()
    s = load().gemm_plan(in_type, c_type, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                         _ref(opts), ctypes.byref(plan))
    return s, plan


def gemm_schedule(kernel, nstage, num_k, ksteps):
    """Event list [(type, slab, slot, arg), ...] of the kernel family's K loop, or None."""
    lib = load()
    n = lib.gemm_schedule(kernel, nstage, num_k, ksteps, None, 0)
    if n < 0:
        return None
    buf = (ctypes.c_int * (4 * max(n, 1)))()
    lib.gemm_schedule(kernel, nstage, num_k, ksteps, buf, n)
    return [tuple(buf[4 * i:4 * i + 4]) for i in range(n)]


def gemm_tune(in_type, c_type, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0, reps=10):
    """(status, GemmOpts of the fastest variant, its ms per call) -- see include/libgemm.h."""
    best = GemmOpts()
    ms = ctypes.c_float(0.0)
    s = load().gemm_tune(in_type, c_type, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, reps,
                         ctypes.byref(best), ctypes.byref(ms))
    return s, best, ms.value


def gemm_tune_ws(in_type, c_type, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0,
                 workspace=0, workspace_bytes=0, reps=10):
    """gemm_tune for the workspace entry points: (status, GemmOpts, ms per call)."""
    best = GemmOpts()
    ms = ctypes.c_float(0.0)
    s = load().gemm_tune_ws(in_type, c_type, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                            workspace, workspace_bytes, reps, ctypes.byref(best), ctypes.byref(ms))
    return s, best, ms.value


def gemm_pipe_copy(dst: int, src: int, nbytes: int, nstage: int = 0, stream: int = 0) -> int:
    """dst[0, nbytes) = src[0, nbytes) through the nStage LDS ring (device pointers)."""
    return load().gemm_pipe_copy(dst, src, nbytes, nstage, stream)


def gemm_mfma_ceiling(in_type: int, shape: int, frags: int, sums: int, grid: int, iters: int,
                      stream: int = 0) -> int:
    """Matrix instructions on register operands (device pointers): grid * 8 * iters * 2^20
    FLOPs; one fp32 accumulator sum per thread into sums."""
    return load().gemm_mfma_ceiling(in_type, shape, frags, sums, grid, iters, stream)


def gemm_h2d_staged(dst: int, src: int, nbytes: int, staging: int, chunk_bytes: int, nstage: int = 2,
                    stream: int = 0) -> int:
    """dst (device) = src (pageable host) through nstage page-locked staging slots."""
    return load().gemm_h2d_staged(dst, src, nbytes, staging, chunk_bytes, nstage, stream)


def gemm_h2d_staged_async(dst: int, src: int, nbytes: int, staging: int, chunk_bytes: int, nstage: int = 2,
                          stream: int = 0) -> int:
    """gemm_h2d_staged returning before the last DMAs finish (sync `stream` before reusing staging)."""
    return load().gemm_h2d_staged_async(dst, src, nbytes, staging, chunk_bytes, nstage, stream)


def gemm_status_string(s: int) -> str:
    return load().gemm_status_string(int(s)).decode()


def gemm_last_error() -> str:
    return load().gemm_last_error().decode()


def status_name(s: int) -> str:
    try:
        return gemm_status_string(s)
    except Exception:  # library not loadable: still give the number
        return f"status {s}"


def check(status: int):
    if status != GEMM_OK:
        raise GemmError(status, gemm_last_error())


# ------------------------------------------------------------------ torch convenience

def _layout_of(t, rows, cols):
    """(layout, ld) of a 2-D tensor view, or None if it is neither row- nor column-major."""
    s0, s1 = t.stride()
    if cols == 1 and rows == 1:
        return GEMM_ROW_MAJOR, 1
    if s1 == 1 and (rows == 1 or s0 >= cols):
        return GEMM_ROW_MAJOR, max(s0, cols) if rows > 1 else cols
    if s0 == 1 and (cols == 1 or s1 >= rows):
        return GEMM_COL_MAJOR, max(s1, rows) if cols > 1 else rows
    return None


def matmul(A, B, C=None, alpha: float = 1.0, beta: float = 0.0, out_dtype=None, stream=None,
           nstage: int = 0, kernel: int = 0, tile: int = 0, flags: int = 0, workspace=None):
    """C = alpha*A@B + beta*C on device tensors (A: M x K, B: K x N, any of the two
    layouts per operand, C row-major).  Returns C.  16-bit inputs: `workspace` (a device
    tensor, 256-byte aligned, at least gemm_workspace_size bytes; "auto" = allocate one
    with torch) lets the direct ring take operands it cannot read in place."""
    import torch
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shapes {tuple(A.shape)} @ {tuple(B.shape)}")
    if A.dtype != B.dtype:
        raise ValueError("A and B must have the same dtype")
    M, K = A.shape
    N = B.shape[1]
    la = _layout_of(A, M, K)
    lb = _layout_of(B, K, N)
    if la is None or lb is None:
        raise ValueError("operands must be row- or column-major views")
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
        if out_dtype is None:
            out_dtype = A.dtype
        C = torch.empty((M, N), dtype=out_dtype, device=A.device)
    if C.dim() != 2 or tuple(C.shape) != (M, N) or (N > 1 and C.stride(1) != 1):
        raise ValueError("C must be an M x N row-major view")
    if M > 1 and C.stride(0) < N:
        # an expanded or row-overlapping view: the kernels would write past its storage
        raise ValueError(f"C rows overlap (stride {C.stride(0)} < N = {N})")
    ldc = C.stride(0) if M > 1 else max(N, 1)
    st = stream if stream is not None else torch.cuda.current_stream(A.device).cuda_stream
    o = _opts(nstage, kernel, tile, flags)
    if A.dtype == torch.float32:
        if C.dtype != torch.float32:
            raise ValueError("fp32 inputs give fp32 C")
        s = gemm_f32_ex(la[0], lb[0], M, N, K, alpha, A.data_ptr(), la[1], B.data_ptr(), lb[1],
                        beta, C.data_ptr(), ldc, st, o)
    elif A.dtype in (torch.bfloat16, torch.float16):
        ct = {torch.float32: GEMM_F32, torch.bfloat16: GEMM_BF16, torch.float16: GEMM_F16}[C.dtype]
        if workspace is None:
            fn = gemm_bf16_ex if A.dtype == torch.bfloat16 else gemm_f16_ex
            s = fn(la[0], lb[0], M, N, K, alpha, A.data_ptr(), la[1], B.data_ptr(), lb[1],
                   beta, C.data_ptr(), ct, ldc, st, o)
        else:
            if isinstance(workspace, str):
                if workspace != "auto":
                    raise ValueError("workspace: a device tensor or 'auto'")
                it = GEMM_BF16 if A.dtype == torch.bfloat16 else GEMM_F16
                s, nbytes, _ = gemm_workspace_size(it, ct, la[0], lb[0], M, N, K, alpha, A.data_ptr(), la[1],
                                                   B.data_ptr(), lb[1], beta, C.data_ptr(), ldc, o)
                check(s)
                workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=A.device)
                if st != torch.cuda.current_stream(A.device).cuda_stream:
                    # the caching allocator orders reuse against the allocating stream only:
                    # tie the block to the stream the pack and the multiply run on, so that
                    # it is not handed out again before they have finished
                    workspace.record_stream(torch.cuda.ExternalStream(st, device=A.device))
            fn = gemm_bf16_ws if A.dtype == torch.bfloat16 else gemm_f16_ws
            s = fn(la[0], lb[0], M, N, K, alpha, A.data_ptr(), la[1], B.data_ptr(), lb[1],
                   beta, C.data_ptr(), ct, ldc, st, o, workspace.data_ptr(),
                   workspace.numel() * workspace.element_size())
    else:
        raise ValueError(f"unsupported dtype {A.dtype}")
    check(s)
    return C


def gemm_operands(in_dtype: str, out_dtype: str, la, lb, M, N, K, alpha, A_ptr, lda, B_ptr, ldb,
                  beta, C_ptr, ldc, stream=0, nstage=0, kernel=0, tile=0, flags=0, ws_ptr=0, ws_bytes=0) -> int:
    """Dispatch on dtype names ('f32' / 'bf16' / 'f16') with raw pointers (16-bit inputs
    with ws_ptr != 0: the workspace entry points)."""
    o = _opts(nstage, kernel, tile, flags)
    if in_dtype == "f32":
        return gemm_f32_ex(la, lb, M, N, K, alpha, A_ptr, lda, B_ptr, ldb, beta, C_ptr, ldc, stream, o)
    ct = {"f32": GEMM_F32, "bf16": GEMM_BF16, "f16": GEMM_F16}[out_dtype]
    if ws_ptr:
        fn = gemm_bf16_ws if in_dtype == "bf16" else gemm_f16_ws
        return fn(la, lb, M, N, K, alpha, A_ptr, lda, B_ptr, ldb, beta, C_ptr, ct, ldc, stream, o, ws_ptr, ws_bytes)
    fn = gemm_bf16_ex if in_dtype == "bf16" else gemm_f16_ex
    return fn(la, lb, M, N, K, alpha, A_ptr, lda, B_ptr, ldb, beta, C_ptr, ct, ldc, stream, o)
