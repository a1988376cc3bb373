/*
 * libgemm.h -- C ABI of the tiled, software-pipelined GEMM library for AMD MI355X (gfx950).
 *
 * Operation (every entry point):   C = alpha * A * B + beta * C
 *
 *   The accumulation C += A * B, looped over the K dimension one tile ("K-slab") at a
 *   time with hierarchical block / wave / thread tiles, is sections 1-4 of the page
 *   "CUTLASS-Cute 初步(6)：CUDA GEMM 计算优化、Multi-Stage 与软流水"; alpha and beta
 *   follow the BLAS convention.  While one K-slab is multiplied out of LDS, the next
 *   slab(s) stream from HBM into other buffers of an nStage LDS ring ("Software
 *   Pipelining and Double Buffering", sections "Double buffering with shared memory"
 *   and "Multi-stage pipelines"; the N-stage ring of "Matrix multiplication").
 *
 * Storage (BLAS index form), all leading dimensions in ELEMENTS:
 *   A (M x K): GEMM_ROW_MAJOR -> A[m*lda + k],  GEMM_COL_MAJOR -> A[k*lda + m]
 *   B (K x N): GEMM_ROW_MAJOR -> B[k*ldb + n],  GEMM_COL_MAJOR -> B[n*ldb + k]
 *   C (M x N): always row-major, C[m*ldc + n]
 *   ("NT" = A row-major, B column-major: both operands K-contiguous.)
 *
 * Arithmetic: products of the inputs are accumulated in fp32.  FP32 inputs use one
 *   fused multiply-add chain per output in ascending k (VALU path).  bf16 / f16 inputs
 *   use the matrix cores (v_mfma_f32_16x16x32_{bf16,f16} in the default 256x256 and
 *   192x256 tiles, v_mfma_f32_32x32x16_{bf16,f16} in the others).  The epilogue computes, in
 *   fp32, alpha*acc when beta == 0 (C is then never read, so NaN in C does not leak)
 *   and fmaf(alpha, acc, beta*C) otherwise, then rounds to the C type with
 *   round-to-nearest-even.  f16 subnormal inputs are not flushed.  The k order seen by
 *   every accumulator does not depend on nstage, so results are bit-identical across
 *   stage counts and across runs.
 *
 * Pointers: A, B and C are DEVICE pointers owned by the caller.  The library allocates
 *   nothing, keeps no pointer after returning and holds no mutable global state apart
 *   from a thread-local error string, a per-device cache of the compute-unit count and,
 *   for gemm_ws_static only, that entry's static device workspace and a per-device cache
 *   of its address (the caches are atomic: first calls from several threads at once are
 *   safe); calls are reentrant and may come from any number of host threads (calls of
 *   gemm_ws_static that may overlap on one GPU must be serialised, see there).  C must not overlap A or B
 *   (not checked).  Misaligned pointers or leading dimensions are never an error: they
 *   select a slower load path, or, given a caller-owned workspace (gemm_*_ws), a
 *   one-pass rewrite of the operands for the fast path.  (gemm_h2d_staged alone takes
 *   host memory.)
 *
 * Streams: the work is enqueued on `stream` (NULL = the null stream) and the call
 *   returns without synchronising.  Faults during execution surface at the caller's
 *   next synchronisation.
 *
 * Errors: argument checks run before anything is launched; on a non-OK status nothing
 *   was enqueued and gemm_last_error() describes the problem.
 *   GEMM_ERR_INVALID_ARG -- negative size, leading dimension below the minimum
 *       (lda >= (la == ROW ? K : M), ldb >= (lb == ROW ? N : K), ldc >= N; each >= 1),
 *       NULL pointer where it would be dereferenced (A and B when alpha != 0 and K > 0;
 *       C when M*N > 0), bad enum value, a C type that the entry point does not offer.
 *   GEMM_ERR_UNSUPPORTED -- gemm_opts_t asks for a kernel / stage count / tile that
 *       cannot run this problem (e.g. the direct-to-LDS ring on a misaligned operand,
 *       or a ring that exceeds the 160 KiB of LDS).
 *   GEMM_ERR_HIP -- the HIP runtime refused the launch (message in gemm_last_error()).
 *   Quick returns (BLAS): M == 0 or N == 0 -> OK, nothing launched.  K == 0 or
 *   alpha == 0 -> C = beta*C (beta == 0 writes zeros without reading C).
 *
 * Debugging: with GEMM_DEBUG set to anything but "" or "0" in the environment (read
 *   once, at the first planning call), every kernel choice is printed to stderr -- the
 *   problem, the kernel family / tile / stage count / grid / LDS picked and, when the
 *   automatic choice passed over the direct global->LDS ring, why -- as is every
 *   non-OK status and every operand rewrite of the workspace path.  Planning probes
 *   (gemm_workspace_size, the tuner, the workspace path's first try) print too.
 */
#ifndef LIBGEMM_H
#define LIBGEMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gemm_status {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = 1,
    GEMM_ERR_UNSUPPORTED = 2,
    GEMM_ERR_HIP = 3
} gemm_status_t;

typedef enum gemm_layout { GEMM_ROW_MAJOR = 0, GEMM_COL_MAJOR = 1 } gemm_layout_t;

typedef enum gemm_dtype { GEMM_F32 = 0, GEMM_BF16 = 1, GEMM_F16 = 2 } gemm_dtype_t;

/* Kernel families (gemm_opts_t.kernel). */
typedef enum gemm_kernel {
    GEMM_KERNEL_AUTO = 0,
    GEMM_KERNEL_VALU_RING = 1,   /* fp32 VALU, direct global->LDS nStage ring (A row-major, B row-major) */
    GEMM_KERNEL_VALU_STAGED = 2, /* fp32 VALU, loads staged through registers, any layout / alignment */
    GEMM_KERNEL_MFMA_RING = 3,   /* bf16/f16 MFMA, direct global->LDS nStage ring (A and B K-contiguous;
                                    tile 30: row-major A of any pitch and row-major B, read as they are) */
    GEMM_KERNEL_MFMA_STAGED = 4, /* bf16/f16 MFMA, loads staged through registers, any layout / alignment */
    GEMM_KERNEL_SCALE = 5        /* C = beta*C only (K == 0 or alpha == 0) */
} gemm_kernel_t;

#define GEMM_MAX_NSTAGE 4

/* Optional knobs for tests and benchmarks.  All-zero = library default. */
typedef struct gemm_opts {
    int nstage; /* 0 = default, else 1..GEMM_MAX_NSTAGE: number of LDS slab buffers.
                   1 = single buffer (load; barrier; compute; barrier), 2 = double buffer,
                   n = n-1 slabs in flight while one is computed. Staged kernels: 1 or 2. */
    int kernel; /* gemm_kernel_t; 0 = automatic choice */
    int tile;   /* 0 = default tile of the kernel family, else a tile id (gemm_plan_t.tile) */
    int flags;  /* GEMM_FLAG_* bits below; other bits must be 0 */
} gemm_opts_t;

/* Plain row-major tile order instead of the grouped, XCD-aware workgroup order (results
 * are unchanged: every output tile is computed the same way wherever it runs). */
#define GEMM_FLAG_NO_XCD_REMAP 1
/* Allocate, whatever the stage count, the LDS of the deepest ring the tile offers, so that
 * nStage variants run at the same occupancy (the fair comparison: at natural occupancy a
 * shallower ring leaves room for more resident workgroups).  Results are unchanged. */
#define GEMM_FLAG_EQUAL_LDS 2
/* Debugging: the LDS-poisoning variant of the ring kernel.  Right after the barrier that
 * releases a ring slot (all its reads done, nothing yet copied into it) the workgroup
 * overwrites the slot with all-ones bits (NaN in bf16, f16 and fp32) and meets at a second
 * barrier before the next copy into it is issued, so a pipeline that read a slot outside
 * its live range would produce NaN instead of a plausible stale value.  Built for the
 * default tiles only -- fp32 ring tiles 5 and 10 (nstage 1-4), bf16 ring tiles 31 and 30 (nstage
 * 1, 2) -- and not for the kernels that run on rewritten operands in the workspace path;
 * any other plan with this flag is GEMM_ERR_UNSUPPORTED.  Results are unchanged; the
 * extra stores and barrier per slab make it slower. */
#define GEMM_FLAG_POISON_LDS 4

/* What a call would launch (filled by gemm_plan; no GPU needed). */
typedef struct gemm_plan {
    int kernel;        /* gemm_kernel_t actually chosen */
    int nstage;
    int tile;          /* tile id within the family */
    int bm, bn, bk;    /* block tile (C rows, C cols, K-slab depth) */
    int threads;       /* threads per workgroup */
    int lds_bytes;     /* LDS per workgroup */
    int64_t grid;      /* workgroups launched (0 if nothing is launched); for the persistent
                          MFMA ring tiles (19, 28) the number of output tiles, which one
                          workgroup per compute unit walks */
    int packed;        /* gemm_workspace_size only: bit 0 / bit 1 = A / B is first rewritten
                          into the workspace (then the fields above describe the multiply of
                          the rewritten operands, K rounded up to a multiple of 64); else 0 */
} gemm_plan_t;

/* fp32 A, B, C. */
gemm_status_t gemm_f32(gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K,
                       float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                       float beta, float* C, int64_t ldc, hipStream_t stream);

/* bf16 A, B (raw 16-bit words); C is bf16 (c_type = GEMM_BF16) or fp32 (GEMM_F32). */
gemm_status_t gemm_bf16(gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K,
                        float alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
                        float beta, void* C, gemm_dtype_t c_type, int64_t ldc, hipStream_t stream);

/* f16 A, B; C is f16 (c_type = GEMM_F16) or fp32 (GEMM_F32). */
gemm_status_t gemm_f16(gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K,
                       float alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
                       float beta, void* C, gemm_dtype_t c_type, int64_t ldc, hipStream_t stream);

/* Same, with explicit knobs (opts may be NULL = defaults). */
gemm_status_t gemm_f32_ex(gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K,
                          float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                          float beta, float* C, int64_t ldc, hipStream_t stream,
                          const gemm_opts_t* opts);
gemm_status_t gemm_bf16_ex(gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K,
                           float alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
                           float beta, void* C, gemm_dtype_t c_type, int64_t ldc, hipStream_t stream,
                           const gemm_opts_t* opts);
gemm_status_t gemm_f16_ex(gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K,
                          float alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
                          float beta, void* C, gemm_dtype_t c_type, int64_t ldc, hipStream_t stream,
                          const gemm_opts_t* opts);

/* Same as gemm_bf16_ex / gemm_f16_ex, with a caller-owned device workspace that lets the
 * direct-to-LDS ring take operands it cannot read in place.  The ring copies 16-byte
 * chunks of K-contiguous rows straight into LDS, a whole K-slab at a time (the page
 * "Software Pipelining and Double Buffering", section "Multi-stage pipelines"; the
 * staged loads of the other kernels take any layout but pass through registers).  A ring
 * that reads the operands as they are needs no rewrite (row-major A and B: tile 30, which
 * takes B's N-contiguous slabs as they lie and A through registers).  Otherwise, when an
 * operand is N- or M-contiguous (B row-major, A column-major), has a base or pitch
 * off 16 bytes, or K is not a multiple of 64, that operand is first rewritten into the
 * workspace as K-contiguous rows of K' = K rounded up to a multiple of 64 elements, the
 * extra columns zero (they add +0 to every sum), by one bandwidth-bound pass enqueued on
 * `stream` before the multiply; the ring then runs on the rewritten operands.
 * workspace: device memory, 256-byte aligned, not overlapping A, B or C; its contents on
 * entry do not matter and on return are unspecified.  workspace_bytes: its size; the
 * size needed is given by gemm_workspace_size.  With a NULL or too small workspace, or a
 * problem the ring runs as it is or cannot run even rewritten (fp32 input, a problem
 * smaller than the tile, a forced staged kernel), the call is exactly gemm_*_ex.
 * The result equals that of the ring on the unpadded problem: same k order per output.
 * Errors: as gemm_*_ex, plus GEMM_ERR_INVALID_ARG for a workspace not 256-byte aligned.
 * The workspace must stay untouched until the enqueued work has finished. */
gemm_status_t gemm_bf16_ws(gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K,
                           float alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
                           float beta, void* C, gemm_dtype_t c_type, int64_t ldc, hipStream_t stream,
                           const gemm_opts_t* opts, void* workspace, size_t workspace_bytes);
gemm_status_t gemm_f16_ws(gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K,
                          float alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
                          float beta, void* C, gemm_dtype_t c_type, int64_t ldc, hipStream_t stream,
                          const gemm_opts_t* opts, void* workspace, size_t workspace_bytes);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): gemm_bf16_ws (in_type GEMM_BF16) or
 * gemm_f16_ws (GEMM_F16) with the workspace taken from a static device array of the
 * library, GEMM_STATIC_WS_BYTES per GPU (held by each GPU the library runs on until the
 * process ends), instead of a caller buffer.  Allocates nothing: no hipMalloc / hipFree,
 * no allocating library call.  A, B, C, the other arguments, the result and the k order
 * are exactly those of gemm_*_ws given a large enough workspace.
 * Every call on one GPU shares that GPU's array: calls that may overlap on one GPU
 * (different streams, different host threads without ordering) race on it and must be
 * serialised by the caller.  Its contents carry over between calls; a call rewrites every
 * byte it reads, so stale contents never reach a result.
 * Errors: as gemm_*_ws (checks run before anything is enqueued), plus
 *   GEMM_ERR_INVALID_ARG -- in_type not bf16 / f16;
 *   GEMM_ERR_UNSUPPORTED -- the rewritten operands need more than GEMM_STATIC_WS_BYTES
 *       (gemm_workspace_size reports the bytes; use gemm_*_ws with a caller workspace);
 *   GEMM_ERR_HIP -- the array's device address could not be looked up, or a launch failed. */
#define GEMM_STATIC_WS_BYTES 33554432
gemm_status_t gemm_ws_static(gemm_dtype_t in_type, gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N,
                             int64_t K, float alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
                             float beta, void* C, gemm_dtype_t c_type, int64_t ldc, hipStream_t stream,
                             const gemm_opts_t* opts);

/* Workspace bytes a gemm_*_ws call with these arguments needs in order to rewrite its
 * operands (0 when it would not rewrite any), and, if plan is not NULL, what that call
 * launches when given at least that many bytes (gemm_plan_t.packed says which operands
 * are rewritten).  Host only; pointers are inspected for NULL and alignment, never
 * dereferenced.  The size is M*K'*2 (A rewritten) plus N*K'*2 (B rewritten), each
 * rounded up to 256 bytes, K' = K rounded up to a multiple of 64.
 * Errors: as gemm_plan, GEMM_ERR_INVALID_ARG for a NULL bytes. */
gemm_status_t gemm_workspace_size(gemm_dtype_t in_type, gemm_dtype_t c_type, gemm_layout_t la, gemm_layout_t lb,
                                  int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                                  const void* B, int64_t ldb, float beta, const void* C, int64_t ldc,
                                  const gemm_opts_t* opts, size_t* bytes, gemm_plan_t* plan);

/* Validate and choose exactly as the corresponding gemm_*_ex call would, without
 * launching anything (host only; pointers are inspected for NULL and alignment, never
 * dereferenced).  in_type: GEMM_F32 / GEMM_BF16 / GEMM_F16.  Returns the status the
 * call would return before launching; *plan is filled when it returns GEMM_OK. */
gemm_status_t gemm_plan(gemm_dtype_t in_type, gemm_dtype_t c_type, gemm_layout_t la, gemm_layout_t lb,
                        int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                        const void* B, int64_t ldb, float beta, const void* C, int64_t ldc,
                        const gemm_opts_t* opts, gemm_plan_t* plan);

/* Stage / tile tuner: launch every (kernel family, tile, stage count) that gemm_plan
 * accepts for this problem -- one warm-up call and `reps` timed calls each, HIP events on
 * `stream` -- and return the fastest as *best (pass it to gemm_*_ex) with its average
 * time per call in *best_ms.  The stage count is chosen against the measured curve rather
 * than a model (the page "Software Pipelining and Double Buffering", section
 * "Multi-stage pipelines", ties the useful depth to the shared-memory budget; section 7
 * of "CUTLASS-Cute 初步(6)：CUDA GEMM 计算优化、Multi-Stage 与软流水" models it from
 * bandwidth and compute rates).
 * Arguments as gemm_plan plus: C is overwritten by the timed calls (with beta != 0 its
 * contents afterwards are unspecified: the calls accumulate); reps 1..100000.
 * Synchronises `stream`.  Empty problems and quick returns report the default plan with
 * *best_ms = 0.  Different tiles sum in different orders, so results differ in the last
 * bits between choices (each choice is deterministic).
 * Errors: as gemm_plan, GEMM_ERR_INVALID_ARG for NULL best / best_ms or reps out of
 * range, GEMM_ERR_HIP for a failed launch or timing. */
gemm_status_t gemm_tune(gemm_dtype_t in_type, gemm_dtype_t c_type, gemm_layout_t la, gemm_layout_t lb,
                        int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                        const void* B, int64_t ldb, float beta, void* C, int64_t ldc, hipStream_t stream,
                        int reps, gemm_opts_t* best, float* best_ms);

/* gemm_tune for the workspace entry points (16-bit inputs): the candidates are every
 * variant a gemm_bf16_ws / gemm_f16_ws call with this workspace accepts -- ring variants
 * on rewritten operands that fit in `workspace_bytes` included -- each timed as that call
 * (the rewrite counted); pass *best to the same call.  Arguments as gemm_tune plus the
 * workspace (as in gemm_*_ws; its contents afterwards are unspecified).
 * Errors: as gemm_tune, GEMM_ERR_INVALID_ARG for fp32 input or a workspace not 256-byte
 * aligned. */
gemm_status_t gemm_tune_ws(gemm_dtype_t in_type, gemm_dtype_t c_type, gemm_layout_t la, gemm_layout_t lb,
                           int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                           const void* B, int64_t ldb, float beta, void* C, int64_t ldc, hipStream_t stream,
                           void* workspace, size_t workspace_bytes, int reps, gemm_opts_t* best, float* best_ms);

/* The K-loop protocol of a kernel family, as the event list its mainloop executes
 * (host only, for checking the pipeline on the CPU).  nstage: 1..5 for the ring
 * families (the protocol itself; kernels are built up to GEMM_MAX_NSTAGE), 1..2 for the
 * staged ones.  Each event is 4 ints
 * {type, slab, slot, arg}:
 *   1 ISSUE    slab -> slot: asynchronous global->LDS copy of K-slab `slab` into ring
 *              slot `slot` (staged kernels: slot == -1, a global->register load);
 *              arg = part | (parts << 8) when the copy is split into parts
 *   2 WAIT     arg = number of the newest issued slabs that may still be in flight
 *   3 BARRIER  all waves of the workgroup
 *   4 COMPUTE  read ring slot `slot`, holding slab `slab` (arg = k-step within the slab,
 *              or -1 for a whole slab)
 *   5 WRITE    staged kernels: registers of slab `slab` -> ring slot `slot`
 *   6 WAIT_LDS the wave's own LDS reads and writes have completed
 * kernel: GEMM_KERNEL_VALU_RING / MFMA_RING / VALU_STAGED / MFMA_STAGED; ksteps = k-steps
 * per slab (2, 4 or 8), plus 16 * code for a ring kernel that splits the copy of each slab
 * into parts (its ISSUE events carry arg = part | (parts << 8)): code 0 = the whole copy at
 * the slab's first k-step, 1 = one part per k-step, c >= 2 = c - 1 parts (at most one per
 * k-step), the first issued right after the barrier that frees the slot.
 * Returns the number of events (writes at most `capacity` of them), or -1 for bad
 * arguments. */
int gemm_schedule(int kernel, int nstage, int num_k, int ksteps, int* events, int capacity);

/* dst[0, bytes) = src[0, bytes), streamed through an nStage LDS ring by the same K-loop
 * protocol and global->LDS copies as the GEMM kernels (16 KiB slabs, each workgroup a
 * contiguous run of them; each slab is copied into LDS, then written out).  It is the
 * bandwidth-bound control of software pipelining: the page "Software Pipelining and
 * Double Buffering" (section "When it pays") says extra stages change nothing for a
 * kernel that already saturates memory bandwidth.
 * dst, src: device pointers, 16-byte aligned, not overlapping; bytes: a multiple of
 * 16384 (0 = no-op); nstage: 1..4 LDS slots (0 = 2).  Enqueued on `stream`.
 * Errors: GEMM_ERR_INVALID_ARG (size, alignment, NULL, overlap), GEMM_ERR_UNSUPPORTED
 * (nstage), GEMM_ERR_HIP (launch). */
gemm_status_t gemm_pipe_copy(void* dst, const void* src, int64_t bytes, int nstage, hipStream_t stream);

/* The compute-bound control, the counterpart of gemm_pipe_copy: matrix instructions on
 * operands held in registers, with no memory access inside the loop, so that its rate is
 * what the matrix cores sustain at the clock the card settles at for that operand data.
 * Set beside a GEMM kernel on operands of the same distribution, it separates what the
 * kernel's feed and overlap lose from what the card cannot give (the page "CUTLASS-Cute
 * 初步(6)", sections 7 and 7.1: more stages fill the gaps between math phases, up to the
 * math rate and never past it).
 * Each of `grid` workgroups runs GEMM_CEIL_THREADS threads (8 waves, two per SIMD).  Every
 * wave reads the whole fragment set once: fragment f, lane l, element e at
 * frags[(f*64 + l)*8 + e] (GEMM_CEIL_FRAG_ELEMS 16-bit values of type in_type).  Fragment
 * f = r*(WA + WB) + i is the first operand of instruction row i of k-step r (i < WA), and
 * f = r*(WA + WB) + WA + j the second operand of column j; lane l of a fragment holds row
 * l mod MI, k = 8*(l / MI) .. +7, of its MI-row block.  shape 16: v_mfma_f32_16x16x32,
 * R = 4, WA = WB = 4; shape 32: v_mfma_f32_32x32x16, R = 8, WA = WB = 2.  The wave then
 * runs `iters` rounds of: for each k-step r, acc[i][j] += X(r,i) * Y(r,j)^T for all i, j
 * (X, Y the MI x KI blocks of fragments (r,i) and (r,j)) -- 2^20 FLOPs per wave and round,
 * so the call does grid * 8 * iters * 2^20 FLOPs.  Finally lane l of wave w of workgroup g
 * writes sums[(g*8 + w)*64 + l] = the sum, in a fixed order, of the accumulator values it
 * holds (for shape 32, registers 4q+t hold rows 8q + 4*(l/32) + t of column l mod 32 of
 * each accumulator; for shape 16, register t holds row 4*(l/16) + t of column l mod 16).
 * frags: device, 16-byte aligned, read-only; sums: device, grid * 512 floats, 4-byte
 * aligned; grid 1..GEMM_CEIL_MAX_GRID; iters >= 0 (0 writes zeros).  Enqueued on `stream`.
 * Errors: GEMM_ERR_UNSUPPORTED (in_type, shape), GEMM_ERR_INVALID_ARG (grid, iters, NULL,
 * alignment), GEMM_ERR_HIP (launch). */
#define GEMM_CEIL_THREADS 512
#define GEMM_CEIL_FRAG_ELEMS 16384
#define GEMM_CEIL_MAX_GRID 65536
gemm_status_t gemm_mfma_ceiling(int in_type, int shape, const void* frags, float* sums, int64_t grid, int64_t iters,
                                hipStream_t stream);

/* dst[0, bytes) = src[0, bytes) from ordinary (pageable) host memory to the device,
 * staged through a ring of `nstage` page-locked slots of `chunk_bytes` each: the CPU
 * copies chunk c into slot c mod nstage while the DMA engine moves the chunks already
 * staged; a slot is refilled only after the DMA that read it has completed (one event per
 * slot).  It is the host-side form of the same ring the kernels run, the one the page
 * "Asynchronous data movement" (CUDA Handbook ch. 17, the paragraph comparing cp.async
 * with CPU/GPU overlap) recalls for pageable copies: with one slot, filling and draining
 * alternate; with two or more they overlap.
 * dst: device memory; src: host memory, not overlapping the staging ring; staging:
 * page-locked host memory (hipHostMalloc), at least nstage * chunk_bytes bytes; nstage
 * 1..4; chunk_bytes >= 1 (the last chunk may be shorter).  The DMAs are enqueued on
 * `stream`; the call returns when all of them have completed (the staging memory is then
 * free again).  Creates and destroys up to 4 HIP events.
 * Errors: GEMM_ERR_INVALID_ARG (sizes, NULL, overlap), GEMM_ERR_UNSUPPORTED (nstage),
 * GEMM_ERR_HIP (a copy, an event or a wait failed). */
gemm_status_t gemm_h2d_staged(void* dst, const void* src, int64_t bytes, void* staging, int64_t chunk_bytes,
                              int nstage, hipStream_t stream);

/* gemm_h2d_staged without the final wait: returns once every chunk has been copied into
 * the staging ring and its DMA enqueued on `stream`, with up to min(nstage, chunks) DMAs
 * still running.  The CPU's part of the copy and the GPU's work on other streams overlap
 * as before; what the caller gains is the host thread, free as soon as the last chunk is
 * staged (the page's CPU/GPU overlap, with the ring's last slots drained by the stream).
 * Contract: `staging` (and `dst`) must stay untouched until `stream` has passed the copies
 * (hipStreamSynchronize(stream), or an event recorded on `stream` after this call).
 * Arguments and errors as gemm_h2d_staged; after an error the call waits for any DMA it
 * enqueued. */
gemm_status_t gemm_h2d_staged_async(void* dst, const void* src, int64_t bytes, void* staging, int64_t chunk_bytes,
                                    int nstage, hipStream_t stream);

const char* gemm_status_string(gemm_status_t status);

/* Thread-local description of the last non-OK status on this thread ("" if none). */
const char* gemm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBGEMM_H */
