// libgemm.cpp -- the C ABI: argument checks, kernel choice and launch.
//
// Everything here runs on the host.  Arguments are checked before anything is
// enqueued; the kernel family, tile and stage count are chosen from the layouts, the
// alignment of the operands and the problem shape; the kernel is launched on the
// caller's stream without synchronising.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "libgemm.h"
#include "launch.hpp"
#include "schedule.hpp"

namespace {

using gemm::GemmParams;

thread_local char g_err[512] = "";

bool debug_on();

gemm_status_t fail(gemm_status_t s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    if (debug_on()) fprintf(stderr, "libgemm: status %d: %s\n", (int)s, g_err);
    return s;
}

struct Tile {
    int id, bm, bn, bk, threads;
    int stages;       // bit s set: nstage = s is instantiated
    int def_stage;    // default nstage
    int stage_bytes;  // LDS per ring slot
};

constexpr int S1 = 1 << 1, S2 = 1 << 2, S3 = 1 << 3, S4 = 1 << 4;

// Instantiated tiles of each family (must match the launch tables of the kernels).
const Tile kValuRing[] = {
    {1, 128, 64, 16, 128, S1 | S2 | S3 | S4, 2, (128 * 16 + 16 * 64) * 4},  // 8x8 per thread, 2-k steps
    {2, 64, 64, 16, 256, S1 | S2 | S3 | S4, 2, (64 * 16 + 16 * 64) * 4},
    {3, 32, 32, 16, 64, S1 | S2 | S3 | S4, 2, (32 * 16 + 16 * 32) * 4},
    {4, 128, 64, 16, 128, S1 | S2 | S3 | S4, 2, (128 * 16 + 16 * 64) * 4},  // tile 1 with 4-k steps
    {5, 128, 64, 16, 256, S1 | S2 | S3 | S4, 4, (128 * 16 + 16 * 64) * 4},  // 8x4 per thread
    {6, 128, 64, 16, 256, S1 | S2 | S3 | S4, 2, (128 * 16 + 16 * 64) * 4},  // 4x8 per thread
    {7, 32, 32, 32, 64, S1 | S2 | S3 | S4, 2, (32 * 32 + 32 * 32) * 4},     // tile 3, 32-deep slabs
    {8, 128, 64, 32, 256, S1 | S2 | S3 | S4, 2, (128 * 32 + 32 * 64) * 4},  // tile 5, 32-deep slabs
    {9, 16, 16, 32, 64, S1 | S2 | S3 | S4, 4, (16 * 32 + 32 * 16) * 4},     // 1x4 per thread, for grids too small for tile 7
    {10, 128, 128, 32, 256, S1 | S2 | S3 | S4, 2, (128 * 32 + 32 * 128) * 4},  // 8x8 per thread
    {11, 128, 128, 16, 512, S1 | S2 | S3 | S4, 4, (128 * 16 + 16 * 128) * 4},  // 512 threads of 8x4
};
// The fp32 ring tile forced kernels default to, and the reference size for the choice of
// the large tile (valu_large_tile): 256 threads of 8x4, 4-k steps, four slots.
constexpr int kValuRingDefault = 5;
const Tile kValuStaged[] = {
    {1, 128, 64, 16, 128, S1 | S2, 2, (128 * 16 + 16 * 64) * 4},
    {3, 32, 32, 16, 64, S1 | S2, 2, (32 * 16 + 16 * 32) * 4},
};
const Tile kMfmaRing[] = {
    {1, 256, 256, 64, 256, S1 | S2, 2, (256 + 256) * 64 * 2},
    {2, 256, 256, 32, 256, S1 | S2 | S3 | S4, 3, (256 + 256) * 32 * 2},
    {3, 128, 128, 64, 256, S1 | S2 | S3 | S4, 2, (128 + 128) * 64 * 2},
    {18, 256, 128, 64, 384, S1 | S2 | S3, 3, (256 + 128) * 64 * 2},  // 4 consumer + 2 producer waves
    {19, 256, 128, 64, 384, S2 | S3, 3, (256 + 128) * 64 * 2},    // tile 18, persistent
    {23, 256, 256, 64, 512, S1 | S2, 2, (256 + 256) * 64 * 2},    // 8 waves (2x4 of 128x64), copies by one wave per SIMD
    {24, 256, 256, 64, 512, S1 | S2, 2, (256 + 256) * 64 * 2},    // tile 23, copies spread
    {25, 256, 256, 32, 512, S3 | S4, 3, (256 + 256) * 32 * 2},    // tile 23 with BK 32, spread
    {26, 256, 192, 64, 512, S1 | S2, 2, (256 + 192) * 64 * 2},    // tile 23's scheme, 4x2 waves of 64x96
    {28, 256, 256, 64, 512, S2, 2, (256 + 256) * 64 * 2},         // tile 23, persistent
    {29, 192, 256, 64, 512, S1 | S2, 2, (192 + 256) * 64 * 2},    // tile 23's scheme, 2x4 waves of 96x64, copies spread
    {30, 192, 256, 64, 512, S1 | S2, 2, (192 + 256) * 64 * 2},    // tile 29 on row-major A (any pitch) and row-major B
    {31, 256, 256, 64, 512, S1 | S2, 2, (256 + 256) * 64 * 2},    // tile 23, 16x16x32, copies right after the barrier (default)
    {32, 192, 256, 64, 512, S1 | S2, 2, (192 + 256) * 64 * 2},    // tile 31's scheme on 192x256
#ifdef GEMM_ALL_TILES  // variants that lose on every workload measured (built on request)
    {4, 256, 256, 64, 256, S2, 2, (256 + 256) * 64 * 2},          // copies spread over the slab
    {5, 256, 256, 32, 256, S3 | S4, 3, (256 + 256) * 32 * 2},     // copies spread
    {6, 128, 128, 64, 256, S2 | S3, 2, (128 + 128) * 64 * 2},     // copies spread
    {7, 256, 256, 64, 512, S2, 2, (256 + 256) * 64 * 2},          // 8 waves 128x64, spread
    {8, 256, 256, 64, 512, S2, 2, (256 + 256) * 64 * 2},          // 8 waves 64x128
    {9, 256, 256, 32, 512, S3 | S4, 3, (256 + 256) * 32 * 2},     // 8 waves, BK 32, spread
    {10, 256, 256, 64, 256, S2, 2, (256 + 256) * 64 * 2},         // 16x16x32 instructions
    {11, 256, 256, 64, 256, S2, 2, (256 + 256) * 64 * 2},         // 16x16x32, spread
    {12, 128, 128, 64, 256, S2 | S3, 2, (128 + 128) * 64 * 2},    // 16x16x32
    {13, 256, 256, 64, 256, S1 | S2, 2, (256 + 256) * 64 * 2},    // tile 1, pinned issue order
    {14, 256, 256, 64, 256, S2, 2, (256 + 256) * 64 * 2},         // tile 4, pinned
    {15, 256, 256, 32, 256, S3 | S4, 3, (256 + 256) * 32 * 2},    // tile 5, pinned
    {16, 256, 256, 32, 512, S3 | S4, 3, (256 + 256) * 32 * 2},    // tile 9, pinned
    {17, 256, 128, 64, 512, S1 | S2 | S3, 3, (256 + 128) * 64 * 2},  // 4 consumer + 4 producer waves
    {20, 256, 128, 64, 512, S3, 3, (256 + 128) * 64 * 2},         // tile 17, persistent
    {22, 256, 128, 64, 320, S3, 3, (256 + 128) * 64 * 2},         // 4 consumer + 1 producer wave
    {21, 256, 256, 64, 512, S1 | S2, 2, (256 + 256) * 64 * 2},    // 8 waves, copies by 4 of them
    {27, 192, 256, 64, 512, S1 | S2, 2, (192 + 256) * 64 * 2},    // tile 23's scheme, 2x4 waves of 96x64
#endif
};
// The MFMA ring tile used when none is named for a problem of >= 128 256x256 tiles (and
// the cost model below keeps 256x256): 256x256x64, two slots, eight waves (2x4 of
// 128x64, two per SIMD) of which one per SIMD issues the copies, 16x16x32 instructions,
// and each slab's copies issued together in the k-step right after the barrier that frees
// its slot (the fastest measured on 8192^3 bf16: 3% ahead of splitting them over the two
// k-steps, 8% ahead of issuing them in the slab's first k-step; on the f16 MLP shape
// within 1% of the split; the 32x32x16 form of the tile, 24, is 2-7% behind).
constexpr int kMfmaRingDefault = 31;

const Tile kMfmaStaged[] = {
    {1, 128, 128, 32, 256, S1 | S2, 2, (128 + 128) * 32 * 2},
    {2, 128, 128, 64, 256, S1 | S2, 2, (128 + 128) * 64 * 2},
};

constexpr int kLdsLimit = 163840;  // bytes of LDS one workgroup may allocate on gfx950
static_assert(gemm::kStaticWsBytes == GEMM_STATIC_WS_BYTES, "static workspace size as the header states");

template <size_t N>
const Tile* find_tile(const Tile (&t)[N], int id) {
    for (size_t i = 0; i < N; ++i)
        if (t[i].id == id) return &t[i];
    return nullptr;
}

struct Problem {
    int in_type, c_type;
    int la, lb;
    int64_t M, N, K;
    float alpha, beta;
    const void* A;
    const void* B;
    const void* C;
    int64_t lda, ldb, ldc;
};

int elem_size(int dt) { return dt == gemm::DT_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

gemm_status_t validate(const Problem& q) {
    if (q.la != GEMM_ROW_MAJOR && q.la != GEMM_COL_MAJOR) return fail(GEMM_ERR_INVALID_ARG, "la: bad layout %d", q.la);
    if (q.lb != GEMM_ROW_MAJOR && q.lb != GEMM_COL_MAJOR) return fail(GEMM_ERR_INVALID_ARG, "lb: bad layout %d", q.lb);
    if (q.M < 0 || q.N < 0 || q.K < 0)
        return fail(GEMM_ERR_INVALID_ARG, "negative size (M=%lld N=%lld K=%lld)", (long long)q.M, (long long)q.N,
                    (long long)q.K);
    if (q.M > INT32_MAX || q.N > INT32_MAX || q.K > INT32_MAX)
        return fail(GEMM_ERR_INVALID_ARG, "sizes must be below 2^31");
    const int64_t min_lda = q.la == GEMM_ROW_MAJOR ? q.K : q.M;
    const int64_t min_ldb = q.lb == GEMM_ROW_MAJOR ? q.N : q.K;
    if (q.lda < 1 || q.lda < min_lda) return fail(GEMM_ERR_INVALID_ARG, "lda=%lld < %lld", (long long)q.lda, (long long)min_lda);
    if (q.ldb < 1 || q.ldb < min_ldb) return fail(GEMM_ERR_INVALID_ARG, "ldb=%lld < %lld", (long long)q.ldb, (long long)min_ldb);
    if (q.ldc < 1 || q.ldc < q.N) return fail(GEMM_ERR_INVALID_ARG, "ldc=%lld < N=%lld", (long long)q.ldc, (long long)q.N);
    if (q.M > 0 && q.N > 0) {
        if (!q.C) return fail(GEMM_ERR_INVALID_ARG, "C is NULL");
        if (q.alpha != 0.0f && q.K > 0) {
            if (!q.A) return fail(GEMM_ERR_INVALID_ARG, "A is NULL");
            if (!q.B) return fail(GEMM_ERR_INVALID_ARG, "B is NULL");
        }
    }
    return GEMM_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// GEMM_DEBUG=1 in the environment: every kernel choice is described on stderr (read once;
// the static's initialisation is thread-safe and it never changes afterwards).
bool debug_on() {
    static const bool on = [] {
        const char* e = getenv("GEMM_DEBUG");
        return e != nullptr && e[0] != 0 && !(e[0] == '0' && e[1] == 0);
    }();
    return on;
}

const char* kernel_name(int k) {
    switch (k) {
        case GEMM_KERNEL_VALU_RING: return "valu_ring";
        case GEMM_KERNEL_VALU_STAGED: return "valu_staged";
        case GEMM_KERNEL_MFMA_RING: return "mfma_ring";
        case GEMM_KERNEL_MFMA_STAGED: return "mfma_staged";
        case GEMM_KERNEL_SCALE: return "scale";
        default: return "none";
    }
}

const char* type_name(int t) { return t == gemm::DT_F32 ? "f32" : t == gemm::DT_BF16 ? "bf16" : "f16"; }

// One line per decision: the problem, what was picked and, when the direct ring was
// passed over, why.
void debug_plan(const Problem& q, const gemm_opts_t& o, const gemm_plan_t& pl, const char* why) {
    if (!debug_on()) return;
    char note[160] = "";
    if (why && why[0]) snprintf(note, sizeof(note), " (direct ring passed over: %s)", why);
    fprintf(stderr,
            "libgemm: %s->%s M=%lld N=%lld K=%lld A=%s B=%s lda=%lld ldb=%lld alpha=%g beta=%g "
            "opts(kernel=%d tile=%d nstage=%d flags=0x%x) -> %s tile %d %dx%dx%d nstage %d grid %lld lds %d%s\n",
            type_name(q.in_type), type_name(q.c_type), (long long)q.M, (long long)q.N, (long long)q.K,
            q.la == GEMM_ROW_MAJOR ? "row" : "col", q.lb == GEMM_ROW_MAJOR ? "row" : "col", (long long)q.lda,
            (long long)q.ldb, q.alpha, q.beta, o.kernel, o.tile, o.nstage, o.flags, kernel_name(pl.kernel), pl.tile,
            pl.bm, pl.bn, pl.bk, pl.nstage, (long long)pl.grid, pl.lds_bytes, note);
}

// LDS a kernel of this tile allocates statically: the ring, or for the split-copy tiles
// with 256 columns and a 16-bit C, at least the C tile (bm x 256 x 2 bytes), which their
// epilogue stages through LDS after the K loop whatever the stage count.
int static_lds(const Tile& t, int S, int kernel, int c_type) {
    int lds = S * t.stage_bytes;
    const bool split = t.id == 21 || t.id == 23 || t.id == 24 || t.id == 25 || t.id == 27 || t.id == 29 || t.id == 30 ||
                       t.id == 31 || t.id == 32;
    if (kernel == GEMM_KERNEL_MFMA_RING && split && c_type != gemm::DT_F32 && t.bn == 256 && lds < t.bm * t.bn * 2)
        lds = t.bm * t.bn * 2;
    return lds;
}

// Tiles of the matrix-core ring that read a row-major A and a row-major (N-contiguous) B
// as they are: A through registers (any pitch or alignment, K tail zero-filled), B's
// K-slabs copied straight into LDS as [k][n] rows and read back with transposing loads.
bool kn_tile(int id) { return id == 30; }

bool kn_ok(const Problem& q, const Tile& t, const char** why) {
    if (q.in_type == gemm::DT_F32) { *why = "16-bit inputs only"; return false; }
    if (!(q.la == GEMM_ROW_MAJOR && q.lb == GEMM_ROW_MAJOR)) { *why = "needs A and B row-major"; return false; }
    if (!aligned16(q.B) || (q.ldb * 2) % 16) { *why = "B rows not 16-byte aligned"; return false; }
    // the last column tile starts at N - bn, where B's 16-byte chunks must begin
    if (q.N % 8) { *why = "N not a multiple of 8"; return false; }
    if (q.K == 0) { *why = "K == 0"; return false; }
    if (q.M < t.bm || q.N < t.bn) { *why = "problem smaller than the tile"; return false; }
    // per-lane 32-bit offsets: a slab of B spans bk rows, a tile of A bm rows
    if ((q.ldb * 2) * (t.bk + 1) >= (int64_t(1) << 31) || (q.lda * 2) * (t.bm + 1) >= (int64_t(1) << 31)) {
        *why = "leading dimension too large"; return false;
    }
    return true;
}

// Can the direct global->LDS ring run this problem with this tile?
bool ring_ok(const Problem& q, const Tile& t, bool mfma, const char** why) {
    if (mfma && kn_tile(t.id)) return kn_ok(q, t, why);
    const int es = elem_size(q.in_type);
    const int vec = 16 / es;
    if (mfma) {
        if (!(q.la == GEMM_ROW_MAJOR && q.lb == GEMM_COL_MAJOR)) { *why = "needs A row-major and B column-major (K-contiguous)"; return false; }
    } else {
        if (!(q.la == GEMM_ROW_MAJOR && q.lb == GEMM_ROW_MAJOR)) { *why = "needs A and B row-major"; return false; }
    }
    if (!aligned16(q.A) || !aligned16(q.B)) { *why = "A/B not 16-byte aligned"; return false; }
    if (q.lda % vec || q.ldb % vec) { *why = "leading dimensions not a multiple of 16 bytes"; return false; }
    if (q.K == 0 || q.K % t.bk) { *why = "K not a multiple of the slab depth"; return false; }
    if (q.M < t.bm || q.N < t.bn) { *why = "problem smaller than the tile"; return false; }
    // The last column tile is shifted inward to start at N - bn; with row-major B (the fp32
    // ring) that column is the start of each copied 16-byte chunk, so it must be a
    // multiple of the vector width.  (The MFMA ring shifts only along K-contiguous rows,
    // whose starts the leading-dimension rule already aligns.)
    if (!mfma && q.N % t.bn && (q.N - t.bn) % vec) {
        *why = "last column tile would start off a 16-byte boundary (N not a multiple of 4)"; return false;
    }
    // per-lane 32-bit offsets span up to one tile of rows (<= 256) of the operand
    if ((q.lda * es) * 256 >= (int64_t(1) << 31) || (q.ldb * es) * 256 >= (int64_t(1) << 31)) {
        *why = "leading dimension too large"; return false;
    }
    return true;
}

// The fp32 ring tile for problems of at least 512 128x64 tiles.  A grid runs in rounds of
// as many workgroups as are resident at once, so each candidate costs
//   ceil(tiles / resident) rounds x resident x tile area / its full-occupancy rate,
// with the residency and rate measured on fp32 squares of 4096-8192 (NN, S at the tile's
// default): tile 5 (128x64, 256 threads of 8x4, 3 per CU) 97.5 TFLOP/s, tile 10 (128x128,
// 256 threads of 8x8, 2 per CU) 100.8.  Against both forced on 16 shapes from 2048^3 to
// 8192^2x4096 (bench.py --fp32-tiles) the model picks the faster on 14 and loses 2-7% on
// 6144^2x2048 and 1536x4096x4096, whose part-filled last round of 128x128 tiles costs less
// than a full one.  (Tile 11, 128x128 with 512 threads of 8x4, one per CU, is never the
// fastest there and stays a forced / tuner choice.)  Only tiles the direct ring accepts for
// this problem compete (tile 10's 32-deep slabs need K % 32 == 0); tile 5 when none does.
const Tile* valu_large_tile(const Problem& q) {
    const int64_t cus = gemm::num_compute_units();
    struct Cand { int id, per_cu; double rate; };
    const Cand cand[] = {{5, 3, 97.5}, {10, 2, 100.8}};
    const Tile* best = nullptr;
    double best_cost = 0.0;
    for (const Cand& c : cand) {
        const Tile* t = find_tile(kValuRing, c.id);
        const char* why = "";
        if (!ring_ok(q, *t, false, &why)) continue;
        const int64_t tiles = cdiv(q.M, t->bm) * cdiv(q.N, t->bn);
        const int64_t resident = c.per_cu * cus;
        const double cost = double(cdiv(tiles, resident)) * double(resident) * double(t->bm * t->bn) / c.rate;
        if (!best || cost < best_cost) { best = t; best_cost = cost; }
    }
    return best ? best : find_tile(kValuRing, kValuRingDefault);
}

gemm_status_t choose(const Problem& q, const gemm_opts_t* o, gemm_plan_t* plan, GemmParams* gp) {
    gemm_opts_t opts = {0, 0, 0, 0};
    if (o) opts = *o;
    if (opts.flags & ~(GEMM_FLAG_NO_XCD_REMAP | GEMM_FLAG_EQUAL_LDS | GEMM_FLAG_POISON_LDS))
        return fail(GEMM_ERR_INVALID_ARG, "unknown flags 0x%x", opts.flags);
    if (opts.nstage < 0 || opts.nstage > GEMM_MAX_NSTAGE) return fail(GEMM_ERR_UNSUPPORTED, "nstage %d out of range", opts.nstage);
    if (opts.kernel < 0 || opts.kernel > GEMM_KERNEL_SCALE) return fail(GEMM_ERR_INVALID_ARG, "kernel %d unknown", opts.kernel);
    if (opts.tile < 0) return fail(GEMM_ERR_INVALID_ARG, "tile %d", opts.tile);
    const bool mfma = q.in_type != gemm::DT_F32;
    if (opts.kernel != 0) {
        const bool k_mfma = opts.kernel == GEMM_KERNEL_MFMA_RING || opts.kernel == GEMM_KERNEL_MFMA_STAGED;
        const bool k_valu = opts.kernel == GEMM_KERNEL_VALU_RING || opts.kernel == GEMM_KERNEL_VALU_STAGED;
        if ((mfma && k_valu) || (!mfma && k_mfma))
            return fail(GEMM_ERR_UNSUPPORTED, "kernel %d does not take this input type", opts.kernel);
    }

    memset(plan, 0, sizeof(*plan));
    memset(gp, 0, sizeof(*gp));
    gp->A = static_cast<const char*>(q.A);
    gp->B = static_cast<const char*>(q.B);
    gp->C = static_cast<char*>(const_cast<void*>(q.C));
    gp->lda = q.lda; gp->ldb = q.ldb; gp->ldc = q.ldc;
    gp->M = (int)q.M; gp->N = (int)q.N; gp->K = (int)q.K;
    gp->alpha = q.alpha; gp->beta = q.beta;
    gp->a_col = q.la == GEMM_COL_MAJOR;
    gp->b_col = q.lb == GEMM_COL_MAJOR;
    gp->out_type = q.c_type;
    gp->xcd_remap = (opts.flags & GEMM_FLAG_NO_XCD_REMAP) ? 0 : 1;
    gp->group_m = 8;
    const int es = elem_size(q.in_type);
    gp->a_vec = aligned16(q.A) && (q.lda * es) % 16 == 0;
    gp->b_vec = aligned16(q.B) && (q.ldb * es) % 16 == 0;

    if (q.M == 0 || q.N == 0) {
        plan->kernel = GEMM_KERNEL_AUTO;
        debug_plan(q, opts, *plan, "");
        return GEMM_OK;  // nothing to do, nothing launched
    }
    if (q.K == 0 || q.alpha == 0.0f || opts.kernel == GEMM_KERNEL_SCALE) {
        if (opts.kernel != 0 && opts.kernel != GEMM_KERNEL_SCALE)
            return fail(GEMM_ERR_UNSUPPORTED, "K == 0 or alpha == 0 only scales C");
        if (opts.kernel == GEMM_KERNEL_SCALE && !(q.K == 0 || q.alpha == 0.0f))
            return fail(GEMM_ERR_UNSUPPORTED, "the scale kernel only runs when K == 0 or alpha == 0");
        plan->kernel = GEMM_KERNEL_SCALE;
        plan->threads = 256;
        int64_t blocks = cdiv(q.M * q.N, 256);
        plan->grid = blocks > 65536 ? 65536 : blocks;
        debug_plan(q, opts, *plan, "");
        return GEMM_OK;
    }

    int kernel = opts.kernel;
    const Tile* t = nullptr;
    const char* why = "";
    if (kernel == 0) {
        // Automatic: the direct ring when the operands allow it, else the staged loader.
        if (!mfma) {
            // small problems: 32x32 tiles with 32-deep slabs (half the barriers of the
            // 16-deep tile 3; fp32 256^3 11.9 vs 12.3 us); while those would be fewer than
            // three per compute unit, 16x16 tiles, each thread one row of four columns, so
            // that every compute unit holds work (one wave per workgroup; fp32 NN 256^3
            // 5.5 vs 11.8 us, 512^3 9.9 vs 21.4, 768^3 23 vs 32; at 1024^3, four 32x32
            // tiles per unit, 45 vs 41)
            const Tile* big = find_tile(kValuRing, kValuRingDefault);
            const bool tiny = cdiv(q.M, 32) * cdiv(q.N, 32) < 3 * int64_t(gemm::num_compute_units());
            const Tile* small = find_tile(kValuRing, tiny ? 9 : 7);
            const bool many = cdiv(q.M, big->bm) * cdiv(q.N, big->bn) >= 512;
            if (many) big = valu_large_tile(q);
            const Tile* pick = (opts.tile ? find_tile(kValuRing, opts.tile) : (many ? big : small));
            if (pick && ring_ok(q, *pick, false, &why)) { kernel = GEMM_KERNEL_VALU_RING; t = pick; }
            else {
                kernel = GEMM_KERNEL_VALU_STAGED;
                t = find_tile(kValuStaged, many ? 1 : 3);
            }
        } else {
            // The 256x256 tile wins as soon as its tiles cover about half the compute
            // units (measured on bf16 NT squares: 3072^3, 144 tiles, 908 vs 758 TFLOP/s
            // for the best smaller tile; 2048^3, 64 tiles, 402 vs 648).
            const Tile* big = find_tile(kMfmaRing, kMfmaRingDefault);
            const Tile* mid = find_tile(kMfmaRing, 3);
            const bool many = cdiv(q.M, big->bm) * cdiv(q.N, big->bn) >= 128;
            if (many) {
                // One workgroup of these tiles is resident per compute unit, so the grid
                // runs in ceil(tiles / CUs) rounds of one tile each: take the shape with
                // the least work per CU, ceil(tiles / CUs) * bm * bn, on the compute units
                // of the current device (the same count the persistent launchers use).
                // Ties keep the earlier shape (256x256 first; 192x256 measured faster
                // than 256x192).
                const int64_t cus = gemm::num_compute_units();
                int64_t best = -1;
                for (int id : {kMfmaRingDefault, 32, 26}) {
                    const Tile* c = find_tile(kMfmaRing, id);
                    const int64_t cost = cdiv(cdiv(q.M, c->bm) * cdiv(q.N, c->bn), cus) * c->bm * c->bn;
                    if (best < 0 || cost < best) { best = cost; big = c; }
                }
            }
            const Tile* pick = opts.tile ? find_tile(kMfmaRing, opts.tile) : (many ? big : mid);
            // row-major A and B: the ring that reads them in place, once its 192x256 tiles
            // give at least a quarter of the compute units work (else the staged kernel)
            const Tile* kn = find_tile(kMfmaRing, 30);
            if (!opts.tile && q.la == GEMM_ROW_MAJOR && q.lb == GEMM_ROW_MAJOR &&
                cdiv(q.M, kn->bm) * cdiv(q.N, kn->bn) >= 64 && kn_ok(q, *kn, &why))
                pick = kn;
            if (pick && ring_ok(q, *pick, true, &why)) { kernel = GEMM_KERNEL_MFMA_RING; t = pick; }
            else {
                kernel = GEMM_KERNEL_MFMA_STAGED;
                t = find_tile(kMfmaStaged, 1);
            }
        }
    } else {
        int id = opts.tile;
        switch (kernel) {
            case GEMM_KERNEL_VALU_RING: t = find_tile(kValuRing, id ? id : kValuRingDefault); break;
            case GEMM_KERNEL_VALU_STAGED: t = find_tile(kValuStaged, id ? id : 1); break;
            case GEMM_KERNEL_MFMA_RING: t = find_tile(kMfmaRing, id ? id : kMfmaRingDefault); break;
            case GEMM_KERNEL_MFMA_STAGED: t = find_tile(kMfmaStaged, id ? id : 1); break;
        }
        if (!t) return fail(GEMM_ERR_UNSUPPORTED, "tile %d not available for kernel %d", opts.tile, kernel);
        if ((kernel == GEMM_KERNEL_VALU_RING || kernel == GEMM_KERNEL_MFMA_RING) &&
            !ring_ok(q, *t, kernel == GEMM_KERNEL_MFMA_RING, &why))
            return fail(GEMM_ERR_UNSUPPORTED, "direct-to-LDS ring cannot run this problem: %s", why);
    }
    if (!t) return fail(GEMM_ERR_UNSUPPORTED, "no tile");

    int S = opts.nstage ? opts.nstage : t->def_stage;
    if (!(t->stages & (1 << S)))
        return fail(GEMM_ERR_UNSUPPORTED, "nstage %d not built for tile %d of kernel %d", S, t->id, kernel);
    const int lds = static_lds(*t, S, kernel, q.c_type);
    if (lds > kLdsLimit)
        return fail(GEMM_ERR_UNSUPPORTED, "ring of %d x %d bytes exceeds the %d bytes of LDS", S, t->stage_bytes, kLdsLimit);

    plan->kernel = kernel;
    plan->nstage = S;
    plan->tile = t->id;
    plan->bm = t->bm; plan->bn = t->bn; plan->bk = t->bk;
    plan->threads = t->threads;
    plan->lds_bytes = lds;
    if (opts.flags & GEMM_FLAG_EQUAL_LDS) {
        int deepest = S;
        for (int d = GEMM_MAX_NSTAGE; d > S; --d)
            if ((t->stages & (1 << d)) && static_lds(*t, d, kernel, q.c_type) <= kLdsLimit) { deepest = d; break; }
        gp->lds_pad = static_lds(*t, deepest, kernel, q.c_type) - lds;
        plan->lds_bytes += gp->lds_pad;
    }
    if (opts.flags & GEMM_FLAG_POISON_LDS) {
        // the debugging variant exists for the default tiles only (the launch tables)
        const bool built = (kernel == GEMM_KERNEL_VALU_RING && (t->id == 5 || t->id == 10)) ||
                           (kernel == GEMM_KERNEL_MFMA_RING && q.in_type == gemm::DT_BF16 && (t->id == 31 || t->id == 30));
        if (!built)
            return fail(GEMM_ERR_UNSUPPORTED, "no LDS-poisoning build of kernel %d tile %d for this input type", kernel,
                        t->id);
        gp->poison = 1;
    }
    gp->tiles_m = (int)cdiv(q.M, t->bm);
    gp->tiles_n = (int)cdiv(q.N, t->bn);
    plan->grid = (int64_t)gp->tiles_m * gp->tiles_n;
    if (plan->grid > INT32_MAX) return fail(GEMM_ERR_UNSUPPORTED, "too many tiles");
    const bool passed_over = opts.kernel == 0 && (kernel == GEMM_KERNEL_VALU_STAGED || kernel == GEMM_KERNEL_MFMA_STAGED);
    debug_plan(q, opts, *plan, passed_over ? why : "");
    return GEMM_OK;
}

gemm_status_t launch(int in_type, const gemm_plan_t& plan, const GemmParams& gp, hipStream_t stream) {
    if (plan.grid == 0) return GEMM_OK;
    hipError_t e = hipSuccess;
    switch (plan.kernel) {
        case GEMM_KERNEL_SCALE: e = gemm::launch_scale(gp, stream); break;
        case GEMM_KERNEL_VALU_RING: e = gemm::launch_valu_ring(plan.tile, plan.nstage, gp, stream); break;
        case GEMM_KERNEL_VALU_STAGED: e = gemm::launch_valu_staged(plan.tile, plan.nstage, gp, stream); break;
        case GEMM_KERNEL_MFMA_RING: e = gemm::launch_mfma_ring(in_type, plan.tile, plan.nstage, gp, stream); break;
        case GEMM_KERNEL_MFMA_STAGED: e = gemm::launch_mfma_staged(in_type, plan.tile, plan.nstage, gp, stream); break;
        default: return fail(GEMM_ERR_UNSUPPORTED, "internal: kernel %d", plan.kernel);
    }
    if (e != hipSuccess) return fail(GEMM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return GEMM_OK;
}

gemm_status_t run(const Problem& q, const gemm_opts_t* opts, hipStream_t stream) {
    g_err[0] = 0;
    gemm_status_t s = validate(q);
    if (s != GEMM_OK) return s;
    gemm_plan_t plan;
    GemmParams gp;
    s = choose(q, opts, &plan, &gp);
    if (s != GEMM_OK) return s;
    return launch(q.in_type, plan, gp, stream);
}

// ------------------------------------------------------------------ repacking path
// A 16-bit problem whose operands the direct ring cannot read as they are (B
// N-contiguous, a row pitch off 16 bytes, a K tail) is run by first rewriting the
// offending operands into a caller-supplied workspace: K-contiguous rows of kp elements,
// kp = K rounded up to kPackK with zeros, which every ring tile divides.
constexpr int64_t kPackK = 64;
constexpr int64_t kWsAlign = 256;

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct PackPlan {
    bool a = false, b = false;  // operand rewritten into the workspace
    int64_t kp = 0;             // K of the problem the ring runs
    int64_t a_bytes = 0, b_bytes = 0;  // workspace bytes per operand (multiples of kWsAlign)
};

// The ring reads this operand in place: K-contiguous (`want` layout), 16-byte aligned
// base and pitch, and a pitch small enough for its 32-bit per-lane offsets.
bool operand_direct(const void* p, int layout, int want, int64_t ld) {
    return layout == want && aligned16(p) && (ld * 2) % 16 == 0 && (ld * 2) * 256 < (int64_t(1) << 31);
}

// What gemm_*_ws runs: fills *pp (packing, if any) and *plan / *gp for the kernel that
// multiplies.  ws: the workspace base, or NULL when only planning (then aligned stand-in
// addresses take the packed operands' place).  Packs only when the operands as given
// cannot take the ring and the packed problem can; otherwise plans as gemm_*_ex.
gemm_status_t plan_ws(const Problem& q, const gemm_opts_t* o, void* ws, PackPlan* pp, gemm_plan_t* plan,
                      GemmParams* gp) {
    *pp = PackPlan();
    // a ring that reads the operands as they are (row-major A and B included) needs no
    // rewrite
    if (choose(q, o, plan, gp) == GEMM_OK && plan->kernel == GEMM_KERNEL_MFMA_RING) return GEMM_OK;
    g_err[0] = 0;
    const int kernel = o ? o->kernel : 0;
    const int64_t kp = round_up(q.K, kPackK);
    const bool candidate = q.in_type != gemm::DT_F32 && q.M > 0 && q.N > 0 && q.K > 0 && q.alpha != 0.0f &&
                           kp <= INT32_MAX && (kernel == 0 || kernel == GEMM_KERNEL_MFMA_RING);
    if (candidate) {
        const bool need_a = kp != q.K || !operand_direct(q.A, q.la, GEMM_ROW_MAJOR, q.lda);
        const bool need_b = kp != q.K || !operand_direct(q.B, q.lb, GEMM_COL_MAJOR, q.ldb);
        if (need_a || need_b) {
            Problem r = q;
            r.K = kp;
            char* base = static_cast<char*>(ws);
            const int64_t a_bytes = need_a ? round_up(q.M * kp * 2, kWsAlign) : 0;
            const int64_t b_bytes = need_b ? round_up(q.N * kp * 2, kWsAlign) : 0;
            const void* stand_in = reinterpret_cast<const void*>(kWsAlign);
            if (need_a) { r.A = base ? base : stand_in; r.la = GEMM_ROW_MAJOR; r.lda = kp; }
            if (need_b) { r.B = base ? base + a_bytes : stand_in; r.lb = GEMM_COL_MAJOR; r.ldb = kp; }
            if (choose(r, o, plan, gp) == GEMM_OK && plan->kernel == GEMM_KERNEL_MFMA_RING) {
                pp->a = need_a; pp->b = need_b; pp->kp = kp;
                pp->a_bytes = a_bytes; pp->b_bytes = b_bytes;
                plan->packed = (need_a ? 1 : 0) | (need_b ? 2 : 0);
                return GEMM_OK;
            }
            g_err[0] = 0;
        }
    }
    return choose(q, o, plan, gp);
}

gemm_status_t run_ws(const Problem& q, const gemm_opts_t* opts, void* ws, size_t ws_bytes, hipStream_t stream) {
    g_err[0] = 0;
    gemm_status_t s = validate(q);
    if (s != GEMM_OK) return s;
    if (ws && (reinterpret_cast<uintptr_t>(ws) % kWsAlign))
        return fail(GEMM_ERR_INVALID_ARG, "workspace must be %lld-byte aligned", (long long)kWsAlign);
    PackPlan pp;
    gemm_plan_t plan;
    GemmParams gp;
    s = plan_ws(q, opts, ws, &pp, &plan, &gp);
    if (s != GEMM_OK) return s;
    if (!(pp.a || pp.b)) return launch(q.in_type, plan, gp, stream);
    if (!ws || (int64_t)ws_bytes < pp.a_bytes + pp.b_bytes) {
        if (debug_on())
            fprintf(stderr, "libgemm: workspace of %zu bytes < the %lld the rewrite needs: the plain call\n", ws_bytes,
                    (long long)(pp.a_bytes + pp.b_bytes));
        return run(q, opts, stream);  // too small: as gemm_*_ex
    }
    if (debug_on())
        fprintf(stderr, "libgemm: workspace path rewrites%s%s K-contiguous, K' = %lld, then the ring above\n",
                pp.a ? " A" : "", pp.b ? " B" : "", (long long)pp.kp);
    gemm::PackParams pk;
    memset(&pk, 0, sizeof(pk));
    char* base = static_cast<char*>(ws);
    if (pp.a) {  // output row m, column k: A[m*lda + k] (row-major) or A[k*lda + m]
        pk.job[0] = {static_cast<const uint16_t*>(q.A), reinterpret_cast<uint16_t*>(base), q.lda, (int)q.M, (int)q.K,
                     (int)pp.kp, q.la == GEMM_COL_MAJOR ? 1 : 0, 0, 0, 0};
    }
    if (pp.b) {  // output row n, column k: B[n*ldb + k] (column-major) or B[k*ldb + n]
        pk.job[1] = {static_cast<const uint16_t*>(q.B), reinterpret_cast<uint16_t*>(base + pp.a_bytes), q.ldb,
                     (int)q.N, (int)q.K, (int)pp.kp, q.lb == GEMM_ROW_MAJOR ? 1 : 0, 0, 0, 0};
    }
    hipError_t e = gemm::launch_pack(pk, stream);
    if (e != hipSuccess) return fail(GEMM_ERR_HIP, "pack launch failed: %s", hipGetErrorString(e));
    return launch(q.in_type, plan, gp, stream);
}

// ------------------------------------------------------------------ schedule recorder
struct Recorder {
    std::vector<int> ev;
    void push(int t, int slab, int slot, int arg) { ev.insert(ev.end(), {t, slab, slot, arg}); }
    template <int N> void wait_slabs() { push(2, -1, -1, N); }
    void barrier() { push(3, -1, -1, 0); }
    template <int BUF> void frag(int slab, int slot, int ks) { push(4, slab, slot, ks); }
    template <int BUF, int HAS, int PARTS> void math(int) {}
    void wait_lds() { push(6, -1, -1, 0); }
    void issue(int slab, int slot, int part, int parts) { push(1, slab, slot, part | (parts << 8)); }
    void load(int slab) { push(1, slab, -1, 0); }
    void write(int slab, int slot) { push(5, slab, slot, 0); }
};

// parts: the PARTS of the ring template (0 = whole slab at the first k-step, 1..KS parts)
template <int S, int KS, int P = 0>
bool rec_ring(Recorder& r, int numK, int parts) {
    if constexpr (P > KS) {
        return false;
    } else {
        if (parts == P) { gemm_sched::ring_mainloop<S, KS, P>(r, numK); return true; }
        return rec_ring<S, KS, P + 1>(r, numK, parts);
    }
}
template <int S, int KS>
void rec_staged(Recorder& r, int numK) { gemm_sched::staged_mainloop<S, KS>(r, numK); }

template <int S>
bool rec_ring_ks(Recorder& r, int ks, int numK, int parts) {
    switch (ks) {
        case 2: return rec_ring<S, 2>(r, numK, parts);
        case 4: return rec_ring<S, 4>(r, numK, parts);
        case 8: return rec_ring<S, 8>(r, numK, parts);
    }
    return false;
}

template <int S>
bool rec_staged_ks(Recorder& r, int ks, int numK) {
    switch (ks) {
        case 2: rec_staged<S, 2>(r, numK); return true;
        case 4: rec_staged<S, 4>(r, numK); return true;
        case 8: rec_staged<S, 8>(r, numK); return true;
    }
    return false;
}

}  // namespace

extern "C" {

gemm_status_t gemm_f32_ex(gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K, float alpha,
                          const float* A, int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                          int64_t ldc, hipStream_t stream, const gemm_opts_t* opts) {
    Problem q{gemm::DT_F32, gemm::DT_F32, (int)la, (int)lb, M, N, K, alpha, beta, A, B, C, lda, ldb, ldc};
    return run(q, opts, stream);
}

static gemm_status_t half_entry(int in_type, gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K,
                                float alpha, const void* A, int64_t lda, const void* B, int64_t ldb, float beta,
                                void* C, gemm_dtype_t c_type, int64_t ldc, hipStream_t stream,
                                const gemm_opts_t* opts) {
    g_err[0] = 0;
    if (c_type != GEMM_F32 && (int)c_type != in_type)
        return fail(GEMM_ERR_INVALID_ARG, "c_type %d not offered by this entry point", (int)c_type);
    Problem q{in_type, (int)c_type, (int)la, (int)lb, M, N, K, alpha, beta, A, B, C, lda, ldb, ldc};
    return run(q, opts, stream);
}

gemm_status_t gemm_bf16_ex(gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K, float alpha,
                           const void* A, int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                           gemm_dtype_t c_type, int64_t ldc, hipStream_t stream, const gemm_opts_t* opts) {
    return half_entry(gemm::DT_BF16, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream, opts);
}

gemm_status_t gemm_f16_ex(gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K, float alpha,
                          const void* A, int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                          gemm_dtype_t c_type, int64_t ldc, hipStream_t stream, const gemm_opts_t* opts) {
    return half_entry(gemm::DT_F16, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream, opts);
}

static gemm_status_t half_entry_ws(int in_type, gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K,
                                   float alpha, const void* A, int64_t lda, const void* B, int64_t ldb, float beta,
                                   void* C, gemm_dtype_t c_type, int64_t ldc, hipStream_t stream,
                                   const gemm_opts_t* opts, void* workspace, size_t workspace_bytes) {
    g_err[0] = 0;
    if (c_type != GEMM_F32 && (int)c_type != in_type)
        return fail(GEMM_ERR_INVALID_ARG, "c_type %d not offered by this entry point", (int)c_type);
    Problem q{in_type, (int)c_type, (int)la, (int)lb, M, N, K, alpha, beta, A, B, C, lda, ldb, ldc};
    return run_ws(q, opts, workspace, workspace_bytes, stream);
}

gemm_status_t gemm_bf16_ws(gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K, float alpha,
                           const void* A, int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                           gemm_dtype_t c_type, int64_t ldc, hipStream_t stream, const gemm_opts_t* opts,
                           void* workspace, size_t workspace_bytes) {
    return half_entry_ws(gemm::DT_BF16, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream, opts,
                         workspace, workspace_bytes);
}

gemm_status_t gemm_f16_ws(gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K, float alpha,
                          const void* A, int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                          gemm_dtype_t c_type, int64_t ldc, hipStream_t stream, const gemm_opts_t* opts,
                          void* workspace, size_t workspace_bytes) {
    return half_entry_ws(gemm::DT_F16, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream, opts,
                         workspace, workspace_bytes);
}

gemm_status_t gemm_ws_static(gemm_dtype_t in_type, gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N,
                             int64_t K, float alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
                             float beta, void* C, gemm_dtype_t c_type, int64_t ldc, hipStream_t stream,
                             const gemm_opts_t* opts) {
    g_err[0] = 0;
    if (in_type != GEMM_BF16 && in_type != GEMM_F16)
        return fail(GEMM_ERR_INVALID_ARG, "in_type %d: gemm_ws_static takes bf16 or f16 inputs", (int)in_type);
    if (c_type != GEMM_F32 && c_type != in_type)
        return fail(GEMM_ERR_INVALID_ARG, "c_type %d not offered for in_type %d", (int)c_type, (int)in_type);
    Problem q{(int)in_type, (int)c_type, (int)la, (int)lb, M, N, K, alpha, beta, A, B, C, lda, ldb, ldc};
    gemm_status_t s = validate(q);
    if (s != GEMM_OK) return s;
    // plan on stand-in addresses first: the size check needs nothing from the device
    PackPlan pp;
    gemm_plan_t plan;
    GemmParams gp;
    s = plan_ws(q, opts, nullptr, &pp, &plan, &gp);
    if (s != GEMM_OK) return s;
    if (!(pp.a || pp.b)) return launch(q.in_type, plan, gp, stream);   // nothing to rewrite
    const int64_t need = pp.a_bytes + pp.b_bytes;
    if (need > gemm::kStaticWsBytes)
        return fail(GEMM_ERR_UNSUPPORTED,
                    "the rewritten operands need %lld bytes, the static workspace holds %lld "
                    "(gemm_*_ws takes a caller workspace of any size)",
                    (long long)need, (long long)gemm::kStaticWsBytes);
    void* ws = nullptr;
    const hipError_t e = gemm::static_workspace(&ws);
    if (e != hipSuccess) return fail(GEMM_ERR_HIP, "static workspace: %s", hipGetErrorString(e));
    return run_ws(q, opts, ws, (size_t)gemm::kStaticWsBytes, stream);
}

gemm_status_t gemm_f32(gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K, float alpha,
                       const float* A, int64_t lda, const float* B, int64_t ldb, float beta, float* C, int64_t ldc,
                       hipStream_t stream) {
    return gemm_f32_ex(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, nullptr);
}

gemm_status_t gemm_bf16(gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K, float alpha,
                        const void* A, int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                        gemm_dtype_t c_type, int64_t ldc, hipStream_t stream) {
    return gemm_bf16_ex(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream, nullptr);
}

gemm_status_t gemm_f16(gemm_layout_t la, gemm_layout_t lb, int64_t M, int64_t N, int64_t K, float alpha,
                       const void* A, int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                       gemm_dtype_t c_type, int64_t ldc, hipStream_t stream) {
    return gemm_f16_ex(la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream, nullptr);
}

gemm_status_t gemm_plan(gemm_dtype_t in_type, gemm_dtype_t c_type, gemm_layout_t la, gemm_layout_t lb, int64_t M,
                        int64_t N, int64_t K, float alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
                        float beta, const void* C, int64_t ldc, const gemm_opts_t* opts, gemm_plan_t* plan) {
    g_err[0] = 0;
    if (!plan) return fail(GEMM_ERR_INVALID_ARG, "plan is NULL");
    if (in_type != GEMM_F32 && in_type != GEMM_BF16 && in_type != GEMM_F16)
        return fail(GEMM_ERR_INVALID_ARG, "in_type %d", (int)in_type);
    if (in_type == GEMM_F32 ? c_type != GEMM_F32 : (c_type != GEMM_F32 && c_type != in_type))
        return fail(GEMM_ERR_INVALID_ARG, "c_type %d not offered for in_type %d", (int)c_type, (int)in_type);
    Problem q{(int)in_type, (int)c_type, (int)la, (int)lb, M, N, K, alpha, beta, A, B, C, lda, ldb, ldc};
    gemm_status_t s = validate(q);
    if (s != GEMM_OK) return s;
    GemmParams gp;
    return choose(q, opts, plan, &gp);
}

gemm_status_t gemm_workspace_size(gemm_dtype_t in_type, gemm_dtype_t c_type, gemm_layout_t la, gemm_layout_t lb,
                                  int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                                  const void* B, int64_t ldb, float beta, const void* C, int64_t ldc,
                                  const gemm_opts_t* opts, size_t* bytes, gemm_plan_t* plan) {
    g_err[0] = 0;
    if (!bytes) return fail(GEMM_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = 0;
    if (in_type != GEMM_F32 && in_type != GEMM_BF16 && in_type != GEMM_F16)
        return fail(GEMM_ERR_INVALID_ARG, "in_type %d", (int)in_type);
    if (in_type == GEMM_F32 ? c_type != GEMM_F32 : (c_type != GEMM_F32 && c_type != in_type))
        return fail(GEMM_ERR_INVALID_ARG, "c_type %d not offered for in_type %d", (int)c_type, (int)in_type);
    Problem q{(int)in_type, (int)c_type, (int)la, (int)lb, M, N, K, alpha, beta, A, B, C, lda, ldb, ldc};
    gemm_status_t s = validate(q);
    if (s != GEMM_OK) return s;
    PackPlan pp;
    gemm_plan_t pl;
    GemmParams gp;
    s = plan_ws(q, opts, nullptr, &pp, &pl, &gp);
    if (s != GEMM_OK) return s;
    *bytes = (size_t)(pp.a_bytes + pp.b_bytes);
    if (plan) *plan = pl;
    return GEMM_OK;
}

}  // extern "C"

namespace {

// The tuner behind gemm_tune / gemm_tune_ws: every (family, tile, stage count) that the
// call with this workspace (NULL: none) would accept, timed as that call.
gemm_status_t tune(gemm_dtype_t in_type, gemm_dtype_t c_type, gemm_layout_t la, gemm_layout_t lb, int64_t M,
                   int64_t N, int64_t K, float alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
                   float beta, void* C, int64_t ldc, hipStream_t stream, void* ws, size_t ws_bytes, int reps,
                   gemm_opts_t* best, float* best_ms) {
    g_err[0] = 0;
    if (!best || !best_ms) return fail(GEMM_ERR_INVALID_ARG, "best / best_ms is NULL");
    if (reps < 1 || reps > 100000) return fail(GEMM_ERR_INVALID_ARG, "reps %d", reps);
    if (in_type != GEMM_F32 && in_type != GEMM_BF16 && in_type != GEMM_F16)
        return fail(GEMM_ERR_INVALID_ARG, "in_type %d", (int)in_type);
    if (in_type == GEMM_F32 ? c_type != GEMM_F32 : (c_type != GEMM_F32 && c_type != in_type))
        return fail(GEMM_ERR_INVALID_ARG, "c_type %d not offered for in_type %d", (int)c_type, (int)in_type);
    if (ws && (reinterpret_cast<uintptr_t>(ws) % kWsAlign))
        return fail(GEMM_ERR_INVALID_ARG, "workspace must be %lld-byte aligned", (long long)kWsAlign);
    Problem q{(int)in_type, (int)c_type, (int)la, (int)lb, M, N, K, alpha, beta, A, B, C, lda, ldb, ldc};
    gemm_status_t s = validate(q);
    if (s != GEMM_OK) return s;

    // the candidates: every (family, tile, stage count) the planner accepts for q (with
    // the workspace: also ring variants on the rewritten operands that fit in it)
    struct Cand { int kernel, tile, nstage; };
    std::vector<Cand> cands;
    const bool mfma = in_type != GEMM_F32;
    const int fams[2] = {mfma ? GEMM_KERNEL_MFMA_RING : GEMM_KERNEL_VALU_RING,
                         mfma ? GEMM_KERNEL_MFMA_STAGED : GEMM_KERNEL_VALU_STAGED};
    for (int fam : fams) {
        const Tile* tab = nullptr;
        size_t n = 0;
        if (fam == GEMM_KERNEL_VALU_RING) { tab = kValuRing; n = sizeof(kValuRing) / sizeof(Tile); }
        if (fam == GEMM_KERNEL_VALU_STAGED) { tab = kValuStaged; n = sizeof(kValuStaged) / sizeof(Tile); }
        if (fam == GEMM_KERNEL_MFMA_RING) { tab = kMfmaRing; n = sizeof(kMfmaRing) / sizeof(Tile); }
        if (fam == GEMM_KERNEL_MFMA_STAGED) { tab = kMfmaStaged; n = sizeof(kMfmaStaged) / sizeof(Tile); }
        for (size_t t = 0; t < n; ++t)
            for (int S = 1; S <= GEMM_MAX_NSTAGE; ++S) {
                gemm_opts_t o = {S, fam, tab[t].id, 0};
                gemm_plan_t pl;
                GemmParams gp;
                PackPlan pp;
                if (ws) {
                    if (plan_ws(q, &o, ws, &pp, &pl, &gp) == GEMM_OK && pl.grid > 0 &&
                        pp.a_bytes + pp.b_bytes <= (int64_t)ws_bytes)
                        cands.push_back({fam, tab[t].id, S});
                } else if (choose(q, &o, &pl, &gp) == GEMM_OK && pl.grid > 0) {
                    cands.push_back({fam, tab[t].id, S});
                }
            }
    }
    g_err[0] = 0;
    if (cands.empty()) {
        // nothing to tune (empty problem or a quick return): report the default choice
        gemm_plan_t pl;
        GemmParams gp;
        s = choose(q, nullptr, &pl, &gp);
        if (s != GEMM_OK) return s;
        *best = {pl.nstage, pl.kernel, pl.tile, 0};
        *best_ms = 0.0f;
        return GEMM_OK;
    }
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return fail(GEMM_ERR_HIP, "hipEventCreate failed");
    if (hipEventCreate(&e1) != hipSuccess) { (void)hipEventDestroy(e0); return fail(GEMM_ERR_HIP, "hipEventCreate failed"); }
    float best_t = -1.0f;
    gemm_status_t result = GEMM_OK;
    for (const Cand& c : cands) {
        gemm_opts_t o = {c.nstage, c.kernel, c.tile, 0};
        auto call = [&]() { return ws ? run_ws(q, &o, ws, ws_bytes, stream) : run(q, &o, stream); };
        s = call();                      // warm-up (code load, caches)
        if (s != GEMM_OK) { result = s; break; }
        hipError_t he = hipEventRecord(e0, stream);
        for (int r = 0; r < reps && s == GEMM_OK; ++r) s = call();
        if (s != GEMM_OK) { result = s; break; }
        if (he == hipSuccess) he = hipEventRecord(e1, stream);
        if (he == hipSuccess) he = hipEventSynchronize(e1);
        float ms = 0.0f;
        if (he == hipSuccess) he = hipEventElapsedTime(&ms, e0, e1);
        if (he != hipSuccess) { result = fail(GEMM_ERR_HIP, "timing failed: %s", hipGetErrorString(he)); break; }
        ms /= (float)reps;
        if (best_t < 0.0f || ms < best_t) { best_t = ms; *best = o; }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (result != GEMM_OK) return result;
    *best_ms = best_t;
    return GEMM_OK;
}

}  // namespace

extern "C" {

gemm_status_t gemm_tune(gemm_dtype_t in_type, gemm_dtype_t c_type, gemm_layout_t la, gemm_layout_t lb, int64_t M,
                        int64_t N, int64_t K, float alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
                        float beta, void* C, int64_t ldc, hipStream_t stream, int reps, gemm_opts_t* best,
                        float* best_ms) {
    return tune(in_type, c_type, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, nullptr, 0, reps,
                best, best_ms);
}

gemm_status_t gemm_tune_ws(gemm_dtype_t in_type, gemm_dtype_t c_type, gemm_layout_t la, gemm_layout_t lb, int64_t M,
                           int64_t N, int64_t K, float alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
                           float beta, void* C, int64_t ldc, hipStream_t stream, void* workspace,
                           size_t workspace_bytes, int reps, gemm_opts_t* best, float* best_ms) {
    if (in_type == GEMM_F32) {
        g_err[0] = 0;
        return fail(GEMM_ERR_INVALID_ARG, "gemm_tune_ws takes 16-bit inputs");
    }
    return tune(in_type, c_type, la, lb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, workspace,
                workspace_bytes, reps, best, best_ms);
}

int gemm_schedule(int kernel, int nstage, int num_k, int ksteps, int* events, int capacity) {
    if (num_k < 0 || capacity < 0 || (capacity > 0 && !events)) return -1;
    Recorder r;
    bool ok = false;
    // ksteps = k-steps per slab (low 4 bits) + 16 * code: code 0 = each slab's copy issued
    // whole at its first k-step, 1 = spread over all k-steps (one part per k-step), c >= 2 =
    // split into c - 1 parts, the first right after the barrier that frees the slot
    const int code = ksteps >> 4;
    ksteps &= 15;
    const int parts = code == 0 ? 0 : code == 1 ? ksteps : code - 1;
    if (parts > ksteps) return -1;
    if (kernel == GEMM_KERNEL_VALU_RING || kernel == GEMM_KERNEL_MFMA_RING) {
        switch (nstage) {
            case 1: ok = rec_ring_ks<1>(r, ksteps, num_k, parts); break;
            case 2: ok = rec_ring_ks<2>(r, ksteps, num_k, parts); break;
            case 3: ok = rec_ring_ks<3>(r, ksteps, num_k, parts); break;
            case 4: ok = rec_ring_ks<4>(r, ksteps, num_k, parts); break;
            case 5: ok = rec_ring_ks<5>(r, ksteps, num_k, parts); break;
        }
    } else if (kernel == GEMM_KERNEL_VALU_STAGED || kernel == GEMM_KERNEL_MFMA_STAGED) {
        if (code != 0) return -1;
        switch (nstage) {
            case 1: ok = rec_staged_ks<1>(r, ksteps, num_k); break;
            case 2: ok = rec_staged_ks<2>(r, ksteps, num_k); break;
        }
    }
    if (!ok) return -1;
    const int n = (int)(r.ev.size() / 4);
    const int w = n < capacity ? n : capacity;
    if (w > 0) memcpy(events, r.ev.data(), sizeof(int) * 4 * (size_t)w);
    return n;
}

gemm_status_t gemm_pipe_copy(void* dst, const void* src, int64_t bytes, int nstage, hipStream_t stream) {
    g_err[0] = 0;
    if (bytes < 0) return fail(GEMM_ERR_INVALID_ARG, "bytes %lld < 0", (long long)bytes);
    if (nstage < 0 || nstage > 4) return fail(GEMM_ERR_UNSUPPORTED, "nstage %d: the copy ring has 1..4 slots", nstage);
    if (bytes % gemm::kCopySlab != 0)
        return fail(GEMM_ERR_INVALID_ARG, "bytes %lld is not a multiple of %d", (long long)bytes, gemm::kCopySlab);
    if (bytes == 0) return GEMM_OK;
    if (!dst || !src) return fail(GEMM_ERR_INVALID_ARG, "null pointer");
    if (!aligned16(dst) || !aligned16(src)) return fail(GEMM_ERR_INVALID_ARG, "dst and src must be 16-byte aligned");
    const char* s0 = static_cast<const char*>(src);
    const char* d0 = static_cast<const char*>(dst);
    if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(GEMM_ERR_INVALID_ARG, "dst and src overlap");
    gemm::CopyParams p;
    p.src = s0;
    p.dst = static_cast<char*>(dst);
    p.slabs = bytes / gemm::kCopySlab;
    // about 8 workgroups per CU, each streaming a contiguous run of slabs
    const int64_t max_wg = 2048;
    p.per_wg = (p.slabs + max_wg - 1) / max_wg;
    const int64_t grid = (p.slabs + p.per_wg - 1) / p.per_wg;
    const hipError_t e = gemm::launch_pipe_copy(nstage ? nstage : 2, p, grid, stream);
    if (e != hipSuccess) return fail(GEMM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return GEMM_OK;
}

gemm_status_t gemm_mfma_ceiling(int in_type, int shape, const void* frags, float* sums, int64_t grid, int64_t iters,
                                hipStream_t stream) {
    g_err[0] = 0;
    if (in_type != GEMM_BF16 && in_type != GEMM_F16)
        return fail(GEMM_ERR_UNSUPPORTED, "in_type %d: the matrix instructions take bf16 or f16", in_type);
    if (shape != 16 && shape != 32) return fail(GEMM_ERR_UNSUPPORTED, "shape %d: 16 (16x16x32) or 32 (32x32x16)", shape);
    if (grid < 1 || grid > GEMM_CEIL_MAX_GRID)
        return fail(GEMM_ERR_INVALID_ARG, "grid %lld outside 1..%d", (long long)grid, GEMM_CEIL_MAX_GRID);
    if (iters < 0) return fail(GEMM_ERR_INVALID_ARG, "iters %lld < 0", (long long)iters);
    if (!frags || !sums) return fail(GEMM_ERR_INVALID_ARG, "null pointer");
    if (!aligned16(frags)) return fail(GEMM_ERR_INVALID_ARG, "frags must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(sums) & 3) return fail(GEMM_ERR_INVALID_ARG, "sums must be 4-byte aligned");
    static_assert(gemm::kCeilFrags * 64 * 8 == GEMM_CEIL_FRAG_ELEMS, "fragment set size");
    static_assert(gemm::kCeilThreads == GEMM_CEIL_THREADS, "threads per workgroup");
    const hipError_t e = gemm::launch_mfma_ceiling(in_type == GEMM_BF16 ? gemm::DT_BF16 : gemm::DT_F16, shape,
                                                   static_cast<const uint16_t*>(frags), sums, grid, iters, stream);
    if (e != hipSuccess) return fail(GEMM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return GEMM_OK;
}

}  // extern "C"

namespace {

// The host-side ring behind gemm_h2d_staged / gemm_h2d_staged_async: the CPU fills
// page-locked slot c mod nstage with chunk c while the DMA engine drains the slots filled
// before; a slot is refilled only once the DMA that read it has completed (one event per
// slot).  drain: wait for the last DMAs too before returning.
gemm_status_t h2d_ring(void* dst, const void* src, int64_t bytes, void* staging, int64_t chunk_bytes, int nstage,
                       hipStream_t stream, bool drain) {
    g_err[0] = 0;
    if (bytes < 0) return fail(GEMM_ERR_INVALID_ARG, "bytes %lld < 0", (long long)bytes);
    if (nstage < 1 || nstage > 4) return fail(GEMM_ERR_UNSUPPORTED, "nstage %d: the staging ring has 1..4 slots", nstage);
    if (chunk_bytes < 1) return fail(GEMM_ERR_INVALID_ARG, "chunk_bytes %lld < 1", (long long)chunk_bytes);
    if (bytes == 0) return GEMM_OK;
    if (!dst || !src || !staging) return fail(GEMM_ERR_INVALID_ARG, "null pointer");
    const char* s0 = static_cast<const char*>(src);
    const char* g0 = static_cast<const char*>(staging);
    const int64_t ring = chunk_bytes * nstage;
    if (s0 < g0 + ring && g0 < s0 + bytes) return fail(GEMM_ERR_INVALID_ARG, "src and staging overlap");
    hipEvent_t ev[4];
    int made = 0;
    gemm_status_t result = GEMM_OK;
    for (; made < nstage; ++made)
        if (hipEventCreateWithFlags(&ev[made], hipEventDisableTiming) != hipSuccess) {
            result = fail(GEMM_ERR_HIP, "hipEventCreateWithFlags failed");
            break;
        }
    char* d0 = static_cast<char*>(dst);
    char* slots = static_cast<char*>(staging);
    const int64_t nchunks = result == GEMM_OK ? (bytes + chunk_bytes - 1) / chunk_bytes : 0;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int slot = (int)(c % nstage);
        const int64_t off = c * chunk_bytes;
        const int64_t len = bytes - off < chunk_bytes ? bytes - off : chunk_bytes;
        hipError_t e = hipSuccess;
        if (c >= nstage) e = hipEventSynchronize(ev[slot]);  // wait until that slot's DMA has read it
        if (e == hipSuccess) {
            memcpy(slots + slot * chunk_bytes, s0 + off, (size_t)len);  // the CPU fills the slot ...
            e = hipMemcpyAsync(d0 + off, slots + slot * chunk_bytes, (size_t)len, hipMemcpyHostToDevice, stream);
        }
        if (e == hipSuccess) e = hipEventRecord(ev[slot], stream);  // ... while the DMA drains the others
        if (e != hipSuccess) { result = fail(GEMM_ERR_HIP, "staged copy failed: %s", hipGetErrorString(e)); break; }
    }
    for (int i = 0; i < made; ++i) {
        // synchronous form: the staging buffer is the caller's again only once every DMA that
        // reads it is done; the asynchronous form leaves the last ones running (an event may be
        // destroyed while its work is pending)
        if ((drain || result != GEMM_OK) && i < nchunks) {
            const hipError_t e = hipEventSynchronize(ev[i]);
            if (e != hipSuccess && result == GEMM_OK) result = fail(GEMM_ERR_HIP, "staged copy failed: %s", hipGetErrorString(e));
        }
        (void)hipEventDestroy(ev[i]);
    }
    return result;
}

}  // namespace

extern "C" {

gemm_status_t gemm_h2d_staged(void* dst, const void* src, int64_t bytes, void* staging, int64_t chunk_bytes,
                              int nstage, hipStream_t stream) {
    return h2d_ring(dst, src, bytes, staging, chunk_bytes, nstage, stream, true);
}

gemm_status_t gemm_h2d_staged_async(void* dst, const void* src, int64_t bytes, void* staging, int64_t chunk_bytes,
                                    int nstage, hipStream_t stream) {
    return h2d_ring(dst, src, bytes, staging, chunk_bytes, nstage, stream, false);
}

const char* gemm_status_string(gemm_status_t s) {
    switch (s) {
        case GEMM_OK: return "GEMM_OK";
        case GEMM_ERR_INVALID_ARG: return "GEMM_ERR_INVALID_ARG";
        case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED";
        case GEMM_ERR_HIP: return "GEMM_ERR_HIP";
    }
    return "GEMM_ERR_UNKNOWN";
}

const char* gemm_last_error(void) { return g_err; }

}  // extern "C"
