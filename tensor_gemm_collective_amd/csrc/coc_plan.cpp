// Host-only validation and pipeline planning.  No HIP calls: everything in
// this file runs (and is tested) without a GPU.
//
// Chunking follows the CoC guide ("Approach", script-level implementation):
// the left matrix of the matmul is split along m into `split` pieces, and m
// must be a multiple of the split count (also the Overlap blog, third layer,
// caveats).  How the pieces map to rows is not stated; the choices below are
// readings:
//   * all-reduce: contiguous row blocks in order;
//   * reduce-scatter: chunk i takes the i-th 1/split of EVERY rank's row
//     slice, so each chunk carries reduction work for this rank (with
//     contiguous blocks all of this rank's reduction would sit in one chunk
//     and nothing would overlap);
//   * all-gather: contiguous row blocks of the gathered matrix, the pipeline
//     starting at the block holding this rank's own shard (available without
//     communication) and wrapping around.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "coc_internal.h"

namespace coc {

namespace {
thread_local std::string g_last_error;

void vset(const char* fmt, va_list ap) {
    char buf[512];
    vsnprintf(buf, sizeof buf, fmt, ap);
    g_last_error = buf;
}
}  // namespace

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vset(fmt, ap);
    va_end(ap);
}

void clear_error() { g_last_error.clear(); }

coc_status fail(coc_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vset(fmt, ap);
    va_end(ap);
    return s;
}

size_t elem_size(coc_dtype dt) { return dt == COC_F32 ? 4 : 2; }

bool dtype_valid(coc_dtype dt) { return dt == COC_F32 || dt == COC_F16 || dt == COC_BF16; }

static const int64_t kMaxElems = int64_t(1) << 31;

coc_status make_plan(coc_op op, int64_t m, int64_t n, int64_t k, coc_dtype dt,
                     int32_t world, int32_t rank, int32_t split, int32_t det, Plan* out) {
    if (!(op >= COC_OP_MATMUL_ALL_REDUCE && op <= COC_OP_MATMUL_ALL_REDUCE_W8A16))
        return fail(COC_ERR_SHAPE, "unknown op %d", int(op));
    if (!(split == 1 || split == 2 || split == 4 || split == 8))
        return fail(COC_ERR_SPLIT, "split must be 1, 2, 4 or 8 (got %d)", split);
    if (world < 1 || world > COC_MAX_WORLD)
        return fail(COC_ERR_WORLD, "world must be in [1, %d] (got %d)", COC_MAX_WORLD, world);
    if (rank < 0 || rank >= world)
        return fail(COC_ERR_WORLD, "rank %d out of range for world %d", rank, world);
    if (op == COC_OP_MATMUL_ALL_REDUCE_W8A16) {
        dt = COC_F16;
    } else if (!dtype_valid(dt)) {
        return fail(COC_ERR_DTYPE, "dtype %d not supported", int(dt));
    }
    if (m < 0 || n < 0 || k < 0)
        return fail(COC_ERR_SHAPE, "negative size (m=%lld n=%lld k=%lld)", (long long)m,
                    (long long)n, (long long)k);
    if (n % 8 != 0 || k % 8 != 0)
        return fail(COC_ERR_SHAPE, "n and k must be multiples of 8 (n=%lld k=%lld)",
                    (long long)n, (long long)k);
    // each dimension below 2^31 first, so the int64 products cannot overflow
    if (m >= kMaxElems || n >= kMaxElems || k >= kMaxElems || m * k >= kMaxElems ||
        k * n >= kMaxElems || m * n >= kMaxElems)
        return fail(COC_ERR_SHAPE, "a matrix has 2^31 or more elements (m=%lld n=%lld k=%lld)",
                    (long long)m, (long long)n, (long long)k);

    Plan p{};
    p.op = op;
    p.dt = dt;
    p.world = world;
    p.rank = rank;
    p.split = split;
    p.det = det ? 1 : 0;
    p.m = m;
    p.n = n;
    p.k = k;
    p.nchunks = split;

    switch (op) {
        case COC_OP_MATMUL_ALL_REDUCE:
        case COC_OP_MATMUL_ALL_REDUCE_W8A16: {
            if (m % split != 0)
                return fail(COC_ERR_SHAPE, "m=%lld is not a multiple of split=%d", (long long)m, split);
            const int64_t cm = m / split;
            for (int i = 0; i < split; ++i) {
                coc_chunk& c = p.chunk[i];
                c.base = i * cm;
                c.stride = 0;
                c.rows_per_blk = cm;
                c.nblk = 1;
                c.order = i;
                c.red_base = c.base;
                c.out_base = c.base;
                c.red_rows = cm;
            }
            break;
        }
        case COC_OP_MATMUL_REDUCE_SCATTER: {
            if (m % world != 0)
                return fail(COC_ERR_SHAPE, "m=%lld is not a multiple of world=%d", (long long)m, world);
            const int64_t slice = m / world;
            if (slice % split != 0)
                return fail(COC_ERR_SHAPE, "m/world=%lld is not a multiple of split=%d",
                            (long long)slice, split);
            const int64_t sub = slice / split;
            for (int i = 0; i < split; ++i) {
                coc_chunk& c = p.chunk[i];
                c.base = i * sub;
                c.stride = slice;
                c.rows_per_blk = sub;
                c.nblk = world;
                c.order = i;
                c.red_base = int64_t(rank) * slice + i * sub;
                c.out_base = i * sub;
                c.red_rows = sub;
            }
            break;
        }
        case COC_OP_ALLGATHER_MATMUL:
        case COC_OP_ALLGATHER_MATMUL_V2: {
            if (m % world != 0)
                return fail(COC_ERR_SHAPE, "m=%lld is not a multiple of world=%d", (long long)m, world);
            if (m % split != 0)
                return fail(COC_ERR_SHAPE, "m=%lld is not a multiple of split=%d", (long long)m, split);
            const int64_t cm = m / split;
            const int64_t shard = m / world;
            const int first = cm ? int((int64_t(rank) * shard) / cm) : 0;
            for (int j = 0; j < split; ++j) {
                const int ci = (first + j) % split;
                coc_chunk& c = p.chunk[j];
                c.base = ci * cm;
                c.stride = 0;
                c.rows_per_blk = cm;
                c.nblk = 1;
                c.order = j;
                c.red_base = c.base;
                c.out_base = c.base;
                c.red_rows = cm;
            }
            break;
        }
    }
    *out = p;
    return COC_OK;
}

size_t workspace_bytes(const Plan& p) {
    if (p.op == COC_OP_ALLGATHER_MATMUL) return size_t(p.m) * size_t(p.k) * elem_size(p.dt);
    return 0;
}

}  // namespace coc

using namespace coc;

extern "C" {

const char* coc_status_string(coc_status s) {
    switch (s) {
        case COC_OK: return "COC_OK";
        case COC_ERR_NULL: return "COC_ERR_NULL";
        case COC_ERR_SPLIT: return "COC_ERR_SPLIT";
        case COC_ERR_SHAPE: return "COC_ERR_SHAPE";
        case COC_ERR_WORLD: return "COC_ERR_WORLD";
        case COC_ERR_DTYPE: return "COC_ERR_DTYPE";
        case COC_ERR_ALIGN: return "COC_ERR_ALIGN";
        case COC_ERR_WORKSPACE: return "COC_ERR_WORKSPACE";
        case COC_ERR_HIP: return "COC_ERR_HIP";
        case COC_ERR_ALIAS: return "COC_ERR_ALIAS";
        case COC_ERR_CAPTURE: return "COC_ERR_CAPTURE";
        case COC_ERR_TIMEOUT: return "COC_ERR_TIMEOUT";
    }
    return "COC_ERR_UNKNOWN";
}

const char* coc_last_error(void) { return g_last_error.c_str(); }

size_t coc_workspace_bytes(int op, int64_t m, int64_t n, int64_t k, coc_dtype dt,
                           int32_t world, int32_t split) {
    if (op < COC_OP_MATMUL_ALL_REDUCE || op > COC_OP_MATMUL_ALL_REDUCE_W8A16) return 0;
    Plan p;
    const std::string saved = g_last_error;
    coc_status s = make_plan((coc_op)op, m, n, k, dt, world, 0, split, 0, &p);
    g_last_error = saved;
    return s == COC_OK ? workspace_bytes(p) : 0;
}

coc_status coc_plan(coc_op op, int64_t m, int32_t world, int32_t rank, int32_t split,
                    coc_chunk* chunks, int32_t max_chunks, int32_t* n_chunks) {
    clear_error();
    Plan p;
    coc_status s = make_plan(op, m, 8, 8, COC_BF16, world, rank, split, 0, &p);
    if (s != COC_OK) return s;
    if (!n_chunks) return fail(COC_ERR_NULL, "n_chunks is NULL");
    *n_chunks = p.nchunks;
    if (chunks) {
        for (int i = 0; i < p.nchunks && i < max_chunks; ++i) chunks[i] = p.chunk[i];
    }
    return COC_OK;
}

}  // extern "C"
