// Internal declarations shared by the host translation units (plan, API) and
// the kernel launchers.  Nothing here is part of the public C ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include "coc.h"

namespace coc {

// ------------------------------------------------------------------ errors
// Thread-local "last error" text behind coc_last_error().
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();
coc_status fail(coc_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

size_t elem_size(coc_dtype dt);
bool dtype_valid(coc_dtype dt);

// ------------------------------------------------------------------ plan
// A validated problem plus the chunk descriptors of its pipeline.
struct Plan {
    coc_op op;
    coc_dtype dt;
    int32_t world, rank, split, det;
    int64_t m, n, k;
    int32_t nchunks;
    coc_chunk chunk[COC_MAX_SPLIT];  // in pipeline order
};

// Shape rules and chunk construction (no pointers, no GPU).  On error sets
// the thread-local message and returns the status.
coc_status make_plan(coc_op op, int64_t m, int64_t n, int64_t k, coc_dtype dt,
                     int32_t world, int32_t rank, int32_t split, int32_t det, Plan* out);

size_t workspace_bytes(const Plan& p);

// ------------------------------------------------------------------ launches
// Kernel classes for timing (match COC_KCLASS_*).
enum KClass { KC_GEMM = 0, KC_REDUCE = 1, KC_GATHER = 2 };

// Matmul over one chunk: C[rows] = A[rows] @ B, rows given by a row map
// { base + b*stride + j : b < nblk, j < rpb }.  A and C are m-row matrices of
// 16-bit or 32-bit elements; B is k x n of the same type, or int8 with fp16
// scales (w8a16).
enum GemmKind { GK_F32 = 0, GK_F16 = 1, GK_BF16 = 2, GK_W8_F16 = 3 };

struct GemmLaunch {
    GemmKind kind;
    const void* a;
    const void* b;
    void* c;
    const void* scales;  // w8a16 only
    int32_t qmode;       // coc_quant_mode, w8a16 only
    int32_t group;       // per-group size, w8a16 only
    int64_t n, k;        // lda = k, ldb = ldc = n
    int64_t base, stride, rpb;
    int32_t nblk;
    int32_t concurrent;  // chunk matmuls expected to run side by side (tile choice only)
};

// Fixed-order sum of nsrc row blocks: dst[dst_row0 + j] = sum_r src[r][src_row0 + j],
// j < rows, all rows n elements wide (leading dimension n).
struct ReduceLaunch {
    coc_dtype dt;
    const void* src[COC_MAX_WORLD];
    int32_t nsrc;
    void* dst;
    int64_t src_row0, dst_row0, rows, n;
    const uint32_t* wait;    // if set, the kernel first waits for *wait >= wait_target
    uint32_t wait_target;
    int32_t own;             // with wait: index of the source being written meanwhile
};

// Bit copy of gathered rows: dst[row] = shard (row / shard_rows), local row
// row % shard_rows, for row in [row0, row0 + rows); rows are k elements wide.
struct GatherLaunch {
    coc_dtype dt;
    const void* src[COC_MAX_WORLD];
    int32_t nsrc;
    int64_t shard_rows;
    void* dst;
    int64_t row0, rows, k;
    uint32_t* signal;        // if set, each workgroup adds 1 once its rows are stored
};

// Matmul over every chunk of an op in one launch (bf16 / fp16, k a positive
// multiple of 32): chunk c's rows come from its row map.  Before its first
// tile of chunk c a workgroup waits for ready[c] >= ready_target[c] (if ready
// is set); after each tile of chunk c it adds 1 to done[c] (if done is set).
struct ChunksLaunch {
    GemmKind kind;
    const void* a;
    const void* b;
    void* c;
    int64_t n, k;
    int32_t nchunks;
    int64_t base[COC_MAX_SPLIT], stride[COC_MAX_SPLIT], rpb[COC_MAX_SPLIT];
    int32_t nblk[COC_MAX_SPLIT];
    uint32_t* done;
    const uint32_t* ready;
    uint32_t ready_target[COC_MAX_SPLIT];
};

// Launchers (kernels.hip).  Return a hipError_t value (0 = success).  The
// caller guarantees that every size and pointer has been validated.
int launch_gemm(const GemmLaunch& g, void* stream);
int launch_reduce(const ReduceLaunch& r, void* stream);
// *groups (if given) receives the number of workgroups launched (signals sent).
int launch_gather(const GatherLaunch& g, void* stream, int32_t* groups = nullptr);

bool chunks_supported(GemmKind kind, int64_t k);
// tiles[c] receives the tile count of chunk c (the completions done[c] gets).
int launch_gemm_chunks(const ChunksLaunch& L, void* stream, int32_t tiles[COC_MAX_SPLIT]);

}  // namespace coc
