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
    int32_t trans_b;     // b holds the weights transposed: n rows of k elements (bf16 / fp16, k % 32 == 0)
};

// Fixed-order sum of nsrc row blocks: dst[dst_row0 + j] = sum_r src[r][src_row0 + j],
// j < rows, all rows n elements wide (leading dimension n).
struct ReduceLaunch {
    coc_dtype dt;
    const void* src[COC_MAX_WORLD];
    int32_t nsrc;
    void* dst;
    int64_t src_row0, dst_row0, rows, n;
    bool wide;   // the launch runs alone (not beside a matmul): more loads in flight per thread
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
    uint32_t* signal;        // if set: ready lines of the chunk; each workgroup adds 1 to one
};

// Matmul over every chunk of an op in one launch (bf16 / fp16, k a positive
// multiple of 32), as a list of pieces walked in order.  Piece i covers the
// output rows of its row map { base + b*stride + j : b < nblk, j < rpb } and
// reads A row (output row + ashift) from a[i].  Before its first tile of
// piece i a workgroup waits for the sum of ready group wait[i]'s lines to
// reach ready_target[wait[i]] (wait[i] >= 0, ready set); after each tile of
// piece i it adds 1 to done[signal[i]] (signal[i] >= 0, done set).  Counter
// layout as below.
constexpr int kMaxPieces = 16;
// How a chunk-walking launch runs the all-gather itself (see
// chunks_fused_gather): chunks [0, early) are copied by all `workgroups` of
// the launch, the rest by `gatherers` of them; each adds 1 per chunk share to
// that chunk's ready lines.  gatherers == 0: the launch cannot (it needs at
// least 16 one-tile workgroups and all workgroups resident at once).
struct FusedGatherPlan {
    int32_t gatherers, early, workgroups;
};

struct ChunksLaunch {
    GemmKind kind;
    const void* b;
    void* c;
    int64_t n, k;
    const void* scales;  // w8a16 only
    int32_t qmode, group;
    // trans_b: b holds the weights transposed (n rows of k elements);
    // trans_a: the single piece's a holds the activations transposed (k rows
    // of lda elements, one per output row; no row map)
    int32_t trans_a, trans_b;
    int64_t lda;
    int32_t npieces;
    const void* a[kMaxPieces];
    const void* bp[kMaxPieces];   // piece i's weights if set (a grouped matmul), else b
    int64_t ashift[kMaxPieces];
    int64_t base[kMaxPieces], stride[kMaxPieces], rpb[kMaxPieces];
    int32_t nblk[kMaxPieces];
    int32_t wait[kMaxPieces];
    int32_t signal[kMaxPieces];
    uint32_t* done;
    uint32_t* ready;
    uint32_t ready_target[COC_MAX_SPLIT];
    // 0: each workgroup walks whole rounds of the list in order, so chunks
    // finish in order (compute first); 1: workgroups with two tiles of the
    // last two rounds start on the first chunks (communicate first)
    int32_t order;
    uint32_t spin_limit;     // polls before a wait gives up (0: the default, about 2 s)
    uint32_t* gave_up;       // set to non-zero by a wait that gives up (may be NULL)
    // All-gather rows that the launch copies itself (gather_nchunks > 0; see
    // chunks_fused_gather): chunk c's rows [gather_row0[c], + gather_rows[c])
    // and [gather_row0b[c], + gather_rowsb[c]) (0 rows: none); gathered row g
    // comes from row g % gather_shard_rows of gather_src[g / gather_shard_rows].
    int32_t gather_nchunks;
    FusedGatherPlan gather_plan;   // as chunks_fused_gather returned it (the launch checks it)
    const void* gather_src[COC_MAX_WORLD];
    void* gather_dst;
    int64_t gather_row_bytes, gather_shard_rows;
    int64_t gather_row0[COC_MAX_SPLIT], gather_rows[COC_MAX_SPLIT];
    int64_t gather_row0b[COC_MAX_SPLIT], gather_rowsb[COC_MAX_SPLIT];
};

// Layout of the chunk hand-over counters (device memory, 32-bit words): each
// counter on its own 128-byte line.  done[c] at line c; ready[c] is spread
// over kReadyLines lines from line COC_MAX_SPLIT + c * kReadyLines (gather
// workgroup b adds to line b % kReadyLines, so its adds do not queue on one
// address) and a waiter sums them.
// The line after them holds the "gave up" word: a wait that gives up stores
// a non-zero value into it (read and cleared by coc_check_waits).
constexpr int kSyncWords = 32;
constexpr int kReadyLines = 16;
constexpr int kGaveUpLine = COC_MAX_SPLIT + COC_MAX_SPLIT * kReadyLines;
constexpr int kSyncLines = kGaveUpLine + 1;

// The reduce that waits beside the one-launch matmul: every chunk in one
// launch, chunk c's rows once done[c] reaches target[c].
struct ReduceChunksLaunch {
    ReduceLaunch r;          // sources, destination, n, dtype; rows fields unused
    int32_t nchunks;
    int64_t src_row0[COC_MAX_SPLIT], dst_row0[COC_MAX_SPLIT], rows[COC_MAX_SPLIT];
    const uint32_t* done;    // counter lines as above
    uint32_t target[COC_MAX_SPLIT];
    int32_t own;             // index of the source the matmul is writing meanwhile
    bool narrow;             // one vector per thread: fits beside a matmul using more registers
    uint32_t spin_limit;     // polls before a wait gives up (0: the default, about 2 s)
    uint32_t* gave_up;       // set to non-zero by a wait that gives up (may be NULL)
};

// The copy of an expert all-to-all, chunk by chunk.  Chunk c covers local
// rows [row0[c], row0[c] + rows[c]) of `local` (the received matrix, or the
// grouped matmul's output), cut into segments seg0[c] .. seg0[c + 1] - 1 in
// row order; segment i pairs its local rows with `rows` rows of remote buffer
// remote[buf] from remote_row on.  to_remote == 0 copies remote -> local
// (dispatch; system-scope stores, then each workgroup adds 1 to one of the
// chunk's ready lines), 1 copies local -> remote (combine; each chunk first
// waits for done[c] to reach target[c], if done is set).  All rows are
// row_bytes wide (a multiple of 16).
constexpr int kMaxA2ASegs = 128;
struct A2ASegment {
    int32_t local_row, remote_row, rows, buf;
};
struct A2ALaunch {
    void* remote[COC_MAX_WORLD];
    void* local;
    int64_t row_bytes;
    int32_t to_remote;
    int32_t nchunks;
    int64_t row0[COC_MAX_SPLIT], rows[COC_MAX_SPLIT];
    int32_t seg0[COC_MAX_SPLIT + 1];
    A2ASegment seg[kMaxA2ASegs];
    uint32_t* ready;            // dispatch: counter lines as above
    const uint32_t* done;       // combine: counter lines as above
    uint32_t target[COC_MAX_SPLIT];
    uint32_t spin_limit;        // polls before a wait gives up (0: the default, about 2 s)
    uint32_t* gave_up;          // set to non-zero by a wait that gives up (may be NULL)
};

// Launchers (kernels.hip).  Return a hipError_t value (0 = success).  The
// caller guarantees that every size and pointer has been validated.
int launch_gemm(const GemmLaunch& g, void* stream);
// Activity stamps for measurement: while buf is set, launches of the matmul,
// reduce and gather kernels take consecutive regions of its `records` slots
// (three words each; layout in kernels.hip); stamp_records_used() is how many
// slots have been handed out since.
void set_stamp_buffer(uint64_t* buf, int64_t records);
int64_t stamp_records_used();
// Zeroes n 32-bit words at p (device memory) on `stream`.
int launch_zero_words(uint32_t* p, int n, void* stream);
int launch_reduce(const ReduceLaunch& r, void* stream);
int launch_reduce_chunks(const ReduceChunksLaunch& r, void* stream);
// *groups (if given) receives the number of workgroups launched (signals sent).
int launch_gather(const GatherLaunch& g, void* stream, int32_t* groups = nullptr);
// Every chunk of an all-gather in one launch (system-scope stores); chunk c's
// workgroups then add 1 each to its ready lines (at ready + c * kReadyLines
// lines).  *per_chunk receives the workgroups per chunk (the adds each gets).
int launch_gather_chunks(const GatherLaunch& g, int nchunks, const int64_t* row0, const int64_t* rows,
                         uint32_t* ready, void* stream, int32_t* per_chunk);

// The all-to-all copy above in one launch.  Dispatch: *per_chunk receives
// the workgroups per chunk (the adds each chunk's ready lines get).  Combine:
// at most one workgroup per CU, walking the chunks in order.
int launch_a2a_chunks(const A2ALaunch& a, void* stream, int32_t* per_chunk);

// Whether the ring kernels take this matmul (bf16 / fp16 with k a positive
// multiple of 32; w8a16 also needs n % 16 == 0 and, per group, group % 32 == 0
// with the tile's scale rows fitting in LDS).
bool chunks_supported(const GemmLaunch& g);
// tiles[i] receives the tile count of piece i (the adds its signal gets) and
// tiles[kMaxPieces] the number of workgroups launched.
int launch_gemm_chunks(const ChunksLaunch& L, void* stream, int32_t tiles[kMaxPieces + 1]);
// Tiles per piece of L's launch, and in tiles[kMaxPieces] its workgroups
// (what launch_gemm_chunks reports), without launching.
void chunks_tiles(const ChunksLaunch& L, int32_t tiles[kMaxPieces + 1]);
// Whether the waiting reduce beside this launch must be the one-vector form
// (the matmul leaves too few VGPRs for the two-vector one to share a CU).
bool chunks_reduce_narrow(const ChunksLaunch& L);
// The plan by which L's launch would run the gather itself (L.gather_nchunks
// set); the caller sets each chunk's ready target from it.
FusedGatherPlan chunks_fused_gather(const ChunksLaunch& L);

}  // namespace coc
