/*
 * coc.h -- fused matmul + tensor-parallel collective ("communication over
 * computation", CoC) for AMD Instinct MI355X (gfx950), one rank's share.
 *
 * Pages cited by title and section:
 *   CoC guide    Ascend PyTorch developer guide, MindSpeed page
 *                "Communication-over-Computation (计算通信并行)".
 *   Overlap blog "MindSpeed LLM通信计算重叠与MC2如何榨干昇腾芯片算力".
 *
 * What is computed (CoC guide, "Problem analysis"): the forward of
 * ColumnParallelLinear / RowParallelLinear is a matmul tightly coupled with a
 * collective -- AllReduce without sequence parallelism, AllGather before /
 * ReduceScatter after the matmul with it.  CoC (CoC guide, "Approach") splits
 * the left matrix along m into 2, 4 or 8 pieces so the matmul of one piece
 * runs while the collective of another is in flight.
 *
 * One-GPU model of a rank.  This library runs rank `rank` of a
 * tensor-parallel group of `world` ranks on a single GPU: what the other
 * ranks would contribute over the interconnect (their partial products or
 * their sequence shards) is handed in as buffers in the same device memory
 * (`peer_bufs`).  The communication step becomes a streaming read of those
 * buffers; the split/pipeline structure is the same one a multi-GPU version
 * would use with remote pointers.
 *
 * Common conventions
 *   - All matrices are dense and row-major.  X is m x k, W is k x n,
 *     Y and partials are m x n (leading dimensions = number of columns).
 *   - Every pointer argument except `peer_bufs` itself is a DEVICE pointer
 *     owned by the caller and must be 16-byte aligned.  `peer_bufs` is a
 *     HOST array of `world` device pointers, read during the call only;
 *     entry `rank` is ignored (may be NULL).  The library never allocates,
 *     frees or retains caller memory.
 *   - Inputs and outputs must not overlap.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *     asynchronous in stream order: work the library puts on its internal
 *     side stream is joined back into `stream` before the call returns, so
 *     later work on `stream` sees the outputs.  Inputs must stay valid until
 *     that work completes.  Different host threads may use different streams
 *     concurrently; two threads must not use the same stream concurrently.
 *     The pipelined forms whose workgroups wait on device counters (the
 *     one-launch pipelines) need their work resident together, so on one
 *     device the library runs them one after another even when they come
 *     from different streams: such a call waits on its stream for the
 *     previous one (unless the stream is being captured into a graph).
 *   - Graph capture: the matmul/collective ops may be captured into a HIP
 *     graph and replayed.  A captured call takes the per-chunk event
 *     pipeline (separate matmul, reduce and gather launches joined by
 *     events), because the one-launch pipelines hand chunks over through
 *     device counters whose targets the host advances call by call and a
 *     replay would repeat.  The first call on a stream creates the
 *     library's side streams and counters for it and synchronises the
 *     device, so it must not be captured: call once on the stream before
 *     capturing it (COC_ERR_CAPTURE otherwise).  The MoE all-to-all pair
 *     works only through those counters and returns COC_ERR_CAPTURE under
 *     capture.  Replays of one graph must not overlap each other.  One
 *     capture holds at most one call of this library: a second call made
 *     while the same capture is open (on any stream) returns
 *     COC_ERR_CAPTURE and enqueues nothing.
 *   - `split` is the number of m-chunks the work is pipelined over: 1
 *     (serial, no overlap), 2, 4 or 8 (CoC guide, "Usage": the split count
 *     options; the m dimension must divide by it, CoC guide "Approach" and
 *     Overlap blog, third-layer caveats).  For the compute-first ops (all-
 *     reduce, reduce-scatter, w8A16) on one GPU the reduction beside the
 *     matmul competes with it for the compute units' memory path and power,
 *     so the library pipelines them only when the reduction would take at
 *     least a sixth of the matmul's time (estimated from the sizes) and some
 *     chunk's tiles all come before the matmul's last round of tiles (a
 *     matmul that fills the GPU once finishes every chunk together);
 *     otherwise the call runs the serial schedule.  Result bits never depend
 *     on the split or on this choice.
 *   - The *_trans_w entry points (matmul all-reduce / reduce-scatter /
 *     all-gather) take the same arguments as the plain ones, but `w` holds
 *     the weights transposed, n rows of k elements, so the backward pass of
 *     a layer (CoC guide, "Approach": forward / backward operator pairs)
 *     multiplies by the forward k x n weight read as its transpose without
 *     copying it: dX = dY @ W^T.  bf16 / fp16 and k % 32 == 0; the result
 *     bits equal those of the plain entry point with the transpose stored.
 *   - `deterministic` != 0 selects the deterministic variants (CoC guide,
 *     "Approach", fused-operator list): partial sums are added in ascending
 *     rank order 0..world-1 in binary32 with this rank's own partial taken
 *     as stored in `partial_out`, and the sum is rounded once to the dtype.
 *     The bits of the result then do not depend on `split`, on the run, or
 *     on which rank computes it.  Non-deterministic mode may use any order.
 *   - Rounding to fp16 / bf16 is round-to-nearest-even everywhere; matmuls
 *     accumulate in binary32.
 *   - Size limits: world in [1, COC_MAX_WORLD], rank in [0, world);
 *     n and k multiples of 8; each of m*k, k*n, m*n below 2^31 elements.
 *     m, n or k may be 0.
 *
 * Errors.  Arguments are validated on the host before anything is enqueued;
 * on any error the call returns a non-zero coc_status, enqueues nothing and
 * writes nothing, and coc_last_error() returns a description (per host
 * thread).  COC_ERR_HIP wraps a failing HIP runtime call and carries its
 * message.  No C++ exception crosses this interface.
 *
 * Hand-over waits.  The pipelined forms hand chunks between kernels through
 * device counters; every wait is bounded (about 2 s), and a wait that gives
 * up writes NaN into the tile or rows it guards instead of hanging, and
 * records that it gave up: coc_check_waits() reports it to the host as
 * COC_ERR_TIMEOUT.  A wait can only give up when the work it waits for
 * cannot run: the one-launch all-gather matmul that copies the gathered rows
 * itself has workgroups waiting for rows other workgroups of the same launch
 * copy, so it needs all its workgroups (one per compute unit) resident at
 * once; a kernel of another process (or of another library) that holds
 * compute units for longer than the bound can starve it.  Calls of this
 * library on one device are chained so that they cannot starve each other.
 * Two environment variables, read at each call, exist to test that path:
 * COC_SPIN_LIMIT=n (polls before giving up) and COC_TEST_UNREACHABLE_WAIT=1
 * (the calls made meanwhile wait for counts that never arrive; the library's
 * own counter bookkeeping stays exact, so later calls are unaffected).
 *
 * Matmul tiles.  The kernel and tile a call runs never change its result
 * bits.  A bf16 / fp16 matmul with transposed weights (the *_trans_w entry
 * points) whose launch shares no compute unit with another kernel (nothing
 * waits beside it; the all-gather forms that copy their rows inside the
 * launch qualify) and fills the device with 256 x 256 tiles, k % 64 == 0,
 * uses a four-wave tile; every other launch the eight-wave one.  COC_FOUR_WAVE=0, read at each call,
 * keeps the eight-wave tile everywhere (for comparisons).
 */
#ifndef COC_H
#define COC_H

#include <stddef.h>
#include <stdint.h>

/* hipStream_t.  A host compiler other than hipcc needs -D__HIP_PLATFORM_AMD__
 * and the ROCm include directory for this header. */
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define COC_MAX_WORLD 8
#define COC_MAX_SPLIT 8

typedef enum coc_dtype {
    COC_F32 = 0,   /* IEEE binary32 */
    COC_F16 = 1,   /* IEEE binary16 */
    COC_BF16 = 2   /* bfloat16 */
} coc_dtype;

typedef enum coc_quant_mode {
    COC_PER_TENSOR = 0,   /* one scale                          */
    COC_PER_CHANNEL = 1,  /* one scale per output column n      */
    COC_PER_GROUP = 2     /* one scale per (k / group, n)       */
} coc_quant_mode;

typedef enum coc_status {
    COC_OK = 0,
    COC_ERR_NULL = 1,       /* a required pointer is NULL                      */
    COC_ERR_SPLIT = 2,      /* split not in {1, 2, 4, 8}                       */
    COC_ERR_SHAPE = 3,      /* sizes inconsistent / not divisible / too large  */
    COC_ERR_WORLD = 4,      /* world or rank out of range                      */
    COC_ERR_DTYPE = 5,      /* dtype or quant mode not supported               */
    COC_ERR_ALIGN = 6,      /* a device pointer is not 16-byte aligned         */
    COC_ERR_WORKSPACE = 7,  /* workspace missing or too small                  */
    COC_ERR_HIP = 8,        /* the HIP runtime reported an error               */
    COC_ERR_ALIAS = 9,      /* an output overlaps an input or another output   */
    COC_ERR_CAPTURE = 10,   /* not possible while the stream is captured        */
    COC_ERR_TIMEOUT = 11    /* a hand-over wait gave up (coc_check_waits)       */
} coc_status;

typedef enum coc_op {
    COC_OP_MATMUL_ALL_REDUCE = 0,
    COC_OP_MATMUL_REDUCE_SCATTER = 1,
    COC_OP_ALLGATHER_MATMUL = 2,
    COC_OP_ALLGATHER_MATMUL_V2 = 3,
    COC_OP_MATMUL_ALL_REDUCE_W8A16 = 4
} coc_op;

/*
 * MATMUL_ALL_REDUCE (CoC guide, "Approach", fused-operator list: compute
 * first, then communicate; with its deterministic variant).  The RowParallel
 * forward without sequence parallelism.
 *
 *   partial_out = round_dt(X @ W)                       (m x n, this rank's send buffer)
 *   y           = round_dt(sum_r P_r),  P_rank = partial_out,
 *                 P_r = peer_bufs[r] (m x n) for r != rank
 *
 * x: m x k, w: k x n, y: m x n, partial_out: m x n, all of dtype `dt`.
 * The left matrix is split into `split` contiguous row blocks; chunk i's
 * matmul overlaps the reduction of chunk i-1.  Requires m % split == 0.
 * `ws` is unused (may be NULL, ws_bytes 0).
 */
coc_status coc_matmul_all_reduce(const void* x, const void* w, void* y, void* partial_out,
                                 const void* const* peer_bufs, int32_t world, int32_t rank,
                                 int64_t m, int64_t n, int64_t k, coc_dtype dt,
                                 int32_t split, int32_t deterministic,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * MATMUL_REDUCE_SCATTER (CoC guide, "Approach", fused-operator list: compute
 * first, then communicate; with its deterministic variant).  The RowParallel
 * forward with sequence parallelism: rank r keeps rows
 * [r*m/world, (r+1)*m/world) of the reduced product.
 *
 *   partial_out = round_dt(X @ W)                                  (m x n)
 *   y[j, :]     = round_dt(sum_r P_r[rank*m/world + j, :]),  j < m/world
 *
 * x: m x k, w: k x n, partial_out: m x n, y: (m/world) x n, peer_bufs[r]:
 * full m x n partials of which only this rank's row slice is read.  Chunk i
 * holds the i-th 1/split of every rank's row slice, so every chunk carries
 * reduction work for this rank.  Requires m % world == 0 and
 * (m/world) % split == 0.  `ws` is unused.
 */
coc_status coc_matmul_reduce_scatter(const void* x, const void* w, void* y, void* partial_out,
                                     const void* const* peer_bufs, int32_t world, int32_t rank,
                                     int64_t m, int64_t n, int64_t k, coc_dtype dt,
                                     int32_t split, int32_t deterministic,
                                     void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ALL_GATHER_MATMUL and ALL_GATHER_MATMUL_V2 (CoC guide, "Approach",
 * fused-operator list: communicate first, then compute; V2 also hands back
 * the all-gathered intermediate).  The ColumnParallel forward with sequence
 * parallelism.
 *
 *   G = [S_0; S_1; ...; S_{world-1}]   (m x k, S_rank = x_shard, S_r = peer_bufs[r])
 *   y = round_dt(G @ W)                 (m x n)
 *
 * x_shard and peer_bufs[r]: (m/world) x k shards; w: k x n; y: m x n.
 * gathered_out == NULL selects ALL_GATHER_MATMUL (G is staged in `ws`, which
 * must hold coc_workspace_bytes(COC_OP_ALLGATHER_MATMUL, ...) bytes; its
 * contents afterwards are unspecified: the matmul may read the own shard's
 * rows from x_shard and leave them out of `ws`);
 * gathered_out != NULL selects ALL_GATHER_MATMUL_V2 and receives G (m x k,
 * bit-exact copy of the shards; `ws` unused).  The gather of chunk i+1
 * overlaps the matmul of chunk i; the pipeline starts with the chunk that
 * holds this rank's own shard.  Requires m % world == 0 and m % split == 0.
 * `deterministic` is accepted; the op is deterministic in either mode.
 */
coc_status coc_allgather_matmul(const void* x_shard, const void* const* peer_bufs, const void* w,
                                void* y, void* gathered_out, int32_t world, int32_t rank,
                                int64_t m, int64_t n, int64_t k, coc_dtype dt,
                                int32_t split, int32_t deterministic,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The same three ops with the weights given transposed (the backward pass of
 * the pair; CoC guide, "Approach": the fused operators come in forward /
 * backward pairs): `w` holds n rows of k elements, the forward layer's
 * k x n weight as stored, and the matmul is round_dt(X @ w^T).  Everything
 * else (arguments, layout, errors, pipeline) is as in the plain entry
 * point.  The RS-layer's input gradient is the all-gather form, AG(dY) @
 * W^T; the AG-layer's is the reduce-scatter form, RS(dY @ W^T).  bf16 / fp16
 * only (COC_ERR_DTYPE otherwise) and k % 32 == 0 (COC_ERR_SHAPE otherwise).
 */
coc_status coc_matmul_all_reduce_trans_w(const void* x, const void* w, void* y, void* partial_out,
                                         const void* const* peer_bufs, int32_t world, int32_t rank,
                                         int64_t m, int64_t n, int64_t k, coc_dtype dt,
                                         int32_t split, int32_t deterministic,
                                         void* ws, size_t ws_bytes, hipStream_t stream);
coc_status coc_matmul_reduce_scatter_trans_w(const void* x, const void* w, void* y, void* partial_out,
                                             const void* const* peer_bufs, int32_t world, int32_t rank,
                                             int64_t m, int64_t n, int64_t k, coc_dtype dt,
                                             int32_t split, int32_t deterministic,
                                             void* ws, size_t ws_bytes, hipStream_t stream);
coc_status coc_allgather_matmul_trans_w(const void* x_shard, const void* const* peer_bufs, const void* w,
                                        void* y, void* gathered_out, int32_t world, int32_t rank,
                                        int64_t m, int64_t n, int64_t k, coc_dtype dt,
                                        int32_t split, int32_t deterministic,
                                        void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Allocation-free ALL_GATHER_MATMUL, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the plain ALL_GATHER_MATMUL above (same arguments,
 * same result bits) with the gathered matrix G and the pipeline's hand-over
 * counters held in a static device array of the library instead of a caller
 * workspace and the library's per-stream allocation.  The call allocates
 * nothing and creates no stream or event: all its work goes to `stream`.
 *
 * Limit: m * k * element size <= 64 MiB (the LLaMA2-70B TP8 gather, 4096 x
 * 8192 bf16, is exactly that); larger problems return COC_ERR_WORKSPACE.
 * The array (64 MiB + 32 KiB) is held on every GPU the library runs on until
 * the process ends.  Every call on one GPU shares that GPU's array, so calls
 * that overlap on one GPU (from different streams or threads, or while
 * another such call's work is still running on another stream) race and
 * must be ordered by the caller; calls on one stream are ordered by it.
 * Its waits report through coc_check_waits() like the other calls'.
 */
coc_status coc_allgather_matmul_noalloc(const void* x_shard, const void* const* peer_bufs, const void* w,
                                        void* y, int32_t world, int32_t rank,
                                        int64_t m, int64_t n, int64_t k, coc_dtype dt,
                                        int32_t split, int32_t deterministic, hipStream_t stream);

/*
 * Weight gradient of the sequence-parallel pair (CoC guide, "Approach": the
 * fused operators come in forward / backward pairs, and V2 hands back the
 * all-gathered G so that the backward pass can reuse it):
 *
 *   dw = round_dt(G^T @ dY)        (k x n)
 *
 * g: m x k (e.g. the gathered_out of ALL_GATHER_MATMUL_V2), dy: m x n,
 * dw: k x n, all bf16 or fp16; accumulation in binary32 over m in
 * increasing order.  Requires m > 0, m % 32 == 0, n and k multiples of 8,
 * 16-byte aligned pointers, dw not overlapping g or dy.  A plain local
 * matmul: no collective.
 */
coc_status coc_weight_grad(const void* g, const void* dy, void* dw, int64_t m, int64_t n, int64_t k,
                           coc_dtype dt, hipStream_t stream);

/*
 * MoE expert all-to-all + grouped matmul, one expert-parallel rank's share
 * (Ampipe page, "Problem analysis": an all-to-all before and one after the
 * expert MLP exchange tokens between the ranks of the expert-parallel group;
 * "Solution": the input is cut along the sequence into independent pieces
 * whose communication and compute are pipelined; the Overlap blog's EP MC2:
 * the all-to-all fused with the experts' grouped matmul into one pipeline).
 *
 * Rows.  counts (HOST array, split x world x experts int64, read during the
 * call only): in sequence piece p, source rank r routes counts[p][r][e] rows
 * to this rank's local expert e.  A source's rows for this rank are ordered
 * piece-major, then by local expert, then in the source's order.  The
 * received matrix R (total x k, total = the sum of counts) orders its rows
 * piece-major, then by local expert, then by source rank, then in the
 * source's order: every (piece, expert) group is one contiguous block.  w
 * holds the local experts' weights, experts x k x n (expert e at offset
 * e * k * n).
 *
 *   coc_alltoall_grouped_matmul (dispatch, then the experts' first matmul):
 *     R = the sources' rows in the received order (bit copy), into recv_out;
 *     y[j] = round_dt(R[j] @ W_e(j))     (total x n), e(j) the row's expert.
 *     x_own: this rank's own rows for itself (source `rank`); peer_bufs[r]:
 *     source r's rows (HOST array of `world` device pointers, entry `rank`
 *     ignored; an entry of a source with no rows may be NULL).
 *
 *   coc_grouped_matmul_alltoall (the experts' second matmul, then combine):
 *     y_local[j] = round_dt(h[j] @ W_e(j))   (total x n, h in the received
 *     order), then every row goes back to its source at the position it had
 *     there: y_own receives this rank's own rows, peer_out[r] source r's
 *     (HOST array of device pointers, entry `rank` ignored; an entry of a
 *     source with no rows may be NULL).
 *
 * Pipeline: piece p's copy overlaps the matmul of other pieces (dispatch:
 * each (piece, expert) group's tiles wait for that piece's copy; combine: a
 * piece's rows go back once all its tiles are stored).  The dispatch
 * overlaps only when recv_out is 128-byte aligned and a row is a whole
 * number of 128-byte lines (k a multiple of 64); otherwise its copy runs
 * before its matmul.  `split` is the
 * number of sequence pieces (the Ampipe degree), 1..COC_MAX_SPLIT; it is the
 * first dimension of counts and fixes the row layout.  A row's result does
 * not depend on the pieces, the run or the other rows (binary32
 * accumulation over k in increasing order).
 *
 * Requirements: bf16 or fp16; world in [1, COC_MAX_WORLD], rank in [0,
 * world); experts in [1, 16]; k > 0 a multiple of 32; n > 0 a multiple of 8;
 * at most 16 non-empty (piece, expert) groups and 128 non-empty (piece,
 * expert, source) blocks; each matrix below 2^31 elements; 16-byte aligned
 * pointers; no output overlapping an input or another output.  A call with
 * no rows does nothing.
 */
coc_status coc_alltoall_grouped_matmul(const void* x_own, const void* const* peer_bufs, const int64_t* counts,
                                       const void* w, void* y, void* recv_out, int32_t world, int32_t rank,
                                       int32_t experts, int64_t n, int64_t k, coc_dtype dt, int32_t split,
                                       hipStream_t stream);
coc_status coc_grouped_matmul_alltoall(const void* h, const void* w, void* y_local, void* y_own,
                                       void* const* peer_out, const int64_t* counts, int32_t world, int32_t rank,
                                       int32_t experts, int64_t n, int64_t k, coc_dtype dt, int32_t split,
                                       hipStream_t stream);

/*
 * w8A16 pseudo-quantised MATMUL_ALL_REDUCE (CoC guide, "Approach", last item
 * of the fused-operator list: fp16, int8 weights, per-tensor / per-channel /
 * per-group scales).  Weight-only symmetric quantisation, no zero point:
 *
 *   W~[kk, j]   = q[kk, j] * s(kk, j)
 *       PER_TENSOR  s = scales[0]
 *       PER_CHANNEL s = scales[j]                    (n scales)
 *       PER_GROUP   s = scales[(kk / group_size) * n + j]   ((k/group_size) x n)
 *   partial_out = round_f16(X @ W~),  y = round_f16(sum_r P_r)  as in
 *   coc_matmul_all_reduce.
 *
 * x_f16: m x k fp16; w_q: k x n int8; scales_f16: fp16 as above; y_f16,
 * partial_out, peer_bufs[r]: m x n fp16.  PER_TENSOR and PER_CHANNEL: the
 * matmul multiplies X by q (each product exact in binary32), and the binary32
 * sums are scaled before rounding to fp16.  PER_GROUP: the weight is
 * dequantised to fp16 (q * s rounded to nearest even) inside the matmul main
 * loop.  Either way the result matches X @ W~ within fp16 accuracy, and is
 * exact when the scales are powers of two and the sums are exact.  PER_GROUP
 * requires group_size > 0, group_size % 8 == 0 and k % group_size == 0
 * (group_size is ignored otherwise).  Requires m % split == 0.  `ws` unused.
 */
coc_status coc_matmul_all_reduce_w8a16(const void* x_f16, const int8_t* w_q, const void* scales_f16,
                                       coc_quant_mode mode, int32_t group_size,
                                       void* y_f16, void* partial_out,
                                       const void* const* peer_bufs, int32_t world, int32_t rank,
                                       int64_t m, int64_t n, int64_t k,
                                       int32_t split, int32_t deterministic,
                                       void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes an op (a coc_op value) needs at these sizes (0 when it needs none).
 * dt is ignored for COC_OP_MATMUL_ALL_REDUCE_W8A16.  Returns 0 for invalid
 * arguments as well; the op call itself reports the error. */
size_t coc_workspace_bytes(int op, int64_t m, int64_t n, int64_t k, coc_dtype dt,
                           int32_t world, int32_t split);

/* Whether a hand-over wait of the library's work on `stream` gave up since
 * the last check (see "Hand-over waits" above).  Waits for the work enqueued
 * on `stream` so far, then returns COC_ERR_TIMEOUT if any wait of that work
 * (or of earlier work of the library on the same stream, or of the
 * allocation-free entry points on the current device) gave up, and clears
 * that record; COC_OK otherwise.  COC_ERR_CAPTURE while `stream` is being
 * captured, COC_ERR_HIP if a HIP call fails. */
coc_status coc_check_waits(hipStream_t stream);

/* Static name of a status code. */
const char* coc_status_string(coc_status s);

/* Description of the last failure on the calling host thread ("" if none).
 * The pointer stays valid until the next call on that thread. */
const char* coc_last_error(void);

/*
 * Row map of one pipeline chunk: the rows
 *   { base + b * stride + j : 0 <= b < nblk, 0 <= j < rows_per_blk }
 * of the m-row left matrix (matmul rows) or of the gathered matrix.
 * `red_base` is the first row of the reduction / gather this chunk carries
 * (for reduce-scatter: the row of the partials; `out_base` is the matching
 * row of y), `red_rows` the number of rows it covers.
 */
typedef struct coc_chunk {
    int64_t base;
    int64_t stride;
    int64_t rows_per_blk;
    int32_t nblk;
    int32_t order;          /* position of this chunk in the pipeline */
    int64_t red_base;
    int64_t out_base;
    int64_t red_rows;
} coc_chunk;

/* Host-only plan introspection: validates (op, m, world, rank, split) like
 * the op calls do (shape rules only; no pointers) and writes up to
 * `max_chunks` chunk descriptors in pipeline order.  Returns the status; on
 * COC_OK *n_chunks is the chunk count.  Touches no GPU state. */
coc_status coc_plan(coc_op op, int64_t m, int32_t world, int32_t rank, int32_t split,
                    coc_chunk* chunks, int32_t max_chunks, int32_t* n_chunks);

/*
 * Kernel timing, for measurement.  While enabled (per process), every
 * matmul, reduce and gather launch of the library is bracketed by a pair of
 * HIP events recorded on the stream that launch goes to.
 * coc_profile_read() waits for the recorded events, adds up their elapsed
 * times per kernel class, fills the arrays (index 0 = matmul, 1 = reduce /
 * reduce-scatter, 2 = gather) and clears the record.  Returns COC_OK or
 * COC_ERR_HIP.  Not for use while another thread issues library calls.
 */
#define COC_KCLASS_GEMM 0
#define COC_KCLASS_REDUCE 1
#define COC_KCLASS_GATHER 2
#define COC_NUM_KCLASS 3
void coc_profile_enable(int32_t on);
coc_status coc_profile_read(double* total_ms, int64_t* launches, double* work_units);

/* Per-launch view of the same record: for each recorded launch, in issue
 * order, its kernel class, start and end in ms relative to the start of the
 * first recorded launch, and its algorithmic work.  Fills at most `max`
 * entries, sets *n to the number of records, and clears the record (like
 * coc_profile_read; use one or the other).  Overlapping intervals mean the
 * launches ran concurrently. */
coc_status coc_profile_records(int32_t* kclass, double* start_ms, double* end_ms, double* work_units,
                               int32_t max, int32_t* n);

/* Activity stamps, for measuring overlap.  coc_profile_stamps(buf, records)
 * hands the library a DEVICE buffer of `records` three-word (64-bit)
 * records, owned by the caller and zeroed by it (NULL turns the stamps off).
 * Each later launch of the library's matmul, reduce and gather kernels takes
 * the next consecutive region of it (one record per workgroup and piece of
 * work); a launch that no longer fits takes none.  coc_profile_stamp_count()
 * returns how many records have been handed out since the buffer was set.
 * A record a workgroup wrote holds:
 *   word 0  1 + kind (0 matmul: first tile started to last tile's stores
 *           issued; 1 reduce: its wait done to its last store issued; 2
 *           gather: copy start to last store issued) | chunk << 8 | XCD << 16
 *   word 1  start, word 2  end: the 100 MHz real-time counter
 * Records left zero had no work.  Per process; not for use while another
 * thread issues library calls. */
void coc_profile_stamps(void* buf, int64_t records);
int64_t coc_profile_stamp_count(void);

/* Diagnostic for measurement (not part of the fused path): the rate the bf16
 * MFMA unit sustains with nothing else running.  Launches `workgroups`
 * workgroups of four waves on `stream`; each wave holds eight independent
 * 32 x 32 fp32 accumulators and, `iters` times, issues one
 * v_mfma_f32_32x32x16_bf16 into each, its operands kept in registers after
 * one load from `operands` (a DEVICE buffer of bf16 values, at least 128
 * bytes, 16-byte aligned; lane t takes vectors (8 t + i) mod count).  Writes
 * one float per thread to `out` (a DEVICE buffer of at least workgroups x 256
 * floats).  Work per launch: workgroups x 4 x iters x 8 x 32768 flops.
 * Random operand values make the arrays toggle as a matmul of random data
 * does; one repeated value barely toggles them, so timing both shows what the
 * operand data alone does to the clock the chip holds.  Errors: NULL
 * pointers (COC_ERR_NULL), misalignment (COC_ERR_ALIGN), sizes out of range
 * (COC_ERR_SHAPE); nothing is launched then. */
coc_status coc_diag_mfma_loop(const void* operands, size_t operand_bytes, float* out, size_t out_floats,
                              int32_t workgroups, int32_t iters, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* COC_H */
