// The C ABI of the fused ops: pointer validation, per-stream contexts and the
// two-stream pipeline that overlaps the matmul of one m-chunk with the
// collective of another.
//
// Pipeline (CoC guide, "Solution": compute and communication cut into finer
// sub-tasks that run as a pipeline; Overlap blog, "core idea": cut both small
// and let them hide each other):
//   compute-first ops (all-reduce, reduce-scatter, w8a16 all-reduce):
//       compute streams: gemm[0] gemm[1] gemm[2] ...  (alternating caller / 2nd stream)
//       comm stream:            reduce[0] reduce[1] ...  (reduce[i] waits on gemm[i])
//   communicate-first ops (all-gather matmul, V2):
//       comm stream:     gather[0] gather[1] gather[2] ...
//       compute streams:          gemm[0]   gemm[1]  ...  (gemm[i] waits on gather[i])
// The chunk matmuls do not depend on each other, so consecutive chunks go to
// two compute streams and the next chunk's workgroups fill the compute units
// the previous chunk's last wave leaves idle.  The library streams are forked
// from and joined back into the caller's stream with events, so a call is
// ordered like a single kernel on that stream.  split == 1 is the serial
// baseline: everything on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "coc_internal.h"

// Chunk matmuls alternate between the caller's stream and a second compute
// stream (2), or all run on the caller's stream (1).
#ifndef COC_COMPUTE_STREAMS
#define COC_COMPUTE_STREAMS 2
#endif
// 1: the all-gather pipeline's copy runs inside its chunk-walking matmul
// launch (by the workgroups with one tile) where the launch allows it; 0: as
// a separate launch on the side stream.
#ifndef COC_FUSED_GATHER
#define COC_FUSED_GATHER 1
#endif
// 1: bf16 / fp16 pipelines with k a multiple of 32 run all chunk matmuls of an
// op in one chunk-walking launch (hand-over through device counters); 0: one
// launch per chunk on the two compute streams.
#ifndef COC_ONE_LAUNCH
#define COC_ONE_LAUNCH 1
#endif

namespace coc {
namespace {

// Testing hooks (see coc.h): COC_SPIN_LIMIT=n makes every hand-over wait give
// up after n polls instead of about 2 s; COC_TEST_UNREACHABLE_WAIT=1 puts the
// targets of the waits of the calls made meanwhile out of reach (the counter
// bookkeeping itself stays exact, so later calls are unaffected).  The
// waiting tiles and rows then come out NaN and every kernel still ends.
uint32_t spin_limit_override() {
    const char* v = getenv("COC_SPIN_LIMIT");
    const long n = v ? strtol(v, nullptr, 10) : 0;
    return n > 0 && n < (1L << 30) ? (uint32_t)n : 0u;
}
uint32_t target_offset() {
    const char* v = getenv("COC_TEST_UNREACHABLE_WAIT");
    return v && v[0] == '1' ? (1u << 30) : 0u;
}

coc_status hip_fail(hipError_t e, const char* what) {
    return fail(COC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define COC_HIP(expr)                                         \
    do {                                                      \
        hipError_t e_ = (expr);                               \
        if (e_ != hipSuccess) return hip_fail(e_, #expr);     \
    } while (0)

#define COC_TRY(expr)                       \
    do {                                    \
        coc_status s_ = (expr);             \
        if (s_ != COC_OK) return s_;        \
    } while (0)

// ------------------------------------------------------------------ contexts
// One side stream plus pipeline events per (device, caller stream).  Streams
// are created with the default priority and never destroyed (the process
// owns them until exit).
struct StreamCtx {
    hipStream_t side = nullptr;    // reduce / gather
    hipStream_t gemm2 = nullptr;   // second compute stream
    hipEvent_t ev[COC_MAX_SPLIT] = {};
    hipEvent_t fork = nullptr;
    hipEvent_t join = nullptr;
    hipEvent_t join2 = nullptr;
    // Chunk hand-over counters of the one-launch pipeline (device memory,
    // layout in coc_internal.h): tiles of chunk c stored, gather workgroups
    // of chunk c done.  They only grow; *_sent hold the values all work
    // enqueued so far brings them to.
    uint32_t* sync = nullptr;
    uint32_t done_sent[COC_MAX_SPLIT] = {};
    uint32_t ready_sent[COC_MAX_SPLIT] = {};
    hipEvent_t tail = nullptr;     // end of this stream's last counter-waiting call
    uint32_t* gave_up() const { return sync + kGaveUpLine * kSyncWords; }
};

std::mutex g_ctx_mu;
std::map<std::pair<int, hipStream_t>, StreamCtx*> g_ctx;

// Whether `s` is being captured into a graph.  The one-launch pipelines hand
// chunks over through device counters whose targets the host advances call by
// call; a replayed graph would repeat the captured targets, so captured calls
// take the per-chunk event pipelines instead.
coc_status capturing(hipStream_t s, bool* out) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    COC_HIP(hipStreamIsCapturing(s, &cs));
    *out = cs != hipStreamCaptureStatusNone;
    return COC_OK;
}

// One capture holds at most one call of the library.  A bench run that
// captured two ops into one graph ended in a host segmentation fault whose
// cause was not found (the two calls record the same context events and
// side-stream joins twice within one capture), so a second call while the
// same capture is open is refused.  Capture ids are unique per capture; the
// last few that took a call are remembered.
std::mutex g_cap_mu;
unsigned long long g_cap_ids[64] = {};
int g_cap_next = 0;

coc_status capture_once(hipStream_t s, bool* cap) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    unsigned long long id = 0;
    COC_HIP(hipStreamGetCaptureInfo(s, &cs, &id));
    *cap = cs != hipStreamCaptureStatusNone;
    if (cs == hipStreamCaptureStatusInvalidated)
        return fail(COC_ERR_CAPTURE, "the stream's capture has been invalidated");
    if (!*cap) return COC_OK;
    std::lock_guard<std::mutex> lk(g_cap_mu);
    for (unsigned long long v : g_cap_ids)
        if (v == id && id != 0)
            return fail(COC_ERR_CAPTURE, "this capture already holds a call of the library; one graph holds "
                                         "at most one (capture each op into a graph of its own)");
    g_cap_ids[g_cap_next] = id;
    g_cap_next = (g_cap_next + 1) % 64;
    return COC_OK;
}

// ------------------------------------------------------------------ scratch memory
// The allocation-free all-gather matmul (coc_allgather_matmul_noalloc) keeps
// what the plain one takes from the caller's workspace (the gathered matrix)
// and from the library's per-stream allocation (the hand-over counters) in
// `scratch`, a file-scope device array that every GPU the library runs on
// holds until the process ends.  Layout: the counter lines (kSyncLines lines
// of 128 bytes, the same layout as a stream context's) from offset 0, then
// the gathered matrix from kScratchGatherOffset (128-byte aligned, as the
// one-launch all-gather needs), at most kScratchGatherBytes.  In host code
// the array's name only stands for the symbol: its device address, one per
// GPU, comes from hipGetSymbolAddress on that GPU.
constexpr size_t kScratchGatherOffset = size_t(32) << 10;
constexpr size_t kScratchGatherBytes = size_t(64) << 20;
static_assert(size_t(kSyncLines) * kSyncWords * sizeof(uint32_t) <= kScratchGatherOffset,
              "the counter lines fit before the gathered matrix");

}  // namespace
}  // namespace coc

static __device__ __align__(256) uint8_t scratch[coc::kScratchGatherOffset + coc::kScratchGatherBytes];

namespace coc {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch[kMaxDevices] = {};   // the address of `scratch` on each device, once set up

// The address of `scratch` on the current device: looked up with that device
// current on its first use there, then kept.
coc_status scratch_base(uint8_t** out) {
    int dev = 0;
    COC_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(COC_ERR_HIP, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        COC_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (p == nullptr) return fail(COC_ERR_HIP, "hipGetSymbolAddress returned no address for the scratch array");
        g_scratch[dev] = (uint8_t*)p;
    }
    *out = g_scratch[dev];
    return COC_OK;
}

// The gave-up word of the scratch counters on device `dev`, or NULL while
// they have not been set up there.
uint32_t* static_gave_up(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    return g_scratch[dev] ? (uint32_t*)g_scratch[dev] + kGaveUpLine * kSyncWords : nullptr;
}

coc_status get_ctx(hipStream_t main, StreamCtx** out) {
    int dev = 0;
    COC_HIP(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lk(g_ctx_mu);
    auto key = std::make_pair(dev, main);
    auto it = g_ctx.find(key);
    if (it != g_ctx.end()) {
        *out = it->second;
        return COC_OK;
    }
    bool cap = false;
    COC_TRY(capturing(main, &cap));
    if (cap)
        return fail(COC_ERR_CAPTURE, "the first call on a stream sets up its side streams and counters (with a "
                                     "device synchronisation) and cannot be captured: call once on this stream "
                                     "before capturing it");
    StreamCtx* c = new StreamCtx;
    COC_HIP(hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking));
    COC_HIP(hipStreamCreateWithFlags(&c->gemm2, hipStreamNonBlocking));
    for (auto& e : c->ev) COC_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    COC_HIP(hipEventCreateWithFlags(&c->fork, hipEventDisableTiming));
    COC_HIP(hipEventCreateWithFlags(&c->join, hipEventDisableTiming));
    COC_HIP(hipEventCreateWithFlags(&c->join2, hipEventDisableTiming));
    COC_HIP(hipEventCreateWithFlags(&c->tail, hipEventDisableTiming));
    COC_HIP(hipMalloc(&c->sync, kSyncLines * kSyncWords * sizeof(uint32_t)));
    COC_HIP(hipMemset(c->sync, 0, kSyncLines * kSyncWords * sizeof(uint32_t)));
    COC_HIP(hipDeviceSynchronize());
    g_ctx[key] = c;
    *out = c;
    return COC_OK;
}

// ------------------------------------------------------------------ waiting calls
// The one-launch pipelines have workgroups that wait on counters other
// workgroups (or a launch beside them) bump, which only works while the
// waiting and the counting work are resident together.  Two such calls
// running at once from different streams could each hold part of the compute
// units while waiting on their own work that no longer fits; the bounded
// waits would then give up and leave NaN.  So, per device, these calls are
// chained: each waits on the caller's stream for the end of the previous one,
// whatever stream that came from (calls on one stream are ordered anyway).  A
// stream being captured into a graph takes no part in the chain.
struct WaitChain {
    std::mutex mu;
    hipEvent_t last = nullptr;       // tail event of the last chained call
    hipStream_t last_stream = nullptr;
};

std::mutex g_chain_mu;
std::map<int, WaitChain*> g_chain;

class ChainedCall {
  public:
    // Takes the device's chain (held until finish() or destruction) and makes
    // `main` wait for the previous chained call on another stream.
    coc_status begin(StreamCtx* c, hipStream_t main) {
        int dev = 0;
        COC_HIP(hipGetDevice(&dev));
        {
            std::lock_guard<std::mutex> lk(g_chain_mu);
            WaitChain*& w = g_chain[dev];
            if (w == nullptr) w = new WaitChain;
            chain_ = w;
        }
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        COC_HIP(hipStreamIsCapturing(main, &cs));
        if (cs != hipStreamCaptureStatusNone) {
            chain_ = nullptr;
            return COC_OK;
        }
        lock_ = std::unique_lock<std::mutex>(chain_->mu);
        if (chain_->last != nullptr && chain_->last_stream != main)
            COC_HIP(hipStreamWaitEvent(main, chain_->last, 0));
        ctx_ = c;
        main_ = main;
        return COC_OK;
    }
    // Marks the end of the call's work on `main` (after every join).
    coc_status finish() {
        if (chain_ == nullptr) return COC_OK;
        COC_HIP(hipEventRecord(ctx_->tail, main_));
        chain_->last = ctx_->tail;
        chain_->last_stream = main_;
        chain_ = nullptr;
        lock_ = std::unique_lock<std::mutex>();
        return COC_OK;
    }

  private:
    WaitChain* chain_ = nullptr;
    std::unique_lock<std::mutex> lock_;
    StreamCtx* ctx_ = nullptr;
    hipStream_t main_ = nullptr;
};

// ------------------------------------------------------------------ timing
struct ProfRec {
    hipEvent_t a, b;
    int cls;
    double work;
};
std::atomic<int> g_prof_on{0};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;

coc_status prof_event(hipEvent_t* e) {
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        if (!g_prof_pool.empty()) {
            *e = g_prof_pool.back();
            g_prof_pool.pop_back();
            return COC_OK;
        }
    }
    COC_HIP(hipEventCreate(e));
    return COC_OK;
}

// Launch through `fn` (returns a hipError_t value), bracketed by timing
// events on `s` when timing is enabled.  `work` is the launch's algorithmic
// flops (matmul) or bytes (reduce, gather).
template <class F>
coc_status launch(int cls, double work, hipStream_t s, F&& fn) {
    if (!g_prof_on.load(std::memory_order_relaxed)) {
        const int e = fn();
        if (e != hipSuccess) return hip_fail(hipError_t(e), "kernel launch");
        return COC_OK;
    }
    hipEvent_t a, b;
    COC_TRY(prof_event(&a));
    COC_TRY(prof_event(&b));
    COC_HIP(hipEventRecord(a, s));
    const int e = fn();
    if (e != hipSuccess) return hip_fail(hipError_t(e), "kernel launch");
    COC_HIP(hipEventRecord(b, s));
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_recs.push_back({a, b, cls, work});
    return COC_OK;
}

// ------------------------------------------------------------------ validation
struct Range {
    uintptr_t lo, hi;  // [lo, hi)
    const char* name;
};

bool overlaps(const Range& a, const Range& b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

Range mk(const void* p, int64_t bytes, const char* name) {
    const uintptr_t lo = (uintptr_t)p;
    return Range{lo, lo + (uintptr_t)(bytes > 0 ? bytes : 0), name};
}

coc_status check_ptr(const void* p, int64_t bytes, const char* name) {
    if (bytes <= 0) return COC_OK;
    if (!p) return fail(COC_ERR_NULL, "%s is NULL", name);
    if ((uintptr_t)p % 16 != 0) return fail(COC_ERR_ALIGN, "%s is not 16-byte aligned", name);
    return COC_OK;
}

coc_status check_alias(const std::vector<Range>& outs, const std::vector<Range>& ins) {
    for (size_t i = 0; i < outs.size(); ++i) {
        for (size_t j = i + 1; j < outs.size(); ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(COC_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
        for (const Range& r : ins)
            if (overlaps(outs[i], r)) return fail(COC_ERR_ALIAS, "%s overlaps %s", outs[i].name, r.name);
    }
    return COC_OK;
}

// Peer pointers: host array of `world` device pointers, entry `rank` ignored.
coc_status check_peers(const void* const* peers, const Plan& P, int64_t bytes, std::vector<Range>* ins) {
    if (P.world == 1 || bytes <= 0) return COC_OK;
    if (!peers) return fail(COC_ERR_NULL, "peer_bufs is NULL");
    static const char* names[COC_MAX_WORLD] = {"peer_bufs[0]", "peer_bufs[1]", "peer_bufs[2]",
                                               "peer_bufs[3]", "peer_bufs[4]", "peer_bufs[5]",
                                               "peer_bufs[6]", "peer_bufs[7]"};
    for (int r = 0; r < P.world; ++r) {
        if (r == P.rank) continue;
        COC_TRY(check_ptr(peers[r], bytes, names[r]));
        ins->push_back(mk(peers[r], bytes, names[r]));
    }
    return COC_OK;
}

// ------------------------------------------------------------------ pipelines
GemmLaunch gemm_for_chunk(const Plan& P, const GemmLaunch& g0, const coc_chunk& c) {
    GemmLaunch g = g0;
    g.base = c.base;
    g.stride = c.stride;
    g.rpb = c.rows_per_blk;
    g.nblk = c.nblk;
    g.concurrent = P.split == 1 ? 1 : COC_COMPUTE_STREAMS;
    return g;
}

double gemm_flops(const Plan& P, const coc_chunk& c) {
    return 2.0 * double(c.rows_per_blk) * double(c.nblk) * double(P.n) * double(P.k);
}

// One piece per chunk, A and output rows by the chunk's row map.
ChunksLaunch chunks_for(const Plan& P, const GemmLaunch& g0) {
    ChunksLaunch L{};
    L.kind = g0.kind;
    L.b = g0.b;
    L.c = g0.c;
    L.n = g0.n;
    L.k = g0.k;
    L.scales = g0.scales;
    L.qmode = g0.qmode;
    L.group = g0.group;
    L.trans_b = g0.trans_b;
    L.npieces = P.nchunks;
    for (int i = 0; i < P.nchunks; ++i) {
        L.a[i] = g0.a;
        L.ashift[i] = 0;
        L.base[i] = P.chunk[i].base;
        L.stride[i] = P.chunk[i].stride;
        L.rpb[i] = P.chunk[i].rows_per_blk;
        L.nblk[i] = P.chunk[i].nblk;
        L.wait[i] = -1;
        L.signal[i] = -1;
    }
    return L;
}

void add_piece(ChunksLaunch* L, const void* a, int64_t ashift, int64_t row0, int64_t rows, int32_t wait) {
    if (rows <= 0) return;
    const int i = L->npieces++;
    L->a[i] = a;
    L->ashift[i] = ashift;
    L->base[i] = row0;
    L->stride[i] = 0;
    L->rpb[i] = rows;
    L->nblk[i] = 1;
    L->wait[i] = wait;
    L->signal[i] = -1;
}

bool one_launch(const Plan& P, const GemmLaunch& g0) {
    return COC_ONE_LAUNCH != 0 && P.split > 1 && chunks_supported(g0);
}

// The one-launch all-gather reads gathered rows through the L2, which needs
// every chunk to start on a 128-byte line (see gemm_ring_chunks).
bool one_launch_gather(const Plan& P, const GemmLaunch& g0) {
    return one_launch(P, g0) && (uintptr_t)g0.a % 128 == 0 && (g0.k * (int64_t)elem_size(P.dt)) % 128 == 0;
}

double total_flops(const Plan& P) {
    double f = 0;
    for (int i = 0; i < P.nchunks; ++i) f += gemm_flops(P, P.chunk[i]);
    return f;
}

// Whether overlapping a compute-first op's reduction with its matmul can pay
// on one GPU.  The reduce beside the matmul shares the compute units' memory
// path and the power budget with it; measured on MI355X, that slows the
// matmul by about as much as a small reduction saves (LLaMA2-70B TP8
// reduce-scatter, 75 MB against a 240 GFLOP matmul: 217 us pipelined
// against 207 us serial), while a large one gains (BLOOM-176B all-reduce,
// 528 MB against 421 GFLOP: 406 against 417 us; the w8A16 all-reduce, 604 MB
// against 240 GFLOP: 293 against 315 us).  The pipeline is used when the
// reduction alone would take at least a sixth of the matmul's time (both
// estimated at measured rates: 5.5 TB/s, 1.2 PFLOP/s); otherwise the call
// runs the serial schedule, which gives the same bits.
constexpr double kReduceBytesPerS = 5.5e12, kMatmulFlopPerS = 1.2e15, kOverlapMinRatio = 1.0 / 6.0;

bool overlap_pays(const Plan& P) {
    const int64_t red_rows = P.op == COC_OP_MATMUL_REDUCE_SCATTER ? P.m / P.world : P.m;
    const double bytes = double(P.world + 1) * double(red_rows) * double(P.n) * double(elem_size(P.dt));
    const double flops = 2.0 * double(P.m) * double(P.n) * double(P.k);
    if (flops <= 0) return false;
    return (bytes / kReduceBytesPerS) >= kOverlapMinRatio * (flops / kMatmulFlopPerS);
}

// Chunks of a compute-first one-launch plan that reduce beside the matmul:
// those whose tiles all fall before the matmul's last round of workgroups
// (the reduce waits on their counters, at most one workgroup per CU).  The
// rest finish with the matmul; their rows (consecutive in every plan) reduce
// in one full-grid launch after it on the caller's stream.  tiles receives
// the per-chunk tile counts (chunks_tiles).
int early_chunks(const Plan& P, const ChunksLaunch& L, int32_t tiles[kMaxPieces + 1]) {
    chunks_tiles(L, tiles);
    const int64_t groups = tiles[kMaxPieces] > 0 ? tiles[kMaxPieces] : 1;
    int64_t total = 0;
    for (int i = 0; i < P.nchunks; ++i) total += tiles[i];
    const int64_t last_round = ((total - 1) / groups) * groups;   // first tile index of the last round
    int early = 0;
    for (int64_t cum = 0; early < P.nchunks - 1 && cum + tiles[early] <= last_round; ++early) cum += tiles[early];
    return early;
}

// One-launch pipeline, compute first: the matmul walks the chunks in order on
// the caller's stream and counts finished tiles per chunk; the reduce of each
// early chunk, on the side stream from the start, waits for that chunk's
// count, and the chunks of the matmul's last round reduce after it on the
// caller's stream.  The host
// enqueues the matmul before the reduces, so if both streams shared one
// hardware queue the matmul would simply finish first.
coc_status run_compute_first_chunks(const Plan& P, const GemmLaunch& g0, const ReduceLaunch& r0,
                                    hipStream_t main) {
    StreamCtx* c = nullptr;
    COC_TRY(get_ctx(main, &c));
    ChainedCall chain;
    COC_TRY(chain.begin(c, main));
    const size_t es = elem_size(P.dt);
    ChunksLaunch L = chunks_for(P, g0);
    int32_t tiles[kMaxPieces + 1];
    const int early = early_chunks(P, L, tiles);
    if (early > 0) {
        COC_HIP(hipEventRecord(c->fork, main));
        COC_HIP(hipStreamWaitEvent(c->side, c->fork, 0));
        for (int i = 0; i < early; ++i) L.signal[i] = i;   // only the chunks reduced beside the matmul
        L.done = c->sync;
    }
    int32_t launched[kMaxPieces + 1];
    COC_TRY(launch(KC_GEMM, total_flops(P), main, [&] { return launch_gemm_chunks(L, main, launched); }));
    if (early > 0) {
        ReduceChunksLaunch R{};
        R.r = r0;
        R.nchunks = early;
        R.done = c->sync;
        R.own = P.rank;
        R.narrow = chunks_reduce_narrow(L);   // fits beside the matmul's two waves per SIMD
        double bytes = 0;
        R.spin_limit = spin_limit_override();
        R.gave_up = c->gave_up();
        const uint32_t off = target_offset();
        for (int i = 0; i < early; ++i) {
            R.target[i] = (c->done_sent[i] += (uint32_t)tiles[i]) + off;
            R.src_row0[i] = P.chunk[i].red_base;
            R.dst_row0[i] = P.chunk[i].out_base;
            R.rows[i] = P.chunk[i].red_rows;
            bytes += double(r0.nsrc + 1) * double(R.rows[i]) * double(P.n) * double(es);
        }
        COC_TRY(launch(KC_REDUCE, bytes, c->side, [&] { return launch_reduce_chunks(R, c->side); }));
    }
    {
        ReduceLaunch r = r0;
        r.src_row0 = P.chunk[early].red_base;
        r.dst_row0 = P.chunk[early].out_base;
        r.wide = true;   // after the matmul on the caller's stream
        r.rows = 0;
        for (int i = early; i < P.nchunks; ++i) r.rows += P.chunk[i].red_rows;
        const double lb = double(r.nsrc + 1) * double(r.rows) * double(P.n) * double(es);
        COC_TRY(launch(KC_REDUCE, lb, main, [&] { return launch_reduce(r, main); }));
    }
    if (early > 0) {
        COC_HIP(hipEventRecord(c->join, c->side));
        COC_HIP(hipStreamWaitEvent(main, c->join, 0));
    }
    return chain.finish();
}

// One-launch pipeline, communicate first: the gathers of all chunks go to the
// side stream first, each workgroup counting itself done; the matmul then
// walks the chunks on the caller's stream.  It starts with this rank's own
// shard, read straight from x_shard (nothing to wait for), then each chunk's
// other rows from the gathered matrix once that chunk's gather is counted
// complete.
// The matmul launch of the one-launch all-gather pipeline: this rank's own
// shard first, read straight from x_shard, then each chunk's rows outside
// it from the gathered matrix, each piece waiting for its chunk's ready
// lines at `ready`.  grow0 / grows receive each chunk's gathered rows.
ChunksLaunch comm_first_launch(const Plan& P, const GemmLaunch& g0, const GatherLaunch& a0, uint32_t* ready,
                               int64_t* grow0, int64_t* grows) {
    const int64_t shard = P.m / P.world;
    const int64_t own0 = P.rank * shard, own1 = own0 + shard;
    ChunksLaunch L{};
    L.kind = g0.kind;
    L.b = g0.b;
    L.c = g0.c;
    L.n = g0.n;
    L.k = g0.k;
    L.ready = ready;
    L.order = 1;
    L.trans_b = g0.trans_b;
    add_piece(&L, a0.src[P.rank], -own0, own0, shard, -1);
    for (int i = 0; i < P.nchunks; ++i) {
        grow0[i] = P.chunk[i].red_base;
        grows[i] = P.chunk[i].red_rows;
        // the chunk's rows outside the own shard (AG chunks are contiguous)
        const int64_t r0 = P.chunk[i].base, r1 = r0 + P.chunk[i].rows_per_blk * P.chunk[i].nblk;
        add_piece(&L, g0.a, 0, r0, (r1 < own0 ? r1 : own0) - r0, i);
        add_piece(&L, g0.a, 0, r0 > own1 ? r0 : own1, r1 - (r0 > own1 ? r0 : own1), i);
    }
    L.gather_nchunks = P.nchunks;   // (the fused-gather plan depends on it)
    return L;
}

// The fused-gather fields of L for plan fp (the launch copies the rows
// itself); the ready targets are left to the caller.  The plain all-gather's
// tiles read the own shard's rows from the shard itself (the first piece of
// comm_first_launch), so its gathered matrix is a workspace whose own rows
// nothing reads: each chunk copies only its rows before and after the own
// shard.  V2 hands the gathered matrix back, so it copies every row.
void set_fused_gather(ChunksLaunch* L, const Plan& P, const GatherLaunch& a0, const FusedGatherPlan& fp,
                      const int64_t* grow0, const int64_t* grows) {
    L->gather_plan = fp;
    for (int r = 0; r < COC_MAX_WORLD; ++r) L->gather_src[r] = a0.src[r < a0.nsrc ? r : 0];
    L->gather_dst = a0.dst;
    L->gather_row_bytes = P.k * (int64_t)elem_size(P.dt);
    L->gather_shard_rows = P.m / P.world;
    const int64_t own0 = P.rank * (P.m / P.world), own1 = own0 + P.m / P.world;
    for (int i = 0; i < P.nchunks; ++i) {
        const int64_t r0 = grow0[i], r1 = grow0[i] + grows[i];
        if (P.op == COC_OP_ALLGATHER_MATMUL) {
            const int64_t a1 = r1 < own0 ? r1 : own0, b0 = r0 > own1 ? r0 : own1;
            L->gather_row0[i] = r0;
            L->gather_rows[i] = a1 > r0 ? a1 - r0 : 0;
            L->gather_row0b[i] = b0;
            L->gather_rowsb[i] = r1 > b0 ? r1 - b0 : 0;
        } else {
            L->gather_row0[i] = r0;
            L->gather_rows[i] = grows[i];
            L->gather_row0b[i] = r1;
            L->gather_rowsb[i] = 0;
        }
    }
}

coc_status run_comm_first_chunks(const Plan& P, const GemmLaunch& g0, const GatherLaunch& a0,
                                 hipStream_t main) {
    StreamCtx* c = nullptr;
    COC_TRY(get_ctx(main, &c));
    ChainedCall chain;
    COC_TRY(chain.begin(c, main));
    const size_t es = elem_size(P.dt);
    int64_t grow0[COC_MAX_SPLIT], grows[COC_MAX_SPLIT];
    ChunksLaunch L = comm_first_launch(P, g0, a0, c->sync + COC_MAX_SPLIT * kSyncWords, grow0, grows);
    double bytes = 0;
    for (int i = 0; i < P.nchunks; ++i) bytes += 2.0 * double(grows[i]) * double(P.k) * double(es);
    int32_t tiles[kMaxPieces + 1];
    L.gave_up = c->gave_up();
    const FusedGatherPlan fp = COC_FUSED_GATHER ? chunks_fused_gather(L) : FusedGatherPlan{};
    if (fp.gatherers > 0) {
        // the matmul launch copies the rows itself, chunk by chunk; the host's
        // running targets advance only once that launch is enqueued
        set_fused_gather(&L, P, a0, fp, grow0, grows);
        L.spin_limit = spin_limit_override();
        const uint32_t off = target_offset();
        uint32_t sent[COC_MAX_SPLIT];
        for (int i = 0; i < P.nchunks; ++i) {
            sent[i] = c->ready_sent[i] + (uint32_t)(i < fp.early ? fp.workgroups : fp.gatherers);
            L.ready_target[i] = sent[i] + off;
        }
        COC_TRY(launch(KC_GEMM, total_flops(P), main, [&] { return launch_gemm_chunks(L, main, tiles); }));
        for (int i = 0; i < P.nchunks; ++i) c->ready_sent[i] = sent[i];
        return chain.finish();
    }
    L.gather_nchunks = 0;
    COC_HIP(hipEventRecord(c->fork, main));
    COC_HIP(hipStreamWaitEvent(c->side, c->fork, 0));
    int32_t per_chunk = 0;
    COC_TRY(launch(KC_GATHER, bytes, c->side, [&] {
        return launch_gather_chunks(a0, P.nchunks, grow0, grows, c->sync + COC_MAX_SPLIT * kSyncWords, c->side,
                                    &per_chunk);
    }));
    // the gather is enqueued: its adds will happen whatever follows
    L.spin_limit = spin_limit_override();
    for (int i = 0; i < P.nchunks; ++i) L.ready_target[i] = (c->ready_sent[i] += (uint32_t)per_chunk) + target_offset();
    COC_TRY(launch(KC_GEMM, total_flops(P), main, [&] { return launch_gemm_chunks(L, main, tiles); }));
    COC_HIP(hipEventRecord(c->join, c->side));
    COC_HIP(hipStreamWaitEvent(main, c->join, 0));
    return chain.finish();
}

// Compute first, then reduce: all-reduce, reduce-scatter, w8a16 all-reduce.
coc_status run_compute_first(const Plan& P, const GemmLaunch& g0, const ReduceLaunch& r0,
                             hipStream_t main, bool cap) {
    const size_t es = elem_size(P.dt);
    auto gemm = [&](int i, hipStream_t s) {
        const GemmLaunch g = gemm_for_chunk(P, g0, P.chunk[i]);
        return launch(KC_GEMM, gemm_flops(P, P.chunk[i]), s, [&] { return launch_gemm(g, s); });
    };
    // alone: the serial form's reduce, after its matmul on the same stream
    auto reduce = [&](int i, hipStream_t s, bool alone) {
        ReduceLaunch r = r0;
        r.src_row0 = P.chunk[i].red_base;
        r.dst_row0 = P.chunk[i].out_base;
        r.rows = P.chunk[i].red_rows;
        r.wide = alone;
        const double bytes = double(r.nsrc + 1) * double(r.rows) * double(P.n) * double(es);
        return launch(KC_REDUCE, bytes, s, [&] { return launch_reduce(r, s); });
    };
    if (P.split == 1) {
        COC_TRY(gemm(0, main));
        return reduce(0, main, true);
    }
    if (one_launch(P, g0) && !cap) return run_compute_first_chunks(P, g0, r0, main);
    StreamCtx* c = nullptr;
    COC_TRY(get_ctx(main, &c));
    COC_HIP(hipEventRecord(c->fork, main));
    COC_HIP(hipStreamWaitEvent(c->gemm2, c->fork, 0));
    for (int i = 0; i < P.nchunks; ++i) {
        hipStream_t cs = (COC_COMPUTE_STREAMS == 2 && (i & 1)) ? c->gemm2 : main;
        COC_TRY(gemm(i, cs));
        COC_HIP(hipEventRecord(c->ev[i], cs));
        COC_HIP(hipStreamWaitEvent(c->side, c->ev[i], 0));
        COC_TRY(reduce(i, c->side, false));
    }
    COC_HIP(hipEventRecord(c->join2, c->gemm2));
    COC_HIP(hipStreamWaitEvent(main, c->join2, 0));
    COC_HIP(hipEventRecord(c->join, c->side));
    COC_HIP(hipStreamWaitEvent(main, c->join, 0));
    return COC_OK;
}

// Communicate first, then compute: all-gather matmul (and V2).
coc_status run_comm_first(const Plan& P, const GemmLaunch& g0, const GatherLaunch& a0,
                          hipStream_t main, bool cap) {
    const size_t es = elem_size(P.dt);
    auto gather = [&](int i, hipStream_t s) {
        GatherLaunch a = a0;
        a.row0 = P.chunk[i].red_base;
        a.rows = P.chunk[i].red_rows;
        const double bytes = 2.0 * double(a.rows) * double(P.k) * double(es);
        return launch(KC_GATHER, bytes, s, [&] { return launch_gather(a, s); });
    };
    auto gemm = [&](int i, hipStream_t s) {
        const GemmLaunch g = gemm_for_chunk(P, g0, P.chunk[i]);
        return launch(KC_GEMM, gemm_flops(P, P.chunk[i]), s, [&] { return launch_gemm(g, s); });
    };
    if (P.split == 1) {
        COC_TRY(gather(0, main));
        return gemm(0, main);
    }
    if (one_launch_gather(P, g0) && !cap) return run_comm_first_chunks(P, g0, a0, main);
    StreamCtx* c = nullptr;
    COC_TRY(get_ctx(main, &c));
    COC_HIP(hipEventRecord(c->fork, main));
    COC_HIP(hipStreamWaitEvent(c->side, c->fork, 0));
    COC_HIP(hipStreamWaitEvent(c->gemm2, c->fork, 0));
    for (int i = 0; i < P.nchunks; ++i) {
        hipStream_t cs = (COC_COMPUTE_STREAMS == 2 && (i & 1)) ? c->gemm2 : main;
        COC_TRY(gather(i, c->side));
        COC_HIP(hipEventRecord(c->ev[i], c->side));
        COC_HIP(hipStreamWaitEvent(cs, c->ev[i], 0));
        COC_TRY(gemm(i, cs));
    }
    // main has waited for the gather of every chunk it ran; gemm2 holds the rest
    COC_HIP(hipEventRecord(c->join2, c->gemm2));
    COC_HIP(hipStreamWaitEvent(main, c->join2, 0));
    COC_HIP(hipEventRecord(c->join, c->side));
    COC_HIP(hipStreamWaitEvent(main, c->join, 0));
    return COC_OK;
}

GemmKind kind_of(coc_dtype dt) {
    return dt == COC_F32 ? GK_F32 : (dt == COC_F16 ? GK_F16 : GK_BF16);
}

// Shared body of the all-reduce / reduce-scatter / w8a16 entry points.
// Weights given transposed (w holds n rows of k elements, the forward
// layer's k x n weight read as its transpose): bf16 / fp16 and k a multiple
// of 32 (the matmul then always runs through the ring kernel).
coc_status check_trans_w(int32_t trans_w, coc_dtype dt, int64_t k) {
    if (!trans_w) return COC_OK;
    if (dt != COC_BF16 && dt != COC_F16) return fail(COC_ERR_DTYPE, "transposed weights need bf16 or fp16");
    if (k % 32 != 0) return fail(COC_ERR_SHAPE, "transposed weights need k %% 32 == 0 (k=%lld)", (long long)k);
    return COC_OK;
}

coc_status compute_first_op(coc_op op, const void* x, const void* w, const void* scales,
                            int32_t qmode, int32_t group, void* y, void* partial,
                            const void* const* peers, int32_t world, int32_t rank, int64_t m,
                            int64_t n, int64_t k, coc_dtype dt, int32_t split, int32_t det,
                            int32_t trans_w, hipStream_t stream) {
    clear_error();
    Plan P;
    COC_TRY(make_plan(op, m, n, k, dt, world, rank, split, det, &P));
    COC_TRY(check_trans_w(trans_w, P.dt, k));
    const bool w8 = op == COC_OP_MATMUL_ALL_REDUCE_W8A16;
    const int64_t es = (int64_t)elem_size(P.dt);
    const int64_t y_rows = op == COC_OP_MATMUL_REDUCE_SCATTER ? m / world : m;
    if (w8) {
        if (qmode != COC_PER_TENSOR && qmode != COC_PER_CHANNEL && qmode != COC_PER_GROUP)
            return fail(COC_ERR_DTYPE, "unknown quant mode %d", qmode);
        if (qmode == COC_PER_GROUP && (group <= 0 || group % 8 != 0 || k % group != 0))
            return fail(COC_ERR_SHAPE, "per-group needs group_size > 0, group_size %% 8 == 0 and "
                                       "k %% group_size == 0 (group_size=%d k=%lld)",
                        group, (long long)k);
    }
    if (m == 0 || n == 0) return COC_OK;  // no output elements

    std::vector<Range> ins, outs;
    COC_TRY(check_ptr(x, m * k * es, "x"));
    COC_TRY(check_ptr(w, k * n * (w8 ? 1 : es), "w"));
    COC_TRY(check_ptr(y, y_rows * n * es, "y"));
    COC_TRY(check_ptr(partial, m * n * es, "partial_out"));
    ins.push_back(mk(x, m * k * es, "x"));
    ins.push_back(mk(w, k * n * (w8 ? 1 : es), "w"));
    int64_t scale_elems = 0;
    if (w8 && k > 0) {
        scale_elems = qmode == COC_PER_TENSOR ? 1 : (qmode == COC_PER_CHANNEL ? n : (k / group) * n);
        COC_TRY(check_ptr(scales, scale_elems * 2, "scales"));
        ins.push_back(mk(scales, scale_elems * 2, "scales"));
    }
    COC_TRY(check_peers(peers, P, m * n * es, &ins));
    outs.push_back(mk(y, y_rows * n * es, "y"));
    outs.push_back(mk(partial, m * n * es, "partial_out"));
    COC_TRY(check_alias(outs, ins));

    GemmLaunch g0{};
    g0.kind = w8 ? GK_W8_F16 : kind_of(P.dt);
    g0.a = x;
    g0.b = w;
    g0.c = partial;
    g0.scales = scales;
    g0.qmode = qmode;
    g0.group = qmode == COC_PER_GROUP ? group : 0;
    g0.n = n;
    g0.k = k;
    g0.trans_b = trans_w;

    ReduceLaunch r0{};
    r0.dt = P.dt;
    r0.nsrc = world;
    for (int r = 0; r < world; ++r) r0.src[r] = (r == rank) ? partial : peers[r];
    r0.dst = y;
    r0.n = n;
    bool cap = false;
    COC_TRY(capture_once(stream, &cap));
    int32_t tiles[kMaxPieces + 1];
    if (P.split > 1 && !cap && one_launch(P, g0) &&
        (!overlap_pays(P) || early_chunks(P, chunks_for(P, g0), tiles) == 0)) {
        // A reduction too small to hide pays less than it costs beside the
        // matmul, and a matmul that finishes every chunk in its last round
        // (BLOOM-7B: one round) leaves nothing to reduce beside it: the serial
        // schedule (the split-1 plan of the same op; its two launches carry
        // less host work than the pipeline's).  The stream's pipeline context
        // is still set up here, so that a later capture of a split call on
        // this stream (which runs the per-chunk pipeline) finds it.
        StreamCtx* ctx = nullptr;
        COC_TRY(get_ctx(stream, &ctx));
        Plan S;
        COC_TRY(make_plan(op, m, n, k, dt, world, rank, 1, det, &S));
        return run_compute_first(S, g0, r0, stream, cap);
    }
    return run_compute_first(P, g0, r0, stream, cap);
}

// ------------------------------------------------------------------ expert all-to-all
// Rows of the MoE expert all-to-all + grouped matmul pair (Ampipe page,
// "Problem analysis" and "Solution"; the Overlap blog's EP MC2): in sequence
// piece p, source rank r routes counts[p][r][e] rows to local expert e.  A
// source's rows are ordered piece, expert; the received matrix piece, expert,
// source, so each (piece, expert) group is one contiguous block.  Pieces are
// the pipeline's chunks; each group is one piece of the chunk-walking matmul.
struct MoePlan {
    int32_t world, rank, experts, split;
    int64_t n, k, total;
    coc_dtype dt;
    int64_t src_rows[COC_MAX_WORLD];
    int64_t chunk_row0[COC_MAX_SPLIT], chunk_rows[COC_MAX_SPLIT];
    int32_t ngroups;
    int64_t group_row0[kMaxPieces], group_rows[kMaxPieces];
    int32_t group_expert[kMaxPieces], group_chunk[kMaxPieces];
    int32_t seg0[COC_MAX_SPLIT + 1];
    A2ASegment seg[kMaxA2ASegs];
};

coc_status make_moe_plan(const int64_t* counts, int32_t world, int32_t rank, int32_t experts, int64_t n,
                         int64_t k, coc_dtype dt, int32_t split, MoePlan* M) {
    if (world < 1 || world > COC_MAX_WORLD || rank < 0 || rank >= world)
        return fail(COC_ERR_WORLD, "world=%d rank=%d out of range", world, rank);
    if (split < 1 || split > COC_MAX_SPLIT)
        return fail(COC_ERR_SPLIT, "expert all-to-all: pieces (split) must be in [1, %d], got %d", COC_MAX_SPLIT,
                    split);
    if (experts < 1 || experts > kMaxPieces)
        return fail(COC_ERR_SHAPE, "local experts must be in [1, %d], got %d", kMaxPieces, experts);
    if (dt != COC_BF16 && dt != COC_F16) return fail(COC_ERR_DTYPE, "expert all-to-all: bf16 or fp16 only");
    if (n <= 0 || k <= 0 || n % 8 != 0 || k % 32 != 0)
        return fail(COC_ERR_SHAPE, "expert all-to-all needs n > 0, n %% 8 == 0, k > 0, k %% 32 == 0 (n=%lld k=%lld)",
                    (long long)n, (long long)k);
    if (!counts) return fail(COC_ERR_NULL, "counts is NULL");
    const int64_t lim = int64_t(1) << 31;
    if (n >= lim || k >= lim || k * n >= lim) return fail(COC_ERR_SHAPE, "an expert weight has 2^31 or more elements");
    MoePlan& P = *M;
    P = MoePlan{};
    P.world = world;
    P.rank = rank;
    P.experts = experts;
    P.split = split;
    P.n = n;
    P.k = k;
    P.dt = dt;
    const int64_t width = n > k ? n : k;
    auto cnt = [&](int p, int r, int e) { return counts[((int64_t)p * world + r) * experts + e]; };
    // each source's first row of (piece p, expert e)
    std::vector<int64_t> src_off((size_t)split * world * experts);
    for (int r = 0; r < world; ++r) {
        int64_t row = 0;
        for (int p = 0; p < split; ++p)
            for (int e = 0; e < experts; ++e) {
                const int64_t c = cnt(p, r, e);
                if (c < 0 || c >= lim) return fail(COC_ERR_SHAPE, "counts[%d][%d][%d] = %lld", p, r, e, (long long)c);
                src_off[((size_t)p * world + r) * experts + e] = row;
                row += c;
                if (row * width >= lim) return fail(COC_ERR_SHAPE, "source %d's rows have 2^31 or more elements", r);
            }
        P.src_rows[r] = row;
    }
    int64_t row = 0;
    int nseg = 0;
    for (int p = 0; p < split; ++p) {
        P.chunk_row0[p] = row;
        P.seg0[p] = nseg;
        for (int e = 0; e < experts; ++e) {
            const int64_t g0 = row;
            for (int r = 0; r < world; ++r) {
                const int64_t c = cnt(p, r, e);
                if (c == 0) continue;
                if (nseg == kMaxA2ASegs)
                    return fail(COC_ERR_SHAPE, "more than %d non-empty (piece, expert, source) blocks", kMaxA2ASegs);
                P.seg[nseg++] = A2ASegment{(int32_t)row, (int32_t)src_off[((size_t)p * world + r) * experts + e],
                                           (int32_t)c, r};
                row += c;
                if (row * width >= lim) return fail(COC_ERR_SHAPE, "the received rows have 2^31 or more elements");
            }
            if (row > g0) {
                if (P.ngroups == kMaxPieces)
                    return fail(COC_ERR_SHAPE, "more than %d non-empty (piece, expert) groups", kMaxPieces);
                const int i = P.ngroups++;
                P.group_row0[i] = g0;
                P.group_rows[i] = row - g0;
                P.group_expert[i] = e;
                P.group_chunk[i] = p;
            }
        }
        P.chunk_rows[p] = row - P.chunk_row0[p];
    }
    P.seg0[split] = nseg;
    P.total = row;
    return COC_OK;
}

double moe_flops(const MoePlan& M) { return 2.0 * double(M.total) * double(M.n) * double(M.k); }

// The grouped matmul: one piece per (piece, expert) group, A = `a` (the
// received-order rows), weights w + e * k * n, output rows as the input's.
ChunksLaunch moe_matmul(const MoePlan& M, const void* a, const void* w, void* y) {
    ChunksLaunch L{};
    L.kind = kind_of(M.dt);
    L.b = w;
    L.c = y;
    L.n = M.n;
    L.k = M.k;
    const size_t wbytes = (size_t)M.k * (size_t)M.n * elem_size(M.dt);
    for (int i = 0; i < M.ngroups; ++i) {
        add_piece(&L, a, 0, M.group_row0[i], M.group_rows[i], -1);
        L.bp[L.npieces - 1] = (const uint8_t*)w + (size_t)M.group_expert[i] * wbytes;
    }
    return L;
}

A2ALaunch moe_a2a(const MoePlan& M, void* local, int64_t row_bytes) {
    A2ALaunch a{};
    a.local = local;
    a.row_bytes = row_bytes;
    a.nchunks = M.split;
    for (int p = 0; p < M.split; ++p) {
        a.row0[p] = M.chunk_row0[p];
        a.rows[p] = M.chunk_rows[p];
    }
    for (int p = 0; p <= M.split; ++p) a.seg0[p] = M.seg0[p];
    for (int i = 0; i < M.seg0[M.split]; ++i) a.seg[i] = M.seg[i];
    return a;
}

// Communicate first: the dispatch copy of every piece on the side stream,
// each workgroup counting itself done per piece; the grouped matmul walks the
// (piece, expert) groups on the caller's stream, each group waiting for its
// piece's count.  The matmul reads the received rows through the L2, which
// is safe only if no 128-byte line holds rows of two pieces (a tile of one
// piece would cache the other's line before its copy): rows of whole lines on
// a 128-byte aligned matrix.  Otherwise the copy runs first on the caller's
// stream and the matmul after it (no overlap).
coc_status run_moe_dispatch(const MoePlan& M, const void* const* src, const void* w, void* y, void* recv,
                            hipStream_t main) {
    bool cap = false;
    COC_TRY(capturing(main, &cap));
    if (cap)
        return fail(COC_ERR_CAPTURE, "the expert all-to-all hands sequence pieces over through device counters "
                                     "and cannot be captured into a graph");
    StreamCtx* c = nullptr;
    COC_TRY(get_ctx(main, &c));
    ChainedCall chain;
    COC_TRY(chain.begin(c, main));
    const size_t es = elem_size(M.dt);
    const bool overlap = (uintptr_t)recv % 128 == 0 && (M.k * (int64_t)es) % 128 == 0;
    A2ALaunch a = moe_a2a(M, recv, M.k * (int64_t)es);
    for (int r = 0; r < M.world; ++r) a.remote[r] = const_cast<void*>(src[r]);
    a.to_remote = 0;
    a.ready = c->sync + COC_MAX_SPLIT * kSyncWords;
    hipStream_t cs = overlap ? c->side : main;
    if (overlap) {
        COC_HIP(hipEventRecord(c->fork, main));
        COC_HIP(hipStreamWaitEvent(c->side, c->fork, 0));
    }
    int32_t per_chunk = 0;
    const double bytes = 2.0 * double(M.total) * double(M.k) * double(es);
    COC_TRY(launch(KC_GATHER, bytes, cs, [&] { return launch_a2a_chunks(a, cs, &per_chunk); }));
    ChunksLaunch L = moe_matmul(M, recv, w, y);
    for (int i = 0; i < L.npieces; ++i) L.wait[i] = overlap ? M.group_chunk[i] : -1;
    L.ready = overlap ? a.ready : nullptr;
    L.order = 1;
    L.spin_limit = spin_limit_override();
    L.gave_up = c->gave_up();
    const uint32_t off = target_offset();
    // the copy's adds happen either way: keep the running targets exact
    for (int p = 0; p < M.split; ++p) L.ready_target[p] = (c->ready_sent[p] += (uint32_t)per_chunk) + off;
    int32_t tiles[kMaxPieces + 1];
    COC_TRY(launch(KC_GEMM, moe_flops(M), main, [&] { return launch_gemm_chunks(L, main, tiles); }));
    if (overlap) {
        COC_HIP(hipEventRecord(c->join, c->side));
        COC_HIP(hipStreamWaitEvent(main, c->join, 0));
    }
    return chain.finish();
}

// Compute first: the grouped matmul walks the groups piece by piece on the
// caller's stream, counting each piece's finished tiles; the combine copy, on
// the side stream from the start, sends a piece's rows back once its count is
// complete.
coc_status run_moe_combine(const MoePlan& M, const void* h, const void* w, void* y_local, void* const* dst,
                           hipStream_t main) {
    bool cap = false;
    COC_TRY(capturing(main, &cap));
    if (cap)
        return fail(COC_ERR_CAPTURE, "the expert all-to-all hands sequence pieces over through device counters "
                                     "and cannot be captured into a graph");
    StreamCtx* c = nullptr;
    COC_TRY(get_ctx(main, &c));
    ChainedCall chain;
    COC_TRY(chain.begin(c, main));
    const size_t es = elem_size(M.dt);
    ChunksLaunch L = moe_matmul(M, h, w, y_local);
    for (int i = 0; i < L.npieces; ++i) L.signal[i] = M.group_chunk[i];
    L.done = c->sync;
    L.order = 0;
    int32_t tiles[kMaxPieces + 1];
    chunks_tiles(L, tiles);
    A2ALaunch a = moe_a2a(M, y_local, M.n * (int64_t)es);
    for (int r = 0; r < M.world; ++r) a.remote[r] = dst[r];
    a.to_remote = 1;
    a.done = c->sync;
    a.spin_limit = spin_limit_override();
    a.gave_up = c->gave_up();
    uint32_t per_piece[COC_MAX_SPLIT] = {};
    for (int i = 0; i < L.npieces; ++i) per_piece[M.group_chunk[i]] += (uint32_t)tiles[i];
    const uint32_t off = target_offset();
    COC_HIP(hipEventRecord(c->fork, main));
    COC_HIP(hipStreamWaitEvent(c->side, c->fork, 0));
    int32_t launched[kMaxPieces + 1];
    COC_TRY(launch(KC_GEMM, moe_flops(M), main, [&] { return launch_gemm_chunks(L, main, launched); }));
    // the matmul is enqueued: its adds will happen, so the running targets advance
    for (int p = 0; p < M.split; ++p) a.target[p] = (c->done_sent[p] += per_piece[p]) + off;
    int32_t unused = 0;
    const double bytes = 2.0 * double(M.total) * double(M.n) * double(es);
    COC_TRY(launch(KC_GATHER, bytes, c->side, [&] { return launch_a2a_chunks(a, c->side, &unused); }));
    COC_HIP(hipEventRecord(c->join, c->side));
    COC_HIP(hipStreamWaitEvent(main, c->join, 0));
    return chain.finish();
}

coc_status allgather_op(const void* x_shard, const void* const* peer_bufs, const void* w, void* y,
                        void* gathered_out, int32_t world, int32_t rank, int64_t m, int64_t n, int64_t k,
                        coc_dtype dt, int32_t split, int32_t deterministic, int32_t trans_w, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
    clear_error();
    const coc_op op = gathered_out ? COC_OP_ALLGATHER_MATMUL_V2 : COC_OP_ALLGATHER_MATMUL;
    Plan P;
    COC_TRY(make_plan(op, m, n, k, dt, world, rank, split, deterministic, &P));
    COC_TRY(check_trans_w(trans_w, P.dt, k));
    const int64_t es = (int64_t)elem_size(P.dt);
    const int64_t shard = m / world;
    if (m == 0 || (n == 0 && !gathered_out) || (n == 0 && k == 0)) return COC_OK;

    void* g = gathered_out;
    if (!g && m * k > 0) {
        const size_t need = workspace_bytes(P);
        if (!ws) return fail(COC_ERR_WORKSPACE, "ALL_GATHER_MATMUL needs a %zu-byte workspace", need);
        if (ws_bytes < need)
            return fail(COC_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
        if ((uintptr_t)ws % 16 != 0) return fail(COC_ERR_ALIGN, "ws is not 16-byte aligned");
        g = ws;
    }
    std::vector<Range> ins, outs;
    COC_TRY(check_ptr(x_shard, shard * k * es, "x_shard"));
    COC_TRY(check_ptr(w, k * n * es, "w"));
    COC_TRY(check_ptr(y, m * n * es, "y"));
    COC_TRY(check_ptr(gathered_out, gathered_out ? m * k * es : 0, "gathered_out"));
    ins.push_back(mk(x_shard, shard * k * es, "x_shard"));
    ins.push_back(mk(w, k * n * es, "w"));
    COC_TRY(check_peers(peer_bufs, P, shard * k * es, &ins));
    outs.push_back(mk(y, m * n * es, "y"));
    outs.push_back(mk(g, m * k * es, gathered_out ? "gathered_out" : "ws"));
    COC_TRY(check_alias(outs, ins));

    GatherLaunch a0{};
    a0.dt = P.dt;
    a0.nsrc = world;
    for (int r = 0; r < world; ++r) a0.src[r] = (r == rank) ? x_shard : peer_bufs[r];
    a0.shard_rows = shard;
    a0.dst = g;
    a0.k = k;

    GemmLaunch g0{};
    g0.kind = kind_of(P.dt);
    g0.a = g;
    g0.b = w;
    g0.c = y;
    g0.n = n;
    g0.k = k;
    g0.trans_b = trans_w;
    bool cap = false;
    COC_TRY(capture_once(stream, &cap));
    return run_comm_first(P, g0, a0, stream, cap);
}

// ALL_GATHER_MATMUL with the gathered matrix and the hand-over counters in
// `scratch`: no allocation, no library stream or event, everything on the
// caller's stream.  The counters are cleared by a kernel at the start of the
// call, so every wait target is absolute.
coc_status allgather_noalloc(const void* x_shard, const void* const* peer_bufs, const void* w, void* y,
                             int32_t world, int32_t rank, int64_t m, int64_t n, int64_t k, coc_dtype dt,
                             int32_t split, int32_t deterministic, hipStream_t stream) {
    clear_error();
    Plan P;
    COC_TRY(make_plan(COC_OP_ALLGATHER_MATMUL, m, n, k, dt, world, rank, split, deterministic, &P));
    const int64_t es = (int64_t)elem_size(P.dt);
    const int64_t shard = m / world;
    if (m == 0 || n == 0) return COC_OK;
    const size_t gbytes = size_t(m) * size_t(k) * size_t(es);
    if (gbytes > kScratchGatherBytes)
        return fail(COC_ERR_WORKSPACE, "the allocation-free all-gather matmul stages at most %zu bytes of "
                                       "gathered rows; m x k needs %zu",
                    kScratchGatherBytes, gbytes);
    std::vector<Range> ins, outs;
    COC_TRY(check_ptr(x_shard, shard * k * es, "x_shard"));
    COC_TRY(check_ptr(w, k * n * es, "w"));
    COC_TRY(check_ptr(y, m * n * es, "y"));
    ins.push_back(mk(x_shard, shard * k * es, "x_shard"));
    ins.push_back(mk(w, k * n * es, "w"));
    COC_TRY(check_peers(peer_bufs, P, shard * k * es, &ins));
    outs.push_back(mk(y, m * n * es, "y"));
    COC_TRY(check_alias(outs, ins));
    uint8_t* base = nullptr;
    COC_TRY(scratch_base(&base));
    bool cap = false;
    COC_TRY(capture_once(stream, &cap));
    uint32_t* sync = (uint32_t*)base;
    void* g = base + kScratchGatherOffset;

    GatherLaunch a0{};
    a0.dt = P.dt;
    a0.nsrc = world;
    for (int r = 0; r < world; ++r) a0.src[r] = (r == rank) ? x_shard : peer_bufs[r];
    a0.shard_rows = shard;
    a0.dst = g;
    a0.k = k;
    GemmLaunch g0{};
    g0.kind = kind_of(P.dt);
    g0.a = g;
    g0.b = w;
    g0.c = y;
    g0.n = n;
    g0.k = k;

    if (P.split > 1 && one_launch_gather(P, g0)) {
        // the counters start from zero (the gave-up line is kept for coc_check_waits)
        COC_HIP(hipError_t(launch_zero_words(sync, kGaveUpLine * kSyncWords, stream)));
        int64_t grow0[COC_MAX_SPLIT], grows[COC_MAX_SPLIT];
        ChunksLaunch L = comm_first_launch(P, g0, a0, sync + COC_MAX_SPLIT * kSyncWords, grow0, grows);
        L.gave_up = sync + kGaveUpLine * kSyncWords;
        L.spin_limit = spin_limit_override();
        const uint32_t off = target_offset();
        const FusedGatherPlan fp = COC_FUSED_GATHER ? chunks_fused_gather(L) : FusedGatherPlan{};
        if (fp.gatherers > 0) {
            set_fused_gather(&L, P, a0, fp, grow0, grows);
            for (int i = 0; i < P.nchunks; ++i)
                L.ready_target[i] = (uint32_t)(i < fp.early ? fp.workgroups : fp.gatherers) + off;
        } else {
            // the copy as its own launch ahead of the matmul on the same stream
            L.gather_nchunks = 0;
            int32_t per_chunk = 0;
            COC_HIP(hipError_t(launch_gather_chunks(a0, P.nchunks, grow0, grows, L.ready, stream, &per_chunk)));
            for (int i = 0; i < P.nchunks; ++i) L.ready_target[i] = (uint32_t)per_chunk + off;
        }
        int32_t tiles[kMaxPieces + 1];
        COC_HIP(hipError_t(launch_gemm_chunks(L, stream, tiles)));
        return COC_OK;
    }
    // every gathered row, then the matmul over them (the serial form)
    GatherLaunch a = a0;
    a.row0 = 0;
    a.rows = m;
    COC_HIP(hipError_t(launch_gather(a, stream)));
    GemmLaunch gg = g0;
    gg.base = 0;
    gg.stride = 0;
    gg.rpb = m;
    gg.nblk = 1;
    gg.concurrent = 1;
    COC_HIP(hipError_t(launch_gemm(gg, stream)));
    return COC_OK;
}


}  // namespace
}  // namespace coc

using namespace coc;

extern "C" {

coc_status coc_matmul_all_reduce(const void* x, const void* w, void* y, void* partial_out,
                                 const void* const* peer_bufs, int32_t world, int32_t rank,
                                 int64_t m, int64_t n, int64_t k, coc_dtype dt, int32_t split,
                                 int32_t deterministic, void* ws, size_t ws_bytes, hipStream_t stream) {
    (void)ws;
    (void)ws_bytes;
    return compute_first_op(COC_OP_MATMUL_ALL_REDUCE, x, w, nullptr, 0, 0, y, partial_out, peer_bufs,
                            world, rank, m, n, k, dt, split, deterministic, 0, stream);
}

coc_status coc_matmul_all_reduce_trans_w(const void* x, const void* w, void* y, void* partial_out,
                                         const void* const* peer_bufs, int32_t world, int32_t rank,
                                         int64_t m, int64_t n, int64_t k, coc_dtype dt, int32_t split,
                                         int32_t deterministic, void* ws, size_t ws_bytes,
                                         hipStream_t stream) {
    (void)ws;
    (void)ws_bytes;
    return compute_first_op(COC_OP_MATMUL_ALL_REDUCE, x, w, nullptr, 0, 0, y, partial_out, peer_bufs,
                            world, rank, m, n, k, dt, split, deterministic, 1, stream);
}

coc_status coc_matmul_reduce_scatter(const void* x, const void* w, void* y, void* partial_out,
                                     const void* const* peer_bufs, int32_t world, int32_t rank,
                                     int64_t m, int64_t n, int64_t k, coc_dtype dt, int32_t split,
                                     int32_t deterministic, void* ws, size_t ws_bytes, hipStream_t stream) {
    (void)ws;
    (void)ws_bytes;
    return compute_first_op(COC_OP_MATMUL_REDUCE_SCATTER, x, w, nullptr, 0, 0, y, partial_out,
                            peer_bufs, world, rank, m, n, k, dt, split, deterministic, 0, stream);
}

coc_status coc_matmul_reduce_scatter_trans_w(const void* x, const void* w, void* y, void* partial_out,
                                             const void* const* peer_bufs, int32_t world, int32_t rank,
                                             int64_t m, int64_t n, int64_t k, coc_dtype dt, int32_t split,
                                             int32_t deterministic, void* ws, size_t ws_bytes,
                                             hipStream_t stream) {
    (void)ws;
    (void)ws_bytes;
    return compute_first_op(COC_OP_MATMUL_REDUCE_SCATTER, x, w, nullptr, 0, 0, y, partial_out,
                            peer_bufs, world, rank, m, n, k, dt, split, deterministic, 1, stream);
}

coc_status coc_matmul_all_reduce_w8a16(const void* x_f16, const int8_t* w_q, const void* scales_f16,
                                       coc_quant_mode mode, int32_t group_size, void* y_f16,
                                       void* partial_out, const void* const* peer_bufs,
                                       int32_t world, int32_t rank, int64_t m, int64_t n, int64_t k,
                                       int32_t split, int32_t deterministic, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
    (void)ws;
    (void)ws_bytes;
    return compute_first_op(COC_OP_MATMUL_ALL_REDUCE_W8A16, x_f16, w_q, scales_f16, (int32_t)mode,
                            group_size, y_f16, partial_out, peer_bufs, world, rank, m, n, k, COC_F16,
                            split, deterministic, 0, stream);
}

coc_status coc_allgather_matmul(const void* x_shard, const void* const* peer_bufs, const void* w,
                                void* y, void* gathered_out, int32_t world, int32_t rank, int64_t m,
                                int64_t n, int64_t k, coc_dtype dt, int32_t split,
                                int32_t deterministic, void* ws, size_t ws_bytes, hipStream_t stream) {
    return allgather_op(x_shard, peer_bufs, w, y, gathered_out, world, rank, m, n, k, dt, split, deterministic,
                        0, ws, ws_bytes, stream);
}

coc_status coc_allgather_matmul_trans_w(const void* x_shard, const void* const* peer_bufs, const void* w,
                                        void* y, void* gathered_out, int32_t world, int32_t rank, int64_t m,
                                        int64_t n, int64_t k, coc_dtype dt, int32_t split,
                                        int32_t deterministic, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
    return allgather_op(x_shard, peer_bufs, w, y, gathered_out, world, rank, m, n, k, dt, split, deterministic,
                        1, ws, ws_bytes, stream);
}

coc_status coc_allgather_matmul_noalloc(const void* x_shard, const void* const* peer_bufs, const void* w,
                                        void* y, int32_t world, int32_t rank, int64_t m, int64_t n, int64_t k,
                                        coc_dtype dt, int32_t split, int32_t deterministic, hipStream_t stream) {
    return allgather_noalloc(x_shard, peer_bufs, w, y, world, rank, m, n, k, dt, split, deterministic, stream);
}

coc_status coc_weight_grad(const void* g, const void* dy, void* dw, int64_t m, int64_t n, int64_t k,
                           coc_dtype dt, hipStream_t stream) {
    clear_error();
    if (dt != COC_BF16 && dt != COC_F16) return fail(COC_ERR_DTYPE, "weight gradient: bf16 or fp16 only");
    if (m < 0 || n < 0 || k < 0) return fail(COC_ERR_SHAPE, "negative size");
    if (n % 8 != 0 || k % 8 != 0) return fail(COC_ERR_SHAPE, "n and k must be multiples of 8 (n=%lld k=%lld)",
                                              (long long)n, (long long)k);
    if (m <= 0 || m % 32 != 0) return fail(COC_ERR_SHAPE, "weight gradient needs m > 0, m %% 32 == 0 (m=%lld)",
                                          (long long)m);
    const int64_t lim = int64_t(1) << 31;
    if (m >= lim || n >= lim || k >= lim || m * k >= lim || m * n >= lim || k * n >= lim)
        return fail(COC_ERR_SHAPE, "a matrix has 2^31 or more elements");
    if (n == 0 || k == 0) return COC_OK;
    const int64_t es = 2;
    std::vector<Range> ins, outs;
    COC_TRY(check_ptr(g, m * k * es, "g"));
    COC_TRY(check_ptr(dy, m * n * es, "dy"));
    COC_TRY(check_ptr(dw, k * n * es, "dw"));
    ins.push_back(mk(g, m * k * es, "g"));
    ins.push_back(mk(dy, m * n * es, "dy"));
    outs.push_back(mk(dw, k * n * es, "dw"));
    COC_TRY(check_alias(outs, ins));
    // dw (k x n) = g^T dy: the activation operand is g read transposed (k
    // output rows, reduction over m), the weight operand dy as stored
    ChunksLaunch L{};
    L.kind = kind_of(dt);
    L.b = dy;
    L.c = dw;
    L.n = n;
    L.k = m;
    L.trans_a = 1;
    L.lda = k;
    L.npieces = 1;
    L.a[0] = g;
    L.rpb[0] = k;
    L.nblk[0] = 1;
    L.wait[0] = -1;
    L.signal[0] = -1;
    int32_t tiles[kMaxPieces + 1];
    bool cap = false;
    COC_TRY(capture_once(stream, &cap));
    return launch(KC_GEMM, 2.0 * double(m) * double(n) * double(k), stream,
                  [&] { return launch_gemm_chunks(L, stream, tiles); });
}

coc_status coc_alltoall_grouped_matmul(const void* x_own, const void* const* peer_bufs, const int64_t* counts,
                                       const void* w, void* y, void* recv_out, int32_t world, int32_t rank,
                                       int32_t experts, int64_t n, int64_t k, coc_dtype dt, int32_t split,
                                       hipStream_t stream) {
    clear_error();
    MoePlan M;
    COC_TRY(make_moe_plan(counts, world, rank, experts, n, k, dt, split, &M));
    if (M.total == 0) return COC_OK;
    const int64_t es = 2;
    static const char* names[COC_MAX_WORLD] = {"peer_bufs[0]", "peer_bufs[1]", "peer_bufs[2]", "peer_bufs[3]",
                                               "peer_bufs[4]", "peer_bufs[5]", "peer_bufs[6]", "peer_bufs[7]"};
    std::vector<Range> ins, outs;
    const void* src[COC_MAX_WORLD] = {};
    for (int r = 0; r < world; ++r) {
        const int64_t bytes = M.src_rows[r] * k * es;
        if (r == rank) {
            COC_TRY(check_ptr(x_own, bytes, "x_own"));
            ins.push_back(mk(x_own, bytes, "x_own"));
            src[r] = x_own;
            continue;
        }
        if (bytes > 0 && !peer_bufs) return fail(COC_ERR_NULL, "peer_bufs is NULL");
        const void* pb = bytes > 0 ? peer_bufs[r] : nullptr;
        COC_TRY(check_ptr(pb, bytes, names[r]));
        ins.push_back(mk(pb, bytes, names[r]));
        src[r] = pb;
    }
    COC_TRY(check_ptr(w, experts * k * n * es, "w"));
    COC_TRY(check_ptr(y, M.total * n * es, "y"));
    COC_TRY(check_ptr(recv_out, M.total * k * es, "recv_out"));
    ins.push_back(mk(w, experts * k * n * es, "w"));
    outs.push_back(mk(y, M.total * n * es, "y"));
    outs.push_back(mk(recv_out, M.total * k * es, "recv_out"));
    COC_TRY(check_alias(outs, ins));
    return run_moe_dispatch(M, src, w, y, recv_out, stream);
}

coc_status coc_grouped_matmul_alltoall(const void* h, const void* w, void* y_local, void* y_own,
                                       void* const* peer_out, const int64_t* counts, int32_t world, int32_t rank,
                                       int32_t experts, int64_t n, int64_t k, coc_dtype dt, int32_t split,
                                       hipStream_t stream) {
    clear_error();
    MoePlan M;
    COC_TRY(make_moe_plan(counts, world, rank, experts, n, k, dt, split, &M));
    if (M.total == 0) return COC_OK;
    const int64_t es = 2;
    static const char* names[COC_MAX_WORLD] = {"peer_out[0]", "peer_out[1]", "peer_out[2]", "peer_out[3]",
                                               "peer_out[4]", "peer_out[5]", "peer_out[6]", "peer_out[7]"};
    std::vector<Range> ins, outs;
    COC_TRY(check_ptr(h, M.total * k * es, "h"));
    COC_TRY(check_ptr(w, experts * k * n * es, "w"));
    COC_TRY(check_ptr(y_local, M.total * n * es, "y_local"));
    ins.push_back(mk(h, M.total * k * es, "h"));
    ins.push_back(mk(w, experts * k * n * es, "w"));
    outs.push_back(mk(y_local, M.total * n * es, "y_local"));
    void* dst[COC_MAX_WORLD] = {};
    for (int r = 0; r < world; ++r) {
        const int64_t bytes = M.src_rows[r] * n * es;
        if (r == rank) {
            COC_TRY(check_ptr(y_own, bytes, "y_own"));
            outs.push_back(mk(y_own, bytes, "y_own"));
            dst[r] = y_own;
            continue;
        }
        if (bytes > 0 && !peer_out) return fail(COC_ERR_NULL, "peer_out is NULL");
        void* pb = bytes > 0 ? peer_out[r] : nullptr;
        COC_TRY(check_ptr(pb, bytes, names[r]));
        outs.push_back(mk(pb, bytes, names[r]));
        dst[r] = pb;
    }
    COC_TRY(check_alias(outs, ins));
    return run_moe_combine(M, h, w, y_local, dst, stream);
}

coc_status coc_check_waits(hipStream_t stream) {
    clear_error();
    bool cap = false;
    COC_TRY(capturing(stream, &cap));
    if (cap) return fail(COC_ERR_CAPTURE, "coc_check_waits reads device memory and cannot be captured");
    int dev = 0;
    COC_HIP(hipGetDevice(&dev));
    StreamCtx* c = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_ctx_mu);
        auto it = g_ctx.find(std::make_pair(dev, stream));
        if (it != g_ctx.end()) c = it->second;
    }
    COC_HIP(hipStreamSynchronize(stream));
    uint32_t* words[2] = {c != nullptr ? c->gave_up() : nullptr, static_gave_up(dev)};
    bool gave_up = false;
    for (uint32_t* w : words) {
        if (w == nullptr) continue;
        uint32_t v = 0;
        COC_HIP(hipMemcpy(&v, w, sizeof v, hipMemcpyDeviceToHost));
        if (v != 0) {
            static const uint32_t zero = 0;
            COC_HIP(hipMemcpy(w, &zero, sizeof zero, hipMemcpyHostToDevice));
            gave_up = true;
        }
    }
    if (gave_up)
        return fail(COC_ERR_TIMEOUT, "a hand-over wait gave up: the rows or tiles it guarded were written as NaN");
    return COC_OK;
}

void coc_profile_enable(int32_t on) { g_prof_on.store(on ? 1 : 0); }

void coc_profile_stamps(void* buf, int64_t records) { set_stamp_buffer((uint64_t*)buf, records); }

int64_t coc_profile_stamp_count(void) { return stamp_records_used(); }

coc_status coc_profile_read(double* total_ms, int64_t* launches, double* work_units) {
    clear_error();
    std::vector<ProfRec> recs;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        recs.swap(g_prof_recs);
    }
    double ms[COC_NUM_KCLASS] = {0, 0, 0};
    int64_t cnt[COC_NUM_KCLASS] = {0, 0, 0};
    double work[COC_NUM_KCLASS] = {0, 0, 0};
    coc_status st = COC_OK;
    for (const ProfRec& r : recs) {
        float t = 0.f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
        if (e != hipSuccess && st == COC_OK) st = hip_fail(e, "hipEventElapsedTime");
        ms[r.cls] += t;
        cnt[r.cls] += 1;
        work[r.cls] += r.work;
    }
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        for (const ProfRec& r : recs) {
            g_prof_pool.push_back(r.a);
            g_prof_pool.push_back(r.b);
        }
    }
    for (int i = 0; i < COC_NUM_KCLASS; ++i) {
        if (total_ms) total_ms[i] = ms[i];
        if (launches) launches[i] = cnt[i];
        if (work_units) work_units[i] = work[i];
    }
    return st;
}

coc_status coc_profile_records(int32_t* kclass, double* start_ms, double* end_ms, double* work_units,
                               int32_t max, int32_t* n) {
    clear_error();
    std::vector<ProfRec> recs;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        recs.swap(g_prof_recs);
    }
    coc_status st = COC_OK;
    if (!n) st = fail(COC_ERR_NULL, "n is NULL");
    int32_t k = 0;
    for (size_t i = 0; i < recs.size() && st == COC_OK; ++i) {
        const ProfRec& r = recs[i];
        float t0 = 0.f, t1 = 0.f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&t0, recs[0].a, r.a);
        if (e == hipSuccess) e = hipEventElapsedTime(&t1, recs[0].a, r.b);
        if (e != hipSuccess) {
            st = hip_fail(e, "hipEventElapsedTime");
            break;
        }
        if (k < max) {
            if (kclass) kclass[k] = r.cls;
            if (start_ms) start_ms[k] = t0;
            if (end_ms) end_ms[k] = t1;
            if (work_units) work_units[k] = r.work;
        }
        ++k;
    }
    if (n) *n = k;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        for (const ProfRec& r : recs) {
            g_prof_pool.push_back(r.a);
            g_prof_pool.push_back(r.b);
        }
    }
    return st;
}

}  // extern "C"
