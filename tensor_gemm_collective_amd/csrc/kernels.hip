// gfx950 kernels of the fused matmul + collective path.
//
//   gemm_ring   m-chunk matmul, bf16 / fp16 inputs, k a multiple of 32:
//               direct-to-LDS loads into an LDS ring, LDS transpose reads,
//               binary32 accumulation on MFMA, round-to-nearest-even to the
//               storage dtype.  The "Matmul" of the CoC guide's
//               matmul/collective pairs ("Problem analysis").
//   gemm_dma    the same for any k (a multiple of 8), 128 x 128 tiles.
//   gemm_w8     the same with int8 weights (w8A16): converted to fp16 in
//               the main loop and scaled there per group, or the fp32 sums
//               scaled in the epilogue per tensor / per channel.
//   gemm_f32    the same for binary32 inputs on the vector ALUs.
//   reduce_rows fixed-order sum of the ranks' partials for a block of rows:
//               the AllReduce / ReduceScatter half of a pair.
//   gather_rows bit copy of sequence shards into the gathered matrix: the
//               AllGather half of the ColumnParallel pair.
//
// Every kernel takes fully validated sizes; all global accesses are guarded by
// the row / column / k bounds passed in.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "coc_internal.h"
#define COC_HD __host__ __device__
#include "coc_schedule.h"

// Build-time tuning knob (default: the measured best): the fewest workgroups
// the chunk matmuls running side by side should have together before the
// ring kernel moves to a larger tile.
// Activations of two consecutive k stages staged together as whole 128-byte
// row segments (k % 64 == 0; transposed weights likewise): measured 1.2-2.8 %
// faster on the LLaMA2-70B shapes with random operands (5-10 % with
// transposed weights), bit-identical results.
#ifndef COC_PAIR_A
#define COC_PAIR_A 1
#endif
#ifndef COC_RING_MIN_TILES
#define COC_RING_MIN_TILES 200
#endif

namespace coc {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ conversions
// binary32 -> bfloat16, round to nearest even: add 0x7fff plus the lowest kept
// bit, then drop the low 16 bits (a carry into the exponent handles rounding
// up to the next binade and to infinity).  NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// binary32 -> binary16 with the hardware conversion (round to nearest even
// in the default mode, binary16 subnormals kept).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    _Float16 h = (_Float16)f;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
}

template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    if constexpr (DT == COC_BF16)
        return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
    else
        return f32_to_f16_bits(lo) | (f32_to_f16_bits(hi) << 16);
}

template <int DT>
__device__ __forceinline__ float unpack_lo(uint32_t w) {
    if constexpr (DT == COC_BF16) return bf16_bits_to_f32(w & 0xffffu);
    else return f16_bits_to_f32(w & 0xffffu);
}
template <int DT>
__device__ __forceinline__ float unpack_hi(uint32_t w) {
    if constexpr (DT == COC_BF16) return bf16_bits_to_f32(w >> 16);
    else return f16_bits_to_f32(w >> 16);
}

// ------------------------------------------------------------------ row maps
// A chunk's rows: { base + b*stride + j : b < nblk, j < rpb }, local index
// r = b*rpb + j.
__device__ __forceinline__ int64_t map_row(int32_t r, int32_t rpb, int64_t base, int64_t stride) {
    const int32_t b = r / rpb;
    return base + (int64_t)b * stride + (r - b * rpb);
}

struct GemmParams {
    const uint8_t* a;
    const uint8_t* b;
    uint8_t* c;
    const uint16_t* scales;
    int64_t base, stride;
    int32_t rpb, rows, n, k;
    int32_t tiles_m, tiles_n;
    int32_t qmode, group;
    int32_t lda;   // transposed activations: elements per stored row
};

// ------------------------------------------------------------------ tile order
// Workgroups are handed to the 8 XCDs (each with its own L2) round-robin by
// id.  The first bijection gives XCD x a contiguous run of tile numbers; the
// second walks tile numbers in groups of up to 4 tile rows, m-fastest inside a
// group.  A short chunk (<= 4 tile rows) thus keeps each weight column block on
// one XCD, and a tall matrix gets 4-row x n blocks per XCD instead of tiles
// from 16 rows whose activation blocks all sit 4 MB apart.
__device__ __forceinline__ int xcd_tile(int b, int total) {
    constexpr int NX = 8;
    const int q = total / NX, r = total % NX;
    const int x = b % NX, local = b / NX;
    return x * q + (x < r ? x : r) + local;
}

__device__ __forceinline__ void grouped_coords(int t, int tiles_m, int tiles_n, int* tm, int* tn) {
    constexpr int GM = 4;
    const int per_group = GM * tiles_n;
    const int g = t / per_group;
    const int rows_in_group = (tiles_m - g * GM) < GM ? (tiles_m - g * GM) : GM;
    const int in_g = t - g * per_group;
    *tm = g * GM + in_g % rows_in_group;
    *tn = in_g / rows_in_group;
}

__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int* tm, int* tn) {
    grouped_coords(xcd_tile(b, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
}

// ------------------------------------------------------------------ cross-kernel sync
// Counters in device memory let one chunk-walking matmul kernel and the
// reduce / gather kernels beside it on another stream hand chunks over without
// a kernel boundary.  The data handed over is written with system-scope
// (write-through, sc0 sc1) stores, and the reduce reads the matmul's partials
// with system-scope loads, so no L2 writeback or invalidate is needed: a
// producer waits for its stores to complete, then bumps the counter; a
// consumer polls the counter, then loads.  (Device-scope fences here would
// write back or invalidate a whole XCD L2 per workgroup, dropping the cached
// weight tiles of the matmul running beside.)  Counters only grow (mod 2^32);
// the host tracks the value each wait must reach.  Waits are bounded: on
// time-out the waiting kernel writes NaN instead of results and carries on,
// so a lost signal shows up in the output instead of hanging the GPU.
constexpr uint32_t kSpinLimit = 1u << 19;   // polls, ~2 s at the longest sleep
// Scope of the counter loads and adds (the data itself is always written and
// read at system scope).
#ifndef COC_SYNC_SYSTEM
#define COC_SYNC_SYSTEM 0
#endif
constexpr int kSyncScope = COC_SYNC_SYSTEM ? __HIP_MEMORY_SCOPE_SYSTEM : __HIP_MEMORY_SCOPE_AGENT;

// Polls back off from ~0.1 us to ~4 us between loads: hundreds of workgroups
// polling one counter at a fixed short interval load its HBM channel enough to
// slow every other stream through it.
// Waits until the sum of `lines` counters (kSyncWords apart) reaches target.
__device__ __forceinline__ bool spin_until(const uint32_t* p, int lines, uint32_t target, uint32_t limit) {
    for (uint32_t i = 0; i < limit; ++i) {
        uint32_t v = 0;
        for (int l = 0; l < lines; ++l) v += __hip_atomic_load(p + l * kSyncWords, __ATOMIC_RELAXED, kSyncScope);
        if ((int32_t)(v - target) >= 0) return true;
        if (i < 4) __builtin_amdgcn_s_sleep(2);
        else if (i < 8) __builtin_amdgcn_s_sleep(16);
        else __builtin_amdgcn_s_sleep(127);
    }
    return false;
}

// Workgroup-wide wait for the counters: thread 0 polls and the outcome goes to
// every wave through LDS.  The barrier orders every later load after the
// poll.  Two calls must be separated by a workgroup barrier (the flag is
// reused).  A wait that gives up also stores 1 into *gave_up (if set), the
// word the host reads back to report the time-out.
__device__ __forceinline__ bool wg_wait(const uint32_t* p, int lines, uint32_t target, uint32_t limit,
                                        uint32_t* gave_up) {
    __shared__ int ok;
    if (threadIdx.x == 0) {
        ok = spin_until(p, lines, target, limit) ? 1 : 0;
        if (!ok && gave_up != nullptr) __hip_atomic_store(gave_up, 1u, __ATOMIC_RELAXED, kSyncScope);
    }
    __syncthreads();
    return ok != 0;
}

// Workgroup-wide signal after system-scope stores: every wave waits for its
// stores to complete, then one thread adds 1 to the counter.
__device__ __forceinline__ void wg_signal(uint32_t* p) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, kSyncScope);
}

// Streaming 16-byte loads and stores (non-temporal: no allocation in the
// caches on the way).  The reduce reads every partial exactly once and the
// gather every shard row exactly once; measured on the 8-source bf16 sum of
// 2048 x 14336 partials after a 512 MB flush: 3.5 TB/s with ordinary loads,
// 5.2 TB/s with non-temporal loads, 5.6 TB/s with non-temporal stores as well.
__device__ __forceinline__ u32x4 load16_stream(const uint8_t* p) {
    return __builtin_nontemporal_load((const u32x4*)p);
}
__device__ __forceinline__ void store16_stream(uint8_t* p, u32x4 v) { __builtin_nontemporal_store(v, (u32x4*)p); }

// ------------------------------------------------------------------ activity stamps
// Measurement only.  A launch given a stamp region (see coc_profile_stamps)
// has thread 0 of each workgroup write one record per piece of work into its
// own slot of the region (slot = workgroup x pieces + piece, assigned by the
// host, so no atomics): {what, start, end}, times from the 100 MHz real-time
// counter (consistent across the XCDs).  `what`: 1 + kind (0 matmul, 1
// reduce, 2 gather) | chunk << 8 | XCD << 16; a slot a workgroup had no work
// for stays zero.  End times are taken when the last store has been issued.
constexpr uint32_t kStampMatmul = 0, kStampReduce = 1, kStampGather = 2;

// The XCD the wave runs on (hardware register XCC_ID, bits 3:0).
__device__ __forceinline__ uint32_t xcd_id() { return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15u; }

__device__ __forceinline__ uint64_t realtime() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ void stamp(uint64_t* region, int slot, uint32_t what, uint64_t t0, uint64_t t1) {
    if (region == nullptr || threadIdx.x != 0) return;
    uint64_t* r = region + 3 * (int64_t)slot;
    r[0] = (uint64_t)(what + 1) | ((uint64_t)xcd_id() << 16);
    r[1] = t0;
    r[2] = t1;
}

// 16-byte system-scope stores go through a buffer resource over the whole
// output (byte offsets < 4 GiB: every matrix has fewer than 2^31 elements):
// one buffer_store_dwordx4 with sc0 sc1 (cache-policy bits 0 and 4), measured
// as fast as a plain store, where two 8-byte atomic stores run at ~60 %.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sys_rsrc(uint8_t* base) {
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)0xffffffff, 0x00020000);
}
__device__ __forceinline__ void store16_sys(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, off, 0, 17);
}

__device__ __forceinline__ u32x4 load16_sys(const uint8_t* src) {
    const u32x2 lo = __builtin_bit_cast(u32x2, __hip_atomic_load((const uint64_t*)src, __ATOMIC_RELAXED,
                                                                  __HIP_MEMORY_SCOPE_SYSTEM));
    const u32x2 hi = __builtin_bit_cast(u32x2, __hip_atomic_load((const uint64_t*)(src + 8), __ATOMIC_RELAXED,
                                                                  __HIP_MEMORY_SCOPE_SYSTEM));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// ------------------------------------------------------------------ MFMA GEMMs
// Both GEMM kernels compute C^T = W^T X^T on v_mfma_f32_32x32x16_{bf16,f16}:
// MFMA operand A is a weight fragment (lane l: column n = l % 32, 8 k values
// (l / 32) * 8 + 0..7 of the current 16-k step), operand B an activation
// fragment (lane l: row m = l % 32, the same 8 k values).  Each lane then
// holds 4 consecutive n of one row m per 32x32 block (one 8-byte store).
// Every kernel and tile shape walks k in the same 16-k steps in increasing
// order, so the bits of an output element depend neither on the tile shape
// nor on the kernel that produced it.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

template <int KIND>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (KIND == GK_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Register-staged kernel for int8 weights (w8A16): tile BM x BN x 64, 256
// threads as 2 x 2 waves.  Each thread loads an 8 k x 8 n block of int8
// weights, converts it to fp16 in registers (per group q * scale, rounded to
// nearest even; otherwise q, and the epilogue scales the fp32 sums) and
// stores it K-contiguous to LDS ([BN columns][64 k]); A goes to
// LDS as [BM rows][64 k].  The 16-byte chunk c of an LDS row sits at
// c ^ swz(row), which keeps the row stores and the MFMA operand reads of 8
// consecutive lanes on distinct banks.
template <int BM, int BN, int KIND>
__global__ __launch_bounds__(256) void gemm_w8(GemmParams p) {
    constexpr int BK = 64;
    constexpr int NT = 256;
    constexpr int WTM = BM / 2, WTN = BN / 2;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int A_ITERS = BM * 8 / NT;   // 16-byte A chunks per thread
    constexpr int NB = BN / 8;             // 8-column blocks of the weight tile
    static_assert(BN <= NT, "one 8x8 weight block per thread at most");
    constexpr int OUT_DT = (KIND == GK_BF16) ? COC_BF16 : COC_F16;

    __shared__ u32x4 smem[2 * (BM + BN) * 8];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // ---- A rows handled by this thread (row map evaluated once)
    const int akc = t & 7;
    const uint8_t* arow[A_ITERS];
    bool aval[A_ITERS];
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) {
        const int r = m0 + (t >> 3) + 32 * i;
        aval[i] = r < p.rows;
        const int64_t gr = aval[i] ? map_row(r, p.rpb, p.base, p.stride) : 0;
        arow[i] = p.a + gr * (int64_t)p.k * 2;
    }
    // ---- weight block handled by this thread
    const bool bact = t < BN;
    const int bkb = t / NB, bnb = t % NB;
    const int bcol = n0 + bnb * 8;
    const bool bcolv = bact && bcol < p.n;

    u32x4 ra[A_ITERS];
    u32x4 rb[8];      // 16-bit weights: 8 k rows x 8 columns
    u32x2 rq[8];      // int8 weights:   8 k rows x 8 columns
    u32x4 rs;         // fp16 scales of the 8 columns (per group)
    if constexpr (KIND == GK_W8_F16) rs = u32x4{0, 0, 0, 0};

    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_ITERS; ++i) {
            const int kk = k0 + akc * 8;
            ra[i] = (aval[i] && kk < p.k) ? *(const u32x4*)(arow[i] + (int64_t)kk * 2)
                                          : u32x4{0, 0, 0, 0};
        }
        const int kr0 = k0 + bkb * 8;
        const bool bv = bcolv && kr0 < p.k;
        if constexpr (KIND == GK_W8_F16) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                rq[j] = bv ? *(const u32x2*)(p.b + (int64_t)(kr0 + j) * p.n + bcol) : u32x2{0, 0};
            if (p.qmode == COC_PER_GROUP && bv)
                rs = *(const u32x4*)(p.scales + (int64_t)(kr0 / p.group) * p.n + bcol);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                rb[j] = bv ? *(const u32x4*)(p.b + ((int64_t)(kr0 + j) * p.n + bcol) * 2)
                           : u32x4{0, 0, 0, 0};
        }
    };

    auto store = [&](int buf) {
        u32x4* As = smem + buf * (BM + BN) * 8;
        u32x4* Bs = As + BM * 8;
#pragma unroll
        for (int i = 0; i < A_ITERS; ++i) {
            const int row = (t >> 3) + 32 * i;
            As[row * 8 + (akc ^ swz(row))] = ra[i];
        }
        if (bact) {
            if constexpr (KIND == GK_W8_F16) {
                // per group dequantise: w = fp16(q) * scale, rounded to nearest
                // even in fp16; per tensor / per channel the tile holds q itself
                // (exact in fp16) and the epilogue scales the fp32 sums
                const bool grouped = p.qmode == COC_PER_GROUP;
                uint32_t h[8][8];
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const uint32_t sb = (c & 1) ? (rs[c >> 1] >> 16) : (rs[c >> 1] & 0xffffu);
                    const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)sb);
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int8_t q = (int8_t)((rq[j][c >> 2] >> (8 * (c & 3))) & 0xffu);
                        const _Float16 w = grouped ? (_Float16)(int)q * sc : (_Float16)(int)q;
                        h[j][c] = __builtin_bit_cast(uint16_t, w);
                    }
                }
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int nl = bnb * 8 + c;
                    u32x4 v;
#pragma unroll
                    for (int pp = 0; pp < 4; ++pp) v[pp] = h[2 * pp][c] | (h[2 * pp + 1][c] << 16);
                    Bs[nl * 8 + (bkb ^ swz(nl))] = v;
                }
            } else {
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int nl = bnb * 8 + c;
                    u32x4 v;
#pragma unroll
                    for (int pp = 0; pp < 4; ++pp) {
                        const uint32_t lo = rb[2 * pp][c >> 1];
                        const uint32_t hi = rb[2 * pp + 1][c >> 1];
                        v[pp] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                        : ((lo & 0xffffu) | (hi << 16));
                    }
                    Bs[nl * 8 + (bkb ^ swz(nl))] = v;
                }
            }
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    constexpr int MFMA_KIND = (KIND == GK_BF16) ? GK_BF16 : GK_F16;
    auto compute = [&](int buf) {
        const u32x4* As = smem + buf * (BM + BN) * 8;
        const u32x4* Bs = As + BM * 8;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int kc = ks * 2 + (lane >> 5);
            u32x4 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * WTM + i * 32 + (lane & 31);
                af[i] = As[row * 8 + (kc ^ swz(row))];
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * WTN + j * 32 + (lane & 31);
                bf[j] = Bs[row * 8 + (kc ^ swz(row))];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<MFMA_KIND>(bf[j], af[i], acc[i][j]);
        }
    };

    const int KT = (p.k + BK - 1) / BK;
    if (KT > 0) {
        load(0);
        store(0);
        __syncthreads();
        for (int kt = 0; kt < KT; ++kt) {
            if (kt + 1 < KT) load((kt + 1) * BK);
            compute(kt & 1);
            if (kt + 1 < KT) store((kt + 1) & 1);
            __syncthreads();
        }
    }

    // ---- epilogue: lane holds n = j*8 + (lane/32)*4 + {0..3} of row m = lane%32
    // (w8A16 per tensor / per channel: sum * scale in fp32, then rounded;
    // n % 8 == 0, so a group of four columns is wholly in range or wholly out)
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int r = m0 + wm * WTM + i * 32 + (lane & 31);
        if (r >= p.rows) continue;
        const int64_t gr = map_row(r, p.rpb, p.base, p.stride);
        uint8_t* crow = p.c + gr * (int64_t)p.n * 2;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = n0 + wn * WTN + j * 32 + q * 8 + (lane >> 5) * 4;
                if (col < p.n) {
                    float sc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
                    if constexpr (KIND == GK_W8_F16) {
                        if (p.qmode == COC_PER_TENSOR) {
                            const float s0 = (float)__builtin_bit_cast(_Float16, p.scales[0]);
#pragma unroll
                            for (int t = 0; t < 4; ++t) sc[t] = s0;
                        } else if (p.qmode == COC_PER_CHANNEL) {
                            const u32x2 sv = *(const u32x2*)(p.scales + col);
#pragma unroll
                            for (int t = 0; t < 4; ++t)
                                sc[t] = (float)__builtin_bit_cast(_Float16, (uint16_t)(sv[t >> 1] >> (16 * (t & 1))));
                        }
                    }
                    u32x2 v;
                    v[0] = pack2<OUT_DT>(acc[i][j][q * 4 + 0] * sc[0], acc[i][j][q * 4 + 1] * sc[1]);
                    v[1] = pack2<OUT_DT>(acc[i][j][q * 4 + 2] * sc[2], acc[i][j][q * 4 + 3] * sc[3]);
                    *(u32x2*)(crow + (int64_t)col * 2) = v;
                }
            }
        }
    }
}

// Direct-to-LDS kernel for bf16 / fp16 (gfx950).  Tile BM x BN, k in stages
// of BK (32 or 64), an LDS ring of STAGES stages, 64 * WM * WN threads (WM x WN
// waves, wave tile BM/WM x BN/WN).
//
//   * Both operands go from global memory straight into LDS with 16-byte
//     global_load_lds_dwordx4 (lane L of a wave-instruction lands at byte
//     16 * L of a 1 KB LDS block); no VGPR staging, no LDS store instructions.
//     Each lane picks the global chunk that belongs at its LDS slot, which is
//     how the XOR swizzles below are applied.
//   * A (X rows, k-contiguous) is stored [BM rows][BK k]; chunk c of row r
//     sits at c ^ gA(r), so the 16-byte MFMA operand reads of 16 consecutive
//     rows hit distinct banks.  With BK = 64 every A row contributes a whole
//     128-byte line per stage.
//   * The weight (k x n row-major in memory) is stored as it comes, [BK k][BN
//     n]; chunk c of k-row K sits at c ^ gB(K).  The MFMA fragment (lane l:
//     column l % 32, 8 consecutive k) is read with two ds_read_b64_tr_b16: in
//     each 16-lane group, lane i receives element i % 4 of the 8-byte chunks
//     addressed by lanes 4j + i / 4 (j = 0..3), so lane 4j + q pointing at
//     k-row K0 + j, columns n0 + 4q .. n0 + 4q + 3 hands lane i column n0 + i
//     at k-rows K0 .. K0 + 3.
//   * Lanes outside the matrix (m, n or k tail) load 16 zero bytes from a
//     device constant instead, so every wave issues the same number of loads
//     per stage and vmcnt counts stay exact; the k tail is zero-filled this way.
//   * Per stage: wait for this wave's loads of the stage, barrier (every
//     wave's loads are then visible and every wave is done with the slot the
//     next loads go to), issue the loads of stage kt + STAGES - 1, then the
//     MFMA k steps with the next step's fragments read ahead.  The DMA loads
//     are issued through inline asm so the compiler does not order every LDS
//     read behind them; the explicit vmcnt wait + s_barrier is the ordering.
__device__ const u32x4 g_zero16 = {0, 0, 0, 0};

#define COC_LDS __attribute__((address_space(3)))
typedef short s16x4 __attribute__((ext_vector_type(4)));

// A rows hold BK/8 16-byte chunks: 4 (BK 32) or 8 (BK 64).
template <int BK>
__device__ __forceinline__ int gA(int r) {
    if constexpr (BK == 32) return ((r >> 2) ^ (r >> 1)) & 3;
    else return (r ^ (r >> 3)) & 7;
}
__device__ __forceinline__ int gB(int K) { return (K & 3) << 2; }
// Paired activation stages (128-byte rows of 8 chunks): chunk c of row r at
// c ^ gP(r).  A 16-lane group of a fragment read takes 16 consecutive rows at
// one chunk; the 8 rows of each parity then land on 8 distinct 16-byte bank
// groups.  The period, 16 rows, divides the 32 rows between a wave's
// fragments, so one offset per lane serves every fragment.
__device__ __forceinline__ int gP(int r) { return (r >> 1) & 7; }

// DEV_SCOPE: device-scope load (sc1), which does not allocate in the
// per-CU L1; each 16-byte chunk is read once per workgroup, so L1 caching buys
// nothing and its miss queue was measured stalling the 256x256 kernel.
template <bool DEV_SCOPE>
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
    if constexpr (DEV_SCOPE)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off sc1"
                     :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory", "m0");
}

// The same copy addressed as an SGPR base plus a 32-bit VGPR offset (device
// scope), so per-stage address updates are scalar adds.
__device__ __forceinline__ void dma16_sbase(uint32_t voff, const void* sbase, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 sc1"
                 :: "v"(voff), "s"(sbase), "s"(lds_base) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return (uint32_t)(uintptr_t)(const COC_LDS void*)p;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int BM, int BN, int WM, int WN, int STAGES, int BK, int KIND, bool DEV_SCOPE>
__global__ __launch_bounds__(64 * WM * WN) void gemm_dma(GemmParams p) {
    constexpr int NW = WM * WN;
    constexpr int KS = BK / 16;    // MFMA k steps per stage
    constexpr int ACH = BK / 8;    // 16-byte chunks per A row
    static_assert(BK == 32 || BK == 64, "stage depth");
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int A_INS = A_BYTES / 1024, B_INS = B_BYTES / 1024;
    static_assert(A_INS % NW == 0 && B_INS % NW == 0, "loads must split evenly over waves");
    static_assert(BN % 128 == 0, "B swizzle works on 16-chunk groups");
    static_assert(STAGES >= 2 && STAGES <= 4, "stage ring");
    constexpr int APW = A_INS / NW, BPW = B_INS / NW, LPW = APW + BPW;
    constexpr int BROW = BN / 8;   // 16-byte chunks per weight k-row
    constexpr int OUT_DT = (KIND == GK_BF16) ? COC_BF16 : COC_F16;
    __shared__ __attribute__((aligned(1024))) uint8_t sm0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t sm1[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t sm2[STAGES >= 3 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t sm3[STAGES == 4 ? STAGE : 16];
    auto stage = [&](auto S) -> uint8_t* {
        constexpr int s_ = decltype(S)::value;
        if constexpr (s_ == 0) return sm0;
        else if constexpr (s_ == 1) return sm1;
        else if constexpr (s_ == 2) return sm2;
        else return sm3;
    };

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave / WN, wn = wave % WN;
    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // global sources of this wave's loads (row map applied once)
    const uint8_t* asrc[APW];
    int akof[APW];
    bool aok[APW];
#pragma unroll
    for (int i = 0; i < APW; ++i) {
        const int q = (wave * APW + i) * 64 + lane;
        const int row = q / ACH;
        aok[i] = m0 + row < p.rows;
        const int64_t gr = aok[i] ? map_row(m0 + row, p.rpb, p.base, p.stride) : 0;
        asrc[i] = p.a + gr * (int64_t)p.k * 2;
        akof[i] = ((q % ACH) ^ gA<BK>(row)) * 8;
    }
    const uint8_t* bsrc[BPW];
    int bkr[BPW];
    bool bok[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
        const int q = (wave * BPW + i) * 64 + lane;
        const int K = q / BROW;
        const int col = n0 + ((q % BROW) ^ gB(K)) * 8;
        bok[i] = col < p.n;
        bkr[i] = K;
        bsrc[i] = p.b + (int64_t)(bok[i] ? col : 0) * 2;
    }
    const uint8_t* zero = (const uint8_t*)&g_zero16;

    auto issue = [&](int kt, auto S) {
        const int k0 = kt * BK;
        uint8_t* st = stage(S);
#pragma unroll
        for (int i = 0; i < APW; ++i) {
            const uint8_t* src =
                (aok[i] && k0 + akof[i] < p.k) ? asrc[i] + (int64_t)(k0 + akof[i]) * 2 : zero;
            dma16<DEV_SCOPE>(src, lds_u32(st + (wave * APW + i) * 1024));
        }
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
            const uint8_t* src =
                (bok[i] && k0 + bkr[i] < p.k) ? bsrc[i] + (int64_t)(k0 + bkr[i]) * p.n * 2 : zero;
            dma16<DEV_SCOPE>(src, lds_u32(st + A_BYTES + (wave * BPW + i) * 1024));
        }
    };

    // fragment offsets within a stage
    int aoff[KS][FM];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * WTM + i * 32 + (lane & 31);
            aoff[ks][i] = row * (BK * 2) + (((ks * 2 + (lane >> 5)) ^ gA<BK>(row)) << 4);
        }
    int boff[KS][2][FN];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int r = lane & 15, grp = (lane >> 4) & 1, hk = lane >> 5;
                const int K = ks * 16 + hk * 8 + h * 4 + (r >> 2);
                const int col = wn * WTN + j * 32 + grp * 16 + 4 * (r & 3);
                boff[ks][h][j] = A_BYTES + K * BN * 2 + (((col >> 3) ^ gB(K)) << 4) + (col & 7) * 2;
            }

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    auto rd = [&](const COC_LDS uint8_t* st, int ks, u32x4* af, u32x4* bf) {
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = *(const COC_LDS u32x4*)(st + aoff[ks][i]);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((COC_LDS s16x4*)(st + boff[ks][0][j]));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((COC_LDS s16x4*)(st + boff[ks][1][j]));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            bf[j] = u32x4{l2[0], l2[1], h2[0], h2[1]};
        }
    };
    auto mm = [&](const u32x4* af, const u32x4* bf) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<KIND>(bf[j], af[i], acc[i][j]);
    };

    const int KT = (p.k + BK - 1) / BK;
    std::integral_constant<int, 0> S0;
    std::integral_constant<int, 1> S1;
    std::integral_constant<int, 2> S2;
    std::integral_constant<int, 3> S3;
    if (0 < KT) issue(0, S0);
    if constexpr (STAGES >= 3) {
        if (1 < KT) issue(1, S1);
    }
    if constexpr (STAGES == 4) {
        if (2 < KT) issue(2, S2);
    }
    auto body = [&](int kt, auto S) {
        constexpr int cs = decltype(S)::value;
        // this wave's loads of stage kt are done; stages issued after it may stay in flight
        const int ahead = KT - 1 - kt;
        if constexpr (STAGES == 4) {
            if (ahead >= 2) wait_vmcnt<2 * LPW>();
            else if (ahead == 1) wait_vmcnt<LPW>();
            else wait_vmcnt<0>();
        } else if constexpr (STAGES == 3) {
            if (ahead >= 1) wait_vmcnt<LPW>();
            else wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
        }
        // every wave's loads of stage kt are visible, and every wave is done
        // reading the slot the next loads go to
        block_barrier();
        if (kt + STAGES - 1 < KT)
            issue(kt + STAGES - 1, std::integral_constant<int, (cs + STAGES - 1) % STAGES>{});
        const COC_LDS uint8_t* st = (const COC_LDS uint8_t*)stage(S);
        u32x4 af[2][FM], bf[2][FN];
        rd(st, 0, af[0], bf[0]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) rd(st, ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
            mm(af[ks & 1], bf[ks & 1]);
        }
    };
    for (int kt = 0; kt < KT; kt += STAGES) {
        body(kt, S0);
        if (kt + 1 < KT) body(kt + 1, S1);
        if constexpr (STAGES >= 3) {
            if (kt + 2 < KT) body(kt + 2, S2);
        }
        if constexpr (STAGES == 4) {
            if (kt + 3 < KT) body(kt + 3, S3);
        }
    }

    // ---- epilogue: lane holds n = q*8 + (lane/32)*4 + {0..3} of row m = lane%32
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int r = m0 + wm * WTM + i * 32 + (lane & 31);
        if (r >= p.rows) continue;
        const int64_t gr = map_row(r, p.rpb, p.base, p.stride);
        uint8_t* crow = p.c + gr * (int64_t)p.n * 2;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = n0 + wn * WTN + j * 32 + q * 8 + (lane >> 5) * 4;
                if (col < p.n) {
                    u32x2 v;
                    v[0] = pack2<OUT_DT>(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]);
                    v[1] = pack2<OUT_DT>(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
                    *(u32x2*)(crow + (int64_t)col * 2) = v;
                }
            }
        }
    }
}

// LDS-ring kernel for bf16 / fp16 with k a positive multiple of 32 (gfx950).
// Tile BM x BN, WM x WN waves of BM/WM x BN/WN, k in stages of 32, an LDS ring
// of S stages.  Measured best: 256 x 256 and 128 x 256 with 2 x 4 waves (two
// waves per SIMD, so one wave's waits are covered by the other's MFMAs), and
// 128 x 128 with 2 x 2 waves (two workgroups per CU).
//
//   * Per 16-k step a wave reads FM + 2 FN fragments (FM = wave rows / 32,
//     FN = wave columns / 32) for FM x FN MFMAs.
//   * Loads are the same direct-to-LDS 16-byte copies and XOR swizzles as
//     gemm_dma, addressed as an SGPR base (the stage's k offset) plus a fixed
//     32-bit VGPR offset per lane.  Rows and columns past the matrix are
//     clamped to valid ones (their results are never stored); k has no tail.
//   * Each stage runs in two phases of FM x FN MFMAs.  Phase 1 computes k step
//     0 while reading the fragments of k step 1.  Then this wave waits for its
//     loads of the next stage and the workgroup meets at a barrier: every
//     wave's loads of stage kt + 1 are then in LDS and every wave has finished
//     reading stage kt - 1.  Phase 2 computes k step 1 while reading the
//     fragments of stage kt + 1 (k step 0) and loading stage kt + S - 1 into
//     the slot stage kt - 1 used.  The MFMA unit thus never waits for a
//     fragment read at a stage boundary.
//   * Fragment reads go 2 per MFMA from the first MFMA of a phase; the DMA
//     instructions are spread evenly over phase 2.  sched_barrier fixes that
//     order against the compiler's scheduler.
//   * With k % 64 == 0 (activations not transposed) the activations of stages
//     2j and 2j + 1 arrive together, whole 128-byte row segments, in one of
//     two pair blocks; the weights keep their four 32-k slots.  The pair is
//     loaded with the weights of stage 2j, in phase 2 of stage 2j - 3, which
//     keeps the same two stages of load slack.  Transposed weights (k
//     contiguous) are paired the same way and load with the activations'
//     pair.  The fragments, and so the bits, are those of the 32-k layout.
//   * Phase 2 runs at wave priority 1 and phase 1 at 0.  The two waves on a
//     SIMD drift apart by up to a phase; the barrier then waits for the one
//     still in phase 2, which the priority lets issue first.  Measured with a
//     shader-cycle counter around the phases: 1229 -> 1153 cycles per stage
//     on a 256 x 256 tile, the barrier wait 268 -> 178.
//   * The k walk (16-k MFMA steps in increasing k, same operand roles) is the
//     one every other kernel here uses, so results are bitwise identical to
//     theirs.
// w8A16 ring tiles keep the tile's per-group fp16 scales in LDS: at most this
// many bytes (k / group rows of BN scales).
constexpr int kW8TableBytes = 32768;
// Kernel-side kind of the int8-weight ring kernels with per-group scales (the
// host passes GK_W8_F16 and the scale mode): the main loop multiplies each
// k-group by its scale, where the GK_W8_F16 kernels scale the fp32 sums in
// the epilogue (per tensor / per channel).
constexpr int GK_W8G_F16 = 4;
constexpr bool is_w8(int kind) { return kind == GK_W8_F16 || kind == GK_W8G_F16; }

template <int BM, int BN, int S, int WM, int WN, int KIND = GK_BF16>
constexpr int ring_lds_bytes() {
    const int ring = S * (BM * 32 * 2 + 32 * BN * (is_w8(KIND) ? 1 : 2)) + (is_w8(KIND) ? kW8TableBytes : 0);
    return ring > BM * BN * 2 ? ring : BM * BN * 2;   // the epilogue stages the tile in the same LDS
}

// One BM x BN output tile at (m0, n0) of a chunk with row map (rows, rpb,
// base, stride); A row = output row + ashift.  `sm` is the workgroup's LDS ring; the caller guarantees that
// every wave has finished with it and has no stores outstanding.  poison:
// store NaN instead of the products (a wait for the tile's inputs timed out).
// SYS: system-scope (write-through) stores, for a tile another kernel reads
// while this one runs.  TA: the activation operand is stored transposed
// (p.a holds its k rows of p.lda elements, m contiguous; one piece, no row
// map); TB: the weight operand is stored transposed (p.b holds n rows of k
// elements).  A transposed operand is staged the way the other one is
// normally (rows of one k step's 64 bytes, or k rows read with the LDS
// transpose), so both come out in the same MFMA fragments and the result
// bits do not change.
template <int BM, int BN, int S, int WM, int WN, int KIND, bool SYS = false, bool TA = false, bool TB = false,
          bool PA = false>
__device__ __forceinline__ void ring_tile(const GemmParams& p, int rows, int rpb, int64_t base, int64_t stride,
                                          int64_t ashift, int m0, int n0, uint8_t* sm, bool poison) {
    constexpr int BK = 32, NW = WM * WN;
    constexpr bool W8 = is_w8(KIND);           // int8 weights, fp16 activations
    constexpr bool grouped = KIND == GK_W8G_F16;   // per-group scales
    constexpr int BE = W8 ? 1 : 2;            // weight bytes per element
    constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 32, FN = WTN / 32;
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * BE, STAGE = A_BYTES + B_BYTES;
    constexpr int APW = A_BYTES / 1024 / NW, BPW = B_BYTES / 1024 / NW, DPW = APW + BPW;
    constexpr int BROW = BN * BE / 16;   // 16-byte chunks per weight k-row
    constexpr int KPI = 64 / BROW;       // weight k-rows per load instruction
    constexpr int WRD = (W8 || TB) ? 1 : 2;   // LDS reads per weight fragment
    constexpr int ARD = TA ? 2 : 1;           // LDS reads per activation fragment
    constexpr int NMM = FM * FN, NRD = ARD * FM + WRD * FN;
    constexpr int AROW = BM * 2 / 16;         // TA: 16-byte chunks per activation k-row
    constexpr int KPA = 64 / AROW;            // TA: activation k-rows per load instruction
    constexpr int OUT_DT = (KIND == GK_BF16) ? COC_BF16 : COC_F16;
    constexpr int TBL = S * STAGE;       // w8: scale table offset in LDS
    static_assert((A_BYTES / 1024) % NW == 0 && (B_BYTES / 1024) % NW == 0, "loads split over the waves");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile of 32 x 32 MFMA blocks");
    static_assert(W8 ? (BROW >= 8 && BROW <= 64) : (BROW >= 16 && BROW <= 64), "weight swizzle");
    static_assert(!(W8 && (TA || TB)) && !(TA && TB), "transposed operands: bf16 / fp16, one at a time");
    static_assert(!TA || (AROW >= 16 && AROW <= 64), "activation swizzle");
    static_assert(S >= 3 && ring_lds_bytes<BM, BN, S, WM, WN, KIND>() <= 160 * 1024, "LDS ring");
    // PA: the activations of two consecutive stages arrive together as whole
    // 128-byte row segments (64 k) into a pair block; LDS holds S / 2 pair
    // blocks (the A of S stages) and then S weight slots.  k % 64 == 0.
    constexpr int A_REG = PA ? S * A_BYTES : 0;
    constexpr int APW2 = 2 * APW;   // PA: load instructions per wave for an A pair
    // PB (PA with the weights stored transposed, k-contiguous like the
    // activations): the weights are paired the same way, in S / 2 pair blocks
    // after the activations', and both pairs load together in odd stages.
    constexpr bool PB = PA && TB;
    constexpr int BPW2 = 2 * BPW;
    static_assert(!PA || (!TA && S == 4), "paired stages: no transposed activations, 4 slots");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const uint32_t lds0 = lds_u32(sm);

    // load offsets from the stage's global base (bytes)
    uint32_t aof[APW], bof[BPW];
#pragma unroll
    for (int i = 0; i < APW; ++i) {
        if constexpr (TA) {
            // k-row K of the stage, columns m0 .. m0 + BM: chunk c at c ^ gB(K)
            const int K = (wave * APW + i) * KPA + lane / AROW;
            const int col = m0 + (((lane % AROW) ^ gB(K)) << 3);
            aof[i] = (uint32_t)K * (uint32_t)p.lda * 2 + (uint32_t)(col < rows ? col : 0) * 2;
            continue;
        }
        const int row = (wave * APW + i) * 16 + (lane >> 2);
        const int r = m0 + row < rows ? m0 + row : rows - 1;
        const int64_t gr = map_row(r, rpb, base, stride) + ashift;
        aof[i] = (uint32_t)(gr * p.k * 2) + (((lane & 3) ^ gA<32>(row)) << 4);
    }
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
        if constexpr (TB) {
            // weight row n0 + row (its k elements contiguous), 64 bytes per stage
            const int row = (wave * BPW + i) * 16 + (lane >> 2);
            const int nr = n0 + row < p.n ? n0 + row : p.n - 1;
            bof[i] = (uint32_t)nr * (uint32_t)p.k * 2 + (((lane & 3) ^ gA<32>(row)) << 4);
            continue;
        }
        const int K = (wave * BPW + i) * KPI + lane / BROW;
        // chunk c of weight k-row K sits at c ^ gB(K) (bf16 / fp16: 8 columns per
        // chunk) or c ^ (K & 7) (int8: 16 columns per chunk)
        const int col = W8 ? n0 + (((lane % BROW) ^ (K & 7)) << 4) : n0 + (((lane % BROW) ^ gB(K)) << 3);
        bof[i] = (uint32_t)K * (uint32_t)p.n * BE + (uint32_t)(col < p.n ? col : 0) * BE;
    }
    // PA: A pair loads, 8 lanes per 128-byte row segment; chunk c of row r at c ^ gP(r)
    uint32_t aofp[PA ? APW2 : 1];
    if constexpr (PA) {
#pragma unroll
        for (int i = 0; i < APW2; ++i) {
            const int q = (wave * APW2 + i) * 64 + lane;
            const int row = q >> 3;
            const int r = m0 + row < rows ? m0 + row : rows - 1;
            const int64_t gr = map_row(r, rpb, base, stride) + ashift;
            aofp[i] = (uint32_t)(gr * p.k * 2) + (((q & 7) ^ gP(row)) << 4);
        }
    }
    // PA: activation fragment offsets in a pair block, per stage half h
    int ardp[PA ? 2 : 1][2];
    if constexpr (PA) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int row = wm * WTM + (lane & 31);
                ardp[h][ks] = row * 128 + (((h * 4 + ks * 2 + (lane >> 5)) ^ gP(row)) << 4);
            }
    }
    // PB: weight pair loads (n rows of 128-byte k segments) and fragment offsets
    uint32_t bofp[PB ? BPW2 : 1];
    int brtp[PB ? 2 : 1][2];
    if constexpr (PB) {
#pragma unroll
        for (int i = 0; i < BPW2; ++i) {
            const int q = (wave * BPW2 + i) * 64 + lane;
            const int row = q >> 3;
            const int nr = n0 + row < p.n ? n0 + row : p.n - 1;
            bofp[i] = (uint32_t)nr * (uint32_t)p.k * 2 + (((q & 7) ^ gP(row)) << 4);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int row = wn * WTN + (lane & 31);
                brtp[h][ks] = row * 128 + (((h * 4 + ks * 2 + (lane >> 5)) ^ gP(row)) << 4);
            }
    }
    // fragment offsets within a stage (the rest are immediates)
    int ard[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int row = wm * WTM + (lane & 31);
        ard[ks] = row * (BK * 2) + (((ks * 2 + (lane >> 5)) ^ gA<32>(row)) << 4);
    }
    // TA: activation fragment i read with the LDS transpose, like a weight
    // fragment (k rows of BM elements)
    int atr[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int r = lane & 15;
        const int K = (lane >> 5) * 8 + (r >> 2);
        const int col = wm * WTM + i * 32 + ((lane >> 4) & 1) * 16 + 4 * (r & 3);
        atr[i] = K * BM * 2 + (((col >> 3) ^ gB(K)) << 4) + (col & 7) * 2;
    }
    // TB: weight fragments read like activation fragments, 16 bytes per lane
    int brt[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int row = wn * WTN + (lane & 31);
        brt[ks] = A_BYTES + row * (BK * 2) + (((ks * 2 + (lane >> 5)) ^ gA<32>(row)) << 4);
    }
    int brd[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int r = lane & 15;
        if constexpr (W8) {
            // ds_read_b64_tr_b8: in each 16-lane group, lane i gets byte i % 8 of
            // the 8-byte chunks addressed by lanes 2j' + i / 8 (j' = 0..7); lane
            // 2j' + h points at k-row K0 + j', columns n0 + 8h .. + 7, so lane i
            // receives column n0 + i at k-rows K0 .. K0 + 7
            const int K = (lane >> 5) * 8 + (r >> 1);
            const int col = wn * WTN + j * 32 + ((lane >> 4) & 1) * 16 + 8 * (r & 1);
            brd[j] = A_BYTES + K * BN + (((col >> 4) ^ (K & 7)) << 4) + (col & 15);
        } else {
            const int K = (lane >> 5) * 8 + (r >> 2);
            const int col = wn * WTN + j * 32 + ((lane >> 4) & 1) * 16 + 4 * (r & 3);
            brd[j] = A_BYTES + K * BN * 2 + (((col >> 3) ^ gB(K)) << 4) + (col & 7) * 2;
        }
    }

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int KT = p.k / BK;   // >= 1 (the launcher sends k == 0 elsewhere)
    const int64_t astep = TA ? (int64_t)BK * p.lda * 2 : (int64_t)BK * 2;
    const int64_t bstep = TB ? (int64_t)BK * 2 : (int64_t)BK * p.n * BE;
    // PA: dma_b, the weights of stage kt into slot `slot`; dma_b2 (PB) and
    // dma_a2, the weights / activations of stages kt and kt + 1 (kt even) into
    // the pair block of slot `slot`
    auto dma_b = [&](int d, int kt, int slot) {
        dma16_sbase(bof[d], p.b + (int64_t)kt * bstep, lds0 + A_REG + slot * B_BYTES + (wave * BPW + d) * 1024);
    };
    auto dma_b2 = [&](int d, int kt, int slot) {
        dma16_sbase(bofp[PB ? d : 0], p.b + (int64_t)kt * bstep,
                    lds0 + A_REG + (slot >> 1) * 2 * B_BYTES + (wave * BPW2 + d) * 1024);
    };
    auto dma_a2 = [&](int d, int kt, int slot) {
        dma16_sbase(aofp[PA ? d : 0], p.a + (int64_t)kt * astep, lds0 + (slot >> 1) * 2 * A_BYTES + (wave * APW2 + d) * 1024);
    };
    auto dma = [&](int d, int kt, int slot) {
        const uint32_t l = lds0 + slot * STAGE;
        if (d < APW)
            dma16_sbase(aof[d], p.a + (int64_t)kt * astep, l + (wave * APW + d) * 1024);
        else
            dma16_sbase(bof[d - APW], p.b + (int64_t)kt * bstep, l + A_BYTES + (wave * BPW + d - APW) * 1024);
    };
    u32x4 af[2][FM], bf[2][FN];
    u32x2 bq[2][FN];   // w8: raw int8 weight fragments, converted right before use
    // fragment r of k step ks of a slot: weight fragments (two halves each, or
    // one int8 read each), then activation rows
    // h: PA, the stage's half of its pair block (kt & 1, a constant at every call)
    auto rdf = [&](int r, int slot, int ks, int buf, int h) {
        // (PA: brd holds the weight offsets past an A_BYTES stage head)
        const COC_LDS uint8_t* st = (const COC_LDS uint8_t*)sm + (PA ? A_REG + slot * B_BYTES - A_BYTES : slot * STAGE);
        if constexpr (PA) {
            if (r >= WRD * FN) {
                af[buf][r - WRD * FN] = *(const COC_LDS u32x4*)((const COC_LDS uint8_t*)sm + (slot >> 1) * 2 * A_BYTES +
                                                              ardp[h][ks] + (r - WRD * FN) * 32 * 128);
                return;
            }
        }
        if constexpr (W8) {
            if (r < FN) {
                bq[buf][r] = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((COC_LDS i32x2*)(st + brd[r] + ks * 16 * BN)));
            } else {
                af[buf][r - FN] = *(const COC_LDS u32x4*)(st + ard[ks] + (r - FN) * 32 * BK * 2);
            }
            return;
        }
        if (r < WRD * FN) {
            if constexpr (PB) {
                bf[buf][r] = *(const COC_LDS u32x4*)((const COC_LDS uint8_t*)sm + A_REG + (slot >> 1) * 2 * B_BYTES +
                                                     brtp[PB ? h : 0][ks] + r * 32 * 128);
            } else if constexpr (TB) {
                bf[buf][r] = *(const COC_LDS u32x4*)(st + brt[ks] + r * 32 * BK * 2);
            } else {
                const int j = r >> 1, h = r & 1;
                const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (COC_LDS s16x4*)(st + brd[j] + (ks * 16 + h * 4) * BN * 2));
                const u32x2 v2 = __builtin_bit_cast(u32x2, v);
                bf[buf][j][2 * h] = v2[0];
                bf[buf][j][2 * h + 1] = v2[1];
            }
        } else if constexpr (TA) {
            const int ra = r - WRD * FN, i = ra >> 1, h = ra & 1;
            const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (COC_LDS s16x4*)(st + atr[i] + (ks * 16 + h * 4) * BM * 2));
            const u32x2 v2 = __builtin_bit_cast(u32x2, v);
            af[buf][i][2 * h] = v2[0];
            af[buf][i][2 * h + 1] = v2[1];
        } else {
            af[buf][r - WRD * FN] = *(const COC_LDS u32x4*)(st + ard[ks] + (r - WRD * FN) * 32 * BK * 2);
        }
    };
    auto reads_at = [&](int s, int slot, int ks, int buf, int h) {
        if (2 * s < NRD) rdf(2 * s, slot, ks, buf, h);
        if (2 * s + 1 < NRD) rdf(2 * s + 1, slot, ks, buf, h);
    };
    auto dmas_at = [&](int s, int kt, int slot) {
#pragma unroll
        for (int d = 0; d < DPW; ++d)
            if ((d * NMM) / DPW == s) dma(d, kt, slot);
    };
    // PA: the weights of stage kt, and with APAIR the activations of stages kt, kt + 1
    auto dmas_pa = [&](int s, int kt, int slot, auto APAIR) {
        if constexpr (PB) {
            // both pairs, in odd stages only
            constexpr int ND = APW2 + BPW2;
#pragma unroll
            for (int d = 0; d < ND; ++d)
                if ((d * NMM) / ND == s) {
                    if (d < APW2) dma_a2(d, kt, slot);
                    else dma_b2(d - APW2, kt, slot);
                }
        } else {
            constexpr int NA = decltype(APAIR)::value ? APW2 : 0, ND = NA + BPW;
#pragma unroll
            for (int d = 0; d < ND; ++d)
                if ((d * NMM) / ND == s) {
                    if (d < NA) dma_a2(d, kt, slot);
                    else dma_b(d - NA, kt, slot);
                }
        }
    };

    // w8A16 scales.  Per tensor and per channel the scale is constant along k,
    // so the main loop multiplies the activations by q itself (every product
    // x * q is exact in fp32) and the epilogue multiplies the fp32 sums by the
    // scale.  Per group (group a multiple of 32, so one k-group per stage) the
    // weight is dequantised in registers: spk[j] = this lane's scale (packed
    // twice) for weight fragment j at the current stage; the tile's k / group
    // rows of BN scales sit in LDS and spn prefetches the next stage's.
    uint32_t spk[FN] = {}, spn[FN] = {};
    auto scales_of = [&](int kt, uint32_t* out) {
        const COC_LDS uint16_t* tbl = (const COC_LDS uint16_t*)((const COC_LDS uint8_t*)sm + TBL);
        const int row = kt * BK / p.group;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const uint32_t s = tbl[row * BN + wn * WTN + j * 32 + (lane & 31)];
            out[j] = s | (s << 16);
        }
    };
    // int8 fragment -> fp16: 0x6400 | (q ^ 0x80) is 1024 + q + 128 exactly, so
    // subtracting 1152 gives q exactly.  Per group one fp16 multiply by the
    // scale then rounds q * scale to nearest even, the dequantised weight.
    auto deq = [&](int buf) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const uint32_t x0 = bq[buf][j][0] ^ 0x80808080u, x1 = bq[buf][j][1] ^ 0x80808080u;
            const uint32_t d[4] = {__builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u),
                                   __builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u),
                                   __builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u),
                                   __builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u)};
            const f16x2 off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
            if constexpr (grouped) {
                const f16x2 sc = __builtin_bit_cast(f16x2, spk[j]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    bf[buf][j][e] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, d[e]) + off) * sc);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    bf[buf][j][e] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, d[e]) + off);
            }
        }
    };
    if constexpr (W8) {
        if constexpr (grouped) {
            const uint16_t* sg = (const uint16_t*)p.scales;
            // the tile's scale rows into LDS: rows of BN fp16, 8 per 16-byte vector
            uint8_t* tbl = sm + TBL;
            const int rows_t = (p.k + p.group - 1) / p.group;
            for (int v = threadIdx.x; v < rows_t * (BN / 8); v += 64 * NW) {
                const int r = v / (BN / 8), c = (v % (BN / 8)) * 8;
                const int col = n0 + c < p.n ? n0 + c : 0;
                *(u32x4*)(tbl + (r * BN + c) * 2) = *(const u32x4*)(sg + (int64_t)r * p.n + col);
            }
            __syncthreads();
            scales_of(0, spn);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" :: "v"(spk[j]), "v"(spn[j]));   // loads done before the DMA
    }

    // prologue: stages 0 .. S-2 in flight, stage 0 visible, its k step 0 read
    if constexpr (PB) {
        // pairs (0, 1) of both operands, then pairs (2, 3) (KT is even)
        for (int d = 0; d < APW2; ++d) dma_a2(d, 0, 0);
        for (int d = 0; d < BPW2; ++d) dma_b2(d, 0, 0);
        if (KT >= 4) {
            for (int d = 0; d < APW2; ++d) dma_a2(d, 2, 2);
            for (int d = 0; d < BPW2; ++d) dma_b2(d, 2, 2);
            wait_vmcnt<APW2 + BPW2>();
        } else {
            wait_vmcnt<0>();
        }
    } else if constexpr (PA) {
        // A pair (0, 1), B 0, B 1, A pair (2, 3), B 2 (KT is even); stage 0 = the first two
        for (int d = 0; d < APW2; ++d) dma_a2(d, 0, 0);
        for (int d = 0; d < BPW; ++d) dma_b(d, 0, 0);
        for (int d = 0; d < BPW; ++d) dma_b(d, 1, 1);
        if (KT >= 4) {
            for (int d = 0; d < APW2; ++d) dma_a2(d, 2, 2);
            for (int d = 0; d < BPW; ++d) dma_b(d, 2, 2);
            wait_vmcnt<2 * BPW + APW2>();
        } else {
            wait_vmcnt<0>();
        }
    } else {
        for (int s = 0; s < S - 1; ++s)
            if (s < KT)
                for (int d = 0; d < DPW; ++d) dma(d, s, s);
        if (KT >= S - 1) wait_vmcnt<(S - 2) * DPW>();
        else wait_vmcnt<0>();
    }
    block_barrier();
    for (int r = 0; r < NRD; ++r) rdf(r, 0, 0, 0, 0);

    auto stage = [&](int kt, auto LOAD, auto MORE, auto WAITN, auto APAIR, auto PAR) {
        constexpr bool load = decltype(LOAD)::value, more = decltype(MORE)::value;
        constexpr int par = decltype(PAR)::value;   // PA: kt & 1
        const int slot = kt % S;
        if constexpr (grouped) {
#pragma unroll
            for (int j = 0; j < FN; ++j) spk[j] = spn[j];
        }
        if constexpr (W8) {
            deq(0);
        }
        // Phase 1 at the low wave priority: a wave that is still in phase 2
        // while the other wave on its SIMD has moved on is the one the
        // barrier waits for, so it issues first.
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < NMM; ++s) {
            acc[s / FN][s % FN] = mfma32<KIND>(bf[0][s % FN], af[0][s / FN], acc[s / FN][s % FN]);
            reads_at(s, slot, 1, 1, par);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (more) {
            wait_vmcnt<decltype(WAITN)::value>();
            block_barrier();
        }
        __builtin_amdgcn_s_setprio(1);
        if constexpr (W8) deq(1);
        __builtin_amdgcn_sched_barrier(0);
        const int nslot = (kt + 1) % S, dslot = (kt + S - 1) % S;
#pragma unroll
        for (int s = 0; s < NMM; ++s) {
            acc[s / FN][s % FN] = mfma32<KIND>(bf[1][s % FN], af[1][s / FN], acc[s / FN][s % FN]);
            if constexpr (more) reads_at(s, nslot, 0, 0, 1 - par);
            if constexpr (load) {
                if constexpr (PA) dmas_pa(s, kt + S - 1, dslot, APAIR);
                else dmas_at(s, kt + S - 1, dslot);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (grouped) {
            if (kt + 1 < KT) scales_of(kt + 1, spn);
        }
    };
    using yes = std::true_type;
    using no = std::false_type;
    int kt = 0;
    // steady state: stages kt+2 .. kt+S-2 may stay in flight at the wait.
    // PA: stage t's phase 2 loads the weights of stage t + 3 and, for odd t, the
    // activation pair (t + 3, t + 4); at stage kt's wait the loads of stage
    // kt - 1's phase 2 may stay in flight.  PB: odd stages load both pairs
    // (t + 3, t + 4), even stages nothing.
    using even = std::integral_constant<int, 0>;
    using odd = std::integral_constant<int, 1>;
    using none = std::integral_constant<int, 0>;
    if constexpr (PB) {
        // odd stages load the next pairs of both operands (two stages ahead),
        // even stages nothing; at an even stage's wait the pairs the previous
        // odd stage loaded may stay in flight
        for (; kt + S < KT; kt += 2) {
            stage(kt, no{}, yes{}, std::integral_constant<int, APW2 + BPW2>{}, no{}, even{});
            stage(kt + 1, yes{}, yes{}, none{}, yes{}, odd{});
        }
        if (kt + S - 1 < KT) {
            stage(kt, no{}, yes{}, std::integral_constant<int, APW2 + BPW2>{}, no{}, even{});
            stage(kt + 1, no{}, yes{}, none{}, no{}, odd{});
            kt += 2;
        }
        stage(kt, no{}, yes{}, none{}, no{}, even{});
        stage(kt + 1, no{}, no{}, none{}, no{}, odd{});
    } else if constexpr (PA) {
        // KT is even: stages run in (even, odd) pairs.  In the loop both stages
        // load (one version of each, so the accumulators keep their registers);
        // then at most one pair whose even stage loads the last weights; then
        // the last pair.
        for (; kt + S < KT; kt += 2) {
            stage(kt, yes{}, yes{}, std::integral_constant<int, BPW + APW2>{}, no{}, even{});
            stage(kt + 1, yes{}, yes{}, std::integral_constant<int, BPW>{}, yes{}, odd{});
        }
        if (kt + S - 1 < KT) {
            stage(kt, yes{}, yes{}, std::integral_constant<int, BPW + APW2>{}, no{}, even{});
            stage(kt + 1, no{}, yes{}, none{}, no{}, odd{});
            kt += 2;
        }
        stage(kt, no{}, yes{}, none{}, no{}, even{});
        stage(kt + 1, no{}, no{}, none{}, no{}, odd{});
    } else {
        for (; kt + S - 1 < KT; ++kt) stage(kt, yes{}, yes{}, std::integral_constant<int, (S - 3) * DPW>{}, no{}, even{});
        for (; kt + 1 < KT; ++kt) stage(kt, no{}, yes{}, none{}, no{}, even{});
        stage(kt, no{}, no{}, none{}, no{}, even{});
    }
    __builtin_amdgcn_s_setprio(0);

    if (poison) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = __builtin_nanf("");
    }
    // w8A16 per tensor / per channel: the staging below stores sum * scale,
    // in fp32, rounded once (lane columns as there; n % 16 == 0 on this path,
    // so a group of four columns is wholly in range or wholly out).
    constexpr bool SCALED = W8 && !grouped;
    float sc[SCALED ? FN : 1][4][4];
    if constexpr (SCALED) {
        const uint16_t* sg = (const uint16_t*)p.scales;
        if (p.qmode == COC_PER_CHANNEL) {
            // (an opaque lane copy, as for the staging addresses below)
            int sl;
            asm volatile("v_mov_b32 %0, %1" : "=v"(sl) : "v"(lane));
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = n0 + wn * WTN + j * 32 + q * 8 + (sl >> 5) * 4;
                    const u32x2 v = col < p.n ? *(const u32x2*)(sg + col) : u32x2{0, 0};
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        sc[j][q][t] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[t >> 1] >> (16 * (t & 1))));
                }
        } else {
            const float s0 = (float)__builtin_bit_cast(_Float16, sg[0]);
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int t = 0; t < 4; ++t) sc[j][q][t] = s0;
        }
    }
    auto outv = [&](int i, int j, int q, int t) {
        if constexpr (SCALED) return acc[i][j][q * 4 + t] * sc[j][q][t];
        else return acc[i][j][q * 4 + t];
    };

    // Epilogue through LDS.  A lane holds n = q*8 + (lane/32)*4 + {0..3} of row
    // m = lane%32 in each 32 x 32 block; stored directly that gives 16-byte
    // pieces of 32 rows per instruction.  Instead each wave (once the whole
    // workgroup is off the ring) writes its WTM x WTN tile, in the storage
    // dtype, into its own LDS region (rows of WTN*2 bytes, 16-byte chunk c of
    // row r at c ^ (r & 7)) and reads it back 16 bytes per lane, WTN/8 lanes
    // per row: every store instruction then writes whole rows of WTN*2
    // contiguous bytes (whole 128-byte lines).
    constexpr int RP = WTN * 2;     // staged row pitch (bytes)
    constexpr int CPR = WTN / 8;    // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;   // rows per store instruction
    static_assert(CPR % 8 == 0 && 64 % CPR == 0 && WTM % RPI == 0, "staging layout");
    static_assert(NW * WTM * RP <= ring_lds_bytes<BM, BN, S, WM, WN, KIND>(), "staging fits in the LDS");
    block_barrier();
    // An opaque copy of the lane index: in the chunk-walking kernel the
    // compiler would otherwise hoist these lane-only LDS addresses out of the
    // tile loop and hold them in registers through the main loop.
    int el;
    asm volatile("v_mov_b32 %0, %1" : "=v"(el) : "v"(lane));
    COC_LDS uint8_t* stg = (COC_LDS uint8_t*)sm + wave * (WTM * RP);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = i * 32 + (el & 31);
                u32x2 v;
                v[0] = pack2<OUT_DT>(outv(i, j, q, 0), outv(i, j, q, 1));
                v[1] = pack2<OUT_DT>(outv(i, j, q, 2), outv(i, j, q, 3));
                *(COC_LDS u32x2*)(stg + row * RP + (((j * 4 + q) ^ (row & 7)) << 4) + (el >> 5) * 8) = v;
            }
    // (keeps the store addresses below from being computed while the
    // accumulators are still live)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < WTM / RPI; ++t) {
        const int row = t * RPI + el / CPR, ch = el % CPR;
        const u32x4 v = *(const COC_LDS u32x4*)(stg + row * RP + ((ch ^ (row & 7)) << 4));
        const int r = m0 + wm * WTM + row, col = n0 + wn * WTN + ch * 8;
        if (r < rows && col < p.n) {
            const int64_t off = map_row(r, rpb, base, stride) * (int64_t)p.n * 2 + (int64_t)col * 2;
            if constexpr (SYS)
                store16_sys(sys_rsrc(p.c), (uint32_t)off, v);
            else
                *(u32x4*)(p.c + off) = v;
        }
    }
}

// ------------------------------------------------------------------ four-wave tile
// The 256 x 256 tile of the bf16 / fp16 launches with transposed weights (W
// stored n x k, so both operands are k-contiguous) that share no CU with
// another kernel (no counter to signal, no wait except for rows the launch
// copies itself), k % 64 == 0: four waves
// of 128 x 128 (2 x 2), v_mfma_f32_16x16x32 (16 rows or columns by 32 k per
// instruction, where ring_tile's v_mfma_f32_32x32x16 takes 32 by 16).  Per
// 32 k the four waves read 64 KB of LDS fragments where ring_tile's eight
// 128 x 64 waves read 96 KB.  One workgroup per CU uses nearly the whole
// register file (one wave per SIMD), so nothing that must share a CU with the
// matmul (a reduce waiting on its counters, a copy whose rows it waits for)
// can run beside it: such launches keep ring_tile.  Both tiles add each output's products
// in the same 8-k steps in increasing k (the MFMA shapes differ only in how
// many steps one instruction takes), so they give the same bits, and no
// result depends on which one ran.
//
// k runs in 64-k stages (whole 128-byte rows of both operands) through two
// LDS slots of 64 KB: the activations as 256 rows of 128 bytes (chunk c of
// row r at c ^ gP(r)), then the weights as 256 n rows of 128 bytes the same
// way.  Within a stage two k steps of 32; each step's 16 fragment reads (one
// activation and eight weight fragments, then seven activation fragments:
// first-use order) run under the previous step's 64 MFMAs.  The barrier sits
// BAR_AT MFMAs into a stage's second step: after it the next stage's
// fragments are read and the stage after next is loaded into the slot just
// read, spread one load every DSTEP MFMAs (its remaining loads go in the next
// stage's first step).
constexpr int kQuadSlot = 256 * 64 * 2 * 2;   // activations + weights of one 64-k stage
constexpr int kQuadLds = 2 * kQuadSlot;        // 128 KB

template <int KIND>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (KIND == GK_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                       0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
}

template <int KIND, bool SYS>
__device__ __forceinline__ void quad_tile(const GemmParams& p, int rows, int rpb, int64_t base, int64_t stride,
                                          int64_t ashift, int m0, int n0, uint8_t* sm, bool poison) {
    constexpr int BK = 64;
    constexpr int A_ST = 256 * BK * 2;   // 32 KB of activations per stage
    constexpr int OUT_DT = (KIND == GK_BF16) ? COC_BF16 : COC_F16;
    constexpr int BAR_AT = 16, DSTEP = 4;
    constexpr int DSPLIT = (64 - BAR_AT + DSTEP - 1) / DSTEP > 16 ? 16 : (64 - BAR_AT + DSTEP - 1) / DSTEP;
    // An opaque copy of the lane index: in a loop over tiles the compiler
    // would otherwise compute every lane-only offset once, before the loop,
    // and hold them all in registers through it (spilling the k loop's).
    int lane;
    asm volatile("v_and_b32 %0, 63, %1" : "=v"(lane) : "v"(threadIdx.x));
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const uint32_t lds0 = lds_u32(sm);

    // loads: each of a wave's 8 activation instructions covers 8 rows of 128
    // bytes, and each of its 8 weight instructions 8 n rows of 128 bytes
    uint32_t aof[8], bof[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = (wave * 8 + i) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ gP(row);
        const int r = m0 + row < rows ? m0 + row : rows - 1;
        const int64_t gr = map_row(r, rpb, base, stride) + ashift;
        aof[i] = (uint32_t)(gr * p.k * 2) + (uint32_t)(c * 16);
        const int nr = n0 + row < p.n ? n0 + row : p.n - 1;
        bof[i] = (uint32_t)nr * (uint32_t)p.k * 2 + (uint32_t)(c * 16);
    }
    auto issue = [&](int d, int kt, int slot) {
        const uint32_t l = lds0 + slot * kQuadSlot;
        if (d < 8) dma16_sbase(aof[d], p.a + (int64_t)kt * BK * 2, l + (wave * 8 + d) * 1024);
        else dma16_sbase(bof[d - 8], p.b + (int64_t)kt * BK * 2, l + A_ST + (wave * 8 + d - 8) * 1024);
    };

    // fragments: lane l holds row (activations) or column (weights) l % 16
    // of its 16-wide block, k 8 (l / 16) .. + 7 of the 32-k step
    const int arow = wm * 128 + (lane & 15), brow = wn * 128 + (lane & 15);
    u32x4 af[2][8], bf[2][8];
    auto read_a = [&](int slot, int ks, int buf, int i) {
        const int c = (ks * 4 + (lane >> 4)) ^ gP(arow);   // gP has a 16-row period
        af[buf][i] = *(const COC_LDS u32x4*)((const COC_LDS uint8_t*)sm + slot * kQuadSlot + (arow + i * 16) * 128 +
                                            c * 16);
    };
    auto read_b = [&](int slot, int ks, int buf, int j) {
        const int c = (ks * 4 + (lane >> 4)) ^ gP(brow);
        bf[buf][j] = *(const COC_LDS u32x4*)((const COC_LDS uint8_t*)sm + slot * kQuadSlot + A_ST + (brow + j * 16) * 128 +
                                            c * 16);
    };
    // read r of a k step's 16, in first-use order: A0, B0 .. B7, A1 .. A7
    auto read_r = [&](int r, int slot, int ks, int buf) {
        if (r == 0) read_a(slot, ks, buf, 0);
        else if (r < 9) read_b(slot, ks, buf, r - 1);
        else read_a(slot, ks, buf, r - 8);
    };

    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int KT = p.k / BK;   // >= 1 (quad_core requires k % 64 == 0)
    for (int d = 0; d < 16; ++d) issue(d, 0, 0);
    if (KT > 1) {
        for (int d = 0; d < 16; ++d) issue(d, 1, 1);
        wait_vmcnt<16>();
    } else {
        wait_vmcnt<0>();
    }
    block_barrier();
    for (int r = 0; r < 16; ++r) read_r(r, 0, 0, 0);

    // MORE: a next stage to read; LOAD2: stage kt + 2 to load; REST: the
    // remaining loads of stage kt + 1 (its first DSPLIT went in stage kt - 1)
    auto stage = [&](int kt, auto MORE, auto LOAD2, auto REST) {
        constexpr bool more = decltype(MORE)::value, load2 = decltype(LOAD2)::value;
        constexpr bool rest = decltype(REST)::value;
        const int slot = kt & 1, nslot = slot ^ 1;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 64; ++s) {
            acc[s >> 3][s & 7] = mfma16<KIND>(bf[0][s & 7], af[0][s >> 3], acc[s >> 3][s & 7]);
            if (s < 16) read_r(s, slot, 1, 1);
            if constexpr (rest) {
                const int g = 64 + s - BAR_AT;
                if (g % DSTEP == 0) {
                    const int d = g / DSTEP;
                    if (d >= DSPLIT && d < 16) issue(d, kt + 1, nslot);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int s = 0; s < BAR_AT; ++s) {
            acc[s >> 3][s & 7] = mfma16<KIND>(bf[1][s & 7], af[1][s >> 3], acc[s >> 3][s & 7]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (more) {
            wait_vmcnt<0>();
            block_barrier();
        }
#pragma unroll
        for (int s = BAR_AT; s < 64; ++s) {
            acc[s >> 3][s & 7] = mfma16<KIND>(bf[1][s & 7], af[1][s >> 3], acc[s >> 3][s & 7]);
            if constexpr (more) {
                if (s - BAR_AT < 16) read_r(s - BAR_AT, nslot, 0, 0);
            }
            if constexpr (load2) {
                const int g = s - BAR_AT;
                if (g % DSTEP == 0 && g / DSTEP < DSPLIT) issue(g / DSTEP, kt + 2, slot);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using yes = std::true_type;
    using no = std::false_type;
    int kt = 0;
    if (KT > 2) {
        stage(0, yes{}, yes{}, no{});
        for (kt = 1; kt + 2 < KT; ++kt) stage(kt, yes{}, yes{}, yes{});
        stage(kt, yes{}, no{}, yes{});
        ++kt;
    } else if (KT == 2) {
        stage(0, yes{}, no{}, no{});
        ++kt;
    }
    stage(kt, no{}, no{}, no{});

    if (poison) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                                         __builtin_nanf("")};
    }

    // Epilogue through LDS: lane l of block (i, j) holds rows m = i*16 + l%16,
    // columns n = j*16 + (l/16)*4 + 0..3.  Each wave stages its 128 x 128 tile
    // in the storage dtype (rows of 256 bytes, 16-byte chunk c of row r at
    // c ^ (r & 15)), then stores whole 256-byte rows, 16 bytes per lane.
    block_barrier();
    int el;
    asm volatile("v_mov_b32 %0, %1" : "=v"(el) : "v"(lane));   // (see ring_tile's epilogue)
    COC_LDS uint8_t* stg = (COC_LDS uint8_t*)sm + wave * (128 * 256);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row = i * 16 + (el & 15);
            const int col = j * 16 + (el >> 4) * 4;
            u32x2 v;
            v[0] = pack2<OUT_DT>(acc[i][j][0], acc[i][j][1]);
            v[1] = pack2<OUT_DT>(acc[i][j][2], acc[i][j][3]);
            *(COC_LDS u32x2*)(stg + row * 256 + (((col >> 3) ^ (row & 15)) << 4) + (col & 7) * 2) = v;
        }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 32; ++t) {
        const int row = t * 4 + (el >> 4), ch = el & 15;
        const u32x4 v = *(const COC_LDS u32x4*)(stg + row * 256 + ((ch ^ (row & 15)) << 4));
        const int r = m0 + wm * 128 + row, col = n0 + wn * 128 + ch * 8;
        if (r < rows && col < p.n) {
            const int64_t off = map_row(r, rpb, base, stride) * (int64_t)p.n * 2 + (int64_t)col * 2;
            if constexpr (SYS)
                store16_sys(sys_rsrc(p.c), (uint32_t)off, v);
            else
                *(u32x4*)(p.c + off) = v;
        }
    }
}

template <int BM, int BN, int S, int WM, int WN, int KIND>
__global__ __launch_bounds__(64 * WM * WN) void gemm_ring(GemmParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t sm[ring_lds_bytes<BM, BN, S, WM, WN, KIND>()];
    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, &tm, &tn);
    ring_tile<BM, BN, S, WM, WN, KIND>(p, p.rows, p.rpb, p.base, p.stride, 0, tm * BM, tn * BN, sm, false);
}

// ------------------------------------------------------------------ gather
// dst row g (g in [row0, row0 + rows)) = row g % shard_rows of shard
// g / shard_rows; 16-byte vector copies.
struct GatherParams {
    const uint8_t* src[COC_MAX_WORLD];
    uint8_t* dst;
    int64_t row_bytes;   // k * element size
    int32_t shard_rows;
    int32_t row0;
    int32_t vpr;
    int32_t total;
    uint32_t* signal;    // if set, each workgroup adds 1 when its rows are stored
    uint64_t* stamps;    // activity records (measurement; may be NULL)
};

// Vector v of the rows from row0 on.  p must be the kernel argument itself
// (not a copy): src[s] then loads from the argument segment instead of
// making a private copy of the pointer array.
__device__ __forceinline__ const uint8_t* gather_src(const GatherParams& p, int row0, int v, int64_t* off) {
    const int row = v / p.vpr;
    const int cv = v - row * p.vpr;
    const int g = row0 + row;
    const int s = g / p.shard_rows;
    const int local = g - s * p.shard_rows;
    *off = (int64_t)g * p.row_bytes + (int64_t)cv * 16;
    return p.src[s] + (int64_t)local * p.row_bytes + (int64_t)cv * 16;
}

// Chunk-walking form of the ring kernel: one launch covers every chunk of an
// op, as a list of pieces (see ChunksLaunch).  8 * per_xcd workgroups (one per
// CU for the 256-wide tiles, two for 128 x 128); workgroup b runs on XCD b % 8
// and walks that XCD's tile list (piece by piece in order, within a piece the
// XCD's run of xcd_tile's split in grouped order) as schedule_item assigns
// it.  A piece can wait for a group of ready counters before its first tile;
// with SIGNAL, tiles are stored write-through and add 1 to their piece's done
// counter.  Gathered rows are read through the L2 as usual: no line of a piece
// can be cached before its wait (rows are whole 128-byte lines and nothing
// reads them earlier in this launch), and the gather writes them through.
//
// Fused all-gather: the launch copies the chunks' rows into the gathered
// matrix itself, chunk by chunk, adding 1 to a chunk's ready lines after each
// share of it.  Chunks [0, early), which the first tiles of the two-tile
// workgroups (below) read, are copied by every workgroup before its first
// tile, so those tiles start together; the rest by the workgroups that own a
// single tile of the last two rounds, which have a tile's time to spare.
struct FusedGather {
    GatherParams p;                    // src, dst, row_bytes, shard_rows, vpr (row0 / total per chunk)
    // a chunk's rows: from row0[c], total[c] vectors, then from row0b[c],
    // totalb[c] vectors (0: none)
    int32_t row0[COC_MAX_SPLIT], total[COC_MAX_SPLIT];
    int32_t row0b[COC_MAX_SPLIT], totalb[COC_MAX_SPLIT];
    int32_t nchunks, early, gatherers; // gatherers == 0: no fused gather
};

struct PersistParams {
    GemmParams g;   // c, n, k, tiles_n (a, b and the row map fields unused)
    const uint8_t* a[kMaxPieces];
    const uint8_t* b[kMaxPieces];   // per piece: one expert's weights in a grouped matmul
    int64_t ashift[kMaxPieces], base[kMaxPieces], stride[kMaxPieces];
    int32_t rpb[kMaxPieces], rows[kMaxPieces], tiles_m[kMaxPieces];
    int32_t wait[kMaxPieces], signal[kMaxPieces];
    uint32_t ready_target[COC_MAX_SPLIT];
    int32_t npieces, per_xcd;
    int32_t order;   // 0: whole rounds in list order; 1: two-tile workgroups first (schedule_item)
    uint32_t spin_limit;   // polls before a wait gives up (the tile is then NaN)
    uint32_t* gave_up;     // set by a wait that gives up (may be NULL)
    uint32_t* done;
    uint32_t* ready;
    uint64_t* stamps;      // activity records (measurement; may be NULL)
    FusedGather fg;
};

// Share gi of ng of chunks [c0, c1), 16 vectors per thread in flight (the
// matmul's registers are free before its first tile), stores written through
// for the other XCDs' matmul workgroups; then 1 added to the chunk's ready
// lines.
__device__ __forceinline__ void fused_gather(const FusedGather& F, int c0, int c1, int gi, int ng, uint32_t* ready) {
    constexpr int U = 16;
    const int nt = blockDim.x;
    const GatherParams& p = F.p;
    for (int c = c0; c < c1; ++c) {
        const uint64_t t0 = p.stamps ? realtime() : 0;
        // the chunk's two row ranges as one run of vectors
        const int row0 = F.row0[c], ta = F.total[c], row0b = F.row0b[c], total = ta + F.totalb[c];
        const int v0 = (int)((int64_t)gi * total / ng), v1 = (int)((int64_t)(gi + 1) * total / ng);
        for (int b = v0 + (int)threadIdx.x; b < v1; b += U * nt) {
            u32x4 x[U];
            int64_t off[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = b + u * nt;
                const bool second = v >= ta;
                if (v < v1) x[u] = load16_stream(gather_src(p, second ? row0b : row0, second ? v - ta : v, &off[u]));
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (b + u * nt >= v1) break;
                store16_sys(sys_rsrc(p.dst), (uint32_t)off[u], x[u]);
            }
        }
        wg_signal(ready + (c * kReadyLines + gi % kReadyLines) * kSyncWords);
        if (p.stamps) stamp(p.stamps, blockIdx.x * (1 + F.nchunks) + 1 + c, kStampGather | (c << 8), t0, realtime());
    }
}

// QUAD: 256 x 256 tiles of quad_tile (four waves, WM = WN = 2; transposed
// weights, nothing to signal, waits only on the launch's own copy).
template <int BM, int BN, int S, int WM, int WN, int KIND, bool SIGNAL, bool TA = false, bool TB = false,
          bool PA = false, bool QUAD = false>
__global__ __launch_bounds__(64 * WM * WN) void gemm_ring_chunks(PersistParams P) {
    static_assert(!QUAD || (BM == 256 && BN == 256 && WM == 2 && WN == 2 && TB && !TA && !SIGNAL),
                  "four-wave tile shape");
    __shared__ __attribute__((aligned(1024))) uint8_t sm[QUAD ? kQuadLds : ring_lds_bytes<BM, BN, S, WM, WN, KIND>()];
    constexpr int NX = 8;
    const int x = blockIdx.x % NX, w = blockIdx.x / NX;
    const int tn_all = P.g.tiles_n;
    const int l = xcd_items(P.tiles_m, tn_all, P.npieces, x);
    if (P.fg.gatherers > 0) {
        int first = -1;
        const int before = singles_before(P.tiles_m, tn_all, P.npieces, P.per_xcd, x, &first);
        fused_gather(P.fg, 0, P.fg.early, blockIdx.x, gridDim.x, P.ready);
        if (first >= 0 && w >= first)
            fused_gather(P.fg, P.fg.early, P.fg.nchunks, before + (w - first), P.fg.gatherers, P.ready);
    }
    int waited = -1;
    bool ok = true;
    uint64_t t_first = 0;
    for (int s = 0;; ++s) {
        // order 0 finishes the list's chunks in order (a compute-first op
        // hands each chunk to its reduce as early as possible)
        const int j = P.order == 0 ? inorder_item(l, P.per_xcd, w, s) : schedule_item(l, P.per_xcd, w, s);
        if (j < 0) break;
        int jj = 0;
        const int c = piece_of_item(P.tiles_m, tn_all, P.npieces, x, j, &jj);
        if (c >= P.npieces) break;
        const int T = P.tiles_m[c] * tn_all;
        int tm, tn;
        grouped_coords(x * (T / NX) + (x < T % NX ? x : T % NX) + jj, P.tiles_m[c], tn_all, &tm, &tn);
        const int wi = P.wait[c];
        if (P.ready != nullptr && wi >= 0 && wi != waited) {
            ok = wg_wait(P.ready + wi * kReadyLines * kSyncWords, kReadyLines, P.ready_target[wi], P.spin_limit,
                         P.gave_up);
            waited = wi;
        }
        // the previous tile's stores are done and every wave is off the LDS ring
        wait_vmcnt<0>();
        block_barrier();
        if (P.stamps != nullptr && t_first == 0) t_first = realtime();
        GemmParams g = P.g;
        g.a = P.a[c];
        g.b = P.b[c];
        if constexpr (QUAD)
            quad_tile<KIND, false>(g, P.rows[c], P.rpb[c], P.base[c], P.stride[c], P.ashift[c], tm * BM, tn * BN, sm,
                                   wi >= 0 && !ok);
        else
            ring_tile<BM, BN, S, WM, WN, KIND, SIGNAL, TA, TB, PA>(g, P.rows[c], P.rpb[c], P.base[c], P.stride[c],
                                                                   P.ashift[c], tm * BM, tn * BN, sm, wi >= 0 && !ok);
        if constexpr (SIGNAL) {
            if (P.signal[c] >= 0) wg_signal(P.done + P.signal[c] * kSyncWords);
        }
    }
    if (P.stamps != nullptr && t_first != 0)
        stamp(P.stamps, blockIdx.x * (1 + P.fg.nchunks), kStampMatmul, t_first, realtime());
}

// ------------------------------------------------------------------ fp32 GEMM
// 64 x 64 x 16 tiles, 256 threads, 4 x 4 outputs per thread, fused
// multiply-add in k order (binary32 throughout).
__global__ __launch_bounds__(256) void gemm_f32(GemmParams p) {
    constexpr int BM = 64, BN = 64, BK = 16;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[BK][BN + 4];
    const int t = threadIdx.x;
    const int tx = t & 15, ty = t >> 4;
    const int tm = blockIdx.x % p.tiles_m, tn = blockIdx.x / p.tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;

    const int ar = t >> 2, akc = (t & 3) * 4;
    const bool arv = m0 + ar < p.rows;
    const float* arow =
        (const float*)p.a + (arv ? map_row(m0 + ar, p.rpb, p.base, p.stride) : 0) * (int64_t)p.k;
    const int bkr = t >> 4, bcol = n0 + (t & 15) * 4;
    const bool bcv = bcol < p.n;

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

    for (int k0 = 0; k0 < p.k; k0 += BK) {
        f32x4 va = {0, 0, 0, 0};
        if (arv && k0 + akc < p.k) va = *(const f32x4*)(arow + k0 + akc);
        f32x4 vb = {0, 0, 0, 0};
        if (bcv && k0 + bkr < p.k) vb = *(const f32x4*)((const float*)p.b + (int64_t)(k0 + bkr) * p.n + bcol);
#pragma unroll
        for (int e = 0; e < 4; ++e) As[akc + e][ar] = va[e];
#pragma unroll
        for (int e = 0; e < 4; ++e) Bs[bkr][(t & 15) * 4 + e] = vb[e];
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
    const int col = n0 + tx * 4;
    if (col >= p.n) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = m0 + ty * 4 + i;
        if (r >= p.rows) continue;
        float* crow = (float*)p.c + map_row(r, p.rpb, p.base, p.stride) * (int64_t)p.n;
        *(f32x4*)(crow + col) = f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
    }
}

// ------------------------------------------------------------------ reduce
// dst[dst_row0 + r][:] = round(sum_{s=0}^{nsrc-1} src[s][src_row0 + r][:]),
// binary32 accumulation in ascending source order.  One 16-byte vector per
// thread per step (8 x 16-bit or 4 x 32-bit elements); the loads of all
// sources are issued before the adds.
struct ReduceParams {
    const uint8_t* src[COC_MAX_WORLD];
    uint8_t* dst;
    int64_t src_row0, dst_row0;
    int64_t row_bytes;   // n * element size
    int32_t nsrc;
    int32_t vpr;         // 16-byte vectors per row
    int32_t total;       // rows * vpr
    uint64_t* stamps;    // activity records (measurement; may be NULL)
};

// Chunk list of the waiting reduce, in pipeline order.
struct ReduceChunks {
    int64_t src_row0[COC_MAX_SPLIT], dst_row0[COC_MAX_SPLIT];
    int32_t total[COC_MAX_SPLIT];     // rows * vpr
    uint32_t target[COC_MAX_SPLIT];
    const uint32_t* done;
    int32_t nchunks, own;
    uint32_t spin_limit;   // polls before a wait gives up (rows then NaN)
    uint32_t* gave_up;     // set by a wait that gives up (may be NULL)
};

// Two sources are loaded at a time and added in rank order before the next
// pair is fetched (scheduling fences keep the compiler from hoisting all
// loads), which keeps the kernel at 32 VGPRs or fewer: the 256x256 matmul
// leaves about that much per SIMD lane free, so reduce waves can share a
// compute unit with a running matmul instead of waiting for it to drain.
template <int DT>
__device__ __forceinline__ void acc_add(float* acc, u32x4 x) {
    if constexpr (DT == COC_F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = acc[e] + __uint_as_float(x[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] = acc[2 * e] + unpack_lo<DT>(x[e]);
            acc[2 * e + 1] = acc[2 * e + 1] + unpack_hi<DT>(x[e]);
        }
    }
}

template <int DT>
__global__ __launch_bounds__(256) void reduce_rows(ReduceParams p) {
    constexpr int E = (DT == COC_F32) ? 4 : 8;
    const int stride = gridDim.x * 256;
    const uint64_t t0 = p.stamps ? realtime() : 0;
    for (int v = blockIdx.x * 256 + threadIdx.x; v < p.total; v += stride) {
        const int row = v / p.vpr;
        const int cv = v - row * p.vpr;
        const int64_t so = (p.src_row0 + row) * p.row_bytes + (int64_t)cv * 16;
        const int64_t dof = (p.dst_row0 + row) * p.row_bytes + (int64_t)cv * 16;
        // binary32 left-to-right sum of the sources in rank order: acc = src0,
        // then acc += src1, acc += src2, ...
        float acc[E];
        {
            const u32x4 x0 = load16_stream(p.src[0] + so);
            u32x4 x1 = {0, 0, 0, 0};
            if (p.nsrc > 1) x1 = load16_stream(p.src[1] + so);
            if constexpr (DT == COC_F32) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = __uint_as_float(x0[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] = unpack_lo<DT>(x0[e]);
                    acc[2 * e + 1] = unpack_hi<DT>(x0[e]);
                }
            }
            if (p.nsrc > 1) acc_add<DT>(acc, x1);
        }
#pragma unroll
        for (int s = 2; s < COC_MAX_WORLD; s += 2) {
            __builtin_amdgcn_sched_barrier(0);
            if (s < p.nsrc) {
                const u32x4 x0 = load16_stream(p.src[s] + so);
                u32x4 x1 = {0, 0, 0, 0};
                if (s + 1 < p.nsrc) x1 = load16_stream(p.src[s + 1] + so);
                acc_add<DT>(acc, x0);
                if (s + 1 < p.nsrc) acc_add<DT>(acc, x1);
            }
        }
        u32x4 out;
        if constexpr (DT == COC_F32) {
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = __float_as_uint(acc[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = pack2<DT>(acc[2 * e], acc[2 * e + 1]);
        }
        *(u32x4*)(p.dst + dof) = out;
    }
    if (p.stamps) stamp(p.stamps, blockIdx.x, kStampReduce, t0, realtime());
}


// The reduce that runs beside the one-launch matmul: one launch walks the
// chunks in pipeline order, each workgroup waiting for chunk c's tiles before
// its share of chunk c's rows.  The partial written meanwhile (source `own`)
// is read with system-scope loads.  At most one workgroup per CU, so however
// the hardware orders the two launches every CU keeps room for the matmul's
// workgroup (the waits could otherwise hold slots the matmul needs).  To keep
// HBM busy with that few waves, each thread loads all sources of two 16-byte
// vectors before adding them (same rank order, same binary32 sums).
template <int DT>
__device__ __forceinline__ void load_sources(const ReduceParams& p, int own, int64_t so, u32x4* x) {
#pragma unroll
    for (int s = 0; s < COC_MAX_WORLD; ++s)
        if (s < p.nsrc) x[s] = s == own ? load16_sys(p.src[s] + so) : load16_stream(p.src[s] + so);
}

template <int DT>
__device__ __forceinline__ u32x4 sum_sources(const ReduceParams& p, const u32x4* x) {
    constexpr int E = (DT == COC_F32) ? 4 : 8;
    float acc[E];
    if constexpr (DT == COC_F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __uint_as_float(x[0][e]);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] = unpack_lo<DT>(x[0][e]);
            acc[2 * e + 1] = unpack_hi<DT>(x[0][e]);
        }
    }
#pragma unroll
    for (int s = 1; s < COC_MAX_WORLD; ++s)
        if (s < p.nsrc) acc_add<DT>(acc, x[s]);
    u32x4 out;
    if constexpr (DT == COC_F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = __float_as_uint(acc[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = pack2<DT>(acc[2 * e], acc[2 * e + 1]);
    }
    return out;
}

// The same sum for a launch that runs alone (after the matmul, or the serial
// form): workgroup b takes the contiguous vectors [b * per, (b + 1) * per),
// and each thread loads every source of U vectors (non-temporal) before
// adding any, so 8 U 16-byte loads are in flight per thread: the reduce is
// bound by the bytes in flight, not by arithmetic.  Same rank order, same
// binary32 sums, same bits as reduce_rows.
template <int DT, int U>
__global__ __launch_bounds__(256) void reduce_rows_wide(ReduceParams p, int per) {
    const uint64_t t0 = p.stamps ? realtime() : 0;
    const int b0 = blockIdx.x * per;
    const int b1 = b0 + per < p.total ? b0 + per : p.total;
    for (int v0 = b0 + (int)threadIdx.x; v0 < b1; v0 += U * 256) {
        u32x4 x[U][COC_MAX_WORLD];
        int64_t dof[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * 256;
            if (v < b1) {
                const int row = v / p.vpr;
                const int cv = v - row * p.vpr;
                const int64_t so = (p.src_row0 + row) * p.row_bytes + (int64_t)cv * 16;
                dof[u] = (p.dst_row0 + row) * p.row_bytes + (int64_t)cv * 16;
#pragma unroll
                for (int s2 = 0; s2 < COC_MAX_WORLD; ++s2)
                    if (s2 < p.nsrc) x[u][s2] = load16_stream(p.src[s2] + so);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (v0 + u * 256 < b1) store16_stream(p.dst + dof[u], sum_sources<DT>(p, x[u]));
    }
    if (p.stamps) stamp(p.stamps, blockIdx.x, kStampReduce, t0, realtime());
}

// U = 2: two vectors per thread (~100 VGPRs); U = 1 (~50 VGPRs) beside a
// matmul that leaves less room.  One workgroup per CU: with 128 or 64 the
// reduce ran longer beside the matmul without speeding it up (BLOOM-176B
// 409 / 488 against 401 us).  Streaming stores for the output (nothing in the
// op reads it again): 0.3-0.6 % faster ops.
template <int DT, int U>
__global__ __launch_bounds__(256) void reduce_chunks_wait(ReduceParams p, ReduceChunks C) {
    const int stride = gridDim.x * 256;
    for (int c = 0; c < C.nchunks; ++c) {
        if (c > 0) __syncthreads();   // wg_wait's flag is reused
        const bool ok = wg_wait(C.done + c * kSyncWords, 1, C.target[c], C.spin_limit, C.gave_up);
        const uint64_t t0 = p.stamps ? realtime() : 0;
        const int total = C.total[c];
        for (int v = blockIdx.x * 256 + threadIdx.x; v < total; v += U * stride) {
            const int v2 = v + stride;
            const bool two = U == 2 && v2 < total;
            const int row = v / p.vpr, row2 = v2 / p.vpr;
            const int64_t so = (C.src_row0[c] + row) * p.row_bytes + (int64_t)(v - row * p.vpr) * 16;
            const int64_t so2 = (C.src_row0[c] + row2) * p.row_bytes + (int64_t)(v2 - row2 * p.vpr) * 16;
            u32x4 x[COC_MAX_WORLD], y[COC_MAX_WORLD];
            load_sources<DT>(p, C.own, so, x);
            if (two) load_sources<DT>(p, C.own, so2, y);
            const u32x4 nan = u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};   // NaN in every format
            const u32x4 o = ok ? sum_sources<DT>(p, x) : nan;
            store16_stream(p.dst + (C.dst_row0[c] + row) * p.row_bytes + (int64_t)(v - row * p.vpr) * 16, o);
            if (two) {
                const u32x4 o2 = ok ? sum_sources<DT>(p, y) : nan;
                store16_stream(p.dst + (C.dst_row0[c] + row2) * p.row_bytes + (int64_t)(v2 - row2 * p.vpr) * 16, o2);
            }
        }
        if (p.stamps) stamp(p.stamps, blockIdx.x * C.nchunks + c, kStampReduce | (c << 8), t0, realtime());
    }
}

// ------------------------------------------------------------------ gather
// (GatherParams and gather_src sit above the chunk-walking matmul, which can
// also run the copy itself.)  Four 16-byte vectors per thread per pass, all
// loaded before any is stored: beside a running matmul only a few gather
// waves fit on each CU, and the copy rate is set by the bytes in flight.
__global__ __launch_bounds__(256) void gather_rows(GatherParams p) {
    constexpr int U = 4;
    const int stride = gridDim.x * 256;
    const uint64_t t0 = p.stamps ? realtime() : 0;
    for (int v0 = blockIdx.x * 256 + threadIdx.x; v0 < p.total; v0 += U * stride) {
        u32x4 x[U];
        int64_t off[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * stride;
            if (v < p.total) x[u] = load16_stream(gather_src(p, p.row0, v, &off[u]));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (v0 + u * stride >= p.total) break;
            if (p.signal != nullptr)
                store16_sys(sys_rsrc(p.dst), (uint32_t)off[u], x[u]);   // read by a matmul already running
            else
                *(u32x4*)(p.dst + off[u]) = x[u];
        }
    }
    if (p.signal != nullptr) wg_signal(p.signal + (blockIdx.x % kReadyLines) * kSyncWords);
    if (p.stamps) stamp(p.stamps, blockIdx.x, kStampGather, t0, realtime());
}

// Every chunk of an all-gather in one launch: workgroups [c*per_chunk,
// (c+1)*per_chunk) copy chunk c (rows row0[c] .. row0[c] + rows[c]) and then
// add 1 to that chunk's ready lines.  Workgroups are dispatched in id order,
// so chunk 0's rows land first, without a kernel boundary between chunks.
struct GatherChunks {
    int32_t row0[COC_MAX_SPLIT], total[COC_MAX_SPLIT];   // first row; rows * vpr
    uint32_t* ready;                                      // chunk c's lines at c * kReadyLines
    int32_t per_chunk;
};

__global__ __launch_bounds__(256) void gather_chunks(GatherParams p, GatherChunks C) {
    constexpr int U = 4;
    const int c = blockIdx.x / C.per_chunk, lb = blockIdx.x % C.per_chunk;
    const int total = C.total[c];
    const int per = (total + C.per_chunk - 1) / C.per_chunk;   // vectors of this workgroup
    const int v_end = (lb + 1) * per < total ? (lb + 1) * per : total;
    const int row0 = C.row0[c];
    const uint64_t t0 = p.stamps ? realtime() : 0;
    for (int v0 = lb * per + threadIdx.x; v0 < v_end; v0 += U * 256) {
        u32x4 x[U];
        int64_t off[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * 256;
            if (v < v_end) x[u] = load16_stream(gather_src(p, row0, v, &off[u]));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (v0 + u * 256 >= v_end) break;
            store16_sys(sys_rsrc(p.dst), (uint32_t)off[u], x[u]);   // read by a matmul already running
        }
    }
    wg_signal(C.ready + (c * kReadyLines + lb % kReadyLines) * kSyncWords);
    if (p.stamps) stamp(p.stamps, blockIdx.x, kStampGather | (c << 8), t0, realtime());
}

// ------------------------------------------------------------------ all-to-all
// The copy of an expert all-to-all (see A2ALaunch): local rows of chunk c are
// consecutive, each segment pairing a run of them with rows of one remote
// buffer.  A thread's vectors only move forward through a chunk, so its
// segment is found by walking the chunk's list forward from the last one.
struct A2AParams {
    uint8_t* remote[COC_MAX_WORLD];
    uint8_t* local;
    int64_t row_bytes;
    int32_t vpr, nchunks, per_chunk;
    int32_t row0[COC_MAX_SPLIT], total[COC_MAX_SPLIT];   // first local row; rows * vpr
    int32_t seg0[COC_MAX_SPLIT + 1];
    const uint32_t* done;
    uint32_t target[COC_MAX_SPLIT];
    uint32_t spin_limit;
    uint32_t* gave_up;     // set by a wait that gives up (may be NULL)
    uint32_t* ready;
    A2ASegment seg[kMaxA2ASegs];
};

// The segment of chunk c holding local row lr, searching from segment s.  p
// must be the kernel argument itself (the table is read from the argument
// segment, not copied).
__device__ __forceinline__ int a2a_segment(const A2AParams& p, int c, int s, int lr) {
    while (s + 1 < p.seg0[c + 1] && lr >= p.seg[s].local_row + p.seg[s].rows) ++s;
    return s;
}

__device__ __forceinline__ int64_t a2a_remote_off(const A2AParams& p, int s, int lr, int cv) {
    return (int64_t)(p.seg[s].remote_row + (lr - p.seg[s].local_row)) * p.row_bytes + (int64_t)cv * 16;
}

// Dispatch: workgroups [c * per_chunk, (c + 1) * per_chunk) copy chunk c's
// rows from the sources into the received matrix, written through for the
// matmul already running, then add 1 each to the chunk's ready lines.
__global__ __launch_bounds__(256) void a2a_dispatch(A2AParams p) {
    constexpr int U = 4;
    const int c = blockIdx.x / p.per_chunk, lb = blockIdx.x % p.per_chunk;
    const int total = p.total[c];
    const int per = (total + p.per_chunk - 1) / p.per_chunk;
    const int v_end = (lb + 1) * per < total ? (lb + 1) * per : total;
    int s = p.seg0[c];
    for (int v0 = lb * per + threadIdx.x; v0 < v_end; v0 += U * 256) {
        u32x4 x[U];
        uint32_t off[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * 256;
            if (v < v_end) {
                const int row = v / p.vpr, cv = v - row * p.vpr;
                const int lr = p.row0[c] + row;
                s = a2a_segment(p, c, s, lr);
                x[u] = load16_stream(p.remote[p.seg[s].buf] + a2a_remote_off(p, s, lr, cv));
                off[u] = (uint32_t)((int64_t)lr * p.row_bytes + (int64_t)cv * 16);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (v0 + u * 256 >= v_end) break;
            store16_sys(sys_rsrc(p.local), off[u], x[u]);
        }
    }
    wg_signal(p.ready + (c * kReadyLines + lb % kReadyLines) * kSyncWords);
}

// Combine: at most one workgroup per CU beside the matmul; chunk by chunk,
// wait until the matmul has counted the chunk's tiles (if done is set), then
// copy its rows of the matmul's output back to the sources (NaN if the wait
// gave up).  The output is read at system scope: the matmul writes it through
// while this kernel runs.
__global__ __launch_bounds__(256) void a2a_combine(A2AParams p) {
    constexpr int U = 4;
    const int stride = gridDim.x * 256;
    const u32x4 nan = u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};   // NaN in every format
    for (int c = 0; c < p.nchunks; ++c) {
        bool ok = true;
        if (p.done != nullptr) {
            if (c > 0) __syncthreads();   // wg_wait's flag is reused
            ok = wg_wait(p.done + c * kSyncWords, 1, p.target[c], p.spin_limit, p.gave_up);
        }
        const int total = p.total[c];
        int s = p.seg0[c];
        for (int v0 = blockIdx.x * 256 + threadIdx.x; v0 < total; v0 += U * stride) {
            u32x4 x[U];
            int64_t off[U];
            uint8_t* dst[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * stride;
                if (v < total) {
                    const int row = v / p.vpr, cv = v - row * p.vpr;
                    const int lr = p.row0[c] + row;
                    s = a2a_segment(p, c, s, lr);
                    x[u] = load16_sys(p.local + (int64_t)lr * p.row_bytes + (int64_t)cv * 16);
                    dst[u] = p.remote[p.seg[s].buf];
                    off[u] = a2a_remote_off(p, s, lr, cv);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (v0 + u * stride >= total) break;
                *(u32x4*)(dst[u] + off[u]) = ok ? x[u] : nan;
            }
        }
    }
}

// Clears n 32-bit words: the allocation-free entry point's hand-over
// counters at the start of each call (a kernel rather than a memset node, so
// that a call captured into a graph clears them on every replay).
__global__ __launch_bounds__(256) void zero_words(uint32_t* p, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

// Activity-stamp buffer for measurement (coc_profile_stamps): records are
// handed out to launches in order; a launch that does not fit gets none.
std::mutex g_stamp_mu;
uint64_t* g_stamp_buf = nullptr;
int64_t g_stamp_cap = 0, g_stamp_next = 0;
uint64_t* stamp_region(int64_t records) {
    std::lock_guard<std::mutex> lk(g_stamp_mu);
    if (g_stamp_buf == nullptr || records <= 0 || g_stamp_next + records > g_stamp_cap) return nullptr;
    uint64_t* r = g_stamp_buf + 3 * g_stamp_next;
    g_stamp_next += records;
    return r;
}

int grid_for(int64_t total_vec, int per_thread = 1) {
    const int64_t want = (total_vec + 256 * per_thread - 1) / (256 * per_thread);
    const int64_t cap = 256 * 8;
    return (int)(want < cap ? (want > 0 ? want : 1) : cap);
}

template <int BM, int BN>
hipError_t launch_w8(GemmParams p, hipStream_t s) {
    p.tiles_m = (p.rows + BM - 1) / BM;
    p.tiles_n = (p.n + BN - 1) / BN;
    hipLaunchKernelGGL((gemm_w8<BM, BN, GK_W8_F16>), dim3(p.tiles_m * p.tiles_n), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_w8_any(GemmParams p, hipStream_t s) {
    const int64_t t256 = ((p.rows + 255) / 256) * ((p.n + 255) / 256);
    const int64_t t256x128 = ((p.rows + 255) / 256) * ((p.n + 127) / 128);
    if (t256 >= 256) return launch_w8<256, 256>(p, s);
    if (t256x128 >= 256) return launch_w8<256, 128>(p, s);
    return launch_w8<128, 128>(p, s);
}

template <int BM, int BN, int WM, int WN, int STAGES, int BK, int KIND, bool DEV_SCOPE>
hipError_t launch_dma(GemmParams p, hipStream_t s) {
    p.tiles_m = (p.rows + BM - 1) / BM;
    p.tiles_n = (p.n + BN - 1) / BN;
    hipLaunchKernelGGL((gemm_dma<BM, BN, WM, WN, STAGES, BK, KIND, DEV_SCOPE>), dim3(p.tiles_m * p.tiles_n),
                       dim3(64 * WM * WN), 0, s, p);
    return hipGetLastError();
}

template <int BM, int BN, int S, int WM, int WN, int KIND>
hipError_t launch_ring(GemmParams p, hipStream_t s) {
    p.tiles_m = (p.rows + BM - 1) / BM;
    p.tiles_n = (p.n + BN - 1) / BN;
    hipLaunchKernelGGL((gemm_ring<BM, BN, S, WM, WN, KIND>), dim3(p.tiles_m * p.tiles_n), dim3(64 * WM * WN), 0,
                       s, p);
    return hipGetLastError();
}

template <int KIND>
hipError_t launch_chunks_kind(const ChunksLaunch& L, hipStream_t s, int32_t* tiles);

template <int KIND>
hipError_t launch_dma_kind(GemmParams p, int concurrent, hipStream_t s, bool trans_b = false) {
    // k a positive multiple of 32: the ring kernel with the largest tile that
    // still gives COC_RING_MIN_TILES workgroups across the chunk matmuls that
    // run side by side.  Otherwise the 128 x 128 direct-to-LDS kernel, which
    // zero-fills the k tail.  Every choice walks k the same way, so it never
    // changes the result bits.
    if (p.k >= 32 && p.k % 32 == 0) {
        if (concurrent <= 1 || is_w8(KIND) || trans_b) {
            // a lone matmul: the chunk-walking launch with one chunk (measured
            // faster than one workgroup per tile: no second dispatch wave)
            ChunksLaunch L{};
            L.kind = (GemmKind)KIND;
            L.b = p.b;
            L.c = p.c;
            L.n = p.n;
            L.k = p.k;
            L.npieces = 1;
            L.scales = p.scales;
            L.qmode = p.qmode;
            L.group = p.group;
            L.trans_b = trans_b;
            L.a[0] = p.a;
            L.base[0] = p.base;
            L.stride[0] = p.stride;
            L.rpb[0] = p.rpb;
            L.nblk[0] = p.rows / (p.rpb > 0 ? p.rpb : 1);
            L.wait[0] = -1;
            L.signal[0] = -1;
            int32_t tiles[kMaxPieces + 1];
            return launch_chunks_kind<KIND>(L, s, tiles);
        }
        if constexpr (!is_w8(KIND)) {
            const int64_t want = COC_RING_MIN_TILES / (concurrent > 1 ? concurrent : 1);
            const int64_t tm256 = (p.rows + 255) / 256, tm128 = (p.rows + 127) / 128;
            const int64_t tn256 = (p.n + 255) / 256;
            if (tm256 * tn256 >= want) return launch_ring<256, 256, 4, 2, 4, KIND>(p, s);
            if (tm128 * tn256 >= want) return launch_ring<128, 256, 4, 2, 4, KIND>(p, s);
            return launch_ring<128, 128, 4, 2, 2, KIND>(p, s);
        }
    }
    // (int8 weights come here only with k % 32 == 0, through the chunk launch)
    if constexpr (is_w8(KIND)) return hipErrorInvalidValue;
    else return launch_dma<128, 128, 2, 2, 4, 32, KIND, false>(p, s);
}

}  // namespace

int launch_gemm(const GemmLaunch& g, void* stream) {
    const int64_t rows = int64_t(g.nblk) * g.rpb;
    if (rows == 0 || g.n == 0) return hipSuccess;
    GemmParams p{};
    p.a = (const uint8_t*)g.a;
    p.b = (const uint8_t*)g.b;
    p.c = (uint8_t*)g.c;
    p.scales = (const uint16_t*)g.scales;
    p.base = g.base;
    p.stride = g.stride;
    p.rpb = (int32_t)g.rpb;
    p.rows = (int32_t)rows;
    p.n = (int32_t)g.n;
    p.k = (int32_t)g.k;
    p.qmode = g.qmode;
    p.group = g.group > 0 ? g.group : 1;
    hipStream_t s = (hipStream_t)stream;
    switch (g.kind) {
        case GK_F32: {
            p.tiles_m = (p.rows + 63) / 64;
            p.tiles_n = (p.n + 63) / 64;
            hipLaunchKernelGGL(gemm_f32, dim3(p.tiles_m * p.tiles_n), dim3(256), 0, s, p);
            return hipGetLastError();
        }
        case GK_F16: return launch_dma_kind<GK_F16>(p, g.concurrent, s, g.trans_b != 0);
        case GK_BF16: return launch_dma_kind<GK_BF16>(p, g.concurrent, s, g.trans_b != 0);
        case GK_W8_F16:
            if (chunks_supported(g)) return launch_dma_kind<GK_W8_F16>(p, 1, s);
            return launch_w8_any(p, s);
    }
    return hipErrorInvalidValue;
}

int launch_zero_words(uint32_t* p, int n, void* stream) {
    if (n <= 0) return hipSuccess;
    const int grid = (n + 255) / 256 < 64 ? (n + 255) / 256 : 64;
    hipLaunchKernelGGL(zero_words, dim3(grid), dim3(256), 0, (hipStream_t)stream, p, n);
    return hipGetLastError();
}

int launch_reduce(const ReduceLaunch& r, void* stream) {
    if (r.rows == 0 || r.n == 0) return hipSuccess;
    ReduceParams p{};
    for (int i = 0; i < COC_MAX_WORLD; ++i) p.src[i] = (const uint8_t*)(i < r.nsrc ? r.src[i] : r.src[0]);
    p.dst = (uint8_t*)r.dst;
    p.src_row0 = r.src_row0;
    p.dst_row0 = r.dst_row0;
    p.row_bytes = r.n * (int64_t)elem_size(r.dt);
    p.nsrc = r.nsrc;
    p.vpr = (int32_t)(p.row_bytes / 16);
    p.total = (int32_t)(r.rows * p.vpr);
    hipStream_t s = (hipStream_t)stream;
    if (r.wide) {
        // up to 16 workgroups per CU, each a contiguous block of at least one
        // pass of U vectors per thread
        constexpr int U = 2;
        const int64_t want = ((int64_t)p.total + U * 256 - 1) / (U * 256);
        const int grid = (int)(want < 4096 ? (want > 0 ? want : 1) : 4096);
        const int per = (int)(((int64_t)p.total + grid - 1) / grid);
        p.stamps = stamp_region(grid);
        switch (r.dt) {
            case COC_F32: hipLaunchKernelGGL((reduce_rows_wide<COC_F32, U>), dim3(grid), dim3(256), 0, s, p, per); break;
            case COC_F16: hipLaunchKernelGGL((reduce_rows_wide<COC_F16, U>), dim3(grid), dim3(256), 0, s, p, per); break;
            case COC_BF16: hipLaunchKernelGGL((reduce_rows_wide<COC_BF16, U>), dim3(grid), dim3(256), 0, s, p, per); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    const int grid = grid_for(p.total);
    p.stamps = stamp_region(grid);
    switch (r.dt) {
        case COC_F32: hipLaunchKernelGGL(reduce_rows<COC_F32>, dim3(grid), dim3(256), 0, s, p); break;
        case COC_F16: hipLaunchKernelGGL(reduce_rows<COC_F16>, dim3(grid), dim3(256), 0, s, p); break;
        case COC_BF16: hipLaunchKernelGGL(reduce_rows<COC_BF16>, dim3(grid), dim3(256), 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int launch_reduce_chunks(const ReduceChunksLaunch& L, void* stream) {
    const ReduceLaunch& r = L.r;
    if (r.n == 0 || L.nchunks == 0) return hipSuccess;
    ReduceParams p{};
    for (int i = 0; i < COC_MAX_WORLD; ++i) p.src[i] = (const uint8_t*)(i < r.nsrc ? r.src[i] : r.src[0]);
    p.dst = (uint8_t*)r.dst;
    p.row_bytes = r.n * (int64_t)elem_size(r.dt);
    p.nsrc = r.nsrc;
    p.vpr = (int32_t)(p.row_bytes / 16);
    ReduceChunks C{};
    int64_t most = 0;
    for (int c = 0; c < L.nchunks; ++c) {
        C.src_row0[c] = L.src_row0[c];
        C.dst_row0[c] = L.dst_row0[c];
        C.total[c] = (int32_t)(L.rows[c] * p.vpr);
        C.target[c] = L.target[c];
        most = C.total[c] > most ? C.total[c] : most;
    }
    C.done = L.done;
    C.nchunks = L.nchunks;
    C.own = L.own;
    C.spin_limit = L.spin_limit > 0 ? L.spin_limit : kSpinLimit;
    C.gave_up = L.gave_up;
    const int grid = grid_for(most) < 256 ? grid_for(most) : 256;   // at most one per CU
    p.stamps = stamp_region((int64_t)grid * C.nchunks);
    hipStream_t s = (hipStream_t)stream;
    auto go = [&](auto DTC) {
        constexpr int DT = decltype(DTC)::value;
        if (L.narrow)
            hipLaunchKernelGGL((reduce_chunks_wait<DT, 1>), dim3(grid), dim3(256), 0, s, p, C);
        else
            hipLaunchKernelGGL((reduce_chunks_wait<DT, 2>), dim3(grid), dim3(256), 0, s, p, C);
    };
    switch (r.dt) {
        case COC_F32: go(std::integral_constant<int, COC_F32>{}); break;
        case COC_F16: go(std::integral_constant<int, COC_F16>{}); break;
        case COC_BF16: go(std::integral_constant<int, COC_BF16>{}); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int launch_gather(const GatherLaunch& g, void* stream, int32_t* groups) {
    if (groups != nullptr) *groups = 0;
    if (g.rows == 0 || g.k == 0) return hipSuccess;
    GatherParams p{};
    for (int i = 0; i < COC_MAX_WORLD; ++i) p.src[i] = (const uint8_t*)(i < g.nsrc ? g.src[i] : g.src[0]);
    p.dst = (uint8_t*)g.dst;
    p.row_bytes = g.k * (int64_t)elem_size(g.dt);
    p.shard_rows = (int32_t)g.shard_rows;
    p.row0 = (int32_t)g.row0;
    p.vpr = (int32_t)(p.row_bytes / 16);
    p.total = (int32_t)(g.rows * p.vpr);
    p.signal = g.signal;
    hipStream_t s = (hipStream_t)stream;
    const int grid = grid_for(p.total, 4);
    p.stamps = stamp_region(grid);
    hipLaunchKernelGGL(gather_rows, dim3(grid), dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess && groups != nullptr) *groups = grid;
    return e;
}

int launch_gather_chunks(const GatherLaunch& g, int nchunks, const int64_t* row0, const int64_t* rows,
                         uint32_t* ready, void* stream, int32_t* per_chunk) {
    *per_chunk = 0;
    if (g.k == 0 || nchunks == 0) return hipSuccess;
    GatherParams p{};
    for (int i = 0; i < COC_MAX_WORLD; ++i) p.src[i] = (const uint8_t*)(i < g.nsrc ? g.src[i] : g.src[0]);
    p.dst = (uint8_t*)g.dst;
    p.row_bytes = g.k * (int64_t)elem_size(g.dt);
    p.shard_rows = (int32_t)g.shard_rows;
    p.vpr = (int32_t)(p.row_bytes / 16);
    GatherChunks C{};
    int64_t most = 0;
    for (int c = 0; c < nchunks; ++c) {
        C.row0[c] = (int32_t)row0[c];
        C.total[c] = (int32_t)(rows[c] * p.vpr);
        most = C.total[c] > most ? C.total[c] : most;
    }
    C.ready = ready;
    // up to 2048 workgroups in all, each with at least 4 passes of 4 vectors per thread
    const int64_t want = (most + 4 * 4 * 256 - 1) / (4 * 4 * 256);
    const int64_t cap = 2048 / nchunks;
    C.per_chunk = (int32_t)(want < cap ? (want > 0 ? want : 1) : cap);
    p.stamps = stamp_region((int64_t)C.per_chunk * nchunks);
    hipLaunchKernelGGL(gather_chunks, dim3(C.per_chunk * nchunks), dim3(256), 0, (hipStream_t)stream, p, C);
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) *per_chunk = C.per_chunk;
    return e;
}

int launch_a2a_chunks(const A2ALaunch& a, void* stream, int32_t* per_chunk) {
    *per_chunk = 0;
    if (a.nchunks <= 0 || a.nchunks > COC_MAX_SPLIT || a.row_bytes <= 0 || a.row_bytes % 16 != 0)
        return hipErrorInvalidValue;
    A2AParams p{};
    for (int i = 0; i < COC_MAX_WORLD; ++i) p.remote[i] = (uint8_t*)a.remote[i];
    p.local = (uint8_t*)a.local;
    p.row_bytes = a.row_bytes;
    p.vpr = (int32_t)(a.row_bytes / 16);
    p.nchunks = a.nchunks;
    int64_t most = 0;
    for (int c = 0; c < a.nchunks; ++c) {
        p.row0[c] = (int32_t)a.row0[c];
        p.total[c] = (int32_t)(a.rows[c] * p.vpr);
        most = p.total[c] > most ? p.total[c] : most;
    }
    for (int c = 0; c <= a.nchunks; ++c) p.seg0[c] = a.seg0[c];
    if (p.seg0[a.nchunks] > kMaxA2ASegs) return hipErrorInvalidValue;
    for (int i = 0; i < p.seg0[a.nchunks]; ++i) p.seg[i] = a.seg[i];
    p.done = a.done;
    for (int c = 0; c < COC_MAX_SPLIT; ++c) p.target[c] = a.target[c];
    p.spin_limit = a.spin_limit > 0 ? a.spin_limit : kSpinLimit;
    p.gave_up = a.gave_up;
    p.ready = a.ready;
    hipStream_t s = (hipStream_t)stream;
    if (a.to_remote == 0) {
        if (a.ready == nullptr) return hipErrorInvalidValue;
        // as the all-gather copy: up to 2048 workgroups, each at least 4
        // passes of 4 vectors per thread
        const int64_t want = (most + 4 * 4 * 256 - 1) / (4 * 4 * 256);
        const int64_t cap = 2048 / a.nchunks;
        p.per_chunk = (int32_t)(want < cap ? (want > 0 ? want : 1) : cap);
        hipLaunchKernelGGL(a2a_dispatch, dim3(p.per_chunk * a.nchunks), dim3(256), 0, s, p);
        const hipError_t e = hipGetLastError();
        if (e == hipSuccess) *per_chunk = p.per_chunk;
        return e;
    }
    const int grid = grid_for(most, 4) < 256 ? grid_for(most, 4) : 256;   // at most one per CU
    hipLaunchKernelGGL(a2a_combine, dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

void set_stamp_buffer(uint64_t* buf, int64_t records) {
    std::lock_guard<std::mutex> lk(g_stamp_mu);
    g_stamp_buf = buf;
    g_stamp_cap = buf != nullptr && records > 0 ? records : 0;
    g_stamp_next = 0;
}

int64_t stamp_records_used() {
    std::lock_guard<std::mutex> lk(g_stamp_mu);
    return g_stamp_next;
}

bool chunks_supported(const GemmLaunch& g) {
    if (g.k < 32 || g.k % 32 != 0) return false;
    if (g.trans_b) return g.kind == GK_BF16 || g.kind == GK_F16;
    if (g.kind == GK_BF16 || g.kind == GK_F16) return true;
    if (g.kind != GK_W8_F16 || g.n % 16 != 0) return false;   // whole 16-byte int8 chunks
    if (g.qmode != COC_PER_GROUP) return true;
    return g.group % 32 == 0 && ((g.k + g.group - 1) / g.group) * 256 * 2 <= kW8TableBytes;
}

namespace {

// Tile shape of a chunk-walking launch: the largest tile that still fills the
// 256 CUs once over the whole op (0: 256 x 256, 1: 128 x 256, 2: 128 x 128).
int chunks_shape(const ChunksLaunch& L, int* bm, int* bn, int* per_cu) {
    int64_t t256 = 0, t128x256 = 0;
    for (int c = 0; c < L.npieces; ++c) {
        const int64_t rows = L.rpb[c] * L.nblk[c];
        t256 += ((rows + 255) / 256) * ((L.n + 255) / 256);
        t128x256 += ((rows + 127) / 128) * ((L.n + 255) / 256);
    }
    if (t256 >= 256) { *bm = 256; *bn = 256; *per_cu = 1; return 0; }
    if (t128x256 >= 256) { *bm = 128; *bn = 256; *per_cu = 1; return 1; }
    *bm = 128; *bn = 128; *per_cu = 2;
    return 2;
}

// Per-piece tiles and workgroups per XCD of a chunk-walking launch.
int chunks_layout(const ChunksLaunch& L, int32_t* tiles, int* per_cu) {
    int bm, bn;
    chunks_shape(L, &bm, &bn, per_cu);
    const int64_t tiles_n = (L.n + bn - 1) / bn;
    int64_t longest = 0;   // XCD 0's list: ceil(T_i / 8) summed over pieces
    for (int c = 0; c < L.npieces; ++c) {
        const int64_t rows = L.rpb[c] * L.nblk[c];
        tiles[c] = (int32_t)(((rows + bm - 1) / bm) * tiles_n);
        longest += (tiles[c] + 7) / 8;
    }
    const int64_t cap = 32 * *per_cu;   // 256 CUs / 8 XCDs, times workgroups per CU
    return (int)(longest < cap ? (longest > 0 ? longest : 1) : cap);
}

int device_cus() {
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cus[dev] = v;
    }
    return cus[dev];
}

template <int BM, int BN, int S, int WM, int WN, int KIND, bool TA, bool TB, bool QUAD = false>
hipError_t launch_chunks_shape(const ChunksLaunch& L, int per_cu, hipStream_t s, int32_t* tiles) {
    PersistParams P{};
    P.g.b = (const uint8_t*)L.b;
    P.g.c = (uint8_t*)L.c;
    P.g.n = (int32_t)L.n;
    P.g.k = (int32_t)L.k;
    P.g.scales = (const uint16_t*)L.scales;
    P.g.qmode = L.qmode;
    P.g.group = L.group > 0 ? L.group : 1;
    P.g.lda = (int32_t)L.lda;
    P.g.tiles_n = (int32_t)((L.n + BN - 1) / BN);
    P.npieces = L.npieces;
    P.order = L.order;
    P.spin_limit = L.spin_limit > 0 ? L.spin_limit : kSpinLimit;
    P.gave_up = L.gave_up;
    bool signal = false;
    int per_cu_chk = 0;
    P.per_xcd = chunks_layout(L, tiles, &per_cu_chk);
    for (int c = 0; c < L.npieces; ++c) {
        const int64_t rows = L.rpb[c] * L.nblk[c];
        P.a[c] = (const uint8_t*)L.a[c];
        P.b[c] = (const uint8_t*)(L.bp[c] != nullptr ? L.bp[c] : L.b);
        P.ashift[c] = L.ashift[c];
        P.base[c] = L.base[c];
        P.stride[c] = L.stride[c];
        P.rpb[c] = (int32_t)(L.rpb[c] > 0 ? L.rpb[c] : 1);
        P.rows[c] = (int32_t)rows;
        P.tiles_m[c] = (int32_t)((rows + BM - 1) / BM);
        P.wait[c] = L.wait[c];
        P.signal[c] = L.signal[c];
        signal = signal || (L.done != nullptr && L.signal[c] >= 0);
    }
    for (int i = 0; i < COC_MAX_SPLIT; ++i) P.ready_target[i] = L.ready_target[i];
    P.done = L.done;
    P.ready = L.ready;
    if (L.gather_nchunks > 0) {
        // the caller's ready targets assume this very plan
        const FusedGatherPlan fp = chunks_fused_gather(L);
        if (fp.gatherers <= 0 || L.ready == nullptr || fp.gatherers != L.gather_plan.gatherers ||
            fp.early != L.gather_plan.early || fp.workgroups != L.gather_plan.workgroups)
            return hipErrorInvalidValue;
        FusedGather& F = P.fg;
        for (int i = 0; i < COC_MAX_WORLD; ++i) F.p.src[i] = (const uint8_t*)L.gather_src[i];
        F.p.dst = (uint8_t*)L.gather_dst;
        F.p.row_bytes = L.gather_row_bytes;
        F.p.shard_rows = (int32_t)L.gather_shard_rows;
        F.p.vpr = (int32_t)(L.gather_row_bytes / 16);
        F.nchunks = L.gather_nchunks;
        for (int c = 0; c < L.gather_nchunks; ++c) {
            F.row0[c] = (int32_t)L.gather_row0[c];
            F.total[c] = (int32_t)(L.gather_rows[c] * F.p.vpr);
            F.row0b[c] = (int32_t)L.gather_row0b[c];
            F.totalb[c] = (int32_t)(L.gather_rowsb[c] * F.p.vpr);
        }
        F.gatherers = fp.gatherers;
        F.early = fp.early;
    }
    tiles[kMaxPieces] = 8 * P.per_xcd;
    P.stamps = stamp_region((int64_t)8 * P.per_xcd * (1 + P.fg.nchunks));
    P.fg.p.stamps = P.stamps;
    if constexpr (QUAD) {
        // (the caller checked quad_ok: nothing signals, and only rows the
        // launch copies itself are waited for)
        if (signal || L.k % 64 != 0) return hipErrorInvalidValue;
        hipLaunchKernelGGL((gemm_ring_chunks<256, 256, 4, 2, 2, KIND, false, false, true, false, true>),
                           dim3(8 * P.per_xcd), dim3(256), 0, s, P);
        return hipGetLastError();
    } else {
        // activations in whole 128-byte row segments, two stages at a time (k % 64 == 0)
        if constexpr (COC_PAIR_A && !TA) {
            if (L.k % 64 == 0) {
                if (signal)
                    hipLaunchKernelGGL((gemm_ring_chunks<BM, BN, S, WM, WN, KIND, true, false, TB, true>),
                                       dim3(8 * P.per_xcd), dim3(64 * WM * WN), 0, s, P);
                else
                    hipLaunchKernelGGL((gemm_ring_chunks<BM, BN, S, WM, WN, KIND, false, false, TB, true>),
                                       dim3(8 * P.per_xcd), dim3(64 * WM * WN), 0, s, P);
                return hipGetLastError();
            }
        }
        if (signal)
            hipLaunchKernelGGL((gemm_ring_chunks<BM, BN, S, WM, WN, KIND, true, TA, TB>), dim3(8 * P.per_xcd),
                               dim3(64 * WM * WN), 0, s, P);
        else
            hipLaunchKernelGGL((gemm_ring_chunks<BM, BN, S, WM, WN, KIND, false, TA, TB>), dim3(8 * P.per_xcd),
                               dim3(64 * WM * WN), 0, s, P);
        return hipGetLastError();
    }
}

// Whether a launch takes the four-wave tile: bf16 / fp16 with transposed
// weights, 256 x 256 tiles, k % 64 == 0, and nothing beside it to share a CU
// with: no counter to signal, and no wait except for rows the launch copies
// itself (its workgroups are then all resident at once, one per CU).
// COC_FOUR_WAVE=0 keeps ring_tile (the result bits are the same; for A/B
// timing).
bool quad_ok(const ChunksLaunch& L) {
    const char* v = getenv("COC_FOUR_WAVE");
    if (v != nullptr && v[0] == '0') return false;
    if (!(L.kind == GK_BF16 || L.kind == GK_F16) || !L.trans_b || L.trans_a || L.k % 64 != 0) return false;
    for (int c = 0; c < L.npieces; ++c)
        if ((L.wait[c] >= 0 && L.gather_nchunks <= 0) || (L.done != nullptr && L.signal[c] >= 0)) return false;
    int bm = 0, bn = 0, per_cu = 0;
    return chunks_shape(L, &bm, &bn, &per_cu) == 0;
}

template <int KIND, bool TA, bool TB>
hipError_t launch_chunks_layout(const ChunksLaunch& L, hipStream_t s, int32_t* tiles) {
    if constexpr ((KIND == GK_BF16 || KIND == GK_F16) && TB && !TA) {
        if (quad_ok(L)) return launch_chunks_shape<256, 256, 4, 2, 2, KIND, false, true, true>(L, 1, s, tiles);
    }
    int bm, bn, per_cu;
    switch (chunks_shape(L, &bm, &bn, &per_cu)) {
        case 0: return launch_chunks_shape<256, 256, 4, 2, 4, KIND, TA, TB>(L, 1, s, tiles);
        case 1: return launch_chunks_shape<128, 256, 4, 2, 4, KIND, TA, TB>(L, 1, s, tiles);
        default: return launch_chunks_shape<128, 128, 4, 2, 2, KIND, TA, TB>(L, 2, s, tiles);
    }
}

template <int KIND>
hipError_t launch_chunks_kind(const ChunksLaunch& L, hipStream_t s, int32_t* tiles) {
    if constexpr (KIND == GK_W8_F16) {
        if (L.trans_a || L.trans_b) return hipErrorInvalidValue;
        for (int c = 0; c < L.npieces; ++c)
            if (L.bp[c] != nullptr) return hipErrorInvalidValue;   // one weight, one scale table
        if (L.qmode == COC_PER_GROUP) return launch_chunks_layout<GK_W8G_F16, false, false>(L, s, tiles);
        return launch_chunks_layout<KIND, false, false>(L, s, tiles);
    } else {
        if (L.trans_a && L.trans_b) return hipErrorInvalidValue;
        // a transposed activation operand has no row map: one piece
        if (L.trans_a && (L.npieces != 1 || L.nblk[0] != 1 || L.ashift[0] != 0)) return hipErrorInvalidValue;
        if (L.trans_a) return launch_chunks_layout<KIND, true, false>(L, s, tiles);
        if (L.trans_b) return launch_chunks_layout<KIND, false, true>(L, s, tiles);
        return launch_chunks_layout<KIND, false, false>(L, s, tiles);
    }
}

}  // namespace

bool chunks_reduce_narrow(const ChunksLaunch& L) {
    // The int8-weight matmuls (199-213 VGPRs) and the 256 x 256 paired-stage
    // ones (208-210) leave 80-96 VGPRs per SIMD lane beside their two waves,
    // too few for the two-vector waiting reduce (104); the others (<= 200)
    // leave 112.
    if (L.kind == GK_W8_F16) return true;
    int bm = 0, bn = 0, per_cu = 0;
    const bool paired = COC_PAIR_A && !L.trans_a && L.k % 64 == 0;
    return paired && chunks_shape(L, &bm, &bn, &per_cu) == 0;
}

void chunks_tiles(const ChunksLaunch& L, int32_t tiles[kMaxPieces + 1]) {
    for (int c = 0; c <= kMaxPieces; ++c) tiles[c] = 0;
    int per_cu = 0;
    tiles[kMaxPieces] = 8 * chunks_layout(L, tiles, &per_cu);
}

FusedGatherPlan chunks_fused_gather(const ChunksLaunch& L) {
    FusedGatherPlan fp{};
    int32_t tiles[kMaxPieces];
    int per_cu = 0;
    const int per_xcd = chunks_layout(L, tiles, &per_cu);
    // every workgroup must be resident at once (one per CU): workgroups wait
    // for rows that others copy
    if (per_cu != 1 || 8 * per_xcd > device_cus()) return fp;
    int first = -1;
    const int g = singles_before(tiles, 1, L.npieces, per_xcd, 8, &first);   // over XCDs 0..7
    if (g < 16) return fp;
    const int early = early_chunks(tiles, L.wait, L.npieces, per_xcd);
    fp.gatherers = g;
    fp.early = early < L.gather_nchunks ? early : L.gather_nchunks;
    fp.workgroups = 8 * per_xcd;
    return fp;
}

int launch_gemm_chunks(const ChunksLaunch& L, void* stream, int32_t tiles[kMaxPieces + 1]) {
    for (int c = 0; c <= kMaxPieces; ++c) tiles[c] = 0;
    hipStream_t s = (hipStream_t)stream;
    switch (L.kind) {
        case GK_F16: return launch_chunks_kind<GK_F16>(L, s, tiles);
        case GK_BF16: return launch_chunks_kind<GK_BF16>(L, s, tiles);
        case GK_W8_F16: return launch_chunks_kind<GK_W8_F16>(L, s, tiles);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace coc
