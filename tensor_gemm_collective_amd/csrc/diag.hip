// Diagnostic for measurement: the rate the bf16 MFMA unit sustains on its own.
//
// Each wave keeps eight independent 32x32 accumulators and, per iteration,
// issues one v_mfma_f32_32x32x16_bf16 into each, with operands that stay in
// registers (loaded once from the caller's buffer): no LDS, no memory traffic
// in the loop.  Random operands make the MFMA arrays toggle as they do in a
// matmul of random data; operands of one repeated value barely toggle them.
// Timing the launch on both kinds shows what operand toggling alone does to
// the rate the chip holds (its clock under the power limit), with nothing
// else drawing power.  This is the instruction and the accumulator count the
// ring matmul's waves use.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "coc.h"
#include "coc_internal.h"

namespace coc {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 8;   // independent accumulators per wave

__global__ __launch_bounds__(256) void mfma_loop(const u32x4* in, int32_t n_in, float* out, int32_t iters) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    u32x4 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = in[(t * 8 + i) % n_in];
        b[i] = in[(t * 8 + 4 + i) % n_in];
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[c & 3]),
                                                             __builtin_bit_cast(bf16x8, b[c >> 2]), acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    out[t] = s;   // keeps the loop from being removed
}

}  // namespace
}  // namespace coc

extern "C" coc_status coc_diag_mfma_loop(const void* operands, size_t operand_bytes, float* out, size_t out_floats,
                                         int32_t workgroups, int32_t iters, hipStream_t stream) {
    using coc::fail;
    coc::clear_error();
    if (operands == nullptr || out == nullptr) return fail(COC_ERR_NULL, "operands and out are required");
    if ((uintptr_t)operands % 16 != 0 || (uintptr_t)out % 16 != 0)
        return fail(COC_ERR_ALIGN, "operands and out must be 16-byte aligned");
    const size_t vecs = operand_bytes / 16;
    if (vecs < 8 || vecs > (size_t)INT32_MAX)
        return fail(COC_ERR_SHAPE, "operand_bytes must hold 8 to 2^31 - 1 16-byte vectors (got %zu bytes)",
                    operand_bytes);
    if (workgroups < 1 || workgroups > 65536 || iters < 1)
        return fail(COC_ERR_SHAPE, "workgroups must be in [1, 65536] and iters >= 1 (got %d, %d)", workgroups, iters);
    if (out_floats < (size_t)workgroups * 256)
        return fail(COC_ERR_SHAPE, "out must hold workgroups * 256 floats (%zu < %zu)", out_floats,
                    (size_t)workgroups * 256);
    hipLaunchKernelGGL(coc::mfma_loop, dim3(workgroups), dim3(256), 0, stream,
                       (const coc::u32x4*)operands, (int32_t)vecs, out, iters);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(COC_ERR_HIP, "mfma_loop launch: %s", hipGetErrorString(e));
    return COC_OK;
}
