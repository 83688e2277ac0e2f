// mfma_rate.hip - calibration kernel for the benchmark: the bf16 matrix-core
// rate this board sustains under its own power management.
//
// Not part of the attention library.  Each wave keeps eight A and eight B
// fragments (16 bytes per lane each, loaded once from a 1 MiB table of
// bf16 values) and issues back-to-back v_mfma bf16 instructions over them
// with four (32x32x16) or eight (16x16x32) independent accumulator chains,
// so the matrix pipe never waits on a dependency and no memory traffic runs
// during the loop.  Every MFMA pairs a different (A, B) fragment pair, so the
// operands change from one instruction to the next as in a real product.
// The FLOPs of one launch are blocks x 4 waves x iters x 64 MFMAs x
// (32768 for 32x32x16, 16384 for 16x16x32).
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTable = 65536;  // bf16x8 entries in the operand table (1 MiB)

template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_rate_kernel(const bf16x8* __restrict__ table, float* __restrict__ out,
                                                        int iters) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    bf16x8 a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = table[(t * 16 + i) & (kTable - 1)];
        b[i] = table[(t * 16 + 8 + i) & (kTable - 1)];
    }
    float s = 0.f;
    if constexpr (SHAPE == 32) {
        f32x16 acc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[(i + j) & 7], acc[i & 3], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) s += acc[j][e];
    } else {
        f32x4 acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[j][e] = 0.f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[(i + j) & 7], acc[i], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) s += acc[j][e];
    }
    out[t] = s;  // keeps the products live
}

}  // namespace

// table: 1 MiB of bf16 (65536 x 8 values), device; out: blocks x 256 floats,
// device; shape 32 or 16.  Returns a hipError_t value (0 on success); any
// other shape or a non-positive size returns hipErrorInvalidValue without a
// launch.
extern "C" __attribute__((visibility("default"))) int mla_calib_mfma_rate(const void* table, void* out, int blocks,
                                                                         int iters, int shape, void* stream) {
    if (!table || !out || blocks <= 0 || iters <= 0 || (shape != 32 && shape != 16)) return (int)hipErrorInvalidValue;
    if (shape == 32)
        hipLaunchKernelGGL(mfma_rate_kernel<32>, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                           (const bf16x8*)table, (float*)out, iters);
    else
        hipLaunchKernelGGL(mfma_rate_kernel<16>, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                           (const bf16x8*)table, (float*)out, iters);
    return (int)hipGetLastError();
}
