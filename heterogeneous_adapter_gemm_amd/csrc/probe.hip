// Measurement probe: the sustained matrix-core rate of this GPU for the two
// bf16 shapes (16x16x32, the GEMM kernels' shape, and 32x32x16).  Every wave
// runs independent chains of matrix operations on register data (no memory
// traffic inside the loop), so the launch time gives the rate the matrix cores
// reach at the clock the chip holds under full load: the ceiling the GEMM
// kernels are compared with next to the published peak.
#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"
#include "lora_gemm.h"

namespace hagemm {
namespace {

constexpr int kProbeChains = 8;   // independent accumulators per wave (hide the matrix-op latency)

typedef float f32x16 __attribute__((ext_vector_type(16)));

// SHAPE 16: v_mfma_f32_16x16x32_bf16 (the GEMM kernels' shape); SHAPE 32: v_mfma_f32_32x32x16_bf16
template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int64_t iters, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const u32x4 a = {0x3f803f80u + (uint32_t)lane, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    const u32x4 b = {0x3c003c00u, 0x3c003c00u + (uint32_t)(threadIdx.x >> 6), 0x3c003c00u, 0x3c003c00u};
    float s = 0.f;
    if constexpr (SHAPE == 16) {
        f32x4 acc[kProbeChains];
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, (float)c};
        for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
            for (int c = 0; c < kProbeChains; ++c) acc[c] = mma_step(a, b, acc[c], bf16_t{});
        }
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c) s += acc[c][0] + acc[c][3];
    } else {
        f32x16 acc[kProbeChains];
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[c][e] = (float)c;
        for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
            for (int c = 0; c < kProbeChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                                 __builtin_bit_cast(bf16x8, b), acc[c], 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c) s += acc[c][0] + acc[c][15];
    }
    s = wave_sum(s);
    if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace
}  // namespace hagemm

extern "C" int lora_probe_mfma(int32_t shape, int64_t iters, int32_t blocks, float* out, void* stream,
                               double* flops) {
    if ((shape != 16 && shape != 32) || iters < 1 || blocks < 1 || !out)
        return hagemm::set_error(LORA_EINVAL, "shape must be 16 or 32, iters and blocks >= 1, out non-NULL");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (shape == 16)
        hipLaunchKernelGGL(hagemm::mfma_probe_kernel<16>, dim3(blocks), dim3(256), 0, st, iters, out);
    else
        hipLaunchKernelGGL(hagemm::mfma_probe_kernel<32>, dim3(blocks), dim3(256), 0, st, iters, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hagemm::set_error(LORA_EHIP, "mfma probe: %s", hipGetErrorString(e));
    // 16 x 16 x 32 and 32 x 32 x 16 ops: 16384 and 32768 multiply-adds
    if (flops) *flops = (double)blocks * 4 * iters * hagemm::kProbeChains * 2.0 * (shape == 16 ? 8192 : 16384);
    return LORA_OK;
}
