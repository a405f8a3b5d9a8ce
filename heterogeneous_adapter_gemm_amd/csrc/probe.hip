// Measurement probes.  The sustained matrix-core rate of this GPU for the two
// bf16 shapes (16x16x32, the GEMM kernels' shape, and 32x32x16).  Every wave
// runs independent chains of matrix operations on register data (no memory
// traffic inside the loop), so the launch time gives the rate the matrix cores
// reach at the clock the chip holds under full load: the ceiling the GEMM
// kernels are compared with next to the published peak.  And the rate at which
// HBM serves the delta kernels' access shape: one 8 KiB chunk per wave (an
// adapter row of 4096 bf16 values in its page) at the offsets the caller
// gives, for the same bytes as a shrink or expand launch moves.
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

// One wave per 8 KiB chunk: the chunk's offset is read first (a dependent load, as a BGMV
// unit's index entry is), then the wave's eight 1 KiB pieces are all in flight at once, as a
// shrink wave's A row is.  Nothing is written unless the checksum takes one fixed value.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint8_t* __restrict__ buf, int64_t n_whole,
                                                         const int64_t* __restrict__ chunk, int32_t n,
                                                         float* __restrict__ out) {
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (w >= n) return;
    const int64_t c = min(max(chunk[w], (int64_t)0), n_whole - 1);
    const uint8_t* p = buf + c * 8192 + lane * 16;
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ld16(p + i * 1024);
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    if (s == 0x9e3779b9u) out[w] = (float)s;
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

extern "C" int lora_probe_read(const void* buf, int64_t buf_bytes, const int64_t* chunk, int32_t n_chunks, float* out,
                               void* stream) {
    if (!buf || !chunk || !out || buf_bytes < 8192 || n_chunks < 1)
        return hagemm::set_error(LORA_EINVAL, "read probe: buf_bytes >= 8192, n_chunks >= 1, non-NULL pointers");
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(hagemm::read_probe_kernel, dim3((unsigned)((n_chunks + 3) / 4)), dim3(256), 0, st,
                       static_cast<const uint8_t*>(buf), buf_bytes / 8192, chunk, n_chunks, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hagemm::set_error(LORA_EHIP, "read probe: %s", hipGetErrorString(e));
    return LORA_OK;
}
