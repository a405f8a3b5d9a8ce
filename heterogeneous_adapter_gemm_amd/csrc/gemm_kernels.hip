// The shared base product y[M][N] = x[M][K] * w[N][K]^T on the gfx950 matrix
// cores: one dense GEMM over the whole batch that reads the base weight once
// ("Multi-LoRA serving: S-LoRA, Punica and adapter batching", The bottleneck).
//
// Both operands are K-contiguous, so either can feed either side of an MFMA.
// The kernel puts w on the MFMA's M side and x on its N side: each lane then
// ends with four consecutive output columns of one row, stored as one 8-byte
// (bf16) or 16-byte (fp32) write.  Tiles of x and w are staged through LDS
// (double-buffered, one barrier per K step, rows padded by 16 bytes); the
// next K step's global loads are in flight while the matrix cores work on the
// current one.  Workgroups are numbered so that consecutive tile ids share an
// XCD (blocks are dealt round-robin over the 8 XCDs) and tiles are visited in
// groups of 8 rows of tiles, so concurrently running tiles on one XCD share
// x and w slices in that XCD's L2.
#include "common.h"
#include "internal.h"

namespace hagemm {
namespace {

constexpr int kXcds = 8;
constexpr int kGroupM = 8;

__device__ __forceinline__ int xcd_logical(int bid, int total) {
    const int q = total / kXcds, rr = total % kXcds;
    const int xcd = bid % kXcds, idx = bid / kXcds;
    return xcd < rr ? xcd * (q + 1) + idx : rr * (q + 1) + (xcd - rr) * q + idx;
}

template <typename E, int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64, 1) void gemm_kernel(const E* __restrict__ x, const E* __restrict__ w,
                                                              E* __restrict__ y, int M, int N, int K, int tiles_m,
                                                              int tiles_n, const int32_t* __restrict__ row_slot,
                                                              float* __restrict__ ybase) {
    constexpr int NT = WM * WN * 64;
    constexpr int V = Elem<E>::kVec;
    constexpr int KG = 4 * V;
    constexpr int LDK = BK + V;  // padded LDS row (elements)
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int VPR = BK / V;  // vectors per tile row
    constexpr int XV = BM * VPR / NT, WV = BN * VPR / NT;
    static_assert(BM * VPR % NT == 0 && BN * VPR % NT == 0, "tile loads must divide evenly");
    static_assert(BK % KG == 0 && FM >= 1 && FN >= 1, "bad tile");
    __shared__ __align__(16) E sx[2][BM * LDK];
    __shared__ __align__(16) E sw[2][BN * LDK];

    const int total = tiles_m * tiles_n;
    const int t = xcd_logical(blockIdx.x, total);
    const int group = t / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int in_group = t - group * kGroupM * tiles_n;
    const int tm = first_m + in_group % gm, tn = in_group / gm;
    const int m0 = tm * BM, n0 = tn * BN;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int li = lane & 15, lg = lane >> 4;
    const u32x4 zero = {0u, 0u, 0u, 0u};

    u32x4 rx[XV], rw[WV];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int v = threadIdx.x + i * NT, row = v / VPR, kv = v - row * VPR;
            const int m = min(m0 + row, M - 1), k = k0 + kv * V;
            rx[i] = k < K ? ld16(x + (int64_t)m * K + k) : zero;
        }
#pragma unroll
        for (int i = 0; i < WV; ++i) {
            const int v = threadIdx.x + i * NT, row = v / VPR, kv = v - row * VPR;
            const int n = min(n0 + row, N - 1), k = k0 + kv * V;
            rw[i] = k < K ? ld16(w + (int64_t)n * K + k) : zero;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int v = threadIdx.x + i * NT, row = v / VPR, kv = v - row * VPR;
            *reinterpret_cast<u32x4*>(&sx[buf][row * LDK + kv * V]) = rx[i];
        }
#pragma unroll
        for (int i = 0; i < WV; ++i) {
            const int v = threadIdx.x + i * NT, row = v / VPR, kv = v - row * VPR;
            *reinterpret_cast<u32x4*>(&sw[buf][row * LDK + kv * V]) = rw[i];
        }
    };

    f32x4 acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const E* cw = sw[cur] + (wn * WTN + li) * LDK + V * lg;
        const E* cx = sx[cur] + (wm * WTM + li) * LDK + V * lg;
#pragma unroll
        for (int kg = 0; kg < BK; kg += KG) {
            u32x4 af[FN], bf[FM];
#pragma unroll
            for (int a = 0; a < FN; ++a) af[a] = *reinterpret_cast<const u32x4*>(cw + a * 16 * LDK + kg);
#pragma unroll
            for (int b = 0; b < FM; ++b) bf[b] = *reinterpret_cast<const u32x4*>(cx + b * 16 * LDK + kg);
#pragma unroll
            for (int a = 0; a < FN; ++a)
#pragma unroll
                for (int b = 0; b < FM; ++b) acc[a][b] = mma_step(af[a], bf[b], acc[a][b], E{});
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }
    // lane holds D[n = 4*lg + i][m = li] of each 16x16 block; rows with an
    // adapter go unrounded to ybase (the delta kernels round them once)
#pragma unroll
    for (int b = 0; b < FM; ++b) {
        const int m = m0 + wm * WTM + b * 16 + li;
        if (m >= M) continue;
        const bool raw = row_slot != nullptr && row_slot[m] >= 0;
#pragma unroll
        for (int a = 0; a < FN; ++a) {
            const int n = n0 + wn * WTN + a * 16 + 4 * lg;
            if (n >= N) continue;
            if (raw) {
                *reinterpret_cast<f32x4*>(ybase + (int64_t)m * N + n) = acc[a][b];
                continue;
            }
            E* yp = y + (int64_t)m * N + n;
            if constexpr (V == 8) {
                u32x2 o;
                o[0] = pack_bf16(acc[a][b][0], acc[a][b][1]);
                o[1] = pack_bf16(acc[a][b][2], acc[a][b][3]);
                *reinterpret_cast<u32x2*>(yp) = o;
            } else {
                *reinterpret_cast<f32x4*>(yp) = acc[a][b];
            }
        }
    }
}

template <typename E, int BM, int BN, int BK, int WM, int WN>
hipError_t run(const void* x, const void* w, void* y, int M, int N, int K, const int32_t* row_slot, float* ybase,
               hipStream_t s) {
    const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    hipLaunchKernelGGL((gemm_kernel<E, BM, BN, BK, WM, WN>), dim3(tm * tn), dim3(WM * WN * 64), 0, s,
                       static_cast<const E*>(x), static_cast<const E*>(w), static_cast<E*>(y), M, N, K, tm, tn,
                       row_slot, ybase);
    return hipGetLastError();
}

}  // namespace

// Tile choice by shape class: a wide tile keeps the matrix cores fed when the
// batch is long (prefill); short batches (decode) are bound by reading w once,
// so they take narrow N tiles to spread w over every CU.
hipError_t launch_gemm(int dtype, const void* x, const void* w, void* y, int64_t M64, int64_t N64, int64_t K64,
                       const int32_t* row_slot, float* ybase, hipStream_t s) {
    const int M = (int)M64, N = (int)N64, K = (int)K64;
    if (dtype == 1) {
        if (M > 256) return run<bf16_t, 256, 256, 64, 2, 2>(x, w, y, M, N, K, row_slot, ybase, s);
        if (M > 64) return run<bf16_t, 256, 64, 64, 4, 1>(x, w, y, M, N, K, row_slot, ybase, s);
        return run<bf16_t, 64, 16, 256, 4, 1>(x, w, y, M, N, K, row_slot, ybase, s);
    }
    if (M > 64) return run<float, 128, 128, 32, 2, 2>(x, w, y, M, N, K, row_slot, ybase, s);
    return run<float, 64, 16, 64, 4, 1>(x, w, y, M, N, K, row_slot, ybase, s);
}

}  // namespace hagemm
