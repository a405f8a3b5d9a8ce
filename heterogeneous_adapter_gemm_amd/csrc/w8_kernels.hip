// The shared base product with an FP8 base weight: y[M][N] = s[n] * sum_k
// x[m][k] * e4m3(q[n][k]), bf16 x, the base weight stored as 8-bit E4M3 codes
// q[N][K] with one fp32 scale s[n] per output channel, fp32 accumulation.  A
// base served quantized while the adapters stay 16-bit ("Multi-LoRA serving:
// S-LoRA, Punica and adapter batching", Interaction with how the adapters were
// trained).  Decode batches are bound by reading the base weight once, so the
// codes halve the bytes that bound them; x keeps its bf16 precision.
//
// The matrix cores run bf16: each lane widens its 8 codes of a K step to bf16
// in registers (v_cvt_pk_f32_fp8, exact for every E4M3 value, then the exact
// fp32 -> bf16 conversion) and the scale is applied to the fp32 accumulators.
//
// gemm_w8_kernel<BM, BK, NB>: one workgroup per 16 NB columns of y (rows of q)
// and BM rows of x (64, 128 or 256), all of K, four waves.  The waves split
// the work of a stage (BK-deep in K: BK / 32 matrix-op K steps) by column
// block, K step and row part, so that each wave holds four 16 x 16 output
// blocks and feeds every q fragment it widens to four matrix ops; where waves
// split K, their partial sums meet in LDS after the K loop and are added in
// wave order.  Both operands go through LDS by direct loads, four stages of
// them: x (BM rows of 2 BK bytes, 16-byte chunks XOR-swizzled as in the bf16
// decode tile) and q (16 NB rows of BK bytes, wave w loading its own rows; a
// wave whose rows take less than a 1 KB wave-load repeats them into the
// slot's unused part, so every wave issues the same loads per step and one
// wait count per step holds).  Each step reads its fragments before it
// issues the next loads: the loads in flight at the reads then target other
// stages only, which the compiler can see, so the reads wait for nothing
// more.  Each column tile starts its K loop at its own offset, so the
// workgroups do not all read the same slice of x at once.
#include "bgmv_device.h"
#include "common.h"
#include "internal.h"

namespace hagemm {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16_pair(f32x2 v) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// eight E4M3 codes (two dwords, code i in byte i) -> eight bf16 (four dwords)
__device__ __forceinline__ u32x4 widen_e4m3(uint32_t lo, uint32_t hi) {
    u32x4 r;
    r[0] = bf16_pair(__builtin_amdgcn_cvt_pk_f32_fp8(lo, false));
    r[1] = bf16_pair(__builtin_amdgcn_cvt_pk_f32_fp8(lo, true));
    r[2] = bf16_pair(__builtin_amdgcn_cvt_pk_f32_fp8(hi, false));
    r[3] = bf16_pair(__builtin_amdgcn_cvt_pk_f32_fp8(hi, true));
    return r;
}

constexpr int kW8Stages = 4;

// BM rows of x, BK-deep stages, NB blocks of 16 output columns per workgroup.
template <int BM, int BK, int NB>
struct W8Cfg {
    static constexpr int XB = BM * BK * 2;                   // x bytes per stage
    static constexpr int R = 4 * NB;                         // q rows each wave loads
    static constexpr int QL = R * BK >= 1024 ? R * BK / 1024 : 1;   // its q wave-loads per step
    static constexpr int QB = 4 * QL * 1024;                 // q bytes per stage (with unused halves)
    static constexpr int LDS = kW8Stages * (XB + QB);
    static constexpr int OCC = LDS <= 80 * 1024 ? 2 : 1;      // workgroups per CU the LDS allows
};

// One workgroup's tile: workgroup bid of the nblocks that run the product.  Rows whose
// delta comes later stay unrounded in ybase: rows with row_slot[m] >= 0, or (row_slot NULL,
// at most 64 rows) the rows whose bit is set in raw_mask.
template <int BM, int BK, int NB>
__device__ __forceinline__ void w8_tile(const bf16_t* __restrict__ x, const uint8_t* __restrict__ q,
                                        const float* __restrict__ scale, bf16_t* __restrict__ y, int M, int N, int K,
                                        const int32_t* __restrict__ row_slot, uint64_t raw_mask,
                                        float* __restrict__ ybase, int bid, int nblocks) {
    using C = W8Cfg<BM, BK, NB>;
    constexpr int S = kW8Stages;
    constexpr int RBX = 2 * BK;          // bytes of an x row per stage
    constexpr int CPX = RBX / 16;        // its 16-byte chunks
    constexpr int RPLX = 1024 / RBX;     // x rows per wave-load (64 lanes x 16 B)
    constexpr int XB = C::XB;
    constexpr int LPX = XB / 1024 / 4;   // x wave-loads per wave per stage
    constexpr int CPW = BK / 16;         // 16-byte chunks of a q row per stage
    constexpr int R = C::R, QL = C::QL, QB = C::QB;
    constexpr int RPLQ = R * BK >= 1024 ? 1024 / BK : R;   // q rows per wave-load
    constexpr int KS = BK / 32;          // matrix-op K steps per stage
    constexpr int KG = KS < 4 / NB ? KS : 4 / NB;   // waves splitting a stage's K steps
    constexpr int KW = KS / KG;          // K steps per wave per stage
    constexpr int MS = 4 / (NB * KG);    // row parts
    constexpr int FM = BM / MS / 16;     // 16-row blocks per wave
    constexpr int L = LPX + QL;          // loads per wave per step
    static_assert(RBX <= 1024 && LPX * 4 * 1024 == XB && NB * KG * MS == 4 && KG * KW == KS && FM == 4, "tile layout");
    static_assert(RPLQ * BK <= 1024 && QL * RPLQ == R, "q layout");
    constexpr int ST = XB + QB;
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[ST];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[ST];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[S > 2 ? ST : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[S > 3 ? ST : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds4[S > 4 ? ST : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds5[S > 5 ? ST : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds6[S > 6 ? ST : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds7[S > 7 ? ST : 16];
    auto stage = [&](int st) -> uint8_t* {
        return st == 0 ? lds0 : st == 1 ? lds1 : st == 2 ? lds2 : st == 3 ? lds3 :
               st == 4 ? lds4 : st == 5 ? lds5 : st == 6 ? lds6 : lds7;
    };
    auto qstage = [&](int st) -> uint8_t* { return stage(st) + XB; };

    // workgroup -> (column tile, row block): the row blocks of a column tile get consecutive
    // logical ids on one XCD, so they stream the same q slab through that XCD's L2 together
    const int row_blocks = (M + BM - 1) / BM;
    const int tiles_n = nblocks / row_blocks;
    const int lid = xcd_logical(bid, nblocks);
    const int tn = lid / row_blocks;
    const int n0 = tn * 16 * NB, m0 = (lid % row_blocks) * BM;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int kq = wave % KG, mq = (wave / KG) % MS, nb = wave / (KG * MS);
    // x: lane -> (row, slot) of each wave-load; slot p of row r holds chunk p ^ ((r / 2) % CPX)
    int xoff[LPX];
#pragma unroll
    for (int i = 0; i < LPX; ++i) {
        const int row = (wave * LPX + i) * RPLX + lane / CPX, slot = lane % CPX;
        xoff[i] = (min(m0 + row, M - 1) * K + (slot ^ ((row / 2) % CPX)) * 8) * 2;
    }
    // q: lane -> (row, slot) of each of the wave's loads; slot p of tile row r holds chunk
    // p ^ (r % CPW); lanes past a load's rows repeat them into the slot's unused part
    int qoff[QL];
#pragma unroll
    for (int i = 0; i < QL; ++i) {
        const int l = lane % (RPLQ * CPW);
        const int row = R * wave + RPLQ * i + l / CPW, slot = l % CPW;
        qoff[i] = min(n0 + row, N - 1) * K + (slot ^ (row % CPW)) * 16;
    }
    const int nk = K / BK;
    const int kshift = (int)(((int64_t)tn * nk) / tiles_n);
    auto issue = [&](int kt, int si) {
        int ke = kt + kshift;
        if (ke >= nk) ke -= nk;
        uint8_t* st = stage(si);
#pragma unroll
        for (int i = 0; i < LPX; ++i) buffer_load_lds16(x, M * K * 2, st + (wave * LPX + i) * 1024, xoff[i], ke * BK * 2);
#pragma unroll
        for (int i = 0; i < QL; ++i) buffer_load_lds16(q, N * K, qstage(si) + (wave * QL + i) * 1024, qoff[i], ke * BK);
    };

    f32x4 acc[FM];
#pragma unroll
    for (int b = 0; b < FM; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    // this wave's fragments of a stage: rows of part mq, column block nb, K steps kq + KG t
    int xfrag[KW][FM], qfrag[KW];
    {
        const int r = nb * 16 + li;   // tile row of q
        const int qbase = ((r / R) * QL + (r % R) / RPLQ) * 1024 + (r % RPLQ) * BK + (lg & 1) * 8;
#pragma unroll
        for (int t = 0; t < KW; ++t) {
            const int kstep = kq + KG * t;
            qfrag[t] = qbase + (((2 * kstep + (lg >> 1)) ^ (r % CPW)) * 16);
#pragma unroll
            for (int b = 0; b < FM; ++b) {
                const int row = (mq * FM + b) * 16 + li;
                xfrag[t][b] = row * RBX + (((kstep * 4 + lg) ^ ((row / 2) % CPX)) * 16);
            }
        }
    }
    u32x4 bf[KW][FM];
    u32x2 qv[KW];
    auto read_frags = [&](int st) {
#pragma unroll
        for (int t = 0; t < KW; ++t) {
            qv[t] = *reinterpret_cast<const u32x2*>(qstage(st) + qfrag[t]);
#pragma unroll
            for (int b = 0; b < FM; ++b) bf[t][b] = *reinterpret_cast<const u32x4*>(stage(st) + xfrag[t][b]);
        }
    };
    auto mma = [&]() {
#pragma unroll
        for (int t = 0; t < KW; ++t) {
            const u32x4 af = widen_e4m3(qv[t][0], qv[t][1]);
#pragma unroll
            for (int b = 0; b < FM; ++b) acc[b] = mma_step(af, bf[t][b], acc[b], bf16_t{});
        }
    };
    // One step: wait for step j's loads (this wave's, then every wave's at the barrier, which
    // also says every wave is done with step j - 1), read its fragments, refill the stage
    // step j - 1 used with step j + S - 1 (past the end: the last step again, into a stage
    // not read again, so every step issues one load group and the wait counts never
    // change), multiply.  The fragments are read before the new loads are issued: the loads
    // outstanding at the reads then target other stages only, and the reads need not wait
    // for them.  Whole groups of S steps run in a loop with no branch inside; the last
    // nk % S steps after it.
    auto step = [&](int j, int st) {
        wait_vmcnt<(S - 2) * L>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        read_frags(st);
        __builtin_amdgcn_sched_barrier(0);
        issue(min(j + S - 1, nk - 1), (st + S - 1) % S);
        mma();
    };
#pragma unroll
    for (int p = 0; p < S - 1; ++p) issue(min(p, nk - 1), p);
    const int nfull = nk - nk % S;
    for (int i = 0; i < nfull; i += S) {
#pragma unroll
        for (int st = 0; st < S; ++st) step(i + st, st);
    }
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
        if (nfull + st < nk) step(nfull + st, st);
    wait_vmcnt<0>();  // no direct load may still be writing LDS when the workgroup ends

    // lane holds D[n = 4 lg + i][m = li] of each 16 x 16 block.  The KG waves of a (row part,
    // column block) hold partial sums over their K steps: the ones past the first put theirs
    // in LDS (the stages are free: every load has landed and, after the barrier, every wave
    // is done reading), and the first adds them in wave order.
    if constexpr (KG > 1) {
        static_assert(4 * FM * 4 * 64 * 4 <= XB, "partial sums fit a stage");
        __syncthreads();
        float* part = reinterpret_cast<float*>(lds0);   // [wave][FM][4][64]
        if (kq > 0) {
#pragma unroll
            for (int b = 0; b < FM; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) part[((wave * FM + b) * 4 + i) * 64 + lane] = acc[b][i];
        }
        __syncthreads();
        if (kq > 0) return;
#pragma unroll
        for (int o = 1; o < KG; ++o)
#pragma unroll
            for (int b = 0; b < FM; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[b][i] += part[(((wave + o) * FM + b) * 4 + i) * 64 + lane];
    }
    // rows whose delta comes later (row_slot >= 0) stay unrounded in ybase
    const int n = n0 + nb * 16 + 4 * lg;
    if (n >= N) return;
    const f32x4 sc = *reinterpret_cast<const f32x4*>(scale + n);
#pragma unroll
    for (int b = 0; b < FM; ++b) {
        const int m = m0 + (mq * FM + b) * 16 + li;
        if (m >= M) continue;
        f32x4 d;
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = acc[b][i] * sc[i];
        const int64_t off = (int64_t)m * N + n;
        const bool raw = row_slot != nullptr ? row_slot[m] >= 0 : m < 64 && ((raw_mask >> m) & 1) != 0;
        if (raw) {
            *reinterpret_cast<f32x4*>(ybase + off) = d;
        } else {
            u32x2 o;
            o[0] = bf16_pair(f32x2{d[0], d[1]});
            o[1] = bf16_pair(f32x2{d[2], d[3]});
            *reinterpret_cast<u32x2*>(y + off) = o;
        }
    }
}

template <int BM, int BK, int NB>
__global__ __launch_bounds__(256, (W8Cfg<BM, BK, NB>::OCC)) void gemm_w8_kernel(
    const bf16_t* __restrict__ x, const uint8_t* __restrict__ q, const float* __restrict__ scale,
    bf16_t* __restrict__ y, int M, int N, int K, const int32_t* __restrict__ row_slot, float* __restrict__ ybase) {
    w8_tile<BM, BK, NB>(x, q, scale, y, M, N, K, row_slot, 0, ybase, blockIdx.x, gridDim.x);
}

// Decode batches of up to 64 rows: the FP8 product's tiles, the BGMV shrink's units and the
// copy of a plan's index in one launch, as the bf16 decode launch does (blocks [0, n_gemm)
// are tiles, then the shrink units, then kCopyBlocks copying cp_n index words).
template <int NB>
__global__ __launch_bounds__(256, (W8Cfg<64, 128, NB>::OCC)) void gemm_w8_shrink_kernel(
    const bf16_t* __restrict__ x, const uint8_t* __restrict__ q, const float* __restrict__ scale,
    bf16_t* __restrict__ y, int M, int N, int K, const int32_t* __restrict__ row_slot, uint64_t raw_mask,
    float* __restrict__ ybase, LoraArgs a, int n_gemm, const uint32_t* __restrict__ cp_src,
    uint32_t* __restrict__ cp_dst, int cp_n) {
    const int b = blockIdx.x;
    if (b < n_gemm)
        w8_tile<64, 128, NB>(x, q, scale, y, M, N, K, row_slot, raw_mask, ybase, b, n_gemm);
    else if (b < n_gemm + a.n_su)
        bgmv_shrink_unit<bf16_t, true>(a, b - n_gemm);
    else
        copy_words(cp_src, cp_dst, cp_n, b - n_gemm - a.n_su);
}

// columns per workgroup of the decode tiles for N output columns (see launch_gemm_w8)
int w8_decode_nb(int N) { return N >= 64 * 160 ? 4 : N >= 32 * 256 ? 2 : 1; }

}  // namespace

bool gemm_w8_ok(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || N < 1 || N % 4 || K < 128 || K % 128) return false;
    return M * K * 2 < INT32_MAX && N * K < INT32_MAX;
}

hipError_t launch_gemm_w8(const void* x, const void* q, const float* scale, void* y, int64_t M64, int64_t N64,
                          int64_t K64, const int32_t* row_slot, float* ybase, hipStream_t s) {
    if (!gemm_w8_ok(M64, N64, K64)) return hipErrorInvalidValue;
    const int M = (int)M64, N = (int)N64, K = (int)K64;
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const uint8_t* qb = static_cast<const uint8_t*>(q);
    bf16_t* yb = static_cast<bf16_t*>(y);
    auto go = [&](auto kern, int bn, int bm) {
        const int64_t grid = (int64_t)((N + bn - 1) / bn) * ((M + bm - 1) / bm);
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, s, xb, qb, scale, yb, M, N, K, row_slot, ybase);
    };
    // Up to 256 rows: 64-row blocks, 16, 32 or 64 columns per workgroup, the widest that
    // still gives about 160 workgroups or more per row block (each workgroup streams all of
    // its rows of x through its CU, so wider tiles move fewer x bytes per q byte; too few
    // workgroups leave CUs idle).  Measured on MI355X, 64 rows: 4096 x 4096 12.8 us with 16
    // columns (14.2 with 32, 19.5 with 64); 4096 -> 11008 20.3 us with 64 (26.8 with 32,
    // 31.3 with 16).  Longer batches: 256-row blocks.
    if (M <= 256) {
        const int nb = w8_decode_nb(N);
        if (nb == 4) go(gemm_w8_kernel<64, 128, 4>, 64, 64);
        else if (nb == 2) go(gemm_w8_kernel<64, 128, 2>, 32, 64);
        else go(gemm_w8_kernel<64, 128, 1>, 16, 64);
    } else {
        go(gemm_w8_kernel<256, 32, 1>, 16, 256);
    }
    return hipGetLastError();
}

bool gemm_w8_shrink_fits(int64_t M, int64_t N, int64_t K, int n_su) {
    return M >= 1 && M <= 64 && n_su > 0 && gemm_w8_ok(M, N, K);
}

hipError_t launch_gemm_w8_shrink(const void* x, const void* q, const float* scale, void* y, int64_t M64, int64_t N64,
                                 int64_t K64, const int32_t* row_slot, uint64_t raw_mask, float* ybase,
                                 const LoraArgs& a, const void* cp_src, void* cp_dst, int64_t cp_n, hipStream_t s) {
    if (!gemm_w8_shrink_fits(M64, N64, K64, a.n_su) || cp_n < 0 || cp_n > INT32_MAX) return hipErrorInvalidValue;
    const int M = (int)M64, N = (int)N64, K = (int)K64;
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const uint8_t* qb = static_cast<const uint8_t*>(q);
    bf16_t* yb = static_cast<bf16_t*>(y);
    const uint32_t* cs = static_cast<const uint32_t*>(cp_src);
    uint32_t* cd = static_cast<uint32_t*>(cp_dst);
    const int ncp = cp_n > 0 ? kCopyBlocks : 0;
    const int* rs = raw_mask != 0 ? nullptr : row_slot;
    const int nb = w8_decode_nb(N);
    const int tn = (N + 16 * nb - 1) / (16 * nb);
    const dim3 grid(tn + a.n_su + ncp);
    if (nb == 4)
        hipLaunchKernelGGL(gemm_w8_shrink_kernel<4>, grid, dim3(256), 0, s, xb, qb, scale, yb, M, N, K, rs, raw_mask,
                           ybase, a, tn, cs, cd, (int)cp_n);
    else if (nb == 2)
        hipLaunchKernelGGL(gemm_w8_shrink_kernel<2>, grid, dim3(256), 0, s, xb, qb, scale, yb, M, N, K, rs, raw_mask,
                           ybase, a, tn, cs, cd, (int)cp_n);
    else
        hipLaunchKernelGGL(gemm_w8_shrink_kernel<1>, grid, dim3(256), 0, s, xb, qb, scale, yb, M, N, K, rs, raw_mask,
                           ybase, a, tn, cs, cd, (int)cp_n);
    return hipGetLastError();
}

}  // namespace hagemm
