// The shared base product y[M][N] = x[M][K] * w[N][K]^T on the gfx950 matrix
// cores: one dense GEMM over the whole batch that reads the base weight once
// ("Multi-LoRA serving: S-LoRA, Punica and adapter batching", The bottleneck).
//
// Both operands are K-contiguous, so either can feed either side of an MFMA.
// All kernels put w on the MFMA's M side and x on its N side: a lane then
// ends with four consecutive output columns of one row, stored as one 8-byte
// (bf16) or 16-byte (fp32) write.
//
//  * gemm_lds_kernel (long batches, bf16, K % 128 == 0): 256 x 256 tiles, 8
//    waves of 64 x 128, one workgroup per CU.  Tiles stream into LDS with
//    direct loads (buffer_load_dwordx4 ... lds: no VGPR staging), four
//    stages of K = 32, so three steps of loads are in flight behind the
//    matrix cores; rows of 64 B with the 16-byte chunks XOR-swizzled so
//    fragment reads are free of bank conflicts.  The partial last round of
//    tiles runs as 256 x 128 half tiles.  Optionally adds the prefill
//    segments' LoRA expand in its epilogue (see below), so those rows are
//    rounded once and written once.
//  * gemm_xlds_kernel (65 to 256 rows, bf16, K % 64 == 0): x and w through
//    LDS by direct loads of whole 128-byte row segments; x is shared by the
//    four waves, each wave's w rows go to a region of its own.
//  * gemm_tile_kernel: register-staged tiles (two K steps in flight) for any
//    K multiple of the vector width; short batches and fp32.
// Workgroups are numbered so that consecutive tile ids share an XCD (blocks
// are dealt round-robin over the 8 XCDs) and tiles are visited in groups of
// 8 rows of tiles, so concurrently running tiles on one XCD share x and w
// slices in that XCD's L2.
#include <type_traits>

#include "bgmv_device.h"

#include "common.h"
#include "internal.h"

namespace hagemm {
namespace {

constexpr int kGroupM = 8;

__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int t = xcd_logical(bid, tiles_m * tiles_n);
    const int group = t / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int in_group = t - group * kGroupM * tiles_n;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}


// store one lane's 4 consecutive outputs of row m: rounded to y, or (rows
// whose delta is still to come) unrounded to ybase
template <typename E>
__device__ __forceinline__ void store4(E* y, float* ybase, bool raw, int64_t off, const f32x4& d) {
    if (raw) {
        *reinterpret_cast<f32x4*>(ybase + off) = d;
    } else if constexpr (Elem<E>::kVec == 8) {
        u32x2 o;
        o[0] = pack_bf16(d[0], d[1]);
        o[1] = pack_bf16(d[2], d[3]);
        *reinterpret_cast<u32x2*>(y + off) = o;
    } else {
        *reinterpret_cast<f32x4*>(y + off) = d;
    }
}

// ---------------------------------------------------------------------------
// Long batches: direct-to-LDS bf16 GEMM with the prefill LoRA expand fused.
//
// Fused expand: after the K loop the LDS is free.  For each prefill segment
// overlapping the tile's rows, the workgroup stages in LDS the segment's B
// rows for the tile's 256 columns, transposed (bt[n][j]), and gamma * v for
// the tile's rows (the SGMV shrink's fp32 v, split into a high
// and a low bf16 half so the product keeps ~16 mantissa bits; rows outside
// the segment zero).  Each wave then adds sum_j bt[n][j] v[m][j] to its
// accumulators on the matrix cores (A side = bt, B side = v, K = rank).
//
// Tile shapes (LdsCfg): BM x BN tiles, BK-deep K steps in S stages, WM x WN
// waves of (BM / WM) x (BN / WN) outputs; UNIT_M x UNIT_N is the tile grid's
// unit (BM x BN for whole tiles; for the pieces of the tiles of the last round,
// the whole tile they are cut from, UNIT_M / BM x UNIT_N / BN pieces each); WPE
// is the waves per SIMD the register budget must allow.
// STAGGER: each column block starts its K loop at its own offset (wrapping around), so
// the workgroups do not all read the same slice of a small, L2-resident x at once.
template <int BM_, int BN_, int BK_, int S_, int WM_, int WN_, bool PIPE_, int UNIT_N_, int WPE_, bool STAGGER_ = false,
          int UNIT_M_ = BM_>
struct LdsCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, S = S_, WM = WM_, WN = WN_, UNIT_N = UNIT_N_, WPE = WPE_;
    static constexpr int UNIT_M = UNIT_M_;
    static constexpr bool PIPE = PIPE_, STAGGER = STAGGER_;
};
// long batches: 256 x 256 tiles, 8 waves, four stages of K = 32, pipelined fragment reads
using CfgLong = LdsCfg<256, 256, 32, 4, 4, 2, true, 256, 1>;
using CfgLongHalf = LdsCfg<256, 128, 32, 4, 4, 2, true, 256, 1>;
// smaller pieces of 256 x 256 tiles, for a last round of few tiles (4, 8 or 16 per tile)
using CfgLongQuarter = LdsCfg<128, 128, 32, 4, 4, 2, true, 256, 1, false, 256>;
using CfgLongEighth = LdsCfg<128, 64, 32, 4, 4, 2, true, 256, 1, false, 256>;
using CfgLongSixteenth = LdsCfg<64, 64, 32, 4, 4, 2, true, 256, 1, false, 256>;
// 192-row tiles: where 256-row tiles leave CUs idle in their last round (e.g. 2,961 rows x
// 4096 columns: 192 tiles of 256 x 256 for 256 CUs, 256 tiles of 192 x 256)
using CfgLong192 = LdsCfg<192, 256, 32, 4, 4, 2, true, 256, 1>;
using CfgLong192Half = LdsCfg<192, 128, 32, 4, 4, 2, true, 256, 1>;
// Decode batches of up to 64 rows: every workgroup streams 16 columns of W (all of K)
// past the whole batch, four waves, four stages of K = 128.  The base GEMM alone and the
// launch shared with the shrink units use this one configuration (same tiles, same K
// order), so their outputs agree bit for bit.
using CfgDecode64 = LdsCfg<64, 16, 128, 4, 4, 1, false, 16, 1, true>;

// The last round of tiles (long batches): with T whole tiles and C resident
// workgroups (one per CU), the first T - T % C tiles (in tile order) run
// whole; the remaining ones run in a second launch cut into P pieces each (P =
// 2, 4, 8 or 16: the most that the chip holds at once, at least 2), so the
// partial last round takes a fraction of a tile's time.  Workgroup b of a
// launch covers tile t0 + b (whole tiles; XCD-aware order) or piece b % P of
// tile t0 + b / P.
//
// S stages of BK-deep K steps: loads for step j + S - 1 are issued while step j
// is computed, so S - 1 steps of loads are in flight behind the matrix cores.
template <bool FUSE, class C>
__device__ __forceinline__ void gemm_lds_tile(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, bf16_t* __restrict__ y, int M, int N, int K,
    int tiles_m, int tiles_n, const int32_t* __restrict__ row_slot, float* __restrict__ ybase, const LoraArgs& seg,
    int t0, int count, int bid, uint64_t raw_mask = 0) {
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, WM = C::WM, WN = C::WN, S = C::S, UNIT_N = C::UNIT_N;
    constexpr int UNIT_M = C::UNIT_M, SUB_M = UNIT_M / BM, SUB_N = UNIT_N / BN, SUBS = SUB_M * SUB_N;
    constexpr bool PIPE = C::PIPE;
    static_assert(SUB_M * BM == UNIT_M && SUB_N * BN == UNIT_N, "pieces tile the unit");
    constexpr int NT = WM * WN * 64, NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 16, FN = WTN / 16;
    constexpr int RB = BK * 2;          // bytes per tile row
    constexpr int CPR = RB / 16;        // 16-byte chunks per row
    constexpr int RPL = 1024 / RB;      // rows per wave-load (64 lanes x 16 B)
    // rows sharing one swizzle value: with 2, the ds_read_b128 fragment reads of 64 B and
    // 128 B rows measure free of bank conflicts on gfx950 (4 and more conflict)
    constexpr int RPB = 2;
    // A stage is GX wave-loads of x rows then GW of w rows (1 KiB each).  When they split
    // evenly over the waves, wave v loads x wave-loads v*GX/NW.. and w wave-loads v*GW/NW..;
    // otherwise wave-load g goes to wave g % NW, and the waves left one short issue a load
    // at an offset past the end of the buffer (it reads nothing and writes zeros into a
    // spare KiB of the stage), so that every wave has the same loads in flight per step.
    constexpr int GX = BM / RPL, GW = BN / RPL, NL = GX + GW;
    constexpr bool EVEN = GX % NW == 0 && GW % NW == 0;
    constexpr int LP = (NL + NW - 1) / NW;  // wave-loads per wave per stage
    constexpr int SPARE = EVEN || LP * NW == NL ? 0 : 1024;
    constexpr int XB = BM * RB;
    // pieces of a tile reserve the whole tile's stage size
    constexpr int STAGE = (UNIT_M + UNIT_N) * RB + SPARE;
    static_assert(S >= 2 && S <= 8 && S * STAGE <= 160 * 1024, "LDS");
    static_assert(CPR >= 4 && RPB >= 1 && GX * RPL == BM && GW * RPL == BN, "load layout");
    static_assert(FM >= 1 && FN >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
    // one array per stage: distinct objects let the compiler see that the stage being
    // filled by direct loads is not the one being read, so reads need not wait for them
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[S > 2 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[S > 3 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds4[S > 4 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds5[S > 5 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds6[S > 6 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds7[S > 7 ? STAGE : 16];
    // stage s (a constant once the K loop is unrolled)
    auto stage = [&](int st) -> uint8_t* {
        return st == 0 ? lds0 : st == 1 ? lds1 : st == 2 ? lds2 : st == 3 ? lds3 :
               st == 4 ? lds4 : st == 5 ? lds5 : st == 6 ? lds6 : lds7;
    };

    // tile of this workgroup (tile grid in units of BM x UNIT_N)
    const int t = SUBS > 1 ? t0 + bid / SUBS : t0 + xcd_logical(bid, count);
    int tm, tn;
    {
        const int group = t / (kGroupM * tiles_n);
        const int first_m = group * kGroupM;
        const int gm = min(tiles_m - first_m, kGroupM);
        const int in_group = t - group * kGroupM * tiles_n;
        tm = first_m + in_group % gm;
        tn = in_group / gm;
    }
    const int piece = SUBS > 1 ? bid % SUBS : 0;
    const int m0 = tm * UNIT_M + (piece / SUB_N) * BM, n0 = tn * UNIT_N + (piece % SUB_N) * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int li = lane & 15, lg = lane >> 4;

    // lane -> (row, slot) of each wave-load; slot p of row r holds chunk p ^ ((r / RPB) % CPR)
    const int lrow = lane / CPR, lslot = lane % CPR;
    // even layout: x offsets xoff[q] and w offsets woff[q] of this wave's wave-loads
    constexpr int LPX = EVEN ? GX / NW : 1, LPW = EVEN ? GW / NW : 1;
    int xoff[LPX], woff[LPW];
    // uneven layout: per wave-load its source, offset and place in the stage
    constexpr int LPU = EVEN ? 1 : LP;
    int voff[LPU], lds_at[LPU], src_bytes[LPU];
    const bf16_t* src[LPU];
    if constexpr (EVEN) {
#pragma unroll
        for (int q = 0; q < LPX; ++q) {
            const int row = (wave * LPX + q) * RPL + lrow;
            xoff[q] = (min(m0 + row, M - 1) * K + (lslot ^ ((row / RPB) % CPR)) * 8) * 2;
        }
#pragma unroll
        for (int q = 0; q < LPW; ++q) {
            const int row = (wave * LPW + q) * RPL + lrow;
            woff[q] = (min(n0 + row, N - 1) * K + (lslot ^ ((row / RPB) % CPR)) * 8) * 2;
        }
    } else {
        const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
        for (int q = 0; q < LP; ++q) {
            const int g = q * NW + wv;
            const bool isw = g >= GX && g < NL;
            const int row = (isw ? g - GX : g) * RPL + lrow;
            const int lim = isw ? N - 1 : M - 1, base = isw ? n0 : m0;
            voff[q] = g < NL ? (min(base + row, lim) * K + (lslot ^ ((row / RPB) % CPR)) * 8) * 2
                             : (int)0x80000000u;   // past the end of x (its size is below 2^31 bytes)
            // the wave-load's source, size and place as wave-uniform (scalar) values
            const uint64_t p = reinterpret_cast<uint64_t>(isw ? w : x);
            const uint32_t plo = __builtin_amdgcn_readfirstlane((uint32_t)p);
            const uint32_t phi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
            src[q] = reinterpret_cast<const bf16_t*>(((uint64_t)phi << 32) | plo);
            src_bytes[q] = __builtin_amdgcn_readfirstlane(isw ? N * K * 2 : M * K * 2);
            lds_at[q] = __builtin_amdgcn_readfirstlane(g < NL ? g * 1024 : (UNIT_M + UNIT_N) * RB);
        }
    }
    // one K step: LP wave-loads of 1 KiB per wave, the K offset in the scalar operand
    const int nk_all = K / BK;
    const int kshift = C::STAGGER ? (int)(((int64_t)tn * nk_all) / tiles_n) : 0;
    auto issue = [&](int kt, uint8_t* bx) {
        int ke = kt + kshift;
        if (ke >= nk_all) ke -= nk_all;
        const int kb = ke * BK * 2;
        if constexpr (EVEN) {
            uint8_t* bw = bx + XB;
#pragma unroll
            for (int q = 0; q < LPX; ++q) buffer_load_lds16(x, M * K * 2, bx + (wave * LPX + q) * 1024, xoff[q], kb);
#pragma unroll
            for (int q = 0; q < LPW; ++q) buffer_load_lds16(w, N * K * 2, bw + (wave * LPW + q) * 1024, woff[q], kb);
        } else {
#pragma unroll
            for (int q = 0; q < LP; ++q) buffer_load_lds16(src[q], src_bytes[q], bx + lds_at[q], voff[q], kb);
        }
    };

    f32x4 acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // swizzle of a fragment row: rows base + li with base a multiple of 16 share it when
    // 16 / RPB is a multiple of CPR (then it depends on li only); otherwise on the base too
    auto swz = [&](int base_row) { return (((16 / RPB) % CPR == 0 ? li : base_row + li) / RPB) % CPR; };
    auto compute = [&](const uint8_t* stage) {
        const uint8_t* bx = stage + (wm * WTM + li) * RB;
        const uint8_t* bw = stage + XB + (wn * WTN + li) * RB;
#pragma unroll
        for (int kg = 0; kg < CPR / 4; ++kg) {
            u32x4 bf[FM];
#pragma unroll
            for (int b = 0; b < FM; ++b)
                bf[b] = *reinterpret_cast<const u32x4*>(bx + b * 16 * RB + ((kg * 4 + lg) ^ swz(wm * WTM + b * 16)) * 16);
#pragma unroll
            for (int a = 0; a < FN; ++a) {
                const u32x4 af =
                    *reinterpret_cast<const u32x4*>(bw + a * 16 * RB + ((kg * 4 + lg) ^ swz(wn * WTN + a * 16)) * 16);
#pragma unroll
                for (int b = 0; b < FM; ++b) acc[a][b] = mma_step(af, bf[b], acc[a][b], bf16_t{});
            }
        }
    };

    // The loop has one exit, so the accumulators stay in place.  Every step issues one load
    // group, so the wait counts are the same in every step: past the end the group re-reads
    // the last step into a stage that is not read again.
    constexpr int L = LP;  // loads per wave per step
    const int nk = K / BK;
    if constexpr (!PIPE) {
        // K / BK need not be a multiple of S here: steps past the end only wait and refill
#pragma unroll
        for (int p = 0; p < S - 1; ++p) issue(min(p, nk - 1), stage(p));
        for (int i = 0; i < nk; i += S) {
#pragma unroll
            for (int st = 0; st < S; ++st) {
                const int j = i + st;
                // this wave's loads of step j are done (those of the S - 2 later steps may not be)
                wait_vmcnt<(S - 2) * L>();
                // every wave's loads of step j are in LDS, and every wave is done with step j - 1
                __builtin_amdgcn_s_barrier();
                // refill the stage step j - 1 used
                issue(min(j + S - 1, nk - 1), stage((st + S - 1) % S));
                if (j < nk) compute(stage(st));
            }
        }
    } else {
        // Fragments of step j + 1 are read from LDS while the matrix cores work on step j, and
        // all S stages hold loads in flight: step j + S is issued into step j's stage once
        // every wave holds step j's fragments in registers.  K / BK is a multiple of S.
        static_assert(CPR == 4 && (16 / RPB) % CPR == 0, "one MFMA K step per stage, swizzle by li");
        const int off = (lg ^ ((li / RPB) % CPR)) * 16;
        auto read_frags = [&](const uint8_t* stg, u32x4 (&af)[FN], u32x4 (&bf)[FM]) {
            const uint8_t* bx = stg + (wm * WTM + li) * RB + off;
            const uint8_t* bw = stg + XB + (wn * WTN + li) * RB + off;
#pragma unroll
            for (int b = 0; b < FM; ++b) bf[b] = *reinterpret_cast<const u32x4*>(bx + b * 16 * RB);
#pragma unroll
            for (int a = 0; a < FN; ++a) af[a] = *reinterpret_cast<const u32x4*>(bw + a * 16 * RB);
        };
        auto mma = [&](const u32x4 (&af)[FN], const u32x4 (&bf)[FM]) {
#pragma unroll
            for (int a = 0; a < FN; ++a)
#pragma unroll
                for (int b = 0; b < FM; ++b) acc[a][b] = mma_step(af[a], bf[b], acc[a][b], bf16_t{});
        };
        u32x4 af0[FN], bf0[FM], af1[FN], bf1[FM];
#pragma unroll
        for (int p = 0; p < S; ++p) issue(min(p, nk - 1), stage(p));
        wait_vmcnt<(S - 1) * L>();
        __builtin_amdgcn_s_barrier();
        read_frags(stage(0), af0, bf0);
        for (int i = 0; i < nk; i += S) {
#pragma unroll
            for (int st = 0; st < S; ++st) {
                const int j = i + st;
                // no instruction moves across the wait and barrier (the scheduler would otherwise
                // hoist the next step's matrix ops above them, together with the waits they need)
                __builtin_amdgcn_sched_barrier(0);
                // this wave's loads of step j + 1 are done, and so are its fragment reads of step j
                wait_vmcnt_lgkm0<(S - 2) * L>();
                // every wave's loads of step j + 1 are in LDS; every wave holds step j's fragments
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                issue(min(j + S, nk - 1), stage(st));
                if (st % 2 == 0) {
                    read_frags(stage((st + 1) % S), af1, bf1);
                    mma(af0, bf0);
                } else {
                    read_frags(stage((st + 1) % S), af0, bf0);
                    mma(af1, bf1);
                }
                // order: the direct loads, then each fragment read followed by two matrix ops,
                // so the reads finish while the rest of the step's matrix ops run
                __builtin_amdgcn_sched_group_barrier(0x020, L, 0);
#pragma unroll
                for (int q = 0; q < FN + FM; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                }
            }
        }
    }
    // no direct load may still be writing LDS when it is reused or released
    wait_vmcnt<0>();

    if constexpr (FUSE) {
        // LDS after the K loop, per 32-wide slice of the rank: bt[n][j] = B[j0+j][n0+n],
        // vh/vl[m][j] = high/low bf16 halves of gamma * v[m0+m][j0+j] for rows of the segment
        // (zero elsewhere and past the rank).  Rows of 40 bf16 (80 B): fragment reads are
        // free of bank conflicts.
        constexpr int LDJ = 40;
        static_assert(BN * LDJ * 2 <= STAGE && (S > 2 ? 1 : 2) * BM * LDJ * 2 <= STAGE, "fused epilogue LDS");
        uint16_t* bt = reinterpret_cast<uint16_t*>(lds0);
        uint16_t* vh = reinterpret_cast<uint16_t*>(lds1);
        uint16_t* vl = S > 2 ? reinterpret_cast<uint16_t*>(lds2) : vh + BM * LDJ;
        const int pmask = (1 << seg.page_shift) - 1;
        for (int s = 0; s < seg.n_segs; ++s) {
            const int sb = seg.s_begin[s], se = seg.s_end[s];
            if (se <= m0 || sb >= m0 + BM) continue;
            const int slot = seg.s_slot[s], r = seg.s_rank[s];
            const float gamma = seg.s_gamma[s];
            const int32_t* tabB =
                seg.page_tab + (int64_t)slot * seg.slot_cap + (int64_t)r * seg.lp_per_rank + r * seg.nci;
            for (int jb = 0; jb < r; jb += 32) {
                __syncthreads();  // LDS free: the K loop, or the previous slice, is done with it
                // item = (pair of rank-rows jp, 8 columns nv): the two rows' values of a column
                // go to LDS as one 32-bit word; the lanes of a wave run along the pairs, so the
                // stores of one instruction fall in distinct banks (at most two-way)
                static_assert(LDJ % 2 == 0, "word-aligned rows");
                uint32_t* btw = reinterpret_cast<uint32_t*>(bt);
                for (int idx = threadIdx.x; idx < 16 * (BN / 8); idx += NT) {
                    const int jp = idx & 15, nv = idx >> 4;
                    const int n = min(n0 + nv * 8, N - 8);
                    const int pg = n >> seg.page_shift, po = n & pmask;
                    const int j0 = jb + 2 * jp;
                    const bf16_t* pages = static_cast<const bf16_t*>(seg.pages);
                    u32x4 v0 = ld16(pages + ((int64_t)tabB[min(j0, r - 1) * seg.nco + pg] << seg.page_shift) + po);
                    u32x4 v1 = ld16(pages + ((int64_t)tabB[min(j0 + 1, r - 1) * seg.nco + pg] << seg.page_shift) + po);
                    const bool nin = n0 + nv * 8 < N;
                    if (j0 >= r || !nin) v0 = u32x4{0u, 0u, 0u, 0u};
                    if (j0 + 1 >= r || !nin) v1 = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        btw[(nv * 8 + 2 * e) * (LDJ / 2) + jp] = (v0[e] & 0xFFFFu) | (v1[e] << 16);
                        btw[(nv * 8 + 2 * e + 1) * (LDJ / 2) + jp] = (v0[e] >> 16) | (v1[e] & 0xFFFF0000u);
                    }
                }
                for (int idx = threadIdx.x; idx < BM * 4; idx += NT) {
                    const int ml = idx >> 2, j = (idx & 3) * 8;
                    const int m = m0 + ml;
                    float vv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) vv[e] = 0.f;
                    if (m >= sb && m < se) {
                        const float* vp = seg.v + (int64_t)m * seg.vstride + jb + j;
                        const f32x4 q0 = *reinterpret_cast<const f32x4*>(vp);
                        const f32x4 q1 = *reinterpret_cast<const f32x4*>(vp + 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            vv[e] = jb + j + e < r ? q0[e] : 0.f;
                            vv[4 + e] = jb + j + 4 + e < r ? q1[e] : 0.f;
                        }
                    }
                    u32x4 hi, lo;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float a0 = gamma * vv[2 * i], a1 = gamma * vv[2 * i + 1];
                        const uint32_t h0 = f32_to_bf16(a0), h1 = f32_to_bf16(a1);
                        hi[i] = h0 | (h1 << 16);
                        lo[i] = pack_bf16(a0 - __uint_as_float(h0 << 16), a1 - __uint_as_float(h1 << 16));
                    }
                    *reinterpret_cast<u32x4*>(&vh[ml * LDJ + j]) = hi;
                    *reinterpret_cast<u32x4*>(&vl[ml * LDJ + j]) = lo;
                }
                __syncthreads();
                const int j0 = 8 * lg;
                u32x4 vhi[FM], vlo[FM];
#pragma unroll
                for (int b = 0; b < FM; ++b) {
                    vhi[b] = *reinterpret_cast<const u32x4*>(&vh[(wm * WTM + b * 16 + li) * LDJ + j0]);
                    vlo[b] = *reinterpret_cast<const u32x4*>(&vl[(wm * WTM + b * 16 + li) * LDJ + j0]);
                }
#pragma unroll
                for (int a = 0; a < FN; ++a) {
                    const u32x4 bfr = *reinterpret_cast<const u32x4*>(&bt[(wn * WTN + a * 16 + li) * LDJ + j0]);
#pragma unroll
                    for (int b = 0; b < FM; ++b) {
                        acc[a][b] = mma_step(bfr, vhi[b], acc[a][b], bf16_t{});
                        acc[a][b] = mma_step(bfr, vlo[b], acc[a][b], bf16_t{});
                    }
                }
            }
        }
    }

    // lane holds D[n = 4*lg + i][m = li] of each 16x16 block
#pragma unroll
    for (int b = 0; b < FM; ++b) {
        const int m = m0 + wm * WTM + b * 16 + li;
        if (m >= M) continue;
        // rows whose delta comes later (decode rows with an adapter) stay unrounded
        // (raw_mask: batches of up to 64 rows, bit m set for rows with an adapter)
        const bool raw = row_slot != nullptr ? row_slot[m] >= 0 && (!FUSE || m >= seg.T_pre)
                                             : m < 64 && ((raw_mask >> m) & 1) != 0;
#pragma unroll
        for (int a = 0; a < FN; ++a) {
            const int n = n0 + wn * WTN + a * 16 + 4 * lg;
            if (n < N) store4(y, ybase, raw, (int64_t)m * N + n, acc[a][b]);
        }
    }
}

template <bool FUSE, class C>
__global__ __launch_bounds__(C::WM* C::WN * 64, C::WPE) void gemm_lds_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, bf16_t* __restrict__ y, int M, int N, int K,
    int tiles_m, int tiles_n, const int32_t* __restrict__ row_slot, float* __restrict__ ybase, LoraArgs seg,
    int t0, int count) {
    gemm_lds_tile<FUSE, C>(x, w, y, M, N, K, tiles_m, tiles_n, row_slot, ybase, seg, t0, count, blockIdx.x);
}

// ---------------------------------------------------------------------------
// Register-staged tiles for any K (multiple of the vector width).  Loads are
// branch-free (rows clamped, K past the end zeroed when stored to LDS) and
// two register sets keep two K steps in flight across the MFMAs.
template <typename E, int BM, int BN, int BK, int WM, int WN>
__device__ __forceinline__ void gemm_tile_body(const E* __restrict__ x, const E* __restrict__ w, E* __restrict__ y,
                                               int M, int N, int K, int tiles_m, int tiles_n,
                                               const int32_t* __restrict__ row_slot, float* __restrict__ ybase,
                                               int bid) {
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

    int tm, tn;
    tile_of(bid, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int li = lane & 15, lg = lane >> 4;
    const u32x4 zero = {0u, 0u, 0u, 0u};

    u32x4 ra[XV + WV], rb[XV + WV];
    auto gload = [&](u32x4 (&r)[XV + WV], int k0) {
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int v = threadIdx.x + i * NT, row = v / VPR, kv = v - row * VPR;
            r[i] = ld16(x + (int64_t)min(m0 + row, M - 1) * K + min(k0 + kv * V, K - V));
        }
#pragma unroll
        for (int i = 0; i < WV; ++i) {
            const int v = threadIdx.x + i * NT, row = v / VPR, kv = v - row * VPR;
            r[XV + i] = ld16(w + (int64_t)min(n0 + row, N - 1) * K + min(k0 + kv * V, K - V));
        }
    };
    auto sstore = [&](const u32x4 (&r)[XV + WV], int buf, int k0) {
        const bool tail = k0 + BK > K;
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int v = threadIdx.x + i * NT, row = v / VPR, kv = v - row * VPR;
            *reinterpret_cast<u32x4*>(&sx[buf][row * LDK + kv * V]) = (tail && k0 + kv * V >= K) ? zero : r[i];
        }
#pragma unroll
        for (int i = 0; i < WV; ++i) {
            const int v = threadIdx.x + i * NT, row = v / VPR, kv = v - row * VPR;
            *reinterpret_cast<u32x4*>(&sw[buf][row * LDK + kv * V]) = (tail && k0 + kv * V >= K) ? zero : r[XV + i];
        }
    };

    f32x4 acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf) {
        const E* cw = sw[buf] + (wn * WTN + li) * LDK + V * lg;
        const E* cx = sx[buf] + (wm * WTM + li) * LDK + V * lg;
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
    };

    const int nk = (K + BK - 1) / BK;
    gload(ra, 0);
    sstore(ra, 0, 0);
    if (nk > 1) gload(rb, BK);
    if (nk > 2) gload(ra, 2 * BK);
    __syncthreads();
    // LDS[0] holds step kt, rb step kt+1, ra step kt+2
    for (int kt = 0; kt < nk; kt += 2) {
        compute(0);
        if (kt + 1 < nk) sstore(rb, 1, (kt + 1) * BK);
        __syncthreads();
        if (kt + 3 < nk) gload(rb, (kt + 3) * BK);
        if (kt + 1 >= nk) break;
        compute(1);
        if (kt + 2 < nk) sstore(ra, 0, (kt + 2) * BK);
        __syncthreads();
        if (kt + 4 < nk) gload(ra, (kt + 4) * BK);
    }
#pragma unroll
    for (int b = 0; b < FM; ++b) {
        const int m = m0 + wm * WTM + b * 16 + li;
        if (m >= M) continue;
        const bool raw = row_slot != nullptr && row_slot[m] >= 0;
#pragma unroll
        for (int a = 0; a < FN; ++a) {
            const int n = n0 + wn * WTN + a * 16 + 4 * lg;
            if (n < N) store4(y, ybase, raw, (int64_t)m * N + n, acc[a][b]);
        }
    }
}

template <typename E, int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64, 1) void gemm_tile_kernel(const E* __restrict__ x, const E* __restrict__ w,
                                                                   E* __restrict__ y, int M, int N, int K, int tiles_m,
                                                                   int tiles_n, const int32_t* __restrict__ row_slot,
                                                                   float* __restrict__ ybase) {
    gemm_tile_body<E, BM, BN, BK, WM, WN>(x, w, y, M, N, K, tiles_m, tiles_n, row_slot, ybase, blockIdx.x);
}

// ---------------------------------------------------------------------------
// Mid-size batches (65 to 256 rows): a tile of BMB x 16 rows of x and 4 WB x 16
// columns.  Both operands go through LDS by direct loads of whole 128-byte row
// segments (a wave-load covers 8 full rows, the access pattern the address
// units serve best): x's rows are shared by the four waves, and each wave's
// WB x 16 rows of w go to a region of its own, since only that wave reads them.
// Steps of 64 K in S stages: the loads of S - 1 steps are in flight behind the
// matrix cores.  Rows of 128 B in LDS, 16-byte chunk c of row r at slot
// c ^ ((r / 2) % 8), so fragment reads are free of bank conflicts.
template <int BMB, int WB, int S>
__device__ __forceinline__ void gemm_xlds_tile(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w,
                                               bf16_t* __restrict__ y, int M, int N, int K, int tiles_m,
                                               int tiles_n, const int32_t* __restrict__ row_slot,
                                               float* __restrict__ ybase, int bid) {
    constexpr int BM = BMB * 16, BN = 64 * WB;
    constexpr int RB = 128;             // bytes of a tile row per step (64 K)
    constexpr int XB = BM * RB;         // x bytes per stage
    constexpr int WR = 16 * WB;         // w rows of one wave
    constexpr int STG = XB + 4 * WR * RB;  // stage: x, then each wave's w rows
    constexpr int LX = BM / 8 / 4;      // x wave-loads (8 rows of 128 B) per wave per step
    constexpr int LW = WR / 8;          // w wave-loads per wave per step
    constexpr int L = LX + LW;          // loads per wave per step
    static_assert(BM % 32 == 0 && S >= 2 && S <= 8 && S * STG <= 160 * 1024, "tile");
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[STG];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[STG];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[S > 2 ? STG : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[S > 3 ? STG : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds4[S > 4 ? STG : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds5[S > 5 ? STG : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds6[S > 6 ? STG : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds7[S > 7 ? STG : 16];
    auto stage = [&](int st) -> uint8_t* {
        return st == 0 ? lds0 : st == 1 ? lds1 : st == 2 ? lds2 : st == 3 ? lds3 :
               st == 4 ? lds4 : st == 5 ? lds5 : st == 6 ? lds6 : lds7;
    };
    int tm, tn;
    tile_of(bid, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int n0 = tn * BN + wave * WR;

    // wave-load q: rows q * 8 + lane / 8 of the wave's share, 16-byte slot lane % 8 holding
    // chunk (lane % 8) ^ ((row / 2) % 8) of the row's 128 bytes
    int xoff[LX], woff[LW];
#pragma unroll
    for (int q = 0; q < LX; ++q) {
        const int row = (wave * LX + q) * 8 + (lane >> 3);
        xoff[q] = (min(m0 + row, M - 1) * K + ((lane & 7) ^ ((row >> 1) & 7)) * 8) * 2;
    }
#pragma unroll
    for (int q = 0; q < LW; ++q) {
        const int row = q * 8 + (lane >> 3);
        woff[q] = (min(n0 + row, N - 1) * K + ((lane & 7) ^ ((row >> 1) & 7)) * 8) * 2;
    }
    const int nk = K / 64;
    const int xbytes = M * K * 2, wbytes = N * K * 2;

    // one step: whole 128-byte row segments of x (shared by the waves) and of this wave's
    // w rows (its own region) go straight into the stage
    auto issue = [&](int kt, int st) {
        const int kb = kt * 128;
        uint8_t* bx = stage(st);
#pragma unroll
        for (int q = 0; q < LX; ++q) buffer_load_lds16(x, xbytes, bx + (wave * LX + q) * 1024, xoff[q], kb);
        uint8_t* bw = bx + XB + wave * WR * RB;
#pragma unroll
        for (int q = 0; q < LW; ++q) buffer_load_lds16(w, wbytes, bw + q * 1024, woff[q], kb);
    };

    f32x4 acc[WB][BMB];
#pragma unroll
    for (int a = 0; a < WB; ++a)
#pragma unroll
        for (int b = 0; b < BMB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int sw = (li >> 1) & 7;  // swizzle of fragment rows 16 b + li
    auto compute = [&](const uint8_t* stg) {
        const uint8_t* bw = stg + XB + wave * WR * RB;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int off = ((4 * h + lg) ^ sw) * 16;
            u32x4 wf[WB], xf[BMB];
#pragma unroll
            for (int a = 0; a < WB; ++a) wf[a] = *reinterpret_cast<const u32x4*>(bw + (16 * a + li) * RB + off);
#pragma unroll
            for (int b = 0; b < BMB; ++b) xf[b] = *reinterpret_cast<const u32x4*>(stg + (16 * b + li) * RB + off);
#pragma unroll
            for (int a = 0; a < WB; ++a)
#pragma unroll
                for (int b = 0; b < BMB; ++b) acc[a][b] = mma_step(wf[a], xf[b], acc[a][b], bf16_t{});
        }
    };

    // every step issues one load group (past the end: the last step again, into a stage
    // that is not read again), so the wait counts are the same in every step
#pragma unroll
    for (int p = 0; p < S - 1; ++p) issue(min(p, nk - 1), p);
    for (int i = 0; i < nk; i += S) {
#pragma unroll
        for (int st = 0; st < S; ++st) {
            const int j = i + st;
            __builtin_amdgcn_sched_barrier(0);
            // this wave's loads of step j are done (those of the S - 2 later steps may not be)
            wait_vmcnt<(S - 2) * L>();
            // every wave's loads of step j are in LDS, and every wave is done with step j - 1
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            issue(min(j + S - 1, nk - 1), (st + S - 1) % S);
            if (j < nk) compute(stage(st));
        }
    }
    wait_vmcnt<0>();

    // lane holds D[w row 4 lg + i][x row li] of each block
#pragma unroll
    for (int b = 0; b < BMB; ++b) {
        const int m = m0 + 16 * b + li;
        if (m >= M) continue;
        const bool raw = row_slot != nullptr && row_slot[m] >= 0;
#pragma unroll
        for (int a = 0; a < WB; ++a) {
            const int n = n0 + 16 * a + 4 * lg;
            if (n < N) store4(y, ybase, raw, (int64_t)m * N + n, acc[a][b]);
        }
    }
}

template <int BMB, int WB, int S>
__global__ __launch_bounds__(256, 2) void gemm_xlds_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w,
                                                           bf16_t* __restrict__ y, int M, int N, int K, int tiles_m,
                                                           int tiles_n, const int32_t* __restrict__ row_slot,
                                                           float* __restrict__ ybase) {
    gemm_xlds_tile<BMB, WB, S>(x, w, y, M, N, K, tiles_m, tiles_n, row_slot, ybase, blockIdx.x);
}

// Decode batches: the base GEMM's tiles and the BGMV shrink's units in one
// launch (independent work: blocks [0, n_gemm) are GEMM tiles, the rest
// shrink units), so the shrink overlaps the GEMM instead of running before it.
// Blocks past the shrink units copy the plan's index words (cp_n of them) from
// cp_src to cp_dst, when the plan's index is read from its host staging buffer by this
// launch and kept in device memory for the later kernels (cp_n = 0 otherwise).

template <class C>
__global__ __launch_bounds__(256) void gemm_lds_shrink_kernel(const bf16_t* __restrict__ x,
                                                               const bf16_t* __restrict__ w, bf16_t* __restrict__ y,
                                                               int M, int N, int K, int tiles_m, int tiles_n,
                                                               const int32_t* __restrict__ row_slot,
                                                               float* __restrict__ ybase, LoraArgs a, int n_gemm,
                                                               const uint32_t* __restrict__ cp_src,
                                                               uint32_t* __restrict__ cp_dst, int cp_n,
                                                               uint64_t raw_mask) {
    static_assert(C::WM * C::WN == 4 && C::BM <= 64, "four waves, as the shrink units; rows in raw_mask");
    const int b = blockIdx.x;
    if (b < n_gemm)
        gemm_lds_tile<false, C>(x, w, y, M, N, K, tiles_m, tiles_n, row_slot, ybase, a, 0, n_gemm, b, raw_mask);
    else if (b < n_gemm + a.n_su)
        bgmv_shrink_unit<bf16_t, true>(a, b - n_gemm);
    else
        copy_words(cp_src, cp_dst, cp_n, b - n_gemm - a.n_su);
}

template <int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(256) void gemm_tile_shrink_kernel(const bf16_t* __restrict__ x,
                                                                const bf16_t* __restrict__ w, bf16_t* __restrict__ y,
                                                                int M, int N, int K, int tiles_m, int tiles_n,
                                                                const int32_t* __restrict__ row_slot,
                                                                float* __restrict__ ybase, LoraArgs a, int n_gemm,
                                                                const uint32_t* __restrict__ cp_src,
                                                                uint32_t* __restrict__ cp_dst, int cp_n) {
    static_assert(WM * WN == 4, "four waves, as the shrink units");
    const int b = blockIdx.x;
    if (b < n_gemm)
        gemm_tile_body<bf16_t, BM, BN, BK, WM, WN>(x, w, y, M, N, K, tiles_m, tiles_n, row_slot, ybase, b);
    else if (b < n_gemm + a.n_su)
        bgmv_shrink_unit<bf16_t>(a, b - n_gemm);
    else
        copy_words(cp_src, cp_dst, cp_n, b - n_gemm - a.n_su);
}

template <typename E, int BM, int BN, int BK, int WM, int WN>
hipError_t run_tile(const void* x, const void* w, void* y, int M, int N, int K, const int32_t* row_slot, float* ybase,
                    hipStream_t s) {
    const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    hipLaunchKernelGGL((gemm_tile_kernel<E, BM, BN, BK, WM, WN>), dim3(tm * tn), dim3(WM * WN * 64), 0, s,
                       static_cast<const E*>(x), static_cast<const E*>(w), static_cast<E*>(y), M, N, K, tm, tn,
                       row_slot, ybase);
    return hipGetLastError();
}

}  // namespace

// Kernel choice by shape class.  Long batches (prefill) are matrix-core
// bound: 256 x 256 direct-to-LDS tiles.  Short batches (decode) are bound by
// reading w once: narrow N tiles spread w over every CU.

// Decode batches on the LDS kernel (CfgDecode64): bf16, up to 64 rows, K % 128 == 0,
// the direct loads' byte offsets within 32 bits.  One rule for every caller.
static bool decode_lds_ok(int dtype, int64_t M, int64_t N, int64_t K) {
    return dtype == 1 && M >= 1 && M <= 64 && K % CfgDecode64::BK == 0 && M * K * 2 < INT32_MAX &&
           N * K * 2 < INT32_MAX;
}
int gemm_cu_count() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cus = n;
        else
            cus = 256;
    }
    return cus;
}

hipError_t launch_gemm(int dtype, const void* x, const void* w, void* y, int64_t M64, int64_t N64, int64_t K64,
                       const int32_t* row_slot, float* ybase, const LoraArgs* seg, bool* fused, hipStream_t s) {
    const int M = (int)M64, N = (int)N64, K = (int)K64;
    if (fused) *fused = false;
    if (dtype == 1) {
        const bf16_t* xb = static_cast<const bf16_t*>(x);
        const bf16_t* wb = static_cast<const bf16_t*>(w);
        bf16_t* yb = static_cast<bf16_t*>(y);
        // byte offsets of the direct loads are 32-bit
        const bool lds_ok = M64 * K64 * 2 < INT32_MAX && N64 * K64 * 2 < INT32_MAX;
        if (M > 256 && K % (CfgLong::S * CfgLong::BK) == 0 && lds_ok) {
            // one workgroup per CU (LDS): the last partial round runs as pieces of tiles.  Tile
            // height 256 or 192, whichever gives the shorter estimated time, in units of a
            // round of 256 x 256 tiles on the whole chip (measured on MI355X at 2,961 rows:
            // a round of 192 x 256 tiles takes 0.85 of one; a round on a fraction u of the
            // CUs 1 - 0.58 (1 - u) of a full one; a round of halves 0.5 (256) or 0.58 x 0.85
            // (192); a round of smaller pieces about 1.5 / P); ties to 256
            const int cus = gemm_cu_count();
            auto pieces = [&](int rem) { return rem * 16 <= cus ? 16 : rem * 8 <= cus ? 8 : rem * 4 <= cus ? 4 : 2; };
            auto plan = [&](int bm, int& tm, int& tn, int& rem) {
                tm = (M + bm - 1) / bm;
                tn = (N + CfgLong::UNIT_N - 1) / CfgLong::UNIT_N;
                const int tiles = tm * tn;
                rem = tiles > cus ? tiles % cus : 0;
                const double f = bm == 256 ? 1.0 : 0.85;
                if (tiles <= cus) return f * (1.0 - 0.58 * (1.0 - (double)tiles / cus));
                double tail = 0.0;
                if (rem) {
                    const int p = bm == 256 ? pieces(rem) : 2;
                    tail = p == 2 ? (bm == 256 ? 0.5 : 0.58) * ((2 * rem + cus - 1) / cus) : 1.5 / p;
                }
                return f * (tiles / cus + tail);
            };
            int tm, tn, rem, tm2, tn2, rem2;
            const bool tall = plan(256, tm, tn, rem) <= plan(192, tm2, tn2, rem2);
            if (!tall) {
                tm = tm2;
                tn = tn2;
                rem = rem2;
            }
            const int n_main = tm * tn - rem;
            const int np = tall && rem ? pieces(rem) : 2;
            const dim3 block(CfgLong::WM * CfgLong::WN * 64);
            const bool fuse = seg != nullptr && seg->n_segs > 0;
            const LoraArgs sa = fuse ? *seg : LoraArgs{};
            auto go = [&](auto whole, auto piece) {
                hipLaunchKernelGGL(whole, dim3(n_main), block, 0, s, xb, wb, yb, M, N, K, tm, tn, row_slot, ybase, sa, 0,
                                   n_main);
                if (rem)
                    hipLaunchKernelGGL(piece, dim3(np * rem), block, 0, s, xb, wb, yb, M, N, K, tm, tn, row_slot,
                                       ybase, sa, n_main, rem);
            };
            auto long_tiles = [&](auto fz) {
                constexpr bool F = decltype(fz)::value;
                if (!tall) go(gemm_lds_kernel<F, CfgLong192>, gemm_lds_kernel<F, CfgLong192Half>);
                else if (np == 16) go(gemm_lds_kernel<F, CfgLong>, gemm_lds_kernel<F, CfgLongSixteenth>);
                else if (np == 8) go(gemm_lds_kernel<F, CfgLong>, gemm_lds_kernel<F, CfgLongEighth>);
                else if (np == 4) go(gemm_lds_kernel<F, CfgLong>, gemm_lds_kernel<F, CfgLongQuarter>);
                else go(gemm_lds_kernel<F, CfgLong>, gemm_lds_kernel<F, CfgLongHalf>);
            };
            if (fuse) long_tiles(std::true_type{});
            else long_tiles(std::false_type{});
            if (fused) *fused = fuse;
            return hipGetLastError();
        }
        if (decode_lds_ok(dtype, M64, N64, K64)) {
            using C = CfgDecode64;
            const int tn = (N + C::BN - 1) / C::BN;
            hipLaunchKernelGGL((gemm_lds_kernel<false, C>), dim3(tn), dim3(C::WM * C::WN * 64), 0, s, xb, wb, yb, M, N,
                               K, 1, tn, row_slot, ybase, LoraArgs{}, 0, tn);
            return hipGetLastError();
        }
        if (M > 64 && M <= 256 && K % 64 == 0 && lds_ok) {
            // the largest tile that still gives about 160 workgroups or more: x is re-read
            // once per column tile, w once per row tile (measured on MI355X, 80 to 256 rows:
            // 4096 x 4096 and 4096 x 11008 take 64 x 64, 11008 x 4096 128 x 64 or 128 x 128)
            auto go = [&](auto kern, int bm, int bn) {
                const int tm = (M + bm - 1) / bm, tn = (N + bn - 1) / bn;
                hipLaunchKernelGGL(kern, dim3(tm * tn), dim3(256), 0, s, xb, wb, yb, M, N, K, tm, tn, row_slot, ybase);
                return hipGetLastError();
            };
            const int64_t t128 = (M + 127) / 128;
            if (M > 128 && t128 * ((N + 127) / 128) >= 160) return go(gemm_xlds_kernel<8, 2, 4>, 128, 128);
            if (t128 * ((N + 63) / 64) >= 160) return go(gemm_xlds_kernel<8, 1, 4>, 128, 64);
            return go(gemm_xlds_kernel<4, 1, 4>, 64, 64);
        }
        if (M > 64) return run_tile<bf16_t, 64, 64, 64, 2, 2>(x, w, y, M, N, K, row_slot, ybase, s);
        return run_tile<bf16_t, 64, 16, 256, 4, 1>(x, w, y, M, N, K, row_slot, ybase, s);
    }
    if (M > 64) return run_tile<float, 64, 64, 32, 2, 2>(x, w, y, M, N, K, row_slot, ybase, s);
    return run_tile<float, 64, 16, 64, 4, 1>(x, w, y, M, N, K, row_slot, ybase, s);
}

// (up to 64 rows: with more rows the shared launch's register budget, set by the shrink
// units, costs the GEMM tiles more occupancy than the shared launch saves)
bool gemm_shrink_fits(int dtype, int64_t M, int n_su) { return dtype == 1 && M >= 1 && M <= 64 && n_su > 0; }

hipError_t launch_gemm_shrink(int dtype, const void* x, const void* w, void* y, int64_t M64, int64_t N64,
                              int64_t K64, const int32_t* row_slot, uint64_t raw_mask, float* ybase,
                              const LoraArgs& a, const void* cp_src, void* cp_dst, int64_t cp_n, hipStream_t s) {
    if (!gemm_shrink_fits(dtype, M64, a.n_su) || cp_n < 0 || cp_n > INT32_MAX) return hipErrorInvalidValue;
    const int M = (int)M64, N = (int)N64, K = (int)K64;
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* wb = static_cast<const bf16_t*>(w);
    bf16_t* yb = static_cast<bf16_t*>(y);
    const uint32_t* cs = static_cast<const uint32_t*>(cp_src);
    uint32_t* cd = static_cast<uint32_t*>(cp_dst);
    const int ncp = cp_n > 0 ? kCopyBlocks : 0;
    if (decode_lds_ok(dtype, M64, N64, K64)) {
        using C = CfgDecode64;
        const int tn = (N + C::BN - 1) / C::BN;
        hipLaunchKernelGGL((gemm_lds_shrink_kernel<C>), dim3(tn + a.n_su + ncp), dim3(256), 0, s, xb, wb, yb, M, N, K,
                           1, tn, raw_mask != 0 ? nullptr : row_slot, ybase, a, tn, cs, cd, (int)cp_n, raw_mask);
    } else {
        const int tn = (N + 15) / 16;
        hipLaunchKernelGGL((gemm_tile_shrink_kernel<64, 16, 256, 4, 1>), dim3(tn + a.n_su + ncp), dim3(256), 0, s, xb,
                           wb, yb, M, N, K, 1, tn, row_slot, ybase, a, tn, cs, cd, (int)cp_n);
    }
    return hipGetLastError();
}

}  // namespace hagemm
