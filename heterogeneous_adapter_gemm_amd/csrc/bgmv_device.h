// Device code of the BGMV shrink, shared by its own kernel and by the decode
// GEMM kernel that runs the shrink units beside its tiles.
#pragma once

#include "common.h"
#include "internal.h"

namespace hagemm {

// Words [blk * 256 + tid, ...) of n, strided over kCopyBlocks workgroups: the copy of a
// plan's index that a decode launch reads from host memory and keeps for later kernels.
__device__ __forceinline__ void copy_words(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst, int n,
                                           int blk) {
    for (int i = blk * 256 + threadIdx.x; i < n; i += kCopyBlocks * 256) dst[i] = src[i];
}

// page-table words of (slot, the call's layer and projection): lp is the projection's offset
// per unit of rank (lp_per_rank, or lp_multi[p] in a launch over several projections)
__device__ __forceinline__ const int32_t* slot_table(const LoraArgs& a, int slot, int rank, int lp) {
    return a.page_tab + (int64_t)slot * a.slot_cap + (int64_t)rank * lp;
}
__device__ __forceinline__ const int32_t* slot_table(const LoraArgs& a, int slot, int rank) {
    return slot_table(a, slot, rank, a.lp_per_rank);
}

// Projection p of a launch over several projections sharing x: its table offset and v
__device__ __forceinline__ int multi_lp(const LoraArgs& a, int p) { return a.n_multi > 1 ? a.lp_multi[p] : a.lp_per_rank; }

// ---------------------------------------------------------------------------
// BGMV shrink: v[row][j] = sum_k x[row][k] * A[j][k] for the rows of one group.
// Workgroup = 4 consecutive rank-rows of one group, one wave each, so the
// group's x rows are fetched from L2 once per workgroup and hit L1 for the
// other waves.  A wave issues its whole A row (up to 8 pages' worth per pass)
// and the pass's x rows (up to kShrinkTokensPerPass) before using any of
// them, then reduces each dot product across the wave in a fixed butterfly
// order.
//
// One pass of a shrink wave over NT rows of its group (NT = rows left, at most
// kShrinkTokensPerPass): loads of A and of exactly NT x rows first.
template <typename E, int NT>
__device__ __forceinline__ void shrink_rows(const LoraArgs& a, const int32_t* tab, int j, const int* row, int lane,
                                            float* v) {
    constexpr int V = Elem<E>::kVec;
    constexpr int S = 8;  // 16-byte vectors per lane per pass: 64*8*V elements
    const E* pages = static_cast<const E*>(a.pages);
    const E* x = static_cast<const E*>(a.x);
    const int pmask = (1 << a.page_shift) - 1;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.f;
    for (int k0 = 0; k0 < a.d_in; k0 += 64 * V * S) {
        // all loads first, from clamped addresses; the K tail is masked at use
        u32x4 av[S], xv[NT][S];
#pragma unroll
        for (int i = 0; i < S; ++i) {
            // the 64 V elements of vector i lie in one page (pages hold a multiple of 64 V), so
            // the page is the same for the whole wave: one scalar table read
            const int kb = min(k0 + i * 64 * V, a.d_in - V);
            const int64_t pg = tab[kb >> a.page_shift];
            const int k = min(k0 + (i * 64 + lane) * V, a.d_in - V);
            av[i] = ld16(pages + (pg << a.page_shift) + (k & pmask));
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < S; ++i) {
                const int k = min(k0 + (i * 64 + lane) * V, a.d_in - V);
                xv[t][i] = ld16(x + (int64_t)row[t] * a.d_in + k);
            }
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const bool kin = k0 + (i * 64 + lane) * V < a.d_in;
            float af[V];
            unpack(kin ? av[i] : zero, af, E{});
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                float xf[V];
                unpack(xv[t][i], xf, E{});
#pragma unroll
                for (int e = 0; e < V; ++e) acc[t] = fmaf(xf[e], af[e], acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const float sum = wave_sum(acc[t]);
        if (lane == 0) v[(int64_t)row[t] * a.vstride + j] = sum;
    }
}

// Shrink unit u (a workgroup of 4 waves): rank-rows j0 .. j0 + 3 of group g,
// for the group's rows first .. first + kShrinkTokensPerUnit - 1.  Its index
// entry (8 words): [0] group, [1] j0 | first << 8, [2] slot, [3] rank | rows
// << 8, [4..7] the unit's rows (the last repeated).  RES reads the resolved
// words [1..7] (one load, then the page table), which shortens the chain of
// dependent loads when the index is read from host memory; otherwise the
// group's table entries are read.
template <typename E, bool RES = false>
__device__ __forceinline__ void bgmv_shrink_unit(const LoraArgs& a, int u, int lp, float* v) {
    constexpr int TB = kShrinkTokensPerPass;
    static_assert(TB == 4 && kShrinkTokensPerUnit == TB, "one pass of 1 to 4 rows");
    const int lane = threadIdx.x & 63;
    if (u >= a.n_su) return;
    int j, slot, r, cnt, first = 0, beg = 0;
    int4 rr{0, 0, 0, 0};
    if constexpr (RES) {
        const int4 h = reinterpret_cast<const int4*>(a.su)[2 * u];
        rr = reinterpret_cast<const int4*>(a.su)[2 * u + 1];
        j = (h.y & 255) + (threadIdx.x >> 6);
        slot = h.z;
        r = h.w & 255;
        cnt = h.w >> 8;
    } else {
        const int2 unit = reinterpret_cast<const int2*>(a.su)[4 * u];
        const int g = unit.x;
        j = (unit.y & 255) + (threadIdx.x >> 6);
        first = unit.y >> 8;
        slot = a.g_slot[g];
        r = a.g_rank[g];
        beg = a.g_begin[g];
        cnt = min(a.g_count[g], first + kShrinkTokensPerUnit);
    }
    if (j >= r) return;
    j = __builtin_amdgcn_readfirstlane(j);   // one rank-row per wave
    const int32_t* tab = slot_table(a, slot, r, lp) + j * a.nci;
    for (int t0 = first; t0 < cnt; t0 += TB) {
        const int nt = min(TB, cnt - t0);
        int row[TB];
        if constexpr (RES) {
            row[0] = rr.x;
            row[1] = rr.y;
            row[2] = rr.z;
            row[3] = rr.w;
        } else {
#pragma unroll
            for (int t = 0; t < TB; ++t) row[t] = a.rows[beg + t0 + min(t, nt - 1)];
        }
        // a pass loads only the x rows it has (a uniform switch)
        switch (nt) {
            case 1: shrink_rows<E, 1>(a, tab, j, row, lane, v); break;
            case 2: shrink_rows<E, 2>(a, tab, j, row, lane, v); break;
            case 3: shrink_rows<E, 3>(a, tab, j, row, lane, v); break;
            default: shrink_rows<E, 4>(a, tab, j, row, lane, v); break;
        }
    }
}
template <typename E, bool RES = false>
__device__ __forceinline__ void bgmv_shrink_unit(const LoraArgs& a, int u) {
    bgmv_shrink_unit<E, RES>(a, u, a.lp_per_rank, a.v);
}

}  // namespace hagemm
