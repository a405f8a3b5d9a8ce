// gfx950 kernels of the adapter path: the per-row LoRA delta computed as a
// shrink v = A x (rank r) and an expand y += gamma B v, reading the adapter's
// rank-rows from scattered pages of the unified pool through the page table
// ("Multi-LoRA serving: S-LoRA, Punica and adapter batching", How the kernels
// work; "S-LoRA: Serving Thousands of Concurrent LoRA Adapters", Unified
// paging and Kernels: gather each request's adapter from non-contiguous pages,
// mixed ranks without padding).
//
//  * BGMV (decode): rows arrive one token each.  The host groups rows by
//    adapter so every A/B page is fetched once per batch however many rows
//    share it.  Shrink: one wave per (group, 4 rank-rows) streams those rows
//    and dots them with each row's x, reducing across the wave with
//    butterfly shuffles.  Expand: one wave per (group, 512-column chunk)
//    streams the chunk of every B rank-row and updates each row's y chunk.
//    Vector ALU only: the work is bound by the page reads, not arithmetic.
//  * SGMV (prefill): rows arrive in contiguous segments sharing an adapter.
//    The two small contractions run on the matrix cores: shrink [64 x d_in]
//    x [d_in x r] per tile, K split over workgroups (partials summed in a
//    fixed order), and expand [64 x r] x [r x 64 columns] (in the long-batch
//    GEMM's epilogue when that kernel runs).
//  * Page-in: one workgroup per page reads the adapter's rows straight from
//    pinned host memory and writes the page, zero past the row's end.
#include <algorithm>

#include "bgmv_device.h"
#include "common.h"
#include "internal.h"

namespace hagemm {
namespace {


// ---------------------------------------------------------------------------
// BGMV shrink (device code in bgmv_device.h)
// In a call with prefill segments whose SGMV shrink split K (S > 1 parts), the
// launch also sums the SGMV partials: blocks past the shrink units are the sum's
// (see sgmv_sum_block), so that small pass costs no launch of its own.
__device__ __forceinline__ void sgmv_sum_block(const LoraArgs& a, int S, int blk, int p);

// With several projections sharing x (n_multi > 1), blocks run projection by projection:
// block b is block b % per of projection b / per.
template <typename E>
__global__ __launch_bounds__(256) void bgmv_shrink_kernel(LoraArgs a, int S) {
    const int per = a.n_su + (S > 1 ? 4 * a.n_tiles : 0);
    const int p = blockIdx.x / per, b = blockIdx.x - p * per;
    if (b < a.n_su) bgmv_shrink_unit<E, true>(a, b, multi_lp(a, p), a.v + p * a.v_pstride);
    else sgmv_sum_block(a, S, b - a.n_su, p);
}

// ---------------------------------------------------------------------------
// BGMV expand: y[row][n] = base + gamma * sum_j v[row][j] * B[j][n] for the
// rows of one group and one 64*V-column chunk.  Workgroup = (group, chunk);
// wave w takes rank-rows j = w, w+4, ... so all of a chunk's B rows are
// fetched at once.  Rows go in batches of four: while the B rows are in
// flight the batch's v rows are staged in LDS and each wave fetches the base
// of the row it finishes; the four partial sums meet in LDS and are added in
// wave order.
// The expand of one (group, chunk) with JW rank-rows per wave (4 JW >= r):
// the B loads are straight-line code, so they all go out before the first use.
// RES: the unit's slot, rank, row count, gamma and first row come resolved in its
// index entry (one load); otherwise through its group's table entries.
// The projection an expand block works for: its output, fp32 base (or NULL), v, width,
// pages per B row and page-table offset per unit of rank.
struct ExpandProj {
    void* y;
    const float* ybase;
    const float* v;
    int d_out, nco, lp;
};

template <typename E, int JW, bool RES>
__device__ __forceinline__ void expand_chunk(const LoraArgs& a, const ExpandProj& q, int e, int ch,
                                             float (&part)[4][kExpandTokensPerPass][Elem<E>::kVec][64],
                                             float (&vs)[kExpandTokensPerPass][kMaxRank]) {
    constexpr int V = Elem<E>::kVec;
    constexpr int TB = kExpandTokensPerPass;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = ch * 64 * V + lane * V;
    const bool nin = n < q.d_out;  // d_out is a multiple of V: a vector is all in or all out
    int slot, r, beg = 0, cnt;
    float gamma;
    int4 rr{0, 0, 0, 0};
    if constexpr (RES) {
        const int4 h = reinterpret_cast<const int4*>(a.eu)[3 * e];
        rr = reinterpret_cast<const int4*>(a.eu)[3 * e + 1];
        slot = h.x;
        r = h.y & 255;
        cnt = h.y >> 8;
        gamma = __int_as_float(h.z);
    } else {
        const int g = a.eu[12 * e + 3], first = a.eu[12 * e + 8];
        slot = a.g_slot[g];
        r = a.g_rank[g];
        beg = a.g_begin[g] + first;
        cnt = min(a.g_count[g] - first, kExpandTokensPerUnit);
        gamma = a.g_gamma[g];
    }
    const int32_t* tabB = slot_table(a, slot, r, q.lp) + r * a.nci;
    const E* pages = static_cast<const E*>(a.pages);
    E* y = static_cast<E*>(q.y);
    const int nc = min(n, q.d_out - V);  // clamped column for the loads
    const int c = nc >> a.page_shift, off = nc & ((1 << a.page_shift) - 1);
    // this wave's B rows for the chunk, all loads in flight together
    u32x4 bv[JW];
#pragma unroll
    for (int i = 0; i < JW; ++i) {
        const int j = min(w + 4 * i, r - 1);
        bv[i] = ld16(pages + ((int64_t)tabB[j * q.nco + c] << a.page_shift) + off);
    }
    static_assert(TB == 4, "wave w finishes row w of a batch");
    for (int t0 = 0; t0 < cnt; t0 += TB) {
        const int nt = min(TB, cnt - t0);
        int row[TB];
        if constexpr (RES) {
            static_assert(kExpandTokensPerUnit == TB, "the entry holds a unit's rows");
            row[0] = rr.x;
            row[1] = rr.y;
            row[2] = rr.z;
            row[3] = rr.w;
        } else {
#pragma unroll
            for (int t = 0; t < TB; ++t) row[t] = a.rows[beg + t0 + min(t, nt - 1)];
        }
        // while the B rows are in flight: the batch's v rows into LDS (one value per thread)
        // and the base of the row this wave finishes
        {
            const int t = threadIdx.x / kMaxRank, j = threadIdx.x % kMaxRank;
            if (j < r) vs[t][j] = q.v[(int64_t)row[t] * a.vstride + j];
        }
        float yv[V];
        if (q.ybase) {
            const float* bp = q.ybase + (int64_t)row[w] * q.d_out + nc;
#pragma unroll
            for (int q = 0; q < V; q += 4) {
                const f32x4 b4 = *reinterpret_cast<const f32x4*>(bp + q);
                yv[q] = b4[0];
                yv[q + 1] = b4[1];
                yv[q + 2] = b4[2];
                yv[q + 3] = b4[3];
            }
        } else {
            unpack(ld16(y + (int64_t)row[w] * q.d_out + nc), yv, E{});
        }
        __syncthreads();
        float acc[TB][V];
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int e = 0; e < V; ++e) acc[t][e] = 0.f;
#pragma unroll
        for (int i = 0; i < JW; ++i) {
            const int j = w + 4 * i;
            if (j < r) {
                float bf[V];
                unpack(bv[i], bf, E{});
#pragma unroll
                for (int t = 0; t < TB; ++t) {
                    const float vv = vs[t][j];
#pragma unroll
                    for (int e = 0; e < V; ++e) acc[t][e] = fmaf(vv, bf[e], acc[t][e]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int e = 0; e < V; ++e) part[w][t][e][lane] = acc[t][e];
        __syncthreads();
        if (w < nt && nin) {
            float sum[V];
#pragma unroll
            for (int e = 0; e < V; ++e) sum[e] = ((part[0][w][e][lane] + part[1][w][e][lane]) + part[2][w][e][lane]) + part[3][w][e][lane];
#pragma unroll
            for (int e = 0; e < V; ++e) yv[e] = fmaf(gamma, sum[e], yv[e]);
            st16(y + (int64_t)row[w] * q.d_out + n, pack(yv, E{}));
        }
        __syncthreads();
    }
}

// Expand unit e's index entry (12 words): slot, rank | rows << 8, gamma (float bits), its
// group; its rows (the last repeated up to four); its first row in the group; three unused.
// The resolved form (RES) shortens the chain of dependent loads in front of the B loads,
// which pays when the grid is about one round of workgroups; the group form keeps the
// kernel's registers lower, which pays when many rounds queue: it is held to 128
// registers, four workgroups per CU (C3 expand 36.4 -> 34.0 us; three dwords spill).
// In a launch over several projections (n_multi > 1) the blocks of projection p are
// [eblk_multi[p], eblk_multi[p + 1]), each projection's expand units times its chunks.
template <typename E, bool RES>
__global__ __launch_bounds__(256, RES ? 1 : 4) void bgmv_expand_kernel(LoraArgs a) {
    constexpr int V = Elem<E>::kVec;
    __shared__ float part[4][kExpandTokensPerPass][V][64];
    __shared__ float vs[kExpandTokensPerPass][kMaxRank];
    int b = blockIdx.x;
    ExpandProj q{a.y, a.ybase, a.v, a.d_out, a.nco, a.lp_per_rank};
    if (a.n_multi > 1) {
        int p = 0;
        while (p + 1 < a.n_multi && b >= a.eblk_multi[p + 1]) ++p;
        b -= a.eblk_multi[p];
        q = ExpandProj{a.y_multi[p], a.ybase ? a.ybase + p * a.ybase_pstride : nullptr, a.v + p * a.v_pstride,
                       a.dout_multi[p], a.nco_multi[p], a.lp_multi[p]};
    }
    const int nchunks = (q.d_out + 64 * V - 1) / (64 * V);
    const int e = b / nchunks, ch = b - e * nchunks;
    const int r = RES ? a.eu[12 * e + 1] & 255 : a.g_rank[a.eu[12 * e + 3]];
    const int jw = (r + 3) / 4;  // rank-rows per wave
    if (jw <= 1) expand_chunk<E, 1, RES>(a, q, e, ch, part, vs);
    else if (jw <= 2) expand_chunk<E, 2, RES>(a, q, e, ch, part, vs);
    else if (jw <= 4) expand_chunk<E, 4, RES>(a, q, e, ch, part, vs);
    else if (jw <= 8) expand_chunk<E, 8, RES>(a, q, e, ch, part, vs);
    else expand_chunk<E, kMaxRank / 4, RES>(a, q, e, ch, part, vs);
}

// ---------------------------------------------------------------------------
// SGMV shrink: v[row][j] = sum_k x[row][k] * A[j][k] for a 64-row tile of one
// segment and every j < r, K split into S parts over S workgroups so that a
// batch of few tiles still covers the chip.  Four waves; wave w owns rows 16w ..
// 16w + 15 of the tile and all NB 16-row blocks of A the rank needs (NB = 1, 2
// or 4: a uniform switch in the kernel).  Per 128-byte step of K, the tile's x
// rows and the A rows go straight from memory into LDS (whole 128-byte row
// pieces, 16-byte chunks placed by a row-dependent swizzle), four steps in
// flight, then into matrix-core fragments.  With S = 1 the workgroup writes v.
// Otherwise each writes its fp32 partial and a later launch (one of its own,
// or the call's BGMV shrink launch when the batch has decode rows too) sums
// the S partials of every output in part order (no workgroup waits for
// another, and no cache maintenance is needed between XCDs: the launch
// boundary orders the partials' writes).
template <typename E, int NB>
__device__ __forceinline__ void sgmv_shrink_part(const LoraArgs& a, uint8_t* lds0, uint8_t* lds1, uint8_t* lds2,
                                                 uint8_t* lds3, int tile, int ks, int S, int pj) {
    constexpr int V = Elem<E>::kVec;   // elements per 16 bytes
    constexpr int BK = 8 * V;          // elements per 128-byte step
    constexpr int NS = 4;              // stages
    constexpr int XS = 64 * 128;       // x bytes of a stage (A follows)
    constexpr int LA = NB == 4 ? 2 : 1;  // A loads per wave per step
    constexpr int L = 2 + LA;          // loads per wave per step
    auto stage = [&](int st) { return st == 0 ? lds0 : st == 1 ? lds1 : st == 2 ? lds2 : lds3; };
    const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = a.t_seg[tile], send = a.s_end[s], row0 = a.t_row0[tile], r = a.s_rank[s];
    const int32_t* tab = slot_table(a, a.s_slot[s], r, multi_lp(a, pj));
    const char* pages = static_cast<const char*>(a.pages);
    const int rowb = a.d_in * (int)sizeof(E);   // bytes of an x row
    const int pmask = (1 << a.page_shift) - 1;
    const int nsteps = (a.d_in + BK - 1) / BK;
    const int st0 = nsteps * ks / S, st1 = nsteps * (ks + 1) / S, nst = st1 - st0;
    // lane -> (row lr of its wave-load's 8, slot p): slot p of row rr holds chunk p ^ (rr % 8)
    const int lr = lane >> 3, p = lane & 7;
    const char* xrow[2];
    int xch[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int rr = 8 * (2 * w + q) + lr;
        xrow[q] = static_cast<const char*>(a.x) + (int64_t)min(row0 + rr, send - 1) * rowb;
        xch[q] = (p ^ (rr & 7)) * 16;
    }
    // A rows of this wave's loads (past r: row r - 1 again, never stored) and their place.
    // NB = 1: waves 0 and 1 load the 16 rows, waves 2 and 3 the same rows again into rows
    // 16 .. 31 of the stage (not read), so every wave issues the same loads
    int arow[LA], ach[LA], adst[LA];
#pragma unroll
    for (int q = 0; q < LA; ++q) {
        const int r8 = NB == 1 ? 8 * (w & 1) : NB == 2 ? 8 * w : 8 * (2 * w + q);   // first row of the load
        const int ar = r8 + lr;
        arow[q] = min(ar, r - 1);
        ach[q] = (p ^ (ar & 7)) * 16;
        adst[q] = XS + (NB == 1 ? 8 * w : r8) * 128;
    }
    int cur_pg = -1;
    const char* apb[LA];
    // x chunks past the row end (a last, partial step) are read at the row's last 16 bytes and
    // zeroed in LDS once they land; A's page tail past the row is zero already
    auto issue = [&](int st, uint8_t* stg) {
        const int kb = st * 128;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int off = min(kb + xch[q], rowb - 16);
            global_load_lds16(xrow[q] + off, stg + (2 * w + q) * 1024);
        }
        const int pg = (st * BK) >> a.page_shift;
        if (pg != cur_pg) {
            cur_pg = pg;
#pragma unroll
            for (int q = 0; q < LA; ++q)
                apb[q] = pages + ((int64_t)tab[arow[q] * a.nci + pg] << a.page_shift) * (int64_t)sizeof(E);
        }
        const int po = ((st * BK) & pmask) * (int)sizeof(E);
#pragma unroll
        for (int q = 0; q < LA; ++q) global_load_lds16(apb[q] + po + ach[q], stg + adst[q]);
    };
    auto at = [](int rr, int cc) { return rr * 128 + ((cc ^ (rr & 7)) << 4); };
    f32x4 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool ragged = a.d_in % BK != 0;
    auto compute = [&](const uint8_t* stg) {
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
            const u32x4 xf = *reinterpret_cast<const u32x4*>(stg + at(16 * w + li, 4 * kq + lg));
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const u32x4 af = *reinterpret_cast<const u32x4*>(stg + XS + at(16 * b + li, 4 * kq + lg));
                acc[b] = mma_step(xf, af, acc[b], E{});
            }
        }
    };
    if (nst > 0) {
#pragma unroll
        for (int q = 0; q < NS - 1; ++q) issue(st0 + min(q, nst - 1), stage(q));
        // unrolled by the stage count, so each stage is a known LDS object: the compiler sees
        // that the stage being filled is not the one being read.  Steps past the end only wait
        // and refill (the last step again), so every wave has the same loads in flight.
        for (int i0 = 0; i0 < nst; i0 += NS) {
#pragma unroll
            for (int u = 0; u < NS; ++u) {
                const int i = i0 + u;
                // no instruction moves across the waits and the barrier
                __builtin_amdgcn_sched_barrier(0);
                // this wave's loads of step i are in LDS (those of the NS - 2 later steps may not be)
                wait_vmcnt<(NS - 2) * L>();
                if (ragged && i < nst && st0 + i == nsteps - 1) {
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        if ((st0 + i) * 128 + xch[q] >= rowb)
                            *reinterpret_cast<u32x4*>(stage(u) + (2 * w + q) * 1024 + lane * 16) =
                                u32x4{0u, 0u, 0u, 0u};
                }
                // (and this wave's LDS stores and fragment reads are done)
                wait_vmcnt_lgkm0<(NS - 2) * L>();
                // every wave's loads of step i are in LDS, and every wave is done with step i - 1
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                issue(st0 + min(i + NS - 1, nst - 1), stage((u + NS - 1) % NS));
                if (i < nst) compute(stage(u));
            }
        }
        wait_vmcnt<0>();   // no load may still be writing LDS when the workgroup ends
    }
    // lane holds D[row = 16 w + 4 lg + i][j = 16 b + li]
    float* out = S == 1 ? a.v + pj * a.v_pstride : a.vpart + pj * a.vpart_pstride + (int64_t)ks * a.vpart_rows * a.vstride;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = row0 + 16 * w + 4 * lg + i, j = 16 * b + li;
            if (row < send && j < r) out[(int64_t)row * a.vstride + j] = acc[b][i];
        }
}

// v[row][j] = sum over the K parts of the partials, in part order.  Block blk: 16 rows of a
// tile (4 per tile); thread: one row, 4 consecutive j, all S partials loaded at once.  Rows
// of no segment are not touched.
__device__ __forceinline__ void sgmv_sum_block(const LoraArgs& a, int S, int blk, int p) {
    const int tile = blk >> 2;
    const int s = a.t_seg[tile], send = a.s_end[s], r = a.s_rank[s];
    const int row = a.t_row0[tile] + 16 * (blk & 3) + (threadIdx.x >> 4), j = (threadIdx.x & 15) * 4;
    if (row >= send || j >= r) return;
    const int64_t pstride = (int64_t)a.vpart_rows * a.vstride;
    const float* pp = a.vpart + p * a.vpart_pstride + (int64_t)row * a.vstride + j;
    f32x4 part[kMaxShrinkSplit];
#pragma unroll
    for (int k = 0; k < kMaxShrinkSplit; ++k)
        if (k < S) part[k] = *reinterpret_cast<const f32x4*>(pp + k * pstride);
    f32x4 sum = part[0];
#pragma unroll
    for (int k = 1; k < kMaxShrinkSplit; ++k)
        if (k < S) sum += part[k];
    float* vp = a.v + p * a.v_pstride + (int64_t)row * a.vstride + j;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (j + e < r) vp[e] = sum[e];
}

__global__ __launch_bounds__(256) void sgmv_shrink_sum_kernel(LoraArgs a, int S) {
    const int per = 4 * a.n_tiles;
    const int p = blockIdx.x / per;
    sgmv_sum_block(a, S, blockIdx.x - p * per, p);
}

// workgroup b: part b / n_tiles of tile b % n_tiles (the tiles of one part run together, so
// the A pieces of a segment's tiles are read while in L2)
template <typename E>
__global__ __launch_bounds__(256) void sgmv_shrink_kernel(LoraArgs a, int S) {
    // one array per stage: distinct objects let the compiler see that the stage being filled
    // by direct loads is not the one being read
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[2 * 64 * 128];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[2 * 64 * 128];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[2 * 64 * 128];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[2 * 64 * 128];
    // projection p = b / (n_tiles * S) of a launch over several projections
    const int per = a.n_tiles * S;
    const int p = blockIdx.x / per, b = blockIdx.x - p * per;
    const int tile = b % a.n_tiles, ks = b / a.n_tiles;
    const int r = a.s_rank[a.t_seg[tile]];
    if (r <= 16) sgmv_shrink_part<E, 1>(a, lds0, lds1, lds2, lds3, tile, ks, S, p);
    else if (r <= 32) sgmv_shrink_part<E, 2>(a, lds0, lds1, lds2, lds3, tile, ks, S, p);
    else sgmv_shrink_part<E, 4>(a, lds0, lds1, lds2, lds3, tile, ks, S, p);
}

// ---------------------------------------------------------------------------
// SGMV expand: y[row][n] += gamma * sum_j v[row][j] * B[j][n] for a 64-row
// tile of one segment and 64 output columns.  The B chunk is staged in LDS
// transposed ([n][j]) so each lane reads its K-contiguous fragment with one
// 16-byte load; v (fp32) enters the bf16
// matrix cores as a high and a low bf16 half.
template <typename E>
__global__ __launch_bounds__(256) void sgmv_expand_kernel(LoraArgs a) {
    constexpr int V = Elem<E>::kVec;
    constexpr int KG = 4 * V;
    constexpr int BNC = 64;          // output columns per tile
    constexpr int LDJ = kMaxRank + V; // LDS row stride (elements) of the transposed B chunk
    __shared__ __align__(16) E bt[BNC * LDJ];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lg = lane >> 4, li = lane & 15;
    const int ncol = (a.d_out + BNC - 1) / BNC;
    const int tile = blockIdx.x / ncol, ct = blockIdx.x - tile * ncol;
    const int s = a.t_seg[tile], row0 = a.t_row0[tile];
    const int slot = a.s_slot[s], r = a.s_rank[s], send = a.s_end[s];
    const float gamma = a.s_gamma[s];
    const int n0 = ct * BNC;
    const int rp = (r + KG - 1) / KG * KG;
    const int32_t* tabB = slot_table(a, slot, r) + r * a.nci;
    const E* pages = static_cast<const E*>(a.pages);
    const int pmask = (1 << a.page_shift) - 1;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // stage B[j][n0 .. n0+63] as bt[n][j], zero for j >= r or n >= d_out
    constexpr int VPR = BNC / V;  // vectors per B row chunk
    for (int idx = threadIdx.x; idx < rp * VPR; idx += 256) {
        const int j = idx / VPR, nv = idx - j * VPR;
        const int n = n0 + nv * V;
        u32x4 val = zero;
        if (j < r && n < a.d_out) val = ld16(pages + ((int64_t)tabB[j * a.nco + (n >> a.page_shift)] << a.page_shift) + (n & pmask));
        const E* pe = reinterpret_cast<const E*>(&val);
#pragma unroll
        for (int e = 0; e < V; ++e) bt[(nv * V + e) * LDJ + j] = pe[e];
    }
    __syncthreads();
    const int myrow = row0 + 16 * w + li;
    const int vrow = min(myrow, send - 1);
    f32x4 acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < rp; kb += KG) {
        // this lane's V consecutive j of v[vrow][*] (zero past the rank)
        float vv[V];
        const int j0 = kb + V * lg;
        const float* vp = a.v + (int64_t)vrow * a.vstride;
#pragma unroll
        for (int e = 0; e < V; ++e) vv[e] = j0 + e < r ? vp[j0 + e] : 0.f;
        u32x4 vhi, vlo;
        if constexpr (V == 8) {
            float lo[8];
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                h[e] = f32_to_bf16(vv[e]);
                lo[e] = vv[e] - __uint_as_float(h[e] << 16);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vhi[i] = h[2 * i] | (h[2 * i + 1] << 16);
                vlo[i] = pack_bf16(lo[2 * i], lo[2 * i + 1]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) vhi[e] = __float_as_uint(vv[e]);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const u32x4 bf = *reinterpret_cast<const u32x4*>(&bt[(16 * b + li) * LDJ + j0]);
            acc[b] = mma_step(bf, vhi, acc[b], E{});
            if constexpr (V == 8) acc[b] = mma_step(bf, vlo, acc[b], E{});
        }
    }
    // lane holds D[n = 16*b + 4*lg + i][row = li]: four consecutive columns of one row
    if (myrow < send) {
        E* yr = static_cast<E*>(a.y) + (int64_t)myrow * a.d_out;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int n = n0 + 16 * b + 4 * lg;
            if (n < a.d_out) {
                f32x4 base;
                if (a.ybase) {
                    base = *reinterpret_cast<const f32x4*>(a.ybase + (int64_t)myrow * a.d_out + n);
                } else if constexpr (V == 8) {
                    const u32x2 old = *reinterpret_cast<const u32x2*>(yr + n);
                    base = f32x4{bf16_lo(old[0]), bf16_hi(old[0]), bf16_lo(old[1]), bf16_hi(old[1])};
                } else {
                    base = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(yr + n));
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) base[i] = fmaf(gamma, acc[b][i], base[i]);
                if constexpr (V == 8) {
                    u32x2 nw;
                    nw[0] = pack_bf16(base[0], base[1]);
                    nw[1] = pack_bf16(base[2], base[3]);
                    *reinterpret_cast<u32x2*>(yr + n) = nw;
                } else {
                    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(yr + n)) = base;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Page-in: page q of the launch (pages block0[k] .. block0[k+1] belong to
// adapter k: n_layers consecutive layers of it) is copied from that adapter's
// rows to its pool page.  The source is either the pinned host blob
// (device-visible pointer, read over PCIe, one layer per launch) or the copy
// of a few layers that the copy engine put in a device staging area (all of
// them in one launch).
// For the host blob a small grid strides over the pages: the copy is bound by
// PCIe, and it runs beside the LoRA-linear kernels, whose occupancy a grid of
// one workgroup per page would take.  A workgroup
// takes kPageInGroup pages per pass and each thread has kPageInLoads 16-byte
// loads of each in flight (with 8 KB pages, one pass covers a page).
// Measured on the Llama-7B stack step with 1.8 GB paged in per step (MI355X):
// over PCIe, 16 workgroups x 2 pages 63.6 ms/step at 44 GB/s, 32 x 1 67.0-67.9
// ms at 52 GB/s (the compute kernels beside it lose more than the copy gains),
// 8 x 4 or 8 x 8 66.9-70.8 ms at 27-29 GB/s (the copy becomes the bound); out
// of the staging area, one workgroup per 2 pages 51.87 ms/step against 52.70
// with 256 striding workgroups (49.1 with every adapter resident), the same
// with 4 or 8 pages per workgroup, and 16 to 64 striding ones slower still.
constexpr int kPageInLoads = 2;
constexpr int kPageInGroup = 2;

template <typename E, int G>
__global__ __launch_bounds__(256) void page_in_kernel(PageInArgs a) {
    constexpr int V = Elem<E>::kVec;
    const int P = 1 << a.page_shift;
    const int total = a.block0[a.n_adapters];
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // one layer per rank-row: pages, A and B elements over the projections
    int pprl = 0, ia = 0, ib = 0;
    for (int p = 0; p < a.n_proj; ++p) {
        pprl += a.nci[p] + a.nco[p];
        ia += a.d_in[p];
        ib += a.d_out[p];
    }
    // source, valid length and destination of launch page qq; an adapter's pages run layer by
    // layer, and so do its page-table entries and its rows in the source
    auto resolve = [&](int qq, const E*& src, int& len, E*& dst) {
        int k = 0;
        while (k + 1 < a.n_adapters && qq >= a.block0[k + 1]) ++k;
        const int q = qq - a.block0[k];
        const int rank = a.rank[k];
        const int layer = q / (rank * pprl);
        int rem = q - layer * rank * pprl, p = 0;
        int64_t aoff = a.a_layer_off[k] + (int64_t)layer * rank * ia;
        int64_t boff = a.b_layer_off[k] + (int64_t)layer * rank * ib;
        for (; p < a.n_proj - 1; ++p) {
            const int np = rank * (a.nci[p] + a.nco[p]);
            if (rem < np) break;
            rem -= np;
            aoff += (int64_t)rank * a.d_in[p];
            boff += (int64_t)rank * a.d_out[p];
        }
        if (rem < rank * a.nci[p]) {
            const int j = rem / a.nci[p], c = rem - j * a.nci[p];
            src = static_cast<const E*>(a.host_A[k]) + aoff + (int64_t)j * a.d_in[p] + (int64_t)c * P;
            len = min(P, a.d_in[p] - c * P);
        } else {
            rem -= rank * a.nci[p];
            const int j = rem / a.nco[p], c = rem - j * a.nco[p];
            src = static_cast<const E*>(a.host_B[k]) + boff + (int64_t)j * a.d_out[p] + (int64_t)c * P;
            len = min(P, a.d_out[p] - c * P);
        }
        const int page = a.tab[k][a.first_page[k] + q];
        dst = static_cast<E*>(a.pages) + ((int64_t)page << a.page_shift);
    };
    // G pages per pass, all their loads in flight before the first store
    for (int q0 = blockIdx.x * G; q0 < total; q0 += gridDim.x * G) {
        const E* src[G];
        E* dst[G];
        int len[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            resolve(min(q0 + g, total - 1), src[g], len[g], dst[g]);
            if (q0 + g >= total) len[g] = 0;  // past the last page: nothing read or written
        }
        for (int e0 = threadIdx.x * V; e0 < P; e0 += 256 * V * kPageInLoads) {
            u32x4 v[G][kPageInLoads];
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int i = 0; i < kPageInLoads; ++i) {
                    const int e = e0 + i * 256 * V;
                    v[g][i] = e < len[g] ? ld16(src[g] + e) : zero;
                }
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int i = 0; i < kPageInLoads; ++i) {
                    const int e = e0 + i * 256 * V;
                    if (len[g] > 0 && e < P) st16(dst[g] + e, v[g][i]);
                }
        }
    }
}

// Index upload: word i of the pinned host staging buffer (read over PCIe through its
// device mapping) to word i of device memory.  A kernel, not a copy command: on the
// stream it is ordered like the LoRA kernels around it, with no copy-engine hand-off.
__global__ __launch_bounds__(256) void upload_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                                                     int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

template <typename E>
hipError_t shrink_bgmv(const LoraArgs& a, int sum_parts, hipStream_t s) {
    const int nsum = sum_parts > 1 ? 4 * a.n_tiles : 0;
    const int np = a.n_multi > 1 ? a.n_multi : 1;
    hipLaunchKernelGGL(bgmv_shrink_kernel<E>, dim3((a.n_su + nsum) * np), dim3(256), 0, s, a, sum_parts);
    return hipGetLastError();
}

template <typename E>
hipError_t expand_bgmv(const LoraArgs& a, hipStream_t s) {
    constexpr int V = Elem<E>::kVec;
    const int nchunks = (a.d_out + 64 * V - 1) / (64 * V);
    const int64_t grid = a.n_multi > 1 ? (int64_t)a.eblk_multi[a.n_multi] : (int64_t)a.n_eu * nchunks;
    // up to about one round of workgroups (three per CU): the resolved entries
    if (grid <= 768)
        hipLaunchKernelGGL((bgmv_expand_kernel<E, true>), dim3((unsigned)grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((bgmv_expand_kernel<E, false>), dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bgmv_shrink(int dtype, const LoraArgs& a, int sum_parts, hipStream_t s) {
    return dtype == 1 ? shrink_bgmv<bf16_t>(a, sum_parts, s) : shrink_bgmv<float>(a, sum_parts, s);
}

int bgmv_expand_chunks(int dtype, int d_out) {
    const int cols = 64 * (dtype == 1 ? Elem<bf16_t>::kVec : Elem<float>::kVec);
    return (d_out + cols - 1) / cols;
}

hipError_t launch_bgmv_expand(int dtype, const LoraArgs& a, hipStream_t s) {
    return dtype == 1 ? expand_bgmv<bf16_t>(a, s) : expand_bgmv<float>(a, s);
}

int sgmv_shrink_parts(int dtype, const LoraArgs& a) {
    // K parts per tile: about two workgroups per CU in all, within the partial buffer; none once
    // the tiles alone cover half the CUs (measured on MI355X: 150 tiles of the 9,551-row
    // prefill take 30.5 us unsplit against 35.2 with 4 parts and their sum; 48 tiles of the
    // stack step's 2,769 prefill rows 15.9 us with 8 parts against 33.1 unsplit)
    if (a.n_tiles <= 0 || a.vpart == nullptr || a.vpart_rows < a.T) return 1;
    const int cus = gemm_cu_count();
    if (2 * a.n_tiles >= cus) return 1;
    const int bk = dtype == 1 ? 64 : 32;
    const int nsteps = (a.d_in + bk - 1) / bk;
    const int S = (2 * cus + a.n_tiles - 1) / a.n_tiles;
    return std::max(1, std::min({S, kMaxShrinkSplit, nsteps}));
}

hipError_t launch_sgmv_shrink(int dtype, const LoraArgs& a, bool sum, hipStream_t s) {
    const int S = sgmv_shrink_parts(dtype, a);
    const int np = a.n_multi > 1 ? a.n_multi : 1;
    const dim3 grid((unsigned)(a.n_tiles * S * np));
    if (dtype == 1)
        hipLaunchKernelGGL((sgmv_shrink_kernel<bf16_t>), grid, dim3(256), 0, s, a, S);
    else
        hipLaunchKernelGGL((sgmv_shrink_kernel<float>), grid, dim3(256), 0, s, a, S);
    if (sum && S > 1)
        hipLaunchKernelGGL(sgmv_shrink_sum_kernel, dim3((unsigned)(4 * a.n_tiles * np)), dim3(256), 0, s, a, S);
    return hipGetLastError();
}

hipError_t launch_sgmv_expand(int dtype, const LoraArgs& a, hipStream_t s) {
    const int ncol = (a.d_out + 63) / 64;
    const dim3 grid((unsigned)(a.n_tiles * ncol));
    if (dtype == 1)
        hipLaunchKernelGGL(sgmv_expand_kernel<bf16_t>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(sgmv_expand_kernel<float>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_upload(const void* src_host_dev, void* dst, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(upload_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint32_t*>(src_host_dev), static_cast<uint32_t*>(dst), n);
    return hipGetLastError();
}

hipError_t launch_page_in(int dtype, const PageInArgs& a, int max_blocks, hipStream_t s) {
    const int pages = a.block0[a.n_adapters];
    if (pages <= 0) return hipSuccess;
    const int groups = (pages + kPageInGroup - 1) / kPageInGroup;
    const int blocks = max_blocks > 0 && max_blocks < groups ? max_blocks : groups;
    if (dtype == 1)
        hipLaunchKernelGGL((page_in_kernel<bf16_t, kPageInGroup>), dim3(blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((page_in_kernel<float, kPageInGroup>), dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace hagemm
