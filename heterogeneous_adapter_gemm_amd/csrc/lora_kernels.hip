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
//    The two small contractions run on the matrix cores: shrink [32 x d_in]
//    x [d_in x r] per workgroup (its 8 waves split K and meet in LDS) and
//    expand [64 x r] x [r x 64 columns] (in the long-batch GEMM's epilogue
//    when that kernel runs).
//  * Page-in: one workgroup per page reads the adapter's rows straight from
//    pinned host memory and writes the page, zero past the row's end.
#include "bgmv_device.h"
#include "common.h"
#include "internal.h"

namespace hagemm {
namespace {


// ---------------------------------------------------------------------------
// BGMV shrink (device code in bgmv_device.h)
template <typename E>
__global__ __launch_bounds__(256) void bgmv_shrink_kernel(LoraArgs a) {
    bgmv_shrink_unit<E>(a, blockIdx.x);
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
template <typename E, int JW, bool RES>
__device__ __forceinline__ void expand_chunk(const LoraArgs& a, int e, int ch,
                                             float (&part)[4][kExpandTokensPerPass][Elem<E>::kVec][64],
                                             float (&vs)[kExpandTokensPerPass][kMaxRank]) {
    constexpr int V = Elem<E>::kVec;
    constexpr int TB = kExpandTokensPerPass;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = ch * 64 * V + lane * V;
    const bool nin = n < a.d_out;  // d_out is a multiple of V: a vector is all in or all out
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
    const int32_t* tabB = slot_table(a, slot, r) + r * a.nci;
    const E* pages = static_cast<const E*>(a.pages);
    E* y = static_cast<E*>(a.y);
    const int nc = min(n, a.d_out - V);  // clamped column for the loads
    const int c = nc >> a.page_shift, off = nc & ((1 << a.page_shift) - 1);
    // this wave's B rows for the chunk, all loads in flight together
    u32x4 bv[JW];
#pragma unroll
    for (int i = 0; i < JW; ++i) {
        const int j = min(w + 4 * i, r - 1);
        bv[i] = ld16(pages + ((int64_t)tabB[j * a.nco + c] << a.page_shift) + off);
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
            if (j < r) vs[t][j] = a.v[(int64_t)row[t] * a.vstride + j];
        }
        float yv[V];
        if (a.ybase) {
            const float* bp = a.ybase + (int64_t)row[w] * a.d_out + nc;
#pragma unroll
            for (int q = 0; q < V; q += 4) {
                const f32x4 b4 = *reinterpret_cast<const f32x4*>(bp + q);
                yv[q] = b4[0];
                yv[q + 1] = b4[1];
                yv[q + 2] = b4[2];
                yv[q + 3] = b4[3];
            }
        } else {
            unpack(ld16(y + (int64_t)row[w] * a.d_out + nc), yv, E{});
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
            st16(y + (int64_t)row[w] * a.d_out + n, pack(yv, E{}));
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
template <typename E, bool RES>
__global__ __launch_bounds__(256, RES ? 1 : 4) void bgmv_expand_kernel(LoraArgs a) {
    constexpr int V = Elem<E>::kVec;
    __shared__ float part[4][kExpandTokensPerPass][V][64];
    __shared__ float vs[kExpandTokensPerPass][kMaxRank];
    const int nchunks = (a.d_out + 64 * V - 1) / (64 * V);
    const int e = blockIdx.x / nchunks, ch = blockIdx.x - e * nchunks;
    const int r = RES ? a.eu[12 * e + 1] & 255 : a.g_rank[a.eu[12 * e + 3]];
    const int jw = (r + 3) / 4;  // rank-rows per wave
    if (jw <= 1) expand_chunk<E, 1, RES>(a, e, ch, part, vs);
    else if (jw <= 2) expand_chunk<E, 2, RES>(a, e, ch, part, vs);
    else if (jw <= 4) expand_chunk<E, 4, RES>(a, e, ch, part, vs);
    else if (jw <= 8) expand_chunk<E, 8, RES>(a, e, ch, part, vs);
    else expand_chunk<E, kMaxRank / 4, RES>(a, e, ch, part, vs);
}

// ---------------------------------------------------------------------------
// SGMV shrink: v[row][j] = sum_k x[row][k] * A[j][k] for 32 rows of one
// segment (half of a 64-row tile; 16 rows when the batch has few tiles) and
// every j < r.  The 8 waves split K into equal ranges of 4V-element steps;
// each wave holds all the workgroup's rows (two 16-row blocks, so every A
// fragment feeds two matrix ops) and keeps the loads of the next U steps in
// flight while it multiplies the current ones.  The
// waves' partial sums meet in LDS and each output is their sum in wave order,
// written once: no K-part partials leave the chip.
// NB = 16-row blocks of A the segment's rank needs (1, 2 or 4: a uniform switch in
// the kernel), so a rank-8 segment loads and multiplies one block, not four.
// RB = 16-row blocks of x per workgroup (2: 32 rows; 1: 16 rows, twice the
// workgroups, for batches with few segment tiles).
template <typename E, int NB, int RB>
__device__ __forceinline__ void sgmv_shrink_tile(const LoraArgs& a, float (&red)[8][32 * 68], int s, int send,
                                                 int row0, int r) {
    constexpr int V = Elem<E>::kVec;
    constexpr int KG = 4 * V;  // K covered by one 16-byte load per lane group
    constexpr int NW = 8, U = 2, RS = 68;  // waves, steps per load batch, LDS row stride (floats)
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lg = lane >> 4, li = lane & 15;
    const int slot = a.s_slot[s];
    const int32_t* tab = slot_table(a, slot, r);
    const E* pages = static_cast<const E*>(a.pages);
    const int pmask = (1 << a.page_shift) - 1;
    const int nsteps = (a.d_in + KG - 1) / KG;
    const int s0 = nsteps * w / NW, s1 = nsteps * (w + 1) / NW;
    const E* xr[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) xr[rb] = static_cast<const E*>(a.x) + (int64_t)min(row0 + 16 * rb + li, send - 1) * a.d_in;
    // rank rows past r repeat row r - 1: their outputs are never stored
    const int32_t* tabj[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) tabj[b] = tab + min(16 * b + li, r - 1) * a.nci;
    // A row bases for the page of the wave's first step and the next one (a 4V-element step
    // never straddles pages, so the page is the same for all lanes); a range that reaches
    // further moves the pair on, which costs one table look-up
    int pg0 = (s0 * KG) >> a.page_shift;
    const E* pb0[NB];
    const E* pb1[NB];
    auto rebase = [&](int pg) {
        pg0 = pg;
        const int pg1 = min(pg + 1, a.nci - 1);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            pb0[b] = pages + ((int64_t)tabj[b][pg] << a.page_shift);
            pb1[b] = pages + ((int64_t)tabj[b][pg1] << a.page_shift);
        }
    };
    rebase(pg0);
    f32x4 acc[RB][NB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[rb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // loads of U steps from step st on: addresses clamped into the rows, masked at use; every
    // wave loads the NB 16-row blocks of A (rows past the rank repeat row r - 1)
    auto load = [&](int st, u32x4 (&xa)[U][RB], u32x4 (&av)[U][NB]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k0 = min((st + u) * KG, (nsteps - 1) * KG);  // step start, clamped
            const int kk = min(k0 + V * lg, a.d_in - V);
            const int pg = k0 >> a.page_shift;
            if (pg > pg0 + 1) rebase(pg);
            const bool first = pg == pg0;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) xa[u][rb] = ld16(xr[rb] + kk);
#pragma unroll
            for (int b = 0; b < NB; ++b) av[u][b] = ld16((first ? pb0[b] : pb1[b]) + (kk & pmask));
        }
    };
    auto mul = [&](int st, const u32x4 (&xa)[U][RB], const u32x4 (&av)[U][NB]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // steps outside this wave's range, and K past the end, contribute zero
            const bool kin = st + u < s1 && (st + u) * KG + V * lg < a.d_in;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const u32x4 xv = kin ? xa[u][rb] : zero;
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[rb][b] = mma_step(xv, av[u][b], acc[rb][b], E{});
            }
        }
    };
    u32x4 x0[U][RB], a0[U][NB], x1[U][RB], a1[U][NB];
    load(s0, x0, a0);
    for (int st = s0; st < s1; st += 2 * U) {
        load(st + U, x1, a1);
        mul(st, x0, a0);
        load(st + 2 * U, x0, a0);
        mul(st + U, x1, a1);
    }
    // lane holds D[row = 16 rb + 4 lg + i][j = 16 b + li]
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[w][(16 * rb + 4 * lg + i) * RS + 16 * b + li] = acc[rb][b][i];
    __syncthreads();
    // (columns j < r < 16 NB only: the blocks this tile wrote)
    for (int idx = threadIdx.x; idx < 16 * RB * 64; idx += NW * 64) {
        const int row = idx >> 6, j = idx & 63;
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < NW; ++q) sum += red[q][row * RS + j];
        if (j < r && row0 + row < send) a.v[(int64_t)(row0 + row) * a.vstride + j] = sum;
    }
}

template <typename E, int RB>
__global__ __launch_bounds__(512) void sgmv_shrink_kernel(LoraArgs a) {
    __shared__ float red[8][32 * 68];
    constexpr int PARTS = 4 / RB;  // workgroups per 64-row tile
    const int tile = blockIdx.x / PARTS;
    const int s = a.t_seg[tile], send = a.s_end[s];
    const int row0 = a.t_row0[tile] + 16 * RB * (blockIdx.x % PARTS);
    if (row0 >= send) return;  // the whole workgroup: the segment ends before its rows
    const int r = a.s_rank[s];
    if (r <= 16) sgmv_shrink_tile<E, 1, RB>(a, red, s, send, row0, r);
    else if (r <= 32) sgmv_shrink_tile<E, 2, RB>(a, red, s, send, row0, r);
    else sgmv_shrink_tile<E, 4, RB>(a, red, s, send, row0, r);
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
// adapter k) is copied from that adapter's rows to its pool page.  The source
// is either the pinned host blob (device-visible pointer, read over PCIe) or
// the copy of the layer that the copy engine put in a device staging area.
// For the host blob a small grid strides over the pages: the copy is bound by
// PCIe, and it runs beside the LoRA-linear kernels, whose occupancy a grid of
// one workgroup per page would take.  A workgroup
// takes kPageInGroup pages per pass and each thread has kPageInLoads 16-byte
// loads of each in flight (with 8 KB pages, one pass covers a page).
// Measured on the Llama-7B stack step with 1.8 GB paged in per step (MI355X):
// 16 workgroups x 2 pages 63.6 ms/step at 44 GB/s over PCIe, 32 x 1 67.0-67.9
// ms at 52 GB/s (the compute kernels beside it lose more than the copy gains),
// 8 x 4 or 8 x 8 66.9-70.8 ms at 27-29 GB/s (the copy becomes the bound).
constexpr int kPageInLoads = 2;
constexpr int kPageInGroup = 2;

template <typename E, int G>
__global__ __launch_bounds__(256) void page_in_kernel(PageInArgs a) {
    constexpr int V = Elem<E>::kVec;
    const int P = 1 << a.page_shift;
    const int total = a.block0[a.n_adapters];
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // source, valid length and destination of launch page qq
    auto resolve = [&](int qq, const E*& src, int& len, E*& dst) {
        int k = 0;
        while (k + 1 < a.n_adapters && qq >= a.block0[k + 1]) ++k;
        const int q = qq - a.block0[k];
        const int rank = a.rank[k];
        int rem = q, p = 0;
        int64_t aoff = a.a_layer_off[k], boff = a.b_layer_off[k];
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
hipError_t shrink_bgmv(const LoraArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(bgmv_shrink_kernel<E>, dim3(a.n_su), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename E>
hipError_t expand_bgmv(const LoraArgs& a, hipStream_t s) {
    constexpr int V = Elem<E>::kVec;
    const int nchunks = (a.d_out + 64 * V - 1) / (64 * V);
    const int64_t grid = (int64_t)a.n_eu * nchunks;
    // up to about one round of workgroups (three per CU): the resolved entries
    if (grid <= 768)
        hipLaunchKernelGGL((bgmv_expand_kernel<E, true>), dim3((unsigned)grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((bgmv_expand_kernel<E, false>), dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bgmv_shrink(int dtype, const LoraArgs& a, hipStream_t s) {
    return dtype == 1 ? shrink_bgmv<bf16_t>(a, s) : shrink_bgmv<float>(a, s);
}

hipError_t launch_bgmv_expand(int dtype, const LoraArgs& a, hipStream_t s) {
    return dtype == 1 ? expand_bgmv<bf16_t>(a, s) : expand_bgmv<float>(a, s);
}

hipError_t launch_sgmv_shrink(int dtype, const LoraArgs& a, hipStream_t s) {
    // 32-row workgroups, or 16-row ones when that would leave CUs idle
    if (a.n_tiles * 2 >= 256) {
        const dim3 grid((unsigned)(a.n_tiles * 2));
        if (dtype == 1)
            hipLaunchKernelGGL((sgmv_shrink_kernel<bf16_t, 2>), grid, dim3(512), 0, s, a);
        else
            hipLaunchKernelGGL((sgmv_shrink_kernel<float, 2>), grid, dim3(512), 0, s, a);
    } else {
        const dim3 grid((unsigned)(a.n_tiles * 4));
        if (dtype == 1)
            hipLaunchKernelGGL((sgmv_shrink_kernel<bf16_t, 1>), grid, dim3(512), 0, s, a);
        else
            hipLaunchKernelGGL((sgmv_shrink_kernel<float, 1>), grid, dim3(512), 0, s, a);
    }
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
    const int blocks = groups < max_blocks ? groups : max_blocks;
    if (dtype == 1)
        hipLaunchKernelGGL((page_in_kernel<bf16_t, kPageInGroup>), dim3(blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((page_in_kernel<float, kPageInGroup>), dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace hagemm
