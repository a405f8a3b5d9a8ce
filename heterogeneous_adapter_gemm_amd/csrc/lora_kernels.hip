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
//    Each workgroup takes a 64-row tile of a segment and runs the two small
//    contractions on the matrix cores: shrink [64 x d_in] x [d_in x r]
//    (K split over workgroups; the partial v are summed by the expand in a
//    fixed order) and expand [64 x r] x [r x 64 columns].
//  * Page-in: one workgroup per page reads the adapter's rows straight from
//    pinned host memory and writes the page, zero past the row's end.
#include "common.h"
#include "internal.h"

namespace hagemm {
namespace {

constexpr int kWaves = 4;  // waves per workgroup

__device__ __forceinline__ const int32_t* slot_table(const LoraArgs& a, int slot, int rank) {
    return a.page_tab + (int64_t)slot * a.slot_cap + (int64_t)rank * a.lp_per_rank;
}

// ---------------------------------------------------------------------------
// BGMV shrink: v[row][j] = sum_k x[row][k] * A[j][k] for the rows of one group
// and rank-rows j0 .. j0+3.
template <typename E>
__global__ __launch_bounds__(256) void bgmv_shrink_kernel(LoraArgs a) {
    constexpr int V = Elem<E>::kVec;
    constexpr int JB = kShrinkRowsPerUnit;
    constexpr int TB = kShrinkTokensPerPass;
    const int lane = threadIdx.x & 63;
    const int u = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (u >= a.n_su) return;
    const int g = a.su_group[u], j0 = a.su_j0[u];
    const int slot = a.g_slot[g], r = a.g_rank[g], beg = a.g_begin[g], cnt = a.g_count[g];
    const int32_t* tab = slot_table(a, slot, r);
    const E* pages = static_cast<const E*>(a.pages);
    const E* x = static_cast<const E*>(a.x);
    const int P = 1 << a.page_shift;
    const int nj = min(JB, r - j0);
    for (int t0 = 0; t0 < cnt; t0 += TB) {
        const int nt = min(TB, cnt - t0);
        int row[TB];
#pragma unroll
        for (int t = 0; t < TB; ++t) row[t] = a.rows[beg + t0 + min(t, nt - 1)];
        float acc[TB][JB];
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int j = 0; j < JB; ++j) acc[t][j] = 0.f;
        for (int c = 0; c < a.nci; ++c) {
            const int kbase = c << a.page_shift;
            const int klen = min(P, a.d_in - kbase);
            const E* pa[JB];
#pragma unroll
            for (int j = 0; j < JB; ++j) pa[j] = pages + ((int64_t)tab[(j0 + min(j, nj - 1)) * a.nci + c] << a.page_shift);
            for (int k = lane * V; k < klen; k += 64 * V) {
                float av[JB][V];
#pragma unroll
                for (int j = 0; j < JB; ++j) unpack(ld16(pa[j] + k), av[j], E{});
#pragma unroll
                for (int t = 0; t < TB; ++t) {
                    float xv[V];
                    unpack(ld16(x + (int64_t)row[t] * a.d_in + kbase + k), xv, E{});
#pragma unroll
                    for (int j = 0; j < JB; ++j)
#pragma unroll
                        for (int e = 0; e < V; ++e) acc[t][j] = fmaf(xv[e], av[j][e], acc[t][j]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int j = 0; j < JB; ++j) {
                const float s = wave_sum(acc[t][j]);
                if (lane == 0 && t < nt && j < nj) a.v[(int64_t)row[t] * a.vstride + j0 + j] = s;
            }
    }
}

// ---------------------------------------------------------------------------
// BGMV expand: y[row][n] += gamma * sum_j v[row][j] * B[j][n] for the rows of
// one group, columns of one 64*V chunk.
template <typename E>
__global__ __launch_bounds__(256) void bgmv_expand_kernel(LoraArgs a) {
    constexpr int V = Elem<E>::kVec;
    constexpr int TB = kExpandTokensPerPass;
    const int lane = threadIdx.x & 63;
    const int nchunks = (a.d_out + 64 * V - 1) / (64 * V);
    const int u = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (u >= a.n_groups * nchunks) return;
    const int g = u / nchunks, ch = u - g * nchunks;
    const int n = ch * 64 * V + lane * V;
    if (n >= a.d_out) return;  // d_out is a multiple of V: a vector is all in or all out
    const int slot = a.g_slot[g], r = a.g_rank[g], beg = a.g_begin[g], cnt = a.g_count[g];
    const float gamma = a.g_gamma[g];
    const int32_t* tabB = slot_table(a, slot, r) + r * a.nci;
    const E* pages = static_cast<const E*>(a.pages);
    E* y = static_cast<E*>(a.y);
    const int c = n >> a.page_shift, off = n & ((1 << a.page_shift) - 1);
    for (int t0 = 0; t0 < cnt; t0 += TB) {
        const int nt = min(TB, cnt - t0);
        int row[TB];
#pragma unroll
        for (int t = 0; t < TB; ++t) row[t] = a.rows[beg + t0 + min(t, nt - 1)];
        float acc[TB][V];
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int e = 0; e < V; ++e) acc[t][e] = 0.f;
#pragma unroll 4
        for (int j = 0; j < r; ++j) {
            float bv[V];
            unpack(ld16(pages + ((int64_t)tabB[j * a.nco + c] << a.page_shift) + off), bv, E{});
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                const float vv = a.v[(int64_t)row[t] * a.vstride + j];
#pragma unroll
                for (int e = 0; e < V; ++e) acc[t][e] = fmaf(vv, bv[e], acc[t][e]);
            }
        }
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            if (t < nt) {
                E* yp = y + (int64_t)row[t] * a.d_out + n;
                float yv[V];
                if (a.ybase) {
                    const float* bp = a.ybase + (int64_t)row[t] * a.d_out + n;
#pragma unroll
                    for (int q = 0; q < V; q += 4) {
                        const f32x4 b4 = *reinterpret_cast<const f32x4*>(bp + q);
                        yv[q] = b4[0]; yv[q + 1] = b4[1]; yv[q + 2] = b4[2]; yv[q + 3] = b4[3];
                    }
                } else {
                    unpack(ld16(yp), yv, E{});
                }
#pragma unroll
                for (int e = 0; e < V; ++e) yv[e] = fmaf(gamma, acc[t][e], yv[e]);
                st16(yp, pack(yv, E{}));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// SGMV shrink: partial v[kp][row][j] = sum_{k in part kp} x[row][k] * A[j][k]
// for a 64-row tile of one segment; wave w owns rows 16w .. 16w+15.
template <typename E>
__global__ __launch_bounds__(256) void sgmv_shrink_kernel(LoraArgs a) {
    constexpr int V = Elem<E>::kVec;
    constexpr int KG = 4 * V;  // K covered by one 16-byte load per lane group
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lg = lane >> 4, li = lane & 15;
    const int tile = blockIdx.x / a.ksplit, kp = blockIdx.x - tile * a.ksplit;
    const int s = a.t_seg[tile], row0 = a.t_row0[tile];
    const int slot = a.s_slot[s], r = a.s_rank[s], send = a.s_end[s];
    const int kb = kp * a.kchunk, ke = min(a.d_in, kb + a.kchunk);
    const int nb = (r + 15) >> 4;
    const int32_t* tab = slot_table(a, slot, r);
    const E* pages = static_cast<const E*>(a.pages);
    const E* xr = static_cast<const E*>(a.x) + (int64_t)min(row0 + 16 * w + li, send - 1) * a.d_in;
    const int pmask = (1 << a.page_shift) - 1;
    f32x4 acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int k = kb; k < ke; k += KG) {
        const int kk = k + V * lg;
        const bool kin = kk < ke;
        const u32x4 xa = kin ? ld16(xr + kk) : zero;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (b < nb) {
                const int j = 16 * b + li;
                u32x4 av = zero;
                if (kin && j < r) av = ld16(pages + ((int64_t)tab[j * a.nci + (kk >> a.page_shift)] << a.page_shift) + (kk & pmask));
                acc[b] = mma_step(xa, av, acc[b], E{});
            }
        }
    }
    // lane holds D[row = 4*lg + i][j = 16*b + li]
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int j = 16 * b + li;
        if (b < nb && j < r) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = row0 + 16 * w + 4 * lg + i;
                if (row < send) a.v[((int64_t)kp * a.T + row) * a.vstride + j] = acc[b][i];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// SGMV expand: y[row][n] += gamma * sum_j v[row][j] * B[j][n] for a 64-row
// tile of one segment and 64 output columns.  The B chunk is staged in LDS
// transposed ([n][j]) so each lane reads its K-contiguous fragment with one
// 16-byte load; v (fp32, summed over the shrink's K parts) enters the bf16
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
        // this lane's V consecutive j of v[vrow][*], summed over the K parts in order
        float vv[V];
#pragma unroll
        for (int e = 0; e < V; ++e) vv[e] = 0.f;
        const int j0 = kb + V * lg;
        for (int p = 0; p < a.ksplit; ++p) {
            const float* vp = a.v + ((int64_t)p * a.T + vrow) * a.vstride;
#pragma unroll
            for (int e = 0; e < V; ++e)
                if (j0 + e < r) vv[e] += vp[j0 + e];
        }
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
// Page-in: workgroup q copies the q-th page of one layer of an adapter from
// the pinned host blob (device-visible pointer) to its pool page.
template <typename E>
__global__ __launch_bounds__(256) void page_in_kernel(PageInArgs a) {
    constexpr int V = Elem<E>::kVec;
    const int q = blockIdx.x;
    int rem = q, p = 0;
    int64_t aoff = a.a_layer_off, boff = a.b_layer_off;
    for (; p < a.n_proj - 1; ++p) {
        const int np = a.rank * (a.nci[p] + a.nco[p]);
        if (rem < np) break;
        rem -= np;
        aoff += (int64_t)a.rank * a.d_in[p];
        boff += (int64_t)a.rank * a.d_out[p];
    }
    const int P = 1 << a.page_shift;
    const E* src;
    int len;
    if (rem < a.rank * a.nci[p]) {
        const int j = rem / a.nci[p], c = rem - j * a.nci[p];
        src = static_cast<const E*>(a.host_A) + aoff + (int64_t)j * a.d_in[p] + (int64_t)c * P;
        len = min(P, a.d_in[p] - c * P);
    } else {
        rem -= a.rank * a.nci[p];
        const int j = rem / a.nco[p], c = rem - j * a.nco[p];
        src = static_cast<const E*>(a.host_B) + boff + (int64_t)j * a.d_out[p] + (int64_t)c * P;
        len = min(P, a.d_out[p] - c * P);
    }
    const int page = a.tab[a.first_page + q];
    E* dst = static_cast<E*>(a.pages) + ((int64_t)page << a.page_shift);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int e = threadIdx.x * V; e < P; e += 256 * V) st16(dst + e, e < len ? ld16(src + e) : zero);
}

template <typename E>
hipError_t shrink_bgmv(const LoraArgs& a, hipStream_t s) {
    const int blocks = (a.n_su + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(bgmv_shrink_kernel<E>, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename E>
hipError_t expand_bgmv(const LoraArgs& a, hipStream_t s) {
    constexpr int V = Elem<E>::kVec;
    const int nchunks = (a.d_out + 64 * V - 1) / (64 * V);
    const int64_t units = (int64_t)a.n_groups * nchunks;
    hipLaunchKernelGGL(bgmv_expand_kernel<E>, dim3((unsigned)((units + kWaves - 1) / kWaves)), dim3(256), 0, s, a);
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
    const dim3 grid((unsigned)(a.n_tiles * a.ksplit));
    if (dtype == 1)
        hipLaunchKernelGGL(sgmv_shrink_kernel<bf16_t>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(sgmv_shrink_kernel<float>, grid, dim3(256), 0, s, a);
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

hipError_t launch_page_in(int dtype, const PageInArgs& a, hipStream_t s) {
    if (a.n_pages <= 0) return hipSuccess;
    if (dtype == 1)
        hipLaunchKernelGGL(page_in_kernel<bf16_t>, dim3(a.n_pages), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(page_in_kernel<float>, dim3(a.n_pages), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace hagemm
