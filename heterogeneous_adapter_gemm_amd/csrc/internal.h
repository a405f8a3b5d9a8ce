// Internal declarations shared by the host side (pool.cpp) and the gfx950
// kernels (lora_kernels.hip, gemm_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct lora_pool;

namespace hagemm {

// Pool queries for the engine layer (engine.cpp): pages an adapter of rank r takes; whether
// a resident slot's page-in copy has finished (queried without waiting).
int64_t pool_pages_for_rank(const lora_pool* p, int32_t rank);
// Set the calling thread's error message (lora_last_error) and return code.
int set_error(int code, const char* fmt, ...);
int pool_copy_done(lora_pool* p, int32_t slot, bool* done);
// Shape and limits of a pool, for the engine layer.
struct PoolInfo {
    bool host_only;
    int32_t elem_bytes, n_layers, n_proj, max_slots, max_rank, max_tokens, max_segments;
    int64_t a_elems_per_rank, b_elems_per_rank;   // one rank-row of A / B over every layer and projection
    uint64_t base_id;
};
PoolInfo pool_info(const lora_pool* p);

// Decode (BGMV) work partition constants.
constexpr int kShrinkRowsPerUnit = 4;   // rank-rows of A per shrink workgroup (one wave each)
constexpr int kShrinkTokensPerPass = 4; // tokens a shrink wave accumulates at once
constexpr int kShrinkTokensPerUnit = 4; // tokens of a group per shrink workgroup: one pass (a heavy group is split)
constexpr int kExpandTokensPerPass = 4; // tokens an expand workgroup accumulates at once
constexpr int kExpandTokensPerUnit = 4; // tokens of a group per expand work item: one pass
// Prefill (SGMV) tiles: 64 rows of one segment per workgroup (4 waves x 16 rows).
constexpr int kSegTileRows = 64;
// The SGMV shrink splits K over up to this many workgroups per tile (fp32 partials of v,
// summed in part order by a second launch).
constexpr int kMaxShrinkSplit = 8;
constexpr int kPlanRing = 4;            // device plan entries per pool (live plans at once)
constexpr int kMaxMulti = 8;            // projections one lora_linear_multi call takes
constexpr int kMaxProj = 16;            // projections per layer the page-in kernel handles
constexpr int kMaxRank = 64;

// Arrays of one plan, as int32 word offsets from the entry base.  Capacities
// derive from the pool's max_tokens / max_segments / max_rank.
struct PlanLayout {
    int64_t g_slot, g_rank, g_begin, g_count, g_gamma, rows;   // decode groups + decode rows
    int64_t s_slot, s_rank, s_gamma, s_begin, s_end;           // non-null segments
    int64_t t_seg, t_row0;                                     // segment row tiles
    int64_t row_slot;                                          // slot of every row, -1 = none
    int64_t eu;                                                // expand units [cap_eu][12] (see the expand kernel)
    int64_t su;                                                // shrink units [cap_su][8] (see the shrink unit)
    int64_t words;                                             // index words (uploaded)
    int64_t v_bytes_off;                                       // [multi][max_tokens][vstride] intermediate v (float)
    int64_t vpart_bytes_off;                                   // [multi][kMaxShrinkSplit][max_tokens][vstride] partials of v
    int64_t ybase_bytes_off;                                   // [multi][max_tokens][max d_out] fp32 base output of adapter rows
    int64_t entry_bytes;                                       // whole entry, 256-aligned
    int64_t v_pstride, vpart_pstride, ybase_pstride;           // floats between consecutive projections' v / partials / base
    int32_t cap_groups, cap_su, cap_eu, cap_segs, cap_tiles, vstride;
    int32_t vpart_rows;                                        // rows of one partial (0: no partial buffer)
    int32_t multi;                                             // projections whose v, partials and base fit
};

PlanLayout plan_layout(int32_t max_tokens, int32_t max_segments, int32_t max_rank, int32_t max_dout,
                       int32_t max_multi = 1);

// Kernel argument block of one LoRA-linear call (passed by value).
struct LoraArgs {
    const void* x;
    void* y;
    const float* ybase;        // fp32 base output of rows with an adapter, or NULL (then y holds the base)
    const void* pages;
    const int32_t* page_tab;   // [max_slots][slot_cap]
    float* v;                  // [T][vstride]
    const int32_t* g_slot;
    const int32_t* g_rank;
    const int32_t* g_begin;
    const int32_t* g_count;
    const float* g_gamma;
    const int32_t* rows;
    const int32_t* su;         // [n_su][8]: group, first rank-row | (first row of the group) << 8, slot, rank | rows << 8, rows[4]
    const int32_t* eu;         // [n_eu][12]: slot, rank | rows << 8, gamma bits, group; rows[4]; first row in the group, 0, 0, 0
    const int32_t* s_slot;
    const int32_t* s_rank;
    const float* s_gamma;
    const int32_t* s_begin;
    const int32_t* s_end;
    const int32_t* t_seg;
    const int32_t* t_row0;
    float* vpart;              // [kMaxShrinkSplit][vpart_rows][vstride] K-part partials of v
    int32_t vpart_rows;
    int32_t n_groups, n_su, n_eu, n_segs, n_tiles;
    int32_t d_in, d_out;
    int32_t page_shift;        // log2(page_elems)
    int32_t slot_cap;          // page-table words per slot
    int32_t lp_per_rank;       // offset of (layer, proj) in a slot's table, per unit of rank
    int32_t nci, nco;          // pages per A row / per B row
    int32_t vstride;           // floats per row of v
    int32_t T;                 // rows of the batch (stride of one v partial)
    int32_t T_pre;             // rows [0, T_pre) are prefill (segment) rows
    // shrinks and expands of several projections sharing x in one launch each
    // (lora_linear_multi): projection p's table offset is lp_multi[p], its v, partials and
    // fp32 base start p * v_pstride, p * vpart_pstride and p * ybase_pstride floats after v,
    // vpart and ybase; its output is y_multi[p], dout_multi[p] wide with nco_multi[p] pages
    // per B row, and its expand blocks are [eblk_multi[p], eblk_multi[p + 1]) of the expand
    // launch.  n_multi <= 1: one projection (lp_per_rank, y, d_out, nco).
    int32_t n_multi;
    int32_t lp_multi[kMaxMulti];
    int32_t dout_multi[kMaxMulti], nco_multi[kMaxMulti];
    int32_t eblk_multi[kMaxMulti + 1];
    void* y_multi[kMaxMulti];
    int64_t v_pstride, vpart_pstride, ybase_pstride;
};

// Page-in of one layer of up to kPageInBatch adapters (one launch).
constexpr int kPageInBatch = 16;
struct PageInArgs {
    void* pages;
    int32_t page_shift;
    int32_t n_proj;
    int32_t n_adapters;
    int32_t n_layers;                       // consecutive layers of each adapter in the launch (>= 1)
    int32_t d_in[kMaxProj];
    int32_t d_out[kMaxProj];
    int32_t nci[kMaxProj];
    int32_t nco[kMaxProj];
    int32_t block0[kPageInBatch + 1];       // first page of each adapter in the launch; block0[n] = total
    const void* host_A[kPageInBatch];       // device-visible pointers to the pinned A / B blobs
    const void* host_B[kPageInBatch];
    const int32_t* tab[kPageInBatch];       // the slot's page-table row (device)
    int32_t rank[kPageInBatch];
    int32_t first_page[kPageInBatch];       // index (in the slot's list) of the first layer's first page
    int64_t a_layer_off[kPageInBatch];      // element offset of the first layer in the A / B source
    int64_t b_layer_off[kPageInBatch];
};

// Compute units of the current device (queried once).
int gemm_cu_count();

// Launchers (return hipGetLastError() after the launch).
// sum_parts > 1: the launch also sums the SGMV shrink's sum_parts K-part partials of v
hipError_t launch_bgmv_shrink(int dtype, const LoraArgs& a, int sum_parts, hipStream_t s);
// column chunks of the BGMV expand per unit of d_out columns (its blocks per expand unit)
int bgmv_expand_chunks(int dtype, int d_out);
hipError_t launch_bgmv_expand(int dtype, const LoraArgs& a, hipStream_t s);
// K parts of the SGMV shrink (1: it writes v itself); with more, its partials are summed by a
// launch of their own (sum) or by the call's BGMV shrink launch
int sgmv_shrink_parts(int dtype, const LoraArgs& a);
hipError_t launch_sgmv_shrink(int dtype, const LoraArgs& a, bool sum, hipStream_t s);
hipError_t launch_sgmv_expand(int dtype, const LoraArgs& a, hipStream_t s);
// max_blocks: workgroups of the launch, each striding over the pages; 0: one short-lived
// workgroup per group of pages.  Reading pinned host memory over PCIe wants a few striding
// ones; a copy out of a device staging area (HBM to HBM) beside the GEMM wants short ones, so
// that no workgroup holds a CU that a GEMM tile is waiting for longer than a page group takes.
hipError_t launch_page_in(int dtype, const PageInArgs& a, int max_blocks, hipStream_t s);
constexpr int kPageInBlocksPcie = 16;
constexpr int kPageInBlocksStaged = 0;
// Layers per copy of a staged page-in (fewer when the staging area cannot hold them)
constexpr int kStageChunkLayers = 4;
// n 32-bit words from pinned host memory (its device mapping) to device memory, by a
// kernel on s (index and page-table uploads)
hipError_t launch_upload(const void* src_host_dev, void* dst, int64_t n, hipStream_t s);
// y = x w^T.  With row_slot != NULL, rows m with row_slot[m] >= 0 are written
// unrounded (fp32) to ybase [M][N] instead of y, for the delta kernels to
// finish with a single rounding.  With seg != NULL the GEMM may instead add
// the segments' LoRA expand (gamma * v B, v from the SGMV shrink) to its
// accumulators before rounding; it then returns *fused = true and the rows
// of those segments need no separate expand.
hipError_t launch_gemm(int dtype, const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                       const int32_t* row_slot, float* ybase, const LoraArgs* seg, bool* fused, hipStream_t s);
// FP8 base: y = (x q^T) * scale[n], x bf16, q E4M3 codes [N][K], scale fp32 [N] (16-byte
// aligned); rows m with row_slot[m] >= 0 go unrounded to ybase.  gemm_w8_ok: N % 4 == 0,
// K % 128 == 0, 32-bit byte offsets.
bool gemm_w8_ok(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_w8(const void* x, const void* q, const float* scale, void* y, int64_t M, int64_t N, int64_t K,
                          const int32_t* row_slot, float* ybase, hipStream_t s);
// FP8 base for decode batches (M <= 64, a.n_su > 0): the product, the BGMV shrink and the
// index copy in one launch, as launch_gemm_shrink (raw_mask as there).
bool gemm_w8_shrink_fits(int64_t M, int64_t N, int64_t K, int n_su);
hipError_t launch_gemm_w8_shrink(const void* x, const void* q, const float* scale, void* y, int64_t M, int64_t N,
                                 int64_t K, const int32_t* row_slot, uint64_t raw_mask, float* ybase,
                                 const LoraArgs& a, const void* cp_src, void* cp_dst, int64_t cp_n, hipStream_t s);
// Decode batches (bf16, M <= 64, a.n_su > 0: gemm_shrink_fits): the base
// GEMM and the BGMV shrink in one launch.  With cp_n > 0 the launch also
// copies cp_n 32-bit words from cp_src to cp_dst (kCopyBlocks workgroups):
// the index of a plan whose first call this is, read by this launch from the
// plan's host staging buffer (device mapping) and kept for later kernels.
// raw_mask (bit m: row m has an adapter) stands for row_slot when nonzero, so
// the GEMM tiles read no index memory.
constexpr int kCopyBlocks = 4;
bool gemm_shrink_fits(int dtype, int64_t M, int n_su);
hipError_t launch_gemm_shrink(int dtype, const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                              const int32_t* row_slot, uint64_t raw_mask, float* ybase, const LoraArgs& a,
                              const void* cp_src, void* cp_dst, int64_t cp_n, hipStream_t s);

}  // namespace hagemm
