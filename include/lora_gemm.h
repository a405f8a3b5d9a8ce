/*
 * lora_gemm.h - C ABI of the MI355X (gfx950) multi-adapter LoRA-linear library.
 *
 * The operation: for every row t of a batch routed to adapter a(t),
 *
 *     y_t = x_t W0^T + (alpha_a / r_a) * (x_t A_a^T) B_a          (none: y_t = x_t W0^T)
 *
 * i.e. the LoRA forward pass y = W0 x + (alpha / r) B A x ("S-LoRA: Serving
 * Thousands of Concurrent Adapters in 2026", The Three Core Pillars) computed
 * unmerged for a batch whose rows use different adapters: one dense product
 * with the shared base weight for the whole batch, then per row a shrink
 * v = A x (rank r) and an expand y += gamma B v ("Multi-LoRA serving: S-LoRA,
 * Punica and adapter batching", How the kernels work).  Decode rows are
 * handled one token at a time (BGMV); prefill rows in contiguous segments
 * that share an adapter (SGMV).  Adapter weights live in a unified pool of
 * fixed-size pages, one hidden-size vector per page, shared with KV blocks,
 * with ranks mixed and unpadded ("S-LoRA: Serving Thousands of Concurrent
 * LoRA Adapters", Unified paging and Kernels and tensor parallelism).
 *
 * Layouts (all row-major, element type = the pool's dtype):
 *   x   [T][d_in]            W0 [d_out][d_in]          y [T][d_out]
 *   A_a r rows of length d_in;  B_a r rows of length d_out (row j = column j
 *   of the d_out x r matrix B).  A vector of length L takes ceil(L / page)
 *   pages holding consecutive chunks; the last page is zero past L.
 *
 * Conventions:
 *   - Every function returns LORA_OK (0) or a negative LORA_E* code; on error
 *     nothing is written through out-parameters and the pool is unchanged;
 *     lora_last_error() then gives a message (thread-local, valid until the
 *     thread's next call).
 *   - Device buffers (pages, meta workspace, x, W0, y) are owned by the caller
 *     (allocated by PyTorch or hipMalloc); the library never allocates device
 *     memory.  It allocates host memory only: its tables, and a small pinned
 *     staging ring per pool (hipHostMalloc) for index uploads.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously; device faults surface at the caller's next synchronise.
 *   - A pool and its plans are not thread-safe: one host thread at a time.
 *   - Element types: LORA_F32 (float) or LORA_BF16 (bfloat16 bits, uint16).
 *     Outputs are rounded to the element type (bf16: nearest-even).
 */
#ifndef LORA_GEMM_H
#define LORA_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    LORA_OK = 0,
    LORA_EINVAL = -1,       /* malformed argument (size, index, pointer, layout) */
    LORA_ENOPAGES = -2,     /* not enough free pages; nothing allocated */
    LORA_ENOTRESIDENT = -3, /* adapter/slot not resident in the pool */
    LORA_EBUSY = -4,        /* adapter still referenced (acquired or in a live plan) */
    LORA_EEXIST = -5,       /* adapter already resident */
    LORA_EBASE = -6,        /* adapter was made for another base model */
    LORA_EHIP = -7,         /* a HIP runtime call failed */
    LORA_ENOSLOT = -8       /* every adapter slot is taken */
};

typedef enum lora_dtype { LORA_F32 = 0, LORA_BF16 = 1 } lora_dtype;

typedef struct lora_pool lora_pool; /* opaque, host side */
typedef struct lora_plan lora_plan; /* opaque per-batch index */

/*
 * Pool description.  The pool covers `num_pages` pages of `page_elems`
 * elements in `pages_dev` (caller-owned device memory, num_pages*page_elems
 * elements), for a model of n_layers x n_proj LoRA-targeted projections with
 * widths d_in[p] -> d_out[p].
 *   free_order   host [num_pages] permutation: the initial free list (the
 *                physical order pages are handed out); NULL = 0..num_pages-1.
 *   max_slots    most adapters resident at once; max_rank: largest rank.
 *   max_tokens   largest batch (rows) of one plan; max_segments: largest
 *                number of prefill segments of one plan.
 *   meta_dev     caller-owned device workspace of at least
 *                lora_pool_meta_bytes() bytes (page tables + plan ring).
 *   base_id      identity of the base model; page-ins must match it
 *                ("Multi-LoRA serving ...", Failure modes: silent wrong base).
 *   stage_dev    optional caller-owned device staging area of stage_bytes
 *                bytes (256-byte aligned) for page-ins: with it, a page-in
 *                copies the host rows into the staging area with the copy
 *                engine (hipMemcpyAsync) and scatters them into the pages
 *                with a kernel (HBM to HBM), so no compute unit waits on PCIe
 *                reads; it must hold one layer of one adapter of max_rank
 *                (max_rank * sum_p (d_in[p] + d_out[p]) elements); four
 *                layers of a whole batch let the batch go in one copy group
 *                per four layers.  NULL
 *                (stage_bytes 0): a kernel gathers the rows straight from the
 *                pinned host memory over PCIe.
 *   max_multi    most projections one lora_linear_multi call takes (0 or 1:
 *                single calls only; at most 8): each plan entry of the
 *                workspace holds that many sets of the shrink's intermediate v,
 *                its K-part partials and the fp32 base of rows with an adapter
 *                (max_tokens x the largest d_out floats each).
 * pages_dev == NULL and meta_dev == NULL together make a host-only pool: the
 * allocator, tables and plans work, no device work is ever issued, and
 * lora_linear* return LORA_EINVAL.
 * Constraints: page_elems a power of two, at least 512 (bf16) or 256 (f32);
 * every d_in, d_out a positive multiple of 8 (bf16) or 4 (f32);
 * 1 <= max_rank <= 64; 1 <= max_tokens <= 2^22; n_layers, n_proj >= 1.
 */
typedef struct lora_pool_desc {
    int32_t dtype;
    int32_t page_elems;
    int64_t num_pages;
    void* pages_dev;
    const int32_t* free_order;
    int32_t n_layers;
    int32_t n_proj;
    const int32_t* d_in;
    const int32_t* d_out;
    int32_t max_slots;
    int32_t max_rank;
    int32_t max_tokens;
    int32_t max_segments;
    void* meta_dev;
    int64_t meta_bytes;
    uint64_t base_id;
    void* stage_dev;
    int64_t stage_bytes;
    int32_t max_multi;
} lora_pool_desc;

/* Bytes of device workspace (meta_dev) the described pool needs. */
int lora_pool_meta_bytes(const lora_pool_desc* desc, int64_t* out_bytes);

/* Create a pool ("S-LoRA: Serving Thousands of Concurrent LoRA Adapters",
 * Unified paging).  Copies desc's host arrays; clears the device page tables
 * with a synchronous copy.  *out owns host memory only. */
int lora_pool_create(const lora_pool_desc* desc, lora_pool** out);

/* Destroy a pool: waits for the pool's outstanding uploads, frees host state.
 * The caller's device buffers are untouched. */
int lora_pool_destroy(lora_pool* pool);

/*
 * Page an adapter in from pinned host memory ("Multi-LoRA serving ...", What
 * the engine does each step: copy a missing adapter into the pool over PCIe;
 * "S-LoRA: Serving Thousands of Concurrent LoRA Adapters", Host memory for
 * adapters).  Allocates rank * (pages per rank-row) pages from the front of
 * the free list - all or none - in the order layer, projection, A before B,
 * rank-row, chunk; takes the lowest free slot; uploads the slot's page table
 * and enqueues the copy on `stream`, in layer order: with a staging area,
 * the copy engine brings up to 4 layers of as many adapters as the staging
 * area holds into it and one kernel scatters those layers into the pages;
 * without one, a gather kernel per layer reads the host rows over PCIe and
 * writes the pages (zero tails included either way).
 *   host_A  pinned (hipHostMalloc / torch pin_memory) array holding, for each
 *           layer then projection, the r x d_in[p] matrix A; host_A_bytes its
 *           size, which must equal sum_p n_layers * r * d_in[p] * elem bytes.
 *   host_B  likewise the r x d_out[p] matrices B (row j = column j of B).
 * The host arrays must stay valid until the work on `stream` has run.  Rows
 * that later kernels read from this adapter wait for the copy of their layer
 * automatically (lora_linear makes its stream wait on the copy's per-layer
 * events), so `stream` may differ from the compute stream.
 * Errors: EINVAL (adapter_id < 0, rank outside 1..max_rank, alpha not
 * finite, wrong sizes, host memory not pinned), EBASE, EEXIST, ENOSLOT,
 * ENOPAGES, EHIP.  Checked in that order. */
int lora_pool_page_in(lora_pool* pool, int32_t adapter_id, int32_t rank, float alpha, uint64_t base_id,
                      const void* host_A, int64_t host_A_bytes, const void* host_B, int64_t host_B_bytes,
                      void* stream, int32_t* out_slot);

/*
 * Page in several adapters at once (the same step of the pages as
 * lora_pool_page_in: the adapters a step needs that are not resident).  The
 * result equals n lora_pool_page_in calls in request order - same slots,
 * same pages, same checks, stopping at the first failing request with nothing
 * changed - except for the order of the copies: the copies are enqueued
 * layer by layer (a staging area's chunk of up to 4 layers at a time, for up to
 * 16 adapters), so layer l of every adapter of the batch is in before the
 * layers after its chunk of any.  A LoRA-linear
 * call of layer l then waits for 1/n_layers of the batch's bytes, not for
 * whole adapters.  Requests name distinct adapters (EEXIST otherwise).
 * out_slots [n] may be NULL.  Errors as lora_pool_page_in. */
typedef struct lora_page_in_req {
    int32_t adapter_id;
    int32_t rank;
    float alpha;
    int32_t reserved;      /* 0 */
    uint64_t base_id;
    const void* host_A;    /* pinned, layout as for lora_pool_page_in */
    int64_t host_A_bytes;
    const void* host_B;
    int64_t host_B_bytes;
} lora_page_in_req;
int lora_pool_page_in_batch(lora_pool* pool, int32_t n, const lora_page_in_req* reqs, void* stream,
                            int32_t* out_slots);

/* Evict a resident adapter: its pages go to the tail of the free list in
 * allocation order and its slot is freed.  EBUSY while acquired or referenced
 * by a live plan: an adapter that a running batch still reads is never the
 * one evicted ("Multi-LoRA serving ...", What the engine does each step: the
 * victim is the least recently used adapter no request is using);
 * ENOTRESIDENT if not resident.  Blocks until device work of earlier plans
 * that read the adapter has finished, so its pages can be reused at once. */
int lora_pool_evict(lora_pool* pool, int32_t adapter_id);

/* Slot of a resident adapter (ENOTRESIDENT otherwise): the engine step's
 * lookup from an adapter to its place in the GPU pool before it builds the
 * batch index ("Multi-LoRA serving ...", What the engine does each step). */
int lora_pool_slot_of(const lora_pool* pool, int32_t adapter_id, int32_t* out_slot);

/* Batch lookup, the per-step index ("Multi-LoRA serving ...", How the kernels
 * work): out_slots[i] = slot of adapter_ids[i], or -1 where adapter_ids[i] < 0.
 * ENOTRESIDENT (nothing written) if any id is not resident. */
int lora_pool_slots_of(const lora_pool* pool, int32_t n, const int32_t* adapter_ids, int32_t* out_slots);

/* Reference counting of a resident slot; an acquired slot cannot be evicted
 * (EBUSY), so a request holding its adapter keeps it resident while it runs
 * ("Multi-LoRA serving ...", What the engine does each step: only adapters no
 * request uses are eviction candidates).  acquire: ENOTRESIDENT on an empty
 * slot; release: EINVAL if the slot holds no reference. */
int lora_pool_acquire(lora_pool* pool, int32_t slot);
int lora_pool_release(lora_pool* pool, int32_t slot);

/* KV blocks share the pool ("S-LoRA: Serving Thousands of Concurrent LoRA
 * Adapters", Unified paging): take n pages from the front of the free list
 * (all or none; ENOPAGES), or return pages (each must be a KV page, listed
 * once; EINVAL otherwise) to the tail in the given order.  The library never
 * reads or writes KV page contents. */
int lora_pool_alloc_kv(lora_pool* pool, int32_t n_pages, int32_t* out_pages);
int lora_pool_free_kv(lora_pool* pool, int32_t n_pages, const int32_t* pages);

/* Read back a slot's pages for (layer, proj): a_pages [r][ceil(d_in/page)],
 * b_pages [r][ceil(d_out/page)] (host arrays, caller-sized). */
int lora_pool_page_table(const lora_pool* pool, int32_t slot, int32_t layer, int32_t proj,
                         int32_t* a_pages, int32_t* b_pages);

/* Pool counters and the free list (host copy; cap = capacity of out). */
int lora_pool_stats(const lora_pool* pool, int64_t* free_pages, int32_t* resident, int64_t* kv_pages);
int lora_pool_free_list(const lora_pool* pool, int64_t cap, int32_t* out, int64_t* n_out);

/* Rank, alpha and adapter id of a resident slot. */
int lora_pool_slot_info(const lora_pool* pool, int32_t slot, int32_t* rank, float* alpha, int32_t* adapter_id);

/*
 * Per-step batch plan: the index built once per step and shared by every
 * LoRA-linear call of the step ("Multi-LoRA serving ...", How the kernels
 * work and What the engine does each step).  Rows [0, seg_start[S]) are
 * prefill rows in S segments; segment s covers rows [seg_start[s],
 * seg_start[s+1]) with adapter slot seg_slot[s] (-1 = none).  The next
 * n_decode rows are decode rows with slots token_slot[i] (-1 = none).
 * All arrays are host arrays.  The plan groups decode rows by slot (stable),
 * splits segments into row tiles, acquires every slot it names (released by
 * lora_plan_destroy) and writes the index to a pinned staging buffer; the
 * index reaches the pool's plan ring on the device with the plan's first
 * lora_linear, on that call's stream (no host wait).  `stream` is where
 * lora_plan_destroy orders the plan's release if no call used it.
 * Errors: EINVAL (seg_start[0] != 0, decreasing, S or rows beyond the pool's
 * max_segments / max_tokens, slot out of range), ENOTRESIDENT (empty slot),
 * EHIP.  S = 0 and n_decode = 0 are allowed. */
int lora_plan_create(lora_pool* pool, const int32_t* seg_start, const int32_t* seg_slot, int32_t n_segments,
                     const int32_t* token_slot, int32_t n_decode, void* stream, lora_plan** out);

/* Release a plan's slots.  A later plan may take its ring entry at once: that
 * plan's upload is ordered after the device work of every lora_linear that
 * used the entry (stream order, or a stream wait when the streams differ),
 * without a host wait. */
int lora_plan_destroy(lora_plan* plan);

/* Read back a plan's decode grouping: groups of decode rows sharing a slot.
 * n_groups out; group_slot/group_begin/group_count [n_groups] and rows
 * [n_decode] (row indices, group g = rows[group_begin[g] .. +group_count[g]]).
 * Any array may be NULL.  Group order is the library's scheduling order. */
int lora_plan_groups(const lora_plan* plan, int32_t* n_groups, int32_t* group_slot, int32_t* group_begin,
                     int32_t* group_count, int32_t* rows);

/*
 * One LoRA-linear for projection (layer, proj) over the plan's batch:
 *   w0 != NULL:  y = x W0^T + delta, rounded once to the element type
 *   w0 == NULL:  y += delta only
 * where delta_t = gamma_a B_a^T (A_a x_t) for rows with an adapter and rows
 * without one are not touched by the delta kernels (so they equal base_gemm's
 * output bit for bit).  x [T][d_in], y [T][d_out] with T = the plan's rows.
 * Decode rows run the BGMV shrink/expand kernels, segments the SGMV kernels.
 * Calls sharing a plan must be ordered on one stream (they share the plan's
 * intermediate buffer and the first call uploads its index).  Errors: EINVAL
 * (null x/y, layer/proj out of range, host-only pool), EHIP. */
int lora_linear(lora_pool* pool, const lora_plan* plan, int32_t layer, int32_t proj,
                const void* x, const void* w0, void* y, void* stream);

/*
 * Several projections of one layer that read the same x (q, k, v, gate and
 * up of a transformer layer), in one call: projection projs[i] writes y[i]
 * from w0[i] exactly as lora_linear(pool, plan, layer, projs[i], x, w0[i],
 * y[i], stream) would, bit for bit.  The shrinks of all n projections run in
 * shared launches (their units are independent, and the launches are bound
 * by the latency of each unit's loads, not by the number of units), then each
 * projection's base GEMM (with the prefill rows' expand), then the decode
 * rows' expands of all n in one launch ("Multi-LoRA serving: S-LoRA, Punica
 * and adapter batching", What the engine does each step: per projection, a
 * shrink and an expand around the base product).  Decode batches of up to
 * 64 rows, whose base GEMM and shrink share one launch per projection, run as
 * n single calls.
 *   n       1 .. the pool's max_multi projections; projs [n] host array, every
 *           projection with the same d_in (x [T][d_in] is shared)
 *   w0, y   host arrays [n] of device pointers (w0 all NULL for y += delta;
 *           the y[i] distinct)
 * Errors: as lora_linear, and EINVAL for n outside 1 .. max_multi, unequal
 * d_in, or w0 given for some projections and not others. */
int lora_linear_multi(lora_pool* pool, const lora_plan* plan, int32_t layer, int32_t n, const int32_t* projs,
                      const void* x, const void* const* w0, void* const* y, void* stream);

/* Decode LoRA-linear (BGMV): T decode rows, host token_slot [T] (-1 = none).
 * Same as lora_plan_create(no segments) + lora_linear + lora_plan_destroy. */
int lora_linear_decode(lora_pool* pool, int32_t layer, int32_t proj, const void* x, const void* w0, void* y,
                       const int32_t* token_slot, int32_t T, void* stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): lora_linear_decode with
 * the plan's index, the shrink output v and the fp32 base of the rows with an
 * adapter in a static device scratch array of the library (16 MiB per GPU,
 * held until the process ends) instead of the pool's workspace.  Allocates no
 * device or pinned memory and takes no plan ring entry.  Results equal
 * lora_linear_decode's bit for bit.  The scratch of one GPU is shared by every
 * call on it and keeps the last call's contents (nothing in it needs to start
 * at zero): calls that overlap on one GPU (other streams, other threads) race;
 * order them on one stream.  Errors: EINVAL when T rows x d_out[proj] outputs
 * need more than the scratch holds (with max_rank 64: 973 rows at
 * d_out = 4096, 373 at 11008) or T > max_tokens, otherwise as
 * lora_linear_decode. */
int lora_linear_decode_noalloc(lora_pool* pool, int32_t layer, int32_t proj, const void* x, const void* w0,
                               void* y, const int32_t* token_slot, int32_t T, void* stream);

/* Prefill LoRA-linear (SGMV): segments as in lora_plan_create, rows
 * [0, seg_start[S]).  Same as lora_plan_create + lora_linear + destroy. */
int lora_linear_prefill(lora_pool* pool, int32_t layer, int32_t proj, const void* x, const void* w0, void* y,
                        const int32_t* seg_start, const int32_t* seg_slot, int32_t n_segments, void* stream);

/*
 * The shared base product, one dense GEMM over the whole batch ("Multi-LoRA
 * serving ...", The bottleneck: one dense GEMM reading W once; "S-LoRA:
 * Serving Thousands of Concurrent LoRA Adapters": x W batched across all
 * requests):  y[M][N] = x[M][K] * w0[N][K]^T, fp32 accumulation, output
 * rounded to dtype.  bf16 runs on the matrix cores (MFMA).  Requires
 * K % 8 == 0 (bf16) or K % 4 == 0 (f32) and 16-byte aligned pointers.
 * M = 0 is a no-op.  Errors: EINVAL, EHIP. */
int base_gemm(int32_t dtype, const void* x, const void* w0, void* y, int64_t M, int64_t N, int64_t K,
              void* stream);

/*
 * FP8 base ("Multi-LoRA serving ...", Interaction with how the adapters were
 * trained: a base served quantized, e.g. FP8, with 16-bit adapters).  The
 * base weight is W0[n][k] = w0_scale[n] * e4m3(w0_code[n][k]): w0_code
 * [N][K] bytes, each an 8-bit E4M3 float (1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits, subnormals, no infinities, 0x7F / 0xFF NaN),
 * w0_scale [N] fp32, one per output channel.  x and y are bf16.
 *   y[M][N] = x[M][K] * W0[N][K]^T, fp32 accumulation (the codes are widened
 *   to bf16 exactly and run on the bf16 matrix cores; the scale multiplies
 *   the accumulators), output rounded to bf16 once.
 * Requires N % 4 == 0, K % 128 == 0, 16-byte aligned pointers, M * K * 2 and
 * N * K below 2^31.  M = 0 is a no-op.  Errors: EINVAL, EHIP. */
int base_gemm_fp8(const void* x, const void* w0_code, const float* w0_scale, void* y, int64_t M, int64_t N, int64_t K,
                  void* stream);

/* lora_linear with an FP8 base (bf16 pool): y = x W0^T + delta with W0 as in
 * base_gemm_fp8 (w0_code [d_out][d_in], w0_scale [d_out]); the delta is
 * lora_linear's, computed from bf16 x and the bf16 adapter pages, and rows
 * with an adapter are rounded once.  Errors as lora_linear, and EINVAL when
 * the pool is not bf16 or the shapes break base_gemm_fp8's requirements. */
int lora_linear_fp8(lora_pool* pool, const lora_plan* plan, int32_t layer, int32_t proj, const void* x,
                    const void* w0_code, const float* w0_scale, void* y, void* stream);

/*
 * Engine layer: memory management and scheduling around the pool.
 * ("S-LoRA: Serving Thousands of Concurrent LoRA Adapters", Host memory for
 * adapters: every adapter has a home in host memory, the GPU holds the ones
 * the running batch uses, and the next batch's adapters are predicted from
 * the waiting queue and copied during the current step.  "Multi-LoRA serving
 * ...", What the engine does each step: an adapter missing from the GPU is
 * taken from the host cache, or loaded from storage into it first; the GPU
 * victim is the least recently used adapter that no request is using; a
 * request becomes ready when its adapter's copy is done; a step takes at most
 * max_step_tokens rows and max_distinct_adapters adapters.)
 *
 * Tiers.  Storage is the caller's two callbacks (info: metadata; fill: the
 * blobs).  The host cache is one arena of host_cache_bytes (pinned for a
 * device pool) holding whole adapters, least recently used dropped first;
 * an entry that a running copy still reads is never dropped.  The GPU tier
 * is the pool: eviction candidates are resident adapters with no running
 * request, whose copy is done and that no waiting request in the look-ahead
 * window (below) wants; the least recently used goes first.
 *
 * Requests.  lora_engine_submit queues a request (adapter -1 = the base
 * model alone) of prompt_tokens prompt rows that then generates max_new_tokens
 * tokens: the step that admits it runs its prompt as one prefill segment and
 * makes its first token; each later step gives it one decode row until it has
 * max_new_tokens tokens; then it finishes and lets go of its adapter (and its
 * KV pages, when the engine manages them).  Arrival time and whether its
 * adapter was on the GPU at arrival are recorded.
 *
 * One step (lora_engine_step):
 *   1. copies that have finished are noted (their adapters become ready);
 *   2. look-ahead: the first prefetch_window waiting requests (those waiting
 *      max_wait_steps steps or more first, then arrival order) name the
 *      adapters to bring in; each that is neither resident nor being copied
 *      is loaded into the host cache if missing, given room in the pool by
 *      evicting candidates, and all of them are paged in with one
 *      lora_pool_page_in_batch on copy_stream.  An adapter with no room
 *      (every candidate gone) waits for a later step;
 *   3. admission, in the same order: a request joins if its adapter is
 *      ready (copy done, or still copying when admit_in_flight is 1: the
 *      layers then wait on the device for their own pages), its prompt fits
 *      in the rows left after one decode row per running request, the step's
 *      distinct adapters stay within max_distinct_adapters, the running
 *      requests within max_running, the segments within the pool's
 *      max_segments, and (kv_pages_per_token > 0) its KV pages - (prompt +
 *      max_new) x kv_pages_per_token, taken whole at admission - can be had,
 *      evicting candidates if needed.  A request that has waited
 *      max_wait_steps steps (> 0) and cannot join for room stops admissions
 *      behind it, so finishing requests make room for it: no request starves;
 *   4. the step's plan: the admitted prompts as segments in admission order,
 *      then one decode row per earlier running request, in admission order.
 * The caller runs the step's lora_linear calls with batch.plan and then calls
 * lora_engine_step_done, which destroys the plan and advances the requests.
 * On an error no batch is formed and nothing is admitted; the engine stays
 * usable (a request whose adapter cannot be loaded can be cancelled).
 * Not thread safe; destroy the engine before its pool.
 */
typedef struct lora_engine lora_engine;
/* Adapter metadata from storage: rank, alpha and base id of adapter_id. 0 = ok. */
typedef int (*lora_adapter_info_fn)(void* user, int32_t adapter_id, int32_t* rank, float* alpha, uint64_t* base_id);
/* Write adapter_id's A and B blobs (layouts of lora_pool_page_in; a_bytes and
 * b_bytes as that call requires) into the host cache buffers.  0 = ok. */
typedef int (*lora_adapter_fill_fn)(void* user, int32_t adapter_id, void* host_A, int64_t a_bytes, void* host_B,
                                    int64_t b_bytes);
typedef struct lora_engine_desc {
    int64_t host_cache_bytes;      /* host tier capacity; must hold one adapter of max_rank */
    int32_t max_step_tokens;       /* rows per step, 1 .. the pool's max_tokens */
    int32_t max_distinct_adapters; /* distinct adapters per step, >= 1 */
    int32_t max_running;           /* admitted, unfinished requests, 1 .. max_step_tokens */
    int32_t prefetch_window;       /* waiting requests looked ahead at, >= 0 */
    int32_t admit_in_flight;       /* 0 or 1, see step 3 */
    int32_t max_wait_steps;        /* starvation bound in steps; 0 = none */
    int32_t kv_pages_per_token;    /* >= 0; 0 = the caller manages KV pages */
    int32_t reserved;              /* 0 */
    lora_adapter_info_fn info;
    lora_adapter_fill_fn fill;
    void* user;                    /* passed to the callbacks */
    void* copy_stream;             /* hipStream_t of the page-ins (NULL = the null stream) */
} lora_engine_desc;
typedef struct lora_engine_batch {
    lora_plan* plan;               /* NULL when the step has no rows */
    int32_t n_requests;            /* prefill requests first, then decode requests */
    int32_t n_prefill;
    int32_t n_rows;                /* rows of the plan */
    int32_t n_distinct;            /* distinct adapters (-1 not counted) */
} lora_engine_batch;
typedef struct lora_engine_stats {
    int64_t steps, rows, admitted, finished, waiting, running, cancelled;
    int64_t arrivals_resident, arrivals_missing; /* GPU tier at arrival (resident or copying = resident) */
    int64_t host_hits, host_misses;              /* per page-in: in the host cache / loaded from storage */
    int64_t page_ins, page_in_bytes, gpu_evictions, host_evictions;
    int64_t room_stalls;                         /* adapters left for a later step: no room in the pool */
    int64_t kv_stalls;                           /* admissions deferred for KV pages */
    double page_in_ms_p50, page_in_ms_p99, page_in_ms_max; /* issue to copy done, GPU clock, per adapter */
    double copy_ms_p50, copy_ms_p99;             /* a page-in batch on the copy stream, start to done */
    double wait_ms_hit_p50, wait_ms_hit_p99;     /* submit to admission, host clock: resident at arrival */
    double wait_ms_miss_p50, wait_ms_miss_p99;   /* ... not resident at arrival */
    double wait_steps_p99, wait_steps_max;       /* submit to admission, in steps */
    double storage_ms_p50, storage_ms_p99;       /* one storage load (fill), host clock */
} lora_engine_stats;
/* Errors: EINVAL (NULL callbacks, a limit outside its range, a host cache
 * too small for one adapter of max_rank), EHIP (host cache allocation). */
int lora_engine_create(lora_pool* pool, const lora_engine_desc* desc, lora_engine** out);
/* Waits for the engine's copies, releases its requests' adapters and KV
 * pages, frees the host cache; resident adapters stay in the pool. */
int lora_engine_destroy(lora_engine* engine);
/* Queue a request.  The adapter's metadata is read (info) on its first use
 * and checked: EINVAL (prompt_tokens outside 1..max_step_tokens,
 * max_new_tokens < 1, request_id already queued or running, rank outside the
 * pool's range, info failed), EBASE (made for another base model: "Multi-LoRA
 * serving ...", Failure modes: silent wrong base). */
int lora_engine_submit(lora_engine* engine, int64_t request_id, int32_t adapter_id, int32_t prompt_tokens,
                       int32_t max_new_tokens);
/* Remove a waiting request (ENOTRESIDENT if it is not waiting). */
int lora_engine_cancel(lora_engine* engine, int64_t request_id);
/* One step (see above).  stream: where the plan's calls run.  EBUSY while the
 * previous step is not done; a failed fill (EINVAL), page-in or plan error as
 * those calls return it. */
int lora_engine_step(lora_engine* engine, void* stream, lora_engine_batch* out);
/* The current step's requests in row order: ids, adapters, rows (prompt
 * length or 1) [n_requests]; any array may be NULL. */
int lora_engine_batch_requests(const lora_engine* engine, int64_t* request_ids, int32_t* adapter_ids,
                               int32_t* n_rows);
/* The step's calls are enqueued: destroy its plan, give every request of the
 * step its token, finish requests that have all their tokens. */
int lora_engine_step_done(lora_engine* engine);
/* KV pages the engine holds for a request (n_out = their number; pages may be
 * NULL; at most cap written).  ENOTRESIDENT if the request is not running. */
int lora_engine_kv_pages(const lora_engine* engine, int64_t request_id, int32_t cap, int32_t* pages, int32_t* n_out);
/* Counters since creation or the last reset (copies in flight are noted first). */
int lora_engine_get_stats(lora_engine* engine, lora_engine_stats* out);
int lora_engine_reset_stats(lora_engine* engine);

/* Per-kernel timing for measurement.  With enable = k > 0, the kernels of
 * every k-th lora_linear / lora_linear_* call on this pool (the first call
 * after this one, then every k-th) and every page-in kernel are bracketed by
 * two HIP events recorded on the launch stream (k > 1 keeps the events' own
 * host cost out of most calls); enable = 0 turns timing off.
 * lora_pool_timing synchronises those events and returns, for kernel class
 * `kernel` (LORA_K_*), the summed elapsed milliseconds and the number of timed
 * launches since timing was last set.  Setting it again resets the counters.
 * Errors: EINVAL (enable < 0, or a host-only pool). */
enum { LORA_K_GEMM = 0, LORA_K_BGMV_SHRINK = 1, LORA_K_BGMV_EXPAND = 2, LORA_K_SGMV_SHRINK = 3,
       LORA_K_SGMV_EXPAND = 4, LORA_K_PAGE_IN = 5,
       LORA_K_GEMM_BGMV_SHRINK = 6, /* decode batches: base GEMM and BGMV shrink in one launch */
       LORA_K_PAGE_IN_BATCH = 7,    /* a whole page-in call: first copy to last page written */
       LORA_K_COUNT = 8 };
int lora_pool_set_timing(lora_pool* pool, int32_t enable);
int lora_pool_timing(lora_pool* pool, int32_t kernel, double* total_ms, int64_t* launches);

/* Measurement probe: `blocks` workgroups of 4 waves each run iters x 8
 * independent bf16 matrix operations of shape 16x16x32 (shape 16) or
 * 32x32x16 (shape 32) on register data and write one checksum per wave to out
 * (device, [4 * blocks] floats).  *flops (may be NULL) receives the launch's
 * flop count; time the launch on `stream` to get the sustained matrix-core
 * rate.  EINVAL for another shape, iters or blocks < 1. */
int lora_probe_mfma(int32_t shape, int64_t iters, int32_t blocks, float* out, void* stream, double* flops);

/* Measurement probe: the rate at which HBM serves the delta kernels' access
 * shape (one adapter row of 8 KiB in its page per wave).  Wave w reads the
 * 8 KiB chunk chunk[w] of buf, i.e. bytes [8192 chunk[w], 8192 chunk[w] +
 * 8192), all of its loads in flight at once; chunk indices outside the buffer's
 * whole chunks are clamped into it.  buf: device, buf_bytes long; chunk:
 * device int64 [n_chunks]; out: device float [n_chunks], written only when a
 * checksum takes one fixed value (it keeps the loads).  Time the launch on
 * `stream`.  EINVAL for buf_bytes < 8192, n_chunks < 1 or a NULL pointer. */
int lora_probe_read(const void* buf, int64_t buf_bytes, const int64_t* chunk, int32_t n_chunks, float* out,
                    void* stream);

/* Message of the calling thread's last error ("" if none). */
const char* lora_last_error(void);

/* Library version string. */
const char* lora_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LORA_GEMM_H */
