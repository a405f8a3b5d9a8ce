// Host side of the LoRA-linear library: the unified page pool (free list,
// slot and page tables, reference counts, KV blocks), per-step batch plans,
// index uploads through a pinned staging ring, and the C ABI that launches
// the gfx950 kernels.  See include/lora_gemm.h for the contract of every
// entry point.
//
// Allocation follows "S-LoRA: Serving Thousands of Concurrent LoRA Adapters"
// (Unified paging: one pool of fixed-size pages, one hidden-size vector per
// page, shared by adapters of any rank and by KV blocks).  Readings of what
// the pages leave open: the free list starts as the caller's physical page
// order and is popped from the front, freed pages go to its tail in list
// order; an adapter's pages are taken in the order layer, projection, A
// before B, rank-row, chunk, all at once or none; a page-in takes the lowest
// free slot.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "internal.h"
#include "lora_gemm.h"

using namespace hagemm;

// Static device scratch of lora_linear_decode_noalloc: the plan index, v and
// the fp32 base of the rows with an adapter, for callers that cannot
// allocate.  Each GPU holds its own copy at its own address until the process
// ends; host code reaches it only through the address hipGetSymbolAddress
// gives for the current device (the array's name in host code is a host-side
// stand-in, not a device address).  Every call on a GPU shares that GPU's
// copy: calls that overlap on one GPU race.
static constexpr int64_t kScratchBytes = int64_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

#define HIP_TRY(expr)                                                                    \
    do {                                                                                 \
        hipError_t e_ = (expr);                                                          \
        if (e_ != hipSuccess) return fail(LORA_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

int ilog2_exact(int64_t v) {
    if (v <= 0 || (v & (v - 1))) return -1;
    int s = 0;
    while ((int64_t(1) << s) < v) ++s;
    return s;
}

enum PageOwner : uint8_t { kFree = 0, kAdapter = 1, kKV = 2, kFreeing = 3 /* inside lora_pool_free_kv only */ };

// staging buffers of page-table uploads (one per adapter of a page-in): a buffer is reused
// only after its upload has run, so a page-in batch of up to kStages adapters enqueues with no
// host wait even when its stream still waits for earlier work
constexpr int kStages = 64;
constexpr int kPlanStages = 8;   // staging buffers of plan uploads (at most kPlanRing in live plans)

struct SlotState {
    int32_t adapter = -1;
    int32_t rank = 0;
    float alpha = 0.f;
    int32_t refs = 0;
    std::vector<int32_t> pages;        // allocation order
    bool copy_pending = false;         // page-in enqueued, completion not yet observed
    int32_t evset = -1;                // per-layer copy events (shared by the adapters of one page-in batch)
    uint64_t stage_gen[kPlanStages] = {};  // per plan stage: its gen at the last plan that read the slot
};

struct StageBuf {
    void* host = nullptr;
    void* host_dev = nullptr;     // its device mapping (read by the upload kernel)
    hipEvent_t ev = nullptr;
    bool recorded = false;
};

// Staging buffer of one plan's index upload.  Its event is recorded once, when
// the plan is destroyed, on the stream of the plan's last call: it then covers
// the upload and every kernel of the plan.  gen counts the buffer's plans; a
// buffer is reused only after a host wait on its event, so a (buffer, gen)
// pair whose gen is no longer current names finished work.
struct PlanStage {
    void* host = nullptr;
    void* host_dev = nullptr;     // its device mapping (read by the upload kernel)
    hipEvent_t ev = nullptr;
    bool recorded = false;
    bool live = false;            // its plan is not destroyed yet
    uint64_t gen = 0;
};

struct RingEntry {
    bool live = false;            // owned by a plan
    int last_stage = -1;          // plan stage of the entry's last destroyed plan
    uint64_t last_gen = 0;
    hipStream_t stream = nullptr; // stream that plan's event was recorded on
};

}  // namespace

struct lora_pool {
    int32_t dtype = 0;
    int32_t page_elems = 0;
    int32_t page_shift = 0;
    int32_t elem_bytes = 0;
    int64_t num_pages = 0;
    void* pages_dev = nullptr;
    void* meta_dev = nullptr;
    void* stage_dev = nullptr;     // optional device staging area of page-ins (caller-owned)
    int64_t stage_bytes = 0;
    int32_t n_layers = 0, n_proj = 0;
    std::vector<int32_t> d_in, d_out, nci, nco;
    std::vector<int32_t> lp_prefix;   // (l * n_proj + p) -> offset per unit rank
    int32_t pages_per_rank = 0;       // over all (layer, proj)
    int32_t pages_per_rank_layer = 0; // one layer
    int32_t max_slots = 0, max_rank = 0, max_tokens = 0, max_segments = 0;
    int32_t max_multi = 1;            // projections one lora_linear_multi call takes
    uint64_t base_id = 0;
    bool host_only = false;
    int32_t slot_cap = 0;
    PlanLayout pl{};
    int64_t ring_off = 0;

    std::deque<int32_t> free_list;
    std::vector<uint8_t> owner;
    std::vector<SlotState> slots;
    std::unordered_map<int32_t, int32_t> adapter_slot;
    int32_t resident = 0;
    int64_t kv_pages = 0;

    RingEntry ring[kPlanRing];
    StageBuf stage[kStages];
    int stage_next = 0;
    PlanStage pstage[kPlanStages];
    int pstage_next = 0;
    std::vector<int32_t> words;        // host image of a plan entry's index words
    size_t stage_cap = 0;

    // measurement: event pairs around each launch, per kernel class, on every
    // timing_period-th lora_linear call (0 = off) and every page-in launch
    int32_t timing_period = 0;
    int64_t linear_calls = 0;
    bool timing = false;
    std::vector<std::pair<int, std::pair<hipEvent_t, hipEvent_t>>> timed;
    std::vector<hipEvent_t> spare_events;

    // per-layer events of page-in batches; a set is reused once no slot refers to it
    struct EvSet { std::vector<hipEvent_t> ev; int32_t refs = 0; };
    std::vector<EvSet> evsets;
    std::vector<int32_t> free_evsets;
};

struct lora_plan {
    lora_pool* pool = nullptr;
    int entry = -1;                  // plan ring entry in the pool's workspace, or -1
    bool scratch = false;            // index, v and ybase in the library's static scratch array
    hagemm::PlanLayout L{};          // layout of the index words and buffers at dev
    uint8_t* dev = nullptr;          // device base of the index words, v and ybase
    int32_t T_pre = 0, T_dec = 0;
    int32_t n_groups = 0, n_su = 0, n_eu = 0, n_segs = 0, n_tiles = 0;
    std::vector<int32_t> g_slot, g_begin, g_count, rows;
    int stage = -1;                  // plan staging buffer (device pools)
    int64_t words = 0;               // index words to upload
    mutable bool uploaded = false;   // the index is in the plan's ring entry
    mutable hipStream_t stream = nullptr;  // creation stream, then the stream of the last lora_linear
    std::vector<int32_t> acquired;   // distinct slots, one reference each
    std::vector<int32_t> pending;    // slots whose page-in may still be copying
};

namespace hagemm {

PlanLayout plan_layout(int32_t max_tokens, int32_t max_segments, int32_t max_rank, int32_t max_dout,
                       int32_t max_multi) {
    PlanLayout L{};
    L.multi = std::max(1, max_multi);
    L.cap_groups = max_tokens;
    // (a group of c rows and rank r has ceil(r / 4) * ceil(c / 4) <= c * ceil(r / 4) units)
    L.cap_su = max_tokens * ((max_rank + kShrinkRowsPerUnit - 1) / kShrinkRowsPerUnit);
    L.cap_eu = max_tokens;
    L.cap_segs = max_segments;
    L.cap_tiles = (max_tokens + kSegTileRows - 1) / kSegTileRows + max_segments;
    L.vstride = (int32_t)align_up(max_rank, 16);
    int64_t w = 0;
    auto take = [&](int64_t n) { int64_t o = w; w += align_up(n, 4); return o; };
    L.g_slot = take(L.cap_groups);
    L.g_rank = take(L.cap_groups);
    L.g_begin = take(L.cap_groups);
    L.g_count = take(L.cap_groups);
    L.g_gamma = take(L.cap_groups);
    L.rows = take(max_tokens);
    L.s_slot = take(L.cap_segs);
    L.s_rank = take(L.cap_segs);
    L.s_gamma = take(L.cap_segs);
    L.s_begin = take(L.cap_segs);
    L.s_end = take(L.cap_segs);
    L.t_seg = take(L.cap_tiles);
    L.t_row0 = take(L.cap_tiles);
    L.row_slot = take(max_tokens);
    L.eu = take(12 * (int64_t)L.cap_eu);
    L.su = take(8 * (int64_t)L.cap_su);   // last: an upload stops after the used units
    L.words = w;
    L.v_bytes_off = align_up(w * 4, 256);
    L.v_pstride = align_up((int64_t)max_tokens * L.vstride, 64);
    L.vpart_bytes_off = align_up(L.v_bytes_off + L.multi * L.v_pstride * 4, 256);
    L.vpart_rows = max_segments > 0 ? max_tokens : 0;
    L.vpart_pstride = align_up((int64_t)kMaxShrinkSplit * L.vpart_rows * L.vstride, 64);
    L.ybase_bytes_off = align_up(L.vpart_bytes_off + L.multi * L.vpart_pstride * 4, 256);
    L.ybase_pstride = align_up((int64_t)max_tokens * max_dout, 64);
    L.entry_bytes = align_up(L.ybase_bytes_off + L.multi * L.ybase_pstride * 4, 256);
    return L;
}

}  // namespace hagemm

namespace {

int check_desc(const lora_pool_desc* d) {
    if (!d) return fail(LORA_EINVAL, "desc is NULL");
    if (d->dtype != LORA_F32 && d->dtype != LORA_BF16) return fail(LORA_EINVAL, "dtype must be LORA_F32 or LORA_BF16");
    const int vec = d->dtype == LORA_BF16 ? 8 : 4;
    const int min_page = d->dtype == LORA_BF16 ? 512 : 256;
    if (d->page_elems < min_page || ilog2_exact(d->page_elems) < 0)
        return fail(LORA_EINVAL, "page_elems must be a power of two >= %d", min_page);
    if (d->num_pages < 1 || d->num_pages > INT32_MAX) return fail(LORA_EINVAL, "num_pages out of range");
    if (d->n_layers < 1 || d->n_proj < 1 || d->n_proj > kMaxProj) return fail(LORA_EINVAL, "n_layers/n_proj out of range");
    if (!d->d_in || !d->d_out) return fail(LORA_EINVAL, "d_in/d_out are NULL");
    for (int p = 0; p < d->n_proj; ++p)
        if (d->d_in[p] < vec || d->d_out[p] < vec || d->d_in[p] % vec || d->d_out[p] % vec)
            return fail(LORA_EINVAL, "projection %d: widths must be positive multiples of %d", p, vec);
    if (d->max_slots < 1 || d->max_rank < 1 || d->max_rank > kMaxRank)
        return fail(LORA_EINVAL, "max_slots must be >= 1 and max_rank in 1..%d", kMaxRank);
    // (rows of a group are packed above the rank-row in a shrink unit's word: < 2^22)
    if (d->max_tokens < 1 || d->max_tokens > (1 << 22) || d->max_segments < 0)
        return fail(LORA_EINVAL, "max_tokens/max_segments out of range");
    if (d->max_multi < 0 || d->max_multi > kMaxMulti)
        return fail(LORA_EINVAL, "max_multi must be 0 .. %d", kMaxMulti);
    if ((d->pages_dev == nullptr) != (d->meta_dev == nullptr))
        return fail(LORA_EINVAL, "pages_dev and meta_dev must both be set (device pool) or both NULL (host-only pool)");
    if (d->stage_dev) {
        if (!d->pages_dev) return fail(LORA_EINVAL, "a host-only pool takes no staging area");
        if ((uintptr_t)d->stage_dev % 256) return fail(LORA_EINVAL, "stage_dev must be 256-byte aligned");
        int64_t per_rank = 0;
        for (int p = 0; p < d->n_proj; ++p) per_rank += d->d_in[p] + d->d_out[p];
        const int64_t need = per_rank * d->max_rank * (d->dtype == LORA_BF16 ? 2 : 4);
        if (d->stage_bytes < need)
            return fail(LORA_EINVAL, "stage_bytes %lld < %lld (one layer of one adapter of max_rank)",
                        (long long)d->stage_bytes, (long long)need);
    } else if (d->stage_bytes != 0) {
        return fail(LORA_EINVAL, "stage_bytes without stage_dev");
    }
    return LORA_OK;
}

struct Geometry {
    std::vector<int32_t> nci, nco, lp_prefix;
    int64_t per_rank = 0, per_rank_layer = 0, slot_cap = 0;
};

Geometry geometry(const lora_pool_desc* d) {
    Geometry g;
    const int64_t P = d->page_elems;
    for (int p = 0; p < d->n_proj; ++p) {
        g.nci.push_back((int32_t)((d->d_in[p] + P - 1) / P));
        g.nco.push_back((int32_t)((d->d_out[p] + P - 1) / P));
        g.per_rank_layer += g.nci.back() + g.nco.back();
    }
    int64_t off = 0;
    for (int l = 0; l < d->n_layers; ++l)
        for (int p = 0; p < d->n_proj; ++p) {
            g.lp_prefix.push_back((int32_t)off);
            off += g.nci[p] + g.nco[p];
        }
    g.per_rank = off;
    g.slot_cap = off * d->max_rank;
    return g;
}

int32_t max_dout(const lora_pool_desc* d) {
    int32_t m = 0;
    for (int p = 0; p < d->n_proj; ++p) m = std::max(m, d->d_out[p]);
    return m;
}

int64_t table_bytes(const lora_pool_desc* d, const Geometry& g) {
    return align_up((int64_t)d->max_slots * g.slot_cap * 4, 256);
}

int acquire_stage(lora_pool* p, size_t bytes, StageBuf** out) {
    if (bytes > p->stage_cap) return fail(LORA_EINVAL, "upload of %zu bytes exceeds the staging buffer", bytes);
    StageBuf& s = p->stage[p->stage_next];
    p->stage_next = (p->stage_next + 1) % kStages;
    if (s.recorded) {
        HIP_TRY(hipEventSynchronize(s.ev));
        s.recorded = false;
    }
    *out = &s;
    return LORA_OK;
}

int upload(lora_pool* p, void* dst_dev, const void* src, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return LORA_OK;
    StageBuf* s = nullptr;
    int rc = acquire_stage(p, bytes, &s);
    if (rc) return rc;
    std::memcpy(s->host, src, bytes);
    HIP_TRY(launch_upload(s->host_dev, dst_dev, (int64_t)(bytes / 4), stream));
    HIP_TRY(hipEventRecord(s->ev, stream));
    s->recorded = true;
    return LORA_OK;
}

int32_t* tab_dev(lora_pool* p) { return reinterpret_cast<int32_t*>(p->meta_dev); }

// the static scratch array's device address, per device (see `scratch` above)
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the scratch array's device address on the current device (resolved once per device)
int scratch_on_current_device(uint8_t** out) {
    int dev = -1;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(LORA_EINVAL, "device %d beyond the %d the library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
        if (!ptr) return fail(LORA_EHIP, "hipGetSymbolAddress gave no address for the scratch array");
        g_scratch_ptr[dev] = ptr;
    }
    *out = static_cast<uint8_t*>(g_scratch_ptr[dev]);
    return LORA_OK;
}

uint8_t* entry_dev(lora_pool* p, int e) {
    return reinterpret_cast<uint8_t*>(p->meta_dev) + p->ring_off + (int64_t)e * p->pl.entry_bytes;
}

hipEvent_t layer_event(lora_pool* p, int32_t slot, int32_t layer) {
    return p->evsets[p->slots[slot].evset].ev[layer];
}

void release_evset(lora_pool* p, SlotState& s) {
    if (s.evset < 0) return;
    if (--p->evsets[s.evset].refs == 0) p->free_evsets.push_back(s.evset);
    s.evset = -1;
}

// Make sure nothing still reads the slot's pages or table on the device.
int quiesce_slot(lora_pool* p, int32_t slot) {
    if (p->host_only) return LORA_OK;
    SlotState& s = p->slots[slot];
    if (s.evset >= 0 && s.copy_pending) {
        HIP_TRY(hipEventSynchronize(layer_event(p, slot, p->n_layers - 1)));
        s.copy_pending = false;
    }
    // plans that read the slot: the slot is released only by destroyed plans
    for (int k = 0; k < kPlanStages; ++k) {
        PlanStage& ps = p->pstage[k];
        if (ps.recorded && s.stage_gen[k] == ps.gen) {
            HIP_TRY(hipEventSynchronize(ps.ev));
            ps.recorded = false;
        }
    }
    return LORA_OK;
}

hipEvent_t take_event(lora_pool* p) {
    if (!p->spare_events.empty()) {
        hipEvent_t e = p->spare_events.back();
        p->spare_events.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Launch `launch` on `st`, bracketed by timing events when measurement is on.
template <typename F>
hipError_t timed_launch(lora_pool* p, int kind, hipStream_t st, F&& launch) {
    if (!p->timing) return launch();
    hipEvent_t a = take_event(p), b = take_event(p);
    if (!a || !b) return hipErrorOutOfMemory;
    hipError_t e = hipEventRecord(a, st);
    if (e == hipSuccess) e = launch();
    if (e == hipSuccess) e = hipEventRecord(b, st);
    p->timed.push_back({kind, {a, b}});
    return e;
}

int check_pinned(const void* ptr, int64_t bytes, const void** dev) {
    hipPointerAttribute_t at;
    std::memset(&at, 0, sizeof at);
    hipError_t e = hipPointerGetAttributes(&at, ptr);
    if (e != hipSuccess || at.type != hipMemoryTypeHost) {
        (void)hipGetLastError();
        return fail(LORA_EINVAL, "host buffer %p is not pinned host memory (allocate it with hipHostMalloc / pin_memory)", ptr);
    }
    const void* last = static_cast<const uint8_t*>(ptr) + (bytes - 1);
    std::memset(&at, 0, sizeof at);
    e = hipPointerGetAttributes(&at, last);
    if (e != hipSuccess || at.type != hipMemoryTypeHost) {
        (void)hipGetLastError();
        return fail(LORA_EINVAL, "host buffer %p: its last byte is not in pinned host memory", ptr);
    }
    void* d = nullptr;
    e = hipHostGetDevicePointer(&d, const_cast<void*>(ptr), 0);
    if (e != hipSuccess || d == nullptr) {
        (void)hipGetLastError();
        return fail(LORA_EINVAL, "host buffer %p has no device mapping", ptr);
    }
    *dev = d;
    return LORA_OK;
}

}  // namespace

extern "C" {

const char* lora_last_error(void) { return g_err.c_str(); }

const char* lora_version(void) { return "hagemm 0.1 gfx950"; }

int lora_pool_meta_bytes(const lora_pool_desc* desc, int64_t* out_bytes) {
    int rc = check_desc(desc);
    if (rc) return rc;
    if (!out_bytes) return fail(LORA_EINVAL, "out_bytes is NULL");
    Geometry g = geometry(desc);
    if ((int64_t)desc->max_slots * g.slot_cap >= INT32_MAX) return fail(LORA_EINVAL, "page table too large for int32 indexing");
    PlanLayout pl = plan_layout(desc->max_tokens, desc->max_segments, desc->max_rank, max_dout(desc), desc->max_multi);
    *out_bytes = table_bytes(desc, g) + (int64_t)kPlanRing * pl.entry_bytes;
    return LORA_OK;
}

int lora_pool_create(const lora_pool_desc* d, lora_pool** out) {
    int rc = check_desc(d);
    if (rc) return rc;
    if (!out) return fail(LORA_EINVAL, "out is NULL");
    Geometry g = geometry(d);
    if ((int64_t)d->max_slots * g.slot_cap >= INT32_MAX) return fail(LORA_EINVAL, "page table too large for int32 indexing");
    PlanLayout pl = plan_layout(d->max_tokens, d->max_segments, d->max_rank, max_dout(d), d->max_multi);
    const int64_t need = table_bytes(d, g) + (int64_t)kPlanRing * pl.entry_bytes;
    const bool host_only = d->meta_dev == nullptr;
    if (!host_only && d->meta_bytes < need)
        return fail(LORA_EINVAL, "meta_bytes %lld < required %lld", (long long)d->meta_bytes, (long long)need);
    if (!host_only && ((uintptr_t)d->meta_dev % 256 || (uintptr_t)d->pages_dev % 16))
        return fail(LORA_EINVAL, "meta_dev must be 256-byte aligned and pages_dev 16-byte aligned");
    // free order must be a permutation
    std::vector<int32_t> order(d->num_pages);
    if (d->free_order) {
        std::vector<uint8_t> seen(d->num_pages, 0);
        for (int64_t i = 0; i < d->num_pages; ++i) {
            int32_t q = d->free_order[i];
            if (q < 0 || q >= d->num_pages || seen[q]) return fail(LORA_EINVAL, "free_order is not a permutation of the pages");
            seen[q] = 1;
            order[i] = q;
        }
    } else {
        for (int64_t i = 0; i < d->num_pages; ++i) order[i] = (int32_t)i;
    }
    auto* p = new lora_pool();
    p->dtype = d->dtype;
    p->page_elems = d->page_elems;
    p->page_shift = ilog2_exact(d->page_elems);
    p->elem_bytes = d->dtype == LORA_BF16 ? 2 : 4;
    p->num_pages = d->num_pages;
    p->pages_dev = d->pages_dev;
    p->meta_dev = d->meta_dev;
    p->stage_dev = d->stage_dev;
    p->stage_bytes = d->stage_bytes;
    p->n_layers = d->n_layers;
    p->n_proj = d->n_proj;
    p->d_in.assign(d->d_in, d->d_in + d->n_proj);
    p->d_out.assign(d->d_out, d->d_out + d->n_proj);
    p->nci = g.nci;
    p->nco = g.nco;
    p->lp_prefix = g.lp_prefix;
    p->pages_per_rank = (int32_t)g.per_rank;
    p->pages_per_rank_layer = (int32_t)g.per_rank_layer;
    p->max_slots = d->max_slots;
    p->max_rank = d->max_rank;
    p->max_tokens = d->max_tokens;
    p->max_segments = d->max_segments;
    p->base_id = d->base_id;
    p->max_multi = std::max(1, d->max_multi);
    p->host_only = host_only;
    p->slot_cap = (int32_t)g.slot_cap;
    p->pl = pl;
    p->ring_off = table_bytes(d, g);
    p->free_list.assign(order.begin(), order.end());
    p->owner.assign(d->num_pages, kFree);
    p->slots.resize(d->max_slots);
    if (!host_only) {
        p->stage_cap = (size_t)g.slot_cap * 4;
        hipError_t e = hipSuccess;
        for (auto& s : p->stage) {
            if (e == hipSuccess) e = hipHostMalloc(&s.host, p->stage_cap, hipHostMallocDefault);
            if (e == hipSuccess) e = hipHostGetDevicePointer(&s.host_dev, s.host, 0);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming);
        }
        for (auto& s : p->pstage) {
            if (e == hipSuccess) e = hipHostMalloc(&s.host, (size_t)pl.words * 4, hipHostMallocDefault);
            if (e == hipSuccess) e = hipHostGetDevicePointer(&s.host_dev, s.host, 0);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming);
        }
        // unused table words read as -1 (no page); a synchronous fill at creation
        if (e == hipSuccess) e = hipMemset(p->meta_dev, 0xFF, (size_t)p->ring_off);
        if (e != hipSuccess) {
            int code = fail(LORA_EHIP, "pool setup: %s", hipGetErrorString(e));
            lora_pool_destroy(p);
            return code;
        }
    }
    *out = p;
    return LORA_OK;
}

int lora_pool_destroy(lora_pool* p) {
    if (!p) return fail(LORA_EINVAL, "pool is NULL");
    for (auto& s : p->stage) {
        if (s.ev) {
            if (s.recorded) (void)hipEventSynchronize(s.ev);
            (void)hipEventDestroy(s.ev);
        }
        if (s.host) (void)hipHostFree(s.host);
    }
    for (auto& s : p->pstage) {
        if (s.ev) {
            if (s.recorded) (void)hipEventSynchronize(s.ev);
            (void)hipEventDestroy(s.ev);
        }
        if (s.host) (void)hipHostFree(s.host);
    }
    for (auto& es : p->evsets)
        for (hipEvent_t e : es.ev) {
            (void)hipEventSynchronize(e);
            (void)hipEventDestroy(e);
        }
    for (auto& t : p->timed) {
        (void)hipEventSynchronize(t.second.second);
        (void)hipEventDestroy(t.second.first);
        (void)hipEventDestroy(t.second.second);
    }
    for (hipEvent_t e : p->spare_events) (void)hipEventDestroy(e);
    delete p;
    return LORA_OK;
}

int lora_pool_set_timing(lora_pool* p, int32_t enable) {
    if (!p) return fail(LORA_EINVAL, "pool is NULL");
    if (p->host_only && enable) return fail(LORA_EINVAL, "host-only pool: nothing to time");
    if (enable < 0) return fail(LORA_EINVAL, "timing period %d < 0", enable);
    for (auto& t : p->timed) {
        HIP_TRY(hipEventSynchronize(t.second.second));
        p->spare_events.push_back(t.second.first);
        p->spare_events.push_back(t.second.second);
    }
    p->timed.clear();
    p->timing_period = enable;
    p->linear_calls = 0;
    p->timing = enable != 0;
    return LORA_OK;
}

int lora_pool_timing(lora_pool* p, int32_t kernel, double* total_ms, int64_t* launches) {
    if (!p || kernel < 0 || kernel >= LORA_K_COUNT) return fail(LORA_EINVAL, "bad arguments");
    double ms = 0.0;
    int64_t n = 0;
    for (auto& t : p->timed) {
        if (t.first != kernel) continue;
        HIP_TRY(hipEventSynchronize(t.second.second));
        float f = 0.f;
        HIP_TRY(hipEventElapsedTime(&f, t.second.first, t.second.second));
        ms += f;
        ++n;
    }
    if (total_ms) *total_ms = ms;
    if (launches) *launches = n;
    return LORA_OK;
}

int lora_pool_page_in_batch(lora_pool* p, int32_t n, const lora_page_in_req* reqs, void* stream, int32_t* out_slots) {
    if (!p) return fail(LORA_EINVAL, "pool is NULL");
    if (n < 0 || (n > 0 && !reqs)) return fail(LORA_EINVAL, "bad request array");
    if (n == 0) return LORA_OK;
    // checks, in the order of the single-adapter call, request by request
    std::vector<const void*> dA(n, nullptr), dB(n, nullptr);
    for (int32_t k = 0; k < n; ++k) {
        const lora_page_in_req& r = reqs[k];
        if (r.adapter_id < 0) return fail(LORA_EINVAL, "request %d: adapter_id must be >= 0", k);
        if (r.rank < 1 || r.rank > p->max_rank) return fail(LORA_EINVAL, "request %d: rank %d outside 1..%d", k, r.rank, p->max_rank);
        if (!std::isfinite(r.alpha)) return fail(LORA_EINVAL, "request %d: alpha is not finite", k);
        int64_t a_elems = 0, b_elems = 0;
        for (int q = 0; q < p->n_proj; ++q) {
            a_elems += (int64_t)p->n_layers * r.rank * p->d_in[q];
            b_elems += (int64_t)p->n_layers * r.rank * p->d_out[q];
        }
        if (!p->host_only || r.host_A || r.host_B) {
            if (!r.host_A || !r.host_B) return fail(LORA_EINVAL, "request %d: host_A/host_B are NULL", k);
            if (r.host_A_bytes != a_elems * p->elem_bytes || r.host_B_bytes != b_elems * p->elem_bytes)
                return fail(LORA_EINVAL, "request %d: host sizes %lld/%lld, expected %lld/%lld bytes", k,
                            (long long)r.host_A_bytes, (long long)r.host_B_bytes, (long long)(a_elems * p->elem_bytes),
                            (long long)(b_elems * p->elem_bytes));
            if (!p->host_only) {
                int rc = check_pinned(r.host_A, r.host_A_bytes, &dA[k]);
                if (rc) return rc;
                rc = check_pinned(r.host_B, r.host_B_bytes, &dB[k]);
                if (rc) return rc;
            }
        }
    }
    for (int32_t k = 0; k < n; ++k)
        if (reqs[k].base_id != p->base_id)
            return fail(LORA_EBASE, "adapter %d was made for base %llu, the pool serves %llu", reqs[k].adapter_id,
                        (unsigned long long)reqs[k].base_id, (unsigned long long)p->base_id);
    for (int32_t k = 0; k < n; ++k) {
        if (p->adapter_slot.count(reqs[k].adapter_id))
            return fail(LORA_EEXIST, "adapter %d already resident", reqs[k].adapter_id);
        for (int32_t j = 0; j < k; ++j)
            if (reqs[j].adapter_id == reqs[k].adapter_id)
                return fail(LORA_EEXIST, "adapter %d requested twice", reqs[k].adapter_id);
    }
    // slots and pages as n single calls in order would take them: lowest free
    // slots, pages from the front of the free list
    std::vector<int32_t> slot(n);
    for (int32_t k = 0, s = 0; k < n; ++k, ++s) {
        while (s < p->max_slots && p->slots[s].adapter >= 0) ++s;
        if (s >= p->max_slots) return fail(LORA_ENOSLOT, "all %d slots taken", p->max_slots);
        slot[k] = s;
    }
    std::vector<int64_t> first(n + 1, 0);
    for (int32_t k = 0; k < n; ++k) {
        first[k + 1] = first[k] + (int64_t)reqs[k].rank * p->pages_per_rank;
        if (first[k + 1] > (int64_t)p->free_list.size())
            return fail(LORA_ENOPAGES, "adapter %d needs %lld pages, %lld free", reqs[k].adapter_id,
                        (long long)(first[k + 1] - first[k]), (long long)((int64_t)p->free_list.size() - first[k]));
    }
    if (!p->host_only) {
        hipStream_t st = static_cast<hipStream_t>(stream);
        // per-layer events shared by the batch
        int32_t es = -1;
        if (!p->free_evsets.empty()) {
            es = p->free_evsets.back();
            p->free_evsets.pop_back();
        } else {
            lora_pool::EvSet set;
            set.ev.assign(p->n_layers, nullptr);
            for (auto& ev : set.ev) {
                hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
                if (e != hipSuccess) {
                    for (hipEvent_t x : set.ev)
                        if (x) (void)hipEventDestroy(x);
                    return fail(LORA_EHIP, "page-in events: %s", hipGetErrorString(e));
                }
            }
            es = (int32_t)p->evsets.size();
            p->evsets.push_back(std::move(set));
        }
        auto give_back = [&] { if (p->evsets[es].refs == 0) p->free_evsets.push_back(es); };
        for (int32_t k = 0; k < n; ++k) {
            std::vector<int32_t> pages(p->free_list.begin() + first[k], p->free_list.begin() + first[k + 1]);
            int rc = upload(p, tab_dev(p) + (int64_t)slot[k] * p->slot_cap, pages.data(), pages.size() * 4, st);
            if (rc) {
                give_back();
                return rc;
            }
        }
        int64_t ia = 0, ib = 0;
        for (int q = 0; q < p->n_proj; ++q) {
            ia += p->d_in[q];
            ib += p->d_out[q];
        }
        p->timing = p->timing_period > 0;
        // layers l .. l + nl - 1 of up to kPageInBatch adapters, rows read from src_A / src_B
        // (device-visible) whose layer l0 starts at element 0; max_blocks as for launch_page_in
        auto scatter = [&](int32_t l, int32_t nl, int32_t l0, int32_t k0, int32_t nk,
                           const std::vector<const void*>& src_A, const std::vector<const void*>& src_B,
                           int max_blocks) -> hipError_t {
            PageInArgs a{};
            a.pages = p->pages_dev;
            a.page_shift = p->page_shift;
            a.n_proj = p->n_proj;
            a.n_adapters = nk;
            a.n_layers = nl;
            for (int q = 0; q < p->n_proj; ++q) {
                a.d_in[q] = p->d_in[q];
                a.d_out[q] = p->d_out[q];
                a.nci[q] = p->nci[q];
                a.nco[q] = p->nco[q];
            }
            a.block0[0] = 0;
            for (int32_t i = 0; i < nk; ++i) {
                const int32_t k = k0 + i, rank = reqs[k].rank;
                a.host_A[i] = src_A[k];
                a.host_B[i] = src_B[k];
                a.tab[i] = tab_dev(p) + (int64_t)slot[k] * p->slot_cap;
                a.rank[i] = rank;
                a.first_page[i] = rank * p->lp_prefix[(int64_t)l * p->n_proj];
                a.a_layer_off[i] = (int64_t)(l - l0) * rank * ia;
                a.b_layer_off[i] = (int64_t)(l - l0) * rank * ib;
                a.block0[i + 1] = a.block0[i] + nl * rank * p->pages_per_rank_layer;
            }
            return timed_launch(p, LORA_K_PAGE_IN, st, [&] { return launch_page_in(p->dtype, a, max_blocks, st); });
        };
        hipError_t e = hipSuccess;
        hipEvent_t span0 = nullptr, span1 = nullptr;
        if (p->timing) {
            span0 = take_event(p);
            span1 = take_event(p);
            if (!span0 || !span1 || (e = hipEventRecord(span0, st)) != hipSuccess) {
                give_back();
                return fail(LORA_EHIP, "page-in timing events");
            }
        }
        if (!p->stage_dev) {
            // layer by layer, so that layer l of every adapter is in before layer l + 1 of any
            for (int32_t l = 0; l < p->n_layers && e == hipSuccess; ++l) {
                for (int32_t k0 = 0; k0 < n && e == hipSuccess; k0 += kPageInBatch)
                    e = scatter(l, 1, 0, k0, std::min(kPageInBatch, n - k0), dA, dB, kPageInBlocksPcie);
                if (e == hipSuccess) e = hipEventRecord(p->evsets[es].ev[l], st);
            }
        } else {
            // through the staging area, a few layers at a time: the copy engine brings
            // kStageChunkLayers layers (fewer if the largest adapter's would not fit) of a group
            // of adapters (as many as the staging area holds, at most kPageInBatch) into the
            // staging area and one kernel scatters those layers into the pages; the staging
            // area is reused after the scatter (stream order).  Each layer's event follows its
            // chunk's scatters, so a layer's first call waits for its chunk only.
            const int64_t eb = p->elem_bytes;
            int64_t row_max = 0;
            for (int32_t k = 0; k < n; ++k) row_max = std::max(row_max, (int64_t)reqs[k].rank * (ia + ib) * eb);
            std::vector<const void*> sA(n), sB(n);
            for (int32_t l0 = 0; l0 < p->n_layers && e == hipSuccess;) {
                int32_t cl = std::min(kStageChunkLayers, p->n_layers - l0);
                while (cl > 1 && cl * row_max > p->stage_bytes) --cl;
                const int32_t l1 = l0 + cl;
                for (int32_t k0 = 0; k0 < n && e == hipSuccess;) {
                    // the adapters [k0, k1) whose layers [l0, l1) fit the staging area together
                    int32_t k1 = k0;
                    int64_t off = 0;
                    while (k1 < n && k1 - k0 < kPageInBatch && e == hipSuccess) {
                        const int64_t la = (int64_t)reqs[k1].rank * ia * eb, lb = (int64_t)reqs[k1].rank * ib * eb;
                        if (off + cl * (la + lb) > p->stage_bytes && k1 > k0) break;
                        uint8_t* dst = static_cast<uint8_t*>(p->stage_dev) + off;
                        const uint8_t* hA = static_cast<const uint8_t*>(reqs[k1].host_A) + (int64_t)l0 * la;
                        const uint8_t* hB = static_cast<const uint8_t*>(reqs[k1].host_B) + (int64_t)l0 * lb;
                        e = hipMemcpyAsync(dst, hA, cl * la, hipMemcpyHostToDevice, st);
                        if (e == hipSuccess) e = hipMemcpyAsync(dst + cl * la, hB, cl * lb, hipMemcpyHostToDevice, st);
                        sA[k1] = dst;
                        sB[k1] = dst + cl * la;
                        off += align_up(cl * (la + lb), 256);
                        ++k1;
                    }
                    if (e == hipSuccess) e = scatter(l0, cl, l0, k0, k1 - k0, sA, sB, kPageInBlocksStaged);
                    k0 = k1;
                }
                for (int32_t l = l0; l < l1 && e == hipSuccess; ++l) e = hipEventRecord(p->evsets[es].ev[l], st);
                l0 = l1;
            }
        }
        if (e == hipSuccess && span1) {
            e = hipEventRecord(span1, st);
            p->timed.push_back({LORA_K_PAGE_IN_BATCH, {span0, span1}});
        }
        if (e != hipSuccess) {
            give_back();
            return fail(LORA_EHIP, "page-in: %s", hipGetErrorString(e));
        }
        for (int32_t k = 0; k < n; ++k) {
            SlotState& s = p->slots[slot[k]];
            release_evset(p, s);
            s.evset = es;
            s.copy_pending = true;
            p->evsets[es].refs++;
        }
    }
    for (int32_t k = 0; k < n; ++k) {
        SlotState& s = p->slots[slot[k]];
        const int64_t need = first[k + 1] - first[k];
        s.pages.resize(need);
        for (int64_t i = 0; i < need; ++i) {
            s.pages[i] = p->free_list.front();
            p->free_list.pop_front();
            p->owner[s.pages[i]] = kAdapter;
        }
        s.adapter = reqs[k].adapter_id;
        s.rank = reqs[k].rank;
        s.alpha = reqs[k].alpha;
        s.refs = 0;
        p->adapter_slot[reqs[k].adapter_id] = slot[k];
        p->resident++;
        if (out_slots) out_slots[k] = slot[k];
    }
    return LORA_OK;
}

int lora_pool_page_in(lora_pool* p, int32_t adapter_id, int32_t rank, float alpha, uint64_t base_id,
                      const void* host_A, int64_t host_A_bytes, const void* host_B, int64_t host_B_bytes,
                      void* stream, int32_t* out_slot) {
    const lora_page_in_req r{adapter_id, rank, alpha, 0, base_id, host_A, host_A_bytes, host_B, host_B_bytes};
    return lora_pool_page_in_batch(p, 1, &r, stream, out_slot);
}

int lora_pool_evict(lora_pool* p, int32_t adapter_id) {
    if (!p) return fail(LORA_EINVAL, "pool is NULL");
    auto it = p->adapter_slot.find(adapter_id);
    if (it == p->adapter_slot.end()) return fail(LORA_ENOTRESIDENT, "adapter %d not resident", adapter_id);
    const int32_t slot = it->second;
    SlotState& s = p->slots[slot];
    if (s.refs > 0) return fail(LORA_EBUSY, "adapter %d is in use (%d references)", adapter_id, s.refs);
    int rc = quiesce_slot(p, slot);
    if (rc) return rc;
    for (int32_t q : s.pages) {
        p->free_list.push_back(q);
        p->owner[q] = kFree;
    }
    s.pages.clear();
    s.adapter = -1;
    s.rank = 0;
    s.alpha = 0.f;
    release_evset(p, s);
    p->adapter_slot.erase(it);
    p->resident--;
    return LORA_OK;
}

int lora_pool_slot_of(const lora_pool* p, int32_t adapter_id, int32_t* out_slot) {
    if (!p || !out_slot) return fail(LORA_EINVAL, "NULL argument");
    auto it = p->adapter_slot.find(adapter_id);
    if (it == p->adapter_slot.end()) return fail(LORA_ENOTRESIDENT, "adapter %d not resident", adapter_id);
    *out_slot = it->second;
    return LORA_OK;
}

int lora_pool_slots_of(const lora_pool* p, int32_t n, const int32_t* ids, int32_t* out) {
    if (!p || n < 0 || (n > 0 && (!ids || !out))) return fail(LORA_EINVAL, "bad arguments");
    for (int32_t i = 0; i < n; ++i)
        if (ids[i] >= 0 && !p->adapter_slot.count(ids[i]))
            return fail(LORA_ENOTRESIDENT, "adapter %d (entry %d) not resident", ids[i], i);
    for (int32_t i = 0; i < n; ++i) out[i] = ids[i] < 0 ? -1 : p->adapter_slot.at(ids[i]);
    return LORA_OK;
}

int lora_pool_acquire(lora_pool* p, int32_t slot) {
    if (!p || slot < 0 || slot >= p->max_slots) return fail(LORA_EINVAL, "slot out of range");
    if (p->slots[slot].adapter < 0) return fail(LORA_ENOTRESIDENT, "slot %d is empty", slot);
    p->slots[slot].refs++;
    return LORA_OK;
}

int lora_pool_release(lora_pool* p, int32_t slot) {
    if (!p || slot < 0 || slot >= p->max_slots) return fail(LORA_EINVAL, "slot out of range");
    if (p->slots[slot].adapter < 0 || p->slots[slot].refs == 0) return fail(LORA_EINVAL, "slot %d not acquired", slot);
    p->slots[slot].refs--;
    return LORA_OK;
}

int lora_pool_alloc_kv(lora_pool* p, int32_t n, int32_t* out_pages) {
    if (!p || n < 0 || (n > 0 && !out_pages)) return fail(LORA_EINVAL, "bad arguments");
    if ((size_t)n > p->free_list.size()) return fail(LORA_ENOPAGES, "%d KV pages asked, %zu free", n, p->free_list.size());
    for (int32_t i = 0; i < n; ++i) {
        int32_t q = p->free_list.front();
        p->free_list.pop_front();
        p->owner[q] = kKV;
        out_pages[i] = q;
    }
    p->kv_pages += n;
    return LORA_OK;
}

int lora_pool_free_kv(lora_pool* p, int32_t n, const int32_t* pages) {
    if (!p || n < 0 || (n > 0 && !pages)) return fail(LORA_EINVAL, "bad arguments");
    // mark each page on the way (a page seen twice finds its mark); on an error
    // the marks are taken back, so the pool is unchanged
    for (int32_t i = 0; i < n; ++i) {
        const int32_t q = pages[i];
        const bool bad = q < 0 || q >= p->num_pages || p->owner[q] != kKV;
        if (bad) {
            const bool twice = q >= 0 && q < p->num_pages && p->owner[q] == kFreeing;
            for (int32_t j = 0; j < i; ++j) p->owner[pages[j]] = kKV;
            return twice ? fail(LORA_EINVAL, "KV page %d is listed twice", q)
                         : fail(LORA_EINVAL, "page %d is not a KV page", q);
        }
        p->owner[q] = kFreeing;
    }
    for (int32_t i = 0; i < n; ++i) {
        p->owner[pages[i]] = kFree;
        p->free_list.push_back(pages[i]);
    }
    p->kv_pages -= n;
    return LORA_OK;
}

int lora_pool_page_table(const lora_pool* p, int32_t slot, int32_t layer, int32_t proj, int32_t* a_pages,
                         int32_t* b_pages) {
    if (!p || slot < 0 || slot >= p->max_slots || layer < 0 || layer >= p->n_layers || proj < 0 || proj >= p->n_proj)
        return fail(LORA_EINVAL, "index out of range");
    const SlotState& s = p->slots[slot];
    if (s.adapter < 0) return fail(LORA_ENOTRESIDENT, "slot %d is empty", slot);
    const int64_t base = (int64_t)s.rank * p->lp_prefix[(int64_t)layer * p->n_proj + proj];
    const int64_t na = (int64_t)s.rank * p->nci[proj], nb = (int64_t)s.rank * p->nco[proj];
    if (a_pages) std::memcpy(a_pages, s.pages.data() + base, na * 4);
    if (b_pages) std::memcpy(b_pages, s.pages.data() + base + na, nb * 4);
    return LORA_OK;
}

int lora_pool_stats(const lora_pool* p, int64_t* free_pages, int32_t* resident, int64_t* kv_pages) {
    if (!p) return fail(LORA_EINVAL, "pool is NULL");
    if (free_pages) *free_pages = (int64_t)p->free_list.size();
    if (resident) *resident = p->resident;
    if (kv_pages) *kv_pages = p->kv_pages;
    return LORA_OK;
}

int lora_pool_free_list(const lora_pool* p, int64_t cap, int32_t* out, int64_t* n_out) {
    if (!p || !n_out || cap < 0 || (cap > 0 && !out)) return fail(LORA_EINVAL, "bad arguments");
    const int64_t n = (int64_t)p->free_list.size();
    if (out) {
        if (cap < n) return fail(LORA_EINVAL, "capacity %lld < %lld free pages", (long long)cap, (long long)n);
        std::copy(p->free_list.begin(), p->free_list.end(), out);
    }
    *n_out = n;
    return LORA_OK;
}

int lora_pool_slot_info(const lora_pool* p, int32_t slot, int32_t* rank, float* alpha, int32_t* adapter_id) {
    if (!p || slot < 0 || slot >= p->max_slots) return fail(LORA_EINVAL, "slot out of range");
    const SlotState& s = p->slots[slot];
    if (s.adapter < 0) return fail(LORA_ENOTRESIDENT, "slot %d is empty", slot);
    if (rank) *rank = s.rank;
    if (alpha) *alpha = s.alpha;
    if (adapter_id) *adapter_id = s.adapter;
    return LORA_OK;
}

}  // extern "C"

namespace hagemm {

int set_error(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int64_t pool_pages_for_rank(const lora_pool* p, int32_t rank) { return (int64_t)rank * p->pages_per_rank; }

PoolInfo pool_info(const lora_pool* p) {
    PoolInfo i{};
    i.host_only = p->host_only;
    i.elem_bytes = p->elem_bytes;
    i.n_layers = p->n_layers;
    i.n_proj = p->n_proj;
    i.max_slots = p->max_slots;
    i.max_rank = p->max_rank;
    i.max_tokens = p->max_tokens;
    i.max_segments = p->max_segments;
    for (int q = 0; q < p->n_proj; ++q) {
        i.a_elems_per_rank += (int64_t)p->n_layers * p->d_in[q];
        i.b_elems_per_rank += (int64_t)p->n_layers * p->d_out[q];
    }
    i.base_id = p->base_id;
    return i;
}

int pool_copy_done(lora_pool* p, int32_t slot, bool* done) {
    if (slot < 0 || slot >= p->max_slots || p->slots[slot].adapter < 0) return fail(LORA_ENOTRESIDENT, "slot %d is empty", slot);
    SlotState& s = p->slots[slot];
    if (p->host_only || !s.copy_pending || s.evset < 0) {
        *done = true;
        return LORA_OK;
    }
    const hipError_t q = hipEventQuery(layer_event(p, slot, p->n_layers - 1));
    if (q == hipSuccess) {
        s.copy_pending = false;
        *done = true;
    } else if (q == hipErrorNotReady) {
        *done = false;
    } else {
        return fail(LORA_EHIP, "page-in event: %s", hipGetErrorString(q));
    }
    return LORA_OK;
}

}  // namespace hagemm

namespace {

// Build a plan whose index words follow layout L.  scratch_dev == NULL: the
// plan takes a ring entry of the pool's workspace (layout p->pl); otherwise
// its index, v and ybase live at scratch_dev.
int plan_create_impl(lora_pool* p, const int32_t* seg_start, const int32_t* seg_slot, int32_t S,
                     const int32_t* token_slot, int32_t n_decode, void* stream, const PlanLayout& L,
                     uint8_t* scratch_dev, lora_plan** out) {
    if (!p || !out) return fail(LORA_EINVAL, "NULL argument");
    if (S < 0 || S > p->max_segments) return fail(LORA_EINVAL, "%d segments, the pool allows %d", S, p->max_segments);
    if (n_decode < 0) return fail(LORA_EINVAL, "n_decode < 0");
    if (S > 0 && (!seg_start || !seg_slot)) return fail(LORA_EINVAL, "seg_start/seg_slot are NULL");
    if (n_decode > 0 && !token_slot) return fail(LORA_EINVAL, "token_slot is NULL");
    int64_t T_pre = 0;
    if (S > 0) {
        if (seg_start[0] != 0) return fail(LORA_EINVAL, "seg_start[0] must be 0");
        for (int32_t s = 0; s < S; ++s)
            if (seg_start[s + 1] < seg_start[s]) return fail(LORA_EINVAL, "seg_start decreases at %d", s);
        T_pre = seg_start[S];
    }
    if (T_pre + n_decode > p->max_tokens)
        return fail(LORA_EINVAL, "%lld rows, the pool allows %d", (long long)(T_pre + n_decode), p->max_tokens);
    auto check_slot = [&](int32_t s, const char* what, int32_t i) -> int {
        if (s < -1 || s >= p->max_slots) return fail(LORA_EINVAL, "%s %d: slot %d out of range", what, i, s);
        if (s >= 0 && p->slots[s].adapter < 0) return fail(LORA_ENOTRESIDENT, "%s %d: slot %d is empty", what, i, s);
        return LORA_OK;
    };
    for (int32_t s = 0; s < S; ++s) {
        int rc = check_slot(seg_slot[s], "segment", s);
        if (rc) return rc;
    }
    for (int32_t t = 0; t < n_decode; ++t) {
        int rc = check_slot(token_slot[t], "decode row", t);
        if (rc) return rc;
    }
    // a free ring entry (plans in the static scratch take none)
    int entry = -1;
    if (!p->host_only && !scratch_dev) {
        for (int e = 0; e < kPlanRing; ++e)
            if (!p->ring[e].live) { entry = e; break; }
        if (entry < 0) return fail(LORA_EBUSY, "all %d plan entries are live; destroy a plan first", kPlanRing);
    }
    auto* plan = new lora_plan();
    plan->pool = p;
    plan->entry = entry;
    plan->scratch = scratch_dev != nullptr;
    plan->L = L;
    plan->dev = scratch_dev ? scratch_dev : (entry >= 0 ? entry_dev(p, entry) : nullptr);
    plan->T_pre = (int32_t)T_pre;
    plan->T_dec = n_decode;
    std::vector<int32_t>& words = p->words;   // host image of the entry; only used parts are written
    if (!p->host_only && (int64_t)words.size() < L.words) words.resize(L.words, 0);
    auto W = [&](int64_t off, int64_t i) -> int32_t& { return words[off + i]; };
    auto put_f = [&](int64_t off, int64_t i, float f) { std::memcpy(&words[off + i], &f, 4); };

    // decode rows grouped by slot, rows ascending within a group (stable)
    std::vector<int32_t> idx;
    idx.reserve(n_decode);
    for (int32_t t = 0; t < n_decode; ++t)
        if (token_slot[t] >= 0) idx.push_back(t);
    std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) { return token_slot[a] < token_slot[b]; });
    struct Grp { int32_t slot, rank, count, first; };   // rows idx[first .. first + count)
    std::vector<Grp> groups;
    for (int32_t i = 0; i < (int32_t)idx.size(); ++i) {
        const int32_t s = token_slot[idx[i]];
        if (groups.empty() || groups.back().slot != s) groups.push_back({s, p->slots[s].rank, 0, i});
        groups.back().count++;
    }
    // scheduling order: heavier groups first (rank, then rows), slot as tie-break
    std::stable_sort(groups.begin(), groups.end(), [](const Grp& a, const Grp& b) {
        if (a.rank != b.rank) return a.rank > b.rank;
        if (a.count != b.count) return a.count > b.count;
        return a.slot < b.slot;
    });
    int32_t pos = 0;
    plan->g_slot.reserve(groups.size());
    plan->g_begin.reserve(groups.size());
    plan->g_count.reserve(groups.size());
    plan->rows.reserve(idx.size());
    for (size_t g = 0; g < groups.size(); ++g) {
        const Grp& G = groups[g];
        plan->g_slot.push_back(G.slot);
        plan->g_begin.push_back(pos);
        plan->g_count.push_back(G.count);
        for (int32_t i = 0; i < G.count; ++i) plan->rows.push_back((int32_t)T_pre + idx[G.first + i]);
        if (!p->host_only) {
            W(L.g_slot, g) = G.slot;
            W(L.g_rank, g) = G.rank;
            W(L.g_begin, g) = pos;
            W(L.g_count, g) = G.count;
            put_f(L.g_gamma, g, p->slots[G.slot].alpha / (float)G.rank);
            for (int32_t i = 0; i < G.count; ++i) W(L.rows, pos + i) = plan->rows[pos + i];
        }
        pos += G.count;
    }
    plan->n_groups = (int32_t)groups.size();
    // shrink units (group, 4 rank-rows, up to kShrinkTokensPerUnit of the group's
    // rows): groups with more rows first (stable in the scheduling order), a
    // group's units in rank-row, then row order.  Expand units (group, up to
    // kExpandTokensPerUnit of its rows), in the scheduling order.  Heavy groups are split by rows, so one adapter
    // shared by many rows does not serialise on a few workgroups.
    std::vector<int32_t> by_rows(groups.size());
    for (size_t g = 0; g < groups.size(); ++g) by_rows[g] = (int32_t)g;
    std::stable_sort(by_rows.begin(), by_rows.end(), [&](int32_t a, int32_t b) { return groups[a].count > groups[b].count; });
    int32_t n_su = 0;
    for (int32_t g : by_rows)
        for (int32_t j0 = 0; j0 < groups[g].rank; j0 += kShrinkRowsPerUnit)
            for (int32_t t0 = 0; t0 < groups[g].count; t0 += kShrinkTokensPerUnit) {
                if (!p->host_only) {
                    const int32_t nt = std::min(kShrinkTokensPerUnit, groups[g].count - t0);
                    const int64_t o = 8 * (int64_t)n_su;
                    W(L.su, o) = g;
                    W(L.su, o + 1) = j0 | (t0 << 8);
                    W(L.su, o + 2) = groups[g].slot;
                    W(L.su, o + 3) = groups[g].rank | (nt << 8);
                    for (int32_t t = 0; t < kShrinkTokensPerUnit; ++t)
                        W(L.su, o + 4 + t) = plan->rows[plan->g_begin[g] + t0 + std::min(t, nt - 1)];
                }
                ++n_su;
            }
    plan->n_su = n_su;
    // expand units: resolved (slot, rank | rows << 8, gamma; the unit's rows) and by group
    // (group, first row of the group)
    int32_t n_eu = 0;
    for (size_t g = 0; g < groups.size(); ++g)
        for (int32_t t0 = 0; t0 < groups[g].count; t0 += kExpandTokensPerUnit) {
            if (!p->host_only) {
                const int32_t nt = std::min(kExpandTokensPerUnit, groups[g].count - t0);
                const int64_t o = 12 * (int64_t)n_eu;
                W(L.eu, o) = groups[g].slot;
                W(L.eu, o + 1) = groups[g].rank | (nt << 8);
                put_f(L.eu, o + 2, p->slots[groups[g].slot].alpha / (float)groups[g].rank);
                W(L.eu, o + 3) = (int32_t)g;
                for (int32_t t = 0; t < kExpandTokensPerUnit; ++t)
                    W(L.eu, o + 4 + t) = plan->rows[plan->g_begin[g] + t0 + std::min(t, nt - 1)];
                W(L.eu, o + 8) = t0;
                W(L.eu, o + 9) = 0;
                W(L.eu, o + 10) = 0;
                W(L.eu, o + 11) = 0;
            }
            ++n_eu;
        }
    plan->n_eu = n_eu;
    // segments with an adapter, split into row tiles (higher rank first)
    struct Seg { int32_t slot, rank, begin, end; };
    std::vector<Seg> segs;
    for (int32_t s = 0; s < S; ++s)
        if (seg_slot[s] >= 0 && seg_start[s + 1] > seg_start[s])
            segs.push_back({seg_slot[s], p->slots[seg_slot[s]].rank, seg_start[s], seg_start[s + 1]});
    std::vector<std::pair<int32_t, int32_t>> tiles;
    for (int32_t s = 0; s < (int32_t)segs.size(); ++s)
        for (int32_t r0 = segs[s].begin; r0 < segs[s].end; r0 += kSegTileRows) tiles.push_back({s, r0});
    std::stable_sort(tiles.begin(), tiles.end(), [&](const std::pair<int32_t, int32_t>& a, const std::pair<int32_t, int32_t>& b) {
        return segs[a.first].rank > segs[b.first].rank;
    });
    plan->n_segs = (int32_t)segs.size();
    plan->n_tiles = (int32_t)tiles.size();
    if (!p->host_only) {
        for (size_t s = 0; s < segs.size(); ++s) {
            W(L.s_slot, s) = segs[s].slot;
            W(L.s_rank, s) = segs[s].rank;
            put_f(L.s_gamma, s, p->slots[segs[s].slot].alpha / (float)segs[s].rank);
            W(L.s_begin, s) = segs[s].begin;
            W(L.s_end, s) = segs[s].end;
        }
        for (size_t t = 0; t < tiles.size(); ++t) {
            W(L.t_seg, t) = tiles[t].first;
            W(L.t_row0, t) = tiles[t].second;
        }
        for (int64_t t = 0; t < T_pre + n_decode; ++t) W(L.row_slot, t) = -1;
        for (const Seg& sg : segs)
            for (int32_t t = sg.begin; t < sg.end; ++t) W(L.row_slot, t) = sg.slot;
        for (int32_t t = 0; t < n_decode; ++t) W(L.row_slot, T_pre + t) = token_slot[t];
    }
    // distinct slots: one reference each for the plan's lifetime
    std::vector<int32_t> distinct;
    for (const Grp& G : groups) distinct.push_back(G.slot);
    for (const Seg& s : segs) distinct.push_back(s.slot);
    std::sort(distinct.begin(), distinct.end());
    distinct.erase(std::unique(distinct.begin(), distinct.end()), distinct.end());
    if (!p->host_only) {
        hipStream_t st = static_cast<hipStream_t>(stream);
        int rc = LORA_OK;
        // a staging buffer whose plan is destroyed; the host waits only for the
        // work of the plan that used it kPlanStages plans ago (at most kPlanRing live)
        int k = -1;
        for (int i = 0; i < kPlanStages && k < 0; ++i) {
            const int c = (p->pstage_next + i) % kPlanStages;
            if (!p->pstage[c].live) k = c;
        }
        PlanStage& ps = p->pstage[k];
        if (ps.recorded) {
            hipError_t e = hipEventSynchronize(ps.ev);
            if (e != hipSuccess) rc = fail(LORA_EHIP, "plan staging wait: %s", hipGetErrorString(e));
        }
        for (int32_t s : distinct) {
            SlotState& ss = p->slots[s];
            if (rc == LORA_OK && ss.copy_pending) {
                hipError_t q = hipEventQuery(layer_event(p, s, p->n_layers - 1));
                if (q == hipSuccess) ss.copy_pending = false;
                else if (q == hipErrorNotReady) plan->pending.push_back(s);
                else rc = fail(LORA_EHIP, "page-in event: %s", hipGetErrorString(q));
            }
        }
        if (rc == LORA_OK) {
            // the index goes to the device with the plan's first call (uploaded before its
            // kernels, or read from this buffer and stored by its first launch)
            ps.recorded = false;
            ps.gen++;
            plan->words = L.su + 8 * (int64_t)n_su;
            std::memcpy(ps.host, words.data(), (size_t)plan->words * 4);
        }
        if (rc) {
            delete plan;
            return rc;
        }
        p->pstage_next = (k + 1) % kPlanStages;
        ps.live = true;
        plan->stage = k;
        plan->stream = st;
        if (entry >= 0) p->ring[entry].live = true;
        for (int32_t s : distinct) p->slots[s].stage_gen[k] = ps.gen;
    }
    for (int32_t s : distinct) p->slots[s].refs++;
    plan->acquired = std::move(distinct);
    *out = plan;
    return LORA_OK;
}

}  // namespace

extern "C" {

int lora_plan_create(lora_pool* p, const int32_t* seg_start, const int32_t* seg_slot, int32_t S,
                     const int32_t* token_slot, int32_t n_decode, void* stream, lora_plan** out) {
    if (!p) return fail(LORA_EINVAL, "NULL argument");
    return plan_create_impl(p, seg_start, seg_slot, S, token_slot, n_decode, stream, p->pl, nullptr, out);
}

int lora_plan_destroy(lora_plan* plan) {
    if (!plan) return fail(LORA_EINVAL, "plan is NULL");
    lora_pool* p = plan->pool;
    int rc = LORA_OK;
    if (plan->stage >= 0) {
        // one event per plan, after its upload and all of its kernels
        PlanStage& ps = p->pstage[plan->stage];
        hipError_t e = hipEventRecord(ps.ev, plan->stream);
        if (e != hipSuccess) {
            (void)hipStreamSynchronize(plan->stream);
            rc = fail(LORA_EHIP, "plan event: %s", hipGetErrorString(e));
        }
        ps.recorded = e == hipSuccess;
        ps.live = false;
        if (plan->entry >= 0) {
            RingEntry& E = p->ring[plan->entry];
            E.live = false;
            E.last_stage = plan->stage;
            E.last_gen = ps.gen;
            E.stream = plan->stream;
        }
    }
    for (int32_t s : plan->acquired) p->slots[s].refs--;
    delete plan;
    return rc;
}

int lora_plan_groups(const lora_plan* plan, int32_t* n_groups, int32_t* group_slot, int32_t* group_begin,
                     int32_t* group_count, int32_t* rows) {
    if (!plan) return fail(LORA_EINVAL, "plan is NULL");
    if (n_groups) *n_groups = plan->n_groups;
    if (group_slot) std::copy(plan->g_slot.begin(), plan->g_slot.end(), group_slot);
    if (group_begin) std::copy(plan->g_begin.begin(), plan->g_begin.end(), group_begin);
    if (group_count) std::copy(plan->g_count.begin(), plan->g_count.end(), group_count);
    if (rows) std::copy(plan->rows.begin(), plan->rows.end(), rows);
    return LORA_OK;
}

}  // extern "C"

namespace {

// One LoRA-linear over the plan's batch.  w0_scale == NULL: w0 is the pool's element type;
// otherwise w0 holds E4M3 codes [d_out][d_in] with w0_scale [d_out] (the FP8 base; bf16 pool).
// n projections of one layer that share x (n = 1: one lora_linear call): their shrinks run in
// shared launches, then each projection's base GEMM and expand
int linear_impl(lora_pool* p, const lora_plan* plan, int32_t layer, int32_t n, const int32_t* projs, const void* x,
                const void* const* w0s, const float* w0_scale, void* const* ys, void* stream) {
    if (!p || !plan || plan->pool != p) return fail(LORA_EINVAL, "plan does not belong to this pool");
    if (p->host_only) return fail(LORA_EINVAL, "host-only pool: no device work");
    if (n < 1 || !projs || !w0s || !ys) return fail(LORA_EINVAL, "no projections");
    if (n > 1 && (n > p->max_multi || n > plan->L.multi))
        return fail(LORA_EINVAL, "%d projections in one call; the pool takes at most %d", n,
                    std::min(p->max_multi, plan->L.multi));
    if (n > 1 && w0_scale) return fail(LORA_EINVAL, "the FP8 base takes one projection per call");
    const int32_t proj = projs[0];
    const void* w0 = w0s[0];
    void* y = ys[0];
    if (layer < 0 || layer >= p->n_layers) return fail(LORA_EINVAL, "layer/proj out of range");
    for (int32_t i = 0; i < n; ++i) {
        if (projs[i] < 0 || projs[i] >= p->n_proj) return fail(LORA_EINVAL, "layer/proj out of range");
        if (p->d_in[projs[i]] != p->d_in[proj]) return fail(LORA_EINVAL, "the projections of one call share x: equal d_in");
        if ((w0s[i] == nullptr) != (w0 == nullptr)) return fail(LORA_EINVAL, "w0 must be given for all projections or none");
    }
    const int32_t T = plan->T_pre + plan->T_dec;
    if (T == 0) return LORA_OK;
    if (!x) return fail(LORA_EINVAL, "x/y are NULL");
    for (int32_t i = 0; i < n; ++i) {
        if (!ys[i]) return fail(LORA_EINVAL, "x/y are NULL");
        if ((uintptr_t)x % 16 || (uintptr_t)ys[i] % 16 || (uintptr_t)w0s[i] % 16)
            return fail(LORA_EINVAL, "x, y, w0 must be 16-byte aligned");
    }
    // decode batches of up to 64 rows run the base GEMM and the BGMV shrink in one launch per
    // projection: there the call is n single calls
    if (n > 1 && w0 && plan->n_tiles == 0 && gemm_shrink_fits(p->dtype, T, plan->n_su)) {
        for (int32_t i = 0; i < n; ++i) {
            const int rc = linear_impl(p, plan, layer, 1, projs + i, x, w0s + i, nullptr, ys + i, stream);
            if (rc) return rc;
        }
        return LORA_OK;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    p->timing = p->timing_period > 0 && p->linear_calls++ % p->timing_period == 0;
    const bool first = !plan->uploaded;
    if (first && plan->entry >= 0) {
        // the entry's earlier device work is ordered before this plan's index reaches it
        // (same stream: stream order; else a stream wait), not by a host wait
        const RingEntry& E = p->ring[plan->entry];
        if (E.last_stage >= 0 && E.stream != st) {
            const PlanStage& last = p->pstage[E.last_stage];
            if (last.gen == E.last_gen && last.recorded) HIP_TRY(hipStreamWaitEvent(st, last.ev, 0));
        }
    }
    // one wait per distinct event (the adapters of one page-in batch share theirs)
    hipEvent_t waited = nullptr;
    for (int32_t s : plan->pending) {
        hipEvent_t ev = layer_event(p, s, layer);
        if (ev != waited) HIP_TRY(hipStreamWaitEvent(st, ev, 0));
        waited = ev;
    }
    const PlanLayout& L = plan->L;
    uint8_t* base = plan->dev;
    auto I = [&](int64_t off) { return reinterpret_cast<const int32_t*>(base) + off; };
    LoraArgs a{};
    a.x = x;
    a.y = y;
    a.pages = p->pages_dev;
    a.page_tab = tab_dev(p);
    a.v = reinterpret_cast<float*>(base + L.v_bytes_off);
    a.g_slot = I(L.g_slot);
    a.g_rank = I(L.g_rank);
    a.g_begin = I(L.g_begin);
    a.g_count = I(L.g_count);
    a.g_gamma = reinterpret_cast<const float*>(I(L.g_gamma));
    a.rows = I(L.rows);
    a.su = I(L.su);
    a.eu = I(L.eu);
    a.s_slot = I(L.s_slot);
    a.s_rank = I(L.s_rank);
    a.s_gamma = reinterpret_cast<const float*>(I(L.s_gamma));
    a.s_begin = I(L.s_begin);
    a.s_end = I(L.s_end);
    a.t_seg = I(L.t_seg);
    a.t_row0 = I(L.t_row0);
    a.vpart = reinterpret_cast<float*>(base + L.vpart_bytes_off);
    a.vpart_rows = L.vpart_rows;
    a.n_groups = plan->n_groups;
    a.n_su = plan->n_su;
    a.n_eu = plan->n_eu;
    a.n_segs = plan->n_segs;
    a.n_tiles = plan->n_tiles;
    a.d_in = p->d_in[proj];
    a.d_out = p->d_out[proj];
    a.page_shift = p->page_shift;
    a.slot_cap = p->slot_cap;
    a.lp_per_rank = p->lp_prefix[(int64_t)layer * p->n_proj + proj];
    a.nci = p->nci[proj];
    a.nco = p->nco[proj];
    a.vstride = L.vstride;
    a.T = T;
    a.T_pre = plan->T_pre;
    if (n > 1) {
        a.n_multi = n;
        a.eblk_multi[0] = 0;
        for (int32_t i = 0; i < n; ++i) {
            const int32_t pi = projs[i];
            a.lp_multi[i] = p->lp_prefix[(int64_t)layer * p->n_proj + pi];
            a.dout_multi[i] = p->d_out[pi];
            a.nco_multi[i] = p->nco[pi];
            a.y_multi[i] = ys[i];
            a.eblk_multi[i + 1] = a.eblk_multi[i] + plan->n_eu * bgmv_expand_chunks(p->dtype, p->d_out[pi]);
        }
        a.v_pstride = L.v_pstride;
        a.vpart_pstride = L.vpart_pstride;
        a.ybase_pstride = L.ybase_pstride;
    }
    hipError_t e = hipSuccess;
    const int dt = p->dtype;
    const bool fp8 = w0_scale != nullptr;
    if (fp8 && (dt != LORA_BF16 || !gemm_w8_ok(T, a.d_out, a.d_in) || (uintptr_t)w0_scale % 16))
        return fail(LORA_EINVAL, "FP8 base: needs a bf16 pool, d_in a multiple of 128, d_out of 4, a 16-byte aligned "
                                 "scale and 32-bit byte offsets");
    const bool any = plan->n_groups > 0 || plan->n_tiles > 0;
    float* ybase = any ? reinterpret_cast<float*>(base + L.ybase_bytes_off) : nullptr;
    const int32_t* rs = any ? I(L.row_slot) : nullptr;
    // decode batches: the base GEMM and the BGMV shrink share one launch
    const bool gemm_done = w0 && a.n_tiles == 0 &&
                           (fp8 ? gemm_w8_shrink_fits(T, a.d_out, a.d_in, a.n_su) : gemm_shrink_fits(dt, T, a.n_su));
    const PlanStage& ps = p->pstage[plan->stage];
    if (first && !gemm_done) {
        // (a batch without adapter rows reads no index)
        if (any && (e = launch_upload(ps.host_dev, base, plan->words, st)) != hipSuccess)
            return fail(LORA_EHIP, "plan upload: %s", hipGetErrorString(e));
        plan->uploaded = true;
    }
    if (gemm_done) {
        // a plan's first call reads the index from the staging buffer (host memory, through
        // its device mapping) and stores it in the ring entry in the same launch
        LoraArgs ah = a;
        const int32_t* rsh = rs;
        if (first) {
            const uint8_t* hb = static_cast<const uint8_t*>(ps.host_dev);
            auto H = [&](int64_t off) { return reinterpret_cast<const int32_t*>(hb) + off; };
            ah.g_slot = H(L.g_slot);
            ah.g_rank = H(L.g_rank);
            ah.g_begin = H(L.g_begin);
            ah.g_count = H(L.g_count);
            ah.g_gamma = reinterpret_cast<const float*>(H(L.g_gamma));
            ah.rows = H(L.rows);
            ah.su = H(L.su);
            ah.eu = H(L.eu);
            ah.s_slot = H(L.s_slot);
            ah.s_rank = H(L.s_rank);
            ah.s_gamma = reinterpret_cast<const float*>(H(L.s_gamma));
            ah.s_begin = H(L.s_begin);
            ah.s_end = H(L.s_end);
            ah.t_seg = H(L.t_seg);
            ah.t_row0 = H(L.t_row0);
            rsh = H(L.row_slot);
        }
        // rows with an adapter (at most 64 rows here): the decode rows in the plan's groups
        uint64_t raw_mask = 0;
        if (T <= 64)
            for (int32_t r : plan->rows) raw_mask |= uint64_t(1) << r;
        e = timed_launch(p, LORA_K_GEMM_BGMV_SHRINK, st, [&] {
            const void* cps = first ? ps.host_dev : nullptr;
            void* cpd = first ? base : nullptr;
            const int64_t cpn = first ? plan->words : 0;
            return fp8 ? launch_gemm_w8_shrink(x, w0, w0_scale, y, T, a.d_out, a.d_in, rsh, raw_mask, ybase, ah, cps,
                                               cpd, cpn, st)
                       : launch_gemm_shrink(dt, x, w0, y, T, a.d_out, a.d_in, rsh, raw_mask, ybase, ah, cps, cpd, cpn,
                                            st);
        });
        if (e != hipSuccess) return fail(LORA_EHIP, "base_gemm + bgmv shrink: %s", hipGetErrorString(e));
        plan->uploaded = true;
        a.ybase = ybase;
    }
    // shrinks first: the base GEMM may consume the prefill v in its epilogue.  With both kinds
    // of rows, the SGMV shrink goes first and the BGMV shrink's launch also sums its K parts
    const bool bgmv = !gemm_done && a.n_su > 0;
    if (a.n_tiles > 0 && (e = timed_launch(p, LORA_K_SGMV_SHRINK, st, [&] {
                              return launch_sgmv_shrink(dt, a, !bgmv, st);
                          })) != hipSuccess)
        return fail(LORA_EHIP, "sgmv shrink: %s", hipGetErrorString(e));
    if (bgmv && (e = timed_launch(p, LORA_K_BGMV_SHRINK, st, [&] {
                     return launch_bgmv_shrink(dt, a, a.n_tiles > 0 ? sgmv_shrink_parts(dt, a) : 1, st);
                 })) != hipSuccess)
        return fail(LORA_EHIP, "bgmv shrink: %s", hipGetErrorString(e));
    for (int32_t i = 0; i < n; ++i) {
        // projection i: its table offset, width, v and base area (the shrinks above wrote all
        // the v's; each GEMM writes its own base area, so one expand launch can follow them all)
        LoraArgs ai = a;
        float* ybase_i = ybase;
        if (n > 1) {
            ai.n_multi = 0;
            ai.lp_per_rank = a.lp_multi[i];
            ai.d_out = p->d_out[projs[i]];
            ai.nco = p->nco[projs[i]];
            ai.v = a.v + i * L.v_pstride;
            ai.y = ys[i];
            if (ybase) ybase_i = ybase + i * L.ybase_pstride;
        }
        const void* wi = w0s[i];
        void* yi = ys[i];
        bool fused = false;
        if (wi && !gemm_done) {
            // rows with an adapter keep the unrounded base for their expand: one rounding in total
            const LoraArgs* seg = plan->n_tiles > 0 ? &ai : nullptr;
            e = timed_launch(p, LORA_K_GEMM, st, [&] {
                return fp8 ? launch_gemm_w8(x, wi, w0_scale, yi, T, ai.d_out, ai.d_in, rs, ybase_i, st)
                           : launch_gemm(dt, x, wi, yi, T, ai.d_out, ai.d_in, rs, ybase_i, seg, &fused, st);
            });
            if (e != hipSuccess) return fail(LORA_EHIP, "base_gemm: %s", hipGetErrorString(e));
            ai.ybase = ybase_i;
            a.ybase = ybase;   // (all of them or none: w0 is given for all projections or none)
        }
        if (n == 1 && ai.n_eu > 0 &&
            (e = timed_launch(p, LORA_K_BGMV_EXPAND, st, [&] { return launch_bgmv_expand(dt, ai, st); })) != hipSuccess)
            return fail(LORA_EHIP, "bgmv expand: %s", hipGetErrorString(e));
        if (ai.n_tiles > 0 && !fused &&
            (e = timed_launch(p, LORA_K_SGMV_EXPAND, st, [&] { return launch_sgmv_expand(dt, ai, st); })) != hipSuccess)
            return fail(LORA_EHIP, "sgmv expand: %s", hipGetErrorString(e));
    }
    // several projections: the decode rows' expands of all of them in one launch
    if (n > 1 && a.n_eu > 0 &&
        (e = timed_launch(p, LORA_K_BGMV_EXPAND, st, [&] { return launch_bgmv_expand(dt, a, st); })) != hipSuccess)
        return fail(LORA_EHIP, "bgmv expand: %s", hipGetErrorString(e));
    plan->stream = st;   // the plan's event is recorded on the stream of its last call
    return LORA_OK;
}

}  // namespace

extern "C" {

int lora_linear(lora_pool* p, const lora_plan* plan, int32_t layer, int32_t proj, const void* x, const void* w0,
                void* y, void* stream) {
    return linear_impl(p, plan, layer, 1, &proj, x, &w0, nullptr, &y, stream);
}

int lora_linear_multi(lora_pool* p, const lora_plan* plan, int32_t layer, int32_t n, const int32_t* projs,
                      const void* x, const void* const* w0, void* const* y, void* stream) {
    return linear_impl(p, plan, layer, n, projs, x, w0, nullptr, y, stream);
}

int lora_linear_fp8(lora_pool* p, const lora_plan* plan, int32_t layer, int32_t proj, const void* x,
                    const void* w0_code, const float* w0_scale, void* y, void* stream) {
    if (!w0_code || !w0_scale) return fail(LORA_EINVAL, "w0_code and w0_scale are required");
    return linear_impl(p, plan, layer, 1, &proj, x, &w0_code, w0_scale, &y, stream);
}

int lora_linear_decode(lora_pool* p, int32_t layer, int32_t proj, const void* x, const void* w0, void* y,
                       const int32_t* token_slot, int32_t T, void* stream) {
    lora_plan* plan = nullptr;
    int rc = lora_plan_create(p, nullptr, nullptr, 0, token_slot, T, stream, &plan);
    if (rc) return rc;
    rc = lora_linear(p, plan, layer, proj, x, w0, y, stream);
    std::string keep = g_err;
    lora_plan_destroy(plan);
    if (rc) g_err = keep;
    return rc;
}

int lora_linear_prefill(lora_pool* p, int32_t layer, int32_t proj, const void* x, const void* w0, void* y,
                        const int32_t* seg_start, const int32_t* seg_slot, int32_t S, void* stream) {
    lora_plan* plan = nullptr;
    int rc = lora_plan_create(p, seg_start, seg_slot, S, nullptr, 0, stream, &plan);
    if (rc) return rc;
    rc = lora_linear(p, plan, layer, proj, x, w0, y, stream);
    std::string keep = g_err;
    lora_plan_destroy(plan);
    if (rc) g_err = keep;
    return rc;
}

int lora_linear_decode_noalloc(lora_pool* p, int32_t layer, int32_t proj, const void* x, const void* w0, void* y,
                               const int32_t* token_slot, int32_t T, void* stream) {
    if (!p) return fail(LORA_EINVAL, "pool is NULL");
    if (p->host_only) return fail(LORA_EINVAL, "host-only pool: no device work");
    if (proj < 0 || proj >= p->n_proj) return fail(LORA_EINVAL, "proj out of range");
    if (T < 0 || T > p->max_tokens) return fail(LORA_EINVAL, "%d rows, the pool allows %d", T, p->max_tokens);
    // a layout sized for this call (no segments), placed at the start of the scratch array
    const PlanLayout L = plan_layout(std::max(T, 1), 0, p->max_rank, p->d_out[proj]);
    if (L.entry_bytes > kScratchBytes)
        return fail(LORA_EINVAL, "%d rows x %d outputs need %lld bytes of scratch; the static scratch holds %lld "
                    "(use lora_linear_decode)", T, p->d_out[proj], (long long)L.entry_bytes, (long long)kScratchBytes);
    if (L.words > p->pl.words) return fail(LORA_EINVAL, "index of %lld words exceeds the staging buffers", (long long)L.words);
    uint8_t* dev = nullptr;
    int rc = scratch_on_current_device(&dev);
    if (rc) return rc;
    lora_plan* plan = nullptr;
    rc = plan_create_impl(p, nullptr, nullptr, 0, token_slot, T, stream, L, dev, &plan);
    if (rc) return rc;
    rc = lora_linear(p, plan, layer, proj, x, w0, y, stream);
    std::string keep = g_err;
    lora_plan_destroy(plan);
    if (rc) g_err = keep;
    return rc;
}

int base_gemm_fp8(const void* x, const void* w0_code, const float* w0_scale, void* y, int64_t M, int64_t N, int64_t K,
                  void* stream) {
    if (M < 0 || N < 1 || K < 1) return fail(LORA_EINVAL, "bad sizes");
    if (M == 0) return LORA_OK;
    if (!gemm_w8_ok(M, N, K)) return fail(LORA_EINVAL, "N must be a multiple of 4 and K of 128, byte offsets 32-bit");
    if (!x || !w0_code || !w0_scale || !y) return fail(LORA_EINVAL, "NULL pointer");
    if ((uintptr_t)x % 16 || (uintptr_t)w0_code % 16 || (uintptr_t)w0_scale % 16 || (uintptr_t)y % 16)
        return fail(LORA_EINVAL, "pointers must be 16-byte aligned");
    hipError_t e = launch_gemm_w8(x, w0_code, w0_scale, y, M, N, K, nullptr, nullptr, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(LORA_EHIP, "base_gemm_fp8: %s", hipGetErrorString(e));
    return LORA_OK;
}

int base_gemm(int32_t dtype, const void* x, const void* w0, void* y, int64_t M, int64_t N, int64_t K, void* stream) {
    if (dtype != LORA_F32 && dtype != LORA_BF16) return fail(LORA_EINVAL, "dtype must be LORA_F32 or LORA_BF16");
    if (M < 0 || N < 1 || K < 1 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return fail(LORA_EINVAL, "bad sizes");
    const int vec = dtype == LORA_BF16 ? 8 : 4;
    if (K % vec || N % 4) return fail(LORA_EINVAL, "K must be a multiple of %d and N of 4", vec);
    if (M == 0) return LORA_OK;
    if (!x || !w0 || !y) return fail(LORA_EINVAL, "NULL pointer");
    if ((uintptr_t)x % 16 || (uintptr_t)w0 % 16 || (uintptr_t)y % 16) return fail(LORA_EINVAL, "pointers must be 16-byte aligned");
    hipError_t e =
        launch_gemm(dtype, x, w0, y, M, N, K, nullptr, nullptr, nullptr, nullptr, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(LORA_EHIP, "base_gemm: %s", hipGetErrorString(e));
    return LORA_OK;
}

}  // extern "C"
