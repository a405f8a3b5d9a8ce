// Adapter engine over the pool: a host cache tier below the GPU pool, a
// least-recently-used GPU tier that never evicts an adapter a request is
// using, page-ins of the adapters the waiting queue will need, and the step's
// admission under a row cap and a distinct-adapter cap ("S-LoRA: Serving
// Thousands of Concurrent LoRA Adapters", Host memory for adapters;
// "Multi-LoRA serving: S-LoRA, Punica and adapter batching", What the engine
// does each step).  Host code only: every device operation goes through the
// pool's C ABI; the engine records events to time its copies.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <climits>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "internal.h"
#include "lora_gemm.h"

using hagemm::set_error;

namespace {

using Clock = std::chrono::steady_clock;

double ms_between(Clock::time_point t0, Clock::time_point t1) {
    return std::chrono::duration<double, std::milli>(t1 - t0).count();
}

// q-quantile by the nearest-rank rule (0 with no samples)
double quantile(std::vector<double> v, double q) {
    if (v.empty()) return 0.0;
    size_t k = (size_t)std::ceil(q * (double)v.size());
    k = k == 0 ? 0 : k - 1;
    if (k >= v.size()) k = v.size() - 1;
    std::nth_element(v.begin(), v.begin() + (std::ptrdiff_t)k, v.end());
    return v[k];
}

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct Request {
    int64_t id = 0;
    int64_t seq = 0;                 // arrival order
    int32_t adapter = -1;
    int32_t prompt = 0, max_new = 0, generated = 0;
    int64_t submit_step = 0;
    Clock::time_point submit_time;
    bool resident_at_arrival = false;
    int32_t slot = -1;               // pool slot acquired while running (adapter >= 0)
    std::vector<int32_t> kv;         // KV pages held while running
};

struct Adapter {
    int32_t rank = 0;
    float alpha = 0.f;
    // GPU tier
    bool resident = false;
    bool copying = false;            // page-in issued, completion not yet seen
    int32_t slot = -1;
    int32_t users = 0;               // running requests
    int64_t last_use = -1;           // step of the last admission, decode row or page-in
    // host tier
    int64_t host_unit = -1;          // first arena unit of its entry; -1 = not cached
    int64_t host_last_use = -1;
    bool host_reading = false;       // a copy in flight reads the entry
};

struct CopyBatch {
    hipEvent_t issue = nullptr;      // on the idle marker stream: the time of issue
    hipEvent_t start = nullptr;      // on the copy stream before the batch
    hipEvent_t end = nullptr;        // on the copy stream after the batch
    std::vector<int32_t> adapters;
};

}  // namespace

struct lora_engine {
    lora_pool* pool = nullptr;
    lora_engine_desc d{};
    hagemm::PoolInfo pi{};
    hipStream_t copy = nullptr;
    hipStream_t marker = nullptr;

    // host arena of n_units units; an adapter of rank r takes entry_units(r) consecutive units:
    // its A blob, then (256-byte aligned) its B blob
    uint8_t* arena = nullptr;
    int64_t a_row_bytes = 0, b_row_bytes = 0, unit_bytes = 0, n_units = 0;
    std::map<int64_t, int64_t> free_runs;  // first unit -> length

    std::unordered_map<int32_t, Adapter> adapters;
    std::unordered_map<int64_t, Request> reqs;
    std::map<int64_t, int64_t> waiting;    // seq -> request id
    std::vector<int64_t> running;          // admitted, unfinished, in admission order
    int64_t next_seq = 0;
    int64_t step_no = 0;

    bool in_step = false;
    lora_plan* plan = nullptr;
    std::vector<int64_t> step_prefill, step_decode;

    std::vector<CopyBatch> inflight;
    std::vector<hipEvent_t> spare;

    lora_engine_stats st{};
    std::vector<double> s_page_in, s_copy, s_wait_hit, s_wait_miss, s_wait_steps, s_storage;
};

namespace {

int64_t b_offset(const lora_engine* e, int32_t rank) { return align_up(rank * e->a_row_bytes, 256); }
int64_t entry_bytes(const lora_engine* e, int32_t rank) { return b_offset(e, rank) + rank * e->b_row_bytes; }
int64_t entry_units(const lora_engine* e, int32_t rank) {
    return (entry_bytes(e, rank) + e->unit_bytes - 1) / e->unit_bytes;
}

// ---- host arena ------------------------------------------------------------------------------

int64_t arena_take(lora_engine* e, int64_t n) {
    for (auto it = e->free_runs.begin(); it != e->free_runs.end(); ++it) {
        if (it->second < n) continue;
        const int64_t at = it->first, len = it->second;
        e->free_runs.erase(it);
        if (len > n) e->free_runs.emplace(at + n, len - n);
        return at;
    }
    return -1;
}

void arena_give(lora_engine* e, int64_t at, int64_t n) {
    auto next = e->free_runs.lower_bound(at);
    if (next != e->free_runs.end() && next->first == at + n) {
        n += next->second;
        next = e->free_runs.erase(next);
    }
    if (next != e->free_runs.begin()) {
        auto prev = std::prev(next);
        if (prev->first + prev->second == at) {
            prev->second += n;
            return;
        }
    }
    e->free_runs.emplace(at, n);
}

// Drop the least recently used host entry that no copy reads (not `keep`); false if none.
bool host_drop_one(lora_engine* e, int32_t keep) {
    int32_t victim = -1;
    int64_t best = LLONG_MAX;
    for (const auto& kv : e->adapters) {
        const Adapter& a = kv.second;
        if (a.host_unit < 0 || a.host_reading || kv.first == keep) continue;
        if (a.host_last_use < best || (a.host_last_use == best && kv.first < victim)) {
            best = a.host_last_use;
            victim = kv.first;
        }
    }
    if (victim < 0) return false;
    Adapter& a = e->adapters[victim];
    arena_give(e, a.host_unit, entry_units(e, a.rank));
    a.host_unit = -1;
    e->st.host_evictions++;
    return true;
}

// Adapter `id` in the host cache: 0 done (*hit says whether it was there), 1 no room now
// (every other entry is being read by a copy), < 0 error (storage load failed).
int host_ensure(lora_engine* e, int32_t id, Adapter& a, bool* hit) {
    a.host_last_use = e->step_no;
    if (a.host_unit >= 0) {
        *hit = true;
        return 0;
    }
    *hit = false;
    const int64_t n = entry_units(e, a.rank);
    int64_t at;
    while ((at = arena_take(e, n)) < 0)
        if (!host_drop_one(e, id)) return 1;
    uint8_t* base = e->arena + at * e->unit_bytes;
    const auto t0 = Clock::now();
    const int rc = e->d.fill(e->d.user, id, base, a.rank * e->a_row_bytes, base + b_offset(e, a.rank),
                             a.rank * e->b_row_bytes);
    e->s_storage.push_back(ms_between(t0, Clock::now()));
    if (rc != 0) {
        arena_give(e, at, n);
        return set_error(LORA_EINVAL, "loading adapter %d from storage failed (fill returned %d)", id, rc);
    }
    a.host_unit = at;
    return 0;
}

// ---- GPU tier ----------------------------------------------------------------------------------

// Evict a resident adapter whose copy is done, that no running request uses and that is not in
// `protect` or `skip`: the least recently used of those the look-ahead window does not want,
// else of those it wants.  1 evicted, 0 no candidate, < 0 error.  An adapter the pool refuses
// as referenced (the caller's acquire or a live plan) goes to `skip`.
int gpu_evict_one(lora_engine* e, const std::unordered_set<int32_t>& protect, std::unordered_set<int32_t>& skip,
                  const std::unordered_set<int32_t>& wanted) {
    for (;;) {
        int32_t victim = -1;
        std::pair<int, int64_t> best{INT_MAX, LLONG_MAX};
        for (const auto& kv : e->adapters) {
            const Adapter& a = kv.second;
            if (!a.resident || a.copying || a.users > 0 || protect.count(kv.first) || skip.count(kv.first)) continue;
            const std::pair<int, int64_t> key{wanted.count(kv.first) ? 1 : 0, a.last_use};
            if (key < best || (key == best && kv.first < victim)) {
                best = key;
                victim = kv.first;
            }
        }
        if (victim < 0) return 0;
        const int rc = lora_pool_evict(e->pool, victim);
        if (rc == LORA_EBUSY) {
            skip.insert(victim);
            continue;
        }
        Adapter& a = e->adapters[victim];
        if (rc == LORA_ENOTRESIDENT) {   // evicted behind the engine's back
            a.resident = false;
            a.slot = -1;
            continue;
        }
        if (rc) return rc;
        a.resident = false;
        a.slot = -1;
        e->st.gpu_evictions++;
        return 1;
    }
}

int pool_room(lora_engine* e, int64_t* free_pages, int32_t* resident) {
    int64_t kv = 0;
    return lora_pool_stats(e->pool, free_pages, resident, &kv);
}

hipEvent_t take_event(lora_engine* e) {
    if (!e->spare.empty()) {
        hipEvent_t ev = e->spare.back();
        e->spare.pop_back();
        return ev;
    }
    hipEvent_t ev = nullptr;
    if (hipEventCreate(&ev) != hipSuccess) return nullptr;
    return ev;
}

void give_events(lora_engine* e, CopyBatch& cb) {
    for (hipEvent_t ev : {cb.issue, cb.start, cb.end})
        if (ev) e->spare.push_back(ev);
    cb.issue = cb.start = cb.end = nullptr;
}

// Note finished copies (wait = block until all have finished).
int poll_copies(lora_engine* e, bool wait) {
    for (size_t i = 0; i < e->inflight.size();) {
        CopyBatch& cb = e->inflight[i];
        const hipError_t q = wait ? hipEventSynchronize(cb.end) : hipEventQuery(cb.end);
        if (q == hipErrorNotReady) {
            ++i;
            continue;
        }
        if (q != hipSuccess) return set_error(LORA_EHIP, "page-in event: %s", hipGetErrorString(q));
        float ms_issue = 0.f, ms_copy = 0.f;
        if (hipEventElapsedTime(&ms_issue, cb.issue, cb.end) != hipSuccess ||
            hipEventElapsedTime(&ms_copy, cb.start, cb.end) != hipSuccess)
            return set_error(LORA_EHIP, "page-in timing events");
        e->s_copy.push_back(ms_copy);
        for (int32_t id : cb.adapters) {
            Adapter& a = e->adapters[id];
            a.copying = false;
            a.host_reading = false;
            e->s_page_in.push_back(ms_issue);
            int32_t slot = -1;
            bool done = false;
            if (a.resident && lora_pool_slot_of(e->pool, id, &slot) == LORA_OK && slot == a.slot)
                (void)hagemm::pool_copy_done(e->pool, slot, &done);
        }
        give_events(e, cb);
        e->inflight.erase(e->inflight.begin() + (std::ptrdiff_t)i);
    }
    return LORA_OK;
}

// One page-in batch on the copy stream, timed from issue to done.
int issue_page_ins(lora_engine* e, const std::vector<lora_page_in_req>& reqs, const std::vector<int32_t>& ids) {
    const int32_t n = (int32_t)reqs.size();
    CopyBatch cb;
    cb.adapters = ids;
    if (!e->pi.host_only) {
        cb.issue = take_event(e);
        cb.start = take_event(e);
        cb.end = take_event(e);
        if (!cb.issue || !cb.start || !cb.end || hipEventRecord(cb.issue, e->marker) != hipSuccess ||
            hipEventRecord(cb.start, e->copy) != hipSuccess) {
            give_events(e, cb);
            for (int32_t id : ids) e->adapters[id].host_reading = false;
            return set_error(LORA_EHIP, "page-in timing events");
        }
    }
    std::vector<int32_t> slots(n, -1);
    const int rc = lora_pool_page_in_batch(e->pool, n, reqs.data(), e->copy, slots.data());
    if (rc) {
        give_events(e, cb);
        for (int32_t id : ids) e->adapters[id].host_reading = false;
        return rc;
    }
    if (!e->pi.host_only && hipEventRecord(cb.end, e->copy) != hipSuccess) {
        // the pages are in the pool; only the timing is lost: wait for the copy here
        (void)hipStreamSynchronize(e->copy);
        give_events(e, cb);
        cb.adapters.clear();
    }
    for (int32_t k = 0; k < n; ++k) {
        Adapter& a = e->adapters[ids[k]];
        a.resident = true;
        a.slot = slots[k];
        a.last_use = e->step_no;
        a.copying = cb.end != nullptr;
        a.host_reading = a.copying;
        e->st.page_ins++;
        e->st.page_in_bytes += reqs[k].host_A_bytes + reqs[k].host_B_bytes;
    }
    if (cb.end) e->inflight.push_back(std::move(cb));
    return LORA_OK;
}

// Waiting requests in scheduling order: those waiting max_wait_steps steps or more first, then
// the rest, each part in arrival order.
std::vector<int64_t> waiting_order(const lora_engine* e) {
    std::vector<int64_t> aged, rest;
    for (const auto& kv : e->waiting) {
        const Request& r = e->reqs.at(kv.second);
        if (e->d.max_wait_steps > 0 && e->step_no - r.submit_step >= e->d.max_wait_steps)
            aged.push_back(kv.second);
        else
            rest.push_back(kv.second);
    }
    aged.insert(aged.end(), rest.begin(), rest.end());
    return aged;
}

bool is_aged(const lora_engine* e, const Request& r) {
    return e->d.max_wait_steps > 0 && e->step_no - r.submit_step >= e->d.max_wait_steps;
}

std::unordered_set<int32_t> window_adapters(const lora_engine* e, const std::vector<int64_t>& order) {
    std::unordered_set<int32_t> w;
    for (size_t i = 0; i < order.size() && (int64_t)i < e->d.prefetch_window; ++i)
        if (e->reqs.at(order[i]).adapter >= 0) w.insert(e->reqs.at(order[i]).adapter);
    return w;
}

// Step 2: bring in the adapters the look-ahead window wants, in window order.  Room for the
// adapter of the request at window position i may come from evicting any candidate except the
// adapters of the requests ahead of it (positions < i), so the head of the queue can always be
// served once running requests let go, and nothing brought in this step is evicted again.
int page_in_ahead(lora_engine* e, const std::vector<int64_t>& order) {
    int64_t free_pages = 0;
    int32_t resident = 0;
    int rc = pool_room(e, &free_pages, &resident);
    if (rc) return rc;
    std::vector<lora_page_in_req> batch;
    std::vector<int32_t> ids;
    std::unordered_set<int32_t> ahead, claimed, skip;
    const std::unordered_set<int32_t> wanted = window_adapters(e, order);
    int64_t claim_pages = 0;
    for (size_t i = 0; i < order.size() && (int64_t)i < e->d.prefetch_window; ++i) {
        const int32_t id = e->reqs.at(order[i]).adapter;
        if (id < 0) continue;
        Adapter& a = e->adapters[id];
        if (a.resident || claimed.count(id)) {
            ahead.insert(id);
            continue;
        }
        const int64_t need = hagemm::pool_pages_for_rank(e->pool, a.rank);
        bool room = true;
        while (resident + (int32_t)claimed.size() + 1 > e->pi.max_slots || free_pages - claim_pages < need) {
            const int ev = gpu_evict_one(e, ahead, skip, wanted);
            if (ev < 0) rc = ev;
            else if (ev == 0) room = false;
            else rc = pool_room(e, &free_pages, &resident);
            if (rc || !room) break;
        }
        if (rc) break;
        if (!room) {
            e->st.room_stalls++;
            break;   // the requests behind it wait too
        }
        bool hit = false;
        const int h = host_ensure(e, id, a, &hit);
        if (h < 0) {
            rc = h;
            break;
        }
        if (h == 1) {
            e->st.room_stalls++;
            break;
        }
        (hit ? e->st.host_hits : e->st.host_misses)++;
        a.host_reading = true;   // until issued: later loads of this batch must not drop it
        uint8_t* base = e->arena + a.host_unit * e->unit_bytes;
        lora_page_in_req r{};
        r.adapter_id = id;
        r.rank = a.rank;
        r.alpha = a.alpha;
        r.base_id = e->pi.base_id;
        r.host_A = base;
        r.host_A_bytes = a.rank * e->a_row_bytes;
        r.host_B = base + b_offset(e, a.rank);
        r.host_B_bytes = a.rank * e->b_row_bytes;
        batch.push_back(r);
        ids.push_back(id);
        claimed.insert(id);
        ahead.insert(id);
        claim_pages += need;
    }
    if (!batch.empty()) {
        const int rc2 = issue_page_ins(e, batch, ids);
        if (rc == LORA_OK) rc = rc2;
    }
    return rc;
}

// Give a running (or admitted) request's adapter reference and KV pages back.
void let_go(lora_engine* e, Request& r) {
    if (r.adapter >= 0 && r.slot >= 0) {
        (void)lora_pool_release(e->pool, r.slot);
        e->adapters[r.adapter].users--;
        r.slot = -1;
    }
    if (!r.kv.empty()) {
        (void)lora_pool_free_kv(e->pool, (int32_t)r.kv.size(), r.kv.data());
        r.kv.clear();
    }
}

}  // namespace

extern "C" {

int lora_engine_create(lora_pool* pool, const lora_engine_desc* d, lora_engine** out) {
    if (!pool || !d || !out) return set_error(LORA_EINVAL, "NULL argument");
    const hagemm::PoolInfo pi = hagemm::pool_info(pool);
    if (!d->info || !d->fill) return set_error(LORA_EINVAL, "info and fill callbacks are required");
    if (d->max_step_tokens < 1 || d->max_step_tokens > pi.max_tokens)
        return set_error(LORA_EINVAL, "max_step_tokens %d outside 1..%d (the pool's max_tokens)", d->max_step_tokens,
                         pi.max_tokens);
    if (pi.max_segments < 1) return set_error(LORA_EINVAL, "the pool takes no prefill segments (max_segments 0)");
    if (d->max_distinct_adapters < 1) return set_error(LORA_EINVAL, "max_distinct_adapters must be >= 1");
    if (d->max_running < 1 || d->max_running > d->max_step_tokens)
        return set_error(LORA_EINVAL, "max_running %d outside 1..max_step_tokens", d->max_running);
    if (d->prefetch_window < 1) return set_error(LORA_EINVAL, "prefetch_window must be >= 1");
    if (d->admit_in_flight != 0 && d->admit_in_flight != 1) return set_error(LORA_EINVAL, "admit_in_flight must be 0 or 1");
    if (d->max_wait_steps < 0 || d->kv_pages_per_token < 0 || d->reserved != 0)
        return set_error(LORA_EINVAL, "max_wait_steps and kv_pages_per_token must be >= 0, reserved 0");
    lora_engine* e = new lora_engine;
    e->pool = pool;
    e->d = *d;
    e->pi = pi;
    e->copy = static_cast<hipStream_t>(d->copy_stream);
    e->a_row_bytes = pi.a_elems_per_rank * pi.elem_bytes;
    e->b_row_bytes = pi.b_elems_per_rank * pi.elem_bytes;
    e->unit_bytes = align_up(e->a_row_bytes + e->b_row_bytes, 256);
    e->n_units = d->host_cache_bytes / e->unit_bytes;
    if (e->n_units < entry_units(e, pi.max_rank)) {
        const long long need = (long long)(entry_units(e, pi.max_rank) * e->unit_bytes);
        delete e;
        return set_error(LORA_EINVAL, "host cache of %lld bytes cannot hold one adapter of rank %d (%lld bytes)",
                         (long long)d->host_cache_bytes, pi.max_rank, need);
    }
    const size_t bytes = (size_t)(e->n_units * e->unit_bytes);
    if (pi.host_only) {
        e->arena = static_cast<uint8_t*>(std::aligned_alloc(256, bytes));
        if (!e->arena) {
            delete e;
            return set_error(LORA_EINVAL, "host cache of %zu bytes: out of memory", bytes);
        }
    } else {
        void* h = nullptr;
        hipError_t he = hipHostMalloc(&h, bytes, hipHostMallocDefault);
        if (he == hipSuccess) he = hipStreamCreateWithFlags(&e->marker, hipStreamNonBlocking);
        if (he != hipSuccess) {
            if (h) (void)hipHostFree(h);
            delete e;
            return set_error(LORA_EHIP, "host cache of %zu bytes: %s", bytes, hipGetErrorString(he));
        }
        e->arena = static_cast<uint8_t*>(h);
    }
    e->free_runs.emplace(0, e->n_units);
    *out = e;
    return LORA_OK;
}

int lora_engine_destroy(lora_engine* e) {
    if (!e) return LORA_OK;
    int rc = poll_copies(e, true);
    if (e->plan) {
        const int r2 = lora_plan_destroy(e->plan);
        if (rc == LORA_OK) rc = r2;
        e->plan = nullptr;
    }
    for (auto& kv : e->reqs) let_go(e, kv.second);
    for (hipEvent_t ev : e->spare) (void)hipEventDestroy(ev);
    if (e->pi.host_only) {
        std::free(e->arena);
    } else {
        (void)hipHostFree(e->arena);
        if (e->marker) (void)hipStreamDestroy(e->marker);
    }
    delete e;
    return rc;
}

int lora_engine_submit(lora_engine* e, int64_t request_id, int32_t adapter_id, int32_t prompt_tokens,
                       int32_t max_new_tokens) {
    if (!e) return set_error(LORA_EINVAL, "engine is NULL");
    if (prompt_tokens < 1 || prompt_tokens > e->d.max_step_tokens)
        return set_error(LORA_EINVAL, "prompt_tokens %d outside 1..%d", prompt_tokens, e->d.max_step_tokens);
    if (max_new_tokens < 1) return set_error(LORA_EINVAL, "max_new_tokens must be >= 1");
    if (e->reqs.count(request_id)) return set_error(LORA_EINVAL, "request %lld is already queued or running",
                                                    (long long)request_id);
    bool resident = false;
    if (adapter_id >= 0) {
        auto it = e->adapters.find(adapter_id);
        if (it == e->adapters.end()) {
            int32_t rank = 0;
            float alpha = 0.f;
            uint64_t base = 0;
            const int rc = e->d.info(e->d.user, adapter_id, &rank, &alpha, &base);
            if (rc != 0) return set_error(LORA_EINVAL, "adapter %d: info returned %d", adapter_id, rc);
            if (rank < 1 || rank > e->pi.max_rank)
                return set_error(LORA_EINVAL, "adapter %d: rank %d outside 1..%d", adapter_id, rank, e->pi.max_rank);
            if (!std::isfinite(alpha)) return set_error(LORA_EINVAL, "adapter %d: alpha is not finite", adapter_id);
            if (base != e->pi.base_id)
                return set_error(LORA_EBASE, "adapter %d was made for base %llu, the pool serves %llu", adapter_id,
                                 (unsigned long long)base, (unsigned long long)e->pi.base_id);
            Adapter a;
            a.rank = rank;
            a.alpha = alpha;
            int32_t slot = -1;   // paged in through the pool before: adopt it
            if (lora_pool_slot_of(e->pool, adapter_id, &slot) == LORA_OK) {
                a.resident = true;
                a.slot = slot;
            }
            it = e->adapters.emplace(adapter_id, a).first;
        }
        resident = it->second.resident;
        (resident ? e->st.arrivals_resident : e->st.arrivals_missing)++;
    }
    Request r;
    r.id = request_id;
    r.seq = e->next_seq++;
    r.adapter = adapter_id;
    r.prompt = prompt_tokens;
    r.max_new = max_new_tokens;
    r.submit_step = e->step_no;
    r.submit_time = Clock::now();
    r.resident_at_arrival = resident;
    e->waiting.emplace(r.seq, request_id);
    e->reqs.emplace(request_id, std::move(r));
    return LORA_OK;
}

int lora_engine_cancel(lora_engine* e, int64_t request_id) {
    if (!e) return set_error(LORA_EINVAL, "engine is NULL");
    auto it = e->reqs.find(request_id);
    if (it == e->reqs.end() || !e->waiting.count(it->second.seq))
        return set_error(LORA_ENOTRESIDENT, "request %lld is not waiting", (long long)request_id);
    e->waiting.erase(it->second.seq);
    e->reqs.erase(it);
    e->st.cancelled++;
    return LORA_OK;
}

int lora_engine_step(lora_engine* e, void* stream, lora_engine_batch* out) {
    if (!e || !out) return set_error(LORA_EINVAL, "NULL argument");
    if (e->in_step) return set_error(LORA_EBUSY, "the previous step is not done (lora_engine_step_done)");
    *out = lora_engine_batch{};
    e->step_no++;
    e->st.steps++;
    int rc = poll_copies(e, false);
    if (rc) return rc;

    // 2. look-ahead page-ins
    const std::vector<int64_t> order = waiting_order(e);
    rc = page_in_ahead(e, order);
    if (rc) return rc;

    // 3. admission
    std::unordered_set<int32_t> distinct;
    for (int64_t rid : e->running)
        if (e->reqs.at(rid).adapter >= 0) distinct.insert(e->reqs.at(rid).adapter);
    int64_t rows_left = (int64_t)e->d.max_step_tokens - (int64_t)e->running.size();
    int64_t n_running = (int64_t)e->running.size();
    std::vector<int64_t> admitted;
    std::unordered_set<int32_t> skip, ahead;   // ahead: adapters of the requests before this one
    const std::unordered_set<int32_t> wanted = window_adapters(e, order);
    for (size_t i = 0; i < order.size(); ahead.insert(e->reqs.at(order[i]).adapter), ++i) {
        const int64_t rid = order[i];
        Request& r = e->reqs.at(rid);
        const bool aged = is_aged(e, r);
        if (r.adapter >= 0) {
            const Adapter& a = e->adapters[r.adapter];
            const bool ready = a.resident && (!a.copying || e->d.admit_in_flight);
            if (!ready) {
                if (aged && !a.copying) break;   // no room for its adapter: hold the others back
                continue;
            }
        }
        const bool fits = r.prompt <= rows_left && n_running + 1 <= e->d.max_running &&
                          (int64_t)admitted.size() + 1 <= e->pi.max_segments &&
                          (r.adapter < 0 || distinct.count(r.adapter) ||
                           (int64_t)distinct.size() + 1 <= e->d.max_distinct_adapters);
        if (!fits) {
            if (aged) break;
            continue;
        }
        if (e->d.kv_pages_per_token > 0) {
            const int64_t need = (int64_t)(r.prompt + r.max_new) * e->d.kv_pages_per_token;
            bool got = false;
            if (need <= INT32_MAX) {
                r.kv.assign((size_t)need, -1);
                std::unordered_set<int32_t> keep = ahead;
                keep.insert(distinct.begin(), distinct.end());
                if (r.adapter >= 0) keep.insert(r.adapter);
                for (;;) {
                    const int k = lora_pool_alloc_kv(e->pool, (int32_t)need, r.kv.data());
                    if (k == LORA_OK) {
                        got = true;
                        break;
                    }
                    if (k != LORA_ENOPAGES) {
                        rc = k;
                        break;
                    }
                    const int ev = gpu_evict_one(e, keep, skip, wanted);
                    if (ev < 0) rc = ev;
                    if (ev <= 0) break;
                }
            }
            if (!got) r.kv.clear();
            if (rc) break;
            if (!got) {
                e->st.kv_stalls++;
                if (aged) break;
                continue;
            }
        }
        if (r.adapter >= 0) {
            Adapter& a = e->adapters[r.adapter];
            rc = lora_pool_acquire(e->pool, a.slot);
            if (rc) {
                let_go(e, r);
                break;
            }
            r.slot = a.slot;
            a.users++;
            a.last_use = e->step_no;
            distinct.insert(r.adapter);
        }
        rows_left -= r.prompt;
        n_running++;
        admitted.push_back(rid);
    }

    // 4. the plan: admitted prompts as segments, then the running requests' decode rows
    if (rc == LORA_OK && (!admitted.empty() || !e->running.empty())) {
        std::vector<int32_t> seg_start(admitted.size() + 1, 0), seg_slot(admitted.size()), token_slot(e->running.size());
        for (size_t s = 0; s < admitted.size(); ++s) {
            const Request& r = e->reqs.at(admitted[s]);
            seg_start[s + 1] = seg_start[s] + r.prompt;
            seg_slot[s] = r.adapter >= 0 ? r.slot : -1;
        }
        for (size_t i = 0; i < e->running.size(); ++i) {
            const Request& r = e->reqs.at(e->running[i]);
            token_slot[i] = r.adapter >= 0 ? r.slot : -1;
        }
        rc = lora_plan_create(e->pool, seg_start.data(), seg_slot.data(), (int32_t)admitted.size(), token_slot.data(),
                              (int32_t)token_slot.size(), stream, &e->plan);
        if (rc == LORA_OK) {
            out->plan = e->plan;
            out->n_rows = seg_start.back() + (int32_t)e->running.size();
        }
    }
    if (rc) {   // nothing admitted: undo this step's admissions
        for (int64_t rid : admitted) let_go(e, e->reqs.at(rid));
        e->plan = nullptr;
        return rc;
    }
    const auto now = Clock::now();
    for (int64_t rid : admitted) {
        const Request& r = e->reqs.at(rid);
        e->waiting.erase(r.seq);
        const double w = ms_between(r.submit_time, now);
        if (r.adapter >= 0) (r.resident_at_arrival ? e->s_wait_hit : e->s_wait_miss).push_back(w);
        else e->s_wait_hit.push_back(w);
        e->s_wait_steps.push_back((double)(e->step_no - r.submit_step));
    }
    for (int64_t rid : e->running) {
        const Request& r = e->reqs.at(rid);
        if (r.adapter >= 0) e->adapters[r.adapter].last_use = e->step_no;
    }
    e->step_prefill = admitted;
    e->step_decode = e->running;
    e->in_step = e->plan != nullptr;
    e->st.admitted += (int64_t)admitted.size();
    e->st.rows += out->n_rows;
    out->n_prefill = (int32_t)admitted.size();
    out->n_requests = (int32_t)(admitted.size() + e->running.size());
    out->n_distinct = (int32_t)distinct.size();
    return LORA_OK;
}

int lora_engine_batch_requests(const lora_engine* e, int64_t* ids, int32_t* adapters, int32_t* rows) {
    if (!e) return set_error(LORA_EINVAL, "engine is NULL");
    size_t k = 0;
    for (int pass = 0; pass < 2; ++pass) {
        for (int64_t rid : pass == 0 ? e->step_prefill : e->step_decode) {
            const Request& r = e->reqs.at(rid);
            if (ids) ids[k] = rid;
            if (adapters) adapters[k] = r.adapter;
            if (rows) rows[k] = pass == 0 ? r.prompt : 1;
            ++k;
        }
    }
    return LORA_OK;
}

int lora_engine_step_done(lora_engine* e) {
    if (!e) return set_error(LORA_EINVAL, "engine is NULL");
    if (!e->in_step) return LORA_OK;
    const int rc = lora_plan_destroy(e->plan);
    e->plan = nullptr;
    e->in_step = false;
    for (int64_t rid : e->step_decode) e->reqs.at(rid).generated++;
    for (int64_t rid : e->step_prefill) {
        e->reqs.at(rid).generated = 1;
        e->running.push_back(rid);
    }
    std::vector<int64_t> still;
    still.reserve(e->running.size());
    for (int64_t rid : e->running) {
        Request& r = e->reqs.at(rid);
        if (r.generated < r.max_new) {
            still.push_back(rid);
            continue;
        }
        let_go(e, r);
        e->reqs.erase(rid);
        e->st.finished++;
    }
    e->running.swap(still);
    e->step_prefill.clear();
    e->step_decode.clear();
    return rc;
}

int lora_engine_kv_pages(const lora_engine* e, int64_t request_id, int32_t cap, int32_t* pages, int32_t* n_out) {
    if (!e || !n_out) return set_error(LORA_EINVAL, "NULL argument");
    auto it = e->reqs.find(request_id);
    if (it == e->reqs.end() || e->waiting.count(it->second.seq))
        return set_error(LORA_ENOTRESIDENT, "request %lld is not running", (long long)request_id);
    const std::vector<int32_t>& kv = it->second.kv;
    *n_out = (int32_t)kv.size();
    if (pages)
        for (int32_t i = 0; i < cap && i < (int32_t)kv.size(); ++i) pages[i] = kv[i];
    return LORA_OK;
}

int lora_engine_get_stats(lora_engine* e, lora_engine_stats* out) {
    if (!e || !out) return set_error(LORA_EINVAL, "NULL argument");
    const int rc = poll_copies(e, false);
    if (rc) return rc;
    lora_engine_stats s = e->st;
    s.waiting = (int64_t)e->waiting.size();
    s.running = (int64_t)e->running.size();
    s.page_in_ms_p50 = quantile(e->s_page_in, 0.50);
    s.page_in_ms_p99 = quantile(e->s_page_in, 0.99);
    s.page_in_ms_max = quantile(e->s_page_in, 1.0);
    s.copy_ms_p50 = quantile(e->s_copy, 0.50);
    s.copy_ms_p99 = quantile(e->s_copy, 0.99);
    s.wait_ms_hit_p50 = quantile(e->s_wait_hit, 0.50);
    s.wait_ms_hit_p99 = quantile(e->s_wait_hit, 0.99);
    s.wait_ms_miss_p50 = quantile(e->s_wait_miss, 0.50);
    s.wait_ms_miss_p99 = quantile(e->s_wait_miss, 0.99);
    s.wait_steps_p99 = quantile(e->s_wait_steps, 0.99);
    s.wait_steps_max = quantile(e->s_wait_steps, 1.0);
    s.storage_ms_p50 = quantile(e->s_storage, 0.50);
    s.storage_ms_p99 = quantile(e->s_storage, 0.99);
    *out = s;
    return LORA_OK;
}

int lora_engine_reset_stats(lora_engine* e) {
    if (!e) return set_error(LORA_EINVAL, "engine is NULL");
    const int rc = poll_copies(e, false);
    e->st = lora_engine_stats{};
    for (auto* v : {&e->s_page_in, &e->s_copy, &e->s_wait_hit, &e->s_wait_miss, &e->s_wait_steps, &e->s_storage})
        v->clear();
    return rc;
}

}  // extern "C"
