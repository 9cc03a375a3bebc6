// Host side of the unified page pool: page bookkeeping, adapter loads, KV growth and queries.
//
// Behaviour follows the pool sketch of "S-LoRA, in depth", section "Unified paging: adapters and
// KV cache in one pool": one free list for KV and adapter pages, allocation from the end of the
// list, frees appended to it, adapters refcounted by their users, idle adapters evicted oldest
// first when an allocation is short, one KV token = 2 * layers pages.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>

#include "internal.h"

using namespace lorapool;

namespace lorapool {

static thread_local std::string g_last_error;

int set_error(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int hip_error(hipError_t e, const char *what) {
    return set_error(LORA_EHIP, "%s failed: %s", what, hipGetErrorString(e));
}

static void clear_error() { g_last_error.clear(); }

}  // namespace lorapool

extern "C" const char *lora_last_error(void) { return g_last_error.c_str(); }

#ifndef LORAPOOL_SRC_HASH
#define LORAPOOL_SRC_HASH "unknown"
#endif
extern "C" const char *lora_version(void) { return "lorapool 0.2 (gfx950) src " LORAPOOL_SRC_HASH; }

extern "C" int64_t lora_pool_pages_for(int32_t rank, int32_t projections, int32_t layers) {
    if (rank < 0 || projections < 0 || layers < 0) return -1;
    return (int64_t)rank * 2 * projections * layers;
}

extern "C" int64_t lora_kv_pages_per_token(int32_t layers) {
    if (layers < 0) return -1;
    return 2 * (int64_t)layers;
}

static void destroy(lora_pool *p) {
    if (!p) return;
    if (!p->bookkeeping_only) {
        DeviceGuard g(p->device);
        for (auto &b : p->load_buf) {
            if (b.done) (void)hipEventSynchronize(b.done);
            if (b.staging) (void)hipFree(b.staging);
            if (b.rows_dev) (void)hipFree(b.rows_dev);
            if (b.rows_host) (void)hipHostFree(b.rows_host);
            if (b.done) (void)hipEventDestroy(b.done);
        }
        if (p->dev_err) (void)hipFree(p->dev_err);
        for (hipEvent_t e : p->prof_events) (void)hipEventDestroy(e);
    }
    delete p;
}

extern "C" int lora_pool_create(void *pages, int64_t num_pages, int32_t hidden, int32_t dtype,
                                int32_t max_rank, int32_t n_slots, int32_t max_adapters,
                                int32_t *page_table, const int64_t *free_order, lora_pool **out) {
    clear_error();
    if (!out) return set_error(LORA_EINVAL, "lora_pool_create: out is NULL");
    *out = nullptr;
    if (num_pages < 1 || num_pages > INT32_MAX)
        return set_error(LORA_EINVAL, "lora_pool_create: num_pages %lld not in [1, 2^31-1]", (long long)num_pages);
    if (hidden < 64 || hidden > 65536 || hidden % 64)
        return set_error(LORA_EINVAL, "lora_pool_create: hidden %d must be a multiple of 64 in [64, 65536]", hidden);
    if (dtype != LORA_F32 && dtype != LORA_BF16)
        return set_error(LORA_EINVAL, "lora_pool_create: unknown dtype %d", dtype);
    if (max_rank < 1 || max_rank > LORA_MAX_RANK)
        return set_error(LORA_ERANK, "lora_pool_create: max_rank %d not in [1, %d]", max_rank, LORA_MAX_RANK);
    if (n_slots < 1 || n_slots > 1 << 16)
        return set_error(LORA_EINVAL, "lora_pool_create: n_slots %d not in [1, 65536]", n_slots);
    if (max_adapters < 1 || max_adapters > LORA_MAX_ADAPTERS)
        return set_error(LORA_EINVAL, "lora_pool_create: max_adapters %d not in [1, %d]", max_adapters, LORA_MAX_ADAPTERS);
    const bool bk = (pages == nullptr && page_table == nullptr);
    if (!bk && (pages == nullptr || page_table == nullptr))
        return set_error(LORA_EINVAL, "lora_pool_create: pages and page_table must both be set or both be NULL");
    if (!bk && ((uintptr_t)pages % 16 || (uintptr_t)page_table % 4))
        return set_error(LORA_EINVAL, "lora_pool_create: pages must be 16-byte and page_table 4-byte aligned");

    lora_pool *p = new (std::nothrow) lora_pool();
    if (!p) return set_error(LORA_ENOMEM, "lora_pool_create: out of host memory");
    p->pages = pages;
    p->num_pages = num_pages;
    p->hidden = hidden;
    p->dtype = dtype;
    p->elem = dtype == LORA_F32 ? 4 : 2;
    p->max_rank = max_rank;
    p->n_slots = n_slots;
    p->max_adapters = max_adapters;
    p->page_table = page_table;
    p->bookkeeping_only = bk;
    try {
        p->free_list.resize((size_t)num_pages);
        if (free_order) {
            std::vector<uint8_t> seen((size_t)num_pages, 0);
            for (int64_t i = 0; i < num_pages; ++i) {
                const int64_t v = free_order[i];
                if (v < 0 || v >= num_pages || seen[(size_t)v]) {
                    delete p;
                    return set_error(LORA_EINVAL, "lora_pool_create: free_order is not a permutation (entry %lld = %lld)",
                                     (long long)i, (long long)v);
                }
                seen[(size_t)v] = 1;
                p->free_list[(size_t)i] = v;
            }
        } else {
            for (int64_t i = 0; i < num_pages; ++i) p->free_list[(size_t)i] = i;
        }
    } catch (...) {
        delete p;
        return set_error(LORA_ENOMEM, "lora_pool_create: out of host memory");
    }
    if (!bk) {
        hipError_t e = hipGetDevice(&p->device);
        if (e != hipSuccess) { destroy(p); return hip_error(e, "hipGetDevice"); }
        // lora_project_noalloc's scratch address on this device; a failure here only disables that
        // entry point (it retries and reports the error), so it does not fail the pool
        if (scratch_setup(p->device) != LORA_OK) clear_error();
        const size_t slot_bytes = 2ull * max_rank * hidden * p->elem;          // A and B of one slot
        const size_t want = slot_bytes * (size_t)n_slots;
        p->staging_bytes = std::max(slot_bytes, std::min(want, (size_t)64 << 20));
        const size_t rows_bytes = (size_t)n_slots * 2 * max_rank * sizeof(int32_t);
        const size_t pt_bytes = (size_t)n_slots * max_adapters * 2 * max_rank * sizeof(int32_t);
        for (auto &b : p->load_buf) {
            if ((e = hipMalloc(&b.staging, p->staging_bytes)) != hipSuccess ||
                (e = hipMalloc((void **)&b.rows_dev, rows_bytes)) != hipSuccess ||
                (e = hipHostMalloc((void **)&b.rows_host, rows_bytes, hipHostMallocDefault)) != hipSuccess ||
                (e = hipEventCreateWithFlags(&b.done, hipEventDisableTiming)) != hipSuccess) {
                destroy(p);
                return hip_error(e, "lora_pool_create load buffers");
            }
        }
        if ((e = hipMalloc((void **)&p->dev_err, 64)) != hipSuccess ||
            (e = hipMemset(p->dev_err, 0, 64)) != hipSuccess ||
            (e = hipMemset(page_table, 0xff, pt_bytes)) != hipSuccess ||
            (e = hipDeviceSynchronize()) != hipSuccess) {
            destroy(p);
            return hip_error(e, "lora_pool_create device setup");
        }
    }
    *out = p;
    return LORA_OK;
}

extern "C" int lora_pool_free(lora_pool *pool) {
    clear_error();
    destroy(pool);
    return LORA_OK;
}

// ---- bookkeeping (caller holds p->mu) ------------------------------------------------------------

static void drop_adapter(lora_pool *p, int32_t aid) {
    auto it = p->adapters.find(aid);
    Adapter &ad = it->second;
    p->free_list.insert(p->free_list.end(), ad.pages.begin(), ad.pages.end());
    p->adapter_total -= (int64_t)ad.pages.size();
    p->adapters.erase(it);
    p->load_order.erase(std::find(p->load_order.begin(), p->load_order.end(), aid));
    p->n_evictions++;
}

static int clear_rows(lora_pool *p, int32_t aid, hipStream_t s) {
    if (p->bookkeeping_only) return LORA_OK;
    DeviceGuard g(p->device);
    hipError_t e = launch_clear_rows(p->page_table, p->max_adapters, 2 * p->max_rank, aid, p->n_slots, s);
    if (e != hipSuccess) return hip_error(e, "clear page-table rows");
    return LORA_OK;
}

// The idle adapters in the order the pool's victim rule evicts them (load order, least recently
// admitted first, or next request in the lookahead farthest first with the ones beyond it least
// recently admitted first).
static std::vector<int32_t> victim_order(lora_pool *p) {
    std::vector<int32_t> idle;
    for (int32_t a : p->load_order)
        if (p->adapters[a].users == 0) idle.push_back(a);
    if (p->victim_rule == LORA_VICTIM_LRU) {
        std::stable_sort(idle.begin(), idle.end(),
                         [&](int32_t a, int32_t b) { return p->adapters[a].last_use < p->adapters[b].last_use; });
    } else if (p->victim_rule == LORA_VICTIM_FARTHEST) {
        const int64_t far = (int64_t)p->lookahead.size();
        std::unordered_map<int32_t, int64_t> next;
        for (int64_t i = far - 1; i >= 0; --i) next[p->lookahead[(size_t)i]] = i;   // first occurrence wins
        auto nx = [&](int32_t a) { auto it = next.find(a); return it == next.end() ? far : it->second; };
        std::stable_sort(idle.begin(), idle.end(), [&](int32_t a, int32_t b) {
            const int64_t na = nx(a), nb = nx(b);
            if (na != nb) return na > nb;
            return p->adapters[a].last_use < p->adapters[b].last_use;
        });
    }
    return idle;
}

// Evict idle adapters in victim order until `need` pages are free; true if enough are free.
static int evict_idle(lora_pool *p, int64_t need, hipStream_t s, bool *enough) {
    for (int32_t a : victim_order(p)) {
        drop_adapter(p, a);
        int rc = clear_rows(p, a, s);
        if (rc) return rc;
        if ((int64_t)p->free_list.size() >= need) { *enough = true; return LORA_OK; }
    }
    *enough = (int64_t)p->free_list.size() >= need;
    return LORA_OK;
}

static bool device_pointer(const void *ptr) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, ptr) != hipSuccess) {
        (void)hipGetLastError();   // pageable host memory is not registered: clear the error
        return false;
    }
    return attr.type == hipMemoryTypeDevice;
}

static int copy_adapter(lora_pool *p, const Adapter &ad, int32_t aid, const void *A_t, const void *B,
                        hipStream_t s) {
    DeviceGuard g(p->device);
    const int32_t r = ad.rank, stride = 2 * p->max_rank, H = p->hidden, S = p->n_slots;
    // the next load buffer; the host waits only if the load that used it last is still queued
    lora_pool::LoadBuf &lb = p->load_buf[p->load_next];
    p->load_next = (p->load_next + 1) % lora_pool::LOAD_RING;
    LP_HIP(hipEventSynchronize(lb.done));
    for (int32_t sl = 0; sl < S; ++sl) {
        int32_t *row = lb.rows_host + (size_t)sl * stride;
        for (int32_t j = 0; j < stride; ++j)
            row[j] = j < 2 * r ? (int32_t)ad.pages[(size_t)sl * 2 * r + j] : -1;
    }
    LP_HIP(hipMemcpyAsync(lb.rows_dev, lb.rows_host, (size_t)S * stride * sizeof(int32_t),
                          hipMemcpyHostToDevice, s));
    if (r > 0) {
        const size_t block = (size_t)r * H * p->elem;   // one slot's A_t (or B) in bytes
        if (device_pointer(A_t) && device_pointer(B)) {
            LP_HIP(launch_scatter_rows(p->pages, H, p->elem, A_t, B, (int64_t)r * H, 0, S, r, lb.rows_dev,
                                       stride, s));
        } else {
            const int32_t per = (int32_t)std::max<size_t>(1, p->staging_bytes / (2 * block));
            for (int32_t s0 = 0; s0 < S; s0 += per) {
                const int32_t n = std::min(per, S - s0);
                char *stA = (char *)lb.staging, *stB = stA + (size_t)n * block;
                LP_HIP(hipMemcpyAsync(stA, (const char *)A_t + (size_t)s0 * block, (size_t)n * block,
                                      hipMemcpyDefault, s));
                LP_HIP(hipMemcpyAsync(stB, (const char *)B + (size_t)s0 * block, (size_t)n * block,
                                      hipMemcpyDefault, s));
                LP_HIP(launch_scatter_rows(p->pages, H, p->elem, stA, stB, (int64_t)r * H, s0, n, r,
                                           lb.rows_dev, stride, s));
            }
        }
    }
    LP_HIP(launch_write_rows(p->page_table, p->max_adapters, stride, aid, lb.rows_dev, S, s));
    LP_HIP(hipEventRecord(lb.done, s));
    return LORA_OK;
}

extern "C" int lora_pool_load_adapter(lora_pool *p, int32_t aid, int32_t rank, const void *A_t,
                                      const void *B, void *stream) {
    clear_error();
    if (!p) return set_error(LORA_EINVAL, "lora_pool_load_adapter: pool is NULL");
    if (aid < 0 || aid >= p->max_adapters)
        return set_error(LORA_EINVAL, "lora_pool_load_adapter: adapter id %d not in [0, %d)", aid, p->max_adapters);
    if (rank < 0 || rank > p->max_rank)
        return set_error(LORA_ERANK, "lora_pool_load_adapter: rank %d not in [0, %d]", rank, p->max_rank);
    if (!p->bookkeeping_only && rank > 0 && (!A_t || !B))
        return set_error(LORA_EINVAL, "lora_pool_load_adapter: A_t and B are required for rank %d", rank);
    hipStream_t s = (hipStream_t)stream;
    std::lock_guard<std::mutex> lk(p->mu);
    auto it = p->adapters.find(aid);
    if (it != p->adapters.end()) {
        if (it->second.rank != rank)
            return set_error(LORA_EEXIST, "lora_pool_load_adapter: adapter %d is resident at rank %d, not %d", aid,
                             it->second.rank, rank);
        it->second.users++;
        it->second.last_use = ++p->tick;
        return LORA_OK;
    }
    const int64_t need = (int64_t)2 * rank * p->n_slots;
    if ((int64_t)p->free_list.size() < need) {
        bool enough = false;
        int rc = evict_idle(p, need, s, &enough);
        if (rc) return rc;
        if (!enough)
            return set_error(LORA_ENOMEM, "lora_pool_load_adapter: adapter %d needs %lld pages, %lld free", aid,
                             (long long)need, (long long)p->free_list.size());
    }
    Adapter ad;
    ad.rank = rank;
    ad.users = 1;
    ad.pages.reserve((size_t)need);
    for (int64_t i = 0; i < need; ++i) {
        ad.pages.push_back(p->free_list.back());
        p->free_list.pop_back();
    }
    if (!p->bookkeeping_only) {
        int rc = copy_adapter(p, ad, aid, A_t, B, s);
        if (rc) {   // give the pages back exactly where they were
            for (auto q = ad.pages.rbegin(); q != ad.pages.rend(); ++q) p->free_list.push_back(*q);
            return rc;
        }
        p->bytes_loaded += need * (int64_t)p->hidden * p->elem;
    }
    p->adapter_total += need;
    ad.last_use = ++p->tick;
    p->adapters.emplace(aid, std::move(ad));
    p->load_order.push_back(aid);
    p->n_loads++;
    return LORA_OK;
}

extern "C" int lora_pool_set_victim_rule(lora_pool *p, int32_t rule) {
    clear_error();
    if (!p) return set_error(LORA_EINVAL, "lora_pool_set_victim_rule: pool is NULL");
    if (rule != LORA_VICTIM_LOAD_ORDER && rule != LORA_VICTIM_LRU && rule != LORA_VICTIM_FARTHEST)
        return set_error(LORA_EINVAL, "lora_pool_set_victim_rule: unknown rule %d", rule);
    std::lock_guard<std::mutex> lk(p->mu);
    p->victim_rule = rule;
    return LORA_OK;
}

extern "C" int lora_pool_set_lookahead(lora_pool *p, const int32_t *ids, int64_t n) {
    clear_error();
    if (!p) return set_error(LORA_EINVAL, "lora_pool_set_lookahead: pool is NULL");
    if (n < 0 || (n > 0 && !ids)) return set_error(LORA_EINVAL, "lora_pool_set_lookahead: %lld ids at %p", (long long)n, (const void *)ids);
    std::lock_guard<std::mutex> lk(p->mu);
    try {
        p->lookahead.assign(ids, ids + n);
    } catch (...) {
        return set_error(LORA_ENOMEM, "lora_pool_set_lookahead: out of host memory");
    }
    return LORA_OK;
}

extern "C" int lora_pool_release_adapter(lora_pool *p, int32_t aid) {
    clear_error();
    if (!p) return set_error(LORA_EINVAL, "lora_pool_release_adapter: pool is NULL");
    std::lock_guard<std::mutex> lk(p->mu);
    auto it = p->adapters.find(aid);
    if (it == p->adapters.end()) return set_error(LORA_ENOENT, "lora_pool_release_adapter: adapter %d is not resident", aid);
    if (it->second.users == 0) return set_error(LORA_EINVAL, "lora_pool_release_adapter: adapter %d has no users", aid);
    it->second.users--;
    return LORA_OK;
}

extern "C" int lora_pool_evict_adapter(lora_pool *p, int32_t aid, void *stream) {
    clear_error();
    if (!p) return set_error(LORA_EINVAL, "lora_pool_evict_adapter: pool is NULL");
    std::lock_guard<std::mutex> lk(p->mu);
    auto it = p->adapters.find(aid);
    if (it == p->adapters.end()) return set_error(LORA_ENOENT, "lora_pool_evict_adapter: adapter %d is not resident", aid);
    if (it->second.users > 0)
        return set_error(LORA_EBUSY, "lora_pool_evict_adapter: adapter %d has %d users", aid, it->second.users);
    drop_adapter(p, aid);
    return clear_rows(p, aid, (hipStream_t)stream);
}

extern "C" int lora_pool_grow_kv(lora_pool *p, int64_t rid, int32_t layers, int64_t *out) {
    clear_error();
    if (!p) return set_error(LORA_EINVAL, "lora_pool_grow_kv: pool is NULL");
    if (layers < 1) return set_error(LORA_EINVAL, "lora_pool_grow_kv: layers %d < 1", layers);
    std::lock_guard<std::mutex> lk(p->mu);
    const int64_t need = 2 * (int64_t)layers;
    if ((int64_t)p->free_list.size() < need)
        return set_error(LORA_ENOMEM, "lora_pool_grow_kv: need %lld pages, %lld free", (long long)need,
                         (long long)p->free_list.size());
    std::vector<int64_t> &v = p->kv[rid];
    for (int64_t i = 0; i < need; ++i) {
        const int64_t pg = p->free_list.back();
        p->free_list.pop_back();
        v.push_back(pg);
        if (out) out[i] = pg;
    }
    p->kv_total += need;
    return LORA_OK;
}

extern "C" int lora_pool_free_kv(lora_pool *p, int64_t rid) {
    clear_error();
    if (!p) return set_error(LORA_EINVAL, "lora_pool_free_kv: pool is NULL");
    std::lock_guard<std::mutex> lk(p->mu);
    auto it = p->kv.find(rid);
    if (it == p->kv.end()) return set_error(LORA_ENOENT, "lora_pool_free_kv: request %lld holds no KV pages", (long long)rid);
    p->free_list.insert(p->free_list.end(), it->second.begin(), it->second.end());
    p->kv_total -= (int64_t)it->second.size();
    p->kv.erase(it);
    return LORA_OK;
}

// ---- queries --------------------------------------------------------------------------------------

extern "C" int lora_pool_stats(const lora_pool *pc, lora_pool_stats_t *out) {
    clear_error();
    if (!pc || !out) return set_error(LORA_EINVAL, "lora_pool_stats: NULL argument");
    lora_pool *p = const_cast<lora_pool *>(pc);
    std::lock_guard<std::mutex> lk(p->mu);
    memset(out, 0, sizeof *out);
    out->num_pages = p->num_pages;
    out->free_pages = (int64_t)p->free_list.size();
    out->kv_pages = p->kv_total;
    out->adapter_pages = p->adapter_total;
    out->resident_adapters = (int32_t)p->adapters.size();
    for (auto &kv : p->adapters) out->idle_adapters += kv.second.users == 0;
    out->kv_requests = (int64_t)p->kv.size();
    out->loads = p->n_loads;
    out->evictions = p->n_evictions;
    out->bytes_loaded = p->bytes_loaded;
    return LORA_OK;
}

extern "C" int lora_pool_page_table(const lora_pool *p, int32_t slot, const int32_t **table, int32_t *row_stride) {
    clear_error();
    if (!p || !table) return set_error(LORA_EINVAL, "lora_pool_page_table: NULL argument");
    if (p->bookkeeping_only) return set_error(LORA_EINVAL, "lora_pool_page_table: bookkeeping-only pool has no table");
    if (slot < 0 || slot >= p->n_slots) return set_error(LORA_EINVAL, "lora_pool_page_table: slot %d not in [0, %d)", slot, p->n_slots);
    *table = p->page_table + (size_t)slot * p->max_adapters * 2 * p->max_rank;
    if (row_stride) *row_stride = 2 * p->max_rank;
    return LORA_OK;
}

extern "C" int lora_pool_adapter_pages(const lora_pool *pc, int32_t aid, int64_t *out, int64_t cap, int64_t *n_out,
                                       int32_t *rank_out, int32_t *users_out) {
    clear_error();
    if (!pc) return set_error(LORA_EINVAL, "lora_pool_adapter_pages: pool is NULL");
    lora_pool *p = const_cast<lora_pool *>(pc);
    std::lock_guard<std::mutex> lk(p->mu);
    auto it = p->adapters.find(aid);
    if (it == p->adapters.end()) return set_error(LORA_ENOENT, "lora_pool_adapter_pages: adapter %d is not resident", aid);
    const auto &pg = it->second.pages;
    if (n_out) *n_out = (int64_t)pg.size();
    if (rank_out) *rank_out = it->second.rank;
    if (users_out) *users_out = it->second.users;
    if ((int64_t)pg.size() > cap || (!out && !pg.empty()))
        return set_error(LORA_EINVAL, "lora_pool_adapter_pages: capacity %lld < %lld", (long long)cap, (long long)pg.size());
    std::copy(pg.begin(), pg.end(), out);
    return LORA_OK;
}

extern "C" int lora_pool_kv_pages(const lora_pool *pc, int64_t rid, int64_t *out, int64_t cap, int64_t *n_out) {
    clear_error();
    if (!pc) return set_error(LORA_EINVAL, "lora_pool_kv_pages: pool is NULL");
    lora_pool *p = const_cast<lora_pool *>(pc);
    std::lock_guard<std::mutex> lk(p->mu);
    auto it = p->kv.find(rid);
    if (it == p->kv.end()) return set_error(LORA_ENOENT, "lora_pool_kv_pages: request %lld holds no KV pages", (long long)rid);
    const auto &pg = it->second;
    if (n_out) *n_out = (int64_t)pg.size();
    if ((int64_t)pg.size() > cap || !out)
        return set_error(LORA_EINVAL, "lora_pool_kv_pages: capacity %lld < %lld", (long long)cap, (long long)pg.size());
    std::copy(pg.begin(), pg.end(), out);
    return LORA_OK;
}

extern "C" int lora_pool_free_list(const lora_pool *pc, int64_t *out, int64_t cap, int64_t *n_out) {
    clear_error();
    if (!pc) return set_error(LORA_EINVAL, "lora_pool_free_list: pool is NULL");
    lora_pool *p = const_cast<lora_pool *>(pc);
    std::lock_guard<std::mutex> lk(p->mu);
    if (n_out) *n_out = (int64_t)p->free_list.size();
    if ((int64_t)p->free_list.size() > cap || (!out && !p->free_list.empty()))
        return set_error(LORA_EINVAL, "lora_pool_free_list: capacity %lld < %lld", (long long)cap,
                         (long long)p->free_list.size());
    std::copy(p->free_list.begin(), p->free_list.end(), out);
    return LORA_OK;
}

extern "C" int lora_pool_resident(const lora_pool *pc, int32_t *out, int32_t cap, int32_t *n_out) {
    clear_error();
    if (!pc) return set_error(LORA_EINVAL, "lora_pool_resident: pool is NULL");
    lora_pool *p = const_cast<lora_pool *>(pc);
    std::lock_guard<std::mutex> lk(p->mu);
    if (n_out) *n_out = (int32_t)p->load_order.size();
    if ((int32_t)p->load_order.size() > cap || (!out && !p->load_order.empty()))
        return set_error(LORA_EINVAL, "lora_pool_resident: capacity %d < %d", cap, (int)p->load_order.size());
    std::copy(p->load_order.begin(), p->load_order.end(), out);
    return LORA_OK;
}
