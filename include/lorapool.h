/*
 * lorapool.h -- unmerged multi-LoRA projection over a unified page pool, for AMD Instinct MI355X
 * (gfx950).  Plain C ABI: opaque pool handle, plain pointers and sizes, int status codes.
 *
 * What it computes ("S-LoRA, in depth", section "Merge or keep adapters separate"): a LoRA adapter
 * turns an h-by-h weight W into W + AB with A h-by-r and B r-by-h; a token with activation x gets
 * xW + (xA)B.  Unmerged serving keeps W shared, batches xW over every token whatever its adapter,
 * and adds the low-rank term per token.  This library computes, for T tokens in one call,
 *
 *     y[t] = x[t] W + s[a] * (x[t] A_a) B_a        a = adapter_ids[t]
 *
 * and y[t] = x[t] W when a == -1 or the adapter has rank 0 (the weightless "identity" adapter of
 * "Switch Adapters by Routing Requests Through Resident, Verified State", its adapter registry).
 * The per-adapter float scale s[a] is this library's reading of the usual LoRA scaling; s = 1
 * gives the page's formula.
 *
 * Where A and B live ("S-LoRA, in depth", section "Unified paging: adapters and KV cache in one
 * pool"): a pool of pages, each one vector of H elements, shared by KV cache and adapters through
 * one free list.  An adapter of rank r on one projection takes 2r pages: the r columns of A and
 * the r rows of B.  Pages need not be contiguous or in order; a per-projection page table maps
 * (adapter, j) to a page, and the projection's gather fetches each token's pages from wherever the
 * pool placed them (same page, section "The architecture").
 *
 * Conventions for every function returning int:
 *   0 = LORA_OK, negative = error (below).  No C++ exception crosses this boundary.  On error,
 *   lora_last_error() returns a message for the calling thread, valid until its next call.
 *   Arguments are validated on the host before any device work; an invalid call leaves every
 *   caller buffer untouched.
 * Streams: `stream` arguments are hipStream_t values passed as void* (NULL = the null stream).
 *   All device work of a call is enqueued on that stream, in call order, so a load followed by a
 *   projection on the same stream sees the new weights.  Ordering across streams is the caller's
 *   job (events).
 * Memory ownership: the caller owns every device buffer (pool pages, page table, x, W, y, ids,
 *   ranks, scales, workspace).  The library owns only host bookkeeping plus two small device
 *   buffers it allocates at pool creation (a staging buffer for loads and a device error word),
 *   freed by lora_pool_free.
 * Threads: calls that change a pool (load, release, evict, KV) take the pool's mutex.
 *   lora_project changes no pool state and holds no "active adapter": adapter choice is per token,
 *   carried by adapter_ids (the routing page's warning against a shared mutable active adapter).
 */
#ifndef LORAPOOL_H
#define LORAPOOL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum lora_status {
    LORA_OK = 0,
    LORA_EINVAL = -1,   /* bad argument: null/misaligned pointer, size, dtype, range            */
    LORA_ENOMEM = -2,   /* not enough free pages (or a library allocation failed)              */
    LORA_ENOENT = -3,   /* unknown adapter / request id                                        */
    LORA_ERANK = -4,    /* rank out of range, or not the rank the adapter was loaded at        */
    LORA_EBUSY = -5,    /* adapter still has users                                             */
    LORA_EEXIST = -6,   /* adapter already resident at another rank                            */
    LORA_EHIP = -7,     /* a HIP runtime call failed (message has the HIP error string)        */
    LORA_EDEVICE = -8   /* an earlier projection found bad ids/ranks/pages on the device       */
};

enum lora_dtype {
    LORA_F32 = 0,       /* pages, x, W, A, B, y in IEEE float32                                 */
    LORA_BF16 = 1       /* ... in bfloat16; products accumulate in float32                      */
};

enum lora_victim_rule {         /* which idle adapter a load that is short of pages evicts first */
    LORA_VICTIM_LOAD_ORDER = 0, /* oldest load first: the pool sketch's rule (the default)        */
    LORA_VICTIM_LRU = 1,        /* least recently admitted first                                  */
    LORA_VICTIM_FARTHEST = 2    /* next request in the lookahead farthest first (Belady's rule);
                                   adapters beyond the lookahead last-admitted-longest-ago first  */
};

#define LORA_MAX_RANK 64        /* largest rank a pool can be created for                       */
#define LORA_MAX_ADAPTERS 8192  /* largest adapter id + 1                                       */
#define LORA_MAX_TOKENS (1 << 22) /* most tokens (T) one projection call takes                  */

typedef struct lora_pool lora_pool;

typedef struct lora_pool_stats {
    int64_t num_pages;          /* pool size                                                    */
    int64_t free_pages;         /* on the free list                                             */
    int64_t kv_pages;           /* held by KV requests                                          */
    int64_t adapter_pages;      /* held by resident adapters                                    */
    int32_t resident_adapters;  /* adapters holding pages (rank-0 adapters count, with 0 pages) */
    int32_t idle_adapters;      /* resident adapters with no users                              */
    int64_t kv_requests;        /* requests holding KV pages                                    */
    int64_t loads;              /* adapter loads that allocated pages (not refcount bumps)      */
    int64_t evictions;          /* adapters whose pages were reclaimed                          */
    int64_t bytes_loaded;       /* bytes copied into pages by loads                             */
} lora_pool_stats_t;

/* ---- pool lifecycle ("Unified paging" section and its pool sketch) ------------------------- */

/*
 * Create a pool over caller-owned device memory.
 *   pages        device, num_pages * hidden elements of `dtype`, 16-byte aligned.  Page p is the
 *                hidden-element vector at pages + p * hidden.
 *   num_pages    >= 1.
 *   hidden       H, the page length and the projection's input and output width; a multiple of
 *                64, 64 <= H <= 65536.
 *   dtype        LORA_F32 or LORA_BF16.
 *   max_rank     1..LORA_MAX_RANK; every adapter's rank must be <= max_rank.
 *   n_slots      projections per adapter (layers * projections, e.g. 32 * 4 for q/k/v/o of a
 *                7B model); each slot has its own page-table block.
 *   max_adapters adapter ids are 0..max_adapters-1 (<= LORA_MAX_ADAPTERS).
 *   page_table   device int32 [n_slots][max_adapters][2*max_rank], caller-owned, 4-byte aligned.
 *                Row (slot, a) lists adapter a's pages for that slot: entries 0..r-1 the columns
 *                of A, r..2r-1 the rows of B, -1 after that.  The library writes it (set to -1
 *                here, synchronously); callers only read it.
 *   free_order   host int64 [num_pages], a permutation of 0..num_pages-1 giving the initial free
 *                list, or NULL for 0..num_pages-1.  Allocation takes pages from the END of the
 *                list and frees append to it (the sketch's pop and extend), so the default hands
 *                out num_pages-1 first.
 *   out          receives the handle.
 * pages and page_table may both be NULL: a bookkeeping-only pool that allocates and accounts
 * pages but touches no device memory (loads copy nothing; projections are refused).
 * Errors: LORA_EINVAL (bad argument, free_order not a permutation), LORA_EHIP.
 */
int lora_pool_create(void *pages, int64_t num_pages, int32_t hidden, int32_t dtype,
                     int32_t max_rank, int32_t n_slots, int32_t max_adapters, int32_t *page_table,
                     const int64_t *free_order, lora_pool **out);

/* Destroy the pool's bookkeeping and library-owned device buffers; waits for the pool's pending
 * loads first.  Caller buffers are untouched.  NULL is accepted.  Returns LORA_OK or LORA_EHIP. */
int lora_pool_free(lora_pool *pool);

/*
 * Make adapter `adapter_id` resident at `rank` (0..max_rank), as the sketch's ensure_adapter:
 *   - already resident at the same rank: one more user (refcount + 1); nothing is copied;
 *   - already resident at another rank: LORA_EEXIST;
 *   - otherwise it needs 2 * rank * n_slots pages; if fewer are free, idle adapters (no users)
 *     are evicted oldest-load first until enough are free; if even that is not enough the call
 *     returns LORA_ENOMEM with no pages taken (idle adapters evicted on the way stay evicted,
 *     as in the sketch).  On success the adapter has one user.
 * The adapter's page list takes pages from the free list in order; list entry i belongs to slot
 * i / (2r), entry i % (2r) of that slot's table row.
 *   A_t  [n_slots][rank][hidden] of the pool dtype: row j of slot s is column j of that slot's A.
 *   B    [n_slots][rank][hidden]: row j of slot s is row j of that slot's B.
 * A_t and B may be host (pageable or pinned) or device memory; they are read during the call
 * for pageable memory and, otherwise, by work on `stream`: keep them alive and unchanged until
 * the stream has passed this call.  Both may be NULL when rank == 0 or the pool is
 * bookkeeping-only.  The copies and the page-table update are enqueued on `stream`, so with
 * pinned memory and a stream of its own a load overlaps projections on other streams (section
 * "Scheduling: prefetch, clustering and early abort"); make the first projection that uses the
 * adapter wait for `stream` (an event).  Host rows are staged through one of two load buffers per
 * pool: the call waits on the host only while the load two calls earlier is still queued.
 * Errors: LORA_EINVAL, LORA_ERANK (rank > max_rank), LORA_EEXIST, LORA_ENOMEM, LORA_EHIP.
 */
int lora_pool_load_adapter(lora_pool *pool, int32_t adapter_id, int32_t rank, const void *A_t,
                           const void *B, void *stream);

/* Choose the victim rule for idle-adapter eviction (enum lora_victim_rule).  The pool sketch of
 * "S-LoRA, in depth" (section "Unified paging") evicts idle adapters in load order; the MoE-offload
 * page ("Cache the Experts You Will Need", sections "A better eviction rule cuts transfers without
 * changing routing" and "Limited foresight") compares least-recently-used eviction with evicting the
 * entry whose next request lies farthest ahead, given a window of upcoming requests.  A "use" is a
 * call of lora_pool_load_adapter that names the adapter (resident or not).  Errors: LORA_EINVAL. */
int lora_pool_set_victim_rule(lora_pool *pool, int32_t rule);

/* The upcoming adapter requests the farthest-future rule looks at: `n` host ids, soonest first (for
 * a scheduler, its waiting queue).  Copied; n == 0 clears it.  Adapters that do not occur count as
 * needed after every one that does.  Errors: LORA_EINVAL (n < 0, or ids NULL with n > 0). */
int lora_pool_set_lookahead(lora_pool *pool, const int32_t *adapter_ids, int64_t n);

/* One user of the adapter finished (refcount - 1).  At zero users it stays resident but idle and
 * becomes evictable.  Errors: LORA_ENOENT (not resident), LORA_EINVAL (already idle). */
int lora_pool_release_adapter(lora_pool *pool, int32_t adapter_id);

/* Reclaim an idle adapter's pages (section "The architecture": an adapter that no active request
 * uses may give its pages back): they return to the end of the free list in page-list
 * order, and the adapter's page-table rows are reset to -1 on `stream`.  The caller must not
 * evict an adapter that queued, unfinished projections still read.
 * Errors: LORA_ENOENT, LORA_EBUSY (has users). */
int lora_pool_evict_adapter(lora_pool *pool, int32_t adapter_id, void *stream);

/* Grow request `request_id`'s KV cache by one token: 2 * layers pages (K and V per layer), as the
 * sketch's grow_kv.  If page_ids_out is not NULL it receives the 2*layers page ids (host int64).
 * Errors: LORA_ENOMEM (no room: the caller has to stop or cut short some request to make room),
 * LORA_EINVAL. */
int lora_pool_grow_kv(lora_pool *pool, int64_t request_id, int32_t layers, int64_t *page_ids_out);

/* Request finished: its KV pages return to the end of the free list.  Errors: LORA_ENOENT. */
int lora_pool_free_kv(lora_pool *pool, int64_t request_id);

/* ---- queries (host only, no device work) ----------------------------------------------------- */

/* Pages for an adapter of `rank` on `projections` projections of `layers` layers:
 * rank * 2 * projections * layers (A and B per projection).  Negative input gives -1. */
int64_t lora_pool_pages_for(int32_t rank, int32_t projections, int32_t layers);

/* KV pages one token takes: 2 * layers (K and V per layer).  Negative input gives -1. */
int64_t lora_kv_pages_per_token(int32_t layers);

int lora_pool_stats(const lora_pool *pool, lora_pool_stats_t *out);

/* Device pointer to `slot`'s page-table block [max_adapters][2*max_rank] and its row stride in
 * elements (2*max_rank).  Errors: LORA_EINVAL (slot out of range, bookkeeping-only pool). */
int lora_pool_page_table(const lora_pool *pool, int32_t slot, const int32_t **table,
                         int32_t *row_stride);

/* Copy adapter `adapter_id`'s page list (2 * rank * n_slots ids, in list order) into out[cap];
 * *n_out = its length, *rank_out = its rank, *users_out = its refcount (each may be NULL).
 * Errors: LORA_ENOENT, LORA_EINVAL (cap too small: *n_out still set). */
int lora_pool_adapter_pages(const lora_pool *pool, int32_t adapter_id, int64_t *out, int64_t cap,
                            int64_t *n_out, int32_t *rank_out, int32_t *users_out);

/* Copy request `request_id`'s KV page list into out[cap]; *n_out = its length.
 * Errors: LORA_ENOENT, LORA_EINVAL (cap too small). */
int lora_pool_kv_pages(const lora_pool *pool, int64_t request_id, int64_t *out, int64_t cap,
                       int64_t *n_out);

/* Copy the free list (front to end; allocation takes from the end) into out[cap]. */
int lora_pool_free_list(const lora_pool *pool, int64_t *out, int64_t cap, int64_t *n_out);

/* Resident adapter ids in load order (oldest first), the order idle eviction follows. */
int lora_pool_resident(const lora_pool *pool, int32_t *out, int32_t cap, int32_t *n_out);

/* ---- the projection --------------------------------------------------------------------------- */

/* Bytes of device workspace lora_project needs for T tokens on this pool (256-byte aligned). */
size_t lora_project_workspace_size(const lora_pool *pool, int64_t T);

/*
 * y = x W + s * (x A) B for T tokens, each on its own adapter (sections "Merge or keep adapters
 * separate" and "The architecture" of "S-LoRA, in depth").
 *   x            device [T][H], pool dtype, row-major, 16-byte aligned.
 *   W            device [H][H], pool dtype, OUT-MAJOR: element (k, n) of W (input k, output n)
 *                is W[n * H + k] -- the layout of a linear layer's weight matrix.  16-byte aligned.
 *   page_table   device: one slot's block [max_adapters][2*max_rank] (lora_pool_page_table).
 *   adapter_ids  device int32 [T]: adapter per token, -1 = none.
 *   ranks        device int32 [max_adapters]: rank per adapter; must equal the loaded rank for
 *                every adapter a token uses (entries of unused adapters are not read).
 *   scale        device float32 [max_adapters]: s per adapter.
 *   y            device [T][H], pool dtype, 16-byte aligned; must not overlap x.  Each element is
 *                accumulated in float32 (base and low-rank parts together) and rounded once to the
 *                pool dtype (round to nearest even).
 *   workspace    device, >= lora_project_workspace_size(pool, T) bytes, 256-byte aligned; its
 *                contents on entry do not matter.  Calls that share a workspace must be ordered
 *                (same stream, or events).
 * T == 0 is a no-op; T above LORA_MAX_TOKENS is LORA_EINVAL.  Ids, ranks and page ids are checked on the device: a token whose adapter id
 * is out of range, whose rank is out of range or differs from the page table, or whose page ids
 * are out of range gets the base product only, and the pool's device error word records the
 * fault; lora_check_device_errors() reports and clears it.
 * Errors (host-side, before any device work): LORA_EINVAL, LORA_EHIP.
 */
int lora_project(lora_pool *pool, const void *x, const void *W, const int32_t *page_table,
                 const int32_t *adapter_ids, const int32_t *ranks, const float *scale, int64_t T,
                 void *y, void *workspace, size_t workspace_bytes, void *stream);

#define LORA_MAX_CALL_SLOTS 4   /* most slots one lora_project_slots call takes                    */

/* Bytes of device workspace lora_project_slots needs for n slots and T tokens (0 if n is out of
 * range): n times lora_project_workspace_size. */
size_t lora_project_slots_workspace_size(const lora_pool *pool, int32_t n, int64_t T);

/*
 * The projection for n (1..LORA_MAX_CALL_SLOTS) slots that share the same tokens: the q, k and v
 * projections of a layer read one x ("S-LoRA, in depth": an adapter has A and B for each of the
 * projections of each layer, and the base product is batched over all tokens).  For each z < n,
 *     y[z][t] = x[t] W[z] + s[a] * (x[t] A_{slots[z],a}) B_{slots[z],a},    a = adapter_ids[t],
 * exactly what lora_project gives for that slot (bit for bit: every sum runs in the same order).
 * One call groups the tokens once and launches each stage once for all n slots, so the base
 * GEMM's tiles of the n slots share the chip (better load balance than n calls).
 *   slots        host int32 [n], distinct or not, each in [0, n_slots); page tables are the pool's
 *   W, y         host arrays of n device pointers, as lora_project's W and y; no two outputs may
 *                overlap each other or x
 *   workspace    >= lora_project_slots_workspace_size(pool, n, T) bytes, 256-byte aligned: n regions
 *                of lora_project_workspace_size(pool, T) bytes, region z for the z-th slot
 * The rest as lora_project.  Float32 pools run the slots one after another.
 * Errors (host-side, before any device work): LORA_EINVAL, LORA_EHIP.  Device checks as
 * lora_project, with one difference for T > 256 (the prefill path, whose grouping serves every
 * slot): an adapter whose page-table row is bad in any slot of the call gets the base product
 * only, in every slot of the call.
 */
int lora_project_slots(lora_pool *pool, int32_t n, const int32_t *slots, const void *x,
                       const void *const *W, const int32_t *adapter_ids, const int32_t *ranks,
                       const float *scale, int64_t T, void *const *y, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * lora_project_slots where each slot reads its own input rows: x is a host array of n device
 * pointers (each as lora_project's x; slots may share one).  The q, k, v and o projections of a layer
 * act on the same tokens but o reads the attention output, not the layer input ("S-LoRA, in depth":
 * an adapter has A and B for each of the projections of each layer); with this call all four go in
 * one launch per stage, so their tiles share the chip.  For each z < n,
 *     y[z][t] = x[z][t] W[z] + s[a] * (x[z][t] A_{slots[z],a}) B_{slots[z],a},   a = adapter_ids[t],
 * bit for bit what lora_project gives for that slot.  No output may overlap any input or another
 * output.  Workspace, errors and device checks as lora_project_slots.
 */
int lora_project_slots_x(lora_pool *pool, int32_t n, const int32_t *slots, const void *const *x,
                         const void *const *W, const int32_t *adapter_ids, const int32_t *ranks,
                         const float *scale, int64_t T, void *const *y, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * The projection with its own indices exposed ("S-LoRA, in depth", section "The architecture": the
 * gather fetches each request's A and B pages from wherever the pool placed them).  Runs exactly the
 * kernels lora_project runs for these arguments -- in instantiations that also record the indices
 * they use -- and writes y bit for bit as lora_project does.  In addition (device int32, caller-owned,
 * 4-byte aligned, filled with -1 by the call first):
 *   gather_out   [T][2*max_rank], input token order: entry j < r is the page whose A column the
 *                shrink multiplied into token t's v[j]; entry r + j the page whose B row the expand
 *                multiplied into token t's y; -1 elsewhere (no adapter, rank 0, past the rank).  An
 *                entry that two workgroups or kernels filled with different pages reads -2.
 *   order_out    [T][2], per sorted position q (the grouping the kernels consumed): the token at q
 *                and the adapter of its segment.  T <= 256 (bfloat16): every token, the ones with a
 *                low-rank term first, grouped by adapter (segments by ceil(r / 16) from 4 down to 1,
 *                then by first token), then the others with adapter -1.  Otherwise: positions
 *                [0, n) hold the n tokens with a low-rank term, grouped by adapter in adapter
 *                order; the rest stay (-1, -1).
 * Other arguments, checks and errors as lora_project.  For tests and debugging; not a fast path.
 */
int lora_debug_project(lora_pool *pool, const void *x, const void *W, const int32_t *page_table,
                       const int32_t *adapter_ids, const int32_t *ranks, const float *scale, int64_t T,
                       void *y, void *workspace, size_t workspace_bytes, int32_t *gather_out,
                       int32_t *order_out, void *stream);

/*
 * Page-table view of the gather (no projection): for every token t (input order) writes the table
 * entries its adapter owns into page_ids_out[t][0..2*max_rank) (device int32): entries 0..r-1 its A
 * columns, r..2r-1 its B rows, -1 elsewhere and for tokens with no adapter or rank 0.  Same inputs
 * and device checks as lora_project (an invalid token gets all -1).  Enqueued on `stream`.  The
 * pages the projection's kernels themselves read come from lora_debug_project.
 */
int lora_debug_gather(lora_pool *pool, const int32_t *page_table, const int32_t *adapter_ids,
                      const int32_t *ranks, int64_t T, int32_t *page_ids_out, void *stream);

/*
 * lora_project for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  No workspace argument: the call uses a scratch
 * array of LORA_NOALLOC_SCRATCH_MB MiB that the library holds on each GPU it runs on until the
 * process ends (its address is taken at pool creation).  It allocates nothing and writes y exactly as
 * lora_project does.  Calls that need more scratch than that (lora_project_workspace_size) are refused
 * with LORA_EINVAL before any device work: at H = 4096 every decode batch (T <= 256) and prefill
 * batches up to about 25k tokens fit.  Every call on a GPU shares that GPU's array: calls that overlap
 * on one GPU (several streams or threads without ordering between them) race and may produce wrong
 * results; order them.  Other arguments, checks and errors as lora_project.
 */
#define LORA_NOALLOC_SCRATCH_MB 32
int lora_project_noalloc(lora_pool *pool, const void *x, const void *W, const int32_t *page_table,
                         const int32_t *adapter_ids, const int32_t *ranks, const float *scale, int64_t T,
                         void *y, void *stream);

/* Wait for all device work, then report and clear the pool's device error word:
 * LORA_OK, or LORA_EDEVICE with a message naming the kinds of fault seen. */
int lora_check_device_errors(lora_pool *pool);

/* ---- per-kernel timing (opt-in, for measurement) ---------------------------------------------- */

typedef struct lora_profile {
    int64_t calls;              /* projections recorded                                          */
    double ms_group;            /* summed device time of the token-grouping kernel (prefill and
                                   float32 paths; the decode path groups inside its first kernel) */
    double ms_first;            /* ... of the first compute launch: decode = shrink + base GEMM
                                   partials; prefill and float32 = shrink                          */
    double ms_second;           /* ... of the second: decode = partial sum + expand + rounding;
                                   prefill and float32 = base GEMM + fused expand                  */
} lora_profile_t;

/* Start recording HIP events around each kernel of the next `max_calls` projections on this
 * pool, on the stream each kernel is launched on.  Recording adds event records between the
 * kernels; time the throughput without it.  Errors: LORA_EINVAL, LORA_EHIP. */
int lora_profile_start(lora_pool *pool, int32_t max_calls);

/* Wait for the recorded work, fill *out with per-kernel sums, and stop recording. */
int lora_profile_stop(lora_pool *pool, lora_profile_t *out);

/* Message for the calling thread's last error ("" if none). */
const char *lora_last_error(void);

/* Library version string. */
const char *lora_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LORAPOOL_H */
