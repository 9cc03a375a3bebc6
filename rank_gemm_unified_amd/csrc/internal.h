// Library-internal declarations shared by the host code and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <deque>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/lorapool.h"

namespace lorapool {

// ---- errors -------------------------------------------------------------------------------------
int set_error(int code, const char *fmt, ...);
int hip_error(hipError_t e, const char *what);
#define LP_HIP(call)                                        \
    do {                                                    \
        hipError_t e_ = (call);                             \
        if (e_ != hipSuccess) return hip_error(e_, #call);  \
    } while (0)

// device error word bits (set by the kernels, reported by lora_check_device_errors)
enum : int {
    DEV_ERR_ID = 1,        // adapter id < -1 or >= max_adapters
    DEV_ERR_RANK = 2,      // ranks[a] < 0 or > max_rank
    DEV_ERR_TABLE = 4,     // page-table row does not hold exactly 2*ranks[a] pages
    DEV_ERR_PAGE = 8,      // page id outside [0, num_pages)
};

// ---- the pool ----------------------------------------------------------------------------------
struct Adapter {
    int32_t rank = 0;
    int32_t users = 0;
    int64_t last_use = 0;         // admission tick of the latest load call that named it
    std::vector<int64_t> pages;   // 2 * rank * n_slots, list order
};

}  // namespace lorapool

struct lora_pool {
    std::mutex mu;
    // geometry (immutable after create)
    void *pages = nullptr;
    int64_t num_pages = 0;
    int32_t hidden = 0;
    int32_t dtype = 0;
    int32_t elem = 0;
    int32_t max_rank = 0;
    int32_t n_slots = 0;
    int32_t max_adapters = 0;
    int32_t *page_table = nullptr;
    bool bookkeeping_only = false;
    int device = 0;
    // bookkeeping
    std::vector<int64_t> free_list;                        // allocation pops from the back
    std::unordered_map<int32_t, lorapool::Adapter> adapters;
    std::vector<int32_t> load_order;                       // resident ids, oldest first
    int32_t victim_rule = LORA_VICTIM_LOAD_ORDER;          // which idle adapter goes first
    std::vector<int32_t> lookahead;                        // upcoming adapter requests, soonest first
    int64_t tick = 0;                                      // admissions so far
    std::unordered_map<int64_t, std::vector<int64_t>> kv;
    int64_t kv_total = 0, adapter_total = 0;
    int64_t n_loads = 0, n_evictions = 0, bytes_loaded = 0;
    // library-owned device/host buffers: a ring of LOAD_RING load buffers, so that a load waits (on
    // the host) only for the load LOAD_RING calls earlier, never for the one just before it
    static constexpr int LOAD_RING = 2;
    struct LoadBuf {
        void *staging = nullptr;      // device, staging_bytes
        int32_t *rows_dev = nullptr;  // device, n_slots * 2 * max_rank int32
        int32_t *rows_host = nullptr; // pinned host, same size
        hipEvent_t done = nullptr;    // recorded after the load that last used this buffer
    };
    LoadBuf load_buf[LOAD_RING];
    int load_next = 0;
    size_t staging_bytes = 0;
    int *dev_err = nullptr;           // device error word
    // opt-in per-kernel timing: 4 events per recorded call
    std::vector<hipEvent_t> prof_events;
    std::atomic<int32_t> prof_next{0};
    int32_t prof_max = 0;
};

namespace lorapool {

// ---- workspace plan ----------------------------------------------------------------------------
enum PathKind : int { PATH_DECODE = 0, PATH_PREFILL = 1, PATH_F32 = 2 };

struct Plan {
    PathKind path;
    int64_t T;
    int32_t chunk;          // tokens per shrink work item
    int32_t n_items_max;    // bound on shrink work items
    int32_t vsplit;         // K-splits of the shrink (partial v buffers)
    int32_t ysplit;         // K-splits of the decode base GEMM
    int32_t n_tiles;        // decode: 64-column tiles
    int32_t mb;             // decode: 16-row blocks per wave
    int32_t rp;             // row stride of v and per-token page lists (max_rank rounded up to 16)
    int32_t stream;         // decode: 1 = k_decode_stream (T <= 64), 0 = k_decode_wide
    int32_t ks;             // decode streaming kernel: max K steps of 32 per wave (a quarter of a split)
    // byte offsets into the workspace
    size_t off_tok_a, off_tok_r, off_perm, off_seg_a, off_seg_start, off_item_seg, off_item_row, off_item_rec,
        off_ctrl, off_v, off_ypart, off_sorted_tok, off_v16, off_spages, total;
};

bool make_plan(const lora_pool *p, int64_t T, Plan *plan);

struct Ws {
    int32_t *tok_a, *tok_r, *perm, *seg_a, *seg_start, *item_seg, *item_row, *ctrl;
    int4 *item_rec;         // prefill: per shrink work item {adapter, rank, first sorted row, rows}; adapter -1 past the last
    float *v, *ypart;
    int32_t *sorted_tok;    // decode: int4 {token, adapter or -1, rank, 0} per sorted position
    uint16_t *v16;          // prefill: v = s x A in bfloat16, [T][rp]
    int32_t *spages;        // decode: B page ids per sorted position, [T][rp]
};
Ws carve(void *base, const Plan &plan);

// Per-slot pointers of one call: up to MAX_CALL_SLOTS slots that share the tokens and their adapter
// ids (the q, k, v and o projections of a layer; q, k and v also share x).  The argument of the several-slot kernels, indexed
// by blockIdx.z (a one-slot call launches the one-slot kernels, whose arguments are the slot's
// pointers themselves); the token grouping of the prefill path lives in slot 0's workspace region
// and serves every slot.
constexpr int MAX_CALL_SLOTS = 4;
struct SlotPtrs {
    const void *x[MAX_CALL_SLOTS];       // the slot's input rows (slots may share one)
    const void *W[MAX_CALL_SLOTS];
    void *y[MAX_CALL_SLOTS];
    const int32_t *pt[MAX_CALL_SLOTS];   // the slot's page table [max_adapters][2 max_rank]
    float *v[MAX_CALL_SLOTS];            // workspace regions, one per slot
    uint16_t *v16[MAX_CALL_SLOTS];
    float *ypart[MAX_CALL_SLOTS];
    int32_t *sorted_tok[MAX_CALL_SLOTS];
    int32_t *spages[MAX_CALL_SLOTS];
};
struct SlotRows {   // the page tables alone (the grouping kernel checks every slot's rows)
    const int32_t *pt[MAX_CALL_SLOTS];
};

// Outputs of the debug instantiations of the kernels (lora_debug_project): every kernel that reads a
// page for a token records the page id where it uses it, and the kernels that consume the token
// grouping record it.  Both buffers are filled with -1 before the launches.
struct DebugOut {
    int32_t *gather;   // [T][2 max_rank], token order: A pages 0..r-1, B pages r..2r-1
    int32_t *order;    // [T][2]: per sorted position, the token and its segment's adapter (-1: none)
};

// ctrl[] slots written by the segment kernel
enum : int { CTRL_NSEG = 0, CTRL_NITEMS = 1, CTRL_NVALID = 2, CTRL_WORDS = 64 };

// ---- launchers (kernels in k_*.hip) -------------------------------------------------------------
hipError_t launch_write_rows(int32_t *page_table, int32_t max_adapters, int32_t row_stride,
                             int32_t adapter, const int32_t *rows, int32_t n_slots,
                             hipStream_t s);
hipError_t launch_clear_rows(int32_t *page_table, int32_t max_adapters, int32_t row_stride,
                             int32_t adapter, int32_t n_slots, hipStream_t s);
hipError_t launch_scatter_rows(void *pages, int32_t hidden, int32_t elem, const void *A_t,
                               const void *B, int64_t src_slot_stride_elems, int32_t slot0,
                               int32_t n_slots_chunk, int32_t rank, const int32_t *rows,
                               int32_t row_stride, hipStream_t s);
hipError_t launch_segments(const lora_pool *p, const Plan &plan, const Ws &ws,
                           const int32_t *ids, const int32_t *ranks, const SlotPtrs &sp, int n,
                           hipStream_t s);
hipError_t launch_debug_gather(const lora_pool *p, const int32_t *pt, const int32_t *ids,
                               const int32_t *ranks, int64_t T, int32_t *out, hipStream_t s);
hipError_t launch_decode_wide(const lora_pool *p, const Plan &plan, const void *x, const int32_t *ids,
                              const int32_t *ranks, const float *scale, const SlotPtrs &sp, int n,
                              hipStream_t s, const DebugOut *dbg = nullptr);
hipError_t launch_decode(const lora_pool *p, const Plan &plan, const void *x, const int32_t *ids,
                         const int32_t *ranks, const float *scale, const SlotPtrs &sp, int n, hipStream_t s,
                         hipEvent_t mid, const DebugOut *dbg = nullptr);
hipError_t launch_prefill(const lora_pool *p, const Plan &plan, const Ws &ws, const void *x,
                          const float *scale, const SlotPtrs &sp, int n, hipStream_t s, hipEvent_t mid,
                          const DebugOut *dbg = nullptr);
hipError_t launch_f32(const lora_pool *p, const Plan &plan, const Ws &ws, const void *x,
                      const void *W, const int32_t *pt, const float *scale, void *y,
                      hipStream_t s, hipEvent_t mid, const DebugOut *dbg = nullptr);
hipError_t launch_fill_i32(int32_t *dst, int64_t n, int32_t value, hipStream_t s);

// Address of the allocation-free entry point's scratch array on device `dev`, taken once per device
// (at pool creation).  Returns a lora_status.
int scratch_setup(int dev);

struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
        if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
    }
    ~DeviceGuard() {
        int cur = -1;
        if (ok && hipGetDevice(&cur) == hipSuccess && cur != prev && prev >= 0) (void)hipSetDevice(prev);
    }
};

}  // namespace lorapool
