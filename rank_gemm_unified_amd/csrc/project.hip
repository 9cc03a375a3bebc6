// lora_project: host-side validation, workspace planning and kernel dispatch.
//
// Per call:  segment kernel (validate ids/ranks/pages, group tokens by adapter)
//            -> shrink  v = s * x A        (gathered A columns)
//            -> base + expand  y = x W + v B  (gathered B rows, one rounding)
// Decode-shaped calls (T <= 256) stream W once with a split-K MFMA kernel; prefill-shaped calls
// use the tiled MFMA GEMM.  The choice depends only on T and the dtype, both known on the host.
#include <algorithm>
#include <cstring>
#include <mutex>

#include "internal.h"

using namespace lorapool;

namespace lorapool {

constexpr int64_t MAX_TOKENS = LORA_MAX_TOKENS;
constexpr int64_t DECODE_MAX_T = 256;

static size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

bool make_plan(const lora_pool *p, int64_t T, Plan *pl) {
    if (!p || T < 0 || T > MAX_TOKENS) return false;
    memset(pl, 0, sizeof *pl);
    pl->T = T;
    const int64_t R = p->max_rank, H = p->hidden;
    if (p->dtype == LORA_F32) {
        pl->path = PATH_F32;
    } else if (T <= DECODE_MAX_T) {
        pl->path = PATH_DECODE;
    } else {
        pl->path = PATH_PREFILL;
    }
    pl->chunk = pl->path == PATH_PREFILL ? 64 : 16;
    pl->n_items_max = (int32_t)((T + pl->chunk - 1) / pl->chunk + std::min<int64_t>(T, p->max_adapters));
    pl->vsplit = 1;
    pl->ysplit = 1;
    pl->n_tiles = 0;
    pl->rp = (int32_t)((R + 15) / 16 * 16);
    if (pl->path == PATH_DECODE) {
        const int64_t ksteps = H / 32;
        if (T <= 64 && H <= 8192) {
            // streaming kernel: 64-column tiles x S splits of K, each split cut into four K quarters
            // (one per wave) of at most 8 steps of 32; S grows towards 256 workgroups when H is small
            pl->stream = 1;
            pl->mb = (int32_t)std::max<int64_t>(1, (T + 15) / 16);
            pl->n_tiles = (int32_t)(H / 64);
            int64_t S = std::max<int64_t>(1, (ksteps + 31) / 32);
            while (S < 8 && pl->n_tiles * S < 256 && 4 * (S + 1) <= ksteps) ++S;
            pl->ysplit = (int32_t)S;
            const int64_t q = (ksteps + 4 * S - 1) / (4 * S);
            pl->ks = q <= 1 ? 1 : q <= 2 ? 2 : q <= 4 ? 4 : 8;
        } else {
            // k_decode_wide: 64-column tiles x S splits of K (chunks of 64) towards 256 workgroups;
            // 16-row blocks of tokens (one or two per wave)
            pl->stream = 0;
            pl->mb = T <= 128 ? 8 : 16;
            pl->n_tiles = (int32_t)(H / 64);
            const int64_t nck = H / 64;
            pl->ysplit = (int32_t)std::max<int64_t>(1, std::min<int64_t>({256 / pl->n_tiles, nck, 8}));
        }
    } else if (pl->path == PATH_PREFILL) {
        pl->vsplit = 4;
        pl->n_tiles = 0;
    }
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o += up256(bytes); return at; };
    pl->off_tok_a = take(T * 4);
    pl->off_tok_r = take(T * 4);
    pl->off_perm = take(T * 4);
    pl->off_seg_a = take((T + 1) * 4);
    pl->off_seg_start = take((T + 2) * 4);
    pl->off_item_seg = take((size_t)pl->n_items_max * 4);
    pl->off_item_row = take((size_t)pl->n_items_max * 4);
    pl->off_item_rec = take((size_t)pl->n_items_max * 16);
    pl->off_ctrl = take(CTRL_WORDS * 4);
    const int64_t sv = pl->path == PATH_DECODE ? pl->ysplit : 1;
    pl->off_v = take(pl->path == PATH_F32 ? (size_t)T * R * 4 : (size_t)pl->vsplit * T * pl->rp * sv * 4);
    pl->off_ypart = take(pl->path == PATH_DECODE ? (size_t)pl->ysplit * T * H * 4 : 0);
    pl->off_sorted_tok = take(pl->path == PATH_DECODE ? (size_t)T * 16 : 0);
    pl->off_v16 = take(pl->path == PATH_PREFILL ? (size_t)T * pl->rp * 2 : 0);
    pl->off_spages = take(pl->path == PATH_DECODE ? (size_t)T * pl->rp * 4 : 0);
    pl->total = o;
    return true;
}

Ws carve(void *base, const Plan &pl) {
    char *b = (char *)base;
    Ws w;
    w.tok_a = (int32_t *)(b + pl.off_tok_a);
    w.tok_r = (int32_t *)(b + pl.off_tok_r);
    w.perm = (int32_t *)(b + pl.off_perm);
    w.seg_a = (int32_t *)(b + pl.off_seg_a);
    w.seg_start = (int32_t *)(b + pl.off_seg_start);
    w.item_seg = (int32_t *)(b + pl.off_item_seg);
    w.item_row = (int32_t *)(b + pl.off_item_row);
    w.item_rec = (int4 *)(b + pl.off_item_rec);
    w.ctrl = (int32_t *)(b + pl.off_ctrl);
    w.v = (float *)(b + pl.off_v);
    w.ypart = (float *)(b + pl.off_ypart);
    w.sorted_tok = (int32_t *)(b + pl.off_sorted_tok);
    w.v16 = (uint16_t *)(b + pl.off_v16);
    w.spages = (int32_t *)(b + pl.off_spages);
    return w;
}

static bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

}  // namespace lorapool

extern "C" size_t lora_project_workspace_size(const lora_pool *p, int64_t T) {
    Plan pl;
    if (!make_plan(p, T, &pl)) return 0;
    return pl.total;
}

namespace {

// One call for n slots that share the tokens (ids, ranks, scale), each with its own x, W and y
// (n = 1: lora_project).  The workspace holds n regions of one plan each; the prefill path's token
// grouping lives in region 0 and serves every slot.  Every argument is checked before any device work.
int project_impl(lora_pool *p, const char *fn, int n, const void *const *X, const void *const *W,
                 const int32_t *const *pt, const int32_t *ids, const int32_t *ranks, const float *scale, int64_t T,
                 void *const *y, void *ws, size_t ws_bytes, void *stream, const DebugOut *dbg = nullptr) {
    if (!p) return set_error(LORA_EINVAL, "%s: pool is NULL", fn);
    if (p->bookkeeping_only) return set_error(LORA_EINVAL, "%s: bookkeeping-only pool", fn);
    if (T < 0 || T > MAX_TOKENS)
        return set_error(LORA_EINVAL, "%s: T = %lld not in [0, %lld]", fn, (long long)T, (long long)MAX_TOKENS);
    if (T == 0) return LORA_OK;
    if (!ids || !ranks || !scale || !ws) return set_error(LORA_EINVAL, "%s: NULL pointer argument", fn);
    if (!aligned(ids, 4) || !aligned(ranks, 4) || !aligned(scale, 4) || !aligned(ws, 256))
        return set_error(LORA_EINVAL, "%s: misaligned pointer (x, W, y: 16 B; ids, ranks, scale, page_table: 4 B; "
                                      "workspace: 256 B)", fn);
    const size_t xbytes = (size_t)T * p->hidden * p->elem;
    for (int z = 0; z < n; ++z) {
        if (!X[z] || !W[z] || !pt[z] || !y[z]) return set_error(LORA_EINVAL, "%s: NULL pointer argument", fn);
        if (!aligned(X[z], 16) || !aligned(W[z], 16) || !aligned(y[z], 16) || !aligned(pt[z], 4))
            return set_error(LORA_EINVAL, "%s: misaligned pointer (x, W, y: 16 B; ids, ranks, scale, page_table: 4 B; "
                                          "workspace: 256 B)", fn);
    }
    for (int z = 0; z < n; ++z) {   // no output may overlap an input or another output
        const char *yb = (const char *)y[z];
        for (int u = 0; u < n; ++u) {
            const char *xb = (const char *)X[u];
            if (xb < yb + xbytes && yb < xb + xbytes) return set_error(LORA_EINVAL, "%s: y overlaps x", fn);
        }
        for (int u = 0; u < z; ++u) {
            const char *ub = (const char *)y[u];
            if (ub < yb + xbytes && yb < ub + xbytes) return set_error(LORA_EINVAL, "%s: two outputs overlap", fn);
        }
    }
    Plan pl;
    make_plan(p, T, &pl);
    if (ws_bytes < pl.total * (size_t)n)
        return set_error(LORA_EINVAL, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, pl.total * (size_t)n);
    // k_decode_wide with several slots: the slots already fill the chip, so each takes fewer K splits
    // (towards 256 workgroups in all).  Every workgroup then pays its fixed costs (the grouping, the
    // unit setup, the first loads) over a longer K range, and the finish reads fewer partials: at
    // 256 tokens, H = 4096 and four slots, one split instead of four, 178 -> 145 us per call.  Sums
    // over K then run in another order than in a one-slot call: the results agree with one call per
    // slot up to one rounding step, and a call of a given shape is still bitwise reproducible.  The
    // buffers were sized for the plan's larger split count.
    if (pl.path == PATH_DECODE && !pl.stream && n > 1)
        pl.ysplit = std::max<int32_t>(1, std::min<int32_t>(pl.ysplit, 256 / (pl.n_tiles * n)));
    DeviceGuard g(p->device);
    if (!g.ok) return set_error(LORA_EHIP, "%s: cannot select the pool's device", fn);
    hipStream_t s = (hipStream_t)stream;
    SlotPtrs sp{};
    for (int z = 0; z < MAX_CALL_SLOTS; ++z) {
        const int k = z < n ? z : 0;
        const Ws wz = carve((char *)ws + (size_t)k * pl.total, pl);
        sp.x[z] = X[k];
        sp.W[z] = W[k];
        sp.y[z] = y[k];
        sp.pt[z] = pt[k];
        sp.v[z] = wz.v;
        sp.v16[z] = wz.v16;
        sp.ypart[z] = wz.ypart;
        sp.sorted_tok[z] = wz.sorted_tok;
        sp.spages[z] = wz.spages;
    }
    const Ws w0 = carve(ws, pl);
    if (dbg) {   // the debug outputs start at -1: kernels record only what they use
        hipError_t e = launch_fill_i32(dbg->gather, T * 2 * p->max_rank, -1, s);
        if (e == hipSuccess) e = launch_fill_i32(dbg->order, 2 * T, -1, s);
        if (e != hipSuccess) return hip_error(e, "debug output fill");
    }
    hipEvent_t *ev = nullptr;
    if (p->prof_max > 0) {
        const int32_t slot = p->prof_next.fetch_add(1);
        if (slot < p->prof_max) ev = &p->prof_events[(size_t)slot * 4];
    }
    if (ev) LP_HIP(hipEventRecord(ev[0], s));
    hipError_t e = hipSuccess;
    if (pl.path != PATH_DECODE) {   // the decode path groups tokens inside its first kernel
        e = launch_segments(p, pl, w0, ids, ranks, sp, n, s);
        if (e != hipSuccess) return hip_error(e, "segment kernel launch");
    }
    if (ev) LP_HIP(hipEventRecord(ev[1], s));
    switch (pl.path) {
        case PATH_DECODE: e = launch_decode(p, pl, X[0], ids, ranks, scale, sp, n, s, ev ? ev[2] : nullptr, dbg); break;
        case PATH_PREFILL: e = launch_prefill(p, pl, w0, X[0], scale, sp, n, s, ev ? ev[2] : nullptr, dbg); break;
        case PATH_F32: e = launch_f32(p, pl, w0, X[0], W[0], pt[0], scale, y[0], s, ev ? ev[2] : nullptr, dbg); break;
    }
    if (e != hipSuccess) return hip_error(e, "projection kernel launch");
    if (ev) LP_HIP(hipEventRecord(ev[3], s));
    return LORA_OK;
}

}  // namespace

extern "C" int lora_project(lora_pool *p, const void *x, const void *W, const int32_t *pt, const int32_t *ids,
                            const int32_t *ranks, const float *scale, int64_t T, void *y, void *ws,
                            size_t ws_bytes, void *stream) {
    return project_impl(p, "lora_project", 1, &x, &W, &pt, ids, ranks, scale, T, &y, ws, ws_bytes, stream);
}

extern "C" size_t lora_project_slots_workspace_size(const lora_pool *p, int32_t n, int64_t T) {
    if (n < 1 || n > MAX_CALL_SLOTS) return 0;
    Plan pl;
    if (!make_plan(p, T, &pl)) return 0;
    return pl.total * (size_t)n;
}

namespace {
int project_slots_impl(lora_pool *p, const char *fn, int32_t n, const int32_t *slots, const void *const *X,
                       const void *const *W, const int32_t *ids, const int32_t *ranks, const float *scale, int64_t T,
                       void *const *y, void *ws, size_t ws_bytes, void *stream) {
    if (!p) return set_error(LORA_EINVAL, "%s: pool is NULL", fn);
    if (n < 1 || n > MAX_CALL_SLOTS) return set_error(LORA_EINVAL, "%s: n = %d not in [1, %d]", fn, n, MAX_CALL_SLOTS);
    if (!slots || !X || !W || !y) return set_error(LORA_EINVAL, "%s: NULL pointer argument", fn);
    const int32_t *pts[MAX_CALL_SLOTS];
    for (int z = 0; z < n; ++z) {
        if (slots[z] < 0 || slots[z] >= p->n_slots)
            return set_error(LORA_EINVAL, "%s: slot %d not in [0, %d)", fn, slots[z], p->n_slots);
        pts[z] = p->page_table ? p->page_table + (size_t)slots[z] * p->max_adapters * 2 * p->max_rank : nullptr;
    }
    if (p->dtype == LORA_F32) {   // the float32 path (parity only) runs the slots one after another
        if (T <= 0 || T > MAX_TOKENS) return project_impl(p, fn, n, X, W, pts, ids, ranks, scale, T, y, ws, ws_bytes,
                                                          stream);   // T = 0: nothing; else the error
        Plan pl;
        if (!make_plan(p, T, &pl)) return set_error(LORA_EINVAL, "%s: bad T", fn);
        if (ws_bytes < pl.total * (size_t)n)
            return set_error(LORA_EINVAL, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, pl.total * (size_t)n);
        const size_t ybytes = (size_t)T * p->hidden * p->elem;
        for (int z = 0; z < n; ++z) {   // all checks before the first launch: no output overlaps an input or output
            const char *a = (const char *)y[z];
            for (int u = 0; u < n; ++u) {
                const char *b = (const char *)X[u], *c = (const char *)y[u];
                if (a && b && a < b + ybytes && b < a + ybytes) return set_error(LORA_EINVAL, "%s: y overlaps x", fn);
                if (u < z && a && c && a < c + ybytes && c < a + ybytes)
                    return set_error(LORA_EINVAL, "%s: two outputs overlap", fn);
            }
        }
        for (int z = 0; z < n; ++z) {
            const int rc = project_impl(p, fn, 1, &X[z], &W[z], &pts[z], ids, ranks, scale, T, &y[z],
                                        (char *)ws + (size_t)z * pl.total, ws_bytes - (size_t)z * pl.total, stream);
            if (rc) return rc;
        }
        return LORA_OK;
    }
    return project_impl(p, fn, n, X, W, pts, ids, ranks, scale, T, y, ws, ws_bytes, stream);
}
}  // namespace

extern "C" int lora_project_slots_x(lora_pool *p, int32_t n, const int32_t *slots, const void *const *x,
                                    const void *const *W, const int32_t *ids, const int32_t *ranks, const float *scale,
                                    int64_t T, void *const *y, void *ws, size_t ws_bytes, void *stream) {
    return project_slots_impl(p, "lora_project_slots_x", n, slots, x, W, ids, ranks, scale, T, y, ws, ws_bytes, stream);
}

extern "C" int lora_project_slots(lora_pool *p, int32_t n, const int32_t *slots, const void *x,
                                  const void *const *W, const int32_t *ids, const int32_t *ranks, const float *scale,
                                  int64_t T, void *const *y, void *ws, size_t ws_bytes, void *stream) {
    const void *X[MAX_CALL_SLOTS] = {x, x, x, x};
    return project_slots_impl(p, "lora_project_slots", n, slots, X, W, ids, ranks, scale, T, y, ws, ws_bytes, stream);
}

extern "C" int lora_profile_start(lora_pool *p, int32_t max_calls) {
    if (!p || p->bookkeeping_only || max_calls < 1 || max_calls > (1 << 20))
        return set_error(LORA_EINVAL, "lora_profile_start: bad pool or max_calls");
    DeviceGuard g(p->device);
    for (hipEvent_t e : p->prof_events) (void)hipEventDestroy(e);
    p->prof_events.assign((size_t)max_calls * 4, nullptr);
    for (auto &e : p->prof_events) LP_HIP(hipEventCreate(&e));
    p->prof_next.store(0);
    p->prof_max = max_calls;
    return LORA_OK;
}

extern "C" int lora_profile_stop(lora_pool *p, lora_profile_t *out) {
    if (!p || !out) return set_error(LORA_EINVAL, "lora_profile_stop: NULL argument");
    DeviceGuard g(p->device);
    memset(out, 0, sizeof *out);
    const int32_t n = std::min(p->prof_next.load(), p->prof_max);
    p->prof_max = 0;
    for (int32_t i = 0; i < n; ++i) {
        hipEvent_t *ev = &p->prof_events[(size_t)i * 4];
        LP_HIP(hipEventSynchronize(ev[3]));
        float a = 0, b = 0, c = 0;
        LP_HIP(hipEventElapsedTime(&a, ev[0], ev[1]));
        LP_HIP(hipEventElapsedTime(&b, ev[1], ev[2]));
        LP_HIP(hipEventElapsedTime(&c, ev[2], ev[3]));
        out->ms_group += a;
        out->ms_first += b;
        out->ms_second += c;
    }
    out->calls = n;
    for (hipEvent_t e : p->prof_events) (void)hipEventDestroy(e);
    p->prof_events.clear();
    return LORA_OK;
}

extern "C" int lora_debug_project(lora_pool *p, const void *x, const void *W, const int32_t *pt, const int32_t *ids,
                                  const int32_t *ranks, const float *scale, int64_t T, void *y, void *ws,
                                  size_t ws_bytes, int32_t *gather_out, int32_t *order_out, void *stream) {
    if (T > 0 && (!gather_out || !order_out))
        return set_error(LORA_EINVAL, "lora_debug_project: NULL pointer argument");
    if (!aligned(gather_out, 4) || !aligned(order_out, 4))
        return set_error(LORA_EINVAL, "lora_debug_project: misaligned debug output");
    const DebugOut dbg{gather_out, order_out};
    return project_impl(p, "lora_debug_project", 1, &x, &W, &pt, ids, ranks, scale, T, &y, ws, ws_bytes, stream, &dbg);
}

// ---- the projection for callers that cannot allocate -------------------------------------------
// The workspace of lora_project_noalloc is this file-scope device array, one copy per GPU, held until
// the process ends.  Host code never passes its name to a kernel (on the host it is a stand-in, not a
// device address): its address on each device comes from hipGetSymbolAddress, taken once per device
// at pool creation with that device current.
namespace {
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(LORA_NOALLOC_SCRATCH_MB) << 20;
static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};
}  // namespace

namespace lorapool {
int scratch_setup(int dev) {
    if (dev < 0 || dev >= MAX_DEVICES) return set_error(LORA_EINVAL, "device %d beyond %d", dev, MAX_DEVICES);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev]) return LORA_OK;
    DeviceGuard g(dev);
    if (!g.ok) return set_error(LORA_EHIP, "cannot select device %d", dev);
    void *ptr = nullptr;
    LP_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    g_scratch_ptr[dev] = ptr;
    return LORA_OK;
}
}  // namespace lorapool

extern "C" int lora_project_noalloc(lora_pool *p, const void *x, const void *W, const int32_t *pt, const int32_t *ids,
                                    const int32_t *ranks, const float *scale, int64_t T, void *y, void *stream) {
    if (!p) return set_error(LORA_EINVAL, "lora_project_noalloc: pool is NULL");
    if (p->bookkeeping_only) return set_error(LORA_EINVAL, "lora_project_noalloc: bookkeeping-only pool");
    Plan pl;
    if (!make_plan(p, T, &pl)) return set_error(LORA_EINVAL, "lora_project_noalloc: T = %lld out of range", (long long)T);
    if (pl.total > NOALLOC_SCRATCH_BYTES)
        return set_error(LORA_EINVAL, "lora_project_noalloc: %lld tokens at H = %d need %zu bytes of scratch, beyond the "
                                      "%d MiB this entry point has; use lora_project with a workspace",
                         (long long)T, p->hidden, pl.total, LORA_NOALLOC_SCRATCH_MB);
    void *ws = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        if (p->device >= 0 && p->device < MAX_DEVICES) ws = g_scratch_ptr[p->device];
    }
    if (!ws) {   // pool creation could not take the address: try once more, and report why not
        const int rc = scratch_setup(p->device);
        if (rc != LORA_OK) return rc;
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        ws = g_scratch_ptr[p->device];
    }
    return project_impl(p, "lora_project_noalloc", 1, &x, &W, &pt, ids, ranks, scale, T, &y, ws, NOALLOC_SCRATCH_BYTES,
                        stream);
}

extern "C" int lora_debug_gather(lora_pool *p, const int32_t *pt, const int32_t *ids, const int32_t *ranks,
                                 int64_t T, int32_t *out, void *stream) {
    if (!p) return set_error(LORA_EINVAL, "lora_debug_gather: pool is NULL");
    if (p->bookkeeping_only) return set_error(LORA_EINVAL, "lora_debug_gather: bookkeeping-only pool");
    if (T < 0 || T > MAX_TOKENS) return set_error(LORA_EINVAL, "lora_debug_gather: bad T %lld", (long long)T);
    if (T == 0) return LORA_OK;
    if (!pt || !ids || !ranks || !out) return set_error(LORA_EINVAL, "lora_debug_gather: NULL pointer argument");
    if (!aligned(pt, 4) || !aligned(ids, 4) || !aligned(ranks, 4) || !aligned(out, 4))
        return set_error(LORA_EINVAL, "lora_debug_gather: misaligned pointer");
    DeviceGuard g(p->device);
    hipError_t e = launch_debug_gather(p, pt, ids, ranks, T, out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_error(e, "debug gather launch");
    return LORA_OK;
}

extern "C" int lora_check_device_errors(lora_pool *p) {
    if (!p) return set_error(LORA_EINVAL, "lora_check_device_errors: pool is NULL");
    if (p->bookkeeping_only) return LORA_OK;
    DeviceGuard g(p->device);
    LP_HIP(hipDeviceSynchronize());
    int word = 0;
    LP_HIP(hipMemcpy(&word, p->dev_err, sizeof word, hipMemcpyDeviceToHost));
    if (!word) return LORA_OK;
    LP_HIP(hipMemset(p->dev_err, 0, sizeof word));
    return set_error(LORA_EDEVICE, "device check failed:%s%s%s%s", word & DEV_ERR_ID ? " adapter-id-out-of-range" : "",
                     word & DEV_ERR_RANK ? " rank-out-of-range" : "",
                     word & DEV_ERR_TABLE ? " adapter-not-loaded-at-this-rank" : "",
                     word & DEV_ERR_PAGE ? " page-id-out-of-range" : "");
}
