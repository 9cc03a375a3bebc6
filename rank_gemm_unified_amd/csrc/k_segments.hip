// Token grouping and validation (one workgroup), and the debug view of the gather.
//
// Grouping tokens that share an adapter lets each adapter's A and B pages be read once per call
// rather than once per token: low-rank work scales with tokens and ranks, adapter memory traffic
// with distinct adapters ("S-LoRA, in depth", section "Kernels for a batch of mixed ranks").
#include "device_common.h"
#include "internal.h"

namespace lorapool {

constexpr int SEG_THREADS = 1024;

// Exclusive scan of a[0..n) in LDS by a 1024-thread block; returns the total to every thread.
// Each thread owns a contiguous run of ceil(n/1024) entries, so the result is deterministic.
__device__ int32_t block_exclusive_scan(int32_t *a, int32_t n, int32_t *scratch) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (n + SEG_THREADS - 1) / SEG_THREADS;
    const int b = tid * per, e = min(n, b + per);
    int32_t local = 0;
    for (int i = b; i < e; ++i) local += a[i];
    const int32_t incl = wave_incl_scan(local, lane);
    if (lane == 63) scratch[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int32_t w = lane < SEG_THREADS / 64 ? scratch[lane] : 0;
        const int32_t wi = wave_incl_scan(w, lane);
        if (lane < SEG_THREADS / 64) scratch[lane] = wi - w;        // exclusive wave offsets
        if (lane == SEG_THREADS / 64 - 1) scratch[SEG_THREADS / 64] = wi;
    }
    __syncthreads();
    int32_t run = scratch[wave] + incl - local;
    for (int i = b; i < e; ++i) {
        const int32_t v = a[i];
        a[i] = run;
        run += v;
    }
    const int32_t total = scratch[SEG_THREADS / 64];
    __syncthreads();
    return total;
}

// LDS counter update: every lane with key >= 0 adds 1 to cnt[key] and gets old + its rank among the
// lanes of its key; -1 for lanes with key < 0.  A wave whose tokens share one key (a prefill run: the
// usual case) issues one atomic for all of them, since per-lane atomics on one counter serialize; a
// wave with several keys (decode-style rows, one adapter each) issues one atomic per lane, and lanes
// sharing a key get distinct slots in an unspecified order (no result depends on the order of tokens
// within a segment).  Looping over the distinct keys instead cost a few LDS round trips per key.
__device__ __forceinline__ int32_t wave_add_rank(int32_t *cnt, int32_t key) {
    const int lane = threadIdx.x & 63;
    const uint64_t valid = __ballot(key >= 0);
    if (!valid) return -1;
    const int leader = __ffsll((unsigned long long)valid) - 1;
    const int32_t lkey = __shfl(key, leader, 64);
    const uint64_t m = __ballot(key == lkey);
    if (m == valid) {
        int32_t old = 0;
        if (lane == leader) old = atomicAdd(&cnt[lkey], __popcll(m));
        old = __shfl(old, leader, 64);
        return key >= 0 ? old + __popcll(m & ((1ull << lane) - 1ull)) : -1;
    }
    return key >= 0 ? atomicAdd(&cnt[key], 1) : -1;
}

// Exclusive scan of three arrays at once (same layout as block_exclusive_scan); returns the totals.
__device__ int3 block_exclusive_scan3(int32_t *a0, int32_t *a1, int32_t *a2, int32_t n, int32_t *scratch) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int NW = SEG_THREADS / 64;
    const int per = (n + SEG_THREADS - 1) / SEG_THREADS;
    const int b = tid * per, e = min(n, b + per);
    int32_t l0 = 0, l1 = 0, l2 = 0;
    for (int i = b; i < e; ++i) { l0 += a0[i]; l1 += a1[i]; l2 += a2[i]; }
    const int32_t i0 = wave_incl_scan(l0, lane), i1 = wave_incl_scan(l1, lane), i2 = wave_incl_scan(l2, lane);
    if (lane == 63) { scratch[wave] = i0; scratch[NW + 1 + wave] = i1; scratch[2 * (NW + 1) + wave] = i2; }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            int32_t *sc = scratch + q * (NW + 1);
            const int32_t w = lane < NW ? sc[lane] : 0;
            const int32_t wi = wave_incl_scan(w, lane);
            if (lane < NW) sc[lane] = wi - w;
            if (lane == NW - 1) sc[NW] = wi;
        }
    }
    __syncthreads();
    int32_t r0 = scratch[wave] + i0 - l0, r1 = scratch[NW + 1 + wave] + i1 - l1,
            r2 = scratch[2 * (NW + 1) + wave] + i2 - l2;
    for (int i = b; i < e; ++i) {
        const int32_t v0 = a0[i], v1 = a1[i], v2 = a2[i];
        a0[i] = r0; a1[i] = r1; a2[i] = r2;
        r0 += v0; r1 += v1; r2 += v2;
    }
    const int3 tot = make_int3(scratch[NW], scratch[2 * (NW + 1) - 1], scratch[3 * (NW + 1) - 1]);
    __syncthreads();
    return tot;
}

// One workgroup of 1024 threads, two dependent rounds of global reads:
//  1. the ids (range-checked; tokens counted per adapter id);
//  2. for every adapter in use, its rank and its whole page-table row in every slot of the call, all
//     loaded together (EPT entries a thread at a time) and checked after they arrive (entries [0, 2r)
//     hold pages in range, entry 2r is -1 when 2r < stride; a bad row in any slot turns the adapter off).
// Tokens of an adapter with rank 0, a bad rank or a bad row get no low-rank term.  Segments are in
// adapter order; tokens of one adapter land in perm in an unspecified order (LDS atomics): no result
// depends on the order of tokens within a segment.  Work items (`chunk` sorted rows of one segment) are
// written as item_seg / item_row and as one record {adapter, rank, first row, rows} each, with
// adapter -1 from the last item up to n_items_max, so a kernel reads its item in one load.
// LDS: cnt | uidx | ulist | rk (max_adapters each) | scratch[3 * 17].
constexpr int KPT = 16;   // tokens per thread held in registers (T <= 16384 reads the ids once)
constexpr int32_t F_OFF = 1 << 30;   // cnt flag: the adapter's tokens get no low-rank term
constexpr int EPT = 4;               // page-table entries per thread and round trip (every slot's at once)

__global__ __launch_bounds__(SEG_THREADS) void k_segments(
    const int32_t *__restrict__ ids, const int32_t *__restrict__ ranks, const SlotRows sp, int32_t n_slots_call,
    int32_t stride, int32_t T, int32_t max_adapters, int32_t max_rank, int64_t num_pages, int32_t chunk,
    int32_t *__restrict__ tok_a, int32_t *__restrict__ tok_r, int32_t *__restrict__ perm,
    int32_t *__restrict__ seg_a, int32_t *__restrict__ seg_start, int32_t *__restrict__ item_seg,
    int32_t *__restrict__ item_row, int4 *__restrict__ item_rec, int32_t n_items_max,
    int32_t *__restrict__ ctrl, int *__restrict__ err) {
    extern __shared__ int32_t lds[];
    int32_t *cnt = lds, *uidx = lds + max_adapters, *ulist = lds + 2 * max_adapters, *rk = lds + 3 * max_adapters;
    int32_t *scratch = lds + 4 * max_adapters;
    __shared__ int s_err;
    const int tid = threadIdx.x;
    const bool cached = T <= KPT * SEG_THREADS;
    int my_err = 0;
    if (tid == 0) s_err = 0;
    for (int a = tid; a < max_adapters; a += SEG_THREADS) cnt[a] = 0;
    __syncthreads();

    // ---- round 1: ids
    int32_t key[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) key[u] = -1;
    for (int t0 = 0; t0 < T; t0 += KPT * SEG_THREADS) {
        // slots u with t0 + u SEG_THREADS >= T hold no token in any lane: skipped (a uniform test)
        int32_t a[KPT];
#pragma unroll
        for (int u = 0; u < KPT; ++u)
            if (t0 + u * SEG_THREADS < T) a[u] = ids[min(t0 + u * SEG_THREADS + tid, T - 1)];
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            if (t0 + u * SEG_THREADS >= T) break;
            const int t = t0 + u * SEG_THREADS + tid;
            int32_t k = -1;
            if (t < T && a[u] != -1) {
                if (a[u] < -1 || a[u] >= max_adapters) my_err |= DEV_ERR_ID;
                else k = a[u];
            }
            wave_add_rank(cnt, k);
            if (t < T && !cached) tok_a[t] = k;
            if (cached) key[u] = k;
        }
    }
    __syncthreads();
    for (int a = tid; a < max_adapters; a += SEG_THREADS) uidx[a] = cnt[a] > 0;
    __syncthreads();
    const int32_t nused = block_exclusive_scan(uidx, max_adapters, scratch);
    for (int a = tid; a < max_adapters; a += SEG_THREADS)
        if (cnt[a] > 0) ulist[uidx[a]] = a;
    __syncthreads();

    // ---- round 2: rank and page-table row of every adapter in use (stride entries each), in every
    // slot of the call (the later kernels read these rows unchecked; one bad row turns the adapter
    // off in all of them)
    const int32_t nent = nused * stride;
    for (int e0 = tid; e0 < nent; e0 += EPT * SEG_THREADS) {
        // the entry's adapter, index and rank are the same in every slot; the entries of all the slots
        // go out together (one round trip, not one per slot), EPT per thread so that they fit the
        // registers of a 1024-thread workgroup
        int32_t av[EPT], jv[EPT], rv[EPT], ev[MAX_CALL_SLOTS][EPT];
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = min(e0 + u * SEG_THREADS, nent - 1);
            av[u] = ulist[e / stride];
            jv[u] = e % stride;
            rv[u] = ranks[av[u]];
        }
#pragma unroll
        for (int z = 0; z < MAX_CALL_SLOTS; ++z) {
            if (z >= n_slots_call) break;   // uniform
            const int32_t *pz = sp.pt[z];
#pragma unroll
            for (int u = 0; u < EPT; ++u) ev[z][u] = pz[(int64_t)av[u] * stride + jv[u]];
        }
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            if (e0 + u * SEG_THREADS >= nent) continue;
            const int32_t r = rv[u], j = jv[u];
            int bad = 0;
            if (r < 0 || r > max_rank) {
                if (j == 0) bad = DEV_ERR_RANK;
            } else if (r > 0) {
#pragma unroll
                for (int z = 0; z < MAX_CALL_SLOTS; ++z) {
                    if (z >= n_slots_call) break;
                    const int32_t ent = ev[z][u];
                    if (j < 2 * r) {
                        if (ent == -1) bad |= DEV_ERR_TABLE;
                        else if (ent < 0 || (int64_t)ent >= num_pages) bad |= DEV_ERR_PAGE;
                    } else if (j == 2 * r && ent != -1) {
                        bad |= DEV_ERR_TABLE;
                    }
                }
            }
            if (j == 0) {
                rk[av[u]] = r;
                if (r <= 0 || r > max_rank) atomicOr(&cnt[av[u]], F_OFF);   // rank 0 or bad: no low-rank term
            }
            if (bad) {
                my_err |= bad;
                atomicOr(&cnt[av[u]], F_OFF);
            }
        }
    }
    __syncthreads();

    // ---- segments: adapters in use with a good row, in adapter order; work items of `chunk` tokens
    for (int a = tid; a < max_adapters; a += SEG_THREADS) {
        const int32_t c = cnt[a];
        const int32_t n = (c & F_OFF) ? 0 : c;
        cnt[a] = n;                       // -> first sorted position
        uidx[a] = n > 0;                  // -> segment index
        ulist[a] = (n + chunk - 1) / chunk;   // -> first work item
    }
    __syncthreads();
    // (a segment's length is re-derived from the scanned offsets of consecutive adapters)
    const int3 tot = block_exclusive_scan3(cnt, uidx, ulist, max_adapters, scratch);
    const int32_t nvalid = tot.x, nseg = tot.y, nitems = tot.z;
    for (int a = tid; a < max_adapters; a += SEG_THREADS) {
        const int32_t next = a + 1 < max_adapters ? cnt[a + 1] : nvalid;
        const int32_t n = next - cnt[a];
        if (n > 0) {
            const int32_t sg = uidx[a];
            seg_a[sg] = a;
            seg_start[sg] = cnt[a];
            int32_t it = ulist[a];
            for (int32_t r0 = cnt[a]; r0 < next; r0 += chunk, ++it) {
                item_seg[it] = sg;
                item_row[it] = r0;
                item_rec[it] = int4{a, rk[a], r0, min(next - r0, chunk)};
            }
        }
    }
    for (int it = nitems + tid; it < n_items_max; it += SEG_THREADS) item_rec[it] = int4{-1, 0, 0, 0};
    if (tid == 0) {
        seg_start[nseg] = nvalid;
        ctrl[CTRL_NSEG] = nseg;
        ctrl[CTRL_NVALID] = nvalid;
        ctrl[CTRL_NITEMS] = nitems;
    }
    __syncthreads();

    // ---- tokens: record, scatter into their segments.  An adapter is live iff its segment index steps
    // up after it (uidx, unlike cnt, is not changed by the scatter).  Every lane takes part in each
    // step: the counter update is wave-wide.
    for (int t0 = 0; t0 < T; t0 += KPT * SEG_THREADS) {
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            if (t0 + u * SEG_THREADS >= T) break;
            const int t = t0 + u * SEG_THREADS + tid;
            int32_t k = t < T ? (cached ? key[u] : tok_a[t]) : -1;
            if (k >= 0 && (k + 1 < max_adapters ? uidx[k + 1] : nseg) == uidx[k]) k = -1;
            if (t < T) {
                tok_a[t] = k;
                tok_r[t] = k >= 0 ? rk[k] : 0;
            }
            const int32_t pos = wave_add_rank(cnt, k);
            if (k >= 0) perm[pos] = t;
        }
    }
    if (my_err) atomicOr(&s_err, my_err);
    __syncthreads();
    if (tid == 0 && s_err) atomicOr(err, s_err);
}

// Debug view of the gather: one workgroup per token, one thread per page-table entry.
__global__ __launch_bounds__(128) void k_debug_gather(const int32_t *__restrict__ ids,
                                                      const int32_t *__restrict__ ranks,
                                                      const int32_t *__restrict__ pt, int32_t stride,
                                                      int32_t max_adapters, int32_t max_rank, int64_t num_pages,
                                                      int32_t *__restrict__ out, int *__restrict__ err) {
    __shared__ int s_bad;
    const int64_t t = blockIdx.x;
    const int j = threadIdx.x;
    if (j == 0) s_bad = 0;
    __syncthreads();
    const int32_t a = ids[t];
    int32_t r = 0;
    int bad = 0;
    if (a != -1) {
        if (a < -1 || a >= max_adapters) {
            bad = DEV_ERR_ID;
        } else {
            r = ranks[a];
            if (r < 0 || r > max_rank) {
                bad = DEV_ERR_RANK;
            } else if (r > 0 && j < stride) {
                bad = check_row_entry(pt + (int64_t)a * stride, j, r, stride, num_pages);
            }
        }
    }
    if (bad) atomicOr(&s_bad, bad);
    __syncthreads();
    const int any = s_bad;
    if (j < stride) {
        int32_t v = -1;
        if (!any && a >= 0 && j < 2 * r) v = pt[(int64_t)a * stride + j];
        out[t * stride + j] = v;
    }
    if (j == 0 && any) atomicOr(err, any);
}

static size_t segments_lds(int32_t max_adapters) { return (size_t)(4 * max_adapters + 3 * 17) * sizeof(int32_t); }

hipError_t launch_segments(const lora_pool *p, const Plan &plan, const Ws &ws, const int32_t *ids,
                           const int32_t *ranks, const SlotPtrs &sp, int n, hipStream_t s) {
    static bool attr_set = false;
    const size_t lds = segments_lds(p->max_adapters);
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)k_segments, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)segments_lds(LORA_MAX_ADAPTERS));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    SlotRows rows;
    for (int z = 0; z < MAX_CALL_SLOTS; ++z) rows.pt[z] = sp.pt[z];
    hipLaunchKernelGGL(k_segments, dim3(1), dim3(SEG_THREADS), lds, s, ids, ranks, rows, n, 2 * p->max_rank,
                       (int32_t)plan.T, p->max_adapters, p->max_rank, p->num_pages, plan.chunk, ws.tok_a, ws.tok_r,
                       ws.perm, ws.seg_a, ws.seg_start, ws.item_seg, ws.item_row, ws.item_rec, plan.n_items_max,
                       ws.ctrl, p->dev_err);
    return hipGetLastError();
}

hipError_t launch_debug_gather(const lora_pool *p, const int32_t *pt, const int32_t *ids, const int32_t *ranks,
                               int64_t T, int32_t *out, hipStream_t s) {
    hipLaunchKernelGGL(k_debug_gather, dim3((unsigned)T), dim3(128), 0, s, ids, ranks, pt, 2 * p->max_rank,
                       p->max_adapters, p->max_rank, p->num_pages, out, p->dev_err);
    return hipGetLastError();
}

}  // namespace lorapool
