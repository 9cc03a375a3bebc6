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
    int32_t incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    if (lane == 63) scratch[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int32_t w = lane < SEG_THREADS / 64 ? scratch[lane] : 0;
        int32_t wi = w;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t y = __shfl_up(wi, off, 64);
            if (lane >= off) wi += y;
        }
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

// One workgroup of 1024 threads.  LDS: hist[max_adapters] | segf[max_adapters] | seglen[max_adapters]
// | scratch[32].  Each thread keeps up to KPT of its tokens (t = tid + 1024 u) in registers, so a
// batch of up to 8192 tokens costs one read of the ids; longer batches re-read them from tok_a.
// Tokens of one adapter land in perm in an unspecified order (LDS atomics): no result depends on
// the order of tokens within a segment.
constexpr int KPT = 8;

__global__ __launch_bounds__(SEG_THREADS) void k_segments(
    const int32_t *__restrict__ ids, const int32_t *__restrict__ ranks, const int32_t *__restrict__ pt,
    int32_t stride, int32_t T, int32_t max_adapters, int32_t max_rank, int64_t num_pages, int32_t chunk,
    int32_t *__restrict__ tok_a, int32_t *__restrict__ tok_r, int32_t *__restrict__ perm,
    int32_t *__restrict__ seg_a, int32_t *__restrict__ seg_start, int32_t *__restrict__ item_seg,
    int32_t *__restrict__ item_row, int32_t *__restrict__ ctrl, int32_t *__restrict__ counters,
    int32_t n_counters, int *__restrict__ err) {
    extern __shared__ int32_t lds[];
    int32_t *hist = lds, *segf = lds + max_adapters, *seglen = lds + 2 * max_adapters;
    int32_t *scratch = lds + 3 * max_adapters;
    __shared__ int s_err;
    const int tid = threadIdx.x;
    const bool cached = T <= KPT * SEG_THREADS;
    int my_err = 0;
    if (tid == 0) s_err = 0;
    for (int i = tid; i < n_counters; i += SEG_THREADS) counters[i] = 0;
    for (int a = tid; a < max_adapters; a += SEG_THREADS) hist[a] = 0;
    __syncthreads();

    // 1. id and rank range checks; count tokens per adapter with rank > 0
    int32_t key[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) key[u] = -1;
    for (int t0 = 0; t0 < T; t0 += KPT * SEG_THREADS) {
        int32_t a[KPT], rr[KPT];
#pragma unroll
        for (int u = 0; u < KPT; ++u) a[u] = ids[min(t0 + u * SEG_THREADS + tid, T - 1)];
#pragma unroll
        for (int u = 0; u < KPT; ++u) rr[u] = ranks[a[u] >= 0 && a[u] < max_adapters ? a[u] : 0];
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int t = t0 + u * SEG_THREADS + tid;
            int32_t k = -1, r = 0;
            if (t < T && a[u] != -1) {
                if (a[u] < -1 || a[u] >= max_adapters) {
                    my_err |= DEV_ERR_ID;
                } else if (rr[u] < 0 || rr[u] > max_rank) {
                    my_err |= DEV_ERR_RANK;
                } else if (rr[u] > 0) {
                    k = a[u];
                    r = rr[u];
                    atomicAdd(&hist[k], 1);
                }
            }
            if (t < T) {
                tok_a[t] = k;
                tok_r[t] = r;
            }
            if (cached) key[u] = k;
        }
    }
    __syncthreads();

    // 2. each adapter in use: its page-table row must hold exactly 2r in-range pages.  The entries
    //    of all used adapters are checked by all threads together (flattened list, 4 loads in flight).
    for (int a = tid; a < max_adapters; a += SEG_THREADS) segf[a] = hist[a] > 0;
    __syncthreads();
    const int32_t nused = block_exclusive_scan(segf, max_adapters, scratch);   // segf := used index
    for (int a = tid; a < max_adapters; a += SEG_THREADS)
        if (hist[a] > 0) seglen[segf[a]] = a;                                   // seglen := used list
    __syncthreads();
    for (int u = tid; u < max_adapters; u += SEG_THREADS)
        segf[u] = u < nused ? min(2 * ranks[seglen[u]] + 1, stride) : 0;
    __syncthreads();
    const int32_t nchk = block_exclusive_scan(segf, max_adapters, scratch);    // segf := entry offsets
    for (int e0 = tid; e0 < nchk; e0 += 4 * SEG_THREADS) {
        int ua[4], j[4];
        int32_t ent[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = min(e0 + u * SEG_THREADS, nchk - 1);
            int lo = 0, hi = nused - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (segf[mid] <= e) lo = mid; else hi = mid - 1;
            }
            ua[u] = seglen[lo];
            j[u] = e - segf[lo];
            ent[u] = pt[(int64_t)ua[u] * stride + j[u]];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (e0 + u * SEG_THREADS >= nchk) continue;
            const int32_t r = ranks[ua[u]];
            int bad = 0;
            if (j[u] < 2 * r) {
                if (ent[u] == -1) bad = DEV_ERR_TABLE;
                else if (ent[u] < 0 || (int64_t)ent[u] >= num_pages) bad = DEV_ERR_PAGE;
            } else if (ent[u] != -1) {
                bad = DEV_ERR_TABLE;
            }
            if (bad) {
                my_err |= bad;
                atomicOr(&hist[ua[u]], 0x40000000);
            }
        }
    }
    __syncthreads();

    // 3. tokens of a faulty adapter get the base product only
    for (int t0 = 0; t0 < T; t0 += KPT * SEG_THREADS) {
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int t = t0 + u * SEG_THREADS + tid;
            if (t >= T) continue;
            const int32_t k = cached ? key[u] : tok_a[t];
            if (k >= 0 && (hist[k] & 0x40000000)) {
                tok_a[t] = -1;
                tok_r[t] = 0;
                if (cached) key[u] = -1;
            }
        }
    }
    __syncthreads();
    for (int a = tid; a < max_adapters; a += SEG_THREADS) {
        const int32_t c = (hist[a] & 0x40000000) ? 0 : hist[a];
        hist[a] = c;
        segf[a] = c > 0;
        seglen[a] = c;
    }
    __syncthreads();
    const int32_t nvalid = block_exclusive_scan(hist, max_adapters, scratch);   // hist := offsets
    const int32_t nseg = block_exclusive_scan(segf, max_adapters, scratch);     // segf := segment index

    // 4. segments in adapter order
    for (int a = tid; a < max_adapters; a += SEG_THREADS) {
        if (seglen[a] > 0) {
            seg_a[segf[a]] = a;
            seg_start[segf[a]] = hist[a];
        }
    }
    if (tid == 0) {
        seg_start[nseg] = nvalid;
        ctrl[CTRL_NSEG] = nseg;
        ctrl[CTRL_NVALID] = nvalid;
    }
    __syncthreads();

    // 5. scatter token ids into their segments
    for (int t0 = 0; t0 < T; t0 += KPT * SEG_THREADS) {
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int t = t0 + u * SEG_THREADS + tid;
            if (t >= T) continue;
            const int32_t k = cached ? key[u] : tok_a[t];
            if (k >= 0) perm[atomicAdd(&hist[k], 1)] = t;
        }
    }
    __syncthreads();

    // 6. shrink work items: each segment split into runs of `chunk` tokens
    for (int s = tid; s < max_adapters; s += SEG_THREADS)
        segf[s] = s < nseg ? (seglen[seg_a[s]] + chunk - 1) / chunk : 0;
    __syncthreads();
    const int32_t nitems = block_exclusive_scan(segf, max_adapters, scratch);
    for (int s = tid; s < nseg; s += SEG_THREADS) {
        const int32_t b = seg_start[s], e = b + seglen[seg_a[s]];
        int32_t it = segf[s];
        for (int32_t r0 = b; r0 < e; r0 += chunk, ++it) {
            item_seg[it] = s;
            item_row[it] = r0;
        }
    }
    if (tid == 0) ctrl[CTRL_NITEMS] = nitems;
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

static size_t segments_lds(int32_t max_adapters) { return (size_t)(3 * max_adapters + 32) * sizeof(int32_t); }

hipError_t launch_segments(const lora_pool *p, const Plan &plan, const Ws &ws, const int32_t *ids,
                           const int32_t *ranks, const int32_t *pt, hipStream_t s) {
    static bool attr_set = false;
    const size_t lds = segments_lds(p->max_adapters);
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)k_segments, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)segments_lds(LORA_MAX_ADAPTERS));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(k_segments, dim3(1), dim3(SEG_THREADS), lds, s, ids, ranks, pt, 2 * p->max_rank,
                       (int32_t)plan.T, p->max_adapters, p->max_rank, p->num_pages, plan.chunk, ws.tok_a, ws.tok_r,
                       ws.perm, ws.seg_a, ws.seg_start, ws.item_seg, ws.item_row, ws.ctrl, ws.counters,
                       plan.n_counters, p->dev_err);
    return hipGetLastError();
}

hipError_t launch_debug_gather(const lora_pool *p, const int32_t *pt, const int32_t *ids, const int32_t *ranks,
                               int64_t T, int32_t *out, hipStream_t s) {
    hipLaunchKernelGGL(k_debug_gather, dim3((unsigned)T), dim3(128), 0, s, ids, ranks, pt, 2 * p->max_rank,
                       p->max_adapters, p->max_rank, p->num_pages, out, p->dev_err);
    return hipGetLastError();
}

}  // namespace lorapool
