// Decode-shaped projection (T <= 256 tokens, typically one per request): memory-bound, so the
// kernels are organised to stream W and the gathered A/B pages from HBM once, with as few
// dependent global round trips as possible and no in-kernel cross-workgroup waits (on this chip a
// device-scope fence writes back and invalidates the whole L2).
//
// Two launches per call:
//   T <= 64:       k_decode_stream   W, x and the batch's A pages in one streaming MFMA pass
//                                    (the shrink x A is extra MFMA columns of the same contraction)
//   64 < T <= 256: k_decode_main     shrink workgroups (one wave per gathered A page) beside split-K
//                                    base workgroups
//   then           k_decode_finish   partial sums in split order + the expand sum_j v_j B_a[j, :]
//                                    from B rows gathered from their pages + one rounding
// ("S-LoRA, in depth", section "Merge or keep adapters separate": xW batched over all tokens
// whatever their adapter, plus two thin low-rank products per adapter; section "Kernels for a batch of
// mixed ranks": low-rank work follows tokens and ranks, adapter traffic follows distinct adapters.)
// Every sum has a fixed order, so results are bitwise reproducible.
//
// The float32 path (parity-only, small shapes) keeps the grouping kernel, a gathered shrink and a
// plain VALU kernel.
#include "device_common.h"
#include "internal.h"

namespace lorapool {

constexpr int CHUNK = 16;      // tokens per shrink work item
constexpr int DEC_T = 256;     // most tokens on the decode path
constexpr int NT = 64;         // columns per base tile (64 < T <= 256 kernel)
constexpr int NB = NT / 16;    // 16-column MFMA blocks per tile

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glob_void;

// s_barrier with no memory fence; the asm statements keep the compiler from moving memory
// accesses across it.  Callers make their own LDS writes complete first.
__device__ __forceinline__ void workgroup_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One wave: v[tok[i]][j] = sc * <x[tok[i]], page> for i < n (1 <= n <= CHUNK).
// Tokens go in groups of G; for each group the page is read in blocks of BLK 16-byte vectors per
// lane together with the group's x rows, all loads of a block issued before the first use
// (indices clamped to valid rows, clamped duplicates discarded): one round trip per block.
template <int EB>
__device__ __forceinline__ void shrink_page_wave(const char *__restrict__ x, const char *__restrict__ Ap,
                                                 int64_t row_bytes, const int32_t *tok, int n, float sc, int j,
                                                 float *__restrict__ v, int R, int lane) {
    constexpr int EPV = 16 / EB;   // elements per 16-byte vector
    constexpr int BLK = 8;         // 16-byte vectors per lane per block (8 KiB per wave)
    constexpr int G = 2;           // tokens per group
#pragma unroll 1
    for (int g0 = 0; g0 < n; g0 += G) {
        const char *xr[G];
#pragma unroll
        for (int i = 0; i < G; ++i) xr[i] = x + (int64_t)tok[min(g0 + i, n - 1)] * row_bytes;
        float acc[G];
#pragma unroll
        for (int i = 0; i < G; ++i) acc[i] = 0.f;
#pragma unroll 1
        for (int64_t base = 0; base < row_bytes; base += 64 * 16 * BLK) {
            int64_t off[BLK];
            bool live[BLK];
#pragma unroll
            for (int b = 0; b < BLK; ++b) {
                const int64_t o = base + (int64_t)(b * 64 + lane) * 16;
                live[b] = o < row_bytes;
                off[b] = live[b] ? o : 0;
            }
            u32x4_t av[BLK], xv[G][BLK];
#pragma unroll
            for (int b = 0; b < BLK; ++b) av[b] = load16(Ap + off[b]);
#pragma unroll
            for (int i = 0; i < G; ++i)
#pragma unroll
                for (int b = 0; b < BLK; ++b) xv[i][b] = load16(xr[i] + off[b]);
#pragma unroll
            for (int b = 0; b < BLK; ++b) {
                float af[EPV];
                if constexpr (EB == 2) {
                    unpack_bf16x8(av[b], af);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) af[e] = __uint_as_float(av[b][e]);
                }
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    float xf[EPV];
                    if constexpr (EB == 2) {
                        unpack_bf16x8(xv[i][b], xf);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) xf[e] = __uint_as_float(xv[i][b][e]);
                    }
                    float d = 0.f;
#pragma unroll
                    for (int e = 0; e < EPV; ++e) d = fmaf(af[e], xf[e], d);
                    acc[i] += live[b] ? d : 0.f;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const float tot = wave_sum(acc[i]);
            if (lane == 0 && g0 + i < n) v[(int64_t)tok[g0 + i] * R + j] = sc * tot;
        }
    }
}

// ---- in-LDS grouping of <= 256 tokens by adapter (thread t handles token t) ---------------------
struct DecGroup {
    int32_t key[DEC_T];        // adapter id, or -1 (none, rank 0, id or rank out of range)
    int32_t r[DEC_T];
    int32_t seg[DEC_T];        // segment of a token with key >= 0
    int32_t seg_a[DEC_T], seg_r[DEC_T], seg_n[DEC_T], seg_bad[DEC_T];
    int32_t seg_off[DEC_T + 1];    // first sorted position of each segment
    int32_t item_off[DEC_T + 1];   // first 16-token shrink item of each segment
    int32_t page_off[DEC_T + 1];   // first page of each segment in the batch's page list
    int32_t chk_off[DEC_T + 1];    // first page-table entry to check of each segment
    int32_t sorted[DEC_T];     // sorted position -> token
    int32_t wsum[8];
    int32_t n_seg, n_valid, n_items, n_pages, n_chk;
};

// exclusive prefix of v over the NTH threads; *total gets the sum (all threads)
template <int NTH>
__device__ int32_t scan_block(int32_t v, int32_t *wsum, int32_t *total) {
    constexpr int NW = NTH / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    __syncthreads();
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        before += w < wave ? wsum[w] : 0;
        tot += wsum[w];
    }
    *total = tot;
    return before + incl - v;
}

// last index s in [0, n) with off[s] <= i (off ascending, off[0] = 0)
__device__ __forceinline__ int find_seg(const int32_t *off, int n, int32_t i) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Every workgroup that needs the grouping derives it from the ids; all derive the same one.
// Returns the id/rank error bits this thread saw.
template <int NTH>
__device__ int dec_group(DecGroup &g, const int32_t *__restrict__ ids, const int32_t *__restrict__ ranks,
                         int32_t T, int32_t max_adapters, int32_t max_rank, int32_t stride) {
    const int t = threadIdx.x;
    const bool tok_thread = t < DEC_T;
    int err = 0;
    int32_t key = -1, r = 0;
    if (t < T) {
        const int32_t a = ids[t];
        const int32_t rr = ranks[a >= 0 && a < max_adapters ? a : 0];
        if (a != -1) {
            if (a < -1 || a >= max_adapters) err |= DEV_ERR_ID;
            else if (rr < 0 || rr > max_rank) err |= DEV_ERR_RANK;
            else if (rr > 0) { key = a; r = rr; }
        }
    }
    if (tok_thread) {
        g.key[t] = key;
        g.r[t] = r;
        g.seg_n[t] = 0;
        g.seg_bad[t] = 0;
    }
    __syncthreads();
    int32_t first = t, rank_in = 0;
    if (key >= 0) {
        for (int u = 0; u < t; ++u) {
            if (g.key[u] == key) {
                if (rank_in == 0) first = u;
                ++rank_in;
            }
        }
    }
    const int is_first = key >= 0 && rank_in == 0;
    int32_t nseg;
    const int32_t sid = scan_block<NTH>(is_first, g.wsum, &nseg);
    if (is_first) {
        g.seg[t] = sid;
        g.seg_a[sid] = key;
        g.seg_r[sid] = r;
    }
    __syncthreads();
    int32_t my_seg = -1;
    if (key >= 0) {
        my_seg = g.seg[first];
        atomicAdd(&g.seg_n[my_seg], 1);
    }
    __syncthreads();
    // per segment (thread s): token offsets, shrink items, pages, entries to check
    const bool seg_thread = t < nseg;
    const int32_t n_s = seg_thread ? g.seg_n[t] : 0;
    const int32_t r_s = seg_thread ? g.seg_r[t] : 0;
    int32_t nvalid, nitems, npages, nchk, nid;
    const int32_t off = scan_block<NTH>(n_s, g.wsum, &nvalid);
    const int32_t ioff = scan_block<NTH>(r_s * ((n_s + CHUNK - 1) / CHUNK), g.wsum, &nitems);
    const int32_t poff = scan_block<NTH>(r_s, g.wsum, &npages);
    const int32_t coff = scan_block<NTH>(seg_thread ? min(2 * r_s + 1, stride) : 0, g.wsum, &nchk);
    // identity / invalid tokens go after the grouped ones, in token order
    const int32_t idpos = scan_block<NTH>(t < T && key < 0, g.wsum, &nid);
    if (seg_thread) {
        g.seg_off[t] = off;
        g.item_off[t] = ioff;
        g.page_off[t] = poff;
        g.chk_off[t] = coff;
    }
    if (t == 0) {
        g.n_seg = nseg;
        g.n_valid = nvalid;
        g.n_items = nitems;
        g.n_pages = npages;
        g.n_chk = nchk;
        g.seg_off[nseg] = nvalid;
        g.item_off[nseg] = nitems;
        g.page_off[nseg] = npages;
        g.chk_off[nseg] = nchk;
    }
    __syncthreads();
    if (t < T) g.sorted[key >= 0 ? g.seg_off[my_seg] + rank_in : nvalid + idpos] = t;
    __syncthreads();
    return err;
}

// Workgroup 0's extra duty: check every page-table row in use (exactly 2r in-range pages, -1 after),
// publish the sorted token list {token, adapter or -1, rank, 0} and, per sorted position, the token's
// B page ids (row entries r..2r-1) for the finishing kernel; report errors.
template <int NTH>
__device__ void dec_publish(DecGroup &g, int err, const int32_t *__restrict__ pt, int32_t stride,
                            int64_t num_pages, int32_t T, int32_t RP, int4 *__restrict__ sorted_tok,
                            int32_t *__restrict__ spages, int *__restrict__ err_word) {
    const int nseg = g.n_seg;
    for (int e0 = threadIdx.x; e0 < g.n_chk; e0 += NTH * 4) {
        int32_t ent[4];
        int sg[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = min(e0 + u * NTH, g.n_chk - 1);
            sg[u] = find_seg(g.chk_off, nseg, e);
            ent[u] = pt[(int64_t)g.seg_a[sg[u]] * stride + (e - g.chk_off[sg[u]])];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + u * NTH;
            if (e >= g.n_chk) continue;
            const int s = sg[u], j = e - g.chk_off[s], r = g.seg_r[s];
            int bad = 0;
            if (j < 2 * r) {
                if (ent[u] == -1) bad = DEV_ERR_TABLE;
                else if (ent[u] < 0 || (int64_t)ent[u] >= num_pages) bad = DEV_ERR_PAGE;
            } else if (ent[u] != -1) {
                bad = DEV_ERR_TABLE;
            }
            if (bad) {
                atomicOr(&g.seg_bad[s], bad);
                err |= bad;
            }
            if (j >= r && j < 2 * r) {   // a B page: give it to every sorted position of the segment
                for (int q = g.seg_off[s]; q < g.seg_off[s + 1]; ++q) spages[(int64_t)q * RP + (j - r)] = ent[u];
            }
        }
    }
    __syncthreads();
    const int p = threadIdx.x;
    if (p < T) {
        const int32_t tt = g.sorted[p];
        int32_t a = -1, r = 0;
        if (p < g.n_valid) {
            const int s = find_seg(g.seg_off, nseg, p);
            if (!g.seg_bad[s]) {
                a = g.seg_a[s];
                r = g.seg_r[s];
            }
        }
        sorted_tok[p] = int4{tt, a, r, 0};
    }
    if (err) atomicOr(err_word, err);
}

// ---- decode, T <= 64: streaming kernel ----------------------------------------------------------
//
// Grid n_tiles x S workgroups, about one per CU.  Workgroup (tile, split) owns output columns
// [16 NW tile, 16 NW (tile + 1)) and the K chunk [kb, ke) of split.  A wave's vector-memory loads
// retire in issue order, so a wave that waits on a dependent chain (ids -> ranks -> page table ->
// pages) must not also have the W stream queued in front of it.  Hence two kinds of wave:
//  * NW W-waves: each issues its whole W slice (16 output columns x the K chunk) at once, stages its
//    share of x's K chunk in LDS (the MFMA A operand of every wave), and writes x W partials;
//  * one meta-wave: reads the ids and ranks, groups the <= 64 tokens by adapter with wave ballots,
//    takes this tile's blocks of 16 pages from the batch's A-page list (adapters in order of first
//    token, pages 0..r-1 each), computes s x A for them over the same K chunk as extra MFMA columns
//    (the shrink), and validates and publishes its share of the adapters' page-table rows.
// Outputs: float32 partials of x W and of s x A, one per split; k_decode_finish adds them in split
// order.  The workgroup has a single barrier (x staged).
template <int MB, int KS, int NW>   // T <= 16 MB; K chunk <= 32 KS; NW W-waves of 16 columns
__global__ __launch_bounds__((NW + 1) * 64, 1) void k_decode_stream(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, const uint16_t *__restrict__ pages,
    int64_t num_pages, const int32_t *__restrict__ pt, int32_t stride, const int32_t *__restrict__ ids,
    const int32_t *__restrict__ ranks, const float *__restrict__ scale, int32_t max_adapters, int32_t max_rank,
    int32_t T, int32_t H, int32_t S, int32_t n_tiles, int32_t RP, float *__restrict__ ypart,
    float *__restrict__ vpart, int4 *__restrict__ sorted_tok, int32_t *__restrict__ spages,
    int *__restrict__ err_word) {
    constexpr int TP = MB * 16;
    constexpr int XS = KS * 32;        // LDS row of x (elements), swizzled in 16-byte pieces
    extern __shared__ __align__(16) char lds_raw[];
    uint16_t *xs = reinterpret_cast<uint16_t *>(lds_raw);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int tile = blockIdx.x % n_tiles, split = blockIdx.x / n_tiles;
    const int ksteps = H / 32;
    const int kb = (int)((int64_t)ksteps * split / S) * 32, ke = (int)((int64_t)ksteps * (split + 1) / S) * 32;
    const int nst = (ke - kb) / 32;
    const int lrow = lane & 15, lk = (lane >> 4) * 8;
    const u32x4_t zero = u32x4_t{0, 0, 0, 0};

    if (wave < NW) {
        // ------------------------------------------------------------------ W-wave
        // x's K chunk goes straight to LDS (no registers); 16-byte piece c of row `row` lands in
        // slot c ^ (row & 15), so the 16 rows an MFMA operand read touches hit distinct banks.
        // Rows >= T and pieces past the chunk hold copies of valid data: their results are never
        // stored and their K steps are never read.
        constexpr int XI = TP * KS * 4 / 64;   // wave-wide direct-to-LDS loads
        for (int i = wave; i < XI; i += NW) {
            const int L = i * 64 + lane;
            const int row = L / (KS * 4), c = (L % (KS * 4)) ^ (row & 15);
            const bool live = row < T && c * 8 < ke - kb;
            const uint16_t *src = x + (int64_t)(live ? row : 0) * H + kb + (live ? c * 8 : 0);
            __builtin_amdgcn_global_load_lds((glob_void *)src, (lds_void *)(xs + i * 64 * 8), 16, 0, 0);
        }
        const int wn = tile * NW * 16 + wave * 16 + lrow;   // output column this lane loads
        const bool wlive = wn < H;
        const uint16_t *wr = W + (int64_t)(wlive ? wn : 0) * H + kb + lk;
        u32x4_t wreg[KS];
#pragma unroll
        for (int st = 0; st < KS; ++st) wreg[st] = load16(wr + 32 * min(st, max(nst - 1, 0)));
        __builtin_amdgcn_sched_barrier(0);   // keep every W load ahead of the barrier
        // vector-memory ops retire in order: waiting until only the KS W loads are outstanding
        // means this wave's x pieces are in LDS.  A plain barrier follows (a __syncthreads
        // fence would wait for the W loads too).
        __builtin_amdgcn_s_waitcnt((KS & 15) | ((KS >> 4) << 14) | 0xF70);
        workgroup_barrier();
        f32x4_t acc[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < KS; ++st) {   // branch-free: steps past the chunk multiply by zero
            const u32x4_t wb = st < nst ? wreg[st] : zero;
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                const int row = m * 16 + lrow;
                const u32x4_t xa = load16(xs + row * XS + (((st * 4 + (lk >> 3)) ^ (row & 15)) << 3));
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa),
                                                                 __builtin_bit_cast(bf16x8_t, wb), acc[m], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);   // keep each K step's LDS reads next to its MFMAs
        }
        // accumulator layout: lane holds rows 4*(lane/16)+i of column lane%16
        if (wlive) {
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = m * 16 + (lane >> 4) * 4 + i;
                    if (t < T) ypart[((int64_t)split * T + t) * H + wn] = acc[m][i];
                }
        }
        return;
    }

    // ---------------------------------------------------------------------- meta-wave (lane = token)
    int err = 0;
    int32_t key = -1, r = 0;
    {
        const int32_t a = lane < T ? ids[lane] : -1;
        const int32_t rr = ranks[a >= 0 && a < max_adapters ? a : 0];
        if (a != -1) {
            if (a < -1 || a >= max_adapters) err |= DEV_ERR_ID;
            else if (rr < 0 || rr > max_rank) err |= DEV_ERR_RANK;
            else if (rr > 0) { key = a; r = rr; }
        }
    }
    // group by key with ballots: rank within key, count, first lane; segments in first-lane order
    int rank_in = 0, cnt = 0, first = lane;
    {
        uint64_t remaining = __ballot(key >= 0);
        while (remaining) {
            const int leader = __ffsll((unsigned long long)remaining) - 1;
            const int32_t lkey = __shfl(key, leader, 64);
            const uint64_t m = __ballot(key == lkey);
            if (key == lkey) {
                rank_in = __popcll(m & ((1ull << lane) - 1ull));
                cnt = __popcll(m);
                first = leader;
            }
            remaining &= ~m;
        }
    }
    const uint64_t first_mask = __ballot(key >= 0 && rank_in == 0);
    const int nseg = __popcll(first_mask);
    const int my_seg = key >= 0 ? __popcll(first_mask & ((1ull << first) - 1ull)) : -1;
    // lane s < nseg describes segment s: the s-th first lane
    int32_t seg_lane = 0;
    {
        uint64_t fm = first_mask;
        for (int s = 0; s < nseg; ++s) {
            const int l = __ffsll((unsigned long long)fm) - 1;
            if (lane == s) seg_lane = l;
            fm &= fm - 1;
        }
    }
    const int32_t seg_a = __shfl(key, seg_lane, 64), seg_r = __shfl(r, seg_lane, 64), seg_n = __shfl(cnt, seg_lane, 64);
    const bool segl = lane < nseg;
    // prefix sums over segments: pages (r) and tokens (n)
    int32_t poff = segl ? seg_r : 0, toff = segl ? seg_n : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t y1 = __shfl_up(poff, off, 64), y2 = __shfl_up(toff, off, 64);
        if (lane >= off) { poff += y1; toff += y2; }
    }
    const int32_t npages = __shfl(poff, 63, 64), nvalid = __shfl(toff, 63, 64);
    poff -= segl ? seg_r : 0;   // exclusive
    toff -= segl ? seg_n : 0;
    // sorted position of this lane's token: grouped tokens first (segments in order), then the rest
    const int idrank = __popcll(__ballot(lane < T && key < 0) & ((1ull << lane) - 1ull));
    const int32_t seg_first_pos = __shfl(toff, max(my_seg, 0), 64);   // every lane shuffles
    const int my_pos = key >= 0 ? seg_first_pos + rank_in : nvalid + idrank;

    // this tile's page blocks: pages [16 b, 16 b + 16) of the list, b = tile + k * n_tiles
    f32x4_t pacc[MB];
    for (int b = tile; b * 16 < npages; b += n_tiles) {
        const int p = min(b * 16 + lrow, npages - 1);
        const bool plive = b * 16 + lrow < npages;
        int sg = 0;   // segment of page p: last s with poff[s] <= p
        for (int s = 1; s < nseg; ++s) sg += __shfl(poff, s, 64) <= p ? 1 : 0;
        const int32_t pa = __shfl(seg_a, sg, 64), pj = p - __shfl(poff, sg, 64);
        int32_t pid = pt[(int64_t)pa * stride + pj];
        if (pid < 0 || (int64_t)pid >= num_pages) pid = 0;   // the row is reported below; token dropped
        const uint16_t *ap = pages + (int64_t)pid * H + kb + lk;
        u32x4_t preg[KS];
#pragma unroll
        for (int st = 0; st < KS; ++st) preg[st] = load16(ap + 32 * min(st, max(nst - 1, 0)));
        if (b == tile) workgroup_barrier();   // x staged (the workgroup's only barrier)
#pragma unroll
        for (int m = 0; m < MB; ++m) pacc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            const u32x4_t bb = plive && st < nst ? preg[st] : zero;
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                const int row = m * 16 + lrow;
                const u32x4_t xa = load16(xs + row * XS + (((st * 4 + (lk >> 3)) ^ (row & 15)) << 3));
                pacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa),
                                                                  __builtin_bit_cast(bf16x8_t, bb), pacc[m], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        const float sc = scale[pa];
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = m * 16 + (lane >> 4) * 4 + i;
                const int32_t key_t = __shfl(key, t & 63, 64);   // outside any condition: all lanes active
                if (plive && t < T && key_t == pa) vpart[((int64_t)t * RP + pj) * S + split] = sc * pacc[m][i];
            }
    }
    if (tile * 16 >= npages) workgroup_barrier();   // no page block: still meet the barrier once

    // publish: segments s = blockIdx.x + k * gridDim.x -- check the page-table row, then write the
    // segment's sorted-token records and B page ids; workgroup 0 also writes the ungrouped tokens
    for (int s = blockIdx.x; s < nseg; s += gridDim.x) {
        const int32_t a = __shfl(seg_a, s, 64), rs = __shfl(seg_r, s, 64);
        const int32_t q0 = __shfl(toff, s, 64), qn = __shfl(seg_n, s, 64);
        const int lim = min(2 * rs + 1, stride);
        int32_t ent[3];
        int bad = 0;
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int j = lane + 64 * u;
            ent[u] = pt[(int64_t)a * stride + min(j, lim - 1)];
        }
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int j = lane + 64 * u;
            if (j >= lim) continue;
            if (j < 2 * rs) {
                if (ent[u] == -1) bad |= DEV_ERR_TABLE;
                else if (ent[u] < 0 || (int64_t)ent[u] >= num_pages) bad |= DEV_ERR_PAGE;
            } else if (ent[u] != -1) {
                bad |= DEV_ERR_TABLE;
            }
        }
        for (int off = 32; off > 0; off >>= 1) bad |= __shfl_xor(bad, off, 64);
        err |= bad;
        // B page ids to every sorted position of the segment
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int j = lane + 64 * u;
            if (j >= rs && j < 2 * rs)
                for (int q = q0; q < q0 + qn; ++q) spages[(int64_t)q * RP + (j - rs)] = ent[u];
        }
        if (key == a) sorted_tok[my_pos] = int4{lane, bad ? -1 : a, bad ? 0 : rs, 0};
    }
    // id/rank faults are per lane and every workgroup sees them: workgroup 0 reports them; page-table
    // faults were already OR-reduced over the wave by the workgroup that checked the row
    for (int off = 32; off > 0; off >>= 1) err |= __shfl_xor(err, off, 64);
    if (blockIdx.x == 0 && lane < T && key < 0) sorted_tok[my_pos] = int4{lane, -1, 0, 0};
    if (lane == 0) {
        const int mine = blockIdx.x == 0 ? err : err & (DEV_ERR_TABLE | DEV_ERR_PAGE);
        if (mine) atomicOr(err_word, mine);
    }
}

// ---- decode, 64 < T <= 256: shrink workgroups + base workgroups side by side ---------------------------
template <int MB, int WM>
__global__ __launch_bounds__(256, 2) void k_decode_main(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, const uint16_t *__restrict__ pages,
    int64_t num_pages, const int32_t *__restrict__ pt, int32_t stride, const int32_t *__restrict__ ids,
    const int32_t *__restrict__ ranks, const float *__restrict__ scale, int32_t max_adapters, int32_t max_rank,
    int32_t T, int32_t H, int32_t n_shrink, int32_t RP, float *__restrict__ vpart, int4 *__restrict__ sorted_tok,
    int32_t *__restrict__ spages, float *__restrict__ ypart, int *__restrict__ err_word) {
    extern __shared__ __align__(16) char lds_raw[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

    if ((int)blockIdx.x < n_shrink) {
        // ------------------------------------------------------------ shrink role
        DecGroup &g = *reinterpret_cast<DecGroup *>(lds_raw);
        const int err = dec_group<256>(g, ids, ranks, T, max_adapters, max_rank, stride);
        if (blockIdx.x == 0) dec_publish<256>(g, err, pt, stride, num_pages, T, RP, sorted_tok, spages, err_word);
        const int nseg = g.n_seg;
        const int nw = n_shrink * 4;
        for (int i = blockIdx.x * 4 + wave; i < g.n_items; i += nw) {
            const int s = find_seg(g.item_off, nseg, i);
            const int32_t r = g.seg_r[s], a = g.seg_a[s];
            const int local = i - g.item_off[s];
            const int chunk = local / r, j = local % r;
            const int32_t page = pt[(int64_t)a * stride + j];
            if (page < 0 || (int64_t)page >= num_pages) continue;   // reported by workgroup 0
            const int n = min(CHUNK, g.seg_n[s] - chunk * CHUNK);
            int32_t tok[CHUNK];
#pragma unroll
            for (int u = 0; u < CHUNK; ++u) tok[u] = u < n ? g.sorted[g.seg_off[s] + chunk * CHUNK + u] : 0;
            shrink_page_wave<2>((const char *)x, (const char *)(pages + (int64_t)page * H), (int64_t)H * 2, tok, n,
                                scale[a], j, vpart, RP, lane);
        }
        return;
    }

    // ---------------------------------------------------------------- base role
    constexpr int WK = 4 / WM;
    constexpr int TP = WM * MB * 16;   // padded rows
    float *red = reinterpret_cast<float *>(lds_raw);   // [WK][TP][NT]
    const int b = blockIdx.x - n_shrink;
    const int n_tiles = H / NT;
    const int tile = b % n_tiles, split = b / n_tiles;
    const int S = (gridDim.x - n_shrink) / n_tiles;
    const int wm = wave % WM, wk = wave / WM;
    const int n0 = tile * NT;
    const int G = S * WK, gi = split * WK + wk;
    const int ksteps = H / 32;
    const int kb = (int)((int64_t)ksteps * gi / G) * 32, ke = (int)((int64_t)ksteps * (gi + 1) / G) * 32;

    f32x4_t acc[MB][NB];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[m][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int lrow = lane & 15, lk = (lane >> 4) * 8;
    const uint16_t *xrow[MB];
    bool xval[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        const int row = (wm * MB + m) * 16 + lrow;
        xval[m] = row < T;
        xrow[m] = x + (int64_t)(xval[m] ? row : 0) * H + lk;
    }
    const uint16_t *wrow[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) wrow[nb] = W + (int64_t)(n0 + nb * 16 + lrow) * H + lk;

    constexpr int U = 2;   // K-steps of 32 in flight per wave
    int k = kb;
    for (; k + 32 * U <= ke; k += 32 * U) {
        u32x4_t xa[U][MB], wb[U][NB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) wb[u][nb] = load16(wrow[nb] + k + 32 * u);
#pragma unroll
            for (int m = 0; m < MB; ++m) xa[u][m] = xval[m] ? load16(xrow[m] + k + 32 * u) : u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa[u][m]),
                                                                         __builtin_bit_cast(bf16x8_t, wb[u][nb]),
                                                                         acc[m][nb], 0, 0, 0);
    }
    for (; k < ke; k += 32) {
        u32x4_t xa[MB], wb[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) wb[nb] = load16(wrow[nb] + k);
#pragma unroll
        for (int m = 0; m < MB; ++m) xa[m] = xval[m] ? load16(xrow[m] + k) : u32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc[m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa[m]),
                                                                     __builtin_bit_cast(bf16x8_t, wb[nb]),
                                                                     acc[m][nb], 0, 0, 0);
    }
    float *mine = red + (size_t)wk * TP * NT;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                mine[((wm * MB + m) * 16 + (lane >> 4) * 4 + i) * NT + nb * 16 + (lane & 15)] = acc[m][nb][i];
    __syncthreads();
    for (int p = threadIdx.x; p < T * (NT / 8); p += 256) {
        const int t = p / (NT / 8), c = (p % (NT / 8)) * 8;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
        for (int q = 0; q < WK; ++q) {
            const float *src = red + ((size_t)q * TP + t) * NT + c;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] += src[e];
        }
        float *dst = ypart + ((int64_t)split * T + t) * H + n0 + c;
        *reinterpret_cast<f32x4_t *>(dst) = f32x4_t{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<f32x4_t *>(dst + 4) = f32x4_t{o[4], o[5], o[6], o[7]};
    }
}

// ---- finishing kernel: sum partials + expand + round ---------------------------------------------------
// Grid (H/64 column tiles, ceil(T/8) groups of sorted tokens), 256 threads.  Round trip 1 reads, by
// sorted position only, the token record and its B page ids; round trip 2 reads the B rows' column
// slices, the v partials (summed in split order into LDS) and the x W partials.  Thread -> (token,
// 8 columns, quarter of j: j in [16 q, 16 q + 16)); quarters meet by lane shuffles.
template <int SY, int SV>
__global__ __launch_bounds__(256) void k_decode_finish(const int4 *__restrict__ sorted_tok,
                                                       const int32_t *__restrict__ spages,
                                                       const float *__restrict__ ypart, const float *__restrict__ vpart,
                                                       int32_t RP, const uint16_t *__restrict__ pages, int32_t H,
                                                       int32_t T, uint16_t *__restrict__ y) {
    __shared__ float s_v[8][64];
    const int n0 = blockIdx.x * 64;
    const int i = threadIdx.x >> 5, c = ((threadIdx.x >> 2) & 7) * 8, q = threadIdx.x & 3;
    const int sp = min((int)blockIdx.y * 8 + i, T - 1);
    const bool live_tok = (int)blockIdx.y * 8 + i < T;
    const int4 st = sorted_tok[sp];
    const int t = st.x, a = live_tok ? st.y : -1, r = st.z;
    const bool has = a >= 0;
    int32_t pid[16];
    {
        const int4 *pr = reinterpret_cast<const int4 *>(spages + (int64_t)sp * RP + 16 * min(q, RP / 16 - 1));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int4 v4 = pr[u];
            pid[4 * u] = v4.x;
            pid[4 * u + 1] = v4.y;
            pid[4 * u + 2] = v4.z;
            pid[4 * u + 3] = v4.w;
        }
    }
    // v[t][j] for j = 2 * (thread within token) + {0, 1}, summed over the SV partials in order
    {
        const int jj = (threadIdx.x & 31) * 2;
        float v0 = 0.f, v1 = 0.f;
        if (has && jj < RP) {
            const float *src = vpart + ((int64_t)t * RP + jj) * SV;
            float pv[2 * SV];
#pragma unroll
            for (int u = 0; u < 2 * SV; ++u) pv[u] = src[u];
#pragma unroll
            for (int u = 0; u < SV; ++u) {
                v0 += pv[u];
                v1 += pv[SV + u];
            }
        }
        s_v[i][jj] = jj < r ? v0 : 0.f;
        s_v[i][jj + 1] = jj + 1 < r ? v1 : 0.f;
    }
    f32x4_t part[SY][2];
    if (q == 0) {   // one lane of each quad needs the x W partials
#pragma unroll
        for (int s = 0; s < SY; ++s) {
            const float *src = ypart + ((int64_t)s * T + t) * H + n0 + c;
            part[s][0] = *reinterpret_cast<const f32x4_t *>(src);
            part[s][1] = *reinterpret_cast<const f32x4_t *>(src + 4);
        }
    }
    const int j0 = 16 * q;
    const bool qlive = has && j0 < r;
    u32x4_t bv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int32_t pg = qlive && j0 + u < r ? pid[u] : pid[0];
        bv[u] = load16(pages + (int64_t)(qlive ? pg : 0) * H + n0 + c);
    }
    __syncthreads();
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        float bf[8];
        unpack_bf16x8(bv[u], bf);
        const float w = (qlive && j0 + u < r) ? s_v[i][j0 + u] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(w, bf[e], o[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        o[e] += __shfl_xor(o[e], 1, 64);
        o[e] += __shfl_xor(o[e], 2, 64);
    }
    if (q == 0 && live_tok) {
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
        for (int s = 0; s < SY; ++s)   // base partials in split order, then the low-rank sum
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] += part[s][0][e];
                acc[e + 4] += part[s][1][e];
            }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += o[e];
        store16(y + (int64_t)t * H + n0 + c, pack_bf16x8(acc));
    }
}

// ---- float32 pools: grouping kernel + gathered shrink + plain VALU kernel ---------------------------
__global__ __launch_bounds__(256) void k_shrink_items_f32(
    const char *__restrict__ x, const char *__restrict__ pages, int32_t H, const int32_t *__restrict__ pt,
    int32_t stride, const float *__restrict__ scale, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ seg_a, const int32_t *__restrict__ seg_start, const int32_t *__restrict__ item_seg,
    const int32_t *__restrict__ item_row, const int32_t *__restrict__ ctrl, const int32_t *__restrict__ tok_r,
    float *__restrict__ v, int32_t R) {
    const int item = blockIdx.x;
    if (item >= ctrl[CTRL_NITEMS]) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int32_t s = item_seg[item], row0 = item_row[item];
    const int32_t n = min(seg_start[s + 1] - row0, CHUNK);
    const int32_t a = seg_a[s];
    const int32_t r = tok_r[perm[row0]];
    const int32_t j = blockIdx.y * 4 + wave;
    if (j >= r) return;
    int32_t tok[CHUNK];
#pragma unroll
    for (int i = 0; i < CHUNK; ++i) tok[i] = i < n ? perm[row0 + i] : 0;
    const int64_t row_bytes = (int64_t)H * 4;
    shrink_page_wave<4>(x, pages + (int64_t)pt[(int64_t)a * stride + j] * row_bytes, row_bytes, tok, n, scale[a], j,
                        v, R, lane);
}

// Grid (H/64 column tiles, ceil(T/16) token blocks); thread -> one token, 4 columns.
__global__ __launch_bounds__(256) void k_project_f32(const float *__restrict__ x, const float *__restrict__ W,
                                                     const float *__restrict__ pages, const int32_t *__restrict__ pt,
                                                     int32_t stride, const int32_t *__restrict__ tok_a,
                                                     const int32_t *__restrict__ tok_r, const float *__restrict__ v,
                                                     int32_t R, int32_t T, int32_t H, float *__restrict__ y) {
    const int t = blockIdx.y * 16 + (threadIdx.x >> 4);
    const int n = blockIdx.x * 64 + (threadIdx.x & 15) * 4;
    if (t >= T) return;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    const float *xr = x + (int64_t)t * H;
    for (int k = 0; k < H; k += 4) {
        const f32x4_t xv = *reinterpret_cast<const f32x4_t *>(xr + k);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const f32x4_t wv = *reinterpret_cast<const f32x4_t *>(W + (int64_t)(n + c) * H + k);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[c] = fmaf(xv[e], wv[e], o[c]);
        }
    }
    const int32_t a = tok_a[t];
    if (a >= 0) {
        const int32_t r = tok_r[t];
        const int32_t *prow = pt + (int64_t)a * stride + r;
        for (int32_t j = 0; j < r; ++j) {
            const f32x4_t b = *reinterpret_cast<const f32x4_t *>(pages + (int64_t)prow[j] * H + n);
            const float vj = v[(int64_t)t * R + j];
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c] = fmaf(vj, b[c], o[c]);
        }
    }
    *reinterpret_cast<f32x4_t *>(y + (int64_t)t * H + n) = f32x4_t{o[0], o[1], o[2], o[3]};
}

// ---- launchers -----------------------------------------------------------------------------------------
template <int MB, int KS, int NW>
static hipError_t launch_stream(const lora_pool *p, const Plan &plan, const Ws &ws, const void *x, const void *W,
                                const int32_t *ids, const int32_t *ranks, const int32_t *pt, const float *scale,
                                hipStream_t s) {
    const size_t lds = (size_t)MB * 16 * KS * 32 * 2;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)k_decode_stream<MB, KS, NW>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((k_decode_stream<MB, KS, NW>), dim3(plan.n_tiles * plan.ysplit), dim3((NW + 1) * 64), lds, s,
                       (const uint16_t *)x, (const uint16_t *)W, (const uint16_t *)p->pages, p->num_pages, pt,
                       2 * p->max_rank, ids, ranks, scale, p->max_adapters, p->max_rank, (int32_t)plan.T, p->hidden,
                       plan.ysplit, plan.n_tiles, plan.rp, ws.ypart, ws.v, (int4 *)ws.sorted_tok, ws.spages, p->dev_err);
    return hipGetLastError();
}

template <int MB, int WM>
static hipError_t launch_main(const lora_pool *p, const Plan &plan, const Ws &ws, const void *x, const void *W,
                              const int32_t *ids, const int32_t *ranks, const int32_t *pt, const float *scale,
                              hipStream_t s) {
    constexpr int WK = 4 / WM;
    const size_t red = (size_t)WK * WM * MB * 16 * NT * sizeof(float);
    const size_t lds = red > sizeof(DecGroup) ? red : sizeof(DecGroup);
    dim3 grid(plan.n_shrink + plan.n_tiles * plan.ysplit);
    hipLaunchKernelGGL((k_decode_main<MB, WM>), grid, dim3(256), lds, s, (const uint16_t *)x, (const uint16_t *)W,
                       (const uint16_t *)p->pages, p->num_pages, pt, 2 * p->max_rank, ids, ranks, scale,
                       p->max_adapters, p->max_rank, (int32_t)plan.T, p->hidden, plan.n_shrink, plan.rp, ws.v,
                       (int4 *)ws.sorted_tok, ws.spages, ws.ypart, p->dev_err);
    return hipGetLastError();
}

template <int SY, int SV>
static void launch_finish_t(const lora_pool *p, const Plan &plan, const Ws &ws, void *y, hipStream_t s) {
    dim3 grid(p->hidden / 64, (unsigned)((plan.T + 7) / 8));
    hipLaunchKernelGGL((k_decode_finish<SY, SV>), grid, dim3(256), 0, s, (const int4 *)ws.sorted_tok, ws.spages,
                       ws.ypart, ws.v, plan.rp, (const uint16_t *)p->pages, p->hidden, (int32_t)plan.T, (uint16_t *)y);
}

static hipError_t launch_finish(const lora_pool *p, const Plan &plan, const Ws &ws, void *y, hipStream_t s) {
    const int sy = plan.ysplit, sv = plan.stream ? plan.ysplit : 1;
    switch (sy * 16 + sv) {
#define LP_CASE(A, B) case A * 16 + B: launch_finish_t<A, B>(p, plan, ws, y, s); break;
        LP_CASE(1, 1) LP_CASE(2, 1) LP_CASE(4, 1) LP_CASE(8, 1)
        LP_CASE(2, 2) LP_CASE(3, 3) LP_CASE(4, 4) LP_CASE(5, 5) LP_CASE(6, 6) LP_CASE(7, 7) LP_CASE(8, 8)
#undef LP_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode(const lora_pool *p, const Plan &plan, const Ws &ws, const void *x, const void *W,
                         const int32_t *ids, const int32_t *ranks, const int32_t *pt, const float *scale, void *y,
                         hipStream_t s, hipEvent_t mid) {
    hipError_t e;
    if (plan.stream) {
        switch (plan.nw * 4096 + plan.mb * 64 + plan.ks) {
#define LP_CASE(M, K, N) case N * 4096 + M * 64 + K: e = launch_stream<M, K, N>(p, plan, ws, x, W, ids, ranks, pt, scale, s); break;
            LP_CASE(1, 8, 4) LP_CASE(1, 16, 4) LP_CASE(1, 32, 4) LP_CASE(1, 8, 8) LP_CASE(1, 16, 8) LP_CASE(1, 32, 8)
            LP_CASE(2, 8, 4) LP_CASE(2, 16, 4) LP_CASE(2, 32, 4) LP_CASE(2, 8, 8) LP_CASE(2, 16, 8) LP_CASE(2, 32, 8)
            LP_CASE(3, 8, 4) LP_CASE(3, 16, 4) LP_CASE(3, 32, 4) LP_CASE(3, 8, 8) LP_CASE(3, 16, 8) LP_CASE(3, 32, 8)
            LP_CASE(4, 8, 4) LP_CASE(4, 16, 4) LP_CASE(4, 32, 4) LP_CASE(4, 8, 8) LP_CASE(4, 16, 8) LP_CASE(4, 32, 8)
#undef LP_CASE
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (plan.wm * 8 + plan.mb) {
            case 2 * 8 + 4: e = launch_main<4, 2>(p, plan, ws, x, W, ids, ranks, pt, scale, s); break;
            case 4 * 8 + 4: e = launch_main<4, 4>(p, plan, ws, x, W, ids, ranks, pt, scale, s); break;
            case 1 * 8 + 1: e = launch_main<1, 1>(p, plan, ws, x, W, ids, ranks, pt, scale, s); break;
            case 1 * 8 + 2: e = launch_main<2, 1>(p, plan, ws, x, W, ids, ranks, pt, scale, s); break;
            case 1 * 8 + 3: e = launch_main<3, 1>(p, plan, ws, x, W, ids, ranks, pt, scale, s); break;
            case 1 * 8 + 4: e = launch_main<4, 1>(p, plan, ws, x, W, ids, ranks, pt, scale, s); break;
            default: return hipErrorInvalidValue;
        }
    }
    if (e != hipSuccess) return e;
    if (mid && (e = hipEventRecord(mid, s)) != hipSuccess) return e;
    return launch_finish(p, plan, ws, y, s);
}

hipError_t launch_f32(const lora_pool *p, const Plan &plan, const Ws &ws, const void *x, const void *W,
                      const int32_t *pt, const float *scale, void *y, hipStream_t s, hipEvent_t mid) {
    dim3 g1(plan.n_items_max, (p->max_rank + 3) / 4);
    hipLaunchKernelGGL(k_shrink_items_f32, g1, dim3(256), 0, s, (const char *)x, (const char *)p->pages, p->hidden,
                       pt, 2 * p->max_rank, scale, ws.perm, ws.seg_a, ws.seg_start, ws.item_seg, ws.item_row, ws.ctrl,
                       ws.tok_r, ws.v, p->max_rank);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (mid && (e = hipEventRecord(mid, s)) != hipSuccess) return e;
    dim3 grid(p->hidden / 64, (unsigned)((plan.T + 15) / 16));
    hipLaunchKernelGGL(k_project_f32, grid, dim3(256), 0, s, (const float *)x, (const float *)W,
                       (const float *)p->pages, pt, 2 * p->max_rank, ws.tok_a, ws.tok_r, ws.v, p->max_rank,
                       (int32_t)plan.T, p->hidden, (float *)y);
    return hipGetLastError();
}

}  // namespace lorapool
