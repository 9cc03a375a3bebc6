// Decode-shaped projection (T <= 256 tokens, typically one per request): memory-bound, so the
// kernels are organised to stream W and the gathered A/B pages from HBM once, with as few
// dependent global round trips as possible.
//
// Two launches per call:
//   k_decode_main    two kinds of workgroup side by side, no waiting on each other:
//                    * shrink workgroups: group the tokens by adapter in LDS (every one of them
//                      derives the same grouping from the ids), then one wave per gathered A page
//                      computes v[t][j] = s_a <x_t, A_a[:, j]> for the tokens of that adapter
//                      (the first of the "two skinny matmuls", "S-LoRA, in depth", section "Merge
//                      or keep adapters separate").  Workgroup 0 also validates the page-table
//                      rows in use and publishes the sorted token list.
//                    * base workgroups: y0 = x W with bf16 MFMA, split over K; each writes a
//                      float32 partial for its 64-column tile.
//   k_decode_finish  per (64-column tile, 8 sorted tokens): sums the K partials in split order,
//                    adds the expand sum_j v[t][j] B_a[j, n] from B rows gathered from their
//                    pages, and rounds once to bfloat16.
// Every sum has a fixed order, so results are bitwise reproducible.
//
// The float32 path (parity-only, small shapes) keeps the grouping kernel, a gathered shrink and
// a plain VALU kernel.
#include "device_common.h"
#include "internal.h"

namespace lorapool {

constexpr int CHUNK = 16;      // tokens per shrink work item
constexpr int DEC_T = 256;     // most tokens on the decode path
constexpr int NT = 64;         // columns per base tile
constexpr int NB = NT / 16;    // 16-column MFMA blocks per tile

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

// ---- in-LDS grouping of <= 256 tokens by adapter (256 threads, thread = token) -------------------
struct DecGroup {
    int32_t key[DEC_T];        // adapter id, or -1 (none, rank 0, id or rank out of range)
    int32_t r[DEC_T];
    int32_t seg[DEC_T];        // segment of a token with key >= 0
    int32_t seg_a[DEC_T], seg_r[DEC_T], seg_n[DEC_T], seg_bad[DEC_T];
    int32_t seg_off[DEC_T + 1];    // first sorted position of each segment
    int32_t item_off[DEC_T + 1];   // first shrink item of each segment
    int32_t chk_off[DEC_T + 1];    // first page-table entry to check of each segment (workgroup 0)
    int32_t sorted[DEC_T];     // sorted position -> token
    int32_t wsum[8];
    int32_t n_seg, n_valid, n_items, n_chk;
};

// exclusive prefix of v over the 256 threads; *total gets the sum (all threads)
__device__ int32_t scan256(int32_t v, int32_t *wsum, int32_t *total) {
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
    int32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
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

__device__ int dec_group(DecGroup &g, const int32_t *__restrict__ ids, const int32_t *__restrict__ ranks,
                         int32_t T, int32_t max_adapters, int32_t max_rank, int32_t stride) {
    const int t = threadIdx.x;
    int err = 0;
    int32_t key = -1, r = 0;
    if (t < T) {
        const int32_t a = ids[t];
        if (a != -1) {
            if (a < -1 || a >= max_adapters) {
                err |= DEV_ERR_ID;
            } else {
                const int32_t rr = ranks[a];
                if (rr < 0 || rr > max_rank) err |= DEV_ERR_RANK;
                else if (rr > 0) { key = a; r = rr; }
            }
        }
    }
    g.key[t] = key;
    g.r[t] = r;
    g.seg_n[t] = 0;
    g.seg_bad[t] = 0;
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
    const int32_t sid = scan256(is_first, g.wsum, &nseg);
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
    // per segment (thread s): token offsets, shrink items, entries to check
    const int32_t n_s = t < nseg ? g.seg_n[t] : 0;
    const int32_t r_s = t < nseg ? g.seg_r[t] : 0;
    int32_t nvalid, nitems, nchk;
    const int32_t off = scan256(n_s, g.wsum, &nvalid);
    const int32_t ioff = scan256(r_s * ((n_s + CHUNK - 1) / CHUNK), g.wsum, &nitems);
    const int32_t coff = scan256(t < nseg ? min(2 * r_s + 1, stride) : 0, g.wsum, &nchk);
    if (t < nseg) {
        g.seg_off[t] = off;
        g.item_off[t] = ioff;
        g.chk_off[t] = coff;
    }
    // identity / invalid tokens go after the grouped ones, in token order
    int32_t nid;
    const int32_t idpos = scan256(t < T && key < 0, g.wsum, &nid);
    if (t == 0) {
        g.n_seg = nseg;
        g.n_valid = nvalid;
        g.n_items = nitems;
        g.n_chk = nchk;
        g.seg_off[nseg] = nvalid;
        g.item_off[nseg] = nitems;
        g.chk_off[nseg] = nchk;
    }
    __syncthreads();
    if (t < T) g.sorted[key >= 0 ? g.seg_off[my_seg] + rank_in : nvalid + idpos] = t;
    __syncthreads();
    return err;
}

// ---- launch 1: shrink workgroups + base workgroups -------------------------------------------------
template <int MB, int WM>
__global__ __launch_bounds__(256, 2) void k_decode_main(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, const uint16_t *__restrict__ pages,
    int64_t num_pages, const int32_t *__restrict__ pt, int32_t stride, const int32_t *__restrict__ ids,
    const int32_t *__restrict__ ranks, const float *__restrict__ scale, int32_t max_adapters, int32_t max_rank,
    int32_t T, int32_t H, int32_t n_shrink, float *__restrict__ v, int4 *__restrict__ sorted_tok,
    float *__restrict__ ypart, int *__restrict__ err_word) {
    extern __shared__ __align__(16) char lds_raw[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int R = max_rank;

    if ((int)blockIdx.x < n_shrink) {
        // ------------------------------------------------------------ shrink role
        DecGroup &g = *reinterpret_cast<DecGroup *>(lds_raw);
        int err = dec_group(g, ids, ranks, T, max_adapters, max_rank, stride);
        const int nseg = g.n_seg;
        if (blockIdx.x == 0) {
            // validate every page-table row in use; publish the sorted token list
            for (int e0 = threadIdx.x; e0 < g.n_chk; e0 += 256 * 8) {
                int32_t ent[8];
                int sg[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int e = e0 + u * 256;
                    sg[u] = -1;
                    if (e < g.n_chk) {
                        sg[u] = find_seg(g.chk_off, nseg, e);
                        const int j = e - g.chk_off[sg[u]];
                        ent[u] = pt[(int64_t)g.seg_a[sg[u]] * stride + j];
                    }
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (sg[u] < 0) continue;
                    const int j = e0 + u * 256 - g.chk_off[sg[u]];
                    const int r = g.seg_r[sg[u]];
                    int bad = 0;
                    if (j < 2 * r) {
                        if (ent[u] == -1) bad = DEV_ERR_TABLE;
                        else if (ent[u] < 0 || (int64_t)ent[u] >= num_pages) bad = DEV_ERR_PAGE;
                    } else if (ent[u] != -1) {
                        bad = DEV_ERR_TABLE;
                    }
                    if (bad) {
                        atomicOr(&g.seg_bad[sg[u]], bad);
                        err |= bad;
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
        // one wave per (segment, token chunk, page j)
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
                                scale[a], j, v, R, lane);
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
    // accumulator layout (16x16 block): lane holds rows 4*(lane/16)+i of column lane%16
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

// ---- launch 2: sum partials + expand + round --------------------------------------------------------
// Grid (H/64 column tiles, ceil(T/8) groups of sorted tokens).  Thread -> (token, 8 columns, quarter
// of j); the four quarters meet by lane shuffles.  All loads are unconditional from valid addresses
// (indices clamped into the token's own page row) so they issue together; only the sums select.
template <int S>
__global__ __launch_bounds__(256) void k_decode_finish(const int4 *__restrict__ sorted_tok,
                                                       const float *__restrict__ ypart,
                                                       const float *__restrict__ v, int32_t R,
                                                       const int32_t *__restrict__ pt, int32_t stride,
                                                       const uint16_t *__restrict__ pages, int32_t H, int32_t T,
                                                       uint16_t *__restrict__ y) {
    const int n0 = blockIdx.x * 64;
    const int i = threadIdx.x >> 5, c = ((threadIdx.x >> 2) & 7) * 8, q = threadIdx.x & 3;
    const int sp = blockIdx.y * 8 + i;
    if (sp >= T) return;   // whole quads leave together
    const int4 st = sorted_tok[sp];
    const int t = st.x, a = st.y, r = st.z;
    f32x4_t part[S][2];
#pragma unroll
    for (int s = 0; s < S; ++s) {   // every lane loads; only quarter 0 adds them in
        const float *src = ypart + ((int64_t)s * T + t) * H + n0 + c;
        part[s][0] = *reinterpret_cast<const f32x4_t *>(src);
        part[s][1] = *reinterpret_cast<const f32x4_t *>(src + 4);
    }
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    if (a >= 0) {
        const int j0 = q * r / 4, j1 = (q + 1) * r / 4;
        const int32_t *prow = pt + (int64_t)a * stride + r;
        const float *vt = v + (int64_t)t * R;
        int32_t pid[16];
        float vj[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int jj = min(j0 + u, r - 1);
            pid[u] = prow[jj];
            vj[u] = vt[jj];
        }
        u32x4_t bv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) bv[u] = load16(pages + (int64_t)pid[u] * H + n0 + c);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            float bf[8];
            unpack_bf16x8(bv[u], bf);
            const float w = j0 + u < j1 ? vj[u] : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = j0 + u < j1 ? fmaf(w, bf[e], o[e]) : o[e];
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        o[e] += __shfl_xor(o[e], 1, 64);
        o[e] += __shfl_xor(o[e], 2, 64);
    }
    if (q == 0) {
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
        for (int s = 0; s < S; ++s)   // base partials in split order, then the low-rank sum
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
template <int MB, int WM>
static hipError_t launch_main(const lora_pool *p, const Plan &plan, const Ws &ws, const void *x, const void *W,
                              const int32_t *ids, const int32_t *ranks, const int32_t *pt, const float *scale,
                              hipStream_t s) {
    constexpr int WK = 4 / WM;
    const size_t red = (size_t)WK * WM * MB * 16 * NT * sizeof(float);
    const size_t lds = red > sizeof(DecGroup) ? red : sizeof(DecGroup);
    const int n_tiles = p->hidden / NT;
    dim3 grid(plan.n_shrink + n_tiles * plan.ysplit);
    hipLaunchKernelGGL((k_decode_main<MB, WM>), grid, dim3(256), lds, s, (const uint16_t *)x, (const uint16_t *)W,
                       (const uint16_t *)p->pages, p->num_pages, pt, 2 * p->max_rank, ids, ranks, scale,
                       p->max_adapters, p->max_rank, (int32_t)plan.T, p->hidden, plan.n_shrink, ws.v,
                       (int4 *)ws.sorted_tok, ws.ypart, p->dev_err);
    return hipGetLastError();
}

hipError_t launch_decode(const lora_pool *p, const Plan &plan, const Ws &ws, const void *x, const void *W,
                         const int32_t *ids, const int32_t *ranks, const int32_t *pt, const float *scale, void *y,
                         hipStream_t s, hipEvent_t mid) {
    hipError_t e;
    switch (plan.wm * 8 + plan.mb) {
        case 1 * 8 + 1: e = launch_main<1, 1>(p, plan, ws, x, W, ids, ranks, pt, scale, s); break;
        case 1 * 8 + 2: e = launch_main<2, 1>(p, plan, ws, x, W, ids, ranks, pt, scale, s); break;
        case 1 * 8 + 3: e = launch_main<3, 1>(p, plan, ws, x, W, ids, ranks, pt, scale, s); break;
        case 1 * 8 + 4: e = launch_main<4, 1>(p, plan, ws, x, W, ids, ranks, pt, scale, s); break;
        case 2 * 8 + 4: e = launch_main<4, 2>(p, plan, ws, x, W, ids, ranks, pt, scale, s); break;
        case 4 * 8 + 4: e = launch_main<4, 4>(p, plan, ws, x, W, ids, ranks, pt, scale, s); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    if (mid && (e = hipEventRecord(mid, s)) != hipSuccess) return e;
    dim3 grid(p->hidden / 64, (unsigned)((plan.T + 7) / 8));
#define LP_FINISH(SS)                                                                                            \
    hipLaunchKernelGGL(k_decode_finish<SS>, grid, dim3(256), 0, s, (const int4 *)ws.sorted_tok, ws.ypart, ws.v,     \
                       p->max_rank, pt, 2 * p->max_rank, (const uint16_t *)p->pages, p->hidden, (int32_t)plan.T, \
                       (uint16_t *)y)
    switch (plan.ysplit) {
        case 1: LP_FINISH(1); break;
        case 2: LP_FINISH(2); break;
        case 4: LP_FINISH(4); break;
        case 8: LP_FINISH(8); break;
        default: return hipErrorInvalidValue;
    }
#undef LP_FINISH
    return hipGetLastError();
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
