// Decode-shaped projection (T <= 256 tokens, typically one per request): memory-bound, so the
// kernels are organised to stream W and the gathered A/B pages from HBM once, with as few
// dependent global round trips as possible and no in-kernel cross-workgroup waits (on this chip a
// device-scope fence writes back and invalidates the whole L2).
//
// Two launches per call:
//   T <= 64:       k_decode_stream   W, x and the batch's A pages in one streaming MFMA pass
//                                    (the shrink x A is extra MFMA columns of the same contraction)
//   64 < T <= 256: k_decode_wide     (k_decode_wide.hip) x streamed through LDS, W and the A pages
//                                    of per-adapter work units in registers, one MFMA pass
//   then           k_decode_finish   partial sums in split order + the expand sum_j v_j B_a[j, :]
//                                    from B rows gathered from their pages + one rounding
// ("S-LoRA, in depth", section "Merge or keep adapters separate": xW batched over all tokens
// whatever their adapter, plus two thin low-rank products per adapter; section "Kernels for a batch of
// mixed ranks": low-rank work follows tokens and ranks, adapter traffic follows distinct adapters.)
// Every sum has a fixed order, so results are bitwise reproducible.
//
// The float32 path (parity-only, small shapes) keeps the grouping kernel, a gathered shrink and a
// plain VALU kernel.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace lorapool {

constexpr int CHUNK = 16;      // tokens per shrink work item of the float32 path

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

// ---- wave-level grouping helpers for the T <= 64 kernel (lane = token) --------------------------------
// Lanes holding the same key >= 0 (itself included), through a wave-private open-addressing table of
// 128 slots in LDS: each lane claims its key's slot by compare-and-swap, then sets its bit in the
// slot's mask.  At most 64 keys, so a free slot always exists.  Lanes with key < 0 get 0.
struct GroupTab {
    int32_t key[128];
    unsigned long long mask[128];
};
__device__ __forceinline__ uint64_t same_key_lanes(int32_t key, int lane, GroupTab *g) {
    g->key[lane] = -1;
    g->key[lane + 64] = -1;
    g->mask[lane] = 0ull;
    g->mask[lane + 64] = 0ull;
    uint64_t m = 0;
    uint32_t h = ((uint32_t)key * 0x9E3779B1u) >> 25;
    if (key >= 0) {
        for (int probe = 0; probe < 128; ++probe) {
            const int32_t old = atomicCAS(&g->key[h], -1, key);
            if (old == -1 || old == key) break;
            h = (h + 1) & 127;
        }
        atomicOr(&g->mask[h], 1ull << lane);
    }
    if (key >= 0) m = g->mask[h];   // LDS operations of one wave complete in order
    return m;
}

// ---- decode, T <= 64: one streaming pass over W, x and the batch's A pages ------------------------
// Grid: n_tiles column tiles of 64 x S splits of K, 256 threads (four waves, one per SIMD).  Wave w
// owns the w-th quarter of its split's K range for all 64 columns of the tile:
//  * x: its T x (K quarter) slice is read with row-contiguous loads, written to a private LDS
//    region and read back in the MFMA operand layout.  A load that covers 16 rows x 64 bytes (the
//    operand layout) costs the CU's load path about twice what a row-contiguous one does;
//  * W: 16 x 32 operand tiles, DS steps in flight.  A shallow queue streams W as fast as a deep
//    one and keeps the latency of the metadata loads queued behind it near one microsecond;
//  * the shrink: block `tile` of the batch's A-page list (adapters in segment order, pages
//    0..r-1 each, 16 pages a block) is 16 extra MFMA columns over the same K quarter.  Each wave
//    works the block out itself (ids -> ranks -> grouping -> page table) at fixed steps of its W
//    loop, so the dependent loads ride between W steps and no wave waits for another.
// The four K-quarter partials are summed in LDS in wave order.  Outputs: float32 partials of x W
// (ypart[split]) and of s x A (vpart[..][split]), and, from the workgroups that own a segment, its
// checked page-table row as sorted-token records and B page ids for k_decode_finish.
template <int MB, int KQ>
struct StreamShape {
    static constexpr int TP = MB * 16;                        // padded token rows
    static constexpr int P = KQ * 4;                          // 16-byte x pieces per row of a K quarter
    static constexpr int RS = 68, PS = 20;                    // row strides (floats) of the sum buffers
    // per wave: its x slice, later overwritten by its x W partial and its block-0 page partial
    static constexpr size_t XSLICE = (size_t)TP * P * 16, PART = (size_t)TP * (RS + PS) * 4;
    static constexpr size_t REGION = XSLICE > PART ? XSLICE : PART;
    static constexpr size_t PBYTES = (size_t)4 * TP * PS * 4;                 // further page blocks' partials
    static constexpr size_t GBYTES = (size_t)4 * sizeof(GroupTab);            // grouping tables
    static constexpr size_t LDS = 4 * REGION + PBYTES + GBYTES;
};

template <int MB, int KQ, bool DBG>
__device__ __forceinline__ void decode_stream_body(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, const uint16_t *__restrict__ pages,
    int64_t num_pages, const int32_t *__restrict__ pt, int32_t stride, const int32_t *__restrict__ ids,
    const int32_t *__restrict__ ranks, const float *__restrict__ scale, int32_t max_adapters, int32_t max_rank,
    int32_t T, int32_t H, int32_t S, int32_t n_tiles, int32_t RP, float *__restrict__ ypart,
    float *__restrict__ vpart, int4 *__restrict__ sorted_tok, int32_t *__restrict__ spages,
    int *__restrict__ err_word, int32_t *__restrict__ dbg_gather) {
    using SH = StreamShape<MB, KQ>;
    constexpr int TP = SH::TP, P = SH::P, RS = SH::RS, PS = SH::PS;
    constexpr int SWZ = P < 16 ? P - 1 : 15;          // piece c of row r sits in slot c ^ (r & SWZ)
    constexpr int DS = KQ < 2 ? KQ : 2;               // W steps in flight ahead of the MFMA step
    constexpr int S1 = KQ > 1 ? 1 : 0;                // step that consumes the ranks (grouping)
    constexpr int S2 = KQ > 5 ? 5 : KQ - 1;           // step that consumes the page-table entries
    constexpr int XI = TP * P / 64;                   // row-contiguous x loads per wave (= MB * KQ)
    extern __shared__ __align__(16) char lds_raw[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int lrow = lane & 15, lq = lane >> 4;
    const u32x4_t zero = u32x4_t{0, 0, 0, 0};

    // XCD-aware order: consecutive workgroups go to the 8 XCDs in turn, so the splits are spread
    // over XCDs and each XCD's L2 holds one or two K chunks of x
    int tile, split;
    if ((gridDim.x & 7) == 0 && 8 % S == 0) {
        const int per = 8 / S;
        split = (blockIdx.x & 7) / per;
        tile = (blockIdx.x >> 3) * per + (blockIdx.x & 7) % per;
    } else {
        tile = blockIdx.x % n_tiles;
        split = blockIdx.x / n_tiles;
    }
    const int ksteps = H / 32, G = 4 * S, gq = split * 4 + wave;
    const int s0 = (int)((int64_t)ksteps * gq / G);
    const int nst = (int)((int64_t)ksteps * (gq + 1) / G) - s0;   // K steps of this wave, <= KQ
    const int kq = s0 * 32;
    const int n0 = tile * 64;
    char *region = lds_raw + (size_t)wave * SH::REGION;
    uint16_t *xs = reinterpret_cast<uint16_t *>(region);
    float *pred = reinterpret_cast<float *>(lds_raw + 4 * SH::REGION);
    GroupTab *gtab = reinterpret_cast<GroupTab *>(lds_raw + 4 * SH::REGION + SH::PBYTES) + wave;

    // ---- issue the ids, then x (row-contiguous).  Every CU of an XCD reads the same x chunk, so each
    // workgroup starts at its own piece (rotation by tile) and the first misses spread over many lines
    // instead of queueing on one.  Rows >= T and pieces past the wave's K steps load valid stand-in
    // data: the MFMA rows and K steps they feed are never stored or never run.
    const int32_t a_raw = ids[min(lane, T - 1)];
    // one W load (step 0, first 16 columns) goes out with x: the first touch of the wave's W rows
    // (address translation, a cold HBM row) then overlaps x's instead of following it
    const uint16_t *wr = W + (int64_t)(n0 + lrow) * H + kq + lq * 8;
    const u32x4_t wfirst = load16(wr);
    __builtin_amdgcn_sched_barrier(0);
    u32x4_t xv[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i) {
        const int L = ((i + tile) % XI) * 64 + lane, row = L / P, c = (L % P) ^ (row & SWZ);
        const bool live = row < T && c < nst * 4;
        xv[i] = load16(x + (int64_t)(live ? row : 0) * H + kq + (live ? c * 8 : 0));
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- ids -> key, then the ranks
    int err = 0;
    const int32_t a_tok = lane < T ? a_raw : -1;
    const int32_t rr = ranks[a_tok >= 0 && a_tok < max_adapters ? a_tok : 0];
    __builtin_amdgcn_sched_barrier(0);

    // ---- x slice to LDS (the wave's own region: no barrier), then the first DS steps of W.  W waits
    // for x: issued together, the W misses delay x, and nothing can use W before x is in LDS.
#pragma unroll
    for (int i = 0; i < XI; ++i) store16(xs + (size_t)(((i + tile) % XI) * 64 + lane) * 8, xv[i]);
    const int slast = max(nst - 1, 0);
    u32x4_t wv[KQ][4];
#pragma unroll
    for (int st = 0; st < DS; ++st)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
            wv[st][nb] = st == 0 && nb == 0 ? wfirst : load16(wr + (int64_t)(16 * nb) * H + 32 * min(st, slast));
    __builtin_amdgcn_sched_barrier(0);

    // metadata produced at steps S1 / S2
    int32_t key = -1, seg_a = 0, seg_r = 0, seg_n = 0, poff = 0, toff = 0, my_pos = 0, nseg = 0, npages = 0;
    int32_t pa = 0, pj = 0, pid = 0, ent[2] = {-1, -1};
    int64_t pidx = 0;
    float sc = 0.f;
    bool plive = false;
    const int32_t *ptc = pt;   // page-table entry of this lane's page (lane % 16)
    u32x4_t pv[KQ];
    f32x4_t acc[MB][4];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[m][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t xk[KQ][MB];   // the A operands of every step, kept for block 0's page MFMAs
    auto xop = [&](int st, int m) {   // MFMA A operand: rows m*16 + lrow, K step st
        const int row = m * 16 + lrow;
        return load16(xs + (size_t)(row * P + ((st * 4 + lq) ^ (row & SWZ))) * 8);
    };

    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < KQ; ++st) {
        if (st + DS < KQ) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                wv[st + DS][nb] = load16(wr + (int64_t)(16 * nb) * H + 32 * min(st + DS, slast));
        }
        if (st == S1) {
            // validate the ids and ranks; key = adapter of a token with a nonzero rank, else -1
            int32_t r = 0, rk = rr;
            asm volatile("" : "+v"(rk));   // keep the first use of the ranks at this step
            if (a_tok != -1) {
                if (a_tok < -1 || a_tok >= max_adapters) err |= DEV_ERR_ID;
                else if (rk < 0 || rk > max_rank) err |= DEV_ERR_RANK;
                else if (rk > 0) { key = a_tok; r = rk; }
            }
            // group: the lanes sharing this lane's key, its first lane, this lane's rank among them
            const uint64_t same = same_key_lanes(key, lane, gtab);
            const int first = key >= 0 ? __ffsll((unsigned long long)same) - 1 : lane;
            const int rank_in = __popcll(same & ((1ull << lane) - 1ull)), cnt = __popcll(same);
            // segments ordered by the quarter count of their rank, ceil(r / 16), from 4 down to 1, then by
            // first token: the finishing kernel's groups of 8 sorted tokens then mostly share their live
            // quarters, and its waves for quarters past every rank of a group skip their loads
            const int cls = key >= 0 ? (r + 15) >> 4 : 0;   // 1..4 (r <= 64)
            const bool fl = key >= 0 && first == lane;
            const uint64_t fm4 = __ballot(fl && cls == 4), fm3 = __ballot(fl && cls == 3), fm2 = __ballot(fl && cls == 2),
                           fm1 = __ballot(fl && cls == 1);
            nseg = __popcll(fm4 | fm3 | fm2 | fm1);
            const uint64_t fmc = cls == 4 ? fm4 : cls == 3 ? fm3 : cls == 2 ? fm2 : fm1;
            const int above = (cls < 4 ? __popcll(fm4) : 0) + (cls < 3 ? __popcll(fm3) : 0) + (cls < 2 ? __popcll(fm2) : 0);
            const int my_seg = key >= 0 ? above + __popcll(fmc & ((1ull << first) - 1ull)) : 0;
            // lane s < nseg describes segment s (segments in the order above): the first
            // lanes write their segment's adapter, rank and token count to the table, lane s reads
            int32_t *segtab = gtab->key;   // the claimed slots are no longer needed
            __builtin_amdgcn_wave_barrier();
            if (key >= 0 && first == lane) {
                segtab[my_seg] = key;
                segtab[64 + my_seg] = r;
                reinterpret_cast<int32_t *>(gtab->mask)[my_seg] = cnt;
            }
            __builtin_amdgcn_wave_barrier();
            const bool segl = lane < nseg;
            seg_a = segl ? segtab[lane] : 0;
            seg_r = segl ? segtab[64 + lane] : 0;
            seg_n = segl ? reinterpret_cast<int32_t *>(gtab->mask)[lane] : 0;
            poff = wave_incl_scan(seg_r, lane);
            toff = wave_incl_scan(seg_n, lane);
            npages = __builtin_amdgcn_readlane(poff, 63);
            const int32_t nvalid = __builtin_amdgcn_readlane(toff, 63);
            poff -= seg_r;   // exclusive
            toff -= seg_n;
            const int idrank = __popcll(__ballot(lane < T && key < 0) & ((1ull << lane) - 1ull));
            const int32_t seg_first_pos = __shfl(toff, my_seg, 64);
            my_pos = key >= 0 ? seg_first_pos + rank_in : nvalid + idrank;
            // page of this lane's column (lane % 16) in the workgroup's first block, and its segment:
            // one ballot per column counts the segments that start at or before the page
            const int p = tile * 16 + lrow;
            plive = p < npages;
            int sg = 0;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const uint64_t mk = __ballot(segl && poff <= tile * 16 + c);
                if (lrow == c) sg = max(__popcll(mk) - 1, 0);
            }
            pa = __shfl(seg_a, sg, 64);
            pj = p - __shfl(poff, sg, 64);
            pidx = plive ? (int64_t)pa * stride + pj : 0;
            ptc = pt + pidx;
            pid = *ptc;
            sc = scale[plive ? pa : 0];
        }
        if (st == S2) {
            // the page-table row of the segment this workgroup publishes first (used at the end)
            const int ps = (int)blockIdx.x < nseg ? (int)blockIdx.x : 0;
            int32_t a_pub = __shfl(seg_a, ps, 64), r_pub = __shfl(seg_r, ps, 64);
            if ((int)blockIdx.x >= nseg) a_pub = r_pub = 0;   // nothing to publish: read entry 0
            const int lim = min(2 * r_pub + 1, stride);
#pragma unroll
            for (int u = 0; u < 2; ++u) ent[u] = pt[(int64_t)a_pub * stride + min(lane + 64 * u, lim - 1)];
            // this block's pages: lane loads page (lane % 16), K rows kq + 32 s + 8 (lane / 16) + [0, 8)
            int32_t pg = pid;
            const bool pok = plive && pg >= 0 && (int64_t)pg < num_pages;   // bad rows are reported by the publisher
            const uint16_t *pr = pok ? pages + (int64_t)pg * H + kq + lq * 8 : x + lq * 8;
#pragma unroll
            for (int s2 = 0; s2 < KQ; ++s2) pv[s2] = load16(pr + 32 * min(s2, slast));
            plive = pok;
        }
        // steps past the wave's K range multiply by zero (branch-free: a branch here would let the
        // compiler sink the W loads into it, after the point they are meant to be issued)
        const bool sl = st < nst;
#pragma unroll
        for (int m = 0; m < MB; ++m) xk[st][m] = xop(st, m);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const u32x4_t wb = sl ? wv[st][nb] : zero;
#pragma unroll
            for (int m = 0; m < MB; ++m)
                acc[m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xk[st][m]),
                                                                     __builtin_bit_cast(bf16x8_t, wb), acc[m][nb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- page blocks: MFMA over the K quarter, scaled by s; the four quarters are summed in wave order
    // (block 0 takes its A operands from registers, further blocks re-read them from LDS)
    auto page_mfma = [&](const u32x4_t *pvb, float sc_col, f32x4_t *pacc, bool from_regs) {
#pragma unroll
        for (int m = 0; m < MB; ++m) pacc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < KQ; ++s2) {   // columns of dead pages hold stand-in data and are never stored
            const u32x4_t bb = s2 < nst ? pvb[s2] : zero;
#pragma unroll
            for (int m = 0; m < MB; ++m)
                pacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, from_regs ? xk[s2][m] : xop(s2, m)),
                                                                  __builtin_bit_cast(bf16x8_t, bb), pacc[m], 0, 0, 0);
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) pacc[m] *= sc_col;
    };
    // thread -> column lrow (its own lane's page), rows lane/16 + 4 (wave + 4 u); the partial of wave
    // w, row t sits at part(w) + t * pstride
    auto page_store = [&](const float *part0, size_t wstride, int pstride, bool live_col, int32_t a_col,
                          int32_t j_col, int32_t pid_col) {
        float v[MB];
#pragma unroll
        for (int u = 0; u < MB; ++u) {
            const int t = lq + 4 * (wave + 4 * u);
            const float *q = part0 + t * pstride + lrow;
            v[u] = ((q[0] + q[wstride]) + q[2 * wstride]) + q[3 * wstride];
        }
#pragma unroll
        for (int u = 0; u < MB; ++u) {
            const int t = lq + 4 * (wave + 4 * u);
            const int32_t key_t = __shfl(key, t & 63, 64), pos_t = __shfl(my_pos, t & 63, 64);
            if (live_col && t < T && key_t == a_col) {
                vpart[((int64_t)pos_t * RP + j_col) * S + split] = v[u];
                if constexpr (DBG) dbg_put(dbg_gather + (int64_t)t * stride + j_col, pid_col);
            }
        }
    };
    f32x4_t pacc0[MB];
    asm volatile("" ::"v"(ent[0]), "v"(ent[1]));   // the publisher's row has landed: keep its loads at S2
    // ---- publish (wave 0): segments s = blockIdx.x + k gridDim.x -- check the page-table row, then
    // write the segment's sorted-token records and B page ids; workgroup 0 also writes the
    // ungrouped tokens.  It needs only the grouping and the row, so it goes out here, while the
    // block's A pages are still in flight, and not after the reduction (the publishing workgroups
    // were the last to end: 0.5 us less per call at 64 tokens)
    if (wave == 0) {
        for (int s = blockIdx.x; s < nseg; s += gridDim.x) {
            const int32_t a = __shfl(seg_a, s, 64), rs = __shfl(seg_r, s, 64);
            const int32_t q0 = __shfl(toff, s, 64), qn = __shfl(seg_n, s, 64);
            const int lim = min(2 * rs + 1, stride);
            if (s != (int)blockIdx.x) {
#pragma unroll
                for (int u = 0; u < 2; ++u) ent[u] = pt[(int64_t)a * stride + min(lane + 64 * u, lim - 1)];
            }
            int bad = 0;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
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
#pragma unroll
            for (int u = 0; u < 2; ++u) {
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
    page_mfma(pv, sc, pacc0, true);
    // further blocks (more pages than 16 n_tiles: rare) while x is still in LDS, through their own buffer
    for (int b = tile + n_tiles; b * 16 < npages; b += n_tiles) {
        const int p = b * 16 + lrow;
        bool live = p < npages;
        int sg = 0;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const uint64_t mk = __ballot(lane < nseg && poff <= b * 16 + c);
            if (lrow == c) sg = max(__popcll(mk) - 1, 0);
        }
        const int32_t a2 = __shfl(seg_a, sg, 64), j2 = p - __shfl(poff, sg, 64);
        const int32_t pg = pt[live ? (int64_t)a2 * stride + j2 : 0];
        const float sc2 = scale[live ? a2 : 0];
        live = live && pg >= 0 && (int64_t)pg < num_pages;
        const uint16_t *pr = live ? pages + (int64_t)pg * H + kq + lq * 8 : x + lq * 8;
        u32x4_t pv2[KQ];
#pragma unroll
        for (int s2 = 0; s2 < KQ; ++s2) pv2[s2] = load16(pr + 32 * min(s2, slast));
        f32x4_t pacc[MB];
        page_mfma(pv2, sc2, pacc, false);
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) pred[((size_t)wave * TP + m * 16 + lq * 4 + i) * PS + lrow] = pacc[m][i];
        __syncthreads();
        page_store(pred, (size_t)TP * PS, PS, live, a2, j2, pg);
        __syncthreads();
    }

    // ---- the wave's x slice is no longer read: its region takes the wave's x W partial [TP][RS] and
    // block-0 page partial [TP][PS]; one barrier, then every wave sums its share in wave order
    {
        float *mine = reinterpret_cast<float *>(region);
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i) mine[(m * 16 + lq * 4 + i) * RS + nb * 16 + lrow] = acc[m][nb][i];
        float *pm = mine + TP * RS;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) pm[(m * 16 + lq * 4 + i) * PS + lrow] = pacc0[m][i];
    }
    __syncthreads();
    {
        const float *red = reinterpret_cast<const float *>(lds_raw);
        constexpr size_t WS = SH::REGION / 4;   // floats between the waves' regions
        f32x4_t v[MB];
#pragma unroll
        for (int u = 0; u < MB; ++u) {          // thread -> row e / 16, columns 4 (e % 16) + [0, 4)
            const int e = threadIdx.x + 256 * u;
            const float *q = red + (size_t)(e >> 4) * RS + 4 * (e & 15);
            v[u] = ((*reinterpret_cast<const f32x4_t *>(q) + *reinterpret_cast<const f32x4_t *>(q + WS)) +
                    *reinterpret_cast<const f32x4_t *>(q + 2 * WS)) + *reinterpret_cast<const f32x4_t *>(q + 3 * WS);
        }
        // written through to memory: the finishing kernel reads each partial once, and lines left dirty
        // in this XCD's L2 would be flushed at the end of the kernel before it can start (measured:
        // 0.2 us less per call for streaming stores than for plain ones, 0.5 us less again written through)
#pragma unroll
        for (int u = 0; u < MB; ++u) {   // row of the token's sorted position, so the finish needs no record to find it
            const int e = threadIdx.x + 256 * u, t = e >> 4;
            const int pos_t = __shfl(my_pos, t & 63, 64);
            if (t < T) store16_wt(ypart + ((int64_t)split * T + pos_t) * H + n0 + 4 * (e & 15), __builtin_bit_cast(u32x4_t, v[u]));
        }
        page_store(red + TP * RS, WS, PS, plive, pa, pj, pid);
    }

}

// The stream kernel for one slot, and for the n slots of one call (blockIdx.z = the slot; the slots
// share x and the ids).  The one-slot kernel keeps the short argument block.
template <int MB, int KQ>
__global__ __launch_bounds__(256, 1) void k_decode_stream(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, const uint16_t *__restrict__ pages,
    int64_t num_pages, const int32_t *__restrict__ pt, int32_t stride, const int32_t *__restrict__ ids,
    const int32_t *__restrict__ ranks, const float *__restrict__ scale, int32_t max_adapters, int32_t max_rank,
    int32_t T, int32_t H, int32_t S, int32_t n_tiles, int32_t RP, float *__restrict__ ypart,
    float *__restrict__ vpart, int4 *__restrict__ sorted_tok, int32_t *__restrict__ spages,
    int *__restrict__ err_word) {
    decode_stream_body<MB, KQ, false>(x, W, pages, num_pages, pt, stride, ids, ranks, scale, max_adapters, max_rank, T,
                                      H, S, n_tiles, RP, ypart, vpart, sorted_tok, spages, err_word, nullptr);
}

// The debug instantiation (lora_debug_project): the same body, recording the A pages it reads per token.
template <int MB, int KQ>
__global__ __launch_bounds__(256, 1) void k_decode_stream_dbg(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, const uint16_t *__restrict__ pages,
    int64_t num_pages, const int32_t *__restrict__ pt, int32_t stride, const int32_t *__restrict__ ids,
    const int32_t *__restrict__ ranks, const float *__restrict__ scale, int32_t max_adapters, int32_t max_rank,
    int32_t T, int32_t H, int32_t S, int32_t n_tiles, int32_t RP, float *__restrict__ ypart,
    float *__restrict__ vpart, int4 *__restrict__ sorted_tok, int32_t *__restrict__ spages,
    int *__restrict__ err_word, int32_t *__restrict__ dbg_gather) {
    decode_stream_body<MB, KQ, true>(x, W, pages, num_pages, pt, stride, ids, ranks, scale, max_adapters, max_rank, T,
                                     H, S, n_tiles, RP, ypart, vpart, sorted_tok, spages, err_word, dbg_gather);
}

template <int MB, int KQ>
__global__ __launch_bounds__(256, 1) void k_decode_stream_slots(
    const SlotPtrs sp, const uint16_t *__restrict__ pages, int64_t num_pages,
    int32_t stride, const int32_t *__restrict__ ids, const int32_t *__restrict__ ranks, const float *__restrict__ scale,
    int32_t max_adapters, int32_t max_rank, int32_t T, int32_t H, int32_t S, int32_t n_tiles, int32_t RP,
    int *__restrict__ err_word) {
    const int z = blockIdx.z;
    decode_stream_body<MB, KQ, false>((const uint16_t *)sp.x[z], (const uint16_t *)sp.W[z], pages, num_pages, sp.pt[z],
                                      stride, ids, ranks,
                                      scale, max_adapters, max_rank, T, H, S, n_tiles, RP, sp.ypart[z], sp.v[z],
                                      (int4 *)sp.sorted_tok[z], sp.spages[z], err_word, nullptr);
}

// ---- finishing kernel: sum partials + expand + round ---------------------------------------------------
// Grid (H/64 column tiles, ceil(T/8) groups of sorted tokens), 256 threads.  Wave q takes quarter q of
// j (j in [16 q, 16 q + 16)) for all 8 tokens of the group; lane -> (token i, 8 columns c).  Two
// dependent round trips:
//  1. by sorted position only: the token record, this quarter's B page ids, the x W partials of splits
//     q, q + 4 and the v partials of two j's (both stored by sorted position);
//  2. the quarter's 16 B-row slices -- skipped by a wave whose quarter lies past the rank of every
//     token of the group (a wave-uniform branch: half the quarters are past the rank at mixed ranks).
// The four waves' sums (x W partials and expand terms) are then added in LDS in a fixed order,
// ((q0 + q1) + (q2 + q3)), and wave 0 rounds and stores.
template <int SY, int SV, bool DBG>
__device__ __forceinline__ void decode_finish_body(const int4 *__restrict__ sorted_tok, const int32_t *__restrict__ spages,
                                                   const float *__restrict__ ypart, const float *__restrict__ vpart,
                                                   int32_t RP, const uint16_t *__restrict__ pages, int64_t num_pages,
                                                   int32_t H, int32_t T, uint16_t *__restrict__ y,
                                                   const DebugOut dbg = DebugOut{}, int32_t stride = 0) {
    constexpr int SQ = (SY + 3) / 4;   // x W splits per wave (wave q takes splits q, q + 4)
    __shared__ float s_v[8][64];
    __shared__ f32x4_t s_o[4][8][8][2];   // [quarter][token][column group][half]
    const int n0 = blockIdx.x * 64;
    const int q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int i = lane >> 3, cg = lane & 7, c = cg * 8;
    const int sp = min((int)blockIdx.y * 8 + i, T - 1);
    const bool live_tok = (int)blockIdx.y * 8 + i < T;
    // ---- round trip 1: the records, the B page ids, and the x W and v partials (stored by sorted
    // position, so they need nothing from the record)
    f32x4_t part[SQ][2];
#pragma unroll
    for (int k = 0; k < SQ; ++k) {
        part[k][0] = part[k][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (q + 4 * k < SY) {   // wave-uniform: with fewer than four splits the other waves load none
            const float *src = ypart + ((int64_t)(q + 4 * k) * T + sp) * H + n0 + c;
            part[k][0] = *reinterpret_cast<const f32x4_t *>(src);
            part[k][1] = *reinterpret_cast<const f32x4_t *>(src + 4);
        }
    }
    const int vi = threadIdx.x >> 5, jj = (threadIdx.x & 31) * 2;   // v: token vi of the group, j's jj, jj + 1
    const int vsp = min((int)blockIdx.y * 8 + vi, T - 1);
    float pv[2 * SV];
    {
        const float *src = vpart + ((int64_t)vsp * RP + min(jj, RP - 2)) * SV;
#pragma unroll
        for (int u = 0; u < 2 * SV; ++u) pv[u] = src[u];
    }
    const int4 st = sorted_tok[sp];
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
    // The records were written (and their page ids checked) by the first kernel; the token index and
    // the page ids are clamped here all the same, so that a workspace overwritten by another call
    // can only give wrong values, never an address outside the buffers.
    const int t = min(max(st.x, 0), T - 1), a = live_tok ? st.y : -1;
    const bool has = a >= 0;
    const int r = has ? st.z : 0;
    const int j0 = 16 * q;
    const bool qlive = has && j0 < r;
    const bool wlive = __builtin_amdgcn_readfirstlane((int)(__ballot(qlive) != 0ull)) != 0;
    if constexpr (DBG) {   // the B pages this thread multiplies into the token's output, and the grouping it used
        if (live_tok) {
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (qlive && j0 + u < r) dbg_put(dbg.gather + (int64_t)t * stride + r + j0 + u, pid[u]);
            if (q == 0 && cg == 0) {
                dbg_put(dbg.order + 2 * sp, t);
                dbg_put(dbg.order + 2 * sp + 1, a);
            }
        }
    }
    // ---- v[t][j] summed over the splits in order (entries past the rank were never written and are
    // never used: the expand below takes j < r only)
    {
        float v0 = 0.f, v1 = 0.f;
#pragma unroll
        for (int u = 0; u < SV; ++u) {
            v0 += pv[u];
            v1 += pv[SV + u];
        }
        s_v[vi][jj] = v0;
        s_v[vi][jj + 1] = v1;
    }
    // ---- this thread's x W splits
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
    for (int k = 0; k < SQ; ++k) {
        if (q + 4 * k < SY) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[e] += part[k][0][e];
                o[e + 4] += part[k][1][e];
            }
        }
    }
    // ---- round trip 2 (live waves; every load unconditional within them, stand-in addresses for dead
    // entries), then the quarter's expand.  Rows past the token's rank load a stand-in row and are
    // zeroed before use: the page they read (page 0, or the token's first B page) may hold any bits,
    // NaN included, and 0 * NaN is NaN.
    const u32x4_t zero = u32x4_t{0, 0, 0, 0};
    u32x4_t bv[16];
    uint32_t okm = 0;   // rows whose page id is in range
    if (wlive) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int32_t pg = qlive && j0 + u < r ? pid[u] : pid[0];
            const bool pok = pg >= 0 && (int64_t)pg < num_pages;
            okm |= pok ? 1u << u : 0u;
            bv[u] = load16(pages + (int64_t)(qlive && pok ? pg : 0) * H + n0 + c);
        }
    }
    __syncthreads();   // s_v
    if (wlive) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const bool lu = qlive && j0 + u < r && ((okm >> u) & 1u);
            float bf[8];
            unpack_bf16x8(lu ? bv[u] : zero, bf);
            const float w = lu ? s_v[i][j0 + u] : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = fmaf(w, bf[e], o[e]);
        }
    }
    s_o[q][i][cg][0] = f32x4_t{o[0], o[1], o[2], o[3]};
    s_o[q][i][cg][1] = f32x4_t{o[4], o[5], o[6], o[7]};
    __syncthreads();
    if (q == 0 && live_tok) {
        float f[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const f32x4_t sum = (s_o[0][i][cg][h] + s_o[1][i][cg][h]) + (s_o[2][i][cg][h] + s_o[3][i][cg][h]);
#pragma unroll
            for (int e = 0; e < 4; ++e) f[4 * h + e] = sum[e];
        }
        store16_nt(y + (int64_t)t * H + n0 + c, pack_bf16x8(f));
    }
}

template <int SY, int SV>
__global__ __launch_bounds__(256) void k_decode_finish(const int4 *__restrict__ sorted_tok, const int32_t *__restrict__ spages,
                                                       const float *__restrict__ ypart, const float *__restrict__ vpart,
                                                       int32_t RP, const uint16_t *__restrict__ pages, int64_t num_pages,
                                                       int32_t H, int32_t T, uint16_t *__restrict__ y) {
    decode_finish_body<SY, SV, false>(sorted_tok, spages, ypart, vpart, RP, pages, num_pages, H, T, y);
}

template <int SY, int SV>
__global__ __launch_bounds__(256) void k_decode_finish_dbg(const int4 *__restrict__ sorted_tok,
                                                           const int32_t *__restrict__ spages,
                                                           const float *__restrict__ ypart, const float *__restrict__ vpart,
                                                           int32_t RP, const uint16_t *__restrict__ pages,
                                                           int64_t num_pages, int32_t H, int32_t T,
                                                           uint16_t *__restrict__ y, const DebugOut dbg, int32_t stride) {
    decode_finish_body<SY, SV, true>(sorted_tok, spages, ypart, vpart, RP, pages, num_pages, H, T, y, dbg, stride);
}

template <int SY, int SV>
__global__ __launch_bounds__(256) void k_decode_finish_slots(const SlotPtrs sl, int32_t RP,
                                                             const uint16_t *__restrict__ pages, int64_t num_pages,
                                                             int32_t H, int32_t T) {
    const int z = blockIdx.z;
    decode_finish_body<SY, SV, false>((const int4 *)sl.sorted_tok[z], sl.spages[z], sl.ypart[z], sl.v[z], RP, pages,
                                      num_pages, H, T, (uint16_t *)sl.y[z]);
}

// ---- float32 pools: grouping kernel + gathered shrink + plain VALU kernel ---------------------------
template <bool DBG>
__global__ __launch_bounds__(256) void k_shrink_items_f32(
    const char *__restrict__ x, const char *__restrict__ pages, int32_t H, const int32_t *__restrict__ pt,
    int32_t stride, const float *__restrict__ scale, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ seg_a, const int32_t *__restrict__ seg_start, const int32_t *__restrict__ item_seg,
    const int32_t *__restrict__ item_row, const int32_t *__restrict__ ctrl, const int32_t *__restrict__ tok_r,
    float *__restrict__ v, int32_t R, const DebugOut dbg) {
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
    const int32_t pg = pt[(int64_t)a * stride + j];
    if constexpr (DBG) {   // the A page this wave multiplies into its tokens' v[j], and the grouping
        if (lane < n) {
            dbg_put(dbg.gather + (int64_t)tok[lane] * stride + j, pg);
            dbg_put(dbg.order + 2 * (row0 + lane), tok[lane]);
            dbg_put(dbg.order + 2 * (row0 + lane) + 1, a);
        }
    }
    shrink_page_wave<4>(x, pages + (int64_t)pg * row_bytes, row_bytes, tok, n, scale[a], j, v, R, lane);
}

// Grid (H/64 column tiles, ceil(T/16) token blocks); thread -> one token, 4 columns.
template <bool DBG>
__global__ __launch_bounds__(256) void k_project_f32(const float *__restrict__ x, const float *__restrict__ W,
                                                     const float *__restrict__ pages, const int32_t *__restrict__ pt,
                                                     int32_t stride, const int32_t *__restrict__ tok_a,
                                                     const int32_t *__restrict__ tok_r, const float *__restrict__ v,
                                                     int32_t R, int32_t T, int32_t H, float *__restrict__ y,
                                                     const DebugOut dbg) {
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
            if constexpr (DBG) dbg_put(dbg.gather + (int64_t)t * stride + r + j, prow[j]);
            const f32x4_t b = *reinterpret_cast<const f32x4_t *>(pages + (int64_t)prow[j] * H + n);
            const float vj = v[(int64_t)t * R + j];
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c] = fmaf(vj, b[c], o[c]);
        }
    }
    *reinterpret_cast<f32x4_t *>(y + (int64_t)t * H + n) = f32x4_t{o[0], o[1], o[2], o[3]};
}

// ---- launchers -----------------------------------------------------------------------------------------
template <int MB, int KQ>
static hipError_t launch_stream(const lora_pool *p, const Plan &plan, const void *x, const int32_t *ids,
                                const int32_t *ranks, const float *scale, const SlotPtrs &sp, int n, hipStream_t s,
                                const DebugOut *dbg) {
    constexpr size_t lds = StreamShape<MB, KQ>::LDS;
    static_assert(lds <= 160 * 1024, "stream kernel LDS");
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)k_decode_stream<MB, KQ>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void *)k_decode_stream_slots<MB, KQ>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void *)k_decode_stream_dbg<MB, KQ>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    if (dbg)
        hipLaunchKernelGGL((k_decode_stream_dbg<MB, KQ>), dim3(plan.n_tiles * plan.ysplit), dim3(256), lds, s,
                           (const uint16_t *)x, (const uint16_t *)sp.W[0], (const uint16_t *)p->pages, p->num_pages,
                           sp.pt[0], 2 * p->max_rank, ids, ranks, scale, p->max_adapters, p->max_rank,
                           (int32_t)plan.T, p->hidden, plan.ysplit, plan.n_tiles, plan.rp, sp.ypart[0], sp.v[0],
                           (int4 *)sp.sorted_tok[0], sp.spages[0], p->dev_err, dbg->gather);
    else if (n == 1)
        hipLaunchKernelGGL((k_decode_stream<MB, KQ>), dim3(plan.n_tiles * plan.ysplit), dim3(256), lds, s,
                           (const uint16_t *)x, (const uint16_t *)sp.W[0], (const uint16_t *)p->pages, p->num_pages,
                           sp.pt[0], 2 * p->max_rank, ids, ranks, scale, p->max_adapters, p->max_rank,
                           (int32_t)plan.T, p->hidden, plan.ysplit, plan.n_tiles, plan.rp, sp.ypart[0], sp.v[0],
                           (int4 *)sp.sorted_tok[0], sp.spages[0], p->dev_err);
    else
        hipLaunchKernelGGL((k_decode_stream_slots<MB, KQ>), dim3(plan.n_tiles * plan.ysplit, 1, n), dim3(256), lds,
                           s, sp, (const uint16_t *)p->pages, p->num_pages, 2 * p->max_rank, ids,
                           ranks, scale, p->max_adapters, p->max_rank, (int32_t)plan.T, p->hidden, plan.ysplit,
                           plan.n_tiles, plan.rp, p->dev_err);
    return hipGetLastError();
}

template <int SY, int SV>
static void launch_finish_t(const lora_pool *p, const Plan &plan, const SlotPtrs &sp, int n, hipStream_t s,
                            const DebugOut *dbg) {
    dim3 grid(p->hidden / 64, (unsigned)((plan.T + 7) / 8), n);
    if (dbg)
        hipLaunchKernelGGL((k_decode_finish_dbg<SY, SV>), grid, dim3(256), 0, s, (const int4 *)sp.sorted_tok[0],
                           sp.spages[0], sp.ypart[0], sp.v[0], plan.rp, (const uint16_t *)p->pages, p->num_pages,
                           p->hidden, (int32_t)plan.T, (uint16_t *)sp.y[0], *dbg, 2 * p->max_rank);
    else if (n == 1)
        hipLaunchKernelGGL((k_decode_finish<SY, SV>), grid, dim3(256), 0, s, (const int4 *)sp.sorted_tok[0],
                           sp.spages[0], sp.ypart[0], sp.v[0], plan.rp, (const uint16_t *)p->pages, p->num_pages,
                           p->hidden, (int32_t)plan.T, (uint16_t *)sp.y[0]);
    else
        hipLaunchKernelGGL((k_decode_finish_slots<SY, SV>), grid, dim3(256), 0, s, sp, plan.rp,
                           (const uint16_t *)p->pages, p->num_pages, p->hidden, (int32_t)plan.T);
}

static hipError_t launch_finish(const lora_pool *p, const Plan &plan, const SlotPtrs &sp, int n, hipStream_t s,
                                const DebugOut *dbg) {
    const int sy = plan.ysplit, sv = plan.ysplit;   // both decode kernels write S v partials
    switch (sy * 16 + sv) {
#define LP_CASE(A, B) case A * 16 + B: launch_finish_t<A, B>(p, plan, sp, n, s, dbg); break;
        LP_CASE(1, 1) LP_CASE(2, 1) LP_CASE(4, 1) LP_CASE(8, 1)
        LP_CASE(2, 2) LP_CASE(3, 3) LP_CASE(4, 4) LP_CASE(5, 5) LP_CASE(6, 6) LP_CASE(7, 7) LP_CASE(8, 8)
#undef LP_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode(const lora_pool *p, const Plan &plan, const void *x, const int32_t *ids,
                         const int32_t *ranks, const float *scale, const SlotPtrs &sp, int n, hipStream_t s,
                         hipEvent_t mid, const DebugOut *dbg) {
    hipError_t e;
    if (plan.stream) {
        switch (plan.mb * 64 + plan.ks) {
#define LP_CASE(M, K) case M * 64 + K: e = launch_stream<M, K>(p, plan, x, ids, ranks, scale, sp, n, s, dbg); break;
            LP_CASE(1, 1) LP_CASE(1, 2) LP_CASE(1, 4) LP_CASE(1, 8)
            LP_CASE(2, 1) LP_CASE(2, 2) LP_CASE(2, 4) LP_CASE(2, 8)
            LP_CASE(3, 1) LP_CASE(3, 2) LP_CASE(3, 4) LP_CASE(3, 8)
            LP_CASE(4, 1) LP_CASE(4, 2) LP_CASE(4, 4) LP_CASE(4, 8)
#undef LP_CASE
            default: return hipErrorInvalidValue;
        }
    } else {
        e = launch_decode_wide(p, plan, x, ids, ranks, scale, sp, n, s, dbg);
    }
    if (e != hipSuccess) return e;
    if (mid && (e = hipEventRecord(mid, s)) != hipSuccess) return e;
    return launch_finish(p, plan, sp, n, s, dbg);
}

hipError_t launch_f32(const lora_pool *p, const Plan &plan, const Ws &ws, const void *x, const void *W,
                      const int32_t *pt, const float *scale, void *y, hipStream_t s, hipEvent_t mid,
                      const DebugOut *dbg) {
    const DebugOut d = dbg ? *dbg : DebugOut{};
    dim3 g1(plan.n_items_max, (p->max_rank + 3) / 4);
    hipLaunchKernelGGL(dbg ? k_shrink_items_f32<true> : k_shrink_items_f32<false>, g1, dim3(256), 0, s,
                       (const char *)x, (const char *)p->pages, p->hidden, pt, 2 * p->max_rank, scale, ws.perm,
                       ws.seg_a, ws.seg_start, ws.item_seg, ws.item_row, ws.ctrl, ws.tok_r, ws.v, p->max_rank, d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (mid && (e = hipEventRecord(mid, s)) != hipSuccess) return e;
    dim3 grid(p->hidden / 64, (unsigned)((plan.T + 15) / 16));
    hipLaunchKernelGGL(dbg ? k_project_f32<true> : k_project_f32<false>, grid, dim3(256), 0, s, (const float *)x,
                       (const float *)W, (const float *)p->pages, pt, 2 * p->max_rank, ws.tok_a, ws.tok_r, ws.v,
                       p->max_rank, (int32_t)plan.T, p->hidden, (float *)y, d);
    return hipGetLastError();
}

// Fill n int32 entries with `value` (the debug outputs start at -1).
__global__ __launch_bounds__(256) void k_fill_i32(int32_t *__restrict__ dst, int64_t n, int32_t value) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) dst[i] = value;
}

hipError_t launch_fill_i32(int32_t *dst, int64_t n, int32_t value, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)blocks), dim3(256), 0, s, dst, n, value);
    return hipGetLastError();
}

}  // namespace lorapool
