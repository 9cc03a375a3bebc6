// Decode-shaped projection for 64 < T <= 256 tokens: one streaming pass over W, x and the batch's A
// pages, then k_decode_finish (split partials + expand + rounding).
//
// ("S-LoRA, in depth", section "Merge or keep adapters separate": x W batched over all tokens whatever
// their adapter, plus two thin low-rank products per adapter; section "Kernels for a batch of mixed
// ranks": low-rank work follows tokens and ranks, adapter traffic follows distinct adapters.)
//
// Grid: n_tiles column tiles of 64 x S splits of K (chunks of 64), 512 threads (two waves per SIMD,
// so one feeds the MFMA pipe while the other waits for LDS).  Wave w owns rows 16 MBW w + [0, 16 MBW)
// (its tokens) x all 64 columns of the tile:
//  * x and W: the split's K range streams through LDS in chunks of 64 (x: [TP rows][64], three
//    stages; W: the tile's [64 rows][64], four stages, as it comes from HBM), loaded straight from
//    global memory into LDS, row-contiguous; each wave reads its own x rows and the chunk's W rows;
//  * the shrink: work units (adapter segment, 16 of its A pages, 16 of its tokens) dealt round robin,
//    tiles first, then waves; a unit's operands are its page rows (loaded row-contiguously into
//    registers, DW K steps in flight, and put into the MFMA operand layout through the wave's LDS
//    buffer) and its tokens' x rows, gathered from the LDS chunk by row index.  So the A pages of the
//    batch are read once per call and x A costs one MFMA per unit and K step.
// The grouping of tokens by adapter (segments by the quarter count of their rank, ceil(r / 16), from 4
// down to 1, then by first token; tokens in order within a segment) is worked out by every
// workgroup from the ids, deterministically, so all agree.
// Outputs as the T <= 64 kernel: float32 partials of x W (ypart[split]) and of s x A
// (vpart[pos][j][split]), rows in sorted-position order; the workgroups that own a segment check its page-table row and publish its
// sorted-token records and B page ids for the finishing kernel.
#include "device_common.h"
#include "internal.h"

namespace lorapool {
namespace wide {

constexpr int WT = 256;       // most tokens (thread t holds token t during the grouping)
constexpr int KC = 64;        // K chunk staged in LDS: two MFMA steps of 32
constexpr int NSTAGE = 3;     // x chunk stages (x chunk c + 2 loads while c computes; x sits in L2)
constexpr int NWS = 4;        // W chunk stages (W chunk c + 3 loads while c computes; W comes from HBM)
constexpr int DW = 8;         // K steps of page loads in flight per wave
#ifndef WIDE_UPW
#define WIDE_UPW 1
#endif
constexpr int UPW = WIDE_UPW;  // shrink units per wave and pass
constexpr int HSLOTS = 256;   // grouping hash slots (at most 256 keys); the hash keeps 8 bits
static_assert(HSLOTS == 256, "hash width");
constexpr int NW = 8;         // waves, one share of the rows each (two per SIMD)
constexpr int NTH = NW * 64;

struct WideGroup {
    int32_t hkey[HSLOTS];
    unsigned long long hmask[HSLOTS][4];   // tokens holding the slot's key, one bit each
    int32_t slot_seg[HSLOTS];
    int32_t seg_a[WT], seg_r[WT], seg_n[WT], seg_toff[WT + 1], seg_uoff[WT + 1];
    int32_t sorted[WT];                     // sorted position -> token
    int32_t pos[WT];                        // token -> sorted position
    int32_t pub_ent[2 * 64 + 1];           // page-table row of the segment being published
    int32_t wsum[3][NW];
    int32_t wcls[4][NW];                    // segment-first tokens per rank class and wave
    int32_t pub_bad, nseg, nvalid, nunits;
};

__device__ __forceinline__ int wswz(int r, int p) { return r * KC + ((p ^ ((r >> 1) & 7)) << 3); }

// Unit page rows are loaded row-contiguously, 8 page rows x 128 bytes (one chunk's K) per load, and each
// wave reorders them into the MFMA operand layout through a 2 KiB LDS buffer of its own (16 rows x 64 K,
// swizzled as wswz): loads of 16 rows x 64 bytes straight in the operand layout cost the load path about
// twice as much (1 us per projection at 2000 adapters).  The buffers sit after the W stages, over the
// grouping's hash arrays (dead once the grouping is done); the group struct moves up by what they do not
// cover.
constexpr int UBUF_BYTES = NW * UPW * 2048;
constexpr int UBUF_OVER = (int)(HSLOTS * 4 + HSLOTS * 4 * 8);   // hkey + hmask: the first fields of WideGroup
constexpr int GROUP_GAP = UBUF_BYTES > UBUF_OVER ? UBUF_BYTES - UBUF_OVER : 0;

// LDS-only barrier: a full __syncthreads would also wait for every outstanding global load
__device__ __forceinline__ void lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// last index s in [0, n) with off[s] <= i (off ascending, off[0] = 0)
__device__ __forceinline__ int last_leq(const int32_t *off, int n, int32_t i) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return lo;
}

}  // namespace wide
using namespace wide;

template <int MB16, bool DBG>
__device__ __forceinline__ void decode_wide_body(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, const uint16_t *__restrict__ pages,
    int64_t num_pages, const int32_t *__restrict__ pt, int32_t stride, const int32_t *__restrict__ ids,
    const int32_t *__restrict__ ranks, const float *__restrict__ scale, int32_t max_adapters, int32_t max_rank,
    int32_t T, int32_t H, int32_t S, int32_t n_tiles, int32_t RP, float *__restrict__ ypart,
    float *__restrict__ vpart, int4 *__restrict__ sorted_tok, int32_t *__restrict__ spages,
    int *__restrict__ err_word, int32_t *__restrict__ dbg_gather) {
    constexpr int TP = MB16 * 16;           // padded token rows
    constexpr int MBW = MB16 / NW;          // 16-row blocks per wave
    constexpr int XSTAGE = TP * KC;         // elements per x stage
    constexpr int WSTAGE = 64 * KC;         // elements per W stage
    constexpr int DX = TP / 64;             // x chunk loads per wave (1 KiB each)
    constexpr int DWL = 64 / 64;            // W chunk loads per wave
    static_assert(MB16 % NW == 0, "rows per wave");
    extern __shared__ __align__(16) char lds_raw[];
    uint16_t *xs = reinterpret_cast<uint16_t *>(lds_raw);
    uint16_t *wst = xs + NSTAGE * XSTAGE;
    WideGroup &g = *reinterpret_cast<WideGroup *>(lds_raw + (size_t)(NSTAGE * XSTAGE + NWS * WSTAGE) * 2 + GROUP_GAP);
    static_assert(offsetof(WideGroup, slot_seg) == UBUF_OVER, "the page buffers may cover hkey and hmask only");
    uint16_t *const ubuf = wst + NWS * WSTAGE;   // the waves' page buffers (used after the grouping)
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lrow = lane & 15, lq = lane >> 4;
    const bool tokt = tid < WT;                // threads 0..255 hold one token each in the grouping
    const u32x4_t zero = u32x4_t{0, 0, 0, 0};

    // XCD-aware order (consecutive workgroups go to the 8 XCDs in turn): the splits are spread over
    // XCDs, so each XCD's L2 holds one or two K ranges of x
    int tile, split;
    if ((gridDim.x & 7) == 0 && 8 % S == 0) {
        const int per = 8 / S;
        split = (blockIdx.x & 7) / per;
        tile = (blockIdx.x >> 3) * per + (blockIdx.x & 7) % per;
    } else {
        tile = blockIdx.x % n_tiles;
        split = blockIdx.x / n_tiles;
    }
    const int nck = H / KC;
    const int c0 = (int)((int64_t)nck * split / S), nch = (int)((int64_t)nck * (split + 1) / S) - c0;
    const int kb = c0 * KC, nst = 2 * nch;   // K steps of 32 of this workgroup
    const int n0 = tile * 64;

    // ---- chunks: one load fills 8 rows x 128 bytes of a stage; lane l lands in row 8c + l / 8, slot
    // l % 8, which holds piece (l % 8) ^ ((row >> 1) & 7) -- the piece the lane fetches.  x rows past T
    // read row T - 1 (never stored); W row n is W's row n0 + n.  Chunks past the split's range reload
    // chunk 0 (never read).
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc((void *)x, (short)0, T * H * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void *)(W + (int64_t)n0 * H), (short)0, 64 * H * 2, 0x00020000);
    uint32_t xoff[DX], woff;
#pragma unroll
    for (int i = 0; i < DX; ++i) {
        const int r = 8 * (NW * i + wave) + (lane >> 3), p = (lane & 7) ^ ((r >> 1) & 7);
        xoff[i] = (uint32_t)(min(r, T - 1) * H + kb + p * 8) * 2u;
    }
    {
        const int r = 8 * wave + (lane >> 3), p = (lane & 7) ^ ((r >> 1) & 7);
        woff = (uint32_t)(r * H + kb + p * 8) * 2u;
    }
    auto dma_x = [&](int c) {
        const int soff = (c < nch ? c : 0) * KC * 2;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < DX; ++i)
            lds_load16(rx, (lds_void *)(xs + (c % NSTAGE) * XSTAGE + 8 * (NW * i + wave) * KC), xoff[i], soff);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto dma_w = [&](int c) {
        const int soff = (c < nch ? c : 0) * KC * 2;
        __builtin_amdgcn_sched_barrier(0);
        lds_load16(rw, (lds_void *)(wst + (c % NWS) * WSTAGE + 8 * wave * KC), woff, soff);
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- ids first (the first wait is for them alone), then the first chunks: their first touches
    // overlap the grouping's round trips
    const int32_t a_raw = tid < T && tid < WT ? ids[tid] : -1;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NWS; ++c) dma_w(c);
#pragma unroll
    for (int c = 0; c < NSTAGE; ++c) dma_x(c);
    __builtin_amdgcn_sched_barrier(0);

    // ---- validate the ids and ranks; key = adapter of a token with a nonzero rank, else -1
    const int32_t rr = ranks[a_raw >= 0 && a_raw < max_adapters ? a_raw : 0];
    for (int i = tid; i < HSLOTS; i += NTH) {
        g.hkey[i] = -1;
#pragma unroll
        for (int w = 0; w < 4; ++w) g.hmask[i][w] = 0ull;
    }
    if (tid == 0) g.pub_bad = 0;
    int err = 0;
    int32_t key = -1, r_tok = 0;
    if (tokt && tid < T && a_raw != -1) {
        if (a_raw < -1 || a_raw >= max_adapters) err |= DEV_ERR_ID;
        else if (rr < 0 || rr > max_rank) err |= DEV_ERR_RANK;
        else if (rr > 0) { key = a_raw; r_tok = rr; }
    }
    lds_sync();

    // ---- grouping: each key claims a hash slot; every token sets its bit in the slot's mask (the
    // masks do not depend on the order of the atomics, so every workgroup derives the same grouping)
    int slot = 0;
    if (key >= 0) {
        uint32_t h = ((uint32_t)key * 0x9E3779B1u) >> 24;   // 8 bits: HSLOTS = 256
        for (int probe = 0; probe < HSLOTS; ++probe) {
            const int32_t old = atomicCAS(&g.hkey[h], -1, key);
            if (old == -1 || old == key) break;
            h = (h + 1) & (HSLOTS - 1);
        }
        slot = (int)h;
        atomicOr(&g.hmask[slot][tid >> 6], 1ull << (tid & 63));
    }
    lds_sync();
    int first = tid, rank_in = 0, cnt = 0;
    if (key >= 0) {
        unsigned long long m[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) m[w] = g.hmask[slot][w];
        first = -1;
#pragma unroll
        for (int w = 3; w >= 0; --w)
            if (m[w]) first = 64 * w + __ffsll((unsigned long long)m[w]) - 1;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            cnt += __popcll(m[w]);
            rank_in += w < (tid >> 6) ? __popcll(m[w]) : w == (tid >> 6) ? __popcll(m[w] & ((1ull << (tid & 63)) - 1ull)) : 0;
        }
    }
    const int is_first = key >= 0 && first == tid;
    // segment ids: by the quarter count of the rank, ceil(r / 16), from 4 down to 1, then by first token
    // (the finishing kernel's groups of 8 sorted tokens then mostly share their live quarters, and its
    // waves for quarters past every rank of a group skip their loads)
    int nseg;
    {
        const int ord = is_first ? 4 - ((r_tok + 15) >> 4) : 0;   // 0..3 (r <= 64)
        uint64_t bl[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) bl[k] = __ballot(is_first && ord == k);
        if (lane == 0) {
#pragma unroll
            for (int k = 0; k < 4; ++k) g.wcls[k][wave] = __popcll(bl[k]);
        }
        lds_sync();
        int before = 0;
        nseg = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const int s = g.wcls[k][w];
                before += k < ord || (k == ord && w < wave) ? s : 0;
                nseg += s;
            }
        const uint64_t mine = ord == 0 ? bl[0] : ord == 1 ? bl[1] : ord == 2 ? bl[2] : bl[3];
        if (is_first) {
            const int sid = before + __popcll(mine & ((1ull << lane) - 1ull));
            g.slot_seg[slot] = sid;
            g.seg_a[sid] = key;
            g.seg_r[sid] = r_tok;
            g.seg_n[sid] = cnt;
        }
    }
    lds_sync();
    const int my_seg = key >= 0 ? g.slot_seg[slot] : -1;
    // per segment (thread s): first sorted position and first unit; per token: rank among the
    // ungrouped tokens
    {
        const bool sl = tokt && tid < nseg;
        const int n_s = sl ? g.seg_n[tid] : 0, r_s = sl ? g.seg_r[tid] : 0;
        const int u_s = ((r_s + 15) >> 4) * ((n_s + 15) >> 4);
        const int ungrouped = tokt && tid < T && key < 0;
        const int i0 = wave_incl_scan(n_s, lane), i1 = wave_incl_scan(u_s, lane), i2 = wave_incl_scan(ungrouped, lane);
        if (lane == 63) {
            g.wsum[0][wave] = i0;
            g.wsum[1][wave] = i1;
            g.wsum[2][wave] = i2;
        }
        lds_sync();
        int b0 = 0, b1 = 0, b2 = 0, t0 = 0, t1 = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            b0 += w < wave ? g.wsum[0][w] : 0;
            b1 += w < wave ? g.wsum[1][w] : 0;
            b2 += w < wave ? g.wsum[2][w] : 0;
            t0 += g.wsum[0][w];
            t1 += g.wsum[1][w];
        }
        if (sl) {
            g.seg_toff[tid] = b0 + i0 - n_s;
            g.seg_uoff[tid] = b1 + i1 - u_s;
        }
        if (tid == 0) {
            g.seg_toff[nseg] = t0;
            g.seg_uoff[nseg] = t1;
            g.nvalid = t0;
            g.nunits = t1;
        }
        lds_sync();
        if (tokt && tid < T) {
            const int q = key >= 0 ? g.seg_toff[my_seg] + rank_in : t0 + b2 + i2 - ungrouped;
            g.sorted[q] = tid;
            g.pos[tid] = q;
        }
        lds_sync();
    }
    const int nvalid = g.nvalid, nunits = g.nunits;

    f32x4_t acc[MBW][4];
#pragma unroll
    for (int m = 0; m < MBW; ++m)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[m][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // ---- passes over the split's K range: pass 0 carries W and the first NW n_tiles UPW units, further
    // passes (more units than that: not at H >= 4096) only units, with W's operand zeroed
    const int cap = NW * n_tiles * UPW;
    const int npass = max(1, (nunits + cap - 1) / cap);
    for (int pass = 0; pass < npass; ++pass) {
        if (pass > 0) {
#pragma unroll
            for (int c = 0; c < NWS; ++c) dma_w(c);
#pragma unroll
            for (int c = 0; c < NSTAGE; ++c) dma_x(c);
            __builtin_amdgcn_sched_barrier(0);
        }
        const bool with_w = pass == 0;
        // this wave's units: u = pass cap + tile + n_tiles (wave + NW e) (uniform per wave): dealt over the
        // tiles first, so every workgroup carries about the same share (3 us less per call on 2000
        // adapters than filling whole workgroups first)
        int32_t u_seg[UPW], u_pb[UPW], u_tc[UPW];
        bool u_live[UPW];
        const uint16_t *urp[UPW][2];   // rows 0..7 and 8..15 of the unit's pages (or stand-ins), this lane's piece
        int32_t u_pid[UPW];
        int u_row[UPW];
        float u_sc[UPW];
#pragma unroll
        for (int e = 0; e < UPW; ++e) {
            const int u = pass * cap + tile + n_tiles * (wave + NW * e);
            u_live[e] = u < nunits;
            const int s = u_live[e] ? last_leq(g.seg_uoff, nseg, u) : 0;
            const int32_t a = g.seg_a[s], rs = g.seg_r[s], ns = g.seg_n[s], to = g.seg_toff[s];
            const int ntc = (ns + 15) >> 4, local = u - g.seg_uoff[s];
            u_seg[e] = s;
            u_pb[e] = u_live[e] ? local / ntc : 0;
            u_tc[e] = u_live[e] ? local % ntc : 0;
            const int j = u_pb[e] * 16 + lrow, it = u_tc[e] * 16 + lrow;
            u_row[e] = g.sorted[u_live[e] ? to + min(it, ns - 1) : 0];
            const int32_t pid = pt[u_live[e] && j < rs ? (int64_t)a * stride + j : 0];
            u_pid[e] = pid;
            const bool pok = u_live[e] && j < rs && pid >= 0 && (int64_t)pid < num_pages;
            {   // lane l loads page row (l >> 3) + 8 h, 16-byte piece l & 7: the page id comes from lane (that row)
                const int rr = lane >> 3;
                const int32_t p0 = __shfl(pid, rr, 64), p1 = __shfl(pid, rr + 8, 64);
                const int ok0 = __shfl((int)pok, rr, 64), ok1 = __shfl((int)pok, rr + 8, 64);
                urp[e][0] = ok0 ? pages + (int64_t)p0 * H + kb + (lane & 7) * 8 : x + (lane & 7) * 8;
                urp[e][1] = ok1 ? pages + (int64_t)p1 * H + kb + (lane & 7) * 8 : x + (lane & 7) * 8;
            }
            u_sc[e] = scale[u_live[e] ? a : 0];
        }
        // the page load of K step sn, for ring slot i (sn = i mod DW): rows 8 (sn & 1) + [0, 8) of chunk sn >> 1;
        // past the range the last step of the same parity, so that the half, i & 1, is known at compile time
        auto page_load = [&](int e, int i, int sn) {
            return load16(urp[e][i & 1] + KC * (min(sn, nst - 2 + (i & 1)) >> 1));
        };
        // A wave whose units are all past the last (with one unit per wave, about half the waves at 256
        // tokens of 137 adapters and 4096 columns) runs the K loop without page loads, buffer work and
        // unit MFMAs: stand-in loads cost the CU's load path as much as real ones.
        const bool any_live = __builtin_amdgcn_readfirstlane((int)u_live[0]) != 0;   // units grow with e
        auto kloop = [&](auto live_c) {
            constexpr bool LIVE = decltype(live_c)::value;
            constexpr int NU = LIVE ? UPW : 0;   // units whose operands this wave loads and multiplies
            u32x4_t pv[UPW][DW];
            if constexpr (LIVE) {
    #pragma unroll
                for (int i = 0; i < DW; ++i)
    #pragma unroll
                    for (int e = 0; e < UPW; ++e) pv[e][i] = page_load(e, i, i);
            }
            f32x4_t uacc[UPW];
    #pragma unroll
            for (int e = 0; e < UPW; ++e) uacc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            // the first chunks have landed (the DW UPW page loads just issued are the only younger ones)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DW * NU) : "memory");
            lds_sync();

            // ---- K loop, in chunks of two steps of 32.  A chunk's one barrier sits between its steps: before
            // it each wave has read both halves of its operands from the chunk's stages and waited for its
            // loads of chunk c + 1; after it the stages of chunk c are free, so they refill with chunks
            // c + NSTAGE (x) and c + NWS (W) while the second step's MFMAs run and the next chunk's first
            // operands are read -- no MFMA waits for LDS at a chunk boundary.  DW steps per round (the
            // ring of page loads in flight is indexed statically).
            u32x4_t wf[2][4], xf[2][MBW], uf[2][UPW];
            auto frags = [&](int c, int half, u32x4_t *wfo, u32x4_t *xfo, u32x4_t *ufo) {
                const uint16_t *stg = xs + (c % NSTAGE) * XSTAGE, *wsg = wst + (c % NWS) * WSTAGE;
                const int pc = half * 4 + lq;           // 16-byte piece of the row for this lane
    #pragma unroll
                for (int nb = 0; nb < 4; ++nb) wfo[nb] = load16(wsg + wswz(16 * nb + lrow, pc));
    #pragma unroll
                for (int m = 0; m < MBW; ++m) xfo[m] = load16(stg + wswz((wave * MBW + m) * 16 + lrow, pc));
                if constexpr (LIVE) {
    #pragma unroll
                    for (int e = 0; e < UPW; ++e) ufo[e] = load16(stg + wswz(u_row[e], pc));
                }
            };
            frags(0, 0, wf[0], xf[0], uf[0]);
            for (int st0 = 0; st0 < nst; st0 += DW) {
    #pragma unroll
                for (int i = 0; i < DW; ++i) {
                    const int st = st0 + i, c = st >> 1, h = i & 1;
                    const bool sl = st < nst;
                    // at a chunk's first step both of its page loads are in (ring slots i and i + 1): the rows go
                    // into the wave's buffer (LDS accesses of one wave are done in order), and each step reads its
                    // operand, pieces 4 h + lq of row lrow, back out
                    u32x4_t pb[UPW];
    #pragma unroll
                    for (int e = 0; e < NU; ++e) {
                        uint16_t *ub = ubuf + (wave * UPW + e) * (16 * KC);
                        if (h == 0) {
                            const int rr = lane >> 3;
                            *reinterpret_cast<u32x4_t *>(ub + wswz(rr, lane & 7)) = pv[e][i];
                            *reinterpret_cast<u32x4_t *>(ub + wswz(rr + 8, lane & 7)) = pv[e][i + 1];
                        }
                        const u32x4_t op = load16(ub + wswz(lrow, h * 4 + lq));
                        pb[e] = sl && u_live[e] ? op : zero;
                    }
                    // the loads of step st + DW refill this slot of the ring (slot i + 1, whose rows went into the
                    // buffer at step st, refills at step st + 1)
    #pragma unroll
                    for (int e = 0; e < NU; ++e) pv[e][i] = page_load(e, i, st + DW);
                    if (h == 1) {   // chunk c's stages are free: refill them
                        dma_w(c + NWS);
                        dma_x(c + NSTAGE);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if (h == 0) frags(c, 1, wf[1], xf[1], uf[1]);
                    else frags(c + 1, 0, wf[0], xf[0], uf[0]);
                    const bool wl = sl && with_w;   // steps past the range and unit-only passes add nothing to x W
    #pragma unroll
                    for (int m = 0; m < MBW; ++m)
    #pragma unroll
                        for (int nb = 0; nb < 4; ++nb)
                            acc[m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, xf[h][m]), __builtin_bit_cast(bf16x8_t, wl ? wf[h][nb] : zero),
                                acc[m][nb], 0, 0, 0);
    #pragma unroll
                    for (int e = 0; e < NU; ++e)
                        uacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, uf[h][e]),
                                                                          __builtin_bit_cast(bf16x8_t, pb[e]), uacc[e], 0, 0, 0);
    #pragma unroll
                    for (int g2 = 0; g2 < MBW * 4 + NU; ++g2) {   // one operand read after each MFMA
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        if (g2 < 4 + MBW + NU) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                    if (h == 0) {
                        // mid-chunk: this wave's loads of x chunk c + 1 (and of the older W chunk c + 1) have
                        // landed.  x chunk c + 1 went out last in chunk c + 1 - NSTAGE; younger are, for
                        // each chunk between, its two steps of page loads and its W and x loads, and this
                        // chunk's first step of page loads
                        __builtin_amdgcn_sched_barrier(0);
                        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NSTAGE - 2) * (2 * NU + DWL + DX) + NU) : "memory");
                        lds_sync();
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the stand-in loads past the end have landed
            lds_sync();

            // ---- units: s v partials of this split (tokens and pages past the segment are dropped; a
            // segment whose page-table row is bad is dropped by the finishing kernel)
    #pragma unroll
            for (int e = 0; e < NU; ++e) {
                if (!u_live[e]) continue;
                const int s = u_seg[e];
                const int32_t rs = g.seg_r[s], ns = g.seg_n[s], to = g.seg_toff[s];
                const int j = u_pb[e] * 16 + lrow;
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int it = u_tc[e] * 16 + 4 * lq + i;
                    if (j < rs && it < ns) {
                        const int t = g.sorted[to + it];
                        vpart[((int64_t)(to + it) * RP + j) * S + split] = u_sc[e] * uacc[e][i];   // by sorted position
                        if constexpr (DBG) dbg_put(dbg_gather + (int64_t)t * stride + j, u_pid[e]);
                    }
                }
            }
        };
        if (any_live) kloop(std::true_type{});
        else kloop(std::false_type{});
    }

    // ---- x W partial of this split: lane holds column 16 nb + lrow, rows 16 (wave MBW + m) + 4 lq + i; each
    // token's row goes to its sorted position, so the finish needs no record to find it
#pragma unroll
    for (int m = 0; m < MBW; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = (wave * MBW + m) * 16 + 4 * lq + i;
            if (t < T) {
                const int q = g.pos[t];
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) store4_wt(ypart + ((int64_t)split * T + q) * H + n0 + 16 * nb + lrow, __float_as_uint(acc[m][nb][i]));
            }
        }

    // ---- publish: segments s = blockIdx.x + k gridDim.x -- check the page-table row (exactly 2r pages
    // in range, -1 after), then write the segment's sorted-token records and B page ids; workgroup 0
    // also writes the ungrouped tokens and reports the id / rank faults every workgroup saw
    for (int s = blockIdx.x; s < nseg; s += gridDim.x) {
        const int32_t a = g.seg_a[s], rs = g.seg_r[s], q0 = g.seg_toff[s], qn = g.seg_n[s];
        const int lim = min(2 * rs + 1, stride);
        if (tid < lim) {
            const int32_t ent = pt[(int64_t)a * stride + tid];
            int bad = 0;
            if (tid < 2 * rs) {
                if (ent == -1) bad = DEV_ERR_TABLE;
                else if (ent < 0 || (int64_t)ent >= num_pages) bad = DEV_ERR_PAGE;
            } else if (ent != -1) {
                bad = DEV_ERR_TABLE;
            }
            g.pub_ent[tid] = ent;
            if (bad) atomicOr(&g.pub_bad, bad);
        }
        lds_sync();
        const int bad = g.pub_bad;
        for (int idx = tid; idx < qn * rs; idx += NTH) {
            const int q = idx / rs, j = idx % rs;
            spages[(int64_t)(q0 + q) * RP + j] = g.pub_ent[rs + j];
        }
        for (int q = tid; q < qn; q += NTH)
            sorted_tok[q0 + q] = int4{g.sorted[q0 + q], bad ? -1 : a, bad ? 0 : rs, 0};
        if (tid == 0 && bad) atomicOr(err_word, bad);
        lds_sync();
        if (tid == 0) g.pub_bad = 0;
        lds_sync();
    }
    if (blockIdx.x == 0) {
        for (int q = nvalid + tid; q < T; q += NTH) sorted_tok[q] = int4{g.sorted[q], -1, 0, 0};
        const unsigned long long any = __ballot(err != 0);
        if (any) {
            for (int off = 32; off > 0; off >>= 1) err |= __shfl_xor(err, off, 64);
            if (lane == 0) atomicOr(err_word, err);
        }
    }
}

// One slot per launch, and the n slots of one call (blockIdx.z = the slot); the one-slot kernel
// keeps the short argument block.
template <int MB16>
__global__ __launch_bounds__(NTH, 1) void k_decode_wide(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, const uint16_t *__restrict__ pages,
    int64_t num_pages, const int32_t *__restrict__ pt, int32_t stride, const int32_t *__restrict__ ids,
    const int32_t *__restrict__ ranks, const float *__restrict__ scale, int32_t max_adapters, int32_t max_rank,
    int32_t T, int32_t H, int32_t S, int32_t n_tiles, int32_t RP, float *__restrict__ ypart,
    float *__restrict__ vpart, int4 *__restrict__ sorted_tok, int32_t *__restrict__ spages,
    int *__restrict__ err_word) {
    decode_wide_body<MB16, false>(x, W, pages, num_pages, pt, stride, ids, ranks, scale, max_adapters, max_rank, T, H,
                                  S, n_tiles, RP, ypart, vpart, sorted_tok, spages, err_word, nullptr);
}

// The debug instantiation (lora_debug_project): the same body, recording the A pages it reads per token.
template <int MB16>
__global__ __launch_bounds__(NTH, 1) void k_decode_wide_dbg(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, const uint16_t *__restrict__ pages,
    int64_t num_pages, const int32_t *__restrict__ pt, int32_t stride, const int32_t *__restrict__ ids,
    const int32_t *__restrict__ ranks, const float *__restrict__ scale, int32_t max_adapters, int32_t max_rank,
    int32_t T, int32_t H, int32_t S, int32_t n_tiles, int32_t RP, float *__restrict__ ypart,
    float *__restrict__ vpart, int4 *__restrict__ sorted_tok, int32_t *__restrict__ spages,
    int *__restrict__ err_word, int32_t *__restrict__ dbg_gather) {
    decode_wide_body<MB16, true>(x, W, pages, num_pages, pt, stride, ids, ranks, scale, max_adapters, max_rank, T, H,
                                 S, n_tiles, RP, ypart, vpart, sorted_tok, spages, err_word, dbg_gather);
}

template <int MB16>
__global__ __launch_bounds__(NTH, 1) void k_decode_wide_slots(
    const SlotPtrs sp, const uint16_t *__restrict__ pages, int64_t num_pages,
    int32_t stride, const int32_t *__restrict__ ids, const int32_t *__restrict__ ranks, const float *__restrict__ scale,
    int32_t max_adapters, int32_t max_rank, int32_t T, int32_t H, int32_t S, int32_t n_tiles, int32_t RP,
    int *__restrict__ err_word) {
    const int z = blockIdx.z;
    decode_wide_body<MB16, false>((const uint16_t *)sp.x[z], (const uint16_t *)sp.W[z], pages, num_pages, sp.pt[z], stride, ids, ranks, scale,
                                  max_adapters, max_rank, T, H, S, n_tiles, RP, sp.ypart[z], sp.v[z],
                                  (int4 *)sp.sorted_tok[z], sp.spages[z], err_word, nullptr);
}

size_t decode_wide_lds(int mb16) { return (size_t)(NSTAGE * mb16 * 16 + NWS * 64) * KC * 2 + GROUP_GAP + sizeof(WideGroup); }
static_assert((size_t)(NSTAGE * WT + NWS * 64) * KC * 2 + GROUP_GAP + sizeof(WideGroup) <= 160 * 1024, "LDS of the widest case");

template <int MB16>
static hipError_t launch_wide_t(const lora_pool *p, const Plan &plan, const void *x, const int32_t *ids,
                                const int32_t *ranks, const float *scale, const SlotPtrs &sp, int n, hipStream_t s,
                                const DebugOut *dbg) {
    static bool attr_set = false;
    const size_t lds = decode_wide_lds(MB16);
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)k_decode_wide<MB16>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void *)k_decode_wide_slots<MB16>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void *)k_decode_wide_dbg<MB16>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    dim3 grid((unsigned)(plan.n_tiles * plan.ysplit), 1, n);
    if (dbg)
        hipLaunchKernelGGL((k_decode_wide_dbg<MB16>), dim3(grid.x), dim3(NTH), lds, s, (const uint16_t *)x,
                           (const uint16_t *)sp.W[0], (const uint16_t *)p->pages, p->num_pages, sp.pt[0],
                           2 * p->max_rank, ids, ranks, scale, p->max_adapters, p->max_rank, (int32_t)plan.T,
                           p->hidden, plan.ysplit, plan.n_tiles, plan.rp, sp.ypart[0], sp.v[0],
                           (int4 *)sp.sorted_tok[0], sp.spages[0], p->dev_err, dbg->gather);
    else if (n == 1)
        hipLaunchKernelGGL((k_decode_wide<MB16>), grid, dim3(NTH), lds, s, (const uint16_t *)x,
                           (const uint16_t *)sp.W[0], (const uint16_t *)p->pages, p->num_pages, sp.pt[0],
                           2 * p->max_rank, ids, ranks, scale, p->max_adapters, p->max_rank, (int32_t)plan.T,
                           p->hidden, plan.ysplit, plan.n_tiles, plan.rp, sp.ypart[0], sp.v[0],
                           (int4 *)sp.sorted_tok[0], sp.spages[0], p->dev_err);
    else
        hipLaunchKernelGGL((k_decode_wide_slots<MB16>), grid, dim3(NTH), lds, s, sp,
                           (const uint16_t *)p->pages, p->num_pages, 2 * p->max_rank, ids, ranks, scale,
                           p->max_adapters, p->max_rank, (int32_t)plan.T, p->hidden, plan.ysplit, plan.n_tiles,
                           plan.rp, p->dev_err);
    return hipGetLastError();
}

hipError_t launch_decode_wide(const lora_pool *p, const Plan &plan, const void *x, const int32_t *ids,
                              const int32_t *ranks, const float *scale, const SlotPtrs &sp, int n, hipStream_t s,
                              const DebugOut *dbg) {
    switch (plan.mb) {
        case 8: return launch_wide_t<8>(p, plan, x, ids, ranks, scale, sp, n, s, dbg);
        case 16: return launch_wide_t<16>(p, plan, x, ids, ranks, scale, sp, n, s, dbg);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lorapool
