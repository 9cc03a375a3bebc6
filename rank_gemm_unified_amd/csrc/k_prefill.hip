// Prefill-shaped projection (many tokens per request, T > 256): MFMA-bound.
//
//   k_shrink_mfma    partials of X_seg A_a for every 64-row chunk of every adapter segment (tokens
//                    grouped by the grouping kernel), a small tiled bf16 MFMA GEMM against the r
//                    gathered A pages, split over K;
//   k_v_finalize     v = bf16(s_a * the split partials summed in split order);
//   k_prefill_main   y = x W for a 256x256 output tile (bf16 MFMA 32x32x16, LDS double buffer),
//                    then the low-rank term as extra K: for each adapter that owns rows of the
//                    tile, [x | v_a] [W ; B_a] with v_a zero outside its rows and B_a's rows
//                    gathered from their pages; one rounding to bfloat16 at the end.
// ("S-LoRA, in depth", sections "Merge or keep adapters separate" and "Kernels for a batch of
// mixed ranks": the base product is batched over all tokens; the low-rank work follows tokens and
// their ranks.)
#include "device_common.h"
#include "internal.h"

namespace lorapool {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---- shrink ------------------------------------------------------------------------------------
constexpr int SH_ROWS = 64;   // rows per work item
constexpr int VSPLIT = 4;     // K-splits of the shrink

// SNS LDS stages of 16 KiB form the K-tile ring (SNS - 1 tiles in flight).  Six stages (one
// workgroup per CU) when the work items fit one round of the chip (T <= 4096), else four (two per
// CU): measured best at 4096 and at 8448 rows.
//
// Work unit = (work item, split, slot): item = up to 64 tokens of one adapter segment, read as one
// record; split = a K range of H / VSPLIT; slot = a projection of the call.  A persistent grid (as
// many workgroups of 256 threads as the chip holds at once) walks the units in item order and stops
// at the first record past the last item (adapter -1): the item bound the host knows follows from the
// number of tokens, so a grid over it was mostly workgroups that read a record and left -- about
// 14,500 of 18,000 at the 13B stack's shapes, each holding an LDS slot for a round trip.  The slots of one
// (item, split) are consecutive units on one XCD, so the slots that share x (q, k and v) read its
// rows there at about the same time and share its L2.
//
// Per unit, a small tiled GEMM: per K tile of 64, the item's x rows (gathered through perm) and the
// adapter's A pages (<= 64, one per column of v) go from global memory straight into a ring of SNS
// LDS stages, SNS - 1 tiles ahead (the unit's chain is two round trips: the record, then perm and the
// page-table row); four waves compute 32x32 blocks (rows 32 wm.., pages 32 wn..) with 32x32x16 MFMAs.
// (Loading only the 8-row groups below the item's row count and rank -- one group of x rows for a
// decode-row item -- made the 4096-token shrink 1.8 us slower and the 13B stack's 1 us faster.)
// Writes float32 partials vpart[split][t][0..r); k_v_finalize adds
// them in split order.  (No in-kernel cross-workgroup reduction: on this chip a device-scope fence
// writes back and invalidates the whole L2.)
constexpr int SK = 64;                                  // K tile
constexpr int SH_STAGE = (SH_ROWS + 64) * SK;           // x rows + page rows, elements (16 KiB)
__device__ __forceinline__ int sswz(int r, int p) { return r * SK + ((p ^ ((r >> 1) & 7)) << 3); }   // as swz

// One work unit (item, split) of one slot.  Ends with every load landed and a barrier, so that the
// workgroup's next unit may reuse the stages and s_perm.
template <int SNS, bool DBG>
__device__ __forceinline__ void shrink_unit(const uint16_t *__restrict__ x, const uint16_t *__restrict__ pages, int32_t H,
                                            const int32_t *__restrict__ pt, int32_t stride,
                                            const int32_t *__restrict__ perm, const int4 rec, int split,
                                            float *__restrict__ vpart, int32_t T, int32_t R, uint16_t *st,
                                            int32_t *s_perm, int32_t *s_pid, const DebugOut dbg) {
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int32_t a = rec.x, r = rec.y, row0 = rec.z, n = rec.w;   // 1 <= r, 1 <= n <= 64
    const int ktiles = H / SK;
    const int kt0 = (int)((int64_t)ktiles * split / VSPLIT), kt1 = (int)((int64_t)ktiles * (split + 1) / VSPLIT);
    // Loads: one fills 1 KiB of a stage, rows 8d .. 8d + 7 (d < 8: x rows, d >= 8: page rows d - 8);
    // wave w issues d = w, w + 4 (x) and w + 8, w + 12 (pages).  Lane l lands in row 8d + l / 8, slot
    // l % 8, which holds piece (l % 8) ^ ((row >> 1) & 7): the piece the lane fetches.  x rows past the
    // item read its last row and pages past r read page r - 1: their products are never stored.
    const uint16_t *src[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 8 * (wave + 4 * i) + (lane >> 3), p = (lane & 7) ^ ((row >> 1) & 7);
        const int32_t tk = perm[row0 + min(row, n - 1)];
        if ((lane & 7) == 0) s_perm[row] = tk;
        src[i] = x + (int64_t)tk * H + p * 8;
        const int32_t pid = pt[(int64_t)a * stride + min(row, r - 1)];   // checked by the grouping kernel
        src[2 + i] = pages + (int64_t)pid * H + p * 8;
        if constexpr (DBG)
            if ((lane & 7) == 0) s_pid[row] = pid;
    }
    auto dma = [&](int kt, uint16_t *stg) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lds_gload16(src[i] + kt * SK, (lds_void *)(stg + (8 * (wave + 4 * i)) * SK));
    };
    const int nkt = kt1 - kt0;
    // SNS - 1 tiles in flight; tiles past the range reload the first (never read)
#pragma unroll
    for (int u = 0; u < SNS - 1; ++u) dma(kt0 + (u < nkt ? u : 0), st + u * SH_STAGE);
    const int wm = wave >> 1, wn = wave & 1;
    const int frow = lane & 31, fk = lane >> 5;
    f32x16_t acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    for (int u = 0; u < nkt; ++u) {
        // tile u has landed once the SNS - 2 younger tiles (4 loads each per wave) may still be in flight
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(4 * (SNS - 2)) : "memory");
        __builtin_amdgcn_s_barrier();   // every wave's share of tile u is in; tile u - 1 is no longer read
        asm volatile("" ::: "memory");
        const int un = u + SNS - 1;
        dma(kt0 + (un < nkt ? un : 0), st + (un % SNS) * SH_STAGE);
        const uint16_t *S = st + (u % SNS) * SH_STAGE;
#pragma unroll
        for (int ks = 0; ks < SK / 16; ++ks) {
            const u32x4_t fa = load16(S + sswz(wm * 32 + frow, ks * 2 + fk));
            const u32x4_t fb = load16(S + sswz(SH_ROWS + wn * 32 + frow, ks * 2 + fk));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa),
                                                          __builtin_bit_cast(bf16x8_t, fb), acc, 0, 0, 0);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the stand-in loads have landed
    __syncthreads();   // s_perm; every wave is past its last fragment read
    // 32x32 block layout: lane holds column (page) lane%32 and, in register e, row 8 (e/4) + 4 (lane/32) + e%4
    float *vout = vpart + (int64_t)split * T * R;
    const int j = wn * 32 + (lane & 31);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int rr = wm * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e & 3);
        if (rr < n && j < r) {
            vout[(int64_t)s_perm[rr] * R + j] = acc[e];
            if constexpr (DBG) dbg_put(dbg.gather + (int64_t)s_perm[rr] * stride + j, s_pid[j]);
        }
    }
    if constexpr (DBG) {   // the item's sorted rows: token and adapter
        if (tid < n) {
            dbg_put(dbg.order + 2 * (row0 + tid), s_perm[tid]);
            dbg_put(dbg.order + 2 * (row0 + tid) + 1, a);
        }
    }
    __syncthreads();   // s_perm and s_pid are read above; the next unit rewrites them
}

// The units of n slots, walked by a persistent grid (gridDim.x a multiple of 8).  Unit u: XCD lane u % 8
// (the XCD of every workgroup that takes it), slot (u / 8) % n, and (item, split) q = (u / 8n) 8 + u % 8
// as item q / VSPLIT, split q % VSPLIT.  A workgroup's units have non-decreasing items, so the first
// one past the last item ends its walk.
template <int SNS, bool DBG>
__device__ __forceinline__ void shrink_walk(const SlotPtrs &sp, int n, const uint16_t *__restrict__ pages, int32_t H,
                                            int32_t stride, const int32_t *__restrict__ perm,
                                            const int4 *__restrict__ item_rec, int32_t n_items_max,
                                            int32_t T, int32_t R, const DebugOut dbg = DebugOut{}) {
    extern __shared__ __align__(16) uint16_t st[];   // SNS stages
    __shared__ int32_t s_perm[SH_ROWS];
    __shared__ int32_t s_pid[DBG ? SH_ROWS : 1];     // debug: the page of each column of v
    for (int64_t u = blockIdx.x;; u += gridDim.x) {
        const int xl = (int)(u & 7), z = (int)((u >> 3) % n);
        const int64_t q = (u >> 3) / n * 8 + xl;
        const int64_t item = q / VSPLIT;
        const int split = (int)(q % VSPLIT);
        if (item >= n_items_max) break;
        const int4 rec = item_rec[item];
        if (rec.x < 0) break;   // past the last item
        shrink_unit<SNS, DBG>((const uint16_t *)sp.x[z], pages, H, sp.pt[z], stride, perm, rec, split, sp.v[z], T, R,
                              st, s_perm, s_pid, dbg);
    }
}

// One slot (the short argument block), its debug instantiation, and the n slots of one call (the
// slots share the token grouping).
template <int SNS>
__global__ __launch_bounds__(256) void k_shrink_mfma(const uint16_t *__restrict__ x, const uint16_t *__restrict__ pages, int32_t H,
                                                     const int32_t *__restrict__ pt, int32_t stride,
                                                     const int32_t *__restrict__ perm, const int4 *__restrict__ item_rec,
                                                     int32_t n_items_max, float *__restrict__ vpart,
                                                     int32_t T, int32_t R) {
    SlotPtrs sp{};
    sp.x[0] = x;
    sp.pt[0] = pt;
    sp.v[0] = vpart;
    shrink_walk<SNS, false>(sp, 1, pages, H, stride, perm, item_rec, n_items_max, T, R);
}

template <int SNS>
__global__ __launch_bounds__(256) void k_shrink_mfma_dbg(const uint16_t *__restrict__ x,
                                                         const uint16_t *__restrict__ pages, int32_t H,
                                                         const int32_t *__restrict__ pt, int32_t stride,
                                                         const int32_t *__restrict__ perm,
                                                         const int4 *__restrict__ item_rec,
                                                         int32_t n_items_max, float *__restrict__ vpart,
                                                         int32_t T, int32_t R, const DebugOut dbg) {
    SlotPtrs sp{};
    sp.x[0] = x;
    sp.pt[0] = pt;
    sp.v[0] = vpart;
    shrink_walk<SNS, true>(sp, 1, pages, H, stride, perm, item_rec, n_items_max, T, R, dbg);
}

template <int SNS>
__global__ __launch_bounds__(256) void k_shrink_mfma_slots(const uint16_t *__restrict__ pages, int32_t H,
                                                           const SlotPtrs sp, int32_t n, int32_t stride,
                                                           const int32_t *__restrict__ perm,
                                                           const int4 *__restrict__ item_rec,
                                                           int32_t n_items_max, int32_t T, int32_t R) {
    shrink_walk<SNS, false>(sp, n, pages, H, stride, perm, item_rec, n_items_max, T, R);
}

// v16[t][j] = bf16(s_a * sum_split vpart[split][t][j]) for tokens with an adapter; zero for
// j in [r, roundup(r, 4)).  One thread per (token, 4 consecutive j).
__device__ __forceinline__ void v_finalize_body(const float *__restrict__ vpart, const int32_t *__restrict__ tok_a,
                                              const int32_t *__restrict__ tok_r, const float *__restrict__ scale,
                                              int32_t T, int32_t R, uint16_t *__restrict__ v16) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t t = idx / (R / 4);
    const int j0 = (int)(idx % (R / 4)) * 4;
    if (t >= T) return;
    const int32_t a = tok_a[t], r = tok_r[t];
    if (a < 0 || j0 >= r) return;
    f32x4_t pv[VSPLIT];
#pragma unroll
    for (int q = 0; q < VSPLIT; ++q) pv[q] = *reinterpret_cast<const f32x4_t *>(vpart + ((int64_t)q * T + t) * R + j0);
    f32x4_t sum = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < VSPLIT; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) sum[e] += pv[q][e];
    const float sc = scale[a];
    uint32_t w0 = (j0 < r ? f32_to_bf16_bits(sc * sum[0]) : 0u) | ((j0 + 1 < r ? f32_to_bf16_bits(sc * sum[1]) : 0u) << 16);
    uint32_t w1 = (j0 + 2 < r ? f32_to_bf16_bits(sc * sum[2]) : 0u) | ((j0 + 3 < r ? f32_to_bf16_bits(sc * sum[3]) : 0u) << 16);
    *reinterpret_cast<uint2 *>(v16 + t * R + j0) = make_uint2(w0, w1);
}

__global__ __launch_bounds__(256) void k_v_finalize(const float *__restrict__ vpart, const int32_t *__restrict__ tok_a,
                                                    const int32_t *__restrict__ tok_r, const float *__restrict__ scale,
                                                    int32_t T, int32_t R, uint16_t *__restrict__ v16) {
    v_finalize_body(vpart, tok_a, tok_r, scale, T, R, v16);
}

__global__ __launch_bounds__(256) void k_v_finalize_slots(const SlotPtrs sp, const int32_t *__restrict__ tok_a,
                                                          const int32_t *__restrict__ tok_r,
                                                          const float *__restrict__ scale, int32_t T, int32_t R) {
    v_finalize_body(sp.v[blockIdx.z], tok_a, tok_r, scale, T, R, sp.v16[blockIdx.z]);
}

// ---- base GEMM + fused expand --------------------------------------------------------------------
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int STAGE = (BM + BN) * BK;               // elements per pipeline stage (unpadded, swizzled)
// 16-byte piece p of row r of a stage sits in slot p ^ ((r >> 1) & 7).  The LDS serves a 16-byte read
// 16 lanes at a time over 64 banks (256 bytes): two 128-byte rows fill the banks once, so the 16 rows
// of one piece that a fragment read touches must use 8 different slots in each of the two halves --
// rows 2i and 2i + 1 share slot p ^ i.  Tile writes (8 lanes per row) are conflict-free either way.
__device__ __forceinline__ int swz(int r, int p) { return r * BK + ((p ^ ((r >> 1) & 7)) << 3); }
constexpr size_t MAIN_LDS = 2 * STAGE * sizeof(uint16_t);

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 12] (the count is an immediate); larger n waits for all
__device__ __forceinline__ void wait_vmem_le(int n) {
    switch (n) {
#define WV(k) case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
        WV(1) WV(2) WV(3) WV(4) WV(5) WV(6) WV(7) WV(8) WV(9) WV(10) WV(11) WV(12)
#undef WV
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}

// PF_WAVES waves in a 2 x (PF_WAVES / 2) grid over the 256 x 256 tile; wave (wm, wn) computes rows
// WTM wm + [0, WTM) x columns WTN wn + [0, WTN) as WMI x WNI blocks of 32 x 32.
#ifndef PF_WAVES
#define PF_WAVES 8
#endif
constexpr int PF_THREADS = PF_WAVES * 64;
constexpr int WGN = PF_WAVES / 2;
constexpr int WTM = BM / 2, WTN = BN / WGN;
constexpr int WMI = WTM / 32, WNI = WTN / 32;
constexpr int DPW = (BM * BK * 2 / 1024) / PF_WAVES;   // 1 KiB tile chunks per wave per operand per K step
constexpr int LR_K = 64 * (BN / 8) / PF_THREADS;         // B-row pieces per thread of the low-rank term
constexpr int LR_V = BM * (64 / 8) / PF_THREADS;         // v-row pieces per thread of the low-rank term

template <bool DBG>
__device__ __forceinline__ void prefill_main_body(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, const uint16_t *__restrict__ pages,
    const int32_t *__restrict__ pt, int32_t stride, const int32_t *__restrict__ tok_a,
    const int32_t *__restrict__ tok_r, const uint16_t *__restrict__ v16, int32_t R, int32_t T, int32_t H,
    int32_t n_tiles_n, uint16_t *__restrict__ y, int blk, int nblk, const DebugOut dbg = DebugOut{}) {
    extern __shared__ __align__(16) uint16_t sm[];
    __shared__ int32_t s_key[BM], s_list[BM], s_lr[BM], s_wsum[PF_THREADS / 64], s_nlist;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: tile chunk addresses stay scalar
    const int wm = wave / WGN, wn = wave % WGN;
    // Tile order (workgroup blk of the nblk of this output).  The first P0 = roundup(n_tiles_n, 8)
    // workgroups take the last row of tiles, one
    // tile each, spread over the XCDs: when decode rows (one adapter each) follow the prefill rows,
    // that row holds most of the batch's distinct adapters and the longest low-rank term, so it
    // starts first (the rest of the grid then runs beside it).  The others go to the 8 XCDs in turn
    // (consecutive workgroups), each XCD taking a contiguous run of an order that walks groups of 4
    // row tiles across all column tiles, so an XCD's tiles share x rows and W columns in its L2.
    // Workgroups past the last tile of either part leave at once.
    int mt, nt;
    {
        const int tm = (T + BM - 1) / BM, P0 = (n_tiles_n + 7) / 8 * 8;
        const int b = blk;
        if (b < P0) {
            if (b >= n_tiles_n) return;
            mt = tm - 1;
            nt = b;
        } else {
            const int rest = (tm - 1) * n_tiles_n, G = nblk - P0, b2 = b - P0;   // G: multiple of 8
            const int t = (b2 & 7) * (G >> 3) + (b2 >> 3);
            if (t >= rest) return;
            constexpr int GM = 4;
            const int grp = GM * n_tiles_n, g = t / grp, fm = g * GM, gsz = min(tm - 1 - fm, GM);
            mt = fm + (t % grp) % gsz;
            nt = (t % grp) / gsz;
        }
    }
    const int m0 = mt * BM, n0 = nt * BN;

    // ---- the adapters owning rows of this tile, in order of their first row (s_list, ranks s_lr), and
    // the B page ids of the first one (pg0): worked out here, before the first tile load is waited
    // for, so that after the K loop the low-rank term needs one round trip.  Thread t < BM owns row t.
    // The two token loads go out before the tile loads, so waiting for them does not wait for those.
    const bool rowt = tid < BM;
    const int32_t key = rowt && m0 + tid < T ? tok_a[m0 + tid] : -1;
    const int32_t key_r = rowt && m0 + tid < T ? tok_r[m0 + tid] : 0;
    __builtin_amdgcn_sched_barrier(0);

    // Tiles go from global memory straight into LDS (16 bytes per lane, no register staging, no LDS
    // write instructions).  One such load fills 1 KiB of a stage, rows 8c .. 8c + 7: lane l lands in
    // row 8c + l / 8, slot l % 8, the slot of piece (l % 8) ^ ((row >> 1) & 7) -- so that is the piece
    // the lane fetches.  Wave w issues chunks c = PF_WAVES i + w (i < DPW) of the x tile and of the W
    // tile.
    // Loads go through buffer resources based at the tile's first row, with 32-bit row offsets.  Rows
    // past T (x) or H (W) read the last valid row: they only feed output rows or columns that are never
    // stored.
    const int rvx = min(T - m0, BM), rvw = min(H - n0, BN);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc((void *)(x + (int64_t)m0 * H), (short)0, rvx * H * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void *)(W + (int64_t)n0 * H), (short)0, rvw * H * 2, 0x00020000);
    uint32_t offa[DPW], offb[DPW];
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
        const int r = 8 * (PF_WAVES * i + wave) + (lane >> 3), p = (lane & 7) ^ ((r >> 1) & 7);
        offa[i] = (uint32_t)(min(r, rvx - 1) * H + p * 8) * 2u;
        offb[i] = (uint32_t)(min(r, rvw - 1) * H + p * 8) * 2u;
    }
    // half h of tile kt's loads (DPW each): h = 0 the x chunks, h = 1 the W chunks
    auto dma_half = [&](int kt, uint16_t *stage, int h) {
        const int soff = kt * BK * 2;
#pragma unroll
        for (int i = 0; i < DPW; ++i) {
            uint16_t *dst = stage + 8 * (PF_WAVES * i + wave) * BK;
            if (h == 0) lds_load16(rx, (lds_void *)dst, offa[i], soff);
            else lds_load16(rw, (lds_void *)(dst + BM * BK), offb[i], soff);
        }
    };
    auto dma = [&](int kt, uint16_t *stage) {
        dma_half(kt, stage, 0);
        dma_half(kt, stage, 1);
    };
    const int frow = lane & 31, fk = (lane >> 5) * 8;   // 32x32x16 operand: row lane%32, k 8*(lane/32)
    // the fragments of k-substep ks of a stage, in the order the MFMAs consume them
    auto frag = [&](const uint16_t *stage, int ks, u32x4_t *fa, u32x4_t *fb) {
        const uint16_t *As = stage, *Bs = stage + BM * BK;
        const int pc = ks * 2 + (fk >> 3);   // 16-byte piece of the row
        fa[0] = load16(As + swz(wm * WTM + frow, pc));
#pragma unroll
        for (int ni = 0; ni < WNI; ++ni) fb[ni] = load16(Bs + swz(wn * WTN + ni * 32 + frow, pc));
#pragma unroll
        for (int mi = 1; mi < WMI; ++mi) fa[mi] = load16(As + swz(wm * WTM + mi * 32 + frow, pc));
    };

    // one of those reads: u = 0 is fa[0], u = 1 .. WNI fb[u - 1], then fa[1 ..]
    auto frag_one = [&](const uint16_t *stage, int ks, int u, u32x4_t *fa, u32x4_t *fb) {
        const uint16_t *As = stage, *Bs = stage + BM * BK;
        const int pc = ks * 2 + (fk >> 3);
        if (u == 0) fa[0] = load16(As + swz(wm * WTM + frow, pc));
        else if (u <= WNI) fb[u - 1] = load16(Bs + swz(wn * WTN + (u - 1) * 32 + frow, pc));
        else fa[u - WNI] = load16(As + swz(wm * WTM + (u - WNI) * 32 + frow, pc));
    };
    // load i (< DPW) of half h of tile kt
    auto dma_one = [&](int kt, uint16_t *stage, int h, int i) {
        uint16_t *dst = stage + 8 * (PF_WAVES * i + wave) * BK;
        if (h == 0) lds_load16(rx, (lds_void *)dst, offa[i], kt * BK * 2);
        else lds_load16(rw, (lds_void *)(dst + BM * BK), offb[i], kt * BK * 2);
    };

    f32x16_t acc[WMI][WNI];
#pragma unroll
    for (int mi = 0; mi < WMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < WNI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;

    // Pipeline over K steps of BK (two LDS stages; step kt computes from stage kt & 1 in four
    // k-substeps).  The one barrier of a step sits between substeps 2 and 3: each wave first waits for
    // its own loads of tile kt + 1 and for its last reads of stage kt & 1.  After it, substep 3 reads
    // the fragments of step kt + 1's first substep (so no MFMA waits for LDS at a step boundary) and
    // starts the loads of tile kt + 2 into stage kt & 1, which no wave reads any more; the second half
    // of those loads goes out in substep 0 of step kt + 1.
    const int nk = H / BK;
    u32x4_t af[2][WMI], bf[2][WNI];
    dma(0, sm);
    {
        // LDS-only barriers here: a full __syncthreads would also wait for the tile loads
        auto lds_sync = [] {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        if (rowt) s_key[tid] = key;
        lds_sync();
        int first = key >= 0;
        for (int u = 0; u < tid && first; ++u) first = s_key[u] != key;
        const int incl = wave_incl_scan(first, lane);   // exclusive scan of `first` over the row threads
        if (lane == 63) s_wsum[wave] = incl;
        lds_sync();
        int before = 0;
        for (int w = 0; w < wave; ++w) before += s_wsum[w];
        if (first) {
            s_list[before + incl - 1] = key;
            s_lr[before + incl - 1] = key_r;
        }
        if (tid == BM - 1) s_nlist = before + incl;
        lds_sync();
    }
    const int nlist = s_nlist;
    // page ids of B rows j = (tid + PF_THREADS k) / 32 of adapter li (row r - 1 stands in past r)
    auto lr_pages = [&](int li, int32_t *pg) {
        const int32_t a = s_list[li], r = max(s_lr[li], 1);
        const int32_t *prow = pt + (int64_t)a * stride + r;
#pragma unroll
        for (int k = 0; k < LR_K; ++k) pg[k] = prow[min((tid + PF_THREADS * k) >> 5, r - 1)];
    };
    int32_t pg0[LR_K] = {};
    // tile 0 has landed once at most the page-id loads (younger) are in flight; they are first needed
    // near the end of the K loop
    if (nlist > 0) {
        lr_pages(0, pg0);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LR_K) : "memory");
    } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // The low-rank operands, [x | v_a] [W ; B_a] as extra K for adapter s_list[li], fill one pipeline
    // stage (64 KiB):
    //   Bn [64][BN]  B_a's rows j < 64 over the tile's columns; 16-byte piece p of row j sits in slot
    //                p ^ 4 ((j >> 3) & 1), since one MFMA operand read takes rows j and j + 8;
    //   Vs [BM][64]  the tile's v rows (the adapter's tokens; zero elsewhere and past the rank), with
    //                the tile swizzle.
    // Thread -> piece idx = tid + PF_THREADS k (k < LR_K = LR_V) of each: B row idx / 32, slot idx % 32;
    // v row idx / 8, slot idx % 8.  The operands of the first adapter are loaded straight into LDS
    // during the K loop's second-to-last step (into the stage tile nk would have used), so the low-rank
    // term waits for no round trip (with a single K step they go out with tile 0); further adapters of
    // the tile load them through registers after it.
    static_assert(LR_K == LR_V && (size_t)64 * BN + (size_t)BM * 64 <= (size_t)STAGE, "low-rank operands fill one stage");
    auto bslot = [](int j, int p) { return j * BN + ((p ^ (((j >> 3) & 1) << 2)) << 3); };
    auto bsrc = [&](const int32_t *pg, int k) {
        const int idx = tid + PF_THREADS * k, j = idx >> 5, p = (idx & 31) ^ (((j >> 3) & 1) << 2);
        return pages + (int64_t)pg[k] * H + min(n0 + 8 * p, H - 8);
    };
    auto vsrc = [&](int k) {
        const int idx = tid + PF_THREADS * k, row = idx >> 3, p = (idx & 7) ^ ((row >> 1) & 7);
        return v16 + (int64_t)min(m0 + row, T - 1) * R + min(8 * p, R - 8);
    };
    // the first adapter's B rows (h = 0) or the tile's v rows (h = 1), LR_K = LR_V loads a thread
    auto lr_half = [&](uint16_t *stg, int h) {
#pragma unroll
        for (int k = 0; k < LR_K; ++k) {
            if (h == 0) lds_gload16(bsrc(pg0, k), (lds_void *)(stg + (PF_THREADS * k + 64 * wave) * 8));
            else lds_gload16(vsrc(k), (lds_void *)(stg + 64 * BN + (PF_THREADS * k + 64 * wave) * 8));
        }
    };
    auto lr_one = [&](uint16_t *stg, int h, int k) {
        if (h == 0) lds_gload16(bsrc(pg0, k), (lds_void *)(stg + (PF_THREADS * k + 64 * wave) * 8));
        else lds_gload16(vsrc(k), (lds_void *)(stg + 64 * BN + (PF_THREADS * k + 64 * wave) * 8));
    };
    auto lr_dma = [&](uint16_t *stg) {
        lr_half(stg, 0);
        lr_half(stg, 1);
    };
    // The K-extension of adapter li: rp / 16 substeps of 32x32x16 MFMAs on the accumulators.  The v
    // operand (the tile's v rows, all adapters, in Vs) is masked in registers: rows of other adapters and
    // entries past the rank are zero (v16 entries past the rank may hold any bits, NaN included, and
    // 0 * NaN is NaN).  B rows past the rank are stand-ins (row r - 1: finite adapter values) and meet
    // those zeros.  The B operand (8 consecutive j of one column) is gathered with 2-byte reads, lane ->
    // column.
    int32_t rkey[WMI];   // the adapter of each row this lane's v fragments cover
#pragma unroll
    for (int mi = 0; mi < WMI; ++mi) rkey[mi] = s_key[wm * WTM + mi * 32 + frow];
    auto lr_mfma = [&](const uint16_t *Bn, const uint16_t *Vs, int li) {
        const int32_t a = s_list[li], r = s_lr[li], rp = (r + 15) & ~15;
        // a 32-row block of this wave with none of the adapter's rows would add only zeros: its v reads
        // and MFMAs are skipped, and the whole term when no block has one (decode rows: one adapter
        // for every few rows)
        bool blk_live[WMI];
        bool any = false;
#pragma unroll
        for (int mi = 0; mi < WMI; ++mi) {
            blk_live[mi] = __builtin_amdgcn_readfirstlane((int)(__ballot(rkey[mi] == a) != 0ull)) != 0;
            any = any || blk_live[mi];
        }
        if (!any) return;
        for (int ks = 0; ks < rp / 16; ++ks) {
            u32x4_t la[WMI], lb[WNI];
            const int jb = ks * 16 + fk;   // this lane's first j
#pragma unroll
            for (int mi = 0; mi < WMI; ++mi) {
                if (!blk_live[mi]) continue;
                u32x4_t v = load16(Vs + swz(wm * WTM + mi * 32 + frow, ks * 2 + (fk >> 3)));
                const int nv = rkey[mi] == a ? min(max(r - jb, 0), 8) : 0;   // entries kept
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] &= (2 * e < nv ? 0xffffu : 0u) | (2 * e + 1 < nv ? 0xffff0000u : 0u);
                la[mi] = v;
            }
#pragma unroll
            for (int ni = 0; ni < WNI; ++ni) {
                const int col = wn * WTN + ni * 32 + frow, cp = col >> 3, ce = col & 7;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int j = ks * 16 + fk + 2 * w;
                    lb[ni][w] = (uint32_t)Bn[bslot(j, cp) + ce] | ((uint32_t)Bn[bslot(j + 1, cp) + ce] << 16);
                }
            }
#pragma unroll
            for (int mi = 0; mi < WMI; ++mi) {
                if (!blk_live[mi]) continue;
#pragma unroll
                for (int ni = 0; ni < WNI; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, la[mi]),
                                                                          __builtin_bit_cast(bf16x8_t, lb[ni]),
                                                                          acc[mi][ni], 0, 0, 0);
            }
        }
    };
    // B rows of adapter li straight into a buffer of [64][BN]: the rows below its rank rounded up to 16,
    // the rows its MFMAs read (load k of a thread covers rows RPL k .. RPL k + RPL - 1, RPL = PF_THREADS
    // / 32, so nb_of(li) loads per thread; rows from r to that bound are stand-ins, rows past it are left
    // as they are and never read)
    constexpr int RPL = PF_THREADS / 32;
    auto nb_of = [&](int li) {
        return min(max(__builtin_amdgcn_readfirstlane((((s_lr[li] + 15) & ~15) + RPL - 1) / RPL), 1), LR_K);
    };
    auto lr_issue_b = [&](uint16_t *buf, const int32_t *pg, int nb) {
#pragma unroll
        for (int k = 0; k < LR_K; ++k)
            if (k < nb) lds_gload16(bsrc(pg, k), (lds_void *)(buf + (PF_THREADS * k + 64 * wave) * 8));
    };
    // debug: the B page each B row of adapter li was loaded from (as the loads above used it), recorded
    // for every row of the tile that belongs to the adapter (one thread per B row)
    auto dbg_b = [&](int li, const int32_t *pg) {
        if constexpr (DBG) {
            const int32_t a = s_list[li], r = s_lr[li];
#pragma unroll
            for (int k = 0; k < LR_K; ++k) {
                const int idx = tid + PF_THREADS * k, j = idx >> 5;
                if ((idx & 31) == 0 && j < r)
                    for (int row = 0; row < BM; ++row)
                        if (m0 + row < T && s_key[row] == a)
                            dbg_put(dbg.gather + (int64_t)(m0 + row) * stride + r + j, pg[k]);
            }
        }
    };

    if (nk > 1) dma(1, sm + STAGE);
    else lr_dma(sm + STAGE);   // a single K step: stage 1 is the low-rank stage from the start
    frag(sm, 0, af[0], bf[0]);
    // One K step.  A tile's loads go out in two halves, so that the load path takes them over 16
    // MFMAs instead of 8: the x half of tile kt + 2 in substep 3 of step kt (the stage of tile kt is
    // free once the step's barrier is passed), its W half in substep 0 of step kt + 1.  Both have
    // landed at the barrier of step kt + 1.  The low-rank operands take the place of tile nk: the B
    // rows in substep 3 of step nk - 2, the v rows in substep 0 of step nk - 1.
    //   D0: the loads of substep 0 -- 0 none, 1 the W half of tile kt + 1, 2 the v rows;
    //   D3: the loads of substep 3 -- 0 none, 1 the x half of tile kt + 2, 2 the B rows;
    //   LAST: the last step (no fragments of a next step; its barrier waits for no load).
    auto step = [&](int kt, auto d0, auto d3, auto last) {
        constexpr int D0 = decltype(d0)::value, D3 = decltype(d3)::value;
        constexpr bool LAST = decltype(last)::value;
        uint16_t *cur = sm + (kt & 1) * STAGE, *oth = sm + ((kt + 1) & 1) * STAGE;
        __builtin_amdgcn_sched_barrier(0);
        // per k-substep (WMI x WNI MFMAs, operands in buffer ks & 1), in this issue order: MFMA g, the
        // next substep's fragment reads 2g and 2g + 1 (into the other buffer), and in substeps 0 and 3
        // load g of a half (g < DPW).  The order is fixed by scheduling fences: left to the scheduler,
        // the loads and reads of a substep went out together after its first MFMA.
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int g = 0; g < WMI * WNI; ++g) {
                const int mi = g / WNI, ni = g % WNI;
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, af[ks & 1][mi]),
                                                                      __builtin_bit_cast(bf16x8_t, bf[ks & 1][ni]),
                                                                      acc[mi][ni], 0, 0, 0);
#pragma unroll
                for (int u = 2 * g; u < 2 * g + 2; ++u)
                    if (u < WMI + WNI) {
                        if (ks < 3) frag_one(cur, ks + 1, u, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
                        else if (!LAST) frag_one(oth, 0, u, af[0], bf[0]);
                    }
                if (g < DPW) {
                    if (ks == 0) {
                        if constexpr (D0 == 1) dma_one(kt + 1, oth, 1, g);
                        if constexpr (D0 == 2) lr_one(oth, 1, g);
                    }
                    if (ks == 3) {
                        if constexpr (D3 == 1) dma_one(kt + 2, cur, 0, g);
                        if constexpr (D3 == 2) lr_one(cur, 0, g);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (ks == 2) {
                if constexpr (LAST)
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // only the low-rank loads are in flight
                else
                    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using NL = std::false_type;
    using LS = std::true_type;
    if (nk >= 3) {
        step(0, I0(), I1(), NL());   // tile 1 went out whole before the loop
        for (int kt = 1; kt + 2 < nk; ++kt) step(kt, I1(), I1(), NL());
        step(nk - 2, I1(), I2(), NL());
        step(nk - 1, I2(), I0(), LS());
    } else if (nk == 2) {
        step(0, I0(), I2(), NL());
        step(1, I2(), I0(), LS());
    } else {
        step(0, I0(), I0(), LS());   // every low-rank load went out before the loop
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // every load, the low-rank operands' included, has landed

    // ---- low-rank term: one K-extension per adapter owning rows of this tile.  Adapter 0's B rows and
    // the tile's v rows came into stage X during the K loop's second-to-last step.  The B rows of
    // adapter li rotate through three buffers -- X's B part and the two halves of stage Y, free since
    // the last K step -- and go out two adapters ahead of their MFMAs; their page ids two further ahead,
    // in two register sets taken in turn.  Each adapter waits for its own loads only (the count of
    // younger loads is exact: page ids are LR_K loads a thread, an adapter's B rows nb_of loads, both
    // known to every wave), then for one barrier, after which the buffer of adapter li - 1 is free for
    // adapter li + 2.
    if (nlist > 0) {
        uint16_t *const X = sm + (nk & 1) * STAGE, *const Y = sm + ((nk + 1) & 1) * STAGE;
        const uint16_t *const Vs = X + 64 * BN;
        auto buf = [&](int li) { const int m = li % 3; return m == 0 ? X : m == 1 ? Y : Y + 64 * BN; };
        auto lds_barrier = [] {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        int32_t pg1[LR_K] = {}, pgA[LR_K] = {}, pgB[LR_K] = {};
        if (nlist > 1) lr_pages(1, pg1);
        if (nlist > 2) lr_pages(2, pgA);
        if (nlist > 3) lr_pages(3, pgB);
        __builtin_amdgcn_sched_barrier(0);
        if (nlist > 1) {
            lr_issue_b(buf(1), pg1, nb_of(1));
            dbg_b(1, pg1);
        }
        dbg_b(0, pg0);
        __builtin_amdgcn_sched_barrier(0);
        // iteration li: wait for adapter li's B rows (v and adapter 0's rows were waited for after the K
        // loop), barrier, issue adapter li + 2's rows (ids in `use`) and adapter li + 4's ids (into `use`),
        // then adapter li's MFMAs
        auto iter = [&](int li, int32_t *use) {
            if (li >= 1) {
                // loads younger than adapter li's B rows: li = 1: [B(2), ids(4)]; li >= 2: [ids(li + 2),
                // B(li + 1), ids(li + 3)] -- those that were issued (ids: LR_K a thread, B(x): nb_of(x))
                const int n = li == 1 ? (nlist > 2 ? nb_of(2) : 0) + (nlist > 4 ? LR_K : 0)
                                      : (li + 2 < nlist ? LR_K : 0) + (li + 1 < nlist ? nb_of(li + 1) : 0) +
                                            (li + 3 < nlist ? LR_K : 0);
                // (the debug instantiation's atomics count as memory operations too: it waits for all)
                wait_vmem_le(DBG ? 0 : n);
            }
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if (li + 2 < nlist) {
                lr_issue_b(buf(li + 2), use, nb_of(li + 2));
                dbg_b(li + 2, use);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (li + 4 < nlist) lr_pages(li + 4, use);
            __builtin_amdgcn_sched_barrier(0);
            lr_mfma(buf(li), Vs, li);
        };
        for (int li = 0; li < nlist; li += 2) {
            iter(li, pgA);
            if (li + 1 < nlist) iter(li + 1, pgB);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // stand-in loads past the end have landed
    }

    // ---- one rounding (the hardware's round-to-nearest-even convert), and each lane stores its own
    //      elements with 2-byte streaming stores (the 32 lanes of a half-wave cover 64 contiguous bytes
    //      of a row).  32x32 block layout: lane holds column lane%32 and, in register e, row 8*(e/4) +
    //      4*(lane/32) + e%4.  A tile wholly inside y takes a path with no bounds test: each row's
    //      address is a scalar base plus one lane offset worked out once (a per-store 64-bit multiply
    //      and exec-mask branch made the stores take 8.5 us of a tile at the 13B stack's shapes, 2.6 us
    //      without).  At 4096 x 4096 every tile ends at about the same time and y leaves in one burst
    //      at the write rate: stores that keep their lines in the caches made that about 4 us longer,
    //      and 8-byte stores of the transposed block (MFMA operands swapped) 50 us longer.
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    if (m0 + BM <= T && n0 + BN <= H) {
        const uint32_t loff = (uint32_t)(4 * (lane >> 5)) * (uint32_t)H + (uint32_t)(lane & 31);
#pragma unroll
        for (int mi = 0; mi < WMI; ++mi)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int e2 = 0; e2 < 2; ++e2) {
                    // registers e and e + 1: rows 8 g + 2 e2 and the next of the block (+ 4 in the upper half-wave)
                    uint16_t *rb = y + (int64_t)(m0 + wm * WTM + mi * 32 + 8 * g + 2 * e2) * H + n0 + wn * WTN;
                    const int e = 4 * g + 2 * e2;
#pragma unroll
                    for (int ni = 0; ni < WNI; ++ni) {
                        const bf16x2_t pv = {(__bf16)acc[mi][ni][e], (__bf16)acc[mi][ni][e + 1]};
                        const uint32_t w = __builtin_bit_cast(uint32_t, pv);
                        __builtin_nontemporal_store((uint16_t)w, rb + loff + ni * 32);
                        __builtin_nontemporal_store((uint16_t)(w >> 16), rb + H + loff + ni * 32);
                    }
                }
        return;
    }
#pragma unroll
    for (int mi = 0; mi < WMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < WNI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = wm * WTM + mi * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e & 3);
                const int col = wn * WTN + ni * 32 + (lane & 31);
                if (m0 + row < T && n0 + col < H)
                    __builtin_nontemporal_store(__builtin_bit_cast(uint16_t, (__bf16)acc[mi][ni][e]),
                                                y + (int64_t)(m0 + row) * H + n0 + col);
            }
}

// One slot per launch, and the n slots of one call (blockIdx.z = the slot; the slots share x and the
// token grouping); the one-slot kernel keeps the short argument block.
__global__ __launch_bounds__(PF_THREADS, 1) void k_prefill_main(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, const uint16_t *__restrict__ pages,
    const int32_t *__restrict__ pt, int32_t stride, const int32_t *__restrict__ tok_a,
    const int32_t *__restrict__ tok_r, const uint16_t *__restrict__ v16, int32_t R, int32_t T, int32_t H,
    int32_t n_tiles_n, uint16_t *__restrict__ y) {
    prefill_main_body<false>(x, W, pages, pt, stride, tok_a, tok_r, v16, R, T, H, n_tiles_n, y, blockIdx.x, gridDim.x);
}

__global__ __launch_bounds__(PF_THREADS, 1) void k_prefill_main_dbg(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, const uint16_t *__restrict__ pages,
    const int32_t *__restrict__ pt, int32_t stride, const int32_t *__restrict__ tok_a,
    const int32_t *__restrict__ tok_r, const uint16_t *__restrict__ v16, int32_t R, int32_t T, int32_t H,
    int32_t n_tiles_n, uint16_t *__restrict__ y, const DebugOut dbg) {
    prefill_main_body<true>(x, W, pages, pt, stride, tok_a, tok_r, v16, R, T, H, n_tiles_n, y, blockIdx.x, gridDim.x,
                            dbg);
}

__global__ __launch_bounds__(PF_THREADS, 1) void k_prefill_main_slots(
    const SlotPtrs sp, const uint16_t *__restrict__ pages, int32_t stride,
    const int32_t *__restrict__ tok_a, const int32_t *__restrict__ tok_r, int32_t R, int32_t T, int32_t H,
    int32_t n_tiles_n, int32_t n) {
    // One grid of n x nblk workgroups: first the last row of tiles of every slot (P0 each, slot after
    // slot), then the other tiles, slot after slot.  So every slot's longest tiles (the decode rows'
    // adapters) start at the beginning, not only the first slot's; both parts are multiples of 8, so
    // each workgroup keeps the XCD the one-slot order gives it.
    const int P0 = (n_tiles_n + 7) / 8 * 8, nblk = (int)gridDim.x / n, b = blockIdx.x;
    int z, blk;
    if (b < n * P0) {
        z = b / P0;
        blk = b % P0;
    } else {
        const int b2 = b - n * P0, G = nblk - P0;   // G > 0 here: b < n nblk
        z = b2 / G;
        blk = P0 + b2 % G;
    }
    prefill_main_body<false>((const uint16_t *)sp.x[z], (const uint16_t *)sp.W[z], pages, sp.pt[z], stride, tok_a, tok_r,
                             (const uint16_t *)sp.v16[z], R, T, H, n_tiles_n, (uint16_t *)sp.y[z], blk, nblk);
}

hipError_t launch_prefill(const lora_pool *p, const Plan &plan, const Ws &ws, const void *x, const float *scale,
                          const SlotPtrs &sp, int n, hipStream_t s, hipEvent_t mid, const DebugOut *dbg) {
    static bool attr_set = false;
    if (!attr_set) {
        const struct { const void *f; int lds; } attrs[] = {
            {(const void *)k_prefill_main, (int)MAIN_LDS},
            {(const void *)k_prefill_main_slots, (int)MAIN_LDS},
            {(const void *)k_prefill_main_dbg, (int)MAIN_LDS},
            {(const void *)k_shrink_mfma_dbg<6>, (int)(6 * SH_STAGE * 2)},
            {(const void *)k_shrink_mfma_dbg<4>, (int)(4 * SH_STAGE * 2)},
            {(const void *)k_shrink_mfma<6>, (int)(6 * SH_STAGE * 2)},
            {(const void *)k_shrink_mfma_slots<6>, (int)(6 * SH_STAGE * 2)},
            {(const void *)k_shrink_mfma<4>, (int)(4 * SH_STAGE * 2)},
            {(const void *)k_shrink_mfma_slots<4>, (int)(4 * SH_STAGE * 2)},
        };
        for (const auto &a : attrs) {
            const hipError_t e = hipFuncSetAttribute(a.f, hipFuncAttributeMaxDynamicSharedMemorySize, a.lds);
            if (e != hipSuccess) return e;
        }
        attr_set = true;
    }
    if (plan.vsplit != VSPLIT) return hipErrorInvalidValue;
    const uint16_t *xh = (const uint16_t *)x, *pages = (const uint16_t *)p->pages;
    const int32_t stride = 2 * p->max_rank, T = (int32_t)plan.T;
    // the persistent shrink grid: as many workgroups as the chip holds at once (one per CU with six
    // stages, two with four), a multiple of 8
    const int sns = plan.T <= 4096 ? 6 : 4;
    const size_t sh_lds = (size_t)sns * SH_STAGE * 2;
    static int n_cu[64] = {};
    if (p->device < 0 || p->device >= 64) return hipErrorInvalidDevice;
    if (n_cu[p->device] == 0) {
        int c = 0;
        const hipError_t e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, p->device);
        if (e != hipSuccess) return e;
        n_cu[p->device] = c > 0 ? c : 1;
    }
    const dim3 g1((unsigned)((n_cu[p->device] * (sns == 6 ? 1 : 2) + 7) / 8 * 8));
    if (dbg) {
        if (sns == 6)
            hipLaunchKernelGGL(k_shrink_mfma_dbg<6>, g1, dim3(256), sh_lds, s, xh, pages, p->hidden, sp.pt[0], stride,
                               ws.perm, ws.item_rec, plan.n_items_max, sp.v[0], T, plan.rp, *dbg);
        else
            hipLaunchKernelGGL(k_shrink_mfma_dbg<4>, g1, dim3(256), sh_lds, s, xh, pages, p->hidden, sp.pt[0], stride,
                               ws.perm, ws.item_rec, plan.n_items_max, sp.v[0], T, plan.rp, *dbg);
    } else if (n == 1) {
        if (sns == 6)
            hipLaunchKernelGGL(k_shrink_mfma<6>, g1, dim3(256), sh_lds, s, xh, pages, p->hidden, sp.pt[0], stride,
                               ws.perm, ws.item_rec, plan.n_items_max, sp.v[0], T, plan.rp);
        else
            hipLaunchKernelGGL(k_shrink_mfma<4>, g1, dim3(256), sh_lds, s, xh, pages, p->hidden, sp.pt[0], stride,
                               ws.perm, ws.item_rec, plan.n_items_max, sp.v[0], T, plan.rp);
    } else {
        if (sns == 6)
            hipLaunchKernelGGL(k_shrink_mfma_slots<6>, g1, dim3(256), sh_lds, s, pages, p->hidden, sp, (int32_t)n,
                               stride, ws.perm, ws.item_rec, plan.n_items_max, T, plan.rp);
        else
            hipLaunchKernelGGL(k_shrink_mfma_slots<4>, g1, dim3(256), sh_lds, s, pages, p->hidden, sp, (int32_t)n,
                               stride, ws.perm, ws.item_rec, plan.n_items_max, T, plan.rp);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nthr = plan.T * (plan.rp / 4);
    const dim3 gf((unsigned)((nthr + 255) / 256), 1, n);
    if (n == 1)
        hipLaunchKernelGGL(k_v_finalize, gf, dim3(256), 0, s, sp.v[0], ws.tok_a, ws.tok_r, scale, T, plan.rp,
                           sp.v16[0]);
    else
        hipLaunchKernelGGL(k_v_finalize_slots, gf, dim3(256), 0, s, sp, ws.tok_a, ws.tok_r, scale, T, plan.rp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (mid && (e = hipEventRecord(mid, s)) != hipSuccess) return e;
    const int tn = (p->hidden + BN - 1) / BN, tm = (int)((plan.T + BM - 1) / BM);
    const int grid = (tn + 7) / 8 * 8 + ((tm - 1) * tn + 7) / 8 * 8;   // the last row of tiles, then the rest
    if (dbg)
        hipLaunchKernelGGL(k_prefill_main_dbg, dim3(grid), dim3(PF_THREADS), MAIN_LDS, s, xh, (const uint16_t *)sp.W[0],
                           pages, sp.pt[0], stride, ws.tok_a, ws.tok_r, (const uint16_t *)sp.v16[0], plan.rp, T,
                           p->hidden, tn, (uint16_t *)sp.y[0], *dbg);
    else if (n == 1)
        hipLaunchKernelGGL(k_prefill_main, dim3(grid), dim3(PF_THREADS), MAIN_LDS, s, xh, (const uint16_t *)sp.W[0],
                           pages, sp.pt[0], stride, ws.tok_a, ws.tok_r, (const uint16_t *)sp.v16[0], plan.rp, T,
                           p->hidden, tn, (uint16_t *)sp.y[0]);
    else
        hipLaunchKernelGGL(k_prefill_main_slots, dim3(grid * n), dim3(PF_THREADS), MAIN_LDS, s, sp, pages,
                           stride, ws.tok_a, ws.tok_r, plan.rp, T, p->hidden, tn, n);
    return hipGetLastError();
}

}  // namespace lorapool
