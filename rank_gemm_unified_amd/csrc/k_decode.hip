// Decode-shaped projection (few tokens, each request one token): memory-bound, so the kernels are
// organised around streaming W and the gathered A/B pages from HBM exactly once.
//
//   k_shrink_gather  v[t][j] = s_a * <x_t, A_a[:, j]>: one wave per A page (one column of A),
//                    dotted with every token of the adapter's group ("two skinny matmuls", the
//                    first one; "S-LoRA, in depth", section "Merge or keep adapters separate").
//   k_base_expand    y = x W over all tokens (MFMA bf16, split over K across workgroups), plus
//                    v (B rows gathered from their pages), accumulated in float32 and rounded once.
#include "device_common.h"
#include "internal.h"

namespace lorapool {

constexpr int SHRINK_TOK = 16;   // tokens per shrink work item (decode)

// ---- shrink: one wave per (work item, page j) --------------------------------------------------
template <int EB>   // element bytes: 2 = bf16, 4 = f32
__global__ __launch_bounds__(256) void k_shrink_gather(
    const char *__restrict__ x, const char *__restrict__ pages, int32_t H, const int32_t *__restrict__ pt,
    int32_t stride, const float *__restrict__ scale, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ seg_a, const int32_t *__restrict__ seg_start, const int32_t *__restrict__ item_seg,
    const int32_t *__restrict__ item_row, const int32_t *__restrict__ ctrl, const int32_t *__restrict__ tok_r,
    float *__restrict__ v, int32_t R) {
    const int item = blockIdx.x;
    if (item >= ctrl[CTRL_NITEMS]) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int32_t s = item_seg[item], row0 = item_row[item];
    const int32_t n = min(seg_start[s + 1] - row0, SHRINK_TOK);
    const int32_t a = seg_a[s];
    const int32_t r = tok_r[perm[row0]];
    const int32_t j = blockIdx.y * 4 + wave;
    if (j >= r) return;
    const int64_t row_bytes = (int64_t)H * EB;
    const char *Ap = pages + (int64_t)pt[(int64_t)a * stride + j] * row_bytes;
    int32_t tok[SHRINK_TOK];
#pragma unroll
    for (int i = 0; i < SHRINK_TOK; ++i) tok[i] = i < n ? perm[row0 + i] : 0;
    float acc[SHRINK_TOK];
#pragma unroll
    for (int i = 0; i < SHRINK_TOK; ++i) acc[i] = 0.f;
    constexpr int EPV = 16 / EB;   // elements per 16-byte vector
    constexpr int BLK = 8;         // 16-byte vectors per lane per block (8 KiB per wave)
    for (int64_t base = 0; base < row_bytes; base += 64 * 16 * BLK) {
        u32x4_t av[BLK];
        float af[BLK][EPV];
#pragma unroll
        for (int b = 0; b < BLK; ++b) {
            const int64_t off = base + (int64_t)(b * 64 + lane) * 16;
            av[b] = off < row_bytes ? load16(Ap + off) : u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int b = 0; b < BLK; ++b) {
            if constexpr (EB == 2) {
                unpack_bf16x8(av[b], af[b]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) af[b][e] = __uint_as_float(av[b][e]);
            }
        }
#pragma unroll
        for (int i = 0; i < SHRINK_TOK; ++i) {
            if (i < n) {
                const char *xr = x + (int64_t)tok[i] * row_bytes;
                u32x4_t xv[BLK];
#pragma unroll
                for (int b = 0; b < BLK; ++b) {
                    const int64_t off = base + (int64_t)(b * 64 + lane) * 16;
                    xv[b] = off < row_bytes ? load16(xr + off) : u32x4_t{0, 0, 0, 0};
                }
#pragma unroll
                for (int b = 0; b < BLK; ++b) {
                    float xf[EPV];
                    if constexpr (EB == 2) {
                        unpack_bf16x8(xv[b], xf);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) xf[e] = __uint_as_float(xv[b][e]);
                    }
#pragma unroll
                    for (int e = 0; e < EPV; ++e) acc[i] = fmaf(af[b][e], xf[e], acc[i]);
                }
            }
        }
    }
    const float sc = scale[a];
#pragma unroll
    for (int i = 0; i < SHRINK_TOK; ++i) {
        if (i < n) {
            const float tot = wave_sum(acc[i]);
            if (lane == 0) v[(int64_t)tok[i] * R + j] = sc * tot;
        }
    }
}

// ---- base GEMM (bf16 MFMA 16x16x32) + expand, split over K ------------------------------------
//
// Grid (H/64 column tiles, S splits).  256 threads = 4 waves laid out WM (along M) x WK (along K).
// Wave (wm, wk) owns rows [wm*MB*16, (wm+1)*MB*16) and one of the WK*S slices of K; all 64 columns
// of the tile.  Partial sums of the WK waves meet in LDS; each split adds its share of the
// low-rank term (a slice of j for every token), writes a float32 partial, and the last split to
// arrive for a tile adds the S partials in split order, rounds once, and stores y.
constexpr int NT = 64;            // columns per tile
constexpr int NB = NT / 16;       // 16-column MFMA blocks per tile

template <int MB, int WM>
__global__ __launch_bounds__(256) void k_base_expand(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, const uint16_t *__restrict__ pages,
    const int32_t *__restrict__ pt, int32_t stride, const int32_t *__restrict__ tok_a,
    const int32_t *__restrict__ tok_r, const float *__restrict__ v, int32_t R, int32_t T, int32_t H,
    float *__restrict__ ypart, int32_t *__restrict__ counters, uint16_t *__restrict__ y) {
    constexpr int WK = 4 / WM;
    constexpr int TP = WM * MB * 16;   // padded rows
    extern __shared__ float red[];     // [WK][TP][NT] when WK > 1
    __shared__ int s_last;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave % WM, wk = wave / WM;
    const int n0 = blockIdx.x * NT;
    const int S = gridDim.y, split = blockIdx.y;
    const int G = S * WK, g = split * WK + wk;
    const int ksteps = H / 32;
    const int kb = (int)((int64_t)ksteps * g / G) * 32, ke = (int)((int64_t)ksteps * (g + 1) / G) * 32;

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

    constexpr int U = 4;   // K-steps of 32 in flight per wave
    int k = kb;
    for (; k + 32 * U <= ke; k += 32 * U) {
        u32x4_t xa[U][MB], wb[U][NB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) wb[u][nb] = load16(wrow[nb] + k + 32 * u);
#pragma unroll
            for (int m = 0; m < MB; ++m)
                xa[u][m] = xval[m] ? load16(xrow[m] + k + 32 * u) : u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, xa[u][m]), __builtin_bit_cast(bf16x8_t, wb[u][nb]),
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

    // accumulator layout (16x16 block): lane holds rows 4*(lane/16)+i, column lane%16
    float *mine = red + (size_t)wk * TP * NT;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = (wm * MB + m) * 16 + (lane >> 4) * 4 + i;
                mine[row * NT + nb * 16 + (lane & 15)] = acc[m][nb][i];
            }
    __syncthreads();

    // epilogue: thread -> (token t, 8 consecutive columns)
    const bool single = (S == 1);
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
        // this split's slice of the low-rank term: j in [r*split/S, r*(split+1)/S)
        const int32_t a = tok_a[t];
        if (a >= 0) {
            const int32_t r = tok_r[t];
            const int32_t j0 = r * split / S, j1 = r * (split + 1) / S;
            const int32_t *prow = pt + (int64_t)a * stride + r;
            const float *vt = v + (int64_t)t * R;
            for (int32_t j = j0; j < j1; ++j) {
                const u32x4_t b = load16(pages + (int64_t)prow[j] * H + n0 + c);
                float bf[8];
                unpack_bf16x8(b, bf);
                const float vj = vt[j];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = fmaf(vj, bf[e], o[e]);
            }
        }
        if (single) {
            store16(y + (int64_t)t * H + n0 + c, pack_bf16x8(o));
        } else {
            float *dst = ypart + ((int64_t)split * T + t) * H + n0 + c;
            *reinterpret_cast<f32x4_t *>(dst) = f32x4_t{o[0], o[1], o[2], o[3]};
            *reinterpret_cast<f32x4_t *>(dst + 4) = f32x4_t{o[4], o[5], o[6], o[7]};
        }
    }
    if (single) return;

    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) s_last = (atomicAdd(&counters[blockIdx.x], 1) == S - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int p = threadIdx.x; p < T * (NT / 8); p += 256) {
        const int t = p / (NT / 8), c = (p % (NT / 8)) * 8;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
        for (int q = 0; q < S; ++q) {
            const float *src = ypart + ((int64_t)q * T + t) * H + n0 + c;
            const f32x4_t lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(src));
            const f32x4_t hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(src + 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[e] += lo[e];
                o[e + 4] += hi[e];
            }
        }
        store16(y + (int64_t)t * H + n0 + c, pack_bf16x8(o));
    }
}

// ---- float32 pools: plain VALU kernel (correctness path; tiny shapes) --------------------------
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

// ---- launchers -----------------------------------------------------------------------------------
template <int EB>
static hipError_t launch_shrink_gather(const lora_pool *p, const Plan &plan, const Ws &ws, const void *x,
                                       const int32_t *pt, const float *scale, hipStream_t s) {
    dim3 grid(plan.n_items_max, (p->max_rank + 3) / 4);
    hipLaunchKernelGGL(k_shrink_gather<EB>, grid, dim3(256), 0, s, (const char *)x, (const char *)p->pages,
                       p->hidden, pt, 2 * p->max_rank, scale, ws.perm, ws.seg_a, ws.seg_start, ws.item_seg,
                       ws.item_row, ws.ctrl, ws.tok_r, ws.v, p->max_rank);
    return hipGetLastError();
}

template <int MB, int WM>
static hipError_t launch_be(const lora_pool *p, const Plan &plan, const Ws &ws, const void *x, const void *W,
                            const int32_t *pt, void *y, hipStream_t s) {
    constexpr int WK = 4 / WM;
    const size_t lds = (size_t)WK * WM * MB * 16 * NT * sizeof(float);
    dim3 grid(p->hidden / NT, plan.ysplit);
    hipLaunchKernelGGL((k_base_expand<MB, WM>), grid, dim3(256), lds, s, (const uint16_t *)x, (const uint16_t *)W,
                       (const uint16_t *)p->pages, pt, 2 * p->max_rank, ws.tok_a, ws.tok_r, ws.v, p->max_rank,
                       (int32_t)plan.T, p->hidden, ws.ypart, ws.counters, (uint16_t *)y);
    return hipGetLastError();
}

hipError_t launch_decode(const lora_pool *p, const Plan &plan, const Ws &ws, const void *x, const void *W,
                         const int32_t *pt, const float *scale, void *y, hipStream_t s, hipEvent_t mid) {
    hipError_t e = launch_shrink_gather<2>(p, plan, ws, x, pt, scale, s);
    if (e != hipSuccess) return e;
    if (mid && (e = hipEventRecord(mid, s)) != hipSuccess) return e;
    switch (plan.wm * 8 + plan.mb) {
        case 1 * 8 + 1: return launch_be<1, 1>(p, plan, ws, x, W, pt, y, s);
        case 1 * 8 + 2: return launch_be<2, 1>(p, plan, ws, x, W, pt, y, s);
        case 1 * 8 + 3: return launch_be<3, 1>(p, plan, ws, x, W, pt, y, s);
        case 1 * 8 + 4: return launch_be<4, 1>(p, plan, ws, x, W, pt, y, s);
        case 2 * 8 + 4: return launch_be<4, 2>(p, plan, ws, x, W, pt, y, s);
        case 4 * 8 + 4: return launch_be<4, 4>(p, plan, ws, x, W, pt, y, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_f32(const lora_pool *p, const Plan &plan, const Ws &ws, const void *x, const void *W,
                      const int32_t *pt, const float *scale, void *y, hipStream_t s, hipEvent_t mid) {
    hipError_t e = launch_shrink_gather<4>(p, plan, ws, x, pt, scale, s);
    if (e != hipSuccess) return e;
    if (mid && (e = hipEventRecord(mid, s)) != hipSuccess) return e;
    dim3 grid(p->hidden / 64, (unsigned)((plan.T + 15) / 16));
    hipLaunchKernelGGL(k_project_f32, grid, dim3(256), 0, s, (const float *)x, (const float *)W,
                       (const float *)p->pages, pt, 2 * p->max_rank, ws.tok_a, ws.tok_r, ws.v, p->max_rank,
                       (int32_t)plan.T, p->hidden, (float *)y);
    return hipGetLastError();
}

}  // namespace lorapool
