// Device-side helpers shared by the kernels: element conversions, vector types, wave reductions,
// and the page-table row check used by every kernel that gathers pages.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace lorapool {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;   // an LDS address, as the LDS-load builtins take it

// 16 bytes per lane from a buffer resource straight into LDS: lane l's bytes land at dst + 16 l.
// (A non-template device function: a kernel template that names this builtin directly is dropped
// from the host compilation pass.)
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, lds_void *dst, uint32_t voff, int32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}
// The same from a per-lane 64-bit global address (a gather): lane l's 16 bytes land at dst + 16 l.
__device__ __forceinline__ void lds_gload16(const void *src, lds_void *dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even float32 -> bfloat16 bits; NaN stays NaN (quiet bit set).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// 8 bf16 values (one 16-byte load) -> 8 floats
__device__ __forceinline__ void unpack_bf16x8(const u32x4_t &v, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ u32x4_t pack_bf16x8(const float *f) {
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = f32_to_bf16_bits(f[2 * i]) | (f32_to_bf16_bits(f[2 * i + 1]) << 16);
    return v;
}

__device__ __forceinline__ u32x4_t load16(const void *p) { return *reinterpret_cast<const u32x4_t *>(p); }
__device__ __forceinline__ void store16(void *p, const u32x4_t &v) { *reinterpret_cast<u32x4_t *>(p) = v; }
// A streaming store: the line is not kept in the caches (for large outputs this kernel never reads)
__device__ __forceinline__ void store16_nt(void *p, const u32x4_t &v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(p));
}

// Stores of the split partials the next launch of the same call reads: written through to memory at
// system scope, so that they leave no dirty lines in this XCD's L2 for the end-of-kernel write-back
// to flush before that launch can start (measured: 0.5 us less per decode call at 64 tokens, 1.7 us
// per projection at 256 tokens and one call per slot).  The small records and v partials keep plain
// stores: written through, their scattered 4-byte pieces cost more than they save.
__device__ __forceinline__ void store16_wt(void *p, const u32x4_t &v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store4_wt(void *p, uint32_t v) {
    asm volatile("global_store_dword %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
}

// Sum over the 64 lanes of a wave; every lane gets the total.  Fixed butterfly order, so the
// result does not depend on anything but the 64 inputs.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Inclusive prefix sum over the 64 lanes: shifts of 1, 2, 4, 8 inside each row of 16 lanes (DPP;
// lanes shifted in from outside the row read 0), then the row totals carried across rows.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
              r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = lane >> 4;
    return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Debug instantiations record each page id where a kernel uses it.  The first writer of an entry
// sets it; a writer that finds a different value marks the entry -2, so two workgroups (or two
// kernels) that used different pages for the same token and j cannot hide one another.
__device__ __forceinline__ void dbg_put(int32_t *p, int32_t v) {
    const int32_t old = atomicCAS(p, -1, v);
    if (old != -1 && old != v) atomicExch(p, -2);
}

// Check adapter a's page-table row against rank r: entries [0, 2r) must be page ids in
// [0, num_pages) and, when 2r < stride, entry 2r must be -1 (so r is the loaded rank).
// `j` is this thread's entry (threads of a group cover the row together); returns error bits.
__device__ __forceinline__ int check_row_entry(const int32_t *row, int32_t j, int32_t r, int32_t stride,
                                               int64_t num_pages) {
    if (j < 2 * r) {
        const int32_t pg = row[j];
        if (pg == -1) return 4;                                   // DEV_ERR_TABLE
        if (pg < 0 || (int64_t)pg >= num_pages) return 8;         // DEV_ERR_PAGE
    } else if (j == 2 * r && j < stride) {
        if (row[j] != -1) return 4;                               // DEV_ERR_TABLE
    }
    return 0;
}

}  // namespace lorapool
