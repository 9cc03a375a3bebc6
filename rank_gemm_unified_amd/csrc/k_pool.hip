// Kernels behind adapter loads and evictions: copy an adapter's A columns and B rows into the
// pool pages its page list names, and write or clear its page-table rows.
#include "device_common.h"
#include "internal.h"

namespace lorapool {

// One workgroup per (slot, row) of the source; each copies one H-element vector into its page.
__global__ __launch_bounds__(256) void k_scatter_rows(char *__restrict__ pages, int32_t row_bytes,
                                                      const char *__restrict__ A_t, const char *__restrict__ B,
                                                      int64_t slot_stride_bytes, int32_t slot0, int32_t rank,
                                                      const int32_t *__restrict__ rows, int32_t row_stride) {
    const int32_t s = blockIdx.x / (2 * rank);
    const int32_t jj = blockIdx.x % (2 * rank);
    const char *src = jj < rank ? A_t + s * slot_stride_bytes + (int64_t)jj * row_bytes
                                : B + s * slot_stride_bytes + (int64_t)(jj - rank) * row_bytes;
    const int32_t page = rows[(int64_t)(slot0 + s) * row_stride + jj];
    char *dst = pages + (int64_t)page * row_bytes;
    for (int32_t i = threadIdx.x; i < row_bytes / 16; i += blockDim.x) store16(dst + 16 * i, load16(src + 16 * i));
}

__global__ void k_write_rows(int32_t *__restrict__ pt, int32_t max_adapters, int32_t row_stride, int32_t adapter,
                             const int32_t *__restrict__ rows) {
    const int32_t slot = blockIdx.x;
    int32_t *dst = pt + ((int64_t)slot * max_adapters + adapter) * row_stride;
    for (int32_t j = threadIdx.x; j < row_stride; j += blockDim.x) dst[j] = rows[(int64_t)slot * row_stride + j];
}

__global__ void k_clear_rows(int32_t *__restrict__ pt, int32_t max_adapters, int32_t row_stride, int32_t adapter) {
    const int32_t slot = blockIdx.x;
    int32_t *dst = pt + ((int64_t)slot * max_adapters + adapter) * row_stride;
    for (int32_t j = threadIdx.x; j < row_stride; j += blockDim.x) dst[j] = -1;
}

hipError_t launch_scatter_rows(void *pages, int32_t hidden, int32_t elem, const void *A_t, const void *B,
                               int64_t src_slot_stride_elems, int32_t slot0, int32_t n_slots_chunk, int32_t rank,
                               const int32_t *rows, int32_t row_stride, hipStream_t s) {
    if (rank <= 0 || n_slots_chunk <= 0) return hipSuccess;
    const int64_t blocks = (int64_t)n_slots_chunk * 2 * rank;
    hipLaunchKernelGGL(k_scatter_rows, dim3((unsigned)blocks), dim3(256), 0, s, (char *)pages, hidden * elem,
                       (const char *)A_t, (const char *)B, src_slot_stride_elems * elem, slot0, rank, rows, row_stride);
    return hipGetLastError();
}

hipError_t launch_write_rows(int32_t *pt, int32_t max_adapters, int32_t row_stride, int32_t adapter,
                             const int32_t *rows, int32_t n_slots, hipStream_t s) {
    hipLaunchKernelGGL(k_write_rows, dim3(n_slots), dim3(128), 0, s, pt, max_adapters, row_stride, adapter, rows);
    return hipGetLastError();
}

hipError_t launch_clear_rows(int32_t *pt, int32_t max_adapters, int32_t row_stride, int32_t adapter,
                             int32_t n_slots, hipStream_t s) {
    hipLaunchKernelGGL(k_clear_rows, dim3(n_slots), dim3(128), 0, s, pt, max_adapters, row_stride, adapter);
    return hipGetLastError();
}

}  // namespace lorapool
