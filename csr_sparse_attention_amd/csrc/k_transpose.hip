// Transposition of a CSR pattern (the CSR of A^T, i.e. A in CSC) for the
// backward products, and the gather that moves per-entry values into the
// transposed order.  Entries of each column keep the order of their rows (a
// stable sort by column), so the result and every product built on it are
// deterministic.
#include <rocprim/device/device_radix_sort.hpp>

#include "common.h"
#include "launch.h"

namespace csrk {

__global__ void k_iota(int32_t* v, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        v[i] = (int32_t)i;
}

// last row i in [lo, hi] with row_ptr[i] <= e
__device__ __forceinline__ int64_t row_search(const int32_t* row_ptr, int64_t lo, int64_t hi, int64_t e)
{
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (row_ptr[mid] <= e)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// rows[e] = the row holding entry e (the COO row array).  A block covers 256
// consecutive entries: two full searches find the rows of its first and last
// entry, and every entry is then searched only between those two rows (one
// or two steps for rows of tens of entries).
__global__ __launch_bounds__(CSR_BLOCK) void k_coo_rows(const int32_t* row_ptr, int64_t n_rows, int32_t* rows,
                                                        int64_t nnz)
{
    __shared__ int64_t span[2];
    const int64_t e0 = (int64_t)blockIdx.x * CSR_BLOCK;
    if (threadIdx.x < 2) {
        const int64_t e = threadIdx.x == 0 ? e0 : min(e0 + CSR_BLOCK, nnz) - 1;
        span[threadIdx.x] = row_search(row_ptr, 0, n_rows - 1, e);
    }
    __syncthreads();
    const int64_t e = e0 + threadIdx.x;
    if (e < nnz) rows[e] = (int32_t)row_search(row_ptr, span[0], span[1], e);
}

// t_row_ptr[c] = number of sorted column keys below c, for c in [0, n_cols]
__global__ void k_col_starts(const int32_t* keys, int64_t nnz, int32_t* t_row_ptr, int64_t n_cols)
{
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c <= n_cols; c += (int64_t)gridDim.x * blockDim.x) {
        int64_t lo = 0, hi = nnz;
        while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if ((int64_t)keys[mid] < c)
                lo = mid + 1;
            else
                hi = mid;
        }
        t_row_ptr[c] = (int32_t)lo;
    }
}

__global__ void k_gather_rows(const int32_t* perm, const int32_t* src, int32_t* dst, int64_t n)
{
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x)
        dst[k] = src[perm[k]];
}

__global__ void k_gather_values(const int32_t* perm, const float* src, float* dst, int64_t n)
{
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x)
        dst[k] = src[perm[k]];
}

static unsigned grid_of(int64_t n)
{
    int64_t b = (n + CSR_BLOCK - 1) / CSR_BLOCK;
    return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

static int key_bits(int64_t n_cols)
{
    int bits = 1;
    while (bits < 31 && ((int64_t)1 << bits) < n_cols) ++bits;
    return bits;
}

static size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

hipError_t transpose_workspace(int64_t n_cols, int64_t nnz, size_t* bytes)
{
    size_t temp = 0;
    hipError_t e = rocprim::radix_sort_pairs(nullptr, temp, (const int32_t*)nullptr, (int32_t*)nullptr,
                                             (const int32_t*)nullptr, (int32_t*)nullptr, (unsigned)nnz, 0,
                                             key_bits(n_cols));
    if (e != hipSuccess) return e;
    *bytes = 2 * up256((size_t)nnz * 4) + up256(temp);
    return hipSuccess;
}

hipError_t launch_transpose(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_cols,
                            int64_t nnz, int32_t* t_row_ptr, int32_t* t_col_idx, int32_t* t_perm, void* ws,
                            size_t ws_bytes, hipStream_t s)
{
    if (nnz == 0) {
        hipLaunchKernelGGL(k_col_starts, dim3(grid_of(n_cols + 1)), dim3(CSR_BLOCK), 0, s, col_idx, (int64_t)0,
                           t_row_ptr, n_cols);
        return hipGetLastError();
    }
    char* w = static_cast<char*>(ws);
    int32_t* iota = reinterpret_cast<int32_t*>(w);
    int32_t* keys = reinterpret_cast<int32_t*>(w + up256((size_t)nnz * 4));
    void* temp = w + 2 * up256((size_t)nnz * 4);
    size_t temp_bytes = ws_bytes - 2 * up256((size_t)nnz * 4);
    hipLaunchKernelGGL(k_iota, dim3(grid_of(nnz)), dim3(CSR_BLOCK), 0, s, iota, nnz);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = rocprim::radix_sort_pairs(temp, temp_bytes, col_idx, keys, (const int32_t*)iota, t_perm, (unsigned)nnz, 0,
                                  key_bits(n_cols), s);
    if (e != hipSuccess) return e;
    // the sort no longer needs the entry indices: their buffer takes the COO
    // rows, and each transposed entry's row is gathered through the permutation
    int32_t* rows = iota;
    const int64_t blocks = (nnz + CSR_BLOCK - 1) / CSR_BLOCK;
    hipLaunchKernelGGL(k_coo_rows, dim3((unsigned)blocks), dim3(CSR_BLOCK), 0, s, row_ptr, n_rows, rows, nnz);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_gather_rows, dim3(grid_of(nnz)), dim3(CSR_BLOCK), 0, s, (const int32_t*)t_perm,
                       (const int32_t*)rows, t_col_idx, nnz);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_col_starts, dim3(grid_of(n_cols + 1)), dim3(CSR_BLOCK), 0, s, (const int32_t*)keys, nnz,
                       t_row_ptr, n_cols);
    return hipGetLastError();
}

hipError_t launch_coo_rows(const int32_t* row_ptr, int64_t n_rows, int32_t* rows, int64_t nnz, hipStream_t s)
{
    if (nnz == 0) return hipSuccess;
    const int64_t blocks = (nnz + CSR_BLOCK - 1) / CSR_BLOCK;
    hipLaunchKernelGGL(k_coo_rows, dim3((unsigned)blocks), dim3(CSR_BLOCK), 0, s, row_ptr, n_rows, rows, nnz);
    return hipGetLastError();
}

hipError_t launch_gather_values(const int32_t* perm, const float* src, float* dst, int64_t n, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_gather_values, dim3(grid_of(n)), dim3(CSR_BLOCK), 0, s, perm, src, dst, n);
    return hipGetLastError();
}

}  // namespace csrk
