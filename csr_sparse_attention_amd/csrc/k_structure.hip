// Integer kernels of the schedule path: fills, degree histogram, merge-path
// partition, optional CSR validation.
#include "launch.h"
#include "common.h"

namespace csrk {

__global__ void k_fill_i64(int64_t* p, int64_t n, int64_t value)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

// out: int64 [67] = counts[33], degree sums[33], max degree; zeroed beforehand.
// Bucket of degree d: 0 for d = 0, else the bit length of d (floor(log2 d) + 1).
__global__ __launch_bounds__(CSR_BLOCK) void k_degree_hist(const int32_t* row_ptr, int64_t n_rows, int64_t* out)
{
    __shared__ unsigned int cnt[33];
    __shared__ unsigned long long sum[33];
    __shared__ int mx;
    for (int i = threadIdx.x; i < 33; i += blockDim.x) {
        cnt[i] = 0;
        sum[i] = 0;
    }
    if (threadIdx.x == 0) mx = 0;
    __syncthreads();
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_rows; i += (int64_t)gridDim.x * blockDim.x) {
        const int d = row_ptr[i + 1] - row_ptr[i];
        const int b = (d == 0) ? 0 : 32 - __clz(d);
        atomicAdd(&cnt[b], 1u);
        atomicAdd(&sum[b], (unsigned long long)d);
        atomicMax(&mx, d);
    }
    __syncthreads();
    unsigned long long* o = reinterpret_cast<unsigned long long*>(out);
    for (int i = threadIdx.x; i < 33; i += blockDim.x) {
        if (cnt[i]) {
            atomicAdd(&o[i], (unsigned long long)cnt[i]);
            atomicAdd(&o[33 + i], sum[i]);
        }
    }
    if (threadIdx.x == 0) atomicMax(&o[66], (unsigned long long)mx);
}

// Chunk boundary c sits at item d = min(c * items, n_rows + nnz) of the merged
// sequence; x = number of rows i whose end precedes it, i.e. with
// row_ptr[i + 1] + i + 1 <= d (a strictly increasing key), y = d - x.  With
// bounds set, also the entry range of row x: bounds[2c] = row_ptr[x],
// bounds[2c + 1] = row_ptr[x + 1] (both nnz when x = n_rows).
__global__ void k_merge_path(const int32_t* row_ptr, int64_t n_rows, int64_t nnz, int64_t items,
                             int64_t n_chunks, int32_t* coords, int32_t* bounds)
{
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c > n_chunks) return;
    const int64_t total = n_rows + nnz;
    const int64_t d = min(c * items, total);
    int64_t lo = max((int64_t)0, d - nnz), hi = min(d, n_rows);
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if ((int64_t)row_ptr[mid + 1] + mid + 1 <= d)
            lo = mid + 1;
        else
            hi = mid;
    }
    // clamped to the arrays' extents: a row_ptr whose last value is not nnz
    // then gives wrong results instead of reads past the entry arrays
    coords[2 * c] = (int32_t)lo;
    coords[2 * c + 1] = (int32_t)min(d - lo, nnz);
    if (bounds) {
        bounds[2 * c] = lo < n_rows ? (int32_t)min((int64_t)row_ptr[lo], nnz) : (int32_t)nnz;
        bounds[2 * c + 1] = lo < n_rows ? (int32_t)min((int64_t)row_ptr[lo + 1], nnz) : (int32_t)nnz;
    }
}

// Counts violations of the CSR invariants into *bad (zeroed beforehand).
// col_idx may be null (the row softmax and its backward read no columns):
// then only row_ptr is checked.
__global__ void k_validate(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_cols,
                           int64_t nnz, int64_t* bad)
{
    unsigned long long local = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t == 0) local += (row_ptr[0] != 0) + ((int64_t)row_ptr[n_rows] != nnz);
    for (int64_t i = t; i < n_rows; i += stride) local += row_ptr[i + 1] < row_ptr[i];
    if (col_idx) {
        for (int64_t e = t; e < nnz; e += stride) {
            const int c = col_idx[e];
            local += (c < 0) || ((int64_t)c >= n_cols);
        }
    }
    if (local) atomicAdd(reinterpret_cast<unsigned long long*>(bad), local);
}

// Adds to *bad the number of idx[i], i < n, outside [0, bound).
__global__ void k_validate_index(const int32_t* idx, int64_t n, int64_t bound, int64_t* bad)
{
    unsigned long long local = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int v = idx[i];
        local += (v < 0) || ((int64_t)v >= bound);
    }
    if (local) atomicAdd(reinterpret_cast<unsigned long long*>(bad), local);
}

static unsigned grid_for(int64_t n, int64_t cap)
{
    int64_t b = (n + CSR_BLOCK - 1) / CSR_BLOCK;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (unsigned)b;
}

__global__ void k_fill_f32(float* p, int64_t n, float value)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_f32, dim3(grid_for(n, 65536)), dim3(CSR_BLOCK), 0, s, p, n, value);
    return hipGetLastError();
}

hipError_t launch_fill_i64(int64_t* p, int64_t n, int64_t value, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_i64, dim3(grid_for(n, 4096)), dim3(CSR_BLOCK), 0, s, p, n, value);
    return hipGetLastError();
}

hipError_t launch_degree_hist(const int32_t* row_ptr, int64_t n_rows, int64_t* out, hipStream_t s)
{
    hipError_t e = launch_fill_i64(out, 67, 0, s);
    if (e != hipSuccess || n_rows <= 0) return e;
    hipLaunchKernelGGL(k_degree_hist, dim3(grid_for(n_rows, 2048)), dim3(CSR_BLOCK), 0, s, row_ptr, n_rows, out);
    return hipGetLastError();
}

hipError_t launch_merge_path(const int32_t* row_ptr, int64_t n_rows, int64_t nnz, int64_t items,
                             int64_t n_chunks, int32_t* coords, hipStream_t s, int32_t* bounds)
{
    hipLaunchKernelGGL(k_merge_path, dim3(grid_for(n_chunks + 1, 1 << 30)), dim3(CSR_BLOCK), 0, s, row_ptr, n_rows,
                       nnz, items, n_chunks, coords, bounds);
    return hipGetLastError();
}

hipError_t launch_validate(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_cols,
                           int64_t nnz, int64_t* bad, hipStream_t s)
{
    hipError_t e = launch_fill_i64(bad, 1, 0, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_validate, dim3(grid_for(n_rows > nnz ? n_rows : nnz, 4096)), dim3(CSR_BLOCK), 0, s, row_ptr,
                       col_idx, n_rows, n_cols, nnz, bad);
    return hipGetLastError();
}

hipError_t launch_validate_index(const int32_t* idx, int64_t n, int64_t bound, int64_t* bad, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_validate_index, dim3(grid_for(n, 4096)), dim3(CSR_BLOCK), 0, s, idx, n, bound, bad);
    return hipGetLastError();
}

} // namespace csrk
