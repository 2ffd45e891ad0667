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

// rows[e] = the row holding entry e (the COO row array), written row by row:
// a wave takes 64 consecutive rows and fills each row's entries with its
// lanes, so consecutive rows' stores are adjacent and coalesced.  Row i's
// range is [row_ptr[i], row_ptr[i + 1]) clamped to [0, nnz], with the first
// row starting at 0 and the last ending at nnz: any entry x then lies in the
// range of the last row whose start is <= x, so for every row_ptr each entry
// receives a row in [0, n_rows) and no store leaves the array (a valid CSR
// gives exactly its rows).
__global__ __launch_bounds__(CSR_BLOCK) void k_coo_rows(const int32_t* row_ptr, int64_t n_rows, int32_t* rows,
                                                        int64_t nnz)
{
    const int lane = lane_id();
    const int64_t r0 = (int64_t)blockIdx.x * CSR_BLOCK + threadIdx.x - lane;
    if (r0 >= n_rows) return;
    auto bound = [&](int64_t i) -> int32_t {
        if (i == 0) return 0;
        if (i == n_rows) return (int32_t)nnz;
        const int32_t v = row_ptr[i];
        return v < 0 ? 0 : (v > nnz ? (int32_t)nnz : v);
    };
    const int64_t r = r0 + lane;
    const int32_t b = r < n_rows ? bound(r) : 0;
    const int32_t e = r < n_rows ? bound(r + 1) : 0;
    const int nr = (int)min((int64_t)CSR_WAVE, n_rows - r0);
    for (int j = 0; j < nr; ++j) {
        const int32_t bj = __builtin_amdgcn_readlane(b, j), ej = __builtin_amdgcn_readlane(e, j);
        for (int32_t k = bj + lane; k < ej; k += CSR_WAVE) rows[k] = (int32_t)(r0 + j);
    }
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

// dst[k] = src[perm[k]], one entry per thread over a grid that covers all of
// them: the waves in flight then cover one contiguous window of k (about
// 1.8x faster on a power-law transpose than a grid-stride loop, whose
// resident waves spread over the whole array)
template <typename T>
__global__ __launch_bounds__(CSR_BLOCK) void k_gather(const int32_t* perm, const T* src, T* dst, int64_t n)
{
    const int64_t k = (int64_t)blockIdx.x * CSR_BLOCK + threadIdx.x;
    if (k < n) dst[k] = src[perm[k]];
}

// One pass of a two-pass permutation: dst[j] = src[idx[j]] (0 for an index
// outside [0, n)).  Workgroups are dealt to the 8 XCDs in turn, so the grid
// is laid out XCD-major: workgroup b works on range (b % 8) * per + b / 8 of
// the n / 256 ranges, and each XCD takes one contiguous eighth of j.  In the
// first pass j is grouped by the window of src it reads (an XCD then reads
// a few windows, each into its own L2); in the second, each XCD reads the
// contiguous runs of every group that its eighth of the output needs.
// Each thread moves PERM_VEC consecutive entries (one 16-byte index load,
// PERM_VEC gathers in flight, one 16-byte store); the last partial vector is
// moved entry by entry.
constexpr int PERM_VEC = 4;
// 4 values at a 4-byte aligned address: one 16-byte access (the arrays need
// not be 16-byte aligned)
typedef int32_t i32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

__global__ __launch_bounds__(CSR_BLOCK) void k_permute_pass(const int32_t* idx, const float* src, float* dst,
                                                            int64_t n, int64_t per)
{
    const int64_t r = (int64_t)(blockIdx.x % CSR_XCDS) * per + blockIdx.x / CSR_XCDS;
    const int64_t j = (r * CSR_BLOCK + threadIdx.x) * PERM_VEC;
    if (j >= n) return;
    if (j + PERM_VEC <= n) {
        const i32x4_a4 i = *reinterpret_cast<const i32x4_a4*>(idx + j);
        const int32_t ii[PERM_VEC] = {i.x, i.y, i.z, i.w};
        float v[PERM_VEC];
#pragma unroll
        for (int u = 0; u < PERM_VEC; ++u) v[u] = (ii[u] >= 0 && (int64_t)ii[u] < n) ? src[ii[u]] : 0.f;
        *reinterpret_cast<f32x4_a4*>(dst + j) = f32x4_a4{v[0], v[1], v[2], v[3]};
        return;
    }
    for (int64_t k = j; k < n; ++k) {
        const int32_t i = idx[k];
        dst[k] = (i >= 0 && (int64_t)i < n) ? src[i] : 0.f;
    }
}

// keys[e] = q[e] >> wbits (the source window of output e)
__global__ void k_window_keys(const int32_t* q, int32_t* keys, int64_t n, int wbits)
{
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x)
        keys[e] = (int32_t)((uint32_t)q[e] >> wbits);
}

// inv[perm[k]] = k; indices outside [0, n) are skipped
__global__ __launch_bounds__(CSR_BLOCK) void k_invert(const int32_t* perm, int32_t* inv, int64_t n)
{
    const int64_t k = (int64_t)blockIdx.x * CSR_BLOCK + threadIdx.x;
    if (k < n) {
        const int32_t p = perm[k];
        if (p >= 0 && (int64_t)p < n) inv[p] = (int32_t)k;
    }
}

static unsigned full_grid(int64_t n) { return (unsigned)((n + CSR_BLOCK - 1) / CSR_BLOCK); }

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
    e = launch_coo_rows(row_ptr, n_rows, rows, nnz, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_gather<int32_t>, dim3(full_grid(nnz)), dim3(CSR_BLOCK), 0, s, (const int32_t*)t_perm,
                       (const int32_t*)rows, t_col_idx, nnz);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_col_starts, dim3(grid_of(n_cols + 1)), dim3(CSR_BLOCK), 0, s, (const int32_t*)keys, nnz,
                       t_row_ptr, n_cols);
    return hipGetLastError();
}

hipError_t launch_coo_rows(const int32_t* row_ptr, int64_t n_rows, int32_t* rows, int64_t nnz, hipStream_t s)
{
    if (nnz == 0 || n_rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_coo_rows, dim3(full_grid(n_rows)), dim3(CSR_BLOCK), 0, s, row_ptr, n_rows, rows, nnz);
    return hipGetLastError();
}

// workgroups of PERM_VEC * CSR_BLOCK entries per XCD
static int64_t xcd_ranges(int64_t n)
{
    const int64_t per_block = (int64_t)CSR_BLOCK * PERM_VEC;
    return ((n + per_block - 1) / per_block + CSR_XCDS - 1) / CSR_XCDS;
}

hipError_t permutation_plan_workspace(int64_t n, size_t* bytes)
{
    size_t temp = 0;
    hipError_t e = rocprim::radix_sort_pairs(nullptr, temp, (const int32_t*)nullptr, (int32_t*)nullptr,
                                             (const int32_t*)nullptr, (int32_t*)nullptr, (unsigned)n, 0, 31);
    if (e != hipSuccess) return e;
    *bytes = 4 * up256((size_t)n * 4) + up256(temp);
    return hipSuccess;
}

// Plan of dst[e] = src[q[e]] in two passes: the outputs e sorted by the
// window q[e] >> wbits of the source they read (stable: e ascending within
// a window) give order; q1[j] = q[order[j]] (pass 1 reads window after
// window) and pos[order[j]] = j (pass 2 finds output e's value at pos[e]).
hipError_t launch_permutation_plan(const int32_t* q, int64_t n, int wbits, int32_t* q1, int32_t* pos, void* ws,
                                   size_t ws_bytes, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    char* w = static_cast<char*>(ws);
    const size_t arr = up256((size_t)n * 4);
    int32_t* keys = reinterpret_cast<int32_t*>(w);
    int32_t* keys_out = reinterpret_cast<int32_t*>(w + arr);
    int32_t* iota = reinterpret_cast<int32_t*>(w + 2 * arr);
    int32_t* order = reinterpret_cast<int32_t*>(w + 3 * arr);
    void* temp = w + 4 * arr;
    size_t temp_bytes = ws_bytes - 4 * arr;
    hipLaunchKernelGGL(k_window_keys, dim3(grid_of(n)), dim3(CSR_BLOCK), 0, s, q, keys, n, wbits);
    hipLaunchKernelGGL(k_iota, dim3(grid_of(n)), dim3(CSR_BLOCK), 0, s, iota, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int bits = key_bits(((n - 1) >> wbits) + 1);
    size_t need = 0;
    e = rocprim::radix_sort_pairs(nullptr, need, (const int32_t*)nullptr, (int32_t*)nullptr, (const int32_t*)nullptr,
                                  (int32_t*)nullptr, (unsigned)n, 0, bits);
    if (e != hipSuccess) return e;
    if (need > temp_bytes) return hipErrorInvalidValue;
    e = rocprim::radix_sort_pairs(temp, temp_bytes, (const int32_t*)keys, keys_out, (const int32_t*)iota, order,
                                  (unsigned)n, 0, bits, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_gather<int32_t>, dim3(full_grid(n)), dim3(CSR_BLOCK), 0, s, (const int32_t*)order, q, q1, n);
    hipLaunchKernelGGL(k_invert, dim3(full_grid(n)), dim3(CSR_BLOCK), 0, s, (const int32_t*)order, pos, n);
    return hipGetLastError();
}

hipError_t launch_permute(const int32_t* q1, const int32_t* pos, const float* src, float* tmp, float* dst, int64_t n,
                          hipStream_t s)
{
    if (n == 0) return hipSuccess;
    const int64_t per = xcd_ranges(n);
    const unsigned grid = (unsigned)(per * CSR_XCDS);
    hipLaunchKernelGGL(k_permute_pass, dim3(grid), dim3(CSR_BLOCK), 0, s, q1, src, tmp, n, per);
    hipLaunchKernelGGL(k_permute_pass, dim3(grid), dim3(CSR_BLOCK), 0, s, pos, (const float*)tmp, dst, n, per);
    return hipGetLastError();
}

hipError_t launch_invert(const int32_t* perm, int32_t* inv, int64_t n, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_invert, dim3(full_grid(n)), dim3(CSR_BLOCK), 0, s, perm, inv, n);
    return hipGetLastError();
}

// the single pass of a permutation's kernel: 4 entries per thread, XCD-major,
// an index outside [0, n) gives 0
hipError_t launch_gather_values(const int32_t* perm, const float* src, float* dst, int64_t n, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    const int64_t per = xcd_ranges(n);
    hipLaunchKernelGGL(k_permute_pass, dim3((unsigned)(per * CSR_XCDS)), dim3(CSR_BLOCK), 0, s, perm, src, dst, n,
                       per);
    return hipGetLastError();
}

}  // namespace csrk
