// Column-part segment format: construction (the products over it run the
// plain kernels on the segment pattern; the sum of the partial rows is in
// fp32_kernels.h).
//
// The entries are stably sorted by their column part (a radix sort on
// log2(P) + 1 bits; the entries of rows kept whole take part P), which
// groups them by (part, row) with each group in its original order, since
// the CSR entries are already in row order.  A
// segment starts wherever (part, row) changes; segment indices come from an
// inclusive scan of those start flags.  Each row's segment count (integer
// atomic adds: the counts do not depend on their order) gives the row's
// slots by an exclusive scan, and a stable radix sort of the segments by row
// lists each row's segments in increasing index, i.e. part, order.  Every
// step is deterministic.
#include <algorithm>

#include <rocprim/device/device_radix_sort.hpp>
#include <rocprim/device/device_scan.hpp>

#include "common.h"
#include "launch.h"

namespace csrk {

namespace {

unsigned grid_for_n(int64_t n)
{
    int64_t b = (n + CSR_BLOCK - 1) / CSR_BLOCK;
    return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

// bits of a sort key below n (at least 1)
int key_bits(int64_t n)
{
    int b = 1;
    while (b < 31 && ((int64_t)1 << b) < n) ++b;
    return b;
}

#define CSR_GRID_STRIDE(i, n) \
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (n); i += (int64_t)gridDim.x * blockDim.x)

}  // namespace

// part of every entry: its column's part (clamped into [0, P): a column out
// of range cannot send the construction out of bounds), or P for an entry of
// a row with fewer than whole_below entries (kept whole, after all parts)
__global__ void k_entry_parts(const int32_t* col, const int32_t* row_ptr, const int32_t* coo_row, int64_t nnz,
                              int32_t part_cols, int32_t parts, int32_t whole_below, int32_t* out)
{
    CSR_GRID_STRIDE(e, nnz)
    {
        const int32_t r = coo_row[e];
        if (row_ptr[r + 1] - row_ptr[r] < whole_below) {
            out[e] = parts;
        } else {
            const int32_t p = col[e] / part_cols;
            out[e] = p < 0 ? 0 : (p >= parts ? parts - 1 : p);
        }
    }
}

__global__ void k_iota_i32(int32_t* v, int64_t n)
{
    CSR_GRID_STRIDE(i, n) v[i] = (int32_t)i;
}

__global__ void k_fill_i32(int32_t* v, int64_t n, int32_t value)
{
    CSR_GRID_STRIDE(i, n) v[i] = value;
}

// format entry k: its column and its row, both through the permutation
__global__ void k_hyb_gather(const int32_t* perm, const int32_t* col, const int32_t* coo_row, int64_t nnz,
                             int32_t* fcol, int32_t* frow)
{
    CSR_GRID_STRIDE(k, nnz)
    {
        const int32_t e = perm[k];
        fcol[k] = col[e];
        frow[k] = coo_row[e];
    }
}

// 1 where format entry k starts a segment: the first entry, or a change of part or row
__global__ void k_seg_flags(const int32_t* fpart, const int32_t* frow, int64_t nnz, int32_t* flags)
{
    CSR_GRID_STRIDE(k, nnz)
    flags[k] = (k == 0 || fpart[k] != fpart[k - 1] || frow[k] != frow[k - 1]) ? 1 : 0;
}

// segment starts and rows; each row's segment count (cnt zeroed before)
__global__ void k_seg_fill(const int32_t* flags, const int32_t* sid, const int32_t* frow, int64_t nnz,
                           int32_t* seg_ptr, int32_t* seg_row, int32_t* cnt)
{
    CSR_GRID_STRIDE(k, nnz)
    {
        if (flags[k]) {
            const int32_t s = sid[k] - 1;
            seg_ptr[s] = (int32_t)k;
            seg_row[s] = frow[k];
            atomicAdd(&cnt[frow[k]], 1);
        }
        if (k == nnz - 1) seg_ptr[sid[k]] = (int32_t)nnz;
    }
}

// Workspace regions: A (parts, then start flags, then segment indices), B
// (entry indices, then format rows, then sorted segment rows), C (sorted
// parts), D (COO rows, then segment ids), per-row counts, and the sorts' /
// scans' temporary storage.
struct HybLayout {
    size_t a, b, c, d, cnt, temp, temp_bytes, total;
};

static hipError_t hyb_layout(int64_t n_rows, int64_t nnz, int32_t parts, HybLayout* L)
{
    size_t sort_t = 0, row_sort_t = 0, iscan_t = 0, escan_t = 0;
    const unsigned n = (unsigned)(nnz > 0 ? nnz : 1);
    hipError_t e = rocprim::radix_sort_pairs(nullptr, sort_t, (const int32_t*)nullptr, (int32_t*)nullptr,
                                             (const int32_t*)nullptr, (int32_t*)nullptr, n, 0, key_bits(parts + 1));
    if (e != hipSuccess) return e;
    e = rocprim::radix_sort_pairs(nullptr, row_sort_t, (const int32_t*)nullptr, (int32_t*)nullptr,
                                  (const int32_t*)nullptr, (int32_t*)nullptr, n, 0, key_bits(n_rows));
    if (e != hipSuccess) return e;
    e = rocprim::inclusive_scan(nullptr, iscan_t, (const int32_t*)nullptr, (int32_t*)nullptr, (size_t)n,
                                rocprim::plus<int32_t>());
    if (e != hipSuccess) return e;
    e = rocprim::exclusive_scan(nullptr, escan_t, (const int32_t*)nullptr, (int32_t*)nullptr, (int32_t)0,
                                (size_t)(n_rows + 1), rocprim::plus<int32_t>());
    if (e != hipSuccess) return e;
    const size_t ent = up256((size_t)nnz * 4), rows = up256((size_t)(n_rows + 1) * 4);
    L->a = 0;
    L->b = L->a + ent;
    L->c = L->b + ent;
    L->d = L->c + ent;
    L->cnt = L->d + ent;
    L->temp = L->cnt + rows;
    L->temp_bytes = up256(std::max(std::max(sort_t, row_sort_t), std::max(iscan_t, escan_t)));
    L->total = L->temp + L->temp_bytes;
    return hipSuccess;
}

hipError_t hybrid_build_workspace(int64_t n_rows, int64_t nnz, int32_t parts, size_t* bytes)
{
    HybLayout L;
    hipError_t e = hyb_layout(n_rows, nnz, parts, &L);
    if (e == hipSuccess) *bytes = L.total;
    return e;
}

#define CSR_TRY(x)                          \
    do {                                    \
        hipError_t err_ = (x);              \
        if (err_ != hipSuccess) return err_; \
    } while (0)

hipError_t launch_hybrid_build_sort(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t nnz,
                                    int32_t parts, int32_t part_cols, int32_t whole_below, int32_t* perm,
                                    int32_t* fcol, void* ws, size_t ws_bytes, int32_t* seg_count_host, hipStream_t s)
{
    HybLayout L;
    CSR_TRY(hyb_layout(n_rows, nnz, parts, &L));
    if (ws_bytes < L.total) return hipErrorInvalidValue;
    char* w = static_cast<char*>(ws);
    int32_t* A = reinterpret_cast<int32_t*>(w + L.a);
    int32_t* B = reinterpret_cast<int32_t*>(w + L.b);
    int32_t* C = reinterpret_cast<int32_t*>(w + L.c);
    int32_t* D = reinterpret_cast<int32_t*>(w + L.d);
    void* temp = w + L.temp;
    size_t temp_bytes = L.temp_bytes;
    CSR_TRY(launch_coo_rows(row_ptr, n_rows, D, nnz, s));
    hipLaunchKernelGGL(k_entry_parts, dim3(grid_for_n(nnz)), dim3(CSR_BLOCK), 0, s, col_idx, row_ptr,
                       (const int32_t*)D, nnz, part_cols, parts, whole_below, A);
    CSR_TRY(hipGetLastError());
    hipLaunchKernelGGL(k_iota_i32, dim3(grid_for_n(nnz)), dim3(CSR_BLOCK), 0, s, B, nnz);
    CSR_TRY(hipGetLastError());
    CSR_TRY(rocprim::radix_sort_pairs(temp, temp_bytes, (const int32_t*)A, C, (const int32_t*)B, perm, (unsigned)nnz,
                                      0, key_bits(parts + 1), s));
    hipLaunchKernelGGL(k_hyb_gather, dim3(grid_for_n(nnz)), dim3(CSR_BLOCK), 0, s, (const int32_t*)perm, col_idx,
                       (const int32_t*)D, nnz, fcol, B);
    CSR_TRY(hipGetLastError());
    hipLaunchKernelGGL(k_seg_flags, dim3(grid_for_n(nnz)), dim3(CSR_BLOCK), 0, s, (const int32_t*)C,
                       (const int32_t*)B, nnz, A);
    CSR_TRY(hipGetLastError());
    temp_bytes = L.temp_bytes;
    CSR_TRY(rocprim::inclusive_scan(temp, temp_bytes, (const int32_t*)A, D, (size_t)nnz, rocprim::plus<int32_t>(),
                                    s));
    // the segment count: the last scanned flag (into pinned host memory)
    return hipMemcpyAsync(seg_count_host, D + (nnz - 1), sizeof(int32_t), hipMemcpyDeviceToHost, s);
}

hipError_t launch_hybrid_build_segments(int64_t n_rows, int64_t nnz, int32_t parts, int64_t n_seg, int32_t* seg_ptr,
                                        int32_t* seg_row, int32_t* row_seg_ptr, int32_t* row_seg, void* ws,
                                        hipStream_t s)
{
    HybLayout L;
    CSR_TRY(hyb_layout(n_rows, nnz, parts, &L));
    char* w = static_cast<char*>(ws);
    int32_t* A = reinterpret_cast<int32_t*>(w + L.a);  // start flags, then segment indices
    int32_t* B = reinterpret_cast<int32_t*>(w + L.b);  // format rows, then sorted segment rows
    const int32_t* D = reinterpret_cast<const int32_t*>(w + L.d);  // segment ids (1-based)
    int32_t* cnt = reinterpret_cast<int32_t*>(w + L.cnt);
    void* temp = w + L.temp;
    size_t temp_bytes = L.temp_bytes;
    hipLaunchKernelGGL(k_fill_i32, dim3(grid_for_n(n_rows + 1)), dim3(CSR_BLOCK), 0, s, cnt, n_rows + 1, 0);
    CSR_TRY(hipGetLastError());
    if (nnz == 0) {
        hipLaunchKernelGGL(k_fill_i32, dim3(1), dim3(CSR_BLOCK), 0, s, seg_ptr, (int64_t)1, 0);
        CSR_TRY(hipGetLastError());
    } else {
        hipLaunchKernelGGL(k_seg_fill, dim3(grid_for_n(nnz)), dim3(CSR_BLOCK), 0, s, (const int32_t*)A, D,
                           (const int32_t*)B, nnz, seg_ptr, seg_row, cnt);
        CSR_TRY(hipGetLastError());
    }
    CSR_TRY(rocprim::exclusive_scan(temp, temp_bytes, (const int32_t*)cnt, row_seg_ptr, (int32_t)0,
                                    (size_t)(n_rows + 1), rocprim::plus<int32_t>(), s));
    if (n_seg > 0) {
        // each row's segments in part order: a stable sort of the segment
        // indices by row (segments are already in (part, row) order)
        hipLaunchKernelGGL(k_iota_i32, dim3(grid_for_n(n_seg)), dim3(CSR_BLOCK), 0, s, A, n_seg);
        CSR_TRY(hipGetLastError());
        temp_bytes = L.temp_bytes;
        CSR_TRY(rocprim::radix_sort_pairs(temp, temp_bytes, (const int32_t*)seg_row, B, (const int32_t*)A, row_seg,
                                          (unsigned)n_seg, 0, key_bits(n_rows), s));
    }
    (void)parts;
    return hipSuccess;
}

}  // namespace csrk
