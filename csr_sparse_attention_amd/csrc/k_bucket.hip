// Degree classes: the short rows of a CSR pattern packed by degree class,
// slot-major (SparseTIR page, Abstract: composable formats, rows bucketed by
// degree), their SpMM, and the construction.
//
// Construction, every step deterministic: each row gets its class key (the
// bit width of its degree minus one for 1 <= degree < E, else the class
// count); a stable radix sort of the row indices by key lists the packed
// rows class by class, each class in row order; one thread per packed row
// writes its slots.  The other rows' entries (rows of E or more entries;
// empty rows take none) are copied into a CSR of their own on the same row
// numbering, positioned by an exclusive scan of their degrees.
#include <algorithm>

#include <rocprim/device/device_radix_sort.hpp>
#include <rocprim/device/device_scan.hpp>

#include "fp32_kernels.h"
#include "launch.h"

namespace csrk {

namespace {

unsigned grid_n(int64_t n)
{
    int64_t b = (n + CSR_BLOCK - 1) / CSR_BLOCK;
    return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

#define CSR_GRID_LOOP(i, n) \
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (n); i += (int64_t)gridDim.x * blockDim.x)

#define CSR_TRY(x)                           \
    do {                                     \
        hipError_t err_ = (x);               \
        if (err_ != hipSuccess) return err_; \
    } while (0)

struct ClassTable {
    int64_t rows[6], base[6], row0[6];
};

// class of a row of degree d: c for 2^c <= d < 2^(c+1) when 1 <= d < E, else n_classes
__global__ void k_bucket_keys(const int32_t* row_ptr, int64_t n_rows, int32_t E, int32_t n_classes, int32_t* keys,
                              int32_t* idx)
{
    CSR_GRID_LOOP(r, n_rows)
    {
        const int32_t d = row_ptr[r + 1] - row_ptr[r];
        keys[r] = (d >= 1 && d < E) ? 31 - __clz(d) : n_classes;
        idx[r] = (int32_t)r;
    }
}

__global__ void k_bucket_slots(const int32_t* rows, const int32_t* row_ptr, const int32_t* col_idx, int64_t n_short,
                               int32_t n_classes, ClassTable t, int32_t* slot_col, int32_t* slot_pos)
{
    CSR_GRID_LOOP(p, n_short)
    {
        int c = 0;
        while (c + 1 < n_classes && p >= t.row0[c + 1]) ++c;
        const int64_t i = p - t.row0[c], n = t.rows[c];
        const int w = (2 << c) - 1;
        const int32_t r = rows[p];
        const int32_t b = row_ptr[r];
        const int32_t d = row_ptr[r + 1] - b;
        for (int j = 0; j < w; ++j) {
            const int64_t s = t.base[c] + (int64_t)j * n + i;
            slot_col[s] = j < d ? col_idx[b + j] : -1;
            slot_pos[s] = j < d ? b + j : -1;
        }
    }
}

// degree of each row in the long rows' CSR (0 for packed rows), and a 0 at n_rows
__global__ void k_bucket_long_deg(const int32_t* row_ptr, int64_t n_rows, int32_t E, int32_t* deg)
{
    CSR_GRID_LOOP(r, n_rows + 1)
    {
        const int32_t d = r < n_rows ? row_ptr[r + 1] - row_ptr[r] : 0;
        deg[r] = d >= E ? d : 0;
    }
}

__global__ void k_bucket_long_fill(const int32_t* row_ptr, const int32_t* col_idx, const int32_t* coo, int64_t nnz,
                                   int32_t E, const int32_t* long_row_ptr, int32_t* long_col, int32_t* long_pos)
{
    CSR_GRID_LOOP(e, nnz)
    {
        const int32_t r = coo[e];
        const int32_t b = row_ptr[r];
        if (row_ptr[r + 1] - b >= E) {
            const int64_t k = long_row_ptr[r] + (e - b);
            long_col[k] = col_idx[e];
            long_pos[k] = (int32_t)e;
        }
    }
}

__global__ void k_gather_or_zero(const int32_t* pos, const float* src, float* dst, int64_t n)
{
    CSR_GRID_LOOP(k, n)
    {
        const int32_t q = pos[k];
        dst[k] = q >= 0 ? (src ? src[q] : 1.f) : 0.f;
    }
}

struct BuildLayout {
    size_t keys, idx, keys_out, deg, coo, temp, temp_bytes, total;
};

hipError_t build_layout(int64_t n_rows, int64_t nnz, BuildLayout* L)
{
    size_t sort_bytes = 0, scan_bytes = 0;
    CSR_TRY(rocprim::radix_sort_pairs(nullptr, sort_bytes, (const int32_t*)nullptr, (int32_t*)nullptr,
                                      (const int32_t*)nullptr, (int32_t*)nullptr, (unsigned)(n_rows > 0 ? n_rows : 1),
                                      0, 4));
    CSR_TRY(rocprim::exclusive_scan(nullptr, scan_bytes, (const int32_t*)nullptr, (int32_t*)nullptr, (int32_t)0,
                                    (size_t)(n_rows + 1), rocprim::plus<int32_t>()));
    L->keys = 0;
    L->idx = L->keys + up256((size_t)n_rows * 4);
    L->keys_out = L->idx + up256((size_t)n_rows * 4);
    L->deg = L->keys_out + up256((size_t)n_rows * 4);
    L->coo = L->deg + up256((size_t)(n_rows + 1) * 4);
    L->temp = L->coo + up256((size_t)nnz * 4);
    L->temp_bytes = std::max(sort_bytes, scan_bytes);
    L->total = L->temp + up256(L->temp_bytes);
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// SpMM of the packed rows: a group of W lanes per row (lanes over features as
// in the lane-group kernels), slots read U at a time; a row's padding
// follows its entries, so the walk ends at the first padding slot of the
// batch's last entry.  Padding is never multiplied (an infinite feature
// times 0 would give NaN).
// ---------------------------------------------------------------------------
template <typename T, int VEC, int NV, int U>
__global__ __launch_bounds__(CSR_BLOCK) void k_bucket_spmm(BucketArgs a)
{
    const int64_t blk = blockIdx.x;
    int c = 0;
    while (c + 1 < a.n_classes && blk >= a.cls_block0[c + 1]) ++c;
    const int64_t n = a.cls_rows[c];
    const int w = (2 << c) - 1;
    Lanes<VEC, NV> L(a.W);
    const int64_t i = ((blk - a.cls_block0[c]) * CSR_BLOCK + threadIdx.x) / a.W;
    if (i >= n) return;  // whole groups
    const int32_t* col = a.slot_col + a.cls_base[c] + i;
    const float* val = a.slot_val + a.cls_base[c] + i;
    const T* X = static_cast<const T*>(a.X);
    constexpr uint32_t ES = sizeof(T);
    uint32_t off[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) off[j] = L.valid(j, a.F) ? (uint32_t)L.off(j) * ES : 0u;
    const uint32_t row_bytes = (uint32_t)a.ldx * ES;
    const char* xb = reinterpret_cast<const char*>(X);
    float acc[NV][VEC];
    zero(acc);
    for (int j0 = 0; j0 < w; j0 += U) {
        int cu[U];
        float wu[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u;
            cu[u] = j < w ? col[(int64_t)j * n] : -1;
            wu[u] = j < w ? val[(int64_t)j * n] : 0.f;
        }
        float xv[U][NV][VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (cu[u] >= 0) {
                const char* xr = row_at(xb, cu[u], row_bytes);
#pragma unroll
                for (int j = 0; j < NV; ++j) vload_t<T, VEC>(xv[u][j], reinterpret_cast<const T*>(xr + off[j]));
            } else {
                zero(xv[u]);
                wu[u] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < NV; ++j)
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[j][v] = fmaf(wu[u], xv[u][j][v], acc[j][v]);
        if (cu[U - 1] < 0) break;  // this row's padding reached
    }
    store_row<VEC, NV>(a.Y + (int64_t)a.rows[a.cls_row0[c] + i] * a.ldy, acc, L, a.F, 1.f);
}

template <typename T, int VEC, int NV>
hipError_t run_bucket(const BucketArgs& a, hipStream_t s)
{
    const int64_t blocks = a.cls_block0[a.n_classes];
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    constexpr int U = unroll_for(VEC, NV);
    hipLaunchKernelGGL((k_bucket_spmm<T, VEC, NV, U>), dim3((unsigned)blocks), dim3(CSR_BLOCK), 0, s, a);
    return hipGetLastError();
}

}  // namespace

#define CSR_BK_NV(MACRO, VEC) \
    MACRO(VEC, 1) MACRO(VEC, 2) MACRO(VEC, 3) MACRO(VEC, 4) MACRO(VEC, 5) MACRO(VEC, 6) \
    MACRO(VEC, 8) MACRO(VEC, 12) MACRO(VEC, 16)

hipError_t launch_bucket_spmm(int dtype_bf16, int vec, int nv, const BucketArgs& a, hipStream_t s)
{
    if (a.n_classes < 1 || a.n_classes > 6) return hipErrorInvalidValue;
#define CSR_CASE(V, N) \
    if (vec == V && nv == N) return run_bucket<T, V, N>(a, s);
    if (!dtype_bf16) {
        using T = float;
        CSR_BK_NV(CSR_CASE, 1)
        CSR_BK_NV(CSR_CASE, 2)
        CSR_BK_NV(CSR_CASE, 4)
    } else {
        using T = bf16_t;
        CSR_BK_NV(CSR_CASE, 2)
        CSR_BK_NV(CSR_CASE, 4)
        CSR_BK_NV(CSR_CASE, 8)
    }
#undef CSR_CASE
    return hipErrorInvalidValue;
}

hipError_t bucket_build_workspace(int64_t n_rows, int64_t nnz, size_t* bytes)
{
    BuildLayout L;
    CSR_TRY(build_layout(n_rows, nnz, &L));
    *bytes = L.total;
    return hipSuccess;
}

hipError_t launch_bucket_build(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t nnz, int E,
                               int n_classes, const int64_t* cls_rows, const int64_t* cls_base,
                               const int64_t* cls_row0, int32_t* rows, int32_t* slot_col, int32_t* slot_pos,
                               int32_t* long_row_ptr, int32_t* long_col, int32_t* long_pos, void* ws,
                               size_t ws_bytes, hipStream_t s)
{
    if (n_classes < 1 || n_classes > 6 || n_rows < 0 || nnz < 0) return hipErrorInvalidValue;
    BuildLayout L;
    CSR_TRY(build_layout(n_rows, nnz, &L));
    if (ws_bytes < L.total) return hipErrorInvalidValue;
    char* w = static_cast<char*>(ws);
    int32_t* keys = reinterpret_cast<int32_t*>(w + L.keys);
    int32_t* idx = reinterpret_cast<int32_t*>(w + L.idx);
    int32_t* keys_out = reinterpret_cast<int32_t*>(w + L.keys_out);
    int32_t* deg = reinterpret_cast<int32_t*>(w + L.deg);
    int32_t* coo = reinterpret_cast<int32_t*>(w + L.coo);
    void* temp = w + L.temp;
    ClassTable t;
    int64_t n_short = 0;
    for (int c = 0; c < 6; ++c) {
        t.rows[c] = c < n_classes ? cls_rows[c] : 0;
        t.base[c] = c < n_classes ? cls_base[c] : 0;
        t.row0[c] = c < n_classes ? cls_row0[c] : 0;
        if (c < n_classes) n_short += cls_rows[c];
    }
    if (n_rows > 0) {
        hipLaunchKernelGGL(k_bucket_keys, dim3(grid_n(n_rows)), dim3(CSR_BLOCK), 0, s, row_ptr, n_rows, (int32_t)E,
                           (int32_t)n_classes, keys, idx);
        CSR_TRY(hipGetLastError());
        size_t tb = L.temp_bytes;
        int bits = 1;
        while ((1 << bits) <= n_classes) ++bits;
        CSR_TRY(rocprim::radix_sort_pairs(temp, tb, (const int32_t*)keys, keys_out, (const int32_t*)idx, rows,
                                          (unsigned)n_rows, 0, bits, s));
        if (n_short > 0) {
            hipLaunchKernelGGL(k_bucket_slots, dim3(grid_n(n_short)), dim3(CSR_BLOCK), 0, s, (const int32_t*)rows,
                               row_ptr, col_idx, n_short, (int32_t)n_classes, t, slot_col, slot_pos);
            CSR_TRY(hipGetLastError());
        }
    }
    hipLaunchKernelGGL(k_bucket_long_deg, dim3(grid_n(n_rows + 1)), dim3(CSR_BLOCK), 0, s, row_ptr, n_rows,
                       (int32_t)E, deg);
    CSR_TRY(hipGetLastError());
    size_t tb = L.temp_bytes;
    CSR_TRY(rocprim::exclusive_scan(temp, tb, (const int32_t*)deg, long_row_ptr, (int32_t)0, (size_t)(n_rows + 1),
                                    rocprim::plus<int32_t>(), s));
    if (nnz > 0 && n_rows > 0) {
        CSR_TRY(launch_coo_rows(row_ptr, n_rows, coo, nnz, s));
        hipLaunchKernelGGL(k_bucket_long_fill, dim3(grid_n(nnz)), dim3(CSR_BLOCK), 0, s, row_ptr, col_idx,
                           (const int32_t*)coo, nnz, (int32_t)E, (const int32_t*)long_row_ptr, long_col, long_pos);
        CSR_TRY(hipGetLastError());
    }
    return hipSuccess;
}

hipError_t launch_gather_or_zero(const int32_t* pos, const float* src, float* dst, int64_t n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_gather_or_zero, dim3(grid_n(n)), dim3(CSR_BLOCK), 0, s, pos, src, dst, n);
    return hipGetLastError();
}

}  // namespace csrk
