// Host-side runtime logic that needs no GPU: problem and schedule checks,
// lane layouts, workspace layout, default schedule, candidate list, cost
// model, input signature and the cache log format.
#include "host.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>

namespace csrh {

namespace {

bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int64_t next_pow2(int64_t v)
{
    int64_t p = 1;
    while (p < v) p <<= 1;
    return p;
}

bool nv_ok(int nv)
{
    switch (nv) {
    case 1: case 2: case 3: case 4: case 5: case 6: case 8: case 12: case 16: return true;
    default: return false;
    }
}

int nv_up(int64_t nv)
{
    static const int s[] = {1, 2, 3, 4, 5, 6, 8, 12, 16};
    for (int v : s)
        if (v >= nv) return v;
    return -1;
}

int unroll_for(int vec, int nv) { return (vec * nv <= 2) ? 8 : (vec * nv <= 16) ? 4 : 2; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// ops of the lane-group kernels (fp32 accumulation; fp32 or bf16 operands)
bool is_fp32_op(int op)
{
    return op == CSR_OP_SPMM || op == CSR_OP_SDDMM || op == CSR_OP_ATTENTION || op == CSR_OP_ATTENTION_QK ||
           op == CSR_OP_SPMM_SDDMM;
}

bool is_softmax_op(int op) { return op == CSR_OP_ATTENTION || op == CSR_OP_ATTENTION_QK || op == CSR_OP_MHA; }

void fnv(uint64_t& h, int64_t v)
{
    for (int i = 0; i < 8; ++i) {
        h ^= (uint64_t)((uint64_t)v >> (8 * i)) & 0xffu;
        h *= 0x100000001b3ull;
    }
}

}  // namespace

int max_vec_f32(const csr_problem_t& p)
{
    for (int v : {4, 2, 1}) {
        if (p.width % v) continue;
        const size_t bytes = 4u * v;
        bool ok = true;
        if (p.op == CSR_OP_SPMM || p.op == CSR_OP_ATTENTION) {
            ok = (p.ld_b % v == 0) && (p.ld_out % v == 0) && aligned(p.b, bytes) && aligned(p.out, bytes);
        } else if (p.op == CSR_OP_SDDMM) {
            ok = (p.ld_a % v == 0) && (p.ld_b % v == 0) && aligned(p.a, bytes) && aligned(p.b, bytes);
        } else if (p.op == CSR_OP_ATTENTION_QK) {
            ok = (p.ld_a % v == 0) && (p.ld_b % v == 0) && (p.ld_c % v == 0) && (p.ld_out % v == 0) &&
                 aligned(p.a, bytes) && aligned(p.b, bytes) && aligned(p.c, bytes) && aligned(p.out, bytes);
        } else if (p.op == CSR_OP_SPMM_SDDMM) {
            ok = (p.ld_b % v == 0) && (p.ld_c % v == 0) && (p.ld_out % v == 0) && aligned(p.b, bytes) &&
                 aligned(p.c, bytes) && aligned(p.out, bytes);
        }
        if (ok) return v;
    }
    return 1;
}

// bf16 operands are read 8, 4 or 2 values (16, 8 or 4 bytes) per lane
// access; the fp32 output rows of SpMM and attention are written with the
// same lane layout (8 floats as two 16-byte stores).  0: no such access fits
// (an odd width or leading dimension, or operands not 4-byte aligned).
int max_vec_bf16(const csr_problem_t& p)
{
    for (int v : {8, 4, 2}) {
        if (p.width % v) continue;
        const size_t in = 2u * v, outv = (v > 4 ? 4 : v), out = 4u * outv;
        bool ok = true;
        if (p.op == CSR_OP_SPMM || p.op == CSR_OP_ATTENTION) {
            ok = (p.ld_b % v == 0) && (p.ld_out % outv == 0) && aligned(p.b, in) && aligned(p.out, out);
        } else if (p.op == CSR_OP_SDDMM) {
            ok = (p.ld_a % v == 0) && (p.ld_b % v == 0) && aligned(p.a, in) && aligned(p.b, in);
        } else if (p.op == CSR_OP_ATTENTION_QK) {
            ok = (p.ld_a % v == 0) && (p.ld_b % v == 0) && (p.ld_c % v == 0) && (p.ld_out % outv == 0) &&
                 aligned(p.a, in) && aligned(p.b, in) && aligned(p.c, in) && aligned(p.out, out);
        }
        if (ok) return v;
    }
    return 0;
}

int max_vec(const csr_problem_t& p) { return p.dtype == CSR_DTYPE_BF16 ? max_vec_bf16(p) : max_vec_f32(p); }

bool vec_ok(const csr_problem_t& p, int v)
{
    return p.dtype == CSR_DTYPE_BF16 ? (v == 2 || v == 4 || v == 8) : (v == 1 || v == 2 || v == 4);
}

bool natural_layout(int64_t width, int vec, int* W, int* nv)
{
    if (width <= 0 || vec <= 0 || width % vec) return false;
    const int64_t L = width / vec;
    if (L <= 64) {
        *W = (int)next_pow2(L);
        *nv = 1;
        return true;
    }
    const int n = nv_up((L + 63) / 64);
    if (n < 0) return false;
    *W = 64;
    *nv = n;
    return true;
}

int check_problem(const csr_problem_t& p, bool need_ptrs, std::string* why)
{
    auto fail = [&](int code, const char* msg) {
        if (why) *why = msg;
        return code;
    };
    if (p.op < CSR_OP_SPMM || p.op > CSR_OP_SPMM_SDDMM) return fail(CSR_ERR_SHAPE, "unknown op");
    if (p.a_idx) {
        if (p.op != CSR_OP_SPMM && p.op != CSR_OP_SPMM_SDDMM) return fail(CSR_ERR_SHAPE, "a value index serves SpMM");
        if (!aligned(p.a_idx, 4)) return fail(CSR_ERR_ALIGN, "the value index must be 4-byte aligned");
        if (need_ptrs && p.nnz > 0 && !p.a) return fail(CSR_ERR_NULL, "a value index needs the values");
    }
    if (p.out2 || p.out2_idx) {
        if (p.op != CSR_OP_SPMM_SDDMM) return fail(CSR_ERR_SHAPE, "a second output serves the SpMM + SDDMM op");
        if (!aligned(p.out2, 4) || !aligned(p.out2_idx, 4))
            return fail(CSR_ERR_ALIGN, "the per-entry output and its index must be 4-byte aligned");
    }
    if (is_fp32_op(p.op) && p.dtype != CSR_DTYPE_F32 && p.dtype != CSR_DTYPE_BF16)
        return fail(CSR_ERR_DTYPE, "this op takes fp32 or bf16 operands");
    if (p.op == CSR_OP_SPMM_SDDMM && p.dtype != CSR_DTYPE_F32) return fail(CSR_ERR_DTYPE, "SpMM + SDDMM takes fp32 operands");
    if (p.op == CSR_OP_MHA && p.dtype != CSR_DTYPE_BF16) return fail(CSR_ERR_DTYPE, "multi-head attention takes bf16 Q/K/V");
    if (p.op == CSR_OP_ROW_SOFTMAX || p.op == CSR_OP_SOFTMAX_BWD) {
        const int64_t lim = (int64_t)1 << 31;
        if (p.dtype != CSR_DTYPE_F32) return fail(CSR_ERR_DTYPE, "row softmax takes fp32 scores");
        if (p.op == CSR_OP_SOFTMAX_BWD && !aligned(p.b, 4)) return fail(CSR_ERR_ALIGN, "fp32 arrays must be 4-byte aligned");
        if (need_ptrs && p.op == CSR_OP_SOFTMAX_BWD && p.nnz > 0 && !p.b)
            return fail(CSR_ERR_NULL, "grad_probs is NULL");
        if (p.n_rows < 0 || p.nnz < 0) return fail(CSR_ERR_SHAPE, "negative size");
        if (p.n_rows >= lim - 1 || p.nnz >= lim) return fail(CSR_ERR_SHAPE, "sizes must fit int32 indices");
        if (p.nnz > 0 && p.n_rows == 0) return fail(CSR_ERR_SHAPE, "entries but no rows");
        if (!std::isfinite(p.scale)) return fail(CSR_ERR_SHAPE, "scale must be finite");
        if (!aligned(p.a, 4) || !aligned(p.out, 4)) return fail(CSR_ERR_ALIGN, "fp32 arrays must be 4-byte aligned");
        if (need_ptrs) {
            if (!p.row_ptr) return fail(CSR_ERR_NULL, "row_ptr is NULL");
            if (p.nnz > 0 && (!p.a || !p.out)) return fail(CSR_ERR_NULL, "scores or probs is NULL");
        }
        return CSR_OK;
    }
    const int64_t lim = (int64_t)1 << 31;
    if (p.n_rows < 0 || p.n_cols < 0 || p.nnz < 0) return fail(CSR_ERR_SHAPE, "negative size");
    if (p.n_rows >= lim - 1 || p.n_cols >= lim || p.nnz >= lim) return fail(CSR_ERR_SHAPE, "sizes must fit int32 indices");
    if (p.nnz > 0 && p.n_cols == 0) return fail(CSR_ERR_SHAPE, "entries but no columns");
    if (p.nnz > 0 && p.n_rows == 0) return fail(CSR_ERR_SHAPE, "entries but no rows");
    if (is_fp32_op(p.op)) {
        if (p.width < 1 || p.width > 4096) return fail(CSR_ERR_SHAPE, "feature width must be in [1, 4096]");
        if (p.op == CSR_OP_ATTENTION_QK && p.width > 1024)
            return fail(CSR_ERR_SHAPE, "attention from queries and keys: head_dim must be in [1, 1024]");
        int W, nv;
        if (p.dtype == CSR_DTYPE_BF16) {
            if (p.width % 2) return fail(CSR_ERR_SHAPE, "bf16 operands need an even width");
            if (max_vec_bf16(p) == 0)
                return fail(CSR_ERR_ALIGN, "bf16 operands need even leading dimensions and 4-byte aligned rows");
        } else if (!natural_layout(p.width, 1, &W, &nv) && !natural_layout(p.width, 2, &W, &nv) &&
                   !natural_layout(p.width, 4, &W, &nv)) {
            return fail(CSR_ERR_SHAPE, "feature width not supported");
        }
        if (!natural_layout(p.width, max_vec(p), &W, &nv))
            return fail(CSR_ERR_SHAPE, "feature width too large for the operands' alignment");
        // leading dimensions below 2^30 elements: row strides in bytes fit 32 bits
        const int64_t ld_lim = (int64_t)1 << 30;
        if (p.op == CSR_OP_SDDMM) {
            if (p.ld_a < p.width || p.ld_b < p.width) return fail(CSR_ERR_SHAPE, "leading dimension < K");
            if (p.ld_a >= ld_lim || p.ld_b >= ld_lim) return fail(CSR_ERR_SHAPE, "leading dimension >= 2^30");
        } else if (p.op == CSR_OP_SPMM_SDDMM) {
            if (p.ld_b < p.width || p.ld_c < p.width || p.ld_out < p.width) return fail(CSR_ERR_SHAPE, "leading dimension < F");
            if (p.ld_b >= ld_lim || p.ld_c >= ld_lim || p.ld_out >= ld_lim)
                return fail(CSR_ERR_SHAPE, "leading dimension >= 2^30");
        } else if (p.op == CSR_OP_ATTENTION_QK) {
            if (p.ld_a < p.width || p.ld_b < p.width || p.ld_c < p.width || p.ld_out < p.width)
                return fail(CSR_ERR_SHAPE, "leading dimension < head_dim");
            if (p.ld_a >= ld_lim || p.ld_b >= ld_lim || p.ld_c >= ld_lim || p.ld_out >= ld_lim)
                return fail(CSR_ERR_SHAPE, "leading dimension >= 2^30");
        } else {
            if (p.ld_b < p.width || p.ld_out < p.width) return fail(CSR_ERR_SHAPE, "leading dimension < F");
            if (p.ld_b >= ld_lim || p.ld_out >= ld_lim) return fail(CSR_ERR_SHAPE, "leading dimension >= 2^30");
        }
        if (!aligned(p.a, 4) || !aligned(p.b, 4) || !aligned(p.c, 4) || !aligned(p.out, 4))
            return fail(CSR_ERR_ALIGN, "fp32 operands must be 4-byte aligned");
    } else {
        if (p.heads < 1) return fail(CSR_ERR_SHAPE, "heads must be >= 1");
        if (!pow2(p.head_dim) || p.head_dim < 8 || p.head_dim > 512) return fail(CSR_ERR_SHAPE, "head_dim must be a power of two in [8, 512]");
        if ((int64_t)p.heads * p.head_dim > 512) return fail(CSR_ERR_SHAPE, "heads * head_dim must be <= 512");
        if (p.width != (int64_t)p.heads * p.head_dim) return fail(CSR_ERR_SHAPE, "width must equal heads * head_dim");
        if (!aligned(p.a, 16) || !aligned(p.b, 16) || !aligned(p.c, 16) || !aligned(p.out, 16))
            return fail(CSR_ERR_ALIGN, "Q, K, V and out must be 16-byte aligned");
    }
    if (is_softmax_op(p.op) && !std::isfinite(p.scale)) return fail(CSR_ERR_SHAPE, "scale must be finite");
    if (p.probs) {
        if (!is_softmax_op(p.op)) return fail(CSR_ERR_SHAPE, "probabilities are an output of the attention ops");
        if (!aligned(p.probs, 4)) return fail(CSR_ERR_ALIGN, "probs must be 4-byte aligned");
        if (p.probs_stride < 0 || (p.op == CSR_OP_MHA && p.probs_stride > 1))
            return fail(CSR_ERR_SHAPE, "probs_stride must be >= 0 (multi-head: 0, the layout is [nnz, heads])");
    }
    if (need_ptrs) {
        if (!p.row_ptr) return fail(CSR_ERR_NULL, "row_ptr is NULL");
        if (p.nnz > 0 && !p.col_idx) return fail(CSR_ERR_NULL, "col_idx is NULL");
        if (p.op != CSR_OP_SPMM && p.op != CSR_OP_SPMM_SDDMM && p.nnz > 0 && !p.a)
            return fail(CSR_ERR_NULL, "operand a is NULL");
        if (p.nnz > 0 && !p.b) return fail(CSR_ERR_NULL, "operand b is NULL");
        if ((p.op == CSR_OP_MHA || p.op == CSR_OP_ATTENTION_QK) && p.nnz > 0 && !p.c) return fail(CSR_ERR_NULL, "V is NULL");
        if (p.op == CSR_OP_SPMM_SDDMM && p.nnz > 0 && (!p.c || !p.out2))
            return fail(CSR_ERR_NULL, "U or the per-entry output is NULL");
        if (p.op == CSR_OP_SDDMM ? (p.nnz > 0 && !p.out) : (p.n_rows > 0 && !p.out))
            return fail(CSR_ERR_NULL, "output is NULL");
    }
    return CSR_OK;
}

int check_schedule(const csr_problem_t& p, const csr_schedule_t& s, std::string* why)
{
    auto fail = [&](const char* msg) {
        if (why) *why = msg;
        return CSR_ERR_SCHEDULE;
    };
    if (s.version != CSR_SCHEDULE_VERSION) return fail("schedule version mismatch");
    if (s.op != p.op) return fail("schedule is for another op");
    if (s.mapping != CSR_MAP_ROWGROUP && s.mapping != CSR_MAP_MERGEPATH && s.mapping != CSR_MAP_SEGSCAN)
        return fail("unknown mapping");
    if (s.mapping == CSR_MAP_SEGSCAN) {
        if (p.op != CSR_OP_SPMM && p.op != CSR_OP_SDDMM && p.op != CSR_OP_ROW_SOFTMAX && p.op != CSR_OP_SOFTMAX_BWD)
            return fail("the segmented-scan mapping serves SpMM, SDDMM and the row softmax and its backward");
        if (s.group_lanes != 1 || s.passes > 4 || s.long_row != 0)
            return fail("segmented-scan schedules take group_lanes 1, passes <= 4, long_row 0");
    }
    if (s.flags & ~CSR_SCHED_WIDE) return fail("unknown schedule flags");
    for (int r : s.reserved)
        if (r != 0) return fail("reserved schedule fields must be 0");
    if (s.flags & CSR_SCHED_WIDE) {
        // 4 floats per lane at any 4-byte alignment, 64 lanes per row, the
        // last lane's vector ending at the width
        if (p.op != CSR_OP_SPMM || s.mapping != CSR_MAP_ROWGROUP || p.dtype != CSR_DTYPE_F32)
            return fail("wide lanes serve fp32 SpMM with the row-group mapping");
        if (p.width < 4) return fail("wide lanes need a width of at least 4");
        if (s.vec != 4 || s.group_lanes != 64 || s.chunk_items != 0 || s.long_row != 0)
            return fail("wide lanes take vec 4, 64 lanes per row, chunk_items = long_row = 0");
        if (s.passes != nv_up((p.width + 255) / 256))
            return fail("wide lanes take the fewest supported passes covering width / 256");
        return CSR_OK;
    }
    if (s.mapping != CSR_MAP_ROWGROUP) {
        if (s.chunk_items != 256 && s.chunk_items != 512 && s.chunk_items != 1024) return fail("chunk_items must be 256, 512 or 1024");
        if (s.long_row < 0) return fail("long_row must be >= 0");
    } else if (s.chunk_items != 0 || s.long_row != 0) {
        return fail("row-group schedules take chunk_items = long_row = 0");
    }
    if (p.op == CSR_OP_MHA) {
        if (s.vec != 8 || s.passes != 1 || s.group_lanes != p.head_dim / 8) return fail("multi-head layout must be vec 8, W = head_dim / 8, 1 pass");
        return CSR_OK;
    }
    if (p.op == CSR_OP_SOFTMAX_BWD && s.mapping != CSR_MAP_SEGSCAN)
        return fail("the softmax backward runs on lane-owned entry runs (segmented-scan mapping)");
    if (p.op == CSR_OP_ROW_SOFTMAX || p.op == CSR_OP_SOFTMAX_BWD) {
        if (s.vec != 1 || s.passes != 1) return fail("row softmax layout must be vec 1, 1 pass");
        if (s.mapping == CSR_MAP_SEGSCAN) {
            if (s.group_lanes != 1 || s.long_row != 0) return fail("entry-run row softmax takes group_lanes 1, long_row 0");
            if (s.chunk_items > 512) return fail("entry-run row softmax chunks hold at most 512 items");
            return CSR_OK;
        }
        if (s.mapping != CSR_MAP_MERGEPATH) return fail("row softmax runs on the merge-path chunks");
        if (s.chunk_items > 512) return fail("row-segment softmax chunks hold at most 512 items");
        if (!pow2(s.group_lanes) || s.group_lanes > 64) return fail("group_lanes must be a power of two <= 64");
        return CSR_OK;
    }
    if (!vec_ok(p, s.vec)) return fail(p.dtype == CSR_DTYPE_BF16 ? "bf16 vec must be 2, 4 or 8" : "vec must be 1, 2 or 4");
    if (s.vec > max_vec(p) || p.width % s.vec) return fail("vec not allowed by the operands' width or alignment");
    if (!pow2(s.group_lanes) || s.group_lanes > 64) return fail("group_lanes must be a power of two <= 64");
    if (!nv_ok(s.passes)) return fail("unsupported pass count");
    const int64_t per_pass = (int64_t)s.group_lanes * s.vec;
    if (per_pass * s.passes < p.width) return fail("layout does not cover the feature width");
    // canonical: the fewest supported passes that cover the width (a pass
    // count between supported ones may leave a trailing pass all masked)
    if (nv_up((p.width + per_pass - 1) / per_pass) != s.passes) return fail("layout has an avoidable empty pass");
    return CSR_OK;
}

int64_t n_chunks_for(const csr_problem_t& p, int items)
{
    const int64_t total = p.n_rows + p.nnz;
    const int64_t n = (total + items - 1) / items;
    return n < 1 ? 1 : n;
}

WsLayout ws_layout(const csr_problem_t& p, const csr_schedule_t& s)
{
    WsLayout w{};
    w.coords = kHeadBytes;
    w.total = kHeadBytes;
    if (s.mapping == CSR_MAP_ROWGROUP) return w;
    const int64_t nc = n_chunks_for(p, s.chunk_items);
    w.n_chunks = nc;
    w.carry_row = w.coords + up((size_t)(nc + 1) * 2 * 4);
    w.carry_ml = w.carry_row + up((size_t)nc * 2 * 4);
    size_t ml = 0, val = 0;
    if (p.op == CSR_OP_ATTENTION || p.op == CSR_OP_ATTENTION_QK) {
        ml = (size_t)nc * 2 * 2 * 4;
        val = (size_t)nc * 2 * p.width * 4;
    } else if (p.op == CSR_OP_SPMM || p.op == CSR_OP_SPMM_SDDMM) {
        val = (size_t)nc * 2 * p.width * 4;
    } else if (p.op == CSR_OP_MHA) {
        ml = (size_t)nc * 2 * p.heads * 2 * 4;
        val = (size_t)nc * 2 * p.width * 4;
    } else if (p.op == CSR_OP_ROW_SOFTMAX || p.op == CSR_OP_SOFTMAX_BWD) {
        ml = (size_t)nc * 2 * 2 * 4;
        val = (size_t)p.n_rows * 2 * 4;  // per-row statistics
    }
    w.carry_val = w.carry_ml + up(ml);
    w.total = w.carry_val + up(val);
    if ((p.op == CSR_OP_ROW_SOFTMAX || p.op == CSR_OP_SOFTMAX_BWD) && s.mapping == CSR_MAP_SEGSCAN) {
        // entry range of the row at every chunk boundary
        w.bounds = w.total;
        w.total = w.bounds + up((size_t)(nc + 1) * 2 * 4);
    }
    return w;
}

size_t workspace_bytes(const csr_problem_t& p, const csr_schedule_t& s) { return ws_layout(p, s).total; }

static csr_schedule_t blank(const csr_problem_t& p)
{
    csr_schedule_t s;
    std::memset(&s, 0, sizeof s);
    s.version = CSR_SCHEDULE_VERSION;
    s.op = p.op;
    return s;
}

csr_schedule_t default_schedule(const csr_problem_t& p)
{
    csr_schedule_t s = blank(p);
    s.mapping = CSR_MAP_MERGEPATH;
    if (p.op == CSR_OP_MHA) {
        s.vec = 8;
        s.group_lanes = p.head_dim / 8;
        s.passes = 1;
        s.chunk_items = 256;
        s.long_row = 0;
        return s;
    }
    if (p.op == CSR_OP_ROW_SOFTMAX || p.op == CSR_OP_SOFTMAX_BWD) {
        // lane-owned entry runs, one cross-lane scan per chunk
        s.mapping = CSR_MAP_SEGSCAN;
        s.vec = 1;
        s.group_lanes = 1;
        s.passes = 1;
        s.chunk_items = 256;
        s.long_row = 0;
        return s;
    }
    s.vec = max_vec(p);
    int W = 1, nv = 1;
    natural_layout(p.width, s.vec, &W, &nv);
    s.group_lanes = W;
    s.passes = nv;
    s.chunk_items = 512;
    const int G = 64 / W;
    s.long_row = (G > 1) ? G * unroll_for(s.vec, nv) : 0;
    return s;
}

std::vector<csr_schedule_t> candidates(const csr_problem_t& p, const int64_t* hist)
{
    std::vector<csr_schedule_t> out;
    const csr_schedule_t d = default_schedule(p);
    out.push_back(d);
    const int64_t max_deg = hist ? hist[66] : 0;
    auto add = [&](csr_schedule_t s) {
        if (check_schedule(p, s, nullptr) != CSR_OK) return;
        for (const auto& o : out)
            if (std::memcmp(&o, &s, sizeof s) == 0) return;
        out.push_back(s);
    };
    csr_schedule_t s = d;
    if (p.op == CSR_OP_SOFTMAX_BWD) {
        s.chunk_items = 512;
        add(s);
        return out;
    }
    if (p.op == CSR_OP_ROW_SOFTMAX) {
        s.chunk_items = 512;  // lane-owned runs twice as long
        add(s);
        // row segments by groups of W lanes (a whole wave for the long ones)
        for (int w : {1, 4, 16, 64}) {
            s = d;
            s.mapping = CSR_MAP_MERGEPATH;
            s.chunk_items = 512;
            s.group_lanes = w;
            s.long_row = (w == 64) ? 0 : (w == 1 ? 32 : 8 * w);
            add(s);
        }
        return out;
    }
    s.chunk_items = 256;
    add(s);
    s.chunk_items = 1024;
    add(s);
    // row-group: one group per row, no partition or fix-up; only when no row
    // is long enough to leave a tail or a long fp32 accumulation chain
    if (hist && max_deg <= 4096) {
        s = d;
        s.mapping = CSR_MAP_ROWGROUP;
        s.chunk_items = 0;
        s.long_row = 0;
        add(s);
        // wide lanes where the operands allow only narrower aligned accesses
        if (p.op == CSR_OP_SPMM && p.dtype == CSR_DTYPE_F32 && p.width >= 64 && (max_vec_f32(p) < 4 || p.width % 4)) {
            s.vec = 4;
            s.group_lanes = 64;
            s.passes = nv_up((p.width + 255) / 256);
            s.flags = CSR_SCHED_WIDE;
            add(s);
            s.flags = 0;
        }
    }
    if (p.op != CSR_OP_MHA) {
        // half the lanes per row, twice the passes: more rows in flight
        if (d.group_lanes >= 2 && nv_ok(d.passes * 2)) {
            s = d;
            s.group_lanes = d.group_lanes / 2;
            s.passes = d.passes * 2;
            const int G = 64 / s.group_lanes;
            s.long_row = G * unroll_for(s.vec, s.passes);
            add(s);
        }
        if (64 / d.group_lanes > 1) {
            s = d;
            s.long_row = d.long_row * 4;
            add(s);
        }
        // small widths: lanes over entries, segmented scan
        if ((p.op == CSR_OP_SPMM || p.op == CSR_OP_SDDMM) && p.width <= 4 * d.vec) {
            for (int D : {512, 256}) {
                s = d;
                s.mapping = CSR_MAP_SEGSCAN;
                s.group_lanes = 1;
                s.passes = (int)((p.width + d.vec - 1) / d.vec);
                s.chunk_items = D;
                s.long_row = 0;
                add(s);
            }
        }
    }
    return out;
}

double estimate(const csr_problem_t& p, const csr_schedule_t& s, const int64_t* hist, const DeviceInfo& dev)
{
    // Coarse ranking model: time = HBM bytes / bandwidth (lanes left idle by
    // the layout inflate the gather traffic) + a latency-bound tail for the
    // longest row when rows are not split + launch overheads.
    const double bw = 5.0e12, wave_bw = 8.0e9, launch = 4e-6;
    if (p.op == CSR_OP_ROW_SOFTMAX || p.op == CSR_OP_SOFTMAX_BWD) {
        // scores in, probabilities out; the row-segment mapping pays about
        // twice the per-chunk instruction work of the entry runs
        const double nc = (double)n_chunks_for(p, s.chunk_items);
        const double per_chunk = (s.mapping == CSR_MAP_SEGSCAN ? 0.75e-6 : 1.5e-6) * s.chunk_items / 256.0;
        const double cus = dev.cu_count > 0 ? dev.cu_count : 256.0;
        return p.nnz * 8.0 / bw + 3 * launch + nc * per_chunk / (cus * 8.0);
    }
    const double esize = (p.op == CSR_OP_MHA || p.dtype == CSR_DTYPE_BF16) ? 2.0 : 4.0;
    const double gathers = (p.op == CSR_OP_MHA || p.op == CSR_OP_ATTENTION_QK) ? 2.0 : 1.0;
    const double row_bytes = p.width * esize * gathers;
    // wide lanes: idle lanes read lines that their pass reads anyway, and
    // 16-byte accesses gather about 0.82x the time of 8-byte ones (measured)
    const bool wide = (s.flags & CSR_SCHED_WIDE) != 0;
    const double lanes_used = (p.op == CSR_OP_MHA || wide) ? 1.0
        : (double)p.width / ((double)s.group_lanes * s.vec * s.passes);
    double bytes = p.nnz * (8.0 + (wide ? 0.82 : 1.0) * row_bytes / (lanes_used > 0 ? lanes_used : 1.0)) +
                   p.n_rows * p.width * 4.0;
    if (p.op == CSR_OP_SPMM_SDDMM) bytes += p.nnz * 4.0 + p.n_rows * p.width * 4.0;  // z written, U read
    double t = bytes / bw;
    const double max_deg = hist ? (double)hist[66] : 0.0;
    if (s.mapping == CSR_MAP_ROWGROUP) {
        t += max_deg * row_bytes / wave_bw;  // one group walks the longest row alone
        t += launch;
    } else {
        const double nc = (double)n_chunks_for(p, s.chunk_items);
        const double cus = dev.cu_count > 0 ? dev.cu_count : 256.0;
        t += 3 * launch + nc * 2.0e-9 * 64.0 / cus;  // per-chunk staging and bookkeeping
        t += s.chunk_items * row_bytes / wave_bw * 0.25;  // chunk-granularity tail
    }
    return t;
}

// Expected number of non-empty segments with P column parts: a row of
// degree d whose columns are spread uniformly meets P (1 - (1 - 1/P)^d)
// parts; summed over the degree histogram at each bucket's mean degree
// (without a histogram: every row at the mean degree).
static double expected_segments(const csr_problem_t& p, const int64_t* hist, int P)
{
    const double q = 1.0 - 1.0 / P;
    if (!hist) {
        const double d = p.n_rows > 0 ? (double)p.nnz / p.n_rows : 0.0;
        return p.n_rows * P * (1.0 - std::pow(q, d));
    }
    double s = 0.0;
    for (int b = 1; b < 33; ++b) {
        if (hist[b] <= 0) continue;
        const double d = (double)hist[33 + b] / hist[b];
        s += hist[b] * P * (1.0 - std::pow(q, d));
    }
    return s;
}

// Time (ms) per GB of gathered rows when they come from a slice of s bytes
// of the dense operand, measured on MI355X (the power-law graph's SpMM at
// F = 602 over the format at 4 to 256 parts, less the partial rows' share):
// 0.070 while a slice fits one XCD's L2 (4 MiB), rising with log2 of the
// slice through 0.089 (8 MiB), 0.111 (16 MiB), 0.124 (32 MiB) and 0.131
// (64 MiB) to the rate of gathers spread over an operand far beyond the
// caches, 0.137, from 256 MiB on.
static double gather_ms_per_gb(double s)
{
    static const double pts[6][2] = {{4, 0.070}, {8, 0.0894}, {16, 0.1113}, {32, 0.1235}, {64, 0.1313}, {256, 0.137}};
    const double mib = s / (1 << 20);
    if (mib <= pts[0][0]) return pts[0][1];
    for (int i = 0; i < 5; ++i) {
        if (mib <= pts[i + 1][0]) {
            const double x = std::log2(mib / pts[i][0]) / std::log2(pts[i + 1][0] / pts[i][0]);  // 0 .. 1
            return pts[i][1] + (pts[i + 1][1] - pts[i][1]) * x;
        }
    }
    return pts[5][1];
}

// Plan of the column-part segment format (parts 1: the plain CSR path).
// SpMM: a cost model, time(P, T) = gathered GB of the split rows x
// gather_ms_per_gb(slice of n_cols x width x 4 / P bytes) + gathered GB of
// the rows kept whole (fewer than T entries) x gather_ms_per_gb(the whole
// operand) + the partial rows (written and read: width x 8 bytes per
// segment; a whole row is one segment) at 0.118 ms per GB, all measured; a
// gather moves at least one 64-byte sector; the split rows' segments are
// expected from the degree histogram.  P from 4 to 256 with slices of at
// least 2 MiB and T a power of two (or 0) are scored, and the best is used
// when it is estimated at least 5 % faster than the plain path.  SDDMM (no
// partial rows; rows of at most 16 floats, where the per-entry output
// scatter does not cancel the gain): the power of two nearest to (gathered
// bytes / 4 MiB), from 4 to 256, when the expected segments stay under an
// eighth of the entries, every row split.
void hybrid_plan(const csr_problem_t& p, const int64_t* hist, int* parts, int* whole_below)
{
    *parts = 1;
    *whole_below = 0;
    if (p.op != CSR_OP_SPMM && p.op != CSR_OP_SDDMM) return;
    if (p.nnz <= 0 || p.n_cols <= 0 || p.n_rows <= 0) return;
    const double mib = 1 << 20;
    const double row = p.width * (p.dtype == CSR_DTYPE_BF16 ? 2.0 : 4.0);
    const double X = p.n_cols * row;
    if (p.op == CSR_OP_SDDMM) {
        if (p.width > 16) return;
        const double slices = X / (4.0 * mib);
        if (slices < 2.83) return;  // nearest power of two below 4
        int P = 4;
        while (P < 256 && (double)P * 1.41421356 < slices) P *= 2;
        if (2.0 * expected_segments(p, hist, P) <= 0.25 * p.nnz) *parts = P;
        return;
    }
    const double gather_bytes = std::max(row, 64.0) / 1e9;  // GB per gathered row
    const double part_bytes = p.width * 8.0 / 1e9;          // GB per partial row, written and read
    const double plain = p.nnz * gather_bytes * gather_ms_per_gb(X);
    double best = plain;
    // whole-row thresholds T = 2^k: buckets 1 .. k of the histogram (degrees below 2^k) stay whole
    const int kmax = hist ? 12 : 0;
    for (int P = 4; P <= 256 && X / P >= 2.0 * mib; P *= 2) {
        const double q = 1.0 - 1.0 / P;
        for (int k = 0; k <= kmax; ++k) {
            double split_nnz = (double)p.nnz, split_seg = 0.0, whole_rows = 0.0, whole_nnz = 0.0;
            if (hist) {
                split_nnz = 0.0;
                for (int b = 1; b < 33; ++b) {
                    if (hist[b] <= 0) continue;
                    if (b <= k) {
                        whole_rows += hist[b];
                        whole_nnz += hist[33 + b];
                    } else {
                        const double d = (double)hist[33 + b] / hist[b];
                        split_nnz += hist[33 + b];
                        split_seg += hist[b] * P * (1.0 - std::pow(q, d));
                    }
                }
            } else {
                split_seg = expected_segments(p, nullptr, P);
            }
            const double t = split_nnz * gather_bytes * gather_ms_per_gb(X / P) +
                             whole_nnz * gather_bytes * gather_ms_per_gb(X) +
                             0.118 * (split_seg + whole_rows) * part_bytes;
            if (t < best) {
                best = t;
                *parts = P;
                *whole_below = k > 0 ? (1 << k) : 0;
            }
        }
    }
    if (!(best < 0.95 * plain)) {
        *parts = 1;
        *whole_below = 0;
    }
}

int hybrid_parts(const csr_problem_t& p, const int64_t* hist)
{
    int P = 1, T = 0;
    hybrid_plan(p, hist, &P, &T);
    return P;
}

std::vector<size_t> probe_subset(const std::vector<csr_schedule_t>& cand, const std::vector<double>& est, int k)
{
    std::vector<size_t> order(cand.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](size_t x, size_t y) { return est[x] < est[y]; });
    std::vector<size_t> pick;
    std::vector<char> taken(cand.size(), 0);
    for (size_t i : order) {  // the best of each mapping
        if ((int)pick.size() >= k) break;
        bool seen = false;
        for (size_t j : pick) seen = seen || (cand[j].mapping == cand[i].mapping && cand[j].flags == cand[i].flags);
        if (!seen) {
            pick.push_back(i);
            taken[i] = 1;
        }
    }
    for (size_t i : order) {  // then by estimate
        if ((int)pick.size() >= k) break;
        if (!taken[i]) {
            pick.push_back(i);
            taken[i] = 1;
        }
    }
    std::sort(pick.begin(), pick.end());
    return pick;
}

uint64_t signature(const csr_problem_t& p, const int64_t* hist, const DeviceInfo& dev)
{
    uint64_t h = 0xcbf29ce484222325ull;
    fnv(h, 0x43535253);  // 'CSRS'
    fnv(h, kLibVersion);
    fnv(h, p.op);
    fnv(h, p.dtype);
    fnv(h, p.n_rows);
    fnv(h, p.n_cols);
    fnv(h, p.nnz);
    fnv(h, p.width);
    fnv(h, p.op == CSR_OP_MHA ? p.heads : 0);
    fnv(h, p.op == CSR_OP_MHA ? p.head_dim : 0);
    fnv(h, p.op == CSR_OP_MHA ? 8 : (is_fp32_op(p.op) ? max_vec(p) : max_vec_f32(p)));
    fnv(h, dev.cu_count);
    fnv(h, dev.arch);
    for (int i = 0; i < kHistInts; ++i) fnv(h, hist ? hist[i] : 0);
    if (p.a_idx) fnv(h, 0x58444956);  // 'VIDX': values read through an index
    if (p.out2_idx) fnv(h, 0x5844495a);  // 'ZIDX': the per-entry output written through an index
    return h;
}

uint64_t plan_signature(const csr_problem_t& p, const int64_t* hist, const DeviceInfo& dev)
{
    uint64_t h = signature(p, hist, dev);
    fnv(h, 0x4e414c50);  // 'PLAN'
    return h;
}

int64_t segment_bound(const csr_problem_t& p, const int64_t* hist, int P, int T)
{
    if (!hist) return std::min(p.nnz, p.n_rows * (int64_t)P);
    int64_t n = 0;
    for (int b = 1; b < 33; ++b) {
        if (hist[b] <= 0) continue;
        const int64_t lo = (int64_t)1 << (b - 1), hi = (int64_t)1 << b;  // degrees in [lo, hi)
        if (hi <= T)
            n += hist[b];  // every row of the bucket is kept whole
        else
            n += std::min(hist[33 + b], hist[b] * (int64_t)P);
        (void)lo;
    }
    return std::max<int64_t>(0, std::min(n, p.nnz));
}

std::vector<std::pair<int, int>> plan_formats(const csr_problem_t& p, const int64_t* hist)
{
    std::vector<std::pair<int, int>> out;
    if ((p.op != CSR_OP_SPMM && p.op != CSR_OP_SDDMM) || p.nnz <= 0 || p.n_rows <= 0 || p.n_cols <= 0) return out;
    auto add = [&](int P, int T) {
        if (P < 2 || P > 256) return;
        for (const auto& f : out)
            if (f.first == P && f.second == T) return;
        out.push_back({P, T});
    };
    int P = 1, T = 0;
    hybrid_plan(p, hist, &P, &T);
    if (P > 1) {
        add(P, T);
        add(P / 2, T);
        add(P * 2, T);
        if (T > 0) add(P, 0);
    } else {
        const double X = (double)p.n_cols * p.width * (p.dtype == CSR_DTYPE_BF16 ? 2.0 : 4.0);
        if (X / 4 >= 2.0 * (1 << 20)) add(4, 0);
        if (X / 16 >= 2.0 * (1 << 20)) add(16, 0);
    }
    return out;
}

BucketShape bucket_shape(const csr_problem_t& p, const int64_t* hist, int E)
{
    BucketShape b;
    b.E = E;
    int n = 0;
    while ((1 << n) < E && n < CSR_BUCKET_MAX_CLASSES) ++n;
    b.n_classes = n;
    int64_t slots = 0, rows = 0;
    for (int c = 1; c <= n; ++c) {
        const int64_t cnt = hist ? hist[c] : 0;
        b.class_rows[c - 1] = cnt;
        b.class_base[c - 1] = slots;
        b.class_row0[c - 1] = rows;
        slots += cnt * (((int64_t)1 << c) - 1);
        rows += cnt;
        b.nnz_short += hist ? hist[33 + c] : 0;
    }
    b.n_short = rows;
    b.n_slots = slots;
    b.nnz_long = std::max<int64_t>(0, p.nnz - b.nnz_short);
    return b;
}

BucketLayout bucket_layout(const csr_problem_t& p, const BucketShape& b)
{
    auto up = [](size_t v) { return (v + kAlign - 1) / kAlign * kAlign; };
    BucketLayout L{};
    L.rows = 0;
    L.slot_col = L.rows + up((size_t)p.n_rows * 4);
    L.slot_pos = L.slot_col + up((size_t)b.n_slots * 4);
    L.slot_val = L.slot_pos + up((size_t)b.n_slots * 4);
    L.long_row_ptr = L.slot_val + up((size_t)b.n_slots * 4);
    L.long_col = L.long_row_ptr + up((size_t)(p.n_rows + 1) * 4);
    L.long_pos = L.long_col + up((size_t)b.nnz_long * 4);
    L.long_val = L.long_pos + up((size_t)b.nnz_long * 4);
    L.total = L.long_val + up((size_t)b.nnz_long * 4);
    return L;
}

std::vector<int> plan_buckets(const csr_problem_t& p, const int64_t* hist)
{
    std::vector<int> out;
    if (p.op != CSR_OP_SPMM || !hist || p.n_rows <= 0 || p.nnz <= 0 || p.n_cols <= 0) return out;
    for (int E : {8, 32}) {
        const BucketShape b = bucket_shape(p, hist, E);
        if (b.n_short * 4 >= p.n_rows && b.nnz_short * 10 >= p.nnz && b.n_slots - b.nnz_short <= b.nnz_short)
            out.push_back(E);
    }
    return out;
}

std::string format_plan_line(uint64_t sig, const PlanChoice& c, double probe_us)
{
    char buf[288];
    const csr_schedule_t& s = c.sched;
    std::snprintf(buf, sizeof buf,
                  "csrsa-plan v%d %016llx parts=%d whole=%d op=%d map=%d vec=%d w=%d nv=%d chunk=%d long=%d "
                  "flags=%d us=%.3f\n",
                  CSR_SCHEDULE_VERSION, (unsigned long long)sig, c.parts, c.whole_below, s.op, s.mapping, s.vec,
                  s.group_lanes, s.passes, s.chunk_items, s.long_row, s.flags, probe_us);
    return buf;
}

bool parse_plan_line(const std::string& line, uint64_t* sig, PlanChoice* c, double* probe_us)
{
    int ver = 0, n = 0;
    unsigned long long sg = 0;
    PlanChoice t;
    std::memset(&t.sched, 0, sizeof t.sched);
    double us = 0;
    csr_schedule_t& s = t.sched;
    const int got = std::sscanf(line.c_str(),
                                "csrsa-plan v%d %16llx parts=%d whole=%d op=%d map=%d vec=%d w=%d nv=%d chunk=%d "
                                "long=%d flags=%d us=%lf%n",
                                &ver, &sg, &t.parts, &t.whole_below, &s.op, &s.mapping, &s.vec, &s.group_lanes,
                                &s.passes, &s.chunk_items, &s.long_row, &s.flags, &us, &n);
    if (got != 13 || ver != CSR_SCHEDULE_VERSION) return false;
    for (size_t i = (size_t)n; i < line.size(); ++i)
        if (line[i] != '\n' && line[i] != '\r' && line[i] != ' ') return false;
    if (s.op != CSR_OP_SPMM && s.op != CSR_OP_SDDMM) return false;
    if (t.parts == 0) {  // degree classes: whole_below is the short threshold (SpMM)
        const int E = t.whole_below;
        if (s.op != CSR_OP_SPMM || E < 2 || E > (1 << CSR_BUCKET_MAX_CLASSES) || (E & (E - 1))) return false;
    } else if (t.parts < 1 || t.parts > 256 || (t.parts & (t.parts - 1)) || t.whole_below < 0) {
        return false;
    }
    if (s.mapping != CSR_MAP_ROWGROUP && s.mapping != CSR_MAP_MERGEPATH && s.mapping != CSR_MAP_SEGSCAN) return false;
    s.version = CSR_SCHEDULE_VERSION;
    *sig = sg;
    *c = t;
    if (probe_us) *probe_us = us;
    return true;
}

std::string format_cache_line(uint64_t sig, const csr_schedule_t& s, double probe_us)
{
    char buf[256];
    std::snprintf(buf, sizeof buf,
                  "csrsa-cache v%d %016llx op=%d map=%d vec=%d w=%d nv=%d chunk=%d long=%d flags=%d us=%.3f\n",
                  CSR_SCHEDULE_VERSION, (unsigned long long)sig, s.op, s.mapping, s.vec, s.group_lanes, s.passes,
                  s.chunk_items, s.long_row, s.flags, probe_us);
    return buf;
}

bool parse_cache_line(const std::string& line, uint64_t* sig, csr_schedule_t* s, double* probe_us)
{
    int ver = 0, n = 0;
    unsigned long long sg = 0;
    csr_schedule_t t;
    std::memset(&t, 0, sizeof t);
    double us = 0;
    const int got = std::sscanf(line.c_str(),
                                "csrsa-cache v%d %16llx op=%d map=%d vec=%d w=%d nv=%d chunk=%d long=%d flags=%d us=%lf%n",
                                &ver, &sg, &t.op, &t.mapping, &t.vec, &t.group_lanes, &t.passes, &t.chunk_items,
                                &t.long_row, &t.flags, &us, &n);
    if (got != 11 || ver != CSR_SCHEDULE_VERSION) return false;
    for (size_t i = (size_t)n; i < line.size(); ++i)
        if (line[i] != '\n' && line[i] != '\r' && line[i] != ' ') return false;
    if (t.op < CSR_OP_SPMM || t.op > CSR_OP_SPMM_SDDMM) return false;
    if (t.mapping != CSR_MAP_ROWGROUP && t.mapping != CSR_MAP_MERGEPATH && t.mapping != CSR_MAP_SEGSCAN) return false;
    t.version = CSR_SCHEDULE_VERSION;
    *sig = sg;
    *s = t;
    if (probe_us) *probe_us = us;
    return true;
}

}  // namespace csrh
