// Templated fp32 kernels: SpMM, scores-given softmax attention and SDDMM, in
// the row-group mapping and the merge-path mapping.
//
// Lane layout (both mappings).  A wavefront of 64 lanes is cut into G = 64/W
// groups of W lanes.  Within a group, lane lg covers the features
// (j * W + lg) * VEC .. + VEC - 1 for passes j < NV, so a row of F features is
// read with W * NV vector loads of VEC floats each.  W, VEC and NV are chosen
// on the host from F and the alignment of the operands.
//
// Row-group mapping: group k of the grid owns row k and walks its entries.
//
// Merge-path mapping: the rows and entries are merged into one sequence (the
// end of a row follows the row's last entry) and cut into chunks of D items,
// one chunk per wavefront, so every wavefront gets the same amount of work
// whatever the degree skew.  A wave stages its chunk's row_ptr, col_idx and
// per-entry values in LDS, then
//   pass 1: every row segment with at least `long_row` entries is processed
//           by the whole wave, the G groups taking interleaved entries, and
//           reduced across the groups;
//   pass 2: the remaining short rows are dealt round-robin to the groups.
// Rows whose entries are cut by a chunk boundary leave pieces in a carry
// buffer (slot A: the end of a row that began in an earlier chunk, slot B:
// the beginning or middle of a row that continues into the next chunk), and a
// fix-up kernel combines each such row's pieces in chunk order.  No atomics:
// results are bitwise reproducible for a given schedule.
#pragma once

#include "args.h"
#include "common.h"

namespace csrk {

// AttnQK: attention from queries and keys, SDDMM -> row-softmax -> SpMM in one
// pass (U = Q, X = K, V = values): each score is formed on the fly and folded
// into an online softmax.  Dual: an SpMM and an SDDMM on one pattern that
// share the gathered operand X (Y = A X and z_e = <U[row_e], X[col_e]>), each
// gathered row read once for both.
enum class Op { Spmm, Attention, Sddmm, AttnQK, Dual };


template <int VEC, int NV>
struct Lanes {
    int W, lg, g, G;
    __device__ __forceinline__ Lanes(int w) : W(w)
    {
        int lane = lane_id();
        lg = lane & (w - 1);
        g = lane / w;
        G = CSR_WAVE / w;
    }
    __device__ __forceinline__ int off(int j) const { return (j * W + lg) * VEC; }
    __device__ __forceinline__ bool valid(int j, int F) const { return off(j) < F; }
};

template <int VEC, int NV>
__device__ __forceinline__ void zero(float (&a)[NV][VEC])
{
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int v = 0; v < VEC; ++v) a[j][v] = 0.f;
}

// Edge weight: SpMM value (1 if absent) or unnormalised softmax weight.
template <Op OP>
__device__ __forceinline__ float edge_weight(const float* ev, int e, float scale, float m,
                                             const int32_t* ev_idx = nullptr)
{
    if constexpr (OP == Op::Spmm) {
        return ev ? ev[ev_idx ? ev_idx[e] : e] : 1.f;
    } else {
        return exp_neg(ev[e] * scale - m);
    }
}

// Row addresses: leading dimensions are below 2^30 elements, so a row's byte
// offset is one 32 x 32 -> 64-bit multiply-add of the column index.
__device__ __forceinline__ const char* row_at(const char* base, int32_t row, uint32_t row_bytes)
{
    return base + (uint64_t)(uint32_t)row * row_bytes;
}

// acc += sum over entries e = kb, kb + step, ... < ke of w_e * X[col[e], lane features].
// col / ev are indexed directly by e (they may point into LDS or global memory).
// Batches of U entries run without per-entry tests; only the last, partial
// batch is masked.  Lanes past the width read the row's first features (in
// bounds) and accumulate values that are never stored.
template <Op OP, typename T, int VEC, int NV, int U>
__device__ __forceinline__ void gather_acc(float (&acc)[NV][VEC], const int32_t* col, const float* ev,
                                           int kb, int ke, int step, const T* X, int64_t ldx,
                                           const Lanes<VEC, NV>& L, int F, float scale, float m,
                                           const int32_t* ev_idx = nullptr)
{
    constexpr uint32_t ES = sizeof(T);
    uint32_t off[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) off[j] = L.valid(j, F) ? (uint32_t)L.off(j) * ES : 0u;
    const uint32_t row_bytes = (uint32_t)ldx * ES;
    const char* xb = reinterpret_cast<const char*>(X);
    int k = kb;
    for (; k + (U - 1) * step < ke; k += step * U) {
        float xv[U][NV][VEC];
        float w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = k + u * step;
            w[u] = edge_weight<OP>(ev, e, scale, m, ev_idx);
            const char* xr = row_at(xb, col[e], row_bytes);
#pragma unroll
            for (int j = 0; j < NV; ++j) vload_t<T, VEC>(xv[u][j], reinterpret_cast<const T*>(xr + off[j]));
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < NV; ++j)
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[j][v] = fmaf(w[u], xv[u][j][v], acc[j][v]);
    }
    if (k < ke) {
        float xv[U][NV][VEC];
        float w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = k + u * step;
            const bool ok = e < ke;
            w[u] = ok ? edge_weight<OP>(ev, e, scale, m, ev_idx) : 0.f;
            if (ok) {
                const char* xr = row_at(xb, col[e], row_bytes);
#pragma unroll
                for (int j = 0; j < NV; ++j) vload_t<T, VEC>(xv[u][j], reinterpret_cast<const T*>(xr + off[j]));
            } else {
                zero(xv[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < NV; ++j)
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[j][v] = fmaf(w[u], xv[u][j][v], acc[j][v]);
    }
}

// SpMM with one row per wave (W = 64): the row's columns and values are
// read 64 at a time, one entry per lane, and each gather takes its column
// and weight from that lane (readlane), so the gathers of a batch of U
// entries wait on one coalesced load per 64 entries instead of on their own
// column loads.  b and e must be wave-uniform.
template <typename T, int VEC, int NV, int U>
__device__ __forceinline__ void gather_acc_wave(float (&acc)[NV][VEC], const int32_t* col, const float* ev, int b,
                                                int e, const T* X, int64_t ldx, const Lanes<VEC, NV>& L, int F,
                                                const int32_t* ev_idx)
{
    const int lane = lane_id();
    for (int base = b; base < e; base += CSR_WAVE) {
        const int n = min(CSR_WAVE, e - base);
        const int cl = lane < n ? col[base + lane] : 0;
        const float wl = lane < n ? (ev ? ev[ev_idx ? ev_idx[base + lane] : base + lane] : 1.f) : 0.f;
        for (int i = 0; i < n; i += U) {
            float xv[U][NV][VEC];
            float w[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool ok = i + u < n;
                const int k = ok ? i + u : 0;
                const int c = __builtin_amdgcn_readlane(cl, k);
                w[u] = ok ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), k)) : 0.f;
                const T* xr = X + (int64_t)c * ldx;
#pragma unroll
                for (int j = 0; j < NV; ++j) {
                    if (ok && L.valid(j, F)) {
                        vload_t<T, VEC>(xv[u][j], xr + L.off(j));
                    } else {
#pragma unroll
                        for (int v = 0; v < VEC; ++v) xv[u][j][v] = 0.f;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < NV; ++j)
#pragma unroll
                    for (int v = 0; v < VEC; ++v) acc[j][v] = fmaf(w[u], xv[u][j][v], acc[j][v]);
        }
    }
}

// Softmax statistics (max, sum of exp) of scale * ev[e] over e = kb + t, kb + t + n, ...
// for this lane's t, merged over the n lanes (an aligned power-of-two set).
__device__ __forceinline__ void seg_softmax_stats(const float* ev, int kb, int ke, int t, int n,
                                                  float scale, float& m, float& l)
{
    m = -INFINITY;
    l = 0.f;
    for (int e = kb + t; e < ke; e += n) {
        float x = ev[e] * scale;
        if (x > m) {
            l = l * exp_neg(m - x) + 1.f;
            m = x;
        } else {
            l += exp_neg(x - m);
        }
    }
    // merge lanes t ^ 1, t ^ 2, ... within the n-lane set
    for (int s = 1; s < n; s <<= 1) {
        float m2 = shfl_xor(m, s), l2 = shfl_xor(l, s);
        float mm = fmaxf(m, m2);
        float a = (l > 0.f) ? l * exp_neg(m - mm) : 0.f;
        float b = (l2 > 0.f) ? l2 * exp_neg(m2 - mm) : 0.f;
        m = mm;
        l = a + b;
    }
}

// Attention from queries and keys: walks entries e = kb, kb + step, ... < ke
// of one row.  Per batch of U entries the group gathers the K and V rows,
// forms each score t = scale * <q, K[col_e]> (partial products summed over
// the group's W lanes), and folds the batch into the running maximum m, sum
// of exponentials l and weighted sum acc, rescaling them only by the batch's
// new maximum.  With probs, lane 0 of the group stores each entry's t; it is
// turned into the probability once the row's statistics are final.
template <typename T, int VEC, int NV, int U>
__device__ __forceinline__ void qk_walk(const float (&q)[NV][VEC], const int32_t* col, int kb, int ke, int step,
                                        const T* K, int64_t ldk, const T* Vv, int64_t ldv,
                                        const Lanes<VEC, NV>& L, int F, float scale, float& m, float& l,
                                        float (&acc)[NV][VEC], float* probs, int64_t pstride)
{
    // bf16 keys stay packed for the score: the query's pairs are repacked
    // once (exactly) and each key pair enters a two-term dot instruction
    constexpr bool PACKED = sizeof(T) == 2;
    constexpr int VP = PACKED ? VEC / 2 : 1;
    uint32_t qp[NV][VP];
    if constexpr (PACKED) {
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int v = 0; v < VP; ++v) qp[j][v] = pack_bf16_exact(q[j][2 * v], q[j][2 * v + 1]);
    }
    for (int k = kb; k < ke; k += step * U) {
        float kv[U][NV][PACKED ? 1 : VEC], vv[U][NV][VEC];
        uint32_t kp[U][NV][VP];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = k + u * step;
            const bool ok = e < ke;
            const int c = ok ? col[e] : 0;
            const T* kr = K + (int64_t)c * ldk;
            const T* vr = Vv + (int64_t)c * ldv;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                if (ok && L.valid(j, F)) {
                    if constexpr (PACKED)
                        vload_packed<VEC>(kp[u][j], reinterpret_cast<const bf16_t*>(kr + L.off(j)));
                    else
                        vload_t<T, VEC>(kv[u][j], kr + L.off(j));
                    vload_t<T, VEC>(vv[u][j], vr + L.off(j));
                } else {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) vv[u][j][v] = 0.f;
                    if constexpr (PACKED) {
#pragma unroll
                        for (int v = 0; v < VP; ++v) kp[u][j][v] = 0u;
                    } else {
#pragma unroll
                        for (int v = 0; v < VEC; ++v) kv[u][j][v] = 0.f;
                    }
                }
            }
        }
        float t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float d = 0.f;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                if constexpr (PACKED) {
#pragma unroll
                    for (int v = 0; v < VP; ++v) d = dot2_bf16(qp[j][v], kp[u][j][v], d);
                } else {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) d = fmaf(q[j][v], kv[u][j][v], d);
                }
            }
            t[u] = d;
        }
        group_sum_lanes(t, L.W);
        float mn = m;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            t[u] = (k + u * step < ke) ? t[u] * scale : -INFINITY;
            mn = fmaxf(mn, t[u]);
        }
        if (probs && L.lg == 0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = k + u * step;
                if (e < ke) probs[(int64_t)e * pstride] = t[u];
            }
        }
        const float corr = (l > 0.f) ? exp_neg(m - mn) : 0.f;
        l *= corr;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[j][v] *= corr;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = (k + u * step < ke) ? exp_neg(t[u] - mn) : 0.f;
            l += w;
#pragma unroll
            for (int j = 0; j < NV; ++j)
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[j][v] = fmaf(w, vv[u][j][v], acc[j][v]);
        }
        m = mn;
    }
}

// Merges the online-softmax states of a row whose entries the wave's groups
// took in turn (each group of W lanes holds its own m, l, acc): every lane
// ends with the row's maximum, sum and accumulated row.
template <int VEC, int NV>
__device__ __forceinline__ void qk_merge_groups(float& m, float& l, float (&acc)[NV][VEC], int W)
{
    float M = m;
    for (int s = W; s < CSR_WAVE; s <<= 1) M = fmaxf(M, shfl_xor(M, s));
    const float f = (l > 0.f) ? exp_neg(m - M) : 0.f;
    l = xor_sum_from(l * f, W);
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[j][v] = xor_sum_from(acc[j][v] * f, W);
    m = M;
}

// The probabilities of entries e = kb + t0, kb + t0 + n, ... < ke of a row
// whose scores t_e this wave stored in probs: exp(t_e - m) / l.  The fence
// orders the wave's stores of the scores before the lanes read them back.
__device__ __forceinline__ void probs_from_scores(float* probs, int64_t stride, int kb, int ke, int t0, int n,
                                                  float m, float l)
{
    __threadfence_block();
    for (int e = kb + t0; e < ke; e += n) {
        float* p = probs + (int64_t)e * stride;
        *p = exp_neg(*p - m) / l;
    }
}

// The probabilities of the entries of a row with given scores (scale * ev)
// and final statistics (m, l).
__device__ __forceinline__ void probs_from_given(float* probs, int64_t stride, const float* ev, float scale, int kb,
                                                 int ke, int t0, int n, float m, float l)
{
    for (int e = kb + t0; e < ke; e += n) probs[(int64_t)e * stride] = exp_neg(ev[e] * scale - m) / l;
}

// stream: non-temporal stores, for rows that are read again only after the
// kernel (the column-part segment format's partial rows)
template <int VEC, int NV>
__device__ __forceinline__ void store_row(float* dst, const float (&acc)[NV][VEC], const Lanes<VEC, NV>& L,
                                          int F, float mul, bool stream = false)
{
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        if (L.valid(j, F)) {
            float o[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) o[v] = acc[j][v] * mul;
            if (stream)
                vstore_stream<VEC>(dst + L.off(j), o);
            else
                vstore<VEC>(dst + L.off(j), o);
        }
    }
}

template <int VEC, int NV>
__device__ __forceinline__ void store_row_div(float* dst, const float (&acc)[NV][VEC], const Lanes<VEC, NV>& L,
                                              int F, float den)
{
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        if (L.valid(j, F)) {
            float o[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) o[v] = acc[j][v] / den;
            vstore<VEC>(dst + L.off(j), o);
        }
    }
}

// SDDMM: out[e] = <u, X[col[e]]> for e = kb, kb + step, ... < ke; the W lanes
// of the group reduce the partial dot products and lane 0 of the group writes.
template <typename T, int VEC, int NV, int U>
__device__ __forceinline__ void sddmm_edges(const float (&u)[NV][VEC], const int32_t* col, int kb, int ke,
                                            int step, const T* X, int64_t ldx, const Lanes<VEC, NV>& L,
                                            int F, float* out, const int32_t* out_idx)
{
    // bf16 operands stay packed: the row's pairs are repacked once (exactly)
    // and each gathered pair enters a two-term dot instruction
    constexpr bool PACKED = sizeof(T) == 2;
    constexpr int VP = PACKED ? VEC / 2 : 1;
    uint32_t up[NV][VP];
    if constexpr (PACKED) {
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int v = 0; v < VP; ++v) up[j][v] = pack_bf16_exact(u[j][2 * v], u[j][2 * v + 1]);
    }
    for (int k = kb; k < ke; k += step * U) {
        float xv[U][NV][PACKED ? 1 : VEC];
        uint32_t xp[U][NV][VP];
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
            int e = k + uu * step;
            bool ok = e < ke;
            int c = ok ? col[e] : 0;
            const T* xr = X + (int64_t)c * ldx;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                if constexpr (PACKED) {
                    if (ok && L.valid(j, F)) {
                        vload_packed<VEC>(xp[uu][j], reinterpret_cast<const bf16_t*>(xr + L.off(j)));
                    } else {
#pragma unroll
                        for (int v = 0; v < VP; ++v) xp[uu][j][v] = 0u;
                    }
                } else {
                    if (ok && L.valid(j, F)) {
                        vload_t<T, VEC>(xv[uu][j], xr + L.off(j));
                    } else {
#pragma unroll
                        for (int v = 0; v < VEC; ++v) xv[uu][j][v] = 0.f;
                    }
                }
            }
        }
        float d[U];
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                if constexpr (PACKED) {
#pragma unroll
                    for (int v = 0; v < VP; ++v) s = dot2_bf16(up[j][v], xp[uu][j][v], s);
                } else {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) s = fmaf(u[j][v], xv[uu][j][v], s);
                }
            }
            d[uu] = s;
        }
        group_sum_lanes(d, L.W);
        if (L.lg == 0) {
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
                int e = k + uu * step;
                if (e < ke) out[out_idx ? out_idx[e] : e] = d[uu];
            }
        }
    }
}

// The SpMM and the SDDMM of Op::Dual over entries e = kb, kb + step, ... < ke
// of one row: acc += w_e * X[col_e] (w_e = ev[ev_idx[e]], ev[e], or 1 without
// values) and z_e = <u, X[col_e]>, both from one load of each gathered row.
// The W lanes of the group reduce the partial dot products and lane 0 of the
// group writes z_e at Z[z_idx[e]] (or Z[e]).  Lanes past the width read the
// row's first features (in bounds) and zero them: their u is zero and an
// infinite feature must not turn the dot product into NaN.
template <typename T, int VEC, int NV, int U>
__device__ __forceinline__ void dual_walk(float (&acc)[NV][VEC], const float (&u)[NV][VEC], const int32_t* col,
                                          const float* ev, const int32_t* ev_idx, int kb, int ke, int step,
                                          const T* X, int64_t ldx, const Lanes<VEC, NV>& L, int F, float* Z,
                                          const int32_t* z_idx)
{
    constexpr uint32_t ES = sizeof(T);
    uint32_t off[NV];
    bool on[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        on[j] = L.valid(j, F);
        off[j] = on[j] ? (uint32_t)L.off(j) * ES : 0u;
    }
    const uint32_t row_bytes = (uint32_t)ldx * ES;
    const char* xb = reinterpret_cast<const char*>(X);
    for (int k = kb; k < ke; k += step * U) {
        float xv[U][NV][VEC];
        float w[U];
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
            const int e = k + uu * step;
            const bool ok = e < ke;
            w[uu] = ok ? (ev ? ev[ev_idx ? ev_idx[e] : e] : 1.f) : 0.f;
            if (ok) {
                const char* xr = row_at(xb, col[e], row_bytes);
#pragma unroll
                for (int j = 0; j < NV; ++j) {
                    vload_t<T, VEC>(xv[uu][j], reinterpret_cast<const T*>(xr + off[j]));
                    if (!on[j]) {
#pragma unroll
                        for (int v = 0; v < VEC; ++v) xv[uu][j][v] = 0.f;
                    }
                }
            } else {
                zero(xv[uu]);
            }
        }
        float d[U];
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
            float sdot = 0.f;
#pragma unroll
            for (int j = 0; j < NV; ++j)
#pragma unroll
                for (int v = 0; v < VEC; ++v) sdot = fmaf(u[j][v], xv[uu][j][v], sdot);
            d[uu] = sdot;
        }
#pragma unroll
        for (int uu = 0; uu < U; ++uu)
#pragma unroll
            for (int j = 0; j < NV; ++j)
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[j][v] = fmaf(w[uu], xv[uu][j][v], acc[j][v]);
        group_sum_lanes(d, L.W);
        if (L.lg == 0) {
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
                const int e = k + uu * step;
                if (e < ke) Z[z_idx ? z_idx[e] : e] = d[uu];
            }
        }
    }
}

// U row read for pattern row r: its own row, or the row a segment belongs to
__device__ __forceinline__ int64_t u_row_of(const Fp32Args& a, int64_t r) { return a.u_row ? a.u_row[r] : r; }

template <typename T, int VEC, int NV>
__device__ __forceinline__ void load_row(float (&u)[NV][VEC], const T* src, const Lanes<VEC, NV>& L, int F)
{
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        if (L.valid(j, F)) {
            vload_t<T, VEC>(u[j], src + L.off(j));
        } else {
#pragma unroll
            for (int v = 0; v < VEC; ++v) u[j][v] = 0.f;
        }
    }
}

// ---------------------------------------------------------------------------
// Row-group mapping
// ---------------------------------------------------------------------------
template <Op OP, typename T, int VEC, int NV, int U>
__global__ __launch_bounds__(CSR_BLOCK) void k_rowgroup(Fp32Args a)
{
    const T* X = static_cast<const T*>(a.X);
    Lanes<VEC, NV> L(a.W);
    int64_t row = ((int64_t)blockIdx.x * CSR_BLOCK + threadIdx.x) / a.W;
    if (row >= a.n_rows) return;  // groups are whole: no group is split by this test
    int b = a.row_ptr[row], e = a.row_ptr[row + 1];

    if constexpr (OP == Op::Sddmm) {
        float u[NV][VEC];
        load_row<T, VEC, NV>(u, static_cast<const T*>(a.U) + u_row_of(a, row) * a.ldu, L, a.F);
        sddmm_edges<T, VEC, NV, U>(u, a.col_idx, b, e, 1, X, a.ldx, L, a.F, a.Y, a.out_idx);
    } else if constexpr (OP == Op::Dual) {
        float u[NV][VEC], acc[NV][VEC];
        load_row<T, VEC, NV>(u, static_cast<const T*>(a.U) + row * a.ldu, L, a.F);
        zero(acc);
        dual_walk<T, VEC, NV, U>(acc, u, a.col_idx, a.ev, a.ev_idx, b, e, 1, X, a.ldx, L, a.F, a.Z, a.out_idx);
        store_row<VEC, NV>(a.Y + row * a.ldy, acc, L, a.F, 1.f);
    } else if constexpr (OP == Op::AttnQK) {
        constexpr int UQ = U > 1 ? U / 2 : 1;  // K and V rows in flight: half the entries
        float q[NV][VEC], acc[NV][VEC];
        load_row<T, VEC, NV>(q, static_cast<const T*>(a.U) + row * a.ldu, L, a.F);
        zero(acc);
        float m = -INFINITY, l = 0.f;
        qk_walk<T, VEC, NV, UQ>(q, a.col_idx, b, e, 1, X, a.ldx, static_cast<const T*>(a.V), a.ldv, L, a.F, a.scale,
                                m, l, acc, a.probs, a.probs_stride);
        float* dst = a.Y + row * a.ldy;
        if (e > b) {
            store_row_div<VEC, NV>(dst, acc, L, a.F, l);
            if (a.probs) probs_from_scores(a.probs, a.probs_stride, b, e, L.lg, a.W, m, l);
        } else {
            store_row<VEC, NV>(dst, acc, L, a.F, 1.f);
        }
    } else {
        float acc[NV][VEC];
        zero(acc);
        float m = 0.f, l = 1.f;
        if constexpr (OP == Op::Attention) {
            seg_softmax_stats(a.ev, b, e, L.lg, a.W, a.scale, m, l);
            if (a.probs && e > b) probs_from_given(a.probs, a.probs_stride, a.ev, a.scale, b, e, L.lg, a.W, m, l);
        }
        if (OP == Op::Spmm && a.W == CSR_WAVE)
            gather_acc_wave<T, VEC, NV, U>(acc, a.col_idx, a.ev, __builtin_amdgcn_readfirstlane(b),
                                           __builtin_amdgcn_readfirstlane(e), X, a.ldx, L, a.F, a.ev_idx);
        else
            gather_acc<OP, T, VEC, NV, U>(acc, a.col_idx, a.ev, b, e, 1, X, a.ldx, L, a.F, a.scale, m,
                                          OP == Op::Spmm ? a.ev_idx : nullptr);
        float* dst = a.Y + row * a.ldy;
        if (OP == Op::Attention && e > b)
            store_row_div<VEC, NV>(dst, acc, L, a.F, l);
        else
            store_row<VEC, NV>(dst, acc, L, a.F, 1.f, a.stream_y);  // empty rows: acc == 0
    }
}

// 4 floats at a 4-byte aligned address: one 16-byte access (the hardware
// takes dword-aligned multi-dword loads and stores).
typedef float float4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// Row-group SpMM with wide lanes: one row per wave, 4 floats per lane in each
// of NV passes of 64 lanes, over rows that are only 4-byte aligned or whose
// width is not a multiple of 4.  Lane l of pass j covers features
// off = (j * 64 + l) * 4 ..; the lane whose 4 floats would pass the width F
// reads the 4 ending at F instead (shift = off - (F - 4)) and writes the top
// F - off of its sums, so every access stays inside its row; lanes past the
// width read the row's first 4 floats and write nothing.  Columns and values
// are read 64 at a time, one per lane, and each gather takes its column from
// that lane (readlane).
template <int NV, int U>
__global__ __launch_bounds__(CSR_BLOCK) void k_rowgroup_wide(Fp32Args a)
{
    const int lane = lane_id();
    const int64_t row = ((int64_t)blockIdx.x * CSR_BLOCK + threadIdx.x) / CSR_WAVE;
    if (row >= a.n_rows) return;  // whole waves: no wave is split by this test
    const int b = __builtin_amdgcn_readfirstlane(a.row_ptr[row]);
    const int e = __builtin_amdgcn_readfirstlane(a.row_ptr[row + 1]);
    const int F = a.F;
    uint32_t lo[NV];  // byte offset of the lane's 4 floats in a row
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int off = (j * CSR_WAVE + lane) * 4;
        lo[j] = (uint32_t)(off + 4 <= F ? off : (off < F ? F - 4 : 0)) * 4u;
    }
    const uint32_t row_bytes = (uint32_t)a.ldx * 4u;
    const char* xb = static_cast<const char*>(a.X);
    float4_a4 acc[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) acc[j] = float4_a4{0.f, 0.f, 0.f, 0.f};
    for (int base = b; base < e; base += CSR_WAVE) {
        const int n = min(CSR_WAVE, e - base);
        const int cl = lane < n ? a.col_idx[base + lane] : 0;
        const float wl = lane < n ? (a.ev ? a.ev[a.ev_idx ? a.ev_idx[base + lane] : base + lane] : 1.f) : 0.f;
        // U entries per batch, every load issued before the first multiply-add
        auto batch = [&](int i, bool tail) {
            float4_a4 xv[U][NV];
            float w[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (!tail || i + u < n) {
                    const char* xr = row_at(xb, __builtin_amdgcn_readlane(cl, i + u), row_bytes);
                    w[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), i + u));
#pragma unroll
                    for (int j = 0; j < NV; ++j) xv[u][j] = *reinterpret_cast<const float4_a4*>(xr + lo[j]);
                } else {
                    // padding past the batch's entries (the same for the whole
                    // wave, so no load is issued for it) adds exact zeros
                    w[u] = 0.f;
#pragma unroll
                    for (int j = 0; j < NV; ++j) xv[u][j] = float4_a4{0.f, 0.f, 0.f, 0.f};
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < NV; ++j) {
                    acc[j].x = fmaf(w[u], xv[u][j].x, acc[j].x);
                    acc[j].y = fmaf(w[u], xv[u][j].y, acc[j].y);
                    acc[j].z = fmaf(w[u], xv[u][j].z, acc[j].z);
                    acc[j].w = fmaf(w[u], xv[u][j].w, acc[j].w);
                }
        };
        int i = 0;
        for (; i + U <= n; i += U) batch(i, false);
        if (i < n) batch(i, true);
    }
    float* dst = a.Y + row * a.ldy;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int off = (j * CSR_WAVE + lane) * 4;
        if (off + 4 <= F) {
            float4_a4* d = reinterpret_cast<float4_a4*>(dst + off);
            if (a.stream_y)
                __builtin_nontemporal_store(acc[j], d);
            else
                *d = acc[j];
        } else if (off < F) {  // the top F - off of the 4 floats ending at F
            const int sh = off - (F - 4);
            for (int t = 0; t < F - off; ++t) {
                const int i = sh + t;
                dst[off + t] = i == 1 ? acc[j].y : (i == 2 ? acc[j].z : acc[j].w);  // i >= 1 here
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Merge-path mapping
// ---------------------------------------------------------------------------
template <int D>
struct MpShared {
    int32_t rp[CSR_WAVES_PER_BLOCK][D + 2];
    int32_t col[CSR_WAVES_PER_BLOCK][D];
    float ev[CSR_WAVES_PER_BLOCK][D];
};

template <Op OP, typename T, int VEC, int NV, int U, int D>
__global__ __launch_bounds__(CSR_BLOCK) void k_mergepath(Fp32Args a)
{
    __shared__ MpShared<D> sh;
    const T* X = static_cast<const T*>(a.X);
    const T* Urow = static_cast<const T*>(a.U);
    const int wave = threadIdx.x / CSR_WAVE;
    const int lane = lane_id();
    const int64_t chunk = (int64_t)blockIdx.x * CSR_WAVES_PER_BLOCK + wave;
    const bool active = chunk < a.n_chunks;

    int x0 = 0, y0 = 0, x1 = 0, y1 = 0, nrow = 0;
    bool slotA = false, slotB = false;
    if (active) {
        x0 = a.part[2 * chunk];
        y0 = a.part[2 * chunk + 1];
        x1 = a.part[2 * chunk + 2];
        y1 = a.part[2 * chunk + 3];
        // rows x0 .. x1-1 end in this chunk; row x1 may own entries [.., y1).
        // Rows x0 .. x1 (x1 only if it exists): row_ptr[x0 .. min(x1, n_rows - 1) + 1]
        const int nr = (x1 < a.n_rows ? x1 : (int)a.n_rows - 1) - x0 + 2;
        stage_chunk<(D + 2 + CSR_WAVE - 1) / CSR_WAVE, D / CSR_WAVE, OP != Op::Sddmm, float>(
            sh.rp[wave], a.row_ptr + x0, nr, sh.col[wave], a.col_idx + y0, sh.ev[wave],
            a.ev ? (a.ev_idx ? a.ev : a.ev + y0) : nullptr, y1 - y0, a.ev_idx ? a.ev_idx + y0 : nullptr);
    }
    __syncthreads();
    if (!active) return;

    const int32_t* rp = sh.rp[wave];
    const int32_t* col = sh.col[wave] - y0;  // indexed by absolute entry id
    const float* ev = sh.ev[wave] - y0;
    slotB = (x1 < a.n_rows) && (max(rp[x1 - x0], y0) < y1);
    nrow = x1 - x0 + (slotB ? 1 : 0);
    slotA = (x0 < x1) && (rp[0] < y0);
    if (lane == 0) {
        a.carry_row[2 * chunk] = slotA ? x0 : -1;
        a.carry_row[2 * chunk + 1] = slotB ? x1 : -1;
    }

    Lanes<VEC, NV> L(a.W);
    const int G = L.G;
    const int long_row = (G == 1) ? 0 : a.long_row;

    // Emits the result of row index i (row x0 + i) of this chunk: rows
    // x0 .. x1-1 end here and are final unless they began before y0 (slot A,
    // only possible for i == 0); row x1, when present, continues (slot B).
    const int nend = x1 - x0;
    constexpr bool SOFT = OP == Op::Attention || OP == Op::AttnQK;
    auto emit = [&](int i, float (&acc)[NV][VEC], float m, float l, bool whole_wave) {
        const int rs = rp[i], re = rp[i + 1];
        const int64_t row = (int64_t)x0 + i;
        const bool complete = i < nend && rs >= y0;
        if constexpr (SOFT) {
            // a row complete in this chunk: its probabilities, from every lane
            // that holds the row's statistics (a split row gets them in the fix-up)
            if (a.probs && complete && re > rs) {
                const int t0 = whole_wave ? lane : L.lg, n = whole_wave ? CSR_WAVE : a.W;
                if constexpr (OP == Op::Attention)
                    probs_from_given(a.probs, a.probs_stride, ev, a.scale, rs, re, t0, n, m, l);
                else
                    probs_from_scores(a.probs, a.probs_stride, rs, re, t0, n, m, l);
            }
        }
        if (whole_wave && L.g != 0) return;
        if (complete) {
            float* dst = a.Y + row * a.ldy;
            if (SOFT && re > rs)
                store_row_div<VEC, NV>(dst, acc, L, a.F, l);
            else
                store_row<VEC, NV>(dst, acc, L, a.F, 1.f, a.stream_y);
        } else {
            const int64_t slot = 2 * chunk + ((i == nend) ? 1 : 0);
            store_row<VEC, NV>(a.carry_val + slot * a.F, acc, L, a.F, 1.f);
            if (SOFT && L.lg == 0) {
                a.carry_ml[2 * slot] = m;
                a.carry_ml[2 * slot + 1] = l;
            }
        }
    };

    if constexpr (OP == Op::AttnQK) {
        constexpr int UQ = U > 1 ? U / 2 : 1;
        const T* Q = static_cast<const T*>(a.U);
        const T* Vv = static_cast<const T*>(a.V);
        // pass 1: long segments, whole wave (the groups take interleaved
        // entries, then their states are merged)
        for (int i = 0; i < nrow; ++i) {
            const int sb = max(rp[i], y0), se = min(rp[i + 1], y1);
            if (se - sb < long_row) continue;
            float q[NV][VEC], acc[NV][VEC];
            load_row<T, VEC, NV>(q, Q + ((int64_t)x0 + i) * a.ldu, L, a.F);
            zero(acc);
            float m = -INFINITY, l = 0.f;
            qk_walk<T, VEC, NV, UQ>(q, col, sb + L.g, se, G, X, a.ldx, Vv, a.ldv, L, a.F, a.scale, m, l, acc,
                                    a.probs, a.probs_stride);
            if (G > 1) qk_merge_groups<VEC, NV>(m, l, acc, a.W);
            emit(i, acc, m, l, true);
        }
        // pass 2: short segments, one group each
        if (G > 1) {
            for (int i = L.g; i < nrow; i += G) {
                const int sb = max(rp[i], y0), se = min(rp[i + 1], y1);
                if (se - sb >= long_row) continue;
                float q[NV][VEC], acc[NV][VEC];
                load_row<T, VEC, NV>(q, Q + ((int64_t)x0 + i) * a.ldu, L, a.F);
                zero(acc);
                float m = -INFINITY, l = 0.f;
                qk_walk<T, VEC, NV, UQ>(q, col, sb, se, 1, X, a.ldx, Vv, a.ldv, L, a.F, a.scale, m, l, acc, a.probs,
                                        a.probs_stride);
                emit(i, acc, m, l, false);
            }
        }
    } else if constexpr (OP == Op::Dual) {
        // pass 1: long segments, whole wave (the groups take interleaved
        // entries, then their sums are reduced); the values are in LDS
        for (int i = 0; i < nrow; ++i) {
            const int sb = max(rp[i], y0), se = min(rp[i + 1], y1);
            if (se - sb < long_row) continue;
            float u[NV][VEC], acc[NV][VEC];
            load_row<T, VEC, NV>(u, Urow + ((int64_t)x0 + i) * a.ldu, L, a.F);
            zero(acc);
            dual_walk<T, VEC, NV, U>(acc, u, col, ev, nullptr, sb + L.g, se, G, X, a.ldx, L, a.F, a.Z, a.out_idx);
            if (G > 1) {
#pragma unroll
                for (int j = 0; j < NV; ++j)
#pragma unroll
                    for (int v = 0; v < VEC; ++v) acc[j][v] = xor_sum_from(acc[j][v], a.W);
            }
            emit(i, acc, 0.f, 1.f, true);
        }
        // pass 2: short segments, one group each
        if (G > 1) {
            for (int i = L.g; i < nrow; i += G) {
                const int sb = max(rp[i], y0), se = min(rp[i + 1], y1);
                if (se - sb >= long_row) continue;
                float u[NV][VEC], acc[NV][VEC];
                load_row<T, VEC, NV>(u, Urow + ((int64_t)x0 + i) * a.ldu, L, a.F);
                zero(acc);
                dual_walk<T, VEC, NV, U>(acc, u, col, ev, nullptr, sb, se, 1, X, a.ldx, L, a.F, a.Z, a.out_idx);
                emit(i, acc, 0.f, 1.f, false);
            }
        }
    } else if constexpr (OP == Op::Sddmm) {
        // pass 1: long segments, whole wave
        for (int i = 0; i < nrow; ++i) {
            const int sb = max(rp[i], y0), se = min(rp[i + 1], y1);
            if (se - sb < long_row || se <= sb) continue;
            float u[NV][VEC];
            load_row<T, VEC, NV>(u, Urow + u_row_of(a, (int64_t)x0 + i) * a.ldu, L, a.F);
            sddmm_edges<T, VEC, NV, U>(u, col, sb + L.g, se, G, X, a.ldx, L, a.F, a.Y, a.out_idx);
        }
        // pass 2: short segments, one group each
        for (int i = L.g; i < nrow; i += G) {
            const int sb = max(rp[i], y0), se = min(rp[i + 1], y1);
            if (se - sb >= long_row || se <= sb) continue;
            float u[NV][VEC];
            load_row<T, VEC, NV>(u, Urow + u_row_of(a, (int64_t)x0 + i) * a.ldu, L, a.F);
            sddmm_edges<T, VEC, NV, U>(u, col, sb, se, 1, X, a.ldx, L, a.F, a.Y, a.out_idx);
        }
    } else {
        for (int i = 0; i < nrow; ++i) {
            const int sb = max(rp[i], y0), se = min(rp[i + 1], y1);
            if (se - sb < long_row) continue;
            float acc[NV][VEC];
            zero(acc);
            float m = 0.f, l = 1.f;
            if constexpr (OP == Op::Attention) seg_softmax_stats(ev, sb, se, lane, CSR_WAVE, a.scale, m, l);
            gather_acc<OP, T, VEC, NV, U>(acc, col, ev, sb + L.g, se, G, X, a.ldx, L, a.F, a.scale, m);
            if (G > 1) {
#pragma unroll
                for (int j = 0; j < NV; ++j)
#pragma unroll
                    for (int v = 0; v < VEC; ++v) acc[j][v] = xor_sum_from(acc[j][v], a.W);
            }
            emit(i, acc, m, l, true);
        }
        if (G > 1) {
            for (int i = L.g; i < nrow; i += G) {
                const int sb = max(rp[i], y0), se = min(rp[i + 1], y1);
                if (se - sb >= long_row) continue;
                float acc[NV][VEC];
                zero(acc);
                float m = 0.f, l = 1.f;
                if constexpr (OP == Op::Attention) seg_softmax_stats(ev, sb, se, L.lg, a.W, a.scale, m, l);
                gather_acc<OP, T, VEC, NV, U>(acc, col, ev, sb, se, 1, X, a.ldx, L, a.F, a.scale, m);
                emit(i, acc, m, l, false);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Entry-parallel mapping for small widths (segmented scan)
// ---------------------------------------------------------------------------
// The chunk is staged as in the merge-path mapping, but its entries are
// dealt to the lanes in order: lane l takes entries b + l, b + 64 + l, ...,
// and each lane gathers the whole (small) feature row of its entry, so a
// batch of 64 entries costs one round of gathers whatever the row lengths.
// SpMM then sums the products of each row with an inclusive segmented scan
// across the lanes (segments = runs of lanes holding the same row) and a
// carry between batches; the last lane of a row's run writes the row.  SDDMM
// needs no reduction across entries: each lane forms its entry's dot product.
template <Op OP, typename T, int VEC, int NV, int U, int D>
__global__ __launch_bounds__(CSR_BLOCK) void k_segscan(Fp32Args a)
{
    __shared__ MpShared<D> sh;
    const T* X = static_cast<const T*>(a.X);
    const T* Urow = static_cast<const T*>(a.U);
    const int wave = threadIdx.x / CSR_WAVE;
    const int lane = lane_id();
    const int64_t chunk = (int64_t)blockIdx.x * CSR_WAVES_PER_BLOCK + wave;
    const bool active = chunk < a.n_chunks;
    int x0 = 0, y0 = 0, x1 = 0, y1 = 0;
    if (active) {
        x0 = a.part[2 * chunk];
        y0 = a.part[2 * chunk + 1];
        x1 = a.part[2 * chunk + 2];
        y1 = a.part[2 * chunk + 3];
        const int nr = (x1 < a.n_rows ? x1 : (int)a.n_rows - 1) - x0 + 2;
        stage_chunk<(D + 2 + CSR_WAVE - 1) / CSR_WAVE, D / CSR_WAVE, OP != Op::Sddmm, float>(
            sh.rp[wave], a.row_ptr + x0, nr, sh.col[wave], a.col_idx + y0, sh.ev[wave],
            a.ev ? (a.ev_idx ? a.ev : a.ev + y0) : nullptr, y1 - y0, a.ev_idx ? a.ev_idx + y0 : nullptr);
    }
    __syncthreads();
    if (!active) return;
    const int32_t* rp = sh.rp[wave];
    const int32_t* col = sh.col[wave] - y0;
    const float* ev = sh.ev[wave] - y0;
    const bool slotB = (x1 < a.n_rows) && (max(rp[x1 - x0], y0) < y1);
    const int nrow = x1 - x0 + (slotB ? 1 : 0);
    const bool slotA = (x0 < x1) && (rp[0] < y0);
    if (lane == 0) {
        a.carry_row[2 * chunk] = slotA ? x0 : -1;
        a.carry_row[2 * chunk + 1] = slotB ? x1 : -1;
    }
    const int nend = x1 - x0;
    const int F = a.F;

    // chunk row index of entry e: the largest i < nrow with rp[i] <= e
    auto row_of = [&](int e) {
        int lo = 0, hi = nrow - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (rp[mid] <= e)
                lo = mid;
            else
                hi = mid - 1;
        }
        return lo;
    };
    auto load_row = [&](float (&v)[NV][VEC], const T* src) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            if (j * VEC < F) {
                vload_t<T, VEC>(v[j], src + j * VEC);
            } else {
#pragma unroll
                for (int t = 0; t < VEC; ++t) v[j][t] = 0.f;
            }
        }
    };

    if constexpr (OP == Op::Sddmm) {
        for (int b = y0; b < y1; b += CSR_WAVE * U) {
            float uv[U][NV][VEC], xv[U][NV][VEC];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = b + u * CSR_WAVE + lane;
                if (e < y1) {
                    load_row(uv[u], Urow + u_row_of(a, (int64_t)x0 + row_of(e)) * a.ldu);
                    load_row(xv[u], X + (int64_t)col[e] * a.ldx);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = b + u * CSR_WAVE + lane;
                if (e < y1) {
                    float d = 0.f;
#pragma unroll
                    for (int j = 0; j < NV; ++j)
#pragma unroll
                        for (int t = 0; t < VEC; ++t) d = fmaf(uv[u][j][t], xv[u][j][t], d);
                    a.Y[a.out_idx ? a.out_idx[e] : e] = d;
                }
            }
        }
    } else {
        // a row's result, written by one lane: final row, or a piece of a split row
        auto emit = [&](int i, const float (&v)[NV][VEC]) {
            const bool to_y = i < nend && rp[i] >= y0;
            float* dst = to_y ? a.Y + ((int64_t)x0 + i) * a.ldy
                              : a.carry_val + (2 * chunk + ((i == nend) ? 1 : 0)) * F;
            const bool stream = a.stream_y && to_y;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                if (j * VEC < F) {
                    if (stream)
                        vstore_stream<VEC>(dst + j * VEC, v[j]);
                    else
                        vstore<VEC>(dst + j * VEC, v[j]);
                }
            }
        };
        // rows without entries in this chunk: zero rows (or zero pieces)
        for (int i = lane; i < nrow; i += CSR_WAVE) {
            if (max(rp[i], y0) == min(rp[i + 1], y1)) {
                float z[NV][VEC];
                zero(z);
                emit(i, z);
            }
        }
        float carry[NV][VEC];
        zero(carry);
        int carry_row = -1;
        for (int b = y0; b < y1; b += CSR_WAVE * U) {
            float xv[U][NV][VEC];
            float w[U];
            int ri[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = b + u * CSR_WAVE + lane;
                const bool ok = e < y1;
                w[u] = ok ? ev[e] : 0.f;
                ri[u] = ok ? row_of(e) : -1 - lane;  // a lane past the end forms no segment
                if (ok) {
                    load_row(xv[u], X + (int64_t)col[e] * a.ldx);
                } else {
                    zero(xv[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = b + u * CSR_WAVE + lane;
                const int i = ri[u];
                float v[NV][VEC];
#pragma unroll
                for (int j = 0; j < NV; ++j)
#pragma unroll
                    for (int t = 0; t < VEC; ++t) v[j][t] = w[u] * xv[u][j][t];
                // inclusive segmented scan across lanes (row ids never
                // decrease over the lanes holding entries; lanes past the end
                // carry ids no other lane has)
                seg_sum_wave(i, v);
                if (i == carry_row) {
#pragma unroll
                    for (int j = 0; j < NV; ++j)
#pragma unroll
                        for (int t = 0; t < VEC; ++t) v[j][t] += carry[j][t];
                }
                const int inext = next_lane_i(INT_MIN, i);
                const bool ok = e < y1;
                const bool tail = ok && (lane == CSR_WAVE - 1 || inext != i);
                const bool row_last = ok && (e == min(rp[i + 1], y1) - 1);
                if (tail && row_last) emit(i, v);
                // the run of the last lane continues into the next batch unless its row ended
                const int last_i = lane63_i(i);
                const bool last_done = lane63_i((int)row_last) != 0;
                carry_row = last_done ? -1 : last_i;
#pragma unroll
                for (int j = 0; j < NV; ++j)
#pragma unroll
                    for (int t = 0; t < VEC; ++t) carry[j][t] = lane63_f(v[j][t]);
            }
        }
    }
}

// Fix-up of rows split across chunks.  One wave per chunk c whose slot A holds
// a row r: the pieces of r are slot B of chunks k0 .. c-1 (the run of chunks
// right before c whose slot B holds r) and slot A of c.  SpMM adds them;
// attention rescales each piece by exp(m_k - M), M the largest piece maximum.
// The groups of the wave take interleaved pieces and are reduced in a fixed
// order, so the result is reproducible.
template <Op OP, int VEC, int NV>
__device__ __forceinline__ void fixup_one(const Fp32Args& a, int64_t c, int r)
{
    const int lane = lane_id();

    // k0: first chunk of the run of slot-B pieces of row r ending at c - 1
    int64_t k0 = c;
    while (true) {
        int64_t idx = k0 - 1 - lane;
        bool ok = idx >= 0 && a.carry_row[2 * idx + 1] == r;
        uint64_t mask = __ballot(ok);
        int n = (~mask == 0) ? 64 : __builtin_ctzll(~mask);
        k0 -= n;
        if (n < 64) break;
    }
    // pieces: p = 0 .. np-1 -> slot index 2*(k0+p)+1 for p < np-1, 2*c for the last
    const int64_t np = c - k0 + 1;
    auto slot_of = [&](int64_t p) -> int64_t { return (p < np - 1) ? 2 * (k0 + p) + 1 : 2 * c; };

    Lanes<VEC, NV> L(a.W);
    constexpr bool SOFT = OP == Op::Attention || OP == Op::AttnQK;
    float M = 0.f;
    if constexpr (SOFT) {
        float mm = -INFINITY;
        for (int64_t p = lane; p < np; p += CSR_WAVE) {
            int64_t s = slot_of(p);
            if (a.carry_ml[2 * s + 1] > 0.f) mm = fmaxf(mm, a.carry_ml[2 * s]);
        }
        for (int s = 1; s < CSR_WAVE; s <<= 1) mm = fmaxf(mm, shfl_xor(mm, s));
        M = mm;
    }
    float acc[NV][VEC];
    zero(acc);
    float lsum = 0.f;
    for (int64_t p = L.g; p < np; p += L.G) {
        int64_t s = slot_of(p);
        float w = 1.f;
        if constexpr (SOFT) {
            float lp = a.carry_ml[2 * s + 1];
            w = (lp > 0.f) ? exp_neg(a.carry_ml[2 * s] - M) : 0.f;
            lsum = fmaf(w, lp, lsum);
        }
        const float* src = a.carry_val + s * a.F;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            if (L.valid(j, a.F)) {
                float x[VEC];
                vload<VEC>(x, src + L.off(j));
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[j][v] = fmaf(w, x[v], acc[j][v]);
            }
        }
    }
    if (L.G > 1) {
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[j][v] = xor_sum_from(acc[j][v], a.W);
        lsum = xor_sum_from(lsum, a.W);
    }
    if constexpr (SOFT) {
        // the split row's probabilities, now that its statistics are final
        // (the scores t of attention from queries and keys were stored by the
        // main kernel)
        if (a.probs) {
            const int rb = a.row_ptr[r], re = a.row_ptr[r + 1];
            for (int e = rb + lane; e < re; e += CSR_WAVE) {
                float* pp = a.probs + (int64_t)e * a.probs_stride;
                const float t = (OP == Op::AttnQK) ? *pp : a.ev[e] * a.scale;
                *pp = exp_neg(t - M) / lsum;
            }
        }
    }
    if (L.g != 0) return;
    float* dst = a.Y + (int64_t)r * a.ldy;
    if constexpr (SOFT)
        store_row_div<VEC, NV>(dst, acc, L, a.F, lsum);
    else
        store_row<VEC, NV>(dst, acc, L, a.F, 1.f, a.stream_y);
}

// chunks per fix-up wave: each chunk with a split row costs the wave a few
// dependent loads, so a short window lets more waves share that work
constexpr int FP32_FIX_CHUNKS = 16;

template <Op OP, int VEC, int NV>
__global__ __launch_bounds__(CSR_BLOCK) void k_fixup(Fp32Args a)
{
    const int64_t base = ((int64_t)blockIdx.x * CSR_WAVES_PER_BLOCK +
                          __builtin_amdgcn_readfirstlane(threadIdx.x / CSR_WAVE)) * FP32_FIX_CHUNKS;
    if (base >= a.n_chunks) return;
    const int lane = lane_id();
    const int64_t mine = base + lane;
    const int rl = (lane < FP32_FIX_CHUNKS && mine < a.n_chunks) ? a.carry_row[2 * mine] : -1;
    uint64_t todo = __ballot(rl >= 0);
    while (todo) {
        const int j = __builtin_ctzll(todo);
        todo &= todo - 1;
        fixup_one<OP, VEC, NV>(a, base + j, __shfl(rl, j, CSR_WAVE));
    }
}

// Column-part segment format: Y[r] = the sum of row r's segment partial rows
// in segment (= part) order, +0 for a row without segments.  One lane group
// per row, laid out as in the row-group mapping (16-byte lane accesses),
// with 4 partial rows in flight per group; the sum's order is fixed.
template <int VEC, int NV>
__global__ __launch_bounds__(CSR_BLOCK) void k_hyb_reduce_rows(float* Y, int64_t ldy, const float* part, int32_t F,
                                                               int32_t W, const int32_t* row_seg_ptr,
                                                               const int32_t* row_seg, int64_t n_rows)
{
    constexpr int UR = 4;
    Lanes<VEC, NV> L(W);
    const int64_t row = ((int64_t)blockIdx.x * CSR_BLOCK + threadIdx.x) / W;
    if (row >= n_rows) return;  // groups are whole: no group is split by this test
    const int b = row_seg_ptr[row], e = row_seg_ptr[row + 1];
    float acc[NV][VEC];
    zero(acc);
    for (int k = b; k < e; k += UR) {
        float x[UR][NV][VEC];
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int sg = (k + u < e) ? row_seg[k + u] : -1;
            const float* src = part + (int64_t)(sg < 0 ? 0 : sg) * F;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                if (sg >= 0 && L.valid(j, F)) {
                    vload<VEC>(x[u][j], src + L.off(j));
                } else {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) x[u][j][v] = 0.f;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < UR; ++u)
#pragma unroll
            for (int j = 0; j < NV; ++j)
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[j][v] += x[u][j][v];
    }
    store_row<VEC, NV>(Y + row * ldy, acc, L, F, 1.f);
}

} // namespace csrk
