// Multi-head fused CSR attention, bf16 Q/K/V, fp32 accumulation.
//
// One wavefront covers one node's H * Dh values: lane l holds 8 consecutive
// bf16 values (16 bytes) of head l / LPH, LPH = Dh / 8 lanes per head, so a
// gathered K or V row is one 16-byte load per lane, coalesced into H * Dh * 2
// contiguous bytes.  Per entry the lanes of a head form the score
// t = scale * <q, k> with a butterfly over the LPH lanes, then fold it into an
// online softmax state (running maximum m, sum of exponentials l, weighted
// sum acc of V rows), rescaling the state only when the maximum moves.  The
// SDDMM, the row softmax and the SpMM of the pipeline thus run in a single
// pass over K and V.  Rows are split across wavefronts by the same merge-path
// chunks as the fp32 kernels; split rows leave (m, l, acc) pieces that the
// fix-up kernel merges.
#pragma once

#include "args.h"
#include "common.h"

namespace csrk {


__device__ __forceinline__ void bf16x8_to_f32(float (&d)[8], uint4 r)
{
    uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        d[2 * i] = __uint_as_float(w[i] << 16);
        d[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

template <int LPH>
struct MhaLanes {
    int lane, head, valid;
    int64_t off;  // element offset of this lane's 8 values within a node row
    __device__ __forceinline__ MhaLanes(int H, int Dh)
    {
        lane = lane_id();
        head = lane / LPH;
        valid = head < H;
        off = (int64_t)head * Dh + (lane % LPH) * 8;
    }
};

template <int LPH>
__device__ __forceinline__ float head_sum(float v)
{
#pragma unroll
    for (int s = 1; s < LPH; s <<= 1) v += shfl_xor(v, s);
    return v;
}

// Gathers the K and V rows of entries k .. k+U-1 (< ke) of a row.
template <int LPH, int U>
__device__ __forceinline__ void mha_issue(const MhaArgs& a, const MhaLanes<LPH>& L, const int32_t* col, int k, int ke,
                                          uint4 (&kr)[U], uint4 (&vr)[U])
{
    const int64_t ld = (int64_t)a.H * a.Dh;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int e = k + u;
        const bool ok = (e < ke) && L.valid;
        const int c = (e < ke) ? col[e] : 0;
        const int64_t base = (int64_t)c * ld + L.off;
        if (ok) {
            kr[u] = *reinterpret_cast<const uint4*>(a.K + base);
            vr[u] = *reinterpret_cast<const uint4*>(a.V + base);
        } else {
            kr[u] = make_uint4(0, 0, 0, 0);
            vr[u] = make_uint4(0, 0, 0, 0);
        }
    }
}

// Folds entries k .. k+U-1 (< ke), whose K and V rows are in kr / vr, into the
// online softmax state (m, l, acc) of the row whose query is q.
template <int LPH, int U>
__device__ __forceinline__ void mha_fold(const MhaArgs& a, const MhaLanes<LPH>& L, const float (&q)[8], int k, int ke,
                                         const uint4 (&kr)[U], const uint4 (&vr)[U], float& m, float& l,
                                         float (&acc)[8])
{
    // the score's 8 products of this lane: the query repacked (its values
    // are bf16 widened, so exactly) and the key's bf16 pairs, two at a time
    // through the two-term dot instruction
    uint32_t qp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) qp[i] = pack_bf16_exact(q[2 * i], q[2 * i + 1]);
    float t[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float s = dot2_bf16(qp[0], kr[u].x, 0.f);
        s = dot2_bf16(qp[1], kr[u].y, s);
        s = dot2_bf16(qp[2], kr[u].z, s);
        s = dot2_bf16(qp[3], kr[u].w, s);
        s = head_sum<LPH>(s) * a.scale;
        t[u] = (k + u < ke) ? s : -INFINITY;
    }
    float mn = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mn = fmaxf(mn, t[u]);
    if (a.probs && L.valid && (L.lane % LPH) == 0) {
        // the scores, turned into probabilities once the row's statistics are final
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (k + u < ke) a.probs[(int64_t)(k + u) * a.H + L.head] = t[u];
    }
    const float corr = (l > 0.f) ? exp_neg(m - mn) : 0.f;
    l *= corr;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= corr;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float p = (k + u < ke) ? exp_neg(t[u] - mn) : 0.f;
        l += p;
        float vf[8];
        bf16x8_to_f32(vf, vr[u]);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(p, vf[i], acc[i]);
    }
    m = mn;
}

// Online-softmax walk over entries [kb, ke) of one row (col indexed by entry id).
template <int LPH, int U>
__device__ __forceinline__ void mha_walk(const MhaArgs& a, const MhaLanes<LPH>& L, const float (&q)[8],
                                         const int32_t* col, int kb, int ke, float& m, float& l,
                                         float (&acc)[8])
{
    for (int k = kb; k < ke; k += U) {
        uint4 kr[U], vr[U];
        mha_issue<LPH, U>(a, L, col, k, ke, kr, vr);
        mha_fold<LPH, U>(a, L, q, k, ke, kr, vr, m, l, acc);
    }
}

template <int LPH>
__device__ __forceinline__ void mha_load_q(float (&q)[8], const MhaArgs& a, const MhaLanes<LPH>& L, int64_t row)
{
    uint4 r = L.valid ? *reinterpret_cast<const uint4*>(a.Q + row * ((int64_t)a.H * a.Dh) + L.off)
                      : make_uint4(0, 0, 0, 0);
    bf16x8_to_f32(q, r);
}

// The probabilities of entries [kb, ke) of a row, every head: exp(t - m_h) /
// l_h from the scores t the wave stored; (m_h, l_h) are held by the lanes of
// head h, so every lane of the wave takes part (the fence orders the stored
// scores before they are read back).
template <int LPH>
__device__ __forceinline__ void mha_probs(const MhaArgs& a, int kb, int ke, float m, float l)
{
    __threadfence_block();
    const int lane = lane_id();
    const int64_t n = (int64_t)(ke - kb) * a.H;
    const int64_t n_up = (n + CSR_WAVE - 1) / CSR_WAVE * CSR_WAVE;  // the same trip count in every lane
    for (int64_t idx = lane; idx < n_up; idx += CSR_WAVE) {
        const int h = (int)(idx % a.H);
        const float mh = __shfl(m, h * LPH, CSR_WAVE), lh = __shfl(l, h * LPH, CSR_WAVE);
        if (idx < n) {
            float* p = a.probs + ((int64_t)kb + idx / a.H) * a.H + h;
            *p = exp_neg(*p - mh) / lh;
        }
    }
}

__device__ __forceinline__ void store8(float* dst, const float (&v)[8], float den)
{
    float4 o0 = make_float4(v[0] / den, v[1] / den, v[2] / den, v[3] / den);
    float4 o1 = make_float4(v[4] / den, v[5] / den, v[6] / den, v[7] / den);
    reinterpret_cast<float4*>(dst)[0] = o0;
    reinterpret_cast<float4*>(dst)[1] = o1;
}

__device__ __forceinline__ void store8_raw(float* dst, const float (&v)[8])
{
    reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// Row-group mapping: one wavefront per row.
template <int LPH, int U>
__global__ __launch_bounds__(CSR_BLOCK) void k_mha_rowgroup(MhaArgs a)
{
    const int64_t row = ((int64_t)blockIdx.x * CSR_BLOCK + threadIdx.x) / CSR_WAVE;
    if (row >= a.n_rows) return;
    MhaLanes<LPH> L(a.H, a.Dh);
    float q[8];
    mha_load_q<LPH>(q, a, L, row);
    float m = -INFINITY, l = 0.f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int b = a.row_ptr[row], e = a.row_ptr[row + 1];
    mha_walk<LPH, U>(a, L, q, a.col_idx, b, e, m, l, acc);
    if (a.probs && e > b) mha_probs<LPH>(a, b, e, m, l);
    if (!L.valid) return;
    float* dst = a.out + row * ((int64_t)a.H * a.Dh) + L.off;
    if (e > b)
        store8(dst, acc, l);
    else
        store8_raw(dst, acc);
}

template <int D>
struct MhaShared {
    int32_t rp[CSR_WAVES_PER_BLOCK][D + 2];
    int32_t col[CSR_WAVES_PER_BLOCK][D];
};

// Merge-path mapping: one wavefront per chunk of D items.
template <int LPH, int U, int D>
__global__ __launch_bounds__(CSR_BLOCK) void k_mha_mergepath(MhaArgs a)
{
    __shared__ MhaShared<D> sh;
    const int wave = threadIdx.x / CSR_WAVE;
    const int lane = lane_id();
    const int64_t chunk = (int64_t)blockIdx.x * CSR_WAVES_PER_BLOCK + wave;
    const bool active = chunk < a.n_chunks;
    int x0 = 0, y0 = 0, x1 = 0, y1 = 0, nrow = 0;
    bool slotB = false;
    if (active) {
        x0 = a.part[2 * chunk];
        y0 = a.part[2 * chunk + 1];
        x1 = a.part[2 * chunk + 2];
        y1 = a.part[2 * chunk + 3];
        // rows x0 .. x1 (x1 only if it exists): row_ptr[x0 .. min(x1, n_rows - 1) + 1]
        const int nr = (x1 < a.n_rows ? x1 : (int)a.n_rows - 1) - x0 + 2;
        stage_chunk<(D + 2 + CSR_WAVE - 1) / CSR_WAVE, D / CSR_WAVE, false, int32_t>(
            sh.rp[wave], a.row_ptr + x0, nr, sh.col[wave], a.col_idx + y0, nullptr, nullptr, y1 - y0);
    }
    __syncthreads();
    if (!active) return;
    const int32_t* rp = sh.rp[wave];
    const int32_t* col = sh.col[wave] - y0;
    slotB = (x1 < a.n_rows) && (max(rp[x1 - x0], y0) < y1);
    nrow = x1 - x0 + (slotB ? 1 : 0);
    const bool slotA = (x0 < x1) && (rp[0] < y0);
    if (lane == 0) {
        a.carry_row[2 * chunk] = slotA ? x0 : -1;
        a.carry_row[2 * chunk + 1] = slotB ? x1 : -1;
    }
    MhaLanes<LPH> L(a.H, a.Dh);
    const int64_t ld = (int64_t)a.H * a.Dh;
    const int nend = x1 - x0;
    for (int i = 0; i < nrow; ++i) {
        const int rs = rp[i], re = rp[i + 1];
        const int sb = max(rs, y0), se = min(re, y1);
        const int64_t row = (int64_t)x0 + i;
        float q[8];
        mha_load_q<LPH>(q, a, L, row);
        float m = -INFINITY, l = 0.f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        mha_walk<LPH, U>(a, L, q, col, sb, se, m, l, acc);
        const bool complete = i < nend && rs >= y0;
        if (a.probs && complete && re > rs) mha_probs<LPH>(a, rs, re, m, l);
        if (!L.valid) continue;
        if (complete) {
            float* dst = a.out + row * ld + L.off;
            if (re > rs)
                store8(dst, acc, l);
            else
                store8_raw(dst, acc);
        } else {
            const int64_t slot = 2 * chunk + ((i == nend) ? 1 : 0);
            store8_raw(a.carry_val + slot * ld + L.off, acc);
            if (lane % LPH == 0) {
                a.carry_ml[(slot * a.H + L.head) * 2] = m;
                a.carry_ml[(slot * a.H + L.head) * 2 + 1] = l;
            }
        }
    }
}

// Fix-up: merge the (m, l, acc) pieces of each split row in chunk order.
template <int LPH>
__device__ __forceinline__ void mha_fixup_one(const MhaArgs& a, int64_t c, int r)
{
    const int lane = lane_id();
    int64_t k0 = c;
    while (true) {
        int64_t idx = k0 - 1 - lane;
        bool ok = idx >= 0 && a.carry_row[2 * idx + 1] == r;
        uint64_t mask = __ballot(ok);
        int n = (~mask == 0) ? 64 : __builtin_ctzll(~mask);
        k0 -= n;
        if (n < 64) break;
    }
    const int64_t np = c - k0 + 1;
    MhaLanes<LPH> L(a.H, a.Dh);
    const int64_t ld = (int64_t)a.H * a.Dh;
    float M = -INFINITY;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0}, lsum = 0.f;
    if (L.valid) {
        for (int64_t p = 0; p < np; ++p) {
            const int64_t s = (p < np - 1) ? 2 * (k0 + p) + 1 : 2 * c;
            const float* ml = a.carry_ml + (s * a.H + L.head) * 2;
            if (ml[1] > 0.f) M = fmaxf(M, ml[0]);
        }
        for (int64_t p = 0; p < np; ++p) {
            const int64_t s = (p < np - 1) ? 2 * (k0 + p) + 1 : 2 * c;
            const float* ml = a.carry_ml + (s * a.H + L.head) * 2;
            const float w = (ml[1] > 0.f) ? exp_neg(ml[0] - M) : 0.f;
            lsum = fmaf(w, ml[1], lsum);
            const float4* src = reinterpret_cast<const float4*>(a.carry_val + s * ld + L.off);
            float4 v0 = src[0], v1 = src[1];
            float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, v[i], acc[i]);
        }
    }
    // the split row's probabilities (every lane takes part: the heads'
    // statistics are exchanged between lanes)
    if (a.probs) mha_probs<LPH>(a, a.row_ptr[r], a.row_ptr[r + 1], M, lsum);
    if (!L.valid) return;
    store8(a.out + (int64_t)r * ld + L.off, acc, lsum);
}

template <int LPH>
__global__ __launch_bounds__(CSR_BLOCK) void k_mha_fixup(MhaArgs a)
{
    const int64_t base = fixup_window(a.n_chunks);
    if (base < 0) return;
    const int lane = lane_id();
    const int64_t mine = base + lane;
    const int rl = (mine < a.n_chunks) ? a.carry_row[2 * mine] : -1;
    uint64_t todo = __ballot(rl >= 0);
    while (todo) {
        const int j = __builtin_ctzll(todo);
        todo &= todo - 1;
        mha_fixup_one<LPH>(a, base + j, __shfl(rl, j, CSR_WAVE));
    }
}

} // namespace csrk
